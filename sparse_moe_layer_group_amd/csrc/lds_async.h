// LDS copies issued from inline assembly, for kernels whose LDS reads the
// compiler cannot tell apart from the copies' targets.
#pragma once

#include "common.h"

namespace moe {

// The copies of copy16_to_lds issued from inline assembly (4 or 16 bytes per
// lane), for kernels that read LDS with the transposing ds_read_b64_tr_b{8,16}: this
// compiler cannot tell those reads apart from the copies' targets and makes
// each of them wait until every copy in flight has landed (vmcnt(0)), which
// turns a ring of stages into synchronous copies.  Issued as assembly, the
// copies are outside that analysis.  A kernel using these orders its copies
// and LDS reads with its own vmcnt waits and barriers, and must not have a
// vector-memory load of its own in flight across them (the compiler would
// count its waits for that load without these copies).  M0 takes the LDS
// address through the operand constraint; the s_nop covers the M0 -> LDS DMA
// hazard.  The resource and the LDS address must be wave-uniform: the
// compiler places a divergent value for an "s" operand in vector registers,
// which this instruction cannot take.
MOE_DEV void copy_to_lds_async16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* dst) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)dst));
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}
// the 16-byte copy with the non-temporal hint, for data read once
MOE_DEV void copy_to_lds_async16_nt(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* dst) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)dst));
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}
MOE_DEV void copy_to_lds_async4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* dst) {
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)dst));
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}

}  // namespace moe
