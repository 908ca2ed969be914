// Internal helpers of the gfx950 MoE library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#define MOE_DEV __device__ __forceinline__

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte register chunk
typedef uint16_t bf16_t;  // bfloat16 storage

constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16

MOE_DEV float bf16_to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// round to nearest even; NaN stays NaN
MOE_DEV bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

template <typename T> MOE_DEV float to_f32(T v);
template <> MOE_DEV float to_f32<float>(float v) { return v; }
template <> MOE_DEV float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> MOE_DEV T from_f32(float v);
template <> MOE_DEV float from_f32<float>(float v) { return v; }
template <> MOE_DEV bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// ---------------------------------------------------------------- math

// logistic sigmoid in float32 with the device library's expf
MOE_DEV float sigmoidf(float v) { return 1.0f / (1.0f + expf(-v)); }

MOE_DEV float siluf(float v) { return v / (1.0f + expf(-v)); }

// ---------------------------------------------------------------- E4M3

// OCP E4M3FN code of a float32 value, round to nearest even, |v| clamped to 448
MOE_DEV uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  if (a < 0.015625f) {  // below the smallest normal 2^-6: steps of 2^-9
    return sign | uint32_t(rintf(a * 512.0f));  // 8 lands on the smallest normal's code
  }
  uint32_t u = __float_as_uint(a);
  u += 0x7ffffu + ((u >> 20) & 1u);  // round the mantissa to 3 bits, ties to even
  return sign | ((u >> 20) - (120u << 3));  // rebias the exponent 127 -> 7
}

// scale of a quantisation tile from its max-abs value: amax / 448, or 1 where
// that is zero (an all-zero tile, or a max-abs so small that it underflows)
MOE_DEV float e4m3_scale(float amax) {
  const float s = amax / 448.0f;
  return s > 0.f ? s : 1.0f;
}

// value of an E4M3FN code (NaN codes are never produced by e4m3_encode)
MOE_DEV float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? float(m) * 0.001953125f  // subnormal: m * 2^-9
                           : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------- wave helpers

MOE_DEV void argmax_take(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

// one arg-max step with a DPP lane move (CTRL: a 16-lane-row pattern)
template <int CTRL> MOE_DEV void argmax_dpp(float& v, int& i) {
  const float ov =
      __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xf, 0xf, false);
  argmax_take(v, i, ov, oi);
}

// (value, index) arg-max over the wave: larger value wins, equal values go to
// the smaller index.  Every lane returns the winner.  The rule is associative
// and commutative, so any reduction order gives the same winner: quad swaps
// (lane ^ 1, lane ^ 2) and rotations by 4 and 8 within each 16-lane row use
// DPP moves; the last two steps cross rows with lane shuffles.
MOE_DEV void wave_argmax(float& v, int& i) {
  argmax_dpp<0xb1>(v, i);   // quad_perm [1,0,3,2]
  argmax_dpp<0x4e>(v, i);   // quad_perm [2,3,0,1]
  argmax_dpp<0x124>(v, i);  // row_ror:4
  argmax_dpp<0x128>(v, i);  // row_ror:8
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) argmax_take(v, i, __shfl_xor(v, off, kWave),
                                                       __shfl_xor(i, off, kWave));
}

MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

MOE_DEV int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- global -> LDS copies

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over [base, base + bytes) for raw loads (stride 0; dword 3
// selects the 32-bit data format).  Loads past `bytes` return zeros.
MOE_DEV __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// 16 bytes per lane from byte offset voff of the buffer straight into LDS:
// lane l writes dst + 16 l (dst uniform).  The buffer form (MUBUF) is used
// rather than global_load_lds: this compiler treats the FLAT-encoded copy as
// a possible LDS access and then makes every later LDS-read wait drain the
// whole LDS queue (lgkmcnt(0)), serialising fragment reads with the MFMAs.
MOE_DEV void copy16_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t voff, bf16_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff, 0, 0, 0);
}

}  // namespace moe
