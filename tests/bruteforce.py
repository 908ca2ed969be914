"""Brute-force reference computations for tiny inputs (pure Python loops).

Independent of oracle/: written from the method's description by enumeration
instead of sorting, for use as pins of the oracle on tiny sizes.
"""
import itertools
import math

import numpy as np


def logits_loop(x, wr):
    """L[t][e] = sum_h x[t][h] * wr[h][e] by an explicit float64 loop, rounded to float32."""
    T, H = x.shape
    E = wr.shape[1]
    out = np.zeros((T, E), dtype=np.float32)
    for t in range(T):
        for e in range(E):
            acc = 0.0
            for h in range(H):
                acc += float(x[t, h]) * float(wr[h, e])
            out[t, e] = np.float32(acc)
    return out


def select_enumerate(z, n_groups, topk_groups, topk, group_topn=2):
    """Node-limited selection by enumeration of subsets, for one token.

    z: float32 [E] biased scores.  Group score = the largest sum over all
    ``group_topn``-subsets of the group's experts.  The kept groups are the
    ``topk_groups``-subset of groups with the largest total group score; the
    chosen experts are the ``topk``-subset of the kept groups' experts with the
    largest total score.  Equal totals break toward the lexicographically
    smallest index tuple.  Sums are exact (float64 of float32 values).
    """
    E = len(z)
    per = E // n_groups
    zf = [float(v) for v in z]
    gscore = []
    for g in range(n_groups):
        members = range(g * per, (g + 1) * per)
        best = max(sum(zf[i] for i in c) for c in itertools.combinations(members, group_topn))
        gscore.append(best)
    best_g, best_gs = None, -math.inf
    for c in itertools.combinations(range(n_groups), topk_groups):
        tot = sum(gscore[g] for g in c)
        if tot > best_gs:
            best_g, best_gs = c, tot
    elig = [i for g in best_g for i in range(g * per, (g + 1) * per)]
    best_e, best_es = None, -math.inf
    for c in itertools.combinations(sorted(elig), topk):
        tot = sum(zf[i] for i in c)
        if tot > best_es:
            best_e, best_es = c, tot
    return sorted(best_e), sorted(best_g), gscore


def swiglu_loop(xv, wg, wu, wd):
    """One token through one SwiGLU expert by scalar loops.

    h_j = silu(sum_k wg[j][k] x_k) * (sum_k wu[j][k] x_k); y_i = sum_j wd[i][j] h_j.
    """
    I, H = wg.shape
    h = [0.0] * I
    for j in range(I):
        g = 0.0
        u = 0.0
        for k in range(H):
            g += float(wg[j, k]) * float(xv[k])
            u += float(wu[j, k]) * float(xv[k])
        h[j] = g / (1.0 + math.exp(-g)) * u
    y = [0.0] * H
    for i in range(H):
        acc = 0.0
        for j in range(I):
            acc += float(wd[i, j]) * h[j]
        y[i] = acc
    return np.array(y)


def e4m3_slices_loop(v):
    """Quantise-then-dequantise a vector slice by slice, 128 entries a slice.

    Per slice: amax by a loop; scale = amax / 448 in float32 (1 where that is
    zero); each entry's float32 quotient v / scale, saturated at +-448, is
    rounded to an E4M3FN value by torch's float8_e4m3fn conversion (an
    encoder independent of the oracle's); the result is value * scale in
    float64.
    """
    import torch
    out = []
    for s0 in range(0, len(v), 128):
        sl = [np.float32(a) for a in v[s0:s0 + 128]]
        amax = np.float32(0.0)
        for a in sl:
            if abs(a) > amax:
                amax = np.float32(abs(a))
        scale = np.float32(amax / np.float32(448.0))
        if scale == 0:
            scale = np.float32(1.0)
        for a in sl:
            r = min(max(float(np.float32(a / scale)), -448.0), 448.0)
            code = torch.tensor([r], dtype=torch.float32).to(torch.float8_e4m3fn)
            out.append(float(code.to(torch.float64)[0]) * float(scale))
    return np.array(out)


def swiglu_fp8_loop(xv, wg, wu, wd):
    """One token through one expert on the E4M3 forward path, by loops.

    The token's input is quantised per 1x128 slice; h_j = silu(g_j) * u_j from
    exact dot products with the quantised input, rounded to float32 and
    quantised per 1x128 slice; y_i = sum_j wd[i][j] hq_j.
    """
    I, H = wg.shape
    xq = e4m3_slices_loop(xv)
    h = np.zeros(I, dtype=np.float32)
    for j in range(I):
        g = float(np.dot(wg[j], xq))
        u = float(np.dot(wu[j], xq))
        e = math.exp(-g) if g > -700.0 else math.inf     # SiLU(g) -> -0 for very negative g
        h[j] = np.float32(g / (1.0 + e) * u)
    hq = e4m3_slices_loop(h)
    return np.array([float(np.dot(wd[i], hq)) for i in range(H)])
