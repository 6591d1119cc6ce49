// Single-token recurrent decode for gfx950 (aiwiki.thehackersbrain.dev page, "It is
// a linear RNN": constant work per token and a fixed-size state; the mlblogg.com page,
// "The causal recurrence": the token is added before it is read).
//
// One workgroup per (batch, head).  The fp32 state S [D][Dv] is streamed once: every
// thread issues all of its 16-byte loads before using any, updates
// S += phi(k) v^T in registers, writes the rows back with nontemporal stores and
// accumulates its share of phi(q)^T S.  The partial numerators are reduced across
// the row groups of a wave with lane exchanges and across waves through LDS; the
// denominator phi(q) . z is reduced the same way.  The kernel is bound by HBM
// bandwidth: 2 * D * Dv * 4 bytes of state traffic per head against 4 * D * Dv flops.
//
// The gated step decays the state first, S <- g S + phi(k) v^T and z <- g z + phi(k),
// with one gate per head (aicassindra.com page, "RetNet and gated linear attention");
// a NULL gate is 1, and since 1 * s is exact the ungated step is the same arithmetic.
// With a per-dimension decay ga [D] per head (gated linear attention's Diag(alpha)),
// row d of S and z[d] take ga[d] instead.
// In the normaliser-free mode (retention's output, no phi(q)^T z denominator) o is the
// numerator and z, which may then be NULL, is left alone.
#pragma once

#include "device_common.hpp"

namespace linattn {

template <typename E, int D, int DV>
__global__ __launch_bounds__(kThreads) void decode_kernel(const E* __restrict__ q, const E* __restrict__ k,
                                                         const E* __restrict__ v, const float* __restrict__ g,
                                                         const float* __restrict__ ga, float* __restrict__ S,
                                                         float* __restrict__ z, E* __restrict__ o, float eps,
                                                         int normalize) {
    using X = Elem<E>;
    constexpr int CQ = DV / 4;            // 16-byte column quads per state row
    constexpr int RG = kThreads / CQ;     // row groups
    constexpr int RPT = D / RG;           // rows per thread
    static_assert(kThreads % CQ == 0 && D % RG == 0, "decode tiling");

    __shared__ float s_num[kThreads / kWave][DV];
    __shared__ float s_den[kThreads / kWave];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int cq = tid % CQ;
    const int rg = tid / CQ;
    const int w = tid / kWave;
    const int lane = tid % kWave;

    float* Sb = S + size_t(bh) * D * DV;
    const E* qb = q + size_t(bh) * D;
    const E* kb = k + size_t(bh) * D;
    const E* vb = v + size_t(bh) * DV;

    f32x4_t srow[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        srow[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(Sb + size_t(rg + RG * i) * DV + 4 * cq));

    float vv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vv[r] = X::to_f32(vb[4 * cq + r]);
    const float gt = g ? g[bh] : 1.0f;
    const float* gab = ga ? ga + size_t(bh) * D : nullptr;
    // the decay of each of this thread's rows, read once (behind a uniform branch) while
    // the state loads are in flight
    float gd[RPT];
    if (gab) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) gd[i] = gab[rg + RG * i];
    } else {
#pragma unroll
        for (int i = 0; i < RPT; ++i) gd[i] = gt;
    }

    // denominator: z' = g z + phi(k), den = phi(q) . z'
    float den = 0.0f;
    if (z && tid < D) {
        const float zn = fmaf(gab ? gab[tid] : gt, z[size_t(bh) * D + tid], phi(X::to_f32(kb[tid])));
        z[size_t(bh) * D + tid] = zn;
        den = phi(X::to_f32(qb[tid])) * zn;
    }

    f32x4_t num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int d = rg + RG * i;
        const float fk = phi(X::to_f32(kb[d]));
        const float fq = phi(X::to_f32(qb[d]));
        f32x4_t s = srow[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = fmaf(fk, vv[r], gd[i] * s[r]);
        __builtin_nontemporal_store(s, reinterpret_cast<f32x4_t*>(Sb + size_t(d) * DV + 4 * cq));
#pragma unroll
        for (int r = 0; r < 4; ++r) num[r] = fmaf(fq, s[r], num[r]);
    }

    // reduce numerators over the row groups that share this column quad
#pragma unroll
    for (int off = CQ; off < kWave; off <<= 1)
#pragma unroll
        for (int r = 0; r < 4; ++r) num[r] += __shfl_xor(num[r], off, kWave);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) den += __shfl_xor(den, off, kWave);
    if (lane < CQ)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_num[w][4 * cq + r] = num[r];
    if (lane == 0) s_den[w] = den;
    __syncthreads();
    if (tid < DV) {
        float nsum = 0.0f, dsum = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kThreads / kWave; ++ww) { nsum += s_num[ww][tid]; dsum += s_den[ww]; }
        o[size_t(bh) * DV + tid] = X::from_f32(normalize ? nsum / fmaxf(dsum, eps) : nsum);
    }
}

}  // namespace linattn
