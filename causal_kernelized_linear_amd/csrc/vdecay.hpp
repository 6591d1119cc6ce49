// Per-dimension decay (gated linear attention) on gfx950:
//     S_t = Diag(a_t) S_{t-1} + phi(k_t) v_t^T,   z_t = a_t * z_{t-1} + phi(k_t),
//     o_t = S_t^T phi(q_t) / max(phi(q_t) . z_t, eps)   (or the numerator alone)
// with a_t in [2^-8, 1]^D per head and token (aicassindra.com page, "RetNet and gated
// linear attention": S_i = Diag(alpha_i) S_{i-1} + k_i v_i^T; aiwiki.thehackersbrain.dev
// page, "What is actually lost": an elementwise decay G_t of S_{t-1}, here
// G_t[d, e] = a_t[d]).
//
// Chunk algebra for a chunk of C = 64 tokens, with the chunk-local inclusive
// L_i[d] = sum_{l=s..i} log2 a_l[d]:
//     A_ij  = sum_d Fq_i[d] Fk_j[d] 2^(L_i[d] - L_j[d])          (j <= i)
//     num_i = (Fq_i * 2^L_i) S_prev + sum_j A_ij v_j,   den_i alike with z_prev and 1
//     S_next = Diag(2^L_last) S_prev + (Fk * 2^(L_last - L))^T V   (z alike)
// A is no single product: the decay depends on the dimension.  It is formed per pair of
// 16-row blocks (I, J), J <= I, against a reference row R of the key block:
//     A_ij = sum_d (Fq_i[d] 2^(L_i[d] - L_R[d])) (Fk_j[d] 2^(L_R[d] - L_j[d]))
// an MFMA product of operands rescaled on the fly.  For J < I, R is the key block's
// last row and both factors are at most 1; for J = I, R is the block's middle row and
// both exponents stay within 8 rows of decay, 2^64 at most when a >= 2^-8.
//
//   vd_totals_kernel  per (head, chunk): the chunk's decayed total and L_last
//   vd_scan_kernel    per state element: the state after every chunk, from S0
//   vd_out_kernel     per (head, chunk): the outputs from the state in front
#pragma once

#include "bwd.hpp"

namespace linattn {

struct VdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* a;      // [BH][N][D]
    void* o;
    const float* s0;     // [BH][D][Dv] or NULL
    const float* z0;     // [BH][D] or NULL
    float* st;           // [BH][NC][D*Dv] accumulator layout: chunk totals, then (scan) the state after each chunk
    float* zt;           // [BH][NC][D]
    float* lg;           // [BH][NC][D]: L_last of each chunk (log2)
    int N;
    int NC;
    float eps;
    int normalize;
};

template <typename E, int D, int DV>
struct VdShape {
    static constexpr int C = kBwdChunk;
    static constexpr int PAD = 16 / int(sizeof(E));
    static constexpr int LQ = D + PAD;
    static constexpr int LV = DV + PAD;
    static constexpr int LA = C + PAD;
    static constexpr int LL = D + 4;                   // fp32 decay rows
    static constexpr size_t kOffQ = 0;                 // phi(Q) [C][D]
    static constexpr size_t kOffK = kOffQ + size_t(C) * LQ * sizeof(E);   // phi(K) [C][D]
    static constexpr size_t kOffV = kOffK + size_t(C) * LQ * sizeof(E);   // V [C][Dv] (then O)
    static constexpr size_t kOffS = kOffV + size_t(C) * LV * sizeof(E);   // S_prev [D][Dv]
    static constexpr size_t kOffA = kOffS + size_t(D) * LV * sizeof(E);   // A [C][C]
    static constexpr size_t kOffL = kOffA + size_t(C) * LA * sizeof(E);   // L [C][D] fp32
    static constexpr size_t kOffZ = kOffL + size_t(C) * LL * 4;           // z_prev [D] fp32
    static constexpr size_t kBytes = kOffZ + size_t(D) * 4;
    static_assert(kBytes == vd_lds_bytes(int(sizeof(E)), D, DV), "host LDS formula out of step");
    static constexpr int kWaves = int(kMaxLds / kBytes) < 1 ? 1 : int(kMaxLds / kBytes);
    static constexpr int EPG = 16 / int(sizeof(E));
};

// Rows [ts, ts + C) of a [N][W] tensor into registers (16-byte units, rows clamped to the
// last valid one) and from them into a row-major LDS tile (rows past the end zeroed).
template <typename E, int W>
struct VdRows {
    static constexpr int C = kBwdChunk;
    static constexpr int U = C * W * int(sizeof(E)) / 16 / kThreads;
    static constexpr int G = W * int(sizeof(E)) / 16;
    static constexpr int EPG = 16 / int(sizeof(E));
    f32x4_t r[U];

    __device__ __forceinline__ void load(const E* src, int tid, int ts, int nrows) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = (idx % G) * EPG;
            r[u] = *reinterpret_cast<const f32x4_t*>(src + size_t(ts + min(row, nrows - 1)) * W + col);
        }
    }

    template <bool PHI>
    __device__ __forceinline__ void store(E* tile, int ld, int tid, int nrows) const {
        using X = Elem<E>;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = (idx % G) * EPG;
            f32x4_t out = {0.f, 0.f, 0.f, 0.f};
            if (row < nrows) {
                if constexpr (sizeof(E) == 2) {
                    const F8<E> in = __builtin_bit_cast(F8<E>, r[u]);
                    F8<E> o;
#pragma unroll
                    for (int e = 0; e < 8; ++e) o.x[e] = PHI ? X::from_f32(phi(X::to_f32(in.x[e]))) : in.x[e];
                    out = __builtin_bit_cast(f32x4_t, o);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = PHI ? phi(r[u][e]) : r[u][e];
                }
            }
            *reinterpret_cast<f32x4_t*>(tile + row * ld + col) = out;
        }
    }
};

// The decays of the chunk into sL as the inclusive log2 prefix L (rows past the end
// decay by 1).  Loads first, then one thread per dimension walks the rows.
template <int D>
__device__ __forceinline__ void vd_stage_lambda(float* sL, int LL, const float* ab, int tid, int ts, int nrows) {
    constexpr int C = kBwdChunk;
    constexpr int U = C * D / 4 / kThreads;
    f32x4_t r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int idx = tid + u * kThreads, row = idx / (D / 4), col = 4 * (idx % (D / 4));
        r[u] = *reinterpret_cast<const f32x4_t*>(ab + size_t(ts + min(row, nrows - 1)) * D + col);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int idx = tid + u * kThreads, row = idx / (D / 4), col = 4 * (idx % (D / 4));
        f32x4_t x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = row < nrows ? fast_log2(r[u][e]) : 0.0f;
        *reinterpret_cast<f32x4_t*>(sL + row * LL + col) = x;
    }
    __syncthreads();
    if (tid < D) {
        float acc = 0.0f;
        for (int i = 0; i < C; ++i) {
            acc += sL[i * LL + tid];
            sL[i * LL + tid] = acc;
        }
    }
}

// ------------------------------------------------------------ chunk totals ----

template <typename E, int D, int DV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(VdShape<E, D, DV>::kWaves,
                                                                           VdShape<E, D, DV>::kWaves)))
void vd_totals_kernel(VdArgs args) {
    using Sh = VdShape<E, D, DV>;
    using X = Elem<E>;
    constexpr int C = Sh::C, LQ = Sh::LQ, LV = Sh::LV, LL = Sh::LL;
    constexpr int NA = D / 16, NB = DV / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    E* sK = reinterpret_cast<E*>(smem + Sh::kOffK);
    E* sV = reinterpret_cast<E*>(smem + Sh::kOffV);
    float* sL = reinterpret_cast<float*>(smem + Sh::kOffL);
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int N = args.N, NC = args.NC;
    const int c = blockIdx.x % NC, bh = blockIdx.x / NC, ts = c * C, nrows = min(C, N - ts);

    VdRows<E, D> rk;
    VdRows<E, DV> rv;
    rk.load(reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D, tid, ts, nrows);
    rv.load(reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV, tid, ts, nrows);
    vd_stage_lambda<D>(sL, LL, args.a + size_t(bh) * N * D, tid, ts, nrows);
    rk.template store<true>(sK, LQ, tid, nrows);
    rv.template store<false>(sV, LV, tid, nrows);
    __syncthreads();
    // decayed keys Fk_j * 2^(L_last - L_j) in place; z total in fp32 (one thread per dimension)
    const size_t slot = size_t(bh) * NC + c;
    if (tid < D) {
        const float last = sL[(C - 1) * LL + tid];
        float zs = 0.0f;
        for (int j = 0; j < C; ++j) {
            const float x = X::to_f32(sK[j * LQ + tid]) * fast_exp2(last - sL[j * LL + tid]);
            zs += x;
            sK[j * LQ + tid] = X::from_f32(x);
        }
        args.zt[slot * D + tid] = zs;
        args.lg[slot * D + tid] = last;
    }
    __syncthreads();
    // dS = Fk~^T V, tiles dealt to the waves, written in accumulator layout
    constexpr int NT = NA * NB;
#pragma unroll
    for (int u0 = 0; u0 < NT; u0 += 4) {
        const int u = u0 + w;
        if (u < NT) {
            const int ta = u / NB, tb = u % NB;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C / 32; ++ks)
                acc = mma(frag_col(sK, LQ, 32 * ks + 8 * g4, 16 * ta, l16), frag_col(sV, LV, 32 * ks + 8 * g4, 16 * tb, l16),
                          acc);
            *reinterpret_cast<f32x4_t*>(args.st + slot * (D * DV) + (u * kWave + lane) * 4) = acc;
        }
    }
}

// ------------------------------------------------------------------- scan ----

// In place over the NC chunk slots of each head: slot c becomes the state after chunk c,
// S_c = 2^(L_last,c[d]) S_{c-1} + dS_c (rows d), starting from S0 / z0.
template <int D, int DV>
__global__ __launch_bounds__(kThreads) void vd_scan_kernel(float* st, float* zt, const float* lg, const float* s0,
                                                           const float* z0, int NC) {
    constexpr int NS = D * DV;
    constexpr int NBLK = (NS + D + kThreads - 1) / kThreads;
    const int e = (blockIdx.x % NBLK) * kThreads + threadIdx.x;
    const int bh = blockIdx.x / NBLK;
    if (e >= NS + D) return;
    float* base;
    size_t stride, uidx;
    int d;
    const float* init;
    if (e < NS) {
        const int u = e / 256, ln = (e / 4) % 64, r = e % 4;
        const int ta = u / (DV / 16), tb = u % (DV / 16);
        d = 16 * ta + 4 * (ln / 16) + r;
        const int dv = 16 * tb + ln % 16;
        uidx = size_t(bh) * NS + size_t(d) * DV + dv;
        base = st + size_t(bh) * NC * NS + e;
        stride = NS;
        init = s0;
    } else {
        d = e - NS;
        uidx = size_t(bh) * D + d;
        base = zt + size_t(bh) * NC * D + d;
        stride = D;
        init = z0;
    }
    const float* lgb = lg + size_t(bh) * NC * D + d;
    float acc = init ? init[uidx] : 0.0f;
    constexpr int U = 8;                         // loads in flight per thread
    for (int c0 = 0; c0 < NC; c0 += U) {
        float t[U], f[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int c = min(c0 + i, NC - 1);
            t[i] = base[size_t(c) * stride];
            f[i] = fast_exp2(lgb[size_t(c) * D]);
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (c0 + i < NC) {
                acc = f[i] * acc + t[i];
                base[size_t(c0 + i) * stride] = acc;
            }
        }
    }
}

// ----------------------------------------------------------------- outputs ----

template <typename E, int D, int DV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(VdShape<E, D, DV>::kWaves,
                                                                           VdShape<E, D, DV>::kWaves)))
void vd_out_kernel(VdArgs args) {
    using Sh = VdShape<E, D, DV>;
    using X = Elem<E>;
    constexpr int C = Sh::C, LQ = Sh::LQ, LV = Sh::LV, LA = Sh::LA, LL = Sh::LL;
    constexpr int NE = DV / 16, NJ = C / 16, ND = D / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    E* sQ = reinterpret_cast<E*>(smem + Sh::kOffQ);
    E* sK = reinterpret_cast<E*>(smem + Sh::kOffK);
    E* sV = reinterpret_cast<E*>(smem + Sh::kOffV);
    E* sS = reinterpret_cast<E*>(smem + Sh::kOffS);
    E* sA = reinterpret_cast<E*>(smem + Sh::kOffA);
    float* sL = reinterpret_cast<float*>(smem + Sh::kOffL);
    float* sZ = reinterpret_cast<float*>(smem + Sh::kOffZ);
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int N = args.N, NC = args.NC;
    const int c = blockIdx.x % NC, bh = blockIdx.x / NC, ts = c * C, nrows = min(C, N - ts);

    // staging: every load first
    {
        VdRows<E, D> rq, rk;
        VdRows<E, DV> rv;
        constexpr int SU = D * DV / 4 / kThreads;
        f32x4_t rs[SU];
        rq.load(reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D, tid, ts, nrows);
        rk.load(reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D, tid, ts, nrows);
        rv.load(reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV, tid, ts, nrows);
        const size_t pslot = size_t(bh) * NC + (c - 1);
        if (c > 0) {
#pragma unroll
            for (int u = 0; u < SU; ++u)
                rs[u] = *reinterpret_cast<const f32x4_t*>(args.st + pslot * (D * DV) + 4 * (tid + u * kThreads));
        }
        vd_stage_lambda<D>(sL, LL, args.a + size_t(bh) * N * D, tid, ts, nrows);
        rq.template store<true>(sQ, LQ, tid, nrows);
        rk.template store<true>(sK, LQ, tid, nrows);
        rv.template store<false>(sV, LV, tid, nrows);
        if (c > 0) {
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                const int q4 = tid + u * kThreads, t = q4 / kWave, ln = q4 % kWave;
                const int ta = t / (DV / 16), tb = t % (DV / 16);
                const int d = 16 * ta + 4 * (ln >> 4), e = 16 * tb + (ln & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[(d + r) * LV + e] = X::from_f32(rs[u][r]);
            }
            for (int d = tid; d < D; d += kThreads) sZ[d] = args.zt[pslot * D + d];
        } else {
            const float* us = args.s0 ? args.s0 + size_t(bh) * D * DV : nullptr;
            for (int q4 = tid; q4 < D * DV / 4; q4 += kThreads) {
                const int d = q4 / (DV / 4), e = 4 * (q4 % (DV / 4));
                f32x4_t x = {0.f, 0.f, 0.f, 0.f};
                if (us) x = *reinterpret_cast<const f32x4_t*>(us + size_t(d) * DV + e);
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[d * LV + e + r] = X::from_f32(x[r]);
            }
            for (int d = tid; d < D; d += kThreads) sZ[d] = args.z0 ? args.z0[size_t(bh) * D + d] : 0.0f;
        }
    }
    __syncthreads();

    const int i0 = 16 * w;            // this wave's query rows (block I = w)
    // num = (Fq * 2^L_i) S_prev; den = (Fq * 2^L_i) . z_prev
    f32x4_t num[NE];
#pragma unroll
    for (int et = 0; et < NE; ++et) num[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        const int d0 = 32 * ks + 8 * g4;
        const F8<E> fq = frag_row(sQ, LQ, i0 + l16, d0);
        F8<E> a;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            a.x[e] = X::from_f32(X::to_f32(fq.x[e]) * fast_exp2(sL[(i0 + l16) * LL + d0 + e]));
#pragma unroll
        for (int et = 0; et < NE; ++et) num[et] = mma(a, frag_col(sS, LV, d0, 16 * et, l16), num[et]);
    }
    float dz[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * g4 + r;
        float x = 0.0f;
#pragma unroll
        for (int t = 0; t < ND; ++t) {
            const int d = 16 * t + l16;
            x += X::to_f32(sQ[i * LQ + d]) * fast_exp2(sL[i * LL + d]) * sZ[d];
        }
        dz[r] = x;
    }

    // A over the blocks J <= I, each against its reference row, into sA (E); row sums
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (jt <= w) {
            const int ref = jt < w ? 16 * jt + 15 : 16 * jt + 7;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const int d0 = 32 * ks + 8 * g4;
                const F8<E> fq = frag_row(sQ, LQ, i0 + l16, d0);
                const F8<E> fk = frag_row(sK, LQ, 16 * jt + l16, d0);
                F8<E> qa, kb;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float lr = sL[ref * LL + d0 + e];
                    qa.x[e] = X::from_f32(X::to_f32(fq.x[e]) * fast_exp2(sL[(i0 + l16) * LL + d0 + e] - lr));
                    kb.x[e] = X::from_f32(X::to_f32(fk.x[e]) * fast_exp2(lr - sL[(16 * jt + l16) * LL + d0 + e]));
                }
                acc = mma(qa, kb, acc);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = i0 + 4 * g4 + r, j = 16 * jt + l16;
            const E xe = X::from_f32((jt <= w && j <= i) ? acc[r] : 0.0f);
            sA[i * LA + j] = xe;
            rsum[r] += X::to_f32(xe);
        }
    }
    float den[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) den[r] = sum16(rsum[r] + dz[r]);
    __syncthreads();

    // num += A V
    for (int ks = 0; ks <= (w >> 1); ++ks) {
        const F8<E> a = frag_row(sA, LA, i0 + l16, 32 * ks + 8 * g4);
#pragma unroll
        for (int et = 0; et < NE; ++et) num[et] = mma(a, frag_col(sV, LV, 32 * ks + 8 * g4, 16 * et, l16), num[et]);
    }
    __syncthreads();                  // every read of V is done: it takes O
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float inv = args.normalize ? 1.0f / fmaxf(den[r], args.eps) : 1.0f;
#pragma unroll
        for (int et = 0; et < NE; ++et) sV[(i0 + 4 * g4 + r) * LV + 16 * et + l16] = X::from_f32(num[et][r] * inv);
    }
    __syncthreads();
    {
        constexpr int G = DV * int(sizeof(E)) / 16;
        E* ob = reinterpret_cast<E*>(args.o) + size_t(bh) * N * DV;
        for (int u = tid; u < C * G; u += kThreads) {
            const int row = u / G, col = (u % G) * Sh::EPG;
            if (row < nrows)
                *reinterpret_cast<f32x4_t*>(ob + size_t(ts + row) * DV + col) =
                    *reinterpret_cast<const f32x4_t*>(sV + row * LV + col);
        }
    }
}

}  // namespace linattn
