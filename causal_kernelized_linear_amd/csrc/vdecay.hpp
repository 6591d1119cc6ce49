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
// The chunks of each head are walked in runs of LC (as the gradients' passes do): a
// workgroup carries the state through its run in fp32 registers, so state slots exist
// per run, not per chunk.
//   vd_totals_kernel  per (head, run): the run's decayed total and its summed L_last
//   vd_scan_kernel    per state element: the state after every run, from S0
//   vd_out_kernel     per (head, run): the outputs, from the state in front of the run
//                     stepped across each chunk, S <- Diag(2^L_last) S + Fk~^T V with
//                     Fk~ = Fk * 2^(L_last - L); z alike, as an extra column block of
//                     the same product (V's pad column holds 1).
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
    float* st;           // [BH][NR][D*Dv] accumulator layout: run totals, then (scan) the state after each run
    float* zt;           // [BH][NR][D]
    float* lg;           // [BH][NR][D]: the summed L_last of each run (log2)
    int N;
    int NC;              // chunks of C tokens
    int LC;              // chunks per run
    int NR;              // runs, ceil(NC / LC)
    int NT;              // runs whose totals are formed: NR - 1, or NR when the final state is wanted
    float eps;
    int normalize;
};

template <typename E, int D, int DV>
struct VdShape {
    static constexpr int C = kBwdChunk;
    static constexpr int PAD = 16 / int(sizeof(E));
    static constexpr int LQ = D + PAD;
    static constexpr int LV = DV + PAD;
    static constexpr int LL = D + 4;                   // fp32 decay rows
    static constexpr size_t kOffQ = 0;                 // phi(Q) [C][D]
    static constexpr size_t kOffK = kOffQ + size_t(C) * LQ * sizeof(E);   // phi(K) [C][D]
    static constexpr size_t kOffV = kOffK + size_t(C) * LQ * sizeof(E);   // V [C][Dv] (then O)
    static constexpr size_t kOffS = kOffV + size_t(C) * LV * sizeof(E);   // S_prev [D][Dv]
    static constexpr size_t kOffL = kOffS + size_t(D) * LV * sizeof(E);   // L [C][D] fp32
    static constexpr size_t kOffZ = kOffL + size_t(C) * LL * 4;           // z_prev [D] fp32
    static constexpr size_t kBytes = kOffZ + size_t(D) * 4;
    static_assert(kBytes == vd_lds_bytes(int(sizeof(E)), D, DV), "host LDS formula out of step");
    // workgroups (waves per SIMD) per CU the launch plans for and the register target:
    // what the LDS allows, at most two (three, where the LDS would allow it, measured
    // slower: vdecay_bf16 266 against 232 us)
    static constexpr int kLdsWaves = int(kMaxLds / kBytes) < 1 ? 1 : int(kMaxLds / kBytes);
    static constexpr int kWaves = kLdsWaves < 2 ? kLdsWaves : 2;
    // next chunk's rows in flight during this chunk's work (where the registers allow:
    // the totals kernel below 128 x 128 bf16, the output kernel at 64 x 64 bf16)
    static constexpr bool kAhead = sizeof(E) == 2 && D * DV < 128 * 128;
    static constexpr bool kAheadOut = sizeof(E) == 2 && D * DV <= 64 * 64;
    static constexpr int EPG = 16 / int(sizeof(E));
};

// Rows [ts, ts + C) of a [N][W] tensor into registers (16-byte units, rows clamped to the
// last valid one) and from them into a row-major LDS tile (rows past the end zeroed).
// The loads are non-temporal, as are the decays': the output kernel reads every row for
// the last time, and what the totals kernel reads (k, v and the fp32 decays, 268 MB on
// vdecay_bf16) exceeds the 256 MB last-level cache before the output kernel rereads it.
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
            r[u] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4_t*>(src + size_t(ts + min(row, nrows - 1)) * W + col));
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

// The decays of rows [ts, ts + C) as log2 into sL [C][LL] (rows past the end decay by 1),
// for vd_prefix to sum.  load: coalesced 16-byte units (rows clamped); store: log2 into sL
// row-major.
template <int D>
struct VdDecays {
    static constexpr int C = kBwdChunk, U = C * D / 4 / kThreads, G = D / 4;
    f32x4_t r[U];

    __device__ __forceinline__ void load(const float* ab, int tid, int ts, int nrows) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = 4 * (idx % G);
            r[u] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4_t*>(ab + size_t(ts + min(row, nrows - 1)) * D + col));
        }
    }

    __device__ __forceinline__ void store(float* sL, int LL, int tid, int nrows) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = 4 * (idx % G);
            f32x4_t x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = row < nrows ? fast_log2(r[u][e]) : 0.0f;
            *reinterpret_cast<f32x4_t*>(sL + row * LL + col) = x;
        }
    }
};

// The chunk's decay prefix and what the kernels derive from it, formed by each wave for
// the columns of its quarter of D (so no barrier separates them from the prefix).  Lane
// (l16, s) takes column w D/4 + l16 (+ 16 k, k < D/64) over rows 16 s .. 16 s + 15, one
// 16-row block: it sums the staged log2 decays down its rows in registers, then adds the
// totals of the blocks above it (taken from the lanes that hold them), which gives L at
// each of its rows, the block's middle row m = 16 s + 7 and (lanes s = 3) L_last.
//   OUT (the output kernel): every row of phi(Q) and phi(K) is referred to the middle row
//   m(i) = 16 (i / 16) + 7 of its block,
//       Fq^_i = Fq_i 2^(L_i - L_m(i)),   Fk^_j = Fk_j 2^(L_m(j) - L_j)    (2^-64 .. 2^64 when a >= 2^-8),
//   in place, so that A_ij = Fq^_i . (Fk^_j * 2^(L_m(I) - L_m(J))) for J < I and
//   Fq^_i . Fk^_j on the diagonal block, both exponents of a product summing to L_i - L_j.
//   Otherwise (the totals kernel): the keys as seen from the chunk's end,
//   Fk~_j = Fk_j 2^(L_last - L_j), in place.
// The decays are no longer needed then, and rows 0..15 of sL take one factor each:
//     rows 0..3    2^(L_m(I))                   (the carried part's query factor, block I)
//     rows 4..7    2^(L_last - L_m(J))          (the state step's key factor, block J)
//     rows 8..13   2^(L_m(I) - L_m(J)), J < I   (row 8 + I (I - 1) / 2 + J: key block J against query block I)
//     row  14      2^(L_last)                   (the state's decay over the chunk)
//     row  15      L_last
// Lane (l16, s) writes rows 4 s .. 4 s + 3 of its column.
constexpr int kVdRowDecay = 14, kVdRowLast = 15;
__host__ __device__ constexpr int vd_pair_row(int I, int J) { return 8 + I * (I - 1) / 2 + J; }

template <typename E, int D, bool OUT>
__device__ __forceinline__ void vd_prefix(float* sL, int LL, E* sQ, E* sK, int LQ, int w, int lane) {
    using X = Elem<E>;
    constexpr int CPL = D / 64;
    static_assert(kBwdChunk == 64 && D % 64 == 0, "four 16-row blocks, 16 columns per lane group");
    const int s = lane >> 4, l16 = lane & 15;
    float L[CPL][16];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int col = w * (D / 4) + l16 + 16 * k;
        float run = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            run += sL[(16 * s + r) * LL + col];
            L[k][r] = run;
        }
    }
    float fac[CPL][4];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int col = w * (D / 4) + l16 + 16 * k;
        // the totals of the blocks above: lanes l16, l16 + 16, l16 + 32
        const float t0 = __shfl(L[k][15], l16, kWave), t1 = __shfl(L[k][15], l16 + 16, kWave),
                    t2 = __shfl(L[k][15], l16 + 32, kWave);
        const float off = (s > 0 ? t0 : 0.0f) + (s > 1 ? t1 : 0.0f) + (s > 2 ? t2 : 0.0f);
#pragma unroll
        for (int r = 0; r < 16; ++r) L[k][r] += off;
        const float mid = L[k][7];
        float m[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) m[b] = __shfl(mid, l16 + 16 * b, kWave);
        const float last = __shfl(L[k][15], l16 + 48, kWave);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 16 * s + r;
            E* pk = sK + row * LQ + col;
            if constexpr (OUT) {
                E* pq = sQ + row * LQ + col;
                *pq = X::from_f32(X::to_f32(*pq) * fast_exp2(L[k][r] - mid));
                *pk = X::from_f32(X::to_f32(*pk) * fast_exp2(mid - L[k][r]));
            } else {
                *pk = X::from_f32(X::to_f32(*pk) * fast_exp2(fminf(last - L[k][r], 0.0f)));
            }
        }
        // rows 4 s .. 4 s + 3 of the factor table
        float x[4];
        if (s == 0) {
#pragma unroll
            for (int b = 0; b < 4; ++b) x[b] = m[b];
        } else if (s == 1) {
#pragma unroll
            for (int b = 0; b < 4; ++b) x[b] = last - m[b];
        } else if (s == 2) {
            x[0] = m[1] - m[0];
            x[1] = m[2] - m[0];
            x[2] = m[2] - m[1];
            x[3] = m[3] - m[0];
        } else {
            x[0] = m[3] - m[1];
            x[1] = m[3] - m[2];
            x[2] = last;
            x[3] = last;
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) fac[k][b] = (s == 3 && b == 3) ? x[b] : fast_exp2(x[b]);
    }
    __builtin_amdgcn_wave_barrier();   // the wave's reads of its columns' decays come first
#pragma unroll
    for (int k = 0; k < CPL; ++k)
#pragma unroll
        for (int b = 0; b < 4; ++b) sL[(4 * s + b) * LL + w * (D / 4) + l16 + 16 * k] = fac[k][b];
}

// Accumulator-layout state pieces of this thread (tiles w + 4u, as in the gradients):
// loads and stores of a workspace slot, a caller-layout state, and the [D][Dv] staging.
template <typename E, int D, int DV>
struct VdState {
    using X = Elem<E>;
    static constexpr int SU = D * DV / 4 / kThreads, KZ = D / 64;
    static __device__ __forceinline__ void load_slot(f32x4_t (&r)[SU], const float* slot, int tid) {
#pragma unroll
        for (int u = 0; u < SU; ++u) r[u] = *reinterpret_cast<const f32x4_t*>(slot + 4 * (tid + u * kThreads));
    }
    static __device__ __forceinline__ void put_slot(float* slot, const f32x4_t (&r)[SU], int tid) {
#pragma unroll
        for (int u = 0; u < SU; ++u) *reinterpret_cast<f32x4_t*>(slot + 4 * (tid + u * kThreads)) = r[u];
    }
    static __device__ __forceinline__ void load_user(f32x4_t (&r)[SU], const float* S, int tid) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int q4 = tid + u * kThreads, t = q4 / kWave, ln = q4 % kWave;
            const int d = 16 * (t / (DV / 16)) + 4 * (ln >> 4), e = 16 * (t % (DV / 16)) + (ln & 15);
#pragma unroll
            for (int k = 0; k < 4; ++k) r[u][k] = S ? S[size_t(d + k) * DV + e] : 0.0f;
        }
    }
    static __device__ __forceinline__ void stage(E* sS, int LV, const f32x4_t (&r)[SU], int tid) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int q4 = tid + u * kThreads, t = q4 / kWave, ln = q4 % kWave;
            const int d = 16 * (t / (DV / 16)) + 4 * (ln >> 4), e = 16 * (t % (DV / 16)) + (ln & 15);
#pragma unroll
            for (int k = 0; k < 4; ++k) sS[(d + k) * LV + e] = X::from_f32(r[u][k]);
        }
    }
    // A [D] vector in the z-holder lanes (lane l16 = 0 of group g4 in wave w: entries
    // 16 (w + 4 t) + 4 g4 + r of tile t < KZ).
    static __device__ __forceinline__ void load_z(float (&z)[KZ][4], const float* src, int w, int l16, int g4) {
#pragma unroll
        for (int t = 0; t < KZ; ++t) {
            const f32x4_t v = (src && l16 == 0) ? *reinterpret_cast<const f32x4_t*>(src + 16 * (w + 4 * t) + 4 * g4)
                                                : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) z[t][r] = v[r];
        }
    }
    static __device__ __forceinline__ void put_z(float* dst, const float (&z)[KZ][4], int w, int l16, int g4) {
        if (l16 == 0) {
#pragma unroll
            for (int t = 0; t < KZ; ++t)
                *reinterpret_cast<f32x4_t*>(dst + 16 * (w + 4 * t) + 4 * g4) = f32x4_t{z[t][0], z[t][1], z[t][2], z[t][3]};
        }
    }
};

// One 16x16 state tile with the contraction over the chunk's rows: lhs^T rhs for rows a,
// columns b of two row-major tiles.
template <typename E>
__device__ __forceinline__ f32x4_t vd_tile_tn(const E* lhs, int ldl, int a, const E* rhs, int ldr, int b, int g4,
                                              int l16) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kBwdChunk / 32; ++ks)
        acc = mma(frag_col(lhs, ldl, 32 * ks + 8 * g4, 16 * a, l16), frag_col(rhs, ldr, 32 * ks + 8 * g4, 16 * b, l16),
                  acc);
    return acc;
}

// ------------------------------------------------------------ run totals ----

template <typename E, int D, int DV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(VdShape<E, D, DV>::kWaves,
                                                                           VdShape<E, D, DV>::kWaves)))
void vd_totals_kernel(VdArgs args) {
    using Sh = VdShape<E, D, DV>;
    using St = VdState<E, D, DV>;
    constexpr int C = Sh::C, LQ = Sh::LQ, LV = Sh::LV, LL = Sh::LL, SU = St::SU, KZ = St::KZ;
    constexpr int NB = DV / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    E* sK = reinterpret_cast<E*>(smem + Sh::kOffK);
    E* sV = reinterpret_cast<E*>(smem + Sh::kOffV);
    float* sL = reinterpret_cast<float*>(smem + Sh::kOffL);
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int N = args.N, NC = args.NC;
    const int run = blockIdx.x % args.NT, bh = blockIdx.x / args.NT;
    const int c_first = run * args.LC, c_end = min(NC, c_first + args.LC);

    // The run's total, T <- Diag(2^L_last) T + Fk~^T V chunk by chunk, its z part and the
    // summed L_last (z-holder lanes).
    f32x4_t T[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) T[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float tz[KZ][4] = {}, tl[KZ][4] = {};
    // the rows of a chunk; with Sh::kAhead the next chunk's are loaded into the same
    // registers as soon as this chunk's are in LDS, so they arrive during its products
    VdRows<E, D> rk;
    VdRows<E, DV> rv;
    VdDecays<D> ra;
    auto issue = [&](int cn) {
        const int tn = cn * C, nn = min(C, N - tn);
        rk.load(reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D, tid, tn, nn);
        rv.load(reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV, tid, tn, nn);
        ra.load(args.a + size_t(bh) * N * D, tid, tn, nn);
    };
    if (Sh::kAhead && c_first < c_end) issue(c_first);
    for (int c = c_first; c < c_end; ++c) {
        const int ts = c * C, nrows = min(C, N - ts);
        if (!Sh::kAhead) issue(c);
        ra.store(sL, LL, tid, nrows);
        rk.template store<true>(sK, LQ, tid, nrows);
        rv.template store<false>(sV, LV, tid, nrows);
        if (Sh::kAhead && c + 1 < c_end) issue(c + 1);
        // V's pad: a column of ones, so the z part comes out of the state product
        if (tid < C)
            *reinterpret_cast<f32x4_t*>(sV + tid * LV + DV) = split_pad<E>(tid < nrows ? 1.0f : 0.0f);
        __syncthreads();
        // L, the decayed keys Fk~ in place and the factor rows (vd_prefix)
        vd_prefix<E, D, false>(sL, LL, nullptr, sK, LQ, w, lane);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int t = w + 4 * u, a = t / NB, b = t % NB;
            const f32x4_t ds = vd_tile_tn(sK, LQ, a, sV, LV, b, g4, l16);
            const f32x4_t lf = *reinterpret_cast<const f32x4_t*>(sL + kVdRowDecay * LL + 16 * a + 4 * g4);
#pragma unroll
            for (int k = 0; k < 4; ++k) T[u][k] = lf[k] * T[u][k] + ds[k];
        }
#pragma unroll
        for (int t = 0; t < KZ; ++t) {
            const int a = w + 4 * t;
            const f32x4_t dz = vd_tile_tn(sK, LQ, a, sV, LV, NB, g4, l16);
            const f32x4_t lf = *reinterpret_cast<const f32x4_t*>(sL + kVdRowDecay * LL + 16 * a + 4 * g4);
            const f32x4_t ll = *reinterpret_cast<const f32x4_t*>(sL + kVdRowLast * LL + 16 * a + 4 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                tz[t][r] = lf[r] * tz[t][r] + pair01(dz[r]);
                tl[t][r] += ll[r];
            }
        }
        __syncthreads();              // every read of this chunk's tiles is done
    }
    const size_t slot = size_t(bh) * args.NR + run;
    St::put_slot(args.st + slot * (D * DV), T, tid);
    St::put_z(args.zt + slot * D, tz, w, l16, g4);
    St::put_z(args.lg + slot * D, tl, w, l16, g4);
}

// ------------------------------------------------------------------- scan ----

// In place over the first NC slots of each head's `stride_slots` (the run totals): slot c
// becomes the state after run c, S_c = 2^(L_last,c[d]) S_{c-1} + dS_c (rows d), starting
// from S0 / z0.
template <int D, int DV>
__global__ __launch_bounds__(kThreads) void vd_scan_kernel(float* st, float* zt, const float* lg, const float* s0,
                                                           const float* z0, int NC, int stride_slots) {
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
        base = st + size_t(bh) * stride_slots * NS + e;
        stride = NS;
        init = s0;
    } else {
        d = e - NS;
        uidx = size_t(bh) * D + d;
        base = zt + size_t(bh) * stride_slots * D + d;
        stride = D;
        init = z0;
    }
    const float* lgb = lg + size_t(bh) * stride_slots * D + d;
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
    using St = VdState<E, D, DV>;
    using X = Elem<E>;
    constexpr int C = Sh::C, LQ = Sh::LQ, LV = Sh::LV, LL = Sh::LL, SU = St::SU, KZ = St::KZ;
    constexpr int NE = DV / 16, NJ = C / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    E* sQ = reinterpret_cast<E*>(smem + Sh::kOffQ);
    E* sK = reinterpret_cast<E*>(smem + Sh::kOffK);
    E* sV = reinterpret_cast<E*>(smem + Sh::kOffV);
    E* sS = reinterpret_cast<E*>(smem + Sh::kOffS);
    float* sL = reinterpret_cast<float*>(smem + Sh::kOffL);
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int N = args.N, NC = args.NC;
    const int run = blockIdx.x % args.NR, bh = blockIdx.x / args.NR;
    const int c_first = run * args.LC, c_end = min(NC, c_first + args.LC);
    E* ob = reinterpret_cast<E*>(args.o) + size_t(bh) * N * DV;

    // The state in front of the current chunk, carried through the run in fp32: from the
    // scanned slot in front of the run, or S0 / z0.
    f32x4_t sacc[SU];
    float zv[KZ][4];
    if (run > 0) {
        const size_t slot = size_t(bh) * args.NR + (run - 1);
        St::load_slot(sacc, args.st + slot * (D * DV), tid);
        St::load_z(zv, args.zt + slot * D, w, l16, g4);
    } else {
        St::load_user(sacc, args.s0 ? args.s0 + size_t(bh) * D * DV : nullptr, tid);
        St::load_z(zv, args.z0 ? args.z0 + size_t(bh) * D : nullptr, w, l16, g4);
    }

    // the rows of a chunk; with Sh::kAheadOut the next chunk's are loaded into the same
    // registers as soon as this chunk's are in LDS
    VdRows<E, D> rq, rk;
    VdRows<E, DV> rv;
    VdDecays<D> ra;
    auto issue = [&](int cn) {
        const int tn = cn * C, nn = min(C, N - tn);
        rq.load(reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D, tid, tn, nn);
        rk.load(reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D, tid, tn, nn);
        rv.load(reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV, tid, tn, nn);
        ra.load(args.a + size_t(bh) * N * D, tid, tn, nn);
    };
    if (Sh::kAheadOut && c_first < c_end) issue(c_first);

    for (int c = c_first; c < c_end; ++c) {
    const int ts = c * C, nrows = min(C, N - ts);
    // staging: every load first
    {
        if (!Sh::kAheadOut) issue(c);
        St::stage(sS, LV, sacc, tid);
        if (l16 == 0) {
            // z_prev, split, into the state's pad columns: den's z part comes out of num
#pragma unroll
            for (int t = 0; t < KZ; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *reinterpret_cast<f32x4_t*>(sS + (16 * (w + 4 * t) + 4 * g4 + r) * LV + DV) = split_pad<E>(zv[t][r]);
        }
        ra.store(sL, LL, tid, nrows);
        rq.template store<true>(sQ, LQ, tid, nrows);
        rk.template store<true>(sK, LQ, tid, nrows);
        rv.template store<false>(sV, LV, tid, nrows);
        // V's pad: a column of ones, so the z step comes out of the state product
        if (tid < C)
            *reinterpret_cast<f32x4_t*>(sV + tid * LV + DV) = split_pad<E>(tid < nrows ? 1.0f : 0.0f);
        if (Sh::kAheadOut && c + 1 < c_end) issue(c + 1);
    }
    __syncthreads();
    vd_prefix<E, D, true>(sL, LL, sQ, sK, LQ, w, lane);
    __syncthreads();

    // This wave's query rows (block I = w); this lane's row of the transposed tiles.  The
    // rows of phi(Q) and phi(K) in LDS are referred to their blocks' middle rows and sL
    // holds the factor rows (vd_scan_rescale).
    const int i0 = 16 * w, il = i0 + l16;
    // num^T[e][i] = ((Fq * 2^L) S_prev)^T + (A V)^T, with an extra block of rows e = Dv,
    // Dv + 1: S's pad columns hold z_prev split and V's a column of ones, so they end as
    // den's two parts; Fq_i 2^L_i = Fq^_i 2^(L_m(I))
    f32x4_t nt[NE + 1];
#pragma unroll
    for (int et = 0; et <= NE; ++et) nt[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    F8<E> fqr[D / 32];                 // this lane's query row, rescaled, as the products' operand
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) fqr[ks] = frag_row(sQ, LQ, il, 32 * ks + 8 * g4);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        const int d0 = 32 * ks + 8 * g4;
        const F8<E>& fq = fqr[ks];
        const f32x4_t f0 = *reinterpret_cast<const f32x4_t*>(sL + w * LL + d0);
        const f32x4_t f1 = *reinterpret_cast<const f32x4_t*>(sL + w * LL + d0 + 4);
        F8<E> a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a.x[e] = X::from_f32(X::to_f32(fq.x[e]) * f0[e]);
            a.x[4 + e] = X::from_f32(X::to_f32(fq.x[4 + e]) * f1[e]);
        }
#pragma unroll
        for (int et = 0; et <= NE; ++et) nt[et] = mma(frag_col(sS, LV, d0, 16 * et, l16), a, nt[et]);
    }

    // A over the blocks J <= I, transposed: lane (l16, g4) holds query il against keys
    // 16 jt + 4 g4 + r, the operand layout of the 16x16x16 product with V.  Block J < I:
    // the keys carried from their block's middle row to the query block's (a factor of at
    // most 1: a distant key that underflows carries a weight below 2^-85 anyway); the
    // diagonal block takes the rescaled rows as they are.
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (jt < w) {
            const float* fr = sL + vd_pair_row(w, jt) * LL;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const int d0 = 32 * ks + 8 * g4;
                const F8<E> fk = frag_row(sK, LQ, 16 * jt + l16, d0);
                const f32x4_t f0 = *reinterpret_cast<const f32x4_t*>(fr + d0);
                const f32x4_t f1 = *reinterpret_cast<const f32x4_t*>(fr + d0 + 4);
                F8<E> kb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kb.x[e] = X::from_f32(X::to_f32(fk.x[e]) * f0[e]);
                    kb.x[4 + e] = X::from_f32(X::to_f32(fk.x[4 + e]) * f1[e]);
                }
                acc = mma(kb, fqr[ks], acc);
            }
        } else if (jt == w) {
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const int d0 = 32 * ks + 8 * g4;
                acc = mma(frag_row(sK, LQ, 16 * jt + l16, d0), fqr[ks], acc);
            }
        }
        if (jt <= w) {
            f32x4_t x;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = (16 * jt + 4 * g4 + r <= il) ? acc[r] : 0.0f;
            const F4<E> pa = pack4<E>(x);
#pragma unroll
            for (int et = 0; et <= NE; ++et)
                nt[et] = mma4(frag4_col(sV, LV, 16 * jt + 4 * g4, 16 * et, l16), pa, nt[et]);
        }
    }

    // o = num / max(den, eps) (or num): four consecutive columns of row il per lane; den
    // sits in lanes g4 = 0 (rows Dv and Dv + 1 of the extra block)
    {
        const float den = __shfl(nt[NE][0] + nt[NE][1], l16, kWave);
        const float inv = args.normalize ? 1.0f / fmaxf(den, args.eps) : 1.0f;
        if (ts + il < N) {
#pragma unroll
            for (int et = 0; et < NE; ++et) {
                f32x4_t o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = nt[et][r] * inv;
                store4<E>(ob + size_t(ts + il) * DV + 16 * et + 4 * g4, o);
            }
        }
    }
    // the state carried across the chunk: S <- Diag(2^L_last) S + Fk~^T V with
    // Fk~_j = Fk^_j 2^(L_last - L_m(J)), one 16-key block J at a time, its rows d scaled
    // in fp32; z alike (the extra column block: V's pad column of ones).  It reads only
    // tiles the outputs read, so no barrier separates the two.
    auto carried = [&](int a, int b) {
        f32x4_t ds = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J < NJ; ++J) {
            const f32x4_t t = mma4(frag4_col(sK, LQ, 16 * J + 4 * g4, 16 * a, l16),
                                   frag4_col(sV, LV, 16 * J + 4 * g4, 16 * b, l16), f32x4_t{0.f, 0.f, 0.f, 0.f});
            const f32x4_t u = *reinterpret_cast<const f32x4_t*>(sL + (4 + J) * LL + 16 * a + 4 * g4);
#pragma unroll
            for (int k = 0; k < 4; ++k) ds[k] += u[k] * t[k];
        }
        return ds;
    };
#pragma unroll
    for (int u = 0; u < SU; ++u) {
        const int t = w + 4 * u, a = t / NE, b = t % NE;
        const f32x4_t ds = carried(a, b);
        const f32x4_t lf = *reinterpret_cast<const f32x4_t*>(sL + kVdRowDecay * LL + 16 * a + 4 * g4);
#pragma unroll
        for (int k = 0; k < 4; ++k) sacc[u][k] = lf[k] * sacc[u][k] + ds[k];
    }
#pragma unroll
    for (int t = 0; t < KZ; ++t) {
        const int a = w + 4 * t;
        const f32x4_t dzt = carried(a, NE);
        const f32x4_t lf = *reinterpret_cast<const f32x4_t*>(sL + kVdRowDecay * LL + 16 * a + 4 * g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) zv[t][r] = lf[r] * zv[t][r] + pair01(dzt[r]);
    }
    __syncthreads();                  // every read of this chunk's tiles is done
    }
}

}  // namespace linattn
