// Chunked forward of causal kernelized linear attention for gfx950.
//
// The sequence of every (batch, head) is cut into segments of L chunks of CH
// tokens.  Three launches make one forward:
//
//   1. walk<TOTALS>  one workgroup per (head, segment): walks the segment's
//      chunks and accumulates the segment's own state total
//          T = sum_j w_j phi(k_j) v_j^T,  t = sum_j w_j phi(k_j)
//      (w_j = product of the gates after j inside the segment; 1 ungated) and,
//      gated, the log2 of the segment's total decay.  Reads K and V only.
//   2. scan          per (head, state element): exclusive prefix over segments,
//          P_0 = S0,  P_{s+1} = Gamma_s P_s + T_s,
//      in fp32, in place; writes S_N, z_N when asked.
//   3. walk<OUTPUT>  one workgroup per (head, segment): starts from P_s and walks
//      the segment's chunks carrying S and z in registers.  Per chunk it forms
//      the masked quadratic part on MFMA, adds the carried-state part, divides by
//      the clamped denominator, stores O, and folds the chunk into the state.
//
// This is the chunked parallel form of the aiwiki.thehackersbrain.dev page (the
// chunked listing: quadratic inside a chunk, recurrent across chunks, and the
// closing paragraph on the O(c^2) / O(d^2) balance), with the state pass split
// into segment totals plus a scan so every workgroup of the walk is independent.
//
// Chunk algebra for a chunk [s, s + CH) with Fq = phi(Q_c), Fk = phi(K_c):
//     A     = tril(Fq Fk^T)                  (diagonal kept)
//     num   = Fq S_prev + A V_c,   den = Fq z_prev + A 1,   O_c = num / max(den, eps)
//     S_next = S_prev + Fk^T V_c,  z_next = z_prev + Fk^T 1
// Gated (learn.pranaymahendrakar.com page, "Try it yourself": the weighted
// quadratic form), with the chunk-local inclusive Lambda_i = sum_{l=s..i} log2 g_l:
//     A_ij *= 2^(Lambda_i - Lambda_j),  the S_prev / z_prev terms of row i *= 2^Lambda_i,
//     S_next = 2^Lambda_last S_prev + sum_j 2^(Lambda_last - Lambda_j) Fk_j v_j^T  (z alike).
// Every decay factor is 2^(non-positive), so nothing overflows however long the
// sequence or small the gate.
//
// Tile mapping (16x16 MFMA tiles, four waves):
//   * transposed products: the kernel forms A^T = Fk Fq^T and O^T = V^T A^T + S^T Fq^T,
//     so the A^T accumulators of two 16-key tiles are directly the B operand of the
//     next product (the tiles' rows are ordered so lane group g holds keys 8g..8g+7
//     of the 32-key block, matching one 16-byte V^T read), and one lane owns one
//     query row of O^T, so the row sums and the divide stay in the lane.
//   * query strips of 16 rows are dealt to waves in pairs (w, 7-w) so every wave
//     gets the same number of causal tiles.
//   * the [D, Dv] state lives in MFMA accumulators (fp32) spread over the waves,
//     wave w owning the d-tiles [w D/64, (w+1) D/64) for every dv; z rides along as
//     one more tile per d-tile whose B operand is a column of ones, so Fk^T 1 costs
//     one MFMA per d-tile and no extra LDS traffic.  The operand copy S^T (input
//     precision) and z are re-staged in LDS once per chunk.
//   * loads are branch-free: rows past the end are clamped to the last row and their
//     features zeroed; the next chunk's K and V are in flight while this chunk's
//     products run, and its Q while this chunk's state is folded.
//
// LDS per workgroup: Fk [CH][D], Fk^T [D][CH], V^T [Dv][CH], S^T [Dv][D] in the
// input precision, rows padded by 16 bytes, plus z [D] and Lambda [CH] in fp32.
#pragma once

#include "device_common.hpp"

// Register sets for K and V: 2 loads the next chunk at the top of each chunk, 1 loads
// it right after the current chunk is staged (fewer registers, shorter overlap).
#ifndef LINATTN_KV_SETS
#define LINATTN_KV_SETS 1
#endif

namespace linattn {

struct WalkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;      // gated only
    void* o;             // OUTPUT only
    float* st;           // [BH][nseg][D*Dv] state totals/prefixes, accumulator layout
    float* zt;           // [BH][nseg][D]
    float* lg;           // [BH][nseg] log2 of each segment's total decay (gated)
    int N;
    int nseg;            // segments per sequence
    int L;               // chunks per segment
    float eps;
};

template <typename E, int D, int DV, int CH>
struct WalkShape {
    static_assert(CH >= 32 && CH <= 256 && (CH & (CH - 1)) == 0, "chunk must be a power of two in [32, 256]");
    static constexpr int PE = 16 / int(sizeof(E));   // 16-byte row padding, in elements
    static constexpr int LK = D + PE;                 // row stride of Fk   [CH][D]
    static constexpr int LKT = CH + PE;               // row stride of Fk^T [D][CH] and V^T [Dv][CH]
    static constexpr int LS = D + PE;                 // row stride of S^T  [Dv][D]
    static constexpr int NSTRIP = CH / 16;
    static constexpr int MAXS = (NSTRIP + 3) / 4;     // query strips per wave
    static constexpr int NKU = (CH / 4) * (D / 8);    // staging units of K (4 rows x 8 columns)
    static constexpr int NVU = (CH / 4) * (DV / 8);
    static constexpr int KPT = (NKU + kThreads - 1) / kThreads;
    static constexpr int VPT = (NVU + kThreads - 1) / kThreads;
    static constexpr int NA = D / 16, NB = DV / 16;
    static constexpr int ZT = NA / 4;                 // d-tiles owned by each wave
    static constexpr int TPW = ZT * NB;               // state tiles per wave
    static constexpr int GPT = (CH + kWave - 1) / kWave;   // gate values per lane of wave 0

    static constexpr size_t bytes(bool output) {
        return (output ? size_t(CH) * LK * sizeof(E) : 0) + size_t(D) * LKT * sizeof(E) +
               size_t(DV) * LKT * sizeof(E) + (output ? size_t(DV) * LS * sizeof(E) : 0) +
               size_t(D) * 4 + size_t(CH) * 4;
    }
};

// Query strip handled by wave w in its m-th slot, or -1.
template <int NSTRIP>
__device__ __forceinline__ int strip_of(int w, int m) {
    const int pair = m >> 1;
    const int s = (m & 1) ? (pair * 8 + 7 - w) : (pair * 8 + w);
    return s < NSTRIP ? s : -1;
}

// The per-thread machinery of one workgroup walking chunks of one head.
// ROWK: also stage the row-major Fk (needed only when outputs are formed).
template <typename E, int D, int DV, int CH, bool GATED, bool ROWK>
struct ChunkWalker {
    using Sh = WalkShape<E, D, DV, CH>;
    using X = Elem<E>;
    static constexpr int LK = Sh::LK, LKT = Sh::LKT, LS = Sh::LS;

    struct Regs {                       // one chunk of K, V (and gates) in flight
        F8<E> rk[Sh::KPT][4];
        F8<E> rv[Sh::VPT][4];
        float rg[Sh::GPT];
    };
    struct QRegs {                      // this wave's query rows of one chunk
        F8<E> rq[Sh::MAXS][D / 32];
    };

    E* sK;
    E* sKt;
    E* sVt;
    E* sSt;
    float* sZ;
    float* sLam;
    int tid, w, lane, l16, g4;
    int N;
    const E* qb;
    const E* kb;
    const E* vb;
    const float* gb;

    // Fk^T and V^T rows are [CH] keys stored as 16-byte groups of 8 keys; group j of
    // row r sits at slot j ^ ((r / 8) mod (CH / 8)).  The transposed writes of a wave
    // (8 rows x 8 key quads) then spread over all banks, and the MFMA operand reads
    // (16 consecutive rows, one group) stay conflict-free.
    static __device__ __forceinline__ int tidx(int row, int group) {
        return row * LKT + ((group ^ ((row >> 3) & (CH / 8 - 1))) << 3);
    }
    // Fk rows are [D] features in 8-element groups; rows 8..15 of every 16 flip bit 2
    // of the group index, so the operand read of keys {0-3, 8-11, ...} is conflict-free.
    static __device__ __forceinline__ int kidx(int row, int group) {
        return row * LK + ((group ^ (((row >> 3) & 1) << 2)) << 3);
    }

    __device__ __forceinline__ void init(unsigned char* smem, int N_, const E* q, const E* k, const E* v,
                                         const float* g) {
        sK = reinterpret_cast<E*>(smem);
        sKt = sK + (ROWK ? CH * LK : 0);
        sVt = sKt + D * LKT;
        sSt = sVt + DV * LKT;
        sZ = reinterpret_cast<float*>(sSt + (ROWK ? DV * LS : 0));
        sLam = sZ + D;
        tid = threadIdx.x;
        w = tid / kWave;
        lane = tid % kWave;
        l16 = lane & 15;
        g4 = lane >> 4;
        N = N_;
        qb = q;
        kb = k;
        vb = v;
        gb = g;
    }

    // Global -> registers for the chunk starting at token ts.  Rows past N are
    // clamped to N-1 (always in bounds); stage() zeroes their features.
    __device__ __forceinline__ void load(Regs& R, int ts) const {
        const int last = N - 1;
#pragma unroll
        for (int it = 0; it < Sh::KPT; ++it) {
            const int u = tid + it * kThreads;
            const int cg = u % (D / 8), kq = (u / (D / 8)) % (CH / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = min(ts + 4 * kq + r, last);
                R.rk[it][r] = *reinterpret_cast<const F8<E>*>(kb + size_t(row) * D + 8 * cg);
            }
        }
#pragma unroll
        for (int it = 0; it < Sh::VPT; ++it) {
            const int u = tid + it * kThreads;
            const int cg = u % (DV / 8), kq = (u / (DV / 8)) % (CH / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = min(ts + 4 * kq + r, last);
                R.rv[it][r] = *reinterpret_cast<const F8<E>*>(vb + size_t(row) * DV + 8 * cg);
            }
        }
        if constexpr (GATED) {
            if (w == 0) {
#pragma unroll
                for (int i = 0; i < Sh::GPT; ++i) {
                    const int j = lane * Sh::GPT + i;
                    const float gv = gb[min(ts + j, last)];
                    R.rg[i] = (j < CH && ts + j < N) ? gv : 1.0f;
                }
            }
        }
    }

    __device__ __forceinline__ void load_q(QRegs& Q, int ts) const {
        const int last = N - 1;
#pragma unroll
        for (int m = 0; m < Sh::MAXS; ++m) {
            const int s = max(strip_of<Sh::NSTRIP>(w, m), 0);
            const int row = min(ts + 16 * s + l16, last);
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                Q.rq[m][ks] = *reinterpret_cast<const F8<E>*>(qb + size_t(row) * D + 32 * ks + 8 * g4);
        }
    }

    // Wave 0: Lambda_j = inclusive sum of log2 g over the chunk, into sLam.
    __device__ __forceinline__ void lambda(const Regs& R) const {
        if (w != 0) return;
        float loc[Sh::GPT];
        float run = 0.0f;
#pragma unroll
        for (int i = 0; i < Sh::GPT; ++i) {
            run += fast_log2(R.rg[i]);
            loc[i] = run;
        }
        float incl = run;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float y = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += y;
        }
        const float excl = incl - run;
#pragma unroll
        for (int i = 0; i < Sh::GPT; ++i) {
            const int j = lane * Sh::GPT + i;
            if (j < CH) sLam[j] = excl + loc[i];
        }
    }

    // phi(K) -> Fk (row-major, if WITHK) and Fk^T (decayed when gated); V -> V^T.
    template <bool WITHK = ROWK>
    __device__ __forceinline__ void stage(const Regs& R, int ts, float lam_last) const {
#pragma unroll
        for (int it = 0; it < Sh::KPT; ++it) {
            const int u = tid + it * kThreads;
            if (u < Sh::NKU) {
                const int cg = u % (D / 8), kq = u / (D / 8);
                E fr[4][8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float mk = (ts + 4 * kq + r < N) ? 1.0f : 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) fr[r][e] = X::from_f32(phi(X::to_f32(R.rk[it][r].x[e])) * mk);
                    if constexpr (WITHK) {
                        F8<E> t;
#pragma unroll
                        for (int e = 0; e < 8; ++e) t.x[e] = fr[r][e];
                        *reinterpret_cast<F8<E>*>(sK + kidx(4 * kq + r, cg)) = t;
                    }
                }
                float dec[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dec[r] = GATED ? fast_exp2(fminf(lam_last - sLam[4 * kq + r], 0.0f)) : 1.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    F4<E> t;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        t.x[r] = GATED ? X::from_f32(X::to_f32(fr[r][e]) * dec[r]) : fr[r][e];
                    *reinterpret_cast<F4<E>*>(sKt + tidx(8 * cg + e, kq >> 1) + 4 * (kq & 1)) = t;
                }
            }
        }
#pragma unroll
        for (int it = 0; it < Sh::VPT; ++it) {
            const int u = tid + it * kThreads;
            if (u < Sh::NVU) {
                const int cg = u % (DV / 8), kq = u / (DV / 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    F4<E> t;
#pragma unroll
                    for (int r = 0; r < 4; ++r) t.x[r] = R.rv[it][r].x[e];
                    *reinterpret_cast<F4<E>*>(sVt + tidx(8 * cg + e, kq >> 1) + 4 * (kq & 1)) = t;
                }
            }
        }
    }

    __device__ __forceinline__ void phi_q(const QRegs& Q, F8<E> (&fq)[Sh::MAXS][D / 32]) const {
#pragma unroll
        for (int m = 0; m < Sh::MAXS; ++m)
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) fq[m][ks].x[e] = X::from_f32(phi(X::to_f32(Q.rq[m][ks].x[e])));
    }

    // S^T (operand precision) and z into LDS for the carried-state part.
    __device__ __forceinline__ void stage_state(const f32x4_t (&sacc)[Sh::TPW], const f32x4_t (&zacc)[Sh::ZT]) const {
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i) {
            const int a = w * Sh::ZT + i;
#pragma unroll
            for (int b = 0; b < Sh::NB; ++b) {
                F4<E> t;
#pragma unroll
                for (int r = 0; r < 4; ++r) t.x[r] = X::from_f32(sacc[i * Sh::NB + b][r]);
                *reinterpret_cast<F4<E>*>(sSt + (16 * b + l16) * LS + 16 * a + 4 * g4) = t;
            }
            if (l16 == 0) *reinterpret_cast<f32x4_t*>(sZ + 16 * a + 4 * g4) = zacc[i];
        }
    }

    // State fold: S = 2^lam_last S + Fk^T V (Fk^T already decayed), z alike.
    __device__ __forceinline__ void fold(f32x4_t (&sacc)[Sh::TPW], f32x4_t (&zacc)[Sh::ZT], float lam_last) const {
        if constexpr (GATED) {
            const float dl = fast_exp2(lam_last);
#pragma unroll
            for (int j = 0; j < Sh::TPW; ++j) sacc[j] *= dl;
#pragma unroll
            for (int i = 0; i < Sh::ZT; ++i) zacc[i] *= dl;
        }
        F8<E> ones;
#pragma unroll
        for (int e = 0; e < 8; ++e) ones.x[e] = X::from_f32(l16 == 0 ? 1.0f : 0.0f);
#pragma unroll
        for (int kbk = 0; kbk < CH / 32; ++kbk) {
            F8<E> vf[Sh::NB];
#pragma unroll
            for (int b = 0; b < Sh::NB; ++b) vf[b] = lds_f8(sVt + tidx(16 * b + l16, 4 * kbk + g4));
#pragma unroll
            for (int i = 0; i < Sh::ZT; ++i) {
                const int a = w * Sh::ZT + i;
                const F8<E> ka = lds_f8(sKt + tidx(16 * a + l16, 4 * kbk + g4));
#pragma unroll
                for (int b = 0; b < Sh::NB; ++b) sacc[i * Sh::NB + b] = mma(ka, vf[b], sacc[i * Sh::NB + b]);
                zacc[i] = mma(ka, ones, zacc[i]);
            }
        }
    }

    // Walk chunks c0 .. c0+nch-1 of the head, folding each into (sacc, zacc); with OUT
    // also form and store the outputs (S^T and z must then already be staged in LDS).
    // K and V of the next chunk are loaded right after this chunk is staged (or, with
    // two register sets, at the top of the chunk); Q of the next chunk is loaded once
    // this chunk's outputs no longer need the single Q set.  The last chunk's fold is
    // skipped when FOLD_LAST is false.
    template <bool OUT, bool FOLD_LAST>
    __device__ __forceinline__ void walk(int c0, int nch, f32x4_t (&sacc)[Sh::TPW], f32x4_t (&zacc)[Sh::ZT],
                                         float& lg_total, E* ob, float eps) const {
        constexpr bool kTwo = LINATTN_KV_SETS == 2;
        Regs ra, rb_store;
        Regs& rb = kTwo ? rb_store : ra;
        QRegs qr;
        auto step = [&](Regs& cur, Regs& nxt, int n) {
            const int ts = (c0 + n) * CH;
            const bool more = n + 1 < nch;
            if (kTwo && more) load(nxt, ts + CH);
            if constexpr (GATED) {
                lambda(cur);
                __syncthreads();
            }
            const float lam_last = GATED ? sLam[CH - 1] : 0.0f;
            stage<OUT>(cur, ts, lam_last);
            F8<E> fq[Sh::MAXS][D / 32];
            if constexpr (OUT) phi_q(qr, fq);
            if (!kTwo && more) load(nxt, ts + CH);
            __syncthreads();
            if constexpr (OUT) {
                outputs(fq, ts, ob, eps);
                if (more) load_q(qr, ts + CH);
            }
            if (FOLD_LAST || more) fold(sacc, zacc, lam_last);
            lg_total += lam_last;
            __syncthreads();
            if (OUT && more) stage_state(sacc, zacc);
        };
        if (nch <= 0) return;
        load(ra, c0 * CH);
        if constexpr (OUT) load_q(qr, c0 * CH);
        for (int n = 0; n < nch; n += 2) {
            step(ra, rb, n);
            if (n + 1 < nch) step(rb, ra, n + 1);
        }
    }

    // Outputs of the chunk starting at ts for this wave's query strips.
    __device__ __forceinline__ void outputs(const F8<E> (&fq)[Sh::MAXS][D / 32], int ts, E* ob, float eps) const {
#pragma unroll
        for (int m = 0; m < Sh::MAXS; ++m) {
            const int s = strip_of<Sh::NSTRIP>(w, m);
            if (s < 0) continue;
            const int qi = 16 * s + l16;               // query row of this lane within the chunk
            f32x4_t acc[DV / 16];
#pragma unroll
            for (int t = 0; t < DV / 16; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // carried-state part: O^T += S^T Fq^T ; den += Fq . z
            float den = 0.0f;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
                for (int t = 0; t < DV / 16; ++t)
                    acc[t] = mma(lds_f8(sSt + (16 * t + l16) * LS + 32 * ks + 8 * g4), fq[m][ks], acc[t]);
                const f32x4_t z0 = *reinterpret_cast<const f32x4_t*>(sZ + 32 * ks + 8 * g4);
                const f32x4_t z1 = *reinterpret_cast<const f32x4_t*>(sZ + 32 * ks + 8 * g4 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    den += X::to_f32(fq[m][ks].x[e]) * z0[e];
                    den += X::to_f32(fq[m][ks].x[4 + e]) * z1[e];
                }
            }
            float lam_q = 0.0f;
            if constexpr (GATED) {
                lam_q = sLam[qi];
                const float sc = fast_exp2(lam_q);
#pragma unroll
                for (int t = 0; t < DV / 16; ++t) acc[t] *= sc;
                den *= sc;
            }
            // causal part: key blocks of 32 up to the diagonal.  Row m of the first A^T
            // tile is key 8(m/4) + m%4 of the block and row m of the second is that key
            // + 4, so lane group g holds keys 8g..8g+7 of the block: a B operand of
            // consecutive keys, matched by one 16-byte V^T read.
            const int npairs = s / 2 + 1;
            const int krow = 8 * (l16 >> 2) + (l16 & 3);
            for (int p = 0; p < npairs; ++p) {
                f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    a0 = mma(lds_f8(sK + kidx(32 * p + krow, 4 * ks + g4)), fq[m][ks], a0);
                    a1 = mma(lds_f8(sK + kidx(32 * p + krow + 4, 4 * ks + g4)), fq[m][ks], a1);
                }
                F8<E> bA;
                float rs = 0.0f;
                f32x4_t l0 = {0.f, 0.f, 0.f, 0.f}, l1 = {0.f, 0.f, 0.f, 0.f};
                if constexpr (GATED) {
                    l0 = *reinterpret_cast<const f32x4_t*>(sLam + 32 * p + 8 * g4);
                    l1 = *reinterpret_cast<const f32x4_t*>(sLam + 32 * p + 8 * g4 + 4);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int k0 = 32 * p + 8 * g4 + r, k1 = k0 + 4;
                    float x0 = a0[r], x1 = a1[r];
                    if constexpr (GATED) {
                        x0 *= fast_exp2(fminf(lam_q - l0[r], 0.0f));
                        x1 *= fast_exp2(fminf(lam_q - l1[r], 0.0f));
                    }
                    x0 = k0 <= qi ? x0 : 0.0f;
                    x1 = k1 <= qi ? x1 : 0.0f;
                    const E e0 = X::from_f32(x0), e1 = X::from_f32(x1);
                    bA.x[r] = e0;
                    bA.x[4 + r] = e1;
                    rs += X::to_f32(e0) + X::to_f32(e1);
                }
                den += rs;
#pragma unroll
                for (int t = 0; t < DV / 16; ++t)
                    acc[t] = mma(lds_f8(sVt + tidx(16 * t + l16, 4 * p + g4)), bA, acc[t]);
            }
            den += __shfl_xor(den, 16, kWave);
            den += __shfl_xor(den, 32, kWave);
            const float inv = 1.0f / fmaxf(den, eps);
            const int row = ts + qi;
            if (row < N) {
#pragma unroll
                for (int t = 0; t < DV / 16; ++t) {
                    F4<E> outv;
#pragma unroll
                    for (int r = 0; r < 4; ++r) outv.x[r] = X::from_f32(acc[t][r] * inv);
                    *reinterpret_cast<F4<E>*>(ob + size_t(row) * DV + 16 * t + 4 * g4) = outv;
                }
            }
        }
    }
};

template <typename E, int D, int DV, int CH, bool GATED, bool OUTPUT>
__global__ __launch_bounds__(kThreads) void walk_kernel(WalkArgs args) {
    using Sh = WalkShape<E, D, DV, CH>;
    using W = ChunkWalker<E, D, DV, CH, GATED, OUTPUT>;
    extern __shared__ __align__(16) unsigned char smem[];

    const int seg = blockIdx.x % args.nseg;
    const int bh = blockIdx.x / args.nseg;
    const int N = args.N;
    const int nchunks_total = (N + CH - 1) / CH;
    const int c0 = seg * args.L;
    const int nch = min(args.L, nchunks_total - c0);

    W wk;
    wk.init(smem, N, reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D,
            reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D,
            reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV, GATED ? args.g + size_t(bh) * N : nullptr);
    E* ob = OUTPUT ? reinterpret_cast<E*>(args.o) + size_t(bh) * N * DV : nullptr;
    float* stp = args.st + (size_t(bh) * args.nseg + seg) * (D * DV);
    float* ztp = args.zt + (size_t(bh) * args.nseg + seg) * D;

    // persistent state in accumulator tiles
    f32x4_t sacc[Sh::TPW];
    f32x4_t zacc[Sh::ZT];
    if (OUTPUT) {
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j)
            sacc[j] = *reinterpret_cast<const f32x4_t*>(stp + ((wk.w * Sh::TPW + j) * kWave + wk.lane) * 4);
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i) {
            const f32x4_t zv = *reinterpret_cast<const f32x4_t*>(ztp + 16 * (wk.w * Sh::ZT + i) + 4 * wk.g4);
            zacc[i] = wk.l16 == 0 ? zv : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        wk.stage_state(sacc, zacc);
    } else {
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j) sacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i) zacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    float lg_total = 0.0f;

    wk.template walk<OUTPUT, !OUTPUT>(c0, nch, sacc, zacc, lg_total, ob, args.eps);

    if (!OUTPUT) {
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j)
            *reinterpret_cast<f32x4_t*>(stp + ((wk.w * Sh::TPW + j) * kWave + wk.lane) * 4) = sacc[j];
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i)
            if (wk.l16 == 0) *reinterpret_cast<f32x4_t*>(ztp + 16 * (wk.w * Sh::ZT + i) + 4 * wk.g4) = zacc[i];
        if (GATED && wk.tid == 0) args.lg[size_t(bh) * args.nseg + seg] = lg_total;
    }
}

// Exclusive prefix of segment totals, in place, one thread per state element.
// Element e < D*Dv is in accumulator layout: tile u = e / 256 (a = u / (Dv/16),
// b = u % (Dv/16)), lane = (e / 4) % 64, r = e % 4, which is S[16a + 4(lane/16) + r][16b + lane%16].
template <int D, int DV, bool GATED>
__global__ __launch_bounds__(kThreads) void scan_kernel(float* st, float* zt, const float* lg, const float* s0,
                                                       const float* z0, float* s_out, float* z_out, int nseg) {
    constexpr int NS = D * DV;
    constexpr int NBLK = (NS + D + kThreads - 1) / kThreads;   // workgroups per head
    const int e = (blockIdx.x % NBLK) * kThreads + threadIdx.x;
    const int bh = blockIdx.x / NBLK;
    if (e >= NS + D) return;
    float* base;
    size_t stride;
    size_t uidx;      // index into the caller's [D][Dv] or [D] layout
    const float* init;
    float* fin;
    if (e < NS) {
        const int u = e / 256, lane = (e / 4) % 64, r = e % 4;
        const int a = u / (DV / 16), b = u % (DV / 16);
        const int d = 16 * a + 4 * (lane / 16) + r, dv = 16 * b + lane % 16;
        uidx = size_t(bh) * NS + size_t(d) * DV + dv;
        base = st + size_t(bh) * nseg * NS + e;
        stride = NS;
        init = s0;
        fin = s_out;
    } else {
        const int d = e - NS;
        uidx = size_t(bh) * D + d;
        base = zt + size_t(bh) * nseg * D + d;
        stride = D;
        init = z0;
        fin = z_out;
    }
    const float* lgb = GATED ? lg + size_t(bh) * nseg : nullptr;
    float acc = init ? init[uidx] : 0.0f;
    constexpr int U = 8;                         // loads in flight per thread
    for (int s0i = 0; s0i < nseg; s0i += U) {
        float t[U], f[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int s = min(s0i + i, nseg - 1);
            t[i] = base[size_t(s) * stride];
            f[i] = GATED ? fast_exp2(lgb[s]) : 1.0f;
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (s0i + i < nseg) {
                base[size_t(s0i + i) * stride] = acc;
                acc = f[i] * acc + t[i];
            }
        }
    }
    if (fin) fin[uidx] = acc;
}

}  // namespace linattn
