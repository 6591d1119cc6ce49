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
//     so the A^T accumulator of two 16-key tiles is directly the B operand of the
//     next product (its 8 contraction slots hold keys {4g..4g+3, 16+4g..16+4g+3}
//     of lane group g; V^T is read with the same key order), and one lane owns one
//     query row of O^T, so the row sums and the divide stay in the lane.
//   * query strips of 16 rows are dealt to waves in pairs (w, 7-w) so every wave
//     gets the same number of causal tiles.
//   * the [D, Dv] state lives in MFMA accumulators (fp32) spread over the waves;
//     its operand copy S^T (input precision) is re-staged in LDS once per chunk.
//
// LDS per workgroup: Fk [CH][D], Fk^T [D][CH], V^T [Dv][CH], S^T [Dv][D] in the
// input precision, rows padded by 16 bytes, plus z [D] and Lambda [CH] in fp32.
#pragma once

#include "device_common.hpp"

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
    static constexpr int TPW = NA * NB / 4;           // state tiles per wave
    static constexpr int TPD = kThreads / D;          // threads per z entry
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

template <typename E, int D, int DV, int CH, bool GATED, bool OUTPUT>
__global__ __launch_bounds__(kThreads) void walk_kernel(WalkArgs args) {
    using Sh = WalkShape<E, D, DV, CH>;
    using X = Elem<E>;
    constexpr int LK = Sh::LK, LKT = Sh::LKT, LS = Sh::LS;

    extern __shared__ __align__(16) unsigned char smem[];
    E* sK = reinterpret_cast<E*>(smem);
    E* sKt = sK + (OUTPUT ? CH * LK : 0);
    E* sVt = sKt + D * LKT;
    E* sSt = sVt + DV * LKT;
    float* sZ = reinterpret_cast<float*>(sSt + (OUTPUT ? DV * LS : 0));
    float* sLam = sZ + D;

    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid % kWave;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;

    const int seg = blockIdx.x % args.nseg;
    const int bh = blockIdx.x / args.nseg;
    const int N = args.N;
    const int nchunks_total = (N + CH - 1) / CH;
    const int c0 = seg * args.L;
    const int nch = min(args.L, nchunks_total - c0);

    const E* qb = reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D;
    const E* kb = reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D;
    const E* vb = reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV;
    const float* gb = GATED ? args.g + size_t(bh) * N : nullptr;
    E* ob = OUTPUT ? reinterpret_cast<E*>(args.o) + size_t(bh) * N * DV : nullptr;
    float* stp = args.st + (size_t(bh) * args.nseg + seg) * (D * DV);
    float* ztp = args.zt + (size_t(bh) * args.nseg + seg) * D;

    // ---- persistent state: S in accumulator tiles, z in registers ------------
    f32x4_t sacc[Sh::TPW];
    const int zd = tid / Sh::TPD;      // z entry owned (with TPD-1 neighbours)
    const int zsub = tid % Sh::TPD;
    float zr;
    float lg_total = 0.0f;
    if (OUTPUT) {
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j)
            sacc[j] = *reinterpret_cast<const f32x4_t*>(stp + ((w * Sh::TPW + j) * kWave + lane) * 4);
        zr = ztp[zd];
    } else {
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j) sacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        zr = 0.0f;
    }

    // S^T (operand precision) and z go to LDS for the first chunk's carried-state part.
    auto stage_state = [&]() {
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j) {
            const int u = w * Sh::TPW + j;
            const int a = u / Sh::NB, b = u % Sh::NB;
            F4<E> t;
#pragma unroll
            for (int r = 0; r < 4; ++r) t.x[r] = X::from_f32(sacc[j][r]);
            *reinterpret_cast<F4<E>*>(sSt + (16 * b + l16) * LS + 16 * a + 4 * g4) = t;
        }
        if (zsub == 0) sZ[zd] = zr;
    };
    if (OUTPUT) stage_state();

    // ---- register staging of one chunk --------------------------------------
    F8<E> rk[Sh::KPT][4];
    F8<E> rv[Sh::VPT][4];
    F8<E> rq[Sh::MAXS][D / 32];
    float rg[Sh::GPT];

    auto load_chunk = [&](int n) {
        const int ts = (c0 + n) * CH;
#pragma unroll
        for (int it = 0; it < Sh::KPT; ++it) {
            const int u = tid + it * kThreads;
            const int cg = u % (D / 8), kq = u / (D / 8);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = ts + 4 * kq + r;
                rk[it][r] = (u < Sh::NKU && row < N)
                                ? *reinterpret_cast<const F8<E>*>(kb + size_t(row) * D + 8 * cg)
                                : zero8<E>();
            }
        }
#pragma unroll
        for (int it = 0; it < Sh::VPT; ++it) {
            const int u = tid + it * kThreads;
            const int cg = u % (DV / 8), kq = u / (DV / 8);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = ts + 4 * kq + r;
                rv[it][r] = (u < Sh::NVU && row < N)
                                ? *reinterpret_cast<const F8<E>*>(vb + size_t(row) * DV + 8 * cg)
                                : zero8<E>();
            }
        }
        if (OUTPUT) {
#pragma unroll
            for (int m = 0; m < Sh::MAXS; ++m) {
                const int s = strip_of<Sh::NSTRIP>(w, m);
                const int row = ts + 16 * s + l16;
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    rq[m][ks] = (s >= 0 && row < N)
                                    ? *reinterpret_cast<const F8<E>*>(qb + size_t(row) * D + 32 * ks + 8 * g4)
                                    : zero8<E>();
                }
            }
        }
        if (GATED && w == 0) {
#pragma unroll
            for (int i = 0; i < Sh::GPT; ++i) {
                const int j = lane * Sh::GPT + i;
                const int row = ts + j;
                rg[i] = (j < CH && row < N) ? gb[row] : 1.0f;
            }
        }
    };

    if (nch > 0) load_chunk(0);

    for (int n = 0; n < nch; ++n) {
        const int ts = (c0 + n) * CH;

        // ---- Lambda: chunk-local inclusive cumulative log2 gate (wave 0) -------
        if (GATED) {
            if (w == 0) {
                float loc[Sh::GPT];
                float run = 0.0f;
#pragma unroll
                for (int i = 0; i < Sh::GPT; ++i) { run += fast_log2(rg[i]); loc[i] = run; }
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
            __syncthreads();
        }
        const float lam_last = GATED ? sLam[CH - 1] : 0.0f;

        // ---- stage phi(K), phi(K)^T (decayed when gated) and V^T into LDS ------
#pragma unroll
        for (int it = 0; it < Sh::KPT; ++it) {
            const int u = tid + it * kThreads;
            if (u < Sh::NKU) {
                const int cg = u % (D / 8), kq = u / (D / 8);
                float f[4][8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool valid = ts + 4 * kq + r < N;
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[r][e] = valid ? phi(X::to_f32(rk[it][r].x[e])) : 0.0f;
                    if (OUTPUT) {
                        F8<E> t;
#pragma unroll
                        for (int e = 0; e < 8; ++e) t.x[e] = X::from_f32(f[r][e]);
                        *reinterpret_cast<F8<E>*>(sK + (4 * kq + r) * LK + 8 * cg) = t;
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
                    for (int r = 0; r < 4; ++r) {
                        // the decayed copy is rounded from the rounded feature, so the
                        // ungated path stores exactly the values of Fk
                        const float fr = X::to_f32(X::from_f32(f[r][e]));
                        t.x[r] = X::from_f32(GATED ? fr * dec[r] : fr);
                    }
                    *reinterpret_cast<F4<E>*>(sKt + (8 * cg + e) * LKT + 4 * kq) = t;
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
                    for (int r = 0; r < 4; ++r) t.x[r] = rv[it][r].x[e];
                    *reinterpret_cast<F4<E>*>(sVt + (8 * cg + e) * LKT + 4 * kq) = t;
                }
            }
        }
        F8<E> fq[Sh::MAXS][D / 32];
        if (OUTPUT) {
#pragma unroll
            for (int m = 0; m < Sh::MAXS; ++m)
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) fq[m][ks].x[e] = X::from_f32(phi(X::to_f32(rq[m][ks].x[e])));
        }
        if (n + 1 < nch) load_chunk(n + 1);     // next chunk's loads overlap this chunk's math
        __syncthreads();

        // ---- outputs of this chunk -------------------------------------------
        if (OUTPUT) {
#pragma unroll
            for (int m = 0; m < Sh::MAXS; ++m) {
                const int s = strip_of<Sh::NSTRIP>(w, m);
                if (s < 0) continue;
                const int qi = 16 * s + l16;               // query row of this lane
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
#pragma unroll
                    for (int e = 0; e < 8; ++e) den += X::to_f32(fq[m][ks].x[e]) * sZ[32 * ks + 8 * g4 + e];
                }
                float lam_q = 0.0f;
                if (GATED) {
                    lam_q = sLam[qi];
                    const float sc = fast_exp2(lam_q);
#pragma unroll
                    for (int t = 0; t < DV / 16; ++t) acc[t] *= sc;
                    den *= sc;
                }
                // causal part: key pairs of 32 up to the diagonal
                const int npairs = s / 2 + 1;
                for (int p = 0; p < npairs; ++p) {
                    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < D / 32; ++ks) {
                        a0 = mma(lds_f8(sK + (32 * p + l16) * LK + 32 * ks + 8 * g4), fq[m][ks], a0);
                        a1 = mma(lds_f8(sK + (32 * p + 16 + l16) * LK + 32 * ks + 8 * g4), fq[m][ks], a1);
                    }
                    F8<E> bA;
                    float rs = 0.0f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int k0 = 32 * p + 4 * g4 + r, k1 = k0 + 16;
                        float x0 = a0[r], x1 = a1[r];
                        if (GATED) {
                            x0 *= fast_exp2(fminf(lam_q - sLam[k0], 0.0f));
                            x1 *= fast_exp2(fminf(lam_q - sLam[k1], 0.0f));
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
                    for (int t = 0; t < DV / 16; ++t) {
                        const E* vr = sVt + (16 * t + l16) * LKT + 32 * p + 4 * g4;
                        acc[t] = mma(join(lds_f4(vr), lds_f4(vr + 16)), bA, acc[t]);
                    }
                }
                den += __shfl_xor(den, 16, kWave);
                den += __shfl_xor(den, 32, kWave);
                const float inv = 1.0f / fmaxf(den, args.eps);
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

        // ---- fold the chunk into the state -------------------------------------
        {
            const float dl = GATED ? fast_exp2(lam_last) : 1.0f;
#pragma unroll
            for (int j = 0; j < Sh::TPW; ++j)
                if (GATED) sacc[j] *= dl;
#pragma unroll
            for (int kbk = 0; kbk < CH / 32; ++kbk) {
#pragma unroll
                for (int j = 0; j < Sh::TPW; ++j) {
                    const int u = w * Sh::TPW + j;
                    const int a = u / Sh::NB, b = u % Sh::NB;
                    sacc[j] = mma(lds_f8(sKt + (16 * a + l16) * LKT + 32 * kbk + 8 * g4),
                                  lds_f8(sVt + (16 * b + l16) * LKT + 32 * kbk + 8 * g4), sacc[j]);
                }
            }
            float zs = 0.0f;
            constexpr int KP = CH / Sh::TPD;
#pragma unroll 8
            for (int j = 0; j < KP; ++j) zs += X::to_f32(sKt[zd * LKT + zsub * KP + j]);
#pragma unroll
            for (int off = 1; off < Sh::TPD; off <<= 1) zs += __shfl_xor(zs, off, kWave);
            zr = dl * zr + zs;
            lg_total += lam_last;
        }
        __syncthreads();
        if (OUTPUT && n + 1 < nch) stage_state();
    }

    if (!OUTPUT) {
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j)
            *reinterpret_cast<f32x4_t*>(stp + ((w * Sh::TPW + j) * kWave + lane) * 4) = sacc[j];
        if (zsub == 0) ztp[zd] = zr;
        if (GATED && tid == 0) args.lg[size_t(bh) * args.nseg + seg] = lg_total;
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
    float acc = init ? init[uidx] : 0.0f;
    for (int s = 0; s < nseg; ++s) {
        const float t = base[s * stride];
        base[s * stride] = acc;
        const float f = GATED ? fast_exp2(lg[size_t(bh) * nseg + s]) : 1.0f;
        acc = f * acc + t;
    }
    if (fin) fin[uidx] = acc;
}

}  // namespace linattn
