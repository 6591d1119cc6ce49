// Gradients of the chunked forward on gfx950: dq, dk, dv, dg and the initial-state
// gradients, for both output modes.
//
// The pages give the forward only and call the chunked form the training path
// (aiwiki.thehackersbrain.dev page, the chunked listing's closing paragraph;
// learn.pranaymahendrakar.com page, "Implementation reality").  The gradients are
// those of the recurrence S_t = g_t S_{t-1} + phi(k_t) v_t^T, z alike, with
// o_t = S_t^T phi(q_t) / max(phi(q_t) . z_t, eps) (learn.pranaymahendrakar.com page,
// "Derivation" and "Try it yourself"), taken chunk by chunk.  With do the incoming
// gradient, d_i = max(den_i, eps) and, where den_i >= eps,
//     dnum_i = do_i / d_i,   dden_i = -(do_i . o_i) / d_i         (0 below the clamp)
// (dnum_i = do_i and dden_i = 0 without the normaliser), and pairwise weights
// w_ij = prod_{l=j+1..i} g_l for j <= i:
//     dphi(q_i) = sum_{j<=i} w_ij (dnum_i . v_j + dden_i) phi(k_j)   (+ the S0 / z0 terms)
//     dphi(k_j) = sum_{i>=j} w_ij (dnum_i . v_j + dden_i) phi(q_i)
//     dv_j      = sum_{i>=j} w_ij (phi(q_i) . phi(k_j)) dnum_i
//     d log g_l = sum over the pairs j < l <= i of P_ij,  P_ij = w_ij (phi(q_i) . phi(k_j)) (dnum_i . v_j + dden_i)
// the last because log g_l enters exactly the weights w_ij of the pairs it separates
// (the initial state counting as a key in front of token 0).
//
// Work per chunk of C = 64 tokens (four waves, wave w owning rows 16w .. 16w + 15 of the
// chunk), with chunk-local Lambda_i = sum_{l=s..i} log2 g_l.  A workgroup walks a run of
// LC chunks and carries the states through it in fp32 registers, so the state slots in
// memory are per run, not per chunk:
//   bwd_dq_kernel   (run walked forwards, the state S_prev in front of the chunk carried)
//                   recomputes A = (Fq Fk^T) o decay o mask, num and den, forms 1/d and
//                   dden, then dFq = B Fk + 2^Lambda_i (dNum S_prev^T + dden z_prev^T)
//                   with B = (dNum V^T + dden 1^T) o decay o mask; folds the chunk's
//                   adjoint total dR_c = Fq^T (2^Lambda dNum), dr_c = Fq^T (2^Lambda dden)
//                   into the run's, and steps the state across the chunk.
//   bwd_dkv_kernel  (run walked backwards, the adjoint R, r of the state after the chunk
//                   carried): dFk = B^T Fq + 2^(Lambda_last - Lambda_j) (V R^T + 1 r^T),
//                   dV = A^T dNum + 2^(Lambda_last - Lambda_j) Fk R, then
//                   R <- 2^Lambda_last R + dR_c.
// dNum never enters a product rounded: the products take the exact input dout and
// scale by 1/d in fp32 (dNum V^T = diag(1/d) dOut V^T).  With the normaliser, dFq_i is
// orthogonal to Fq_i (its terms cancel), and a rounded dnum breaks that cancellation
// where d is small.
//   bwd_dg_kernel   d log g_l for token l of chunk c as four sums that never leave the
//                   chunk: the pairs inside it (X_l, from fp32 row and column sums of P
//                   in the dq pass), keys in front of it against its queries i >= l
//                   (Y_l, the running sum of Fq_i . dFq_i's carried-state part), its keys
//                   j < l against later queries (Z_l, of Fk_j . dFk_j's carried-state
//                   part) and keys in front against later queries (W_c).  With T_b the
//                   pairs across the boundary b between chunks (keys before, queries
//                   after; T = <R, S> + <r, z> of the state there and its adjoint),
//                   W_c = T_end(c) - K_c and T_end(c-1) = W_c + Y_c, with Y_c, K_c the
//                   chunk's sums of the yq and zk terms: the dk/dv pass forms T at the
//                   run's end from the two fp32 states and steps it back chunk by chunk.
//                   A running sum over the whole sequence would cancel to the initial
//                   state's term and collect the rounding of every token on the way; over
//                   one run it collects that of at most LC chunks.
// The states in front of every run come from the forward's totals walk (one run per
// segment) and its scan; the adjoint states from the same scan run over the runs'
// adjoint totals in reverse order.  Every MFMA operand is staged in LDS as a
// row-major tile; an operand whose contraction index runs down the tile's rows is
// read with ds_read_b64_tr_b16 (bf16) or element by element (fp32).
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;      // NULL: ungated
    const void* dout;
    const float* s0;     // [BH][D][Dv] or NULL
    const float* z0;     // [BH][D] or NULL
    void* dq;
    void* dk;
    void* dv;
    float* fst;          // [BH][NR][D*Dv] accumulator layout: slot r < NR-1 holds the state after run r
    float* fzt;          // [BH][NR][D]
    float* rst;          // [BH][NR+1][D*Dv]: run r's adjoint total at slot NR-1-r; after the
                         // scan slot NR-2-r holds the adjoint of the state after run r, and
                         // slot NR-1 the gradient of S0
    float* rzt;          // [BH][NR+1][D], alike
    float* rlg;          // [BH][NR+1] log2 of each run's total decay, reversed like rst
    float* inv;          // [BH][N]: 1 / max(den, eps) of every token (1 without the normaliser)
    float* dden;         // [BH][N]
    float* xs;           // [BH][N]: X_l, the pairs inside the chunk that straddle l
    float* yq;           // [BH][N]: Fq_i . (carried-state part of dFq_i)
    float* zk;           // [BH][N]: Fk_j . (carried-state part of dFk_j)
    float* wc;           // [BH][NC]: W_c
    int N;
    int NC;              // chunks of C tokens
    int LC;              // chunks per run: one workgroup walks a run, carrying the states through it
    int NR;              // runs, ceil(NC / LC)
    float eps;
    int normalize;
};

constexpr int kBwdChunk = kBwdChunkHost;

template <typename E, int D, int DV>
struct BwdShape {
    static constexpr int C = kBwdChunk;
    static constexpr int PAD = 16 / int(sizeof(E));   // one 16-byte group per row
    static constexpr int LQ = D + PAD;                 // phi(Q), phi(K) [C][D]
    static constexpr int LV = DV + PAD;                // V, dNum [C][Dv]; S_prev / R [D][Dv]
    static constexpr int LA = C + PAD;                 // A or B [C][C]
    static constexpr size_t kOffQ = 0;
    static constexpr size_t kOffK = kOffQ + size_t(C) * LQ * sizeof(E);
    static constexpr size_t kOffV = kOffK + size_t(C) * LQ * sizeof(E);
    static constexpr size_t kOffDn = kOffV + size_t(C) * LV * sizeof(E);
    static constexpr size_t kOffS = kOffDn + size_t(C) * LV * sizeof(E);
    static constexpr size_t kOffA = kOffS + size_t(D) * LV * sizeof(E);
    static constexpr size_t kOffLam = kOffA + size_t(C) * LA * sizeof(E);
    static constexpr size_t kOffDd = kOffLam + size_t(C) * 4;
    static constexpr size_t kOffInv = kOffDd + size_t(C) * 4;
    static constexpr size_t kOffCol = kOffInv + size_t(C) * 4;     // [4][C] per-wave column sums of P
    static constexpr size_t kOffRow = kOffCol + size_t(4) * C * 4;  // [C] row sums of P
    static constexpr size_t kOffZ = kOffRow + size_t(C) * 4;
    static constexpr size_t kBytes = kOffZ + size_t(D) * 4;
    static_assert(kBytes == bwd_lds_bytes(int(sizeof(E)), D, DV), "host LDS formula out of step");
    static_assert(4 * C >= kThreads && kThreads % D == 0, "column-sum slices fit sCol");
    // workgroups (so waves per SIMD) the LDS allows: the register target of both kernels,
    // so the compiler does not squeeze the accumulators for an occupancy out of reach
    static constexpr int kWaves = int(kMaxLds / kBytes) < 1 ? 1 : int(kMaxLds / kBytes);
    // 16-byte pieces per thread of a state in accumulator layout, and of one chunk's four
    // row tiles.  Loading the next chunk's rows during this chunk's products keeps them
    // live across the products, beside the two carried states: done where all of it stays
    // within 32 pieces (128 registers), else the rows are loaded chunk by chunk.
    static constexpr int kStateUnits = D * DV / 4 / kThreads;
    static constexpr int kRowPieces = (2 * C * D + 2 * C * DV) * int(sizeof(E)) / 16 / kThreads;
    static constexpr bool kAhead = kRowPieces + 2 * kStateUnits <= 32;
};

// Operand of 16 rows from a row-major tile: lane supplies row `row`, contraction
// slots k0 .. k0 + 7 (k0 includes the lane group's offset), one 16-byte read (bf16).
template <typename E>
__device__ __forceinline__ F8<E> frag_row(const E* t, int ld, int row, int k0) {
    return lds_f8(t + row * ld + k0);
}

// Operand whose contraction index runs down the rows of a row-major tile: slot e of
// lane l holds t[k0 + e][n0 + l % 16].  bf16: two ds_read_b64_tr_b16, each giving a
// 16-lane block four rows of one column when block lane j points at row k0 + j / 4,
// columns n0 + 4 (j % 4) .. + 3.  fp32: eight reads.
__device__ __forceinline__ F8<uint16_t> frag_col(const uint16_t* t, int ld, int k0, int n0, int l16) {
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4_t* lds_ptr_t;
    const uint16_t* p = t + (k0 + (l16 >> 2)) * ld + n0 + 4 * (l16 & 3);
    const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr_t)(const_cast<uint16_t*>(p)));
    const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr_t)(const_cast<uint16_t*>(p + 4 * ld)));
    F8<uint16_t> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f.x[e] = uint16_t(a[e]);
        f.x[4 + e] = uint16_t(b[e]);
    }
    return f;
}

__device__ __forceinline__ F8<float> frag_col(const float* t, int ld, int k0, int n0, int l16) {
    F8<float> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.x[e] = t[(k0 + e) * ld + n0 + l16];
    return f;
}

// Sum over the 16 lanes of a lane group (the columns of an accumulator row), every lane
// getting the total: DPP moves within each 16-lane row, no LDS round trip.  Quad swaps
// (lanes 1,0,3,2 then 2,3,0,1) leave each quad's sum in all its lanes; the half-row
// mirror (lane i from 7 - i) adds the neighbouring quad, the row mirror (i from 15 - i)
// the other half.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum16(float x) {
    x += dpp_move<0xB1>(x);     // quad_perm [1, 0, 3, 2]
    x += dpp_move<0x4E>(x);     // quad_perm [2, 3, 0, 1]
    x += dpp_move<0x141>(x);    // row_half_mirror
    x += dpp_move<0x140>(x);    // row_mirror
    return x;
}

// The derivative of elu + 1 from its value: phi'(x) = 1 above zero, where phi(x) = x + 1 > 1,
// and exp(x) = phi(x) at or below zero, so phi'(x) = min(phi(x), 1).  Taken from the staged
// features (in the input precision), it adds one rounding of the size of the output's own.
__device__ __forceinline__ float dphi_of(float f) { return fminf(f, 1.0f); }

// The per-workgroup machinery shared by both gradient kernels.
template <typename E, int D, int DV, bool GATED>
struct BwdChunk {
    using Sh = BwdShape<E, D, DV>;
    using X = Elem<E>;
    static constexpr int C = Sh::C, LQ = Sh::LQ, LV = Sh::LV, LA = Sh::LA;
    static constexpr int GQ = D * int(sizeof(E)) / 16;    // 16-byte groups per q/k row
    static constexpr int GV = DV * int(sizeof(E)) / 16;   // per v row
    static constexpr int EPG = 16 / int(sizeof(E));       // elements per group

    E* sQ;
    E* sK;
    E* sV;
    E* sDn;
    E* sS;
    E* sA;
    float* sLam;
    float* sDd;
    float* sInv;
    float* sCol;
    float* sRow;
    float* sZ;
    int tid, w, lane, l16, g4;
    int bh, c, ts, nrows, N, NC, run, c_first, c_end;

    __device__ __forceinline__ void init(unsigned char* smem, int N_, int NC_, int LC) {
        sQ = reinterpret_cast<E*>(smem + Sh::kOffQ);
        sK = reinterpret_cast<E*>(smem + Sh::kOffK);
        sV = reinterpret_cast<E*>(smem + Sh::kOffV);
        sDn = reinterpret_cast<E*>(smem + Sh::kOffDn);
        sS = reinterpret_cast<E*>(smem + Sh::kOffS);
        sA = reinterpret_cast<E*>(smem + Sh::kOffA);
        sLam = reinterpret_cast<float*>(smem + Sh::kOffLam);
        sDd = reinterpret_cast<float*>(smem + Sh::kOffDd);
        sInv = reinterpret_cast<float*>(smem + Sh::kOffInv);
        sCol = reinterpret_cast<float*>(smem + Sh::kOffCol);
        sRow = reinterpret_cast<float*>(smem + Sh::kOffRow);
        sZ = reinterpret_cast<float*>(smem + Sh::kOffZ);
        tid = threadIdx.x;
        w = __builtin_amdgcn_readfirstlane(tid / kWave);
        lane = tid % kWave;
        l16 = lane & 15;
        g4 = lane >> 4;
        N = N_;
        NC = NC_;
        const int ngrp = (NC + LC - 1) / LC;
        bh = blockIdx.x / ngrp;
        run = blockIdx.x % ngrp;
        c_first = run * LC;
        c_end = min(NC, c_first + LC);
        set_chunk(c_first);
    }

    // The lane indices made opaque at the top of every chunk: the compiler then rebuilds
    // the many LDS addresses derived from them inside the chunk loop instead of hoisting
    // them all out of it and holding them in registers across the products.
    __device__ __forceinline__ void refresh() { asm volatile("" : "+v"(tid), "+v"(lane), "+v"(l16), "+v"(g4)); }

    __device__ __forceinline__ void set_chunk(int c_) {
        c = c_;
        ts = c * C;
        nrows = min(C, N - ts);
    }

    // Staging is split into a load phase and a store phase so that every global load of
    // the chunk is in flight at once: a load followed by its use in a loop would make the
    // workgroup wait for each one in turn.
    //
    // Rows [ts, ts + C) of a [N][W] tensor: 16-byte units, rows clamped to the last valid
    // one (the loads are unconditional).
    template <int W>
    static constexpr int kRowUnits = C * W * int(sizeof(E)) / 16 / kThreads;

    template <int W>
    __device__ __forceinline__ void load_rows(f32x4_t (&r)[kRowUnits<W>], const E* src, int ts_, int nrows_) const {
        constexpr int G = W * int(sizeof(E)) / 16;
#pragma unroll
        for (int u = 0; u < kRowUnits<W>; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = (idx % G) * EPG;
            r[u] = *reinterpret_cast<const f32x4_t*>(src + size_t(ts_ + min(row, nrows_ - 1)) * W + col);
        }
    }

    // ... into a row-major tile through phi (or as they are) in fp32; rows past the
    // chunk's end become zero.
    template <int W, bool PHI>
    __device__ __forceinline__ void store_rows(E* tile, int ld, const f32x4_t (&r)[kRowUnits<W>]) const {
        constexpr int G = W * int(sizeof(E)) / 16;
#pragma unroll
        for (int u = 0; u < kRowUnits<W>; ++u) {
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

    // The chunk's valid rows of a row-major tile out to a [N][W] tensor, 16 bytes at a time.
    template <int W>
    __device__ __forceinline__ void store_out(E* dst, const E* tile, int ld) const {
        constexpr int G = W * int(sizeof(E)) / 16;
#pragma unroll
        for (int u = 0; u < kRowUnits<W>; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = (idx % G) * EPG;
            if (row < nrows)
                *reinterpret_cast<f32x4_t*>(dst + size_t(ts + row) * W + col) =
                    *reinterpret_cast<const f32x4_t*>(tile + row * ld + col);
        }
    }

    // A state slot in accumulator layout: D * Dv / 4 16-byte pieces per workgroup.
    static constexpr int kStateUnits = Sh::kStateUnits;

    __device__ __forceinline__ void load_slot(f32x4_t (&r)[kStateUnits], const float* slot) const {
#pragma unroll
        for (int u = 0; u < kStateUnits; ++u) r[u] = *reinterpret_cast<const f32x4_t*>(slot + 4 * (tid + u * kThreads));
    }

    // ... into sS (row-major [D][Dv], operand precision).
    __device__ __forceinline__ void store_slot(const f32x4_t (&r)[kStateUnits]) const {
#pragma unroll
        for (int u = 0; u < kStateUnits; ++u) {
            const int q4 = tid + u * kThreads;
            const int t = q4 / kWave, ln = q4 % kWave;
            const int a = t / (DV / 16), b = t % (DV / 16);
            const int d = 16 * a + 4 * (ln >> 4), e = 16 * b + (ln & 15);
#pragma unroll
            for (int k = 0; k < 4; ++k) sS[(d + k) * LV + e] = X::from_f32(r[u][k]);
        }
    }

    // A caller-layout [D][Dv] state (or zero) into this thread's accumulator-layout pieces.
    __device__ __forceinline__ void load_user(f32x4_t (&r)[kStateUnits], const float* S) const {
#pragma unroll
        for (int u = 0; u < kStateUnits; ++u) {
            const int q4 = tid + u * kThreads;
            const int t = q4 / kWave, ln = q4 % kWave;
            const int a = t / (DV / 16), b = t % (DV / 16);
            const int d = 16 * a + 4 * (ln >> 4), e = 16 * b + (ln & 15);
#pragma unroll
            for (int k = 0; k < 4; ++k) r[u][k] = S ? S[size_t(d + k) * DV + e] : 0.0f;
        }
    }

    // Accumulator-layout pieces out to a workspace slot.
    __device__ __forceinline__ void put_slot(float* slot, const f32x4_t (&r)[kStateUnits]) const {
#pragma unroll
        for (int u = 0; u < kStateUnits; ++u) *reinterpret_cast<f32x4_t*>(slot + 4 * (tid + u * kThreads)) = r[u];
    }

    // One 16x16 state tile, contraction over the chunk's rows: lhs^T rhs for the tile's
    // rows a and columns b of two row-major tiles (this lane's accumulator piece).
    __device__ __forceinline__ f32x4_t tile_tn(const E* lhs, int ldl, int a, const E* rhs, int ldr, int b) const {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C / 32; ++ks)
            acc = mma(frag_col(lhs, ldl, 32 * ks + 8 * g4, 16 * a, l16), frag_col(rhs, ldr, 32 * ks + 8 * g4, 16 * b, l16),
                      acc);
        return acc;
    }

    // The gate of row `lane` of the chunk starting at ts_ (rows clamped), for stage_lambda.
    __device__ __forceinline__ float load_gate(const float* gb, int ts_, int nrows_) const {
        if constexpr (GATED) return gb[ts_ + min(lane, nrows_ - 1)];
        return 1.0f;
    }

    // Chunk-local inclusive log2 cumulative decay into sLam (wave 0) from this lane's
    // gate; rows past the end get a unit gate.  sLam[C - 1] is the chunk's total.
    __device__ __forceinline__ void stage_lambda(float gv) const {
        if constexpr (GATED) {
            if (w == 0) {
                float x = lane < nrows ? fast_log2(gv) : 0.0f;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const float y = __shfl_up(x, off, kWave);
                    if (lane >= off) x += y;
                }
                sLam[lane] = x;
            }
        }
    }

    __device__ __forceinline__ float lam(int i) const {
        if constexpr (GATED) return sLam[i];
        return 0.0f;
    }
};

// ----------------------------------------------------------------- dq pass ----

template <typename E, int D, int DV, bool GATED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BwdShape<E, D, DV>::kWaves,
                                                                           BwdShape<E, D, DV>::kWaves)))
void bwd_dq_kernel(BwdArgs args) {
    using B = BwdChunk<E, D, DV, GATED>;
    using X = Elem<E>;
    constexpr int C = B::C, LQ = B::LQ, LV = B::LV, LA = B::LA;
    constexpr int ND = D / 16, NE = DV / 16, NJ = C / 16;
    constexpr int kParts = kThreads / D, kRowsPer = C / kParts;   // column sums: threads per column, rows each
    extern __shared__ __align__(16) unsigned char smem[];
    B ck;
    ck.init(smem, args.N, args.NC, args.LC);
    const int w = ck.w, bh = ck.bh;
    const int N = args.N, NC = args.NC;
    const E* qb = reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D;
    const E* kb = reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D;
    const E* vb = reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV;
    const E* dob = reinterpret_cast<const E*>(args.dout) + size_t(bh) * N * DV;

    // The state in front of the current chunk, carried through the run in fp32 (this
    // thread's accumulator-layout pieces, z_prev[tid] for tid < D): from the scanned slot
    // in front of the run, or S0 / z0 for the first run.
    f32x4_t sacc[B::kStateUnits];
    float zacc = 0.0f;
    if (ck.run > 0) {
        const size_t fslot = size_t(bh) * args.NR + (ck.run - 1);
        ck.load_slot(sacc, args.fst + fslot * (D * DV));
        if (ck.tid < D) zacc = args.fzt[fslot * D + ck.tid];
    } else {
        ck.load_user(sacc, args.s0 ? args.s0 + size_t(bh) * D * DV : nullptr);
        if (ck.tid < D && args.z0) zacc = args.z0[size_t(bh) * D + ck.tid];
    }
    // The run's adjoint total (what its queries pass to the state in front of it): the sum
    // over its chunks of the chunk's adjoint total times the decay from the run's start to
    // the chunk's start, 2^logp.
    f32x4_t racc[B::kStateUnits];
#pragma unroll
    for (int u = 0; u < B::kStateUnits; ++u) racc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float rzacc = 0.0f, logp = 0.0f;

    // staging registers, loaded one chunk ahead of the products
    f32x4_t sq[B::template kRowUnits<D>], sk[B::template kRowUnits<D>];
    f32x4_t sv[B::template kRowUnits<DV>], so[B::template kRowUnits<DV>];
    float sg = 1.0f;
    auto issue = [&](int cn) {
        const int tn = cn * C, nn = min(C, N - tn);
        ck.template load_rows<D>(sq, qb, tn, nn);
        ck.template load_rows<D>(sk, kb, tn, nn);
        ck.template load_rows<DV>(sv, vb, tn, nn);
        ck.template load_rows<DV>(so, dob, tn, nn);
        if constexpr (GATED) sg = ck.load_gate(args.g + size_t(bh) * N, tn, nn);
    };
    if constexpr (B::Sh::kAhead) issue(ck.c_first);
    for (int c = ck.c_first; c < ck.c_end; ++c) {
    ck.refresh();
    const int lane = ck.lane, l16 = ck.l16, g4 = ck.g4;
    ck.set_chunk(c);
    const int ts = ck.ts;
    if constexpr (!B::Sh::kAhead) issue(c);
    ck.template store_rows<D, true>(ck.sQ, LQ, sq);
    ck.template store_rows<D, true>(ck.sK, LQ, sk);
    ck.template store_rows<DV, false>(ck.sV, LV, sv);
    ck.template store_rows<DV, false>(ck.sDn, LV, so);
    ck.store_slot(sacc);
    if (ck.tid < D) ck.sZ[ck.tid] = zacc;
    ck.stage_lambda(sg);
    __syncthreads();
    if (B::Sh::kAhead && c + 1 < ck.c_end) issue(c + 1);

    const int i0 = 16 * w;            // this wave's query rows
    float lam_r[4], rs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lam_r[r] = ck.lam(i0 + 4 * g4 + r);

    // A = Fq Fk^T, decayed and masked, into sA (rows of this wave); row sums in fp32.
    // acc keeps the undecayed fp32 scores for the pair sums of d log g.
    f32x4_t acc[NJ];
    {
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) acc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const F8<E> a = frag_row(ck.sQ, LQ, i0 + l16, 32 * ks + 8 * g4);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
                if (jt <= w) acc[jt] = mma(a, frag_row(ck.sK, LQ, 16 * jt + l16, 32 * ks + 8 * g4), acc[jt]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) rs[r] = 0.0f;
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            const int j = 16 * jt + l16;
            const float lj = ck.lam(j);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + 4 * g4 + r;
                float x = (jt <= w && j <= i) ? acc[jt][r] : 0.0f;
                if constexpr (GATED) x *= fast_exp2(fminf(lam_r[r] - lj, 0.0f));
                const E xe = X::from_f32(x);
                ck.sA[i * LA + j] = xe;
                rs[r] += X::to_f32(xe);          // the row sum of the values the numerator uses
            }
        }
    }
    // den = 2^Lambda_i Fq_i . z_prev + sum_j A_ij
    float den[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * g4 + r;
        float zt = 0.0f;
#pragma unroll
        for (int t = 0; t < ND; ++t) zt += X::to_f32(ck.sQ[i * LQ + 16 * t + l16]) * ck.sZ[16 * t + l16];
        den[r] = sum16(rs[r] + (GATED ? fast_exp2(lam_r[r]) : 1.0f) * zt);
    }
    __syncthreads();

    // num = 2^Lambda_i Fq S_prev + A V
    f32x4_t num[NE];
#pragma unroll
    for (int et = 0; et < NE; ++et) num[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        const F8<E> a = frag_row(ck.sQ, LQ, i0 + l16, 32 * ks + 8 * g4);
#pragma unroll
        for (int et = 0; et < NE; ++et) num[et] = mma(a, frag_col(ck.sS, LV, 32 * ks + 8 * g4, 16 * et, l16), num[et]);
    }
    if constexpr (GATED) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float f = fast_exp2(lam_r[r]);
#pragma unroll
            for (int et = 0; et < NE; ++et) num[et][r] *= f;
        }
    }
    for (int ks = 0; ks <= (w >> 1); ++ks) {
        const F8<E> a = frag_row(ck.sA, LA, i0 + l16, 32 * ks + 8 * g4);
#pragma unroll
        for (int et = 0; et < NE; ++et) num[et] = mma(a, frag_col(ck.sV, LV, 32 * ks + 8 * g4, 16 * et, l16), num[et]);
    }

    // 1/d and dden = -(dout . num) / d^2 (fp32); dnum = dout / d stays implicit
    float dd[4], inv[4];
    {
        float dsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) inv[r] = args.normalize ? 1.0f / fmaxf(den[r], args.eps) : 1.0f;
#pragma unroll
        for (int et = 0; et < NE; ++et)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dsum[r] += X::to_f32(ck.sDn[(i0 + 4 * g4 + r) * LV + 16 * et + l16]) * num[et][r];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float s = sum16(dsum[r]);
            const int i = i0 + 4 * g4 + r;
            dd[r] = (args.normalize && den[r] >= args.eps) ? -s * inv[r] * inv[r] : 0.0f;
            if (l16 == 0 && ts + i < N) {
                args.dden[size_t(bh) * N + ts + i] = dd[r];
                args.inv[size_t(bh) * N + ts + i] = inv[r];
            }
        }
    }
    __syncthreads();

    // B = (diag(1/d) dOut V^T + dden 1^T) o decay o mask over this wave's rows, into sA
    // (every read of A finished before the barrier above); with it the pair terms
    // P_ij = (Fq_i . Fk_j) B_ij in fp32, summed by row (j < i) and by column (i > j)
    {
        f32x4_t bb[NJ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) bb[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DV / 32; ++ks) {
            const F8<E> a = frag_row(ck.sDn, LV, i0 + l16, 32 * ks + 8 * g4);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
                if (jt <= w) bb[jt] = mma(a, frag_row(ck.sV, LV, 16 * jt + l16, 32 * ks + 8 * g4), bb[jt]);
        }
        float prow[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            const int j = 16 * jt + l16;
            const float lj = ck.lam(j);
            float pcol = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + 4 * g4 + r;
                float x = (jt <= w && j <= i) ? bb[jt][r] * inv[r] + dd[r] : 0.0f;
                if constexpr (GATED) x *= fast_exp2(fminf(lam_r[r] - lj, 0.0f));
                ck.sA[i * LA + j] = X::from_f32(x);
                if constexpr (GATED) {
                    const float pij = j < i ? acc[jt][r] * x : 0.0f;
                    prow[r] += pij;
                    pcol += pij;
                }
            }
            if constexpr (GATED) {
                pcol += __shfl_xor(pcol, 16, kWave);
                pcol += __shfl_xor(pcol, 32, kWave);
                if (g4 == 0) ck.sCol[w * C + j] = pcol;
            }
        }
        if constexpr (GATED) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sr = sum16(prow[r]);
                if (l16 == 0) ck.sRow[i0 + 4 * g4 + r] = sr;
            }
        }
    }
    __syncthreads();
    // X_l = sum_{m < l} (col_m - row_m): the pairs inside the chunk with j < l <= i
    if (GATED && w == 0) {
        const float dm = ck.sCol[lane] + ck.sCol[C + lane] + ck.sCol[2 * C + lane] + ck.sCol[3 * C + lane] -
                         ck.sRow[lane];
        float x = dm;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float y = __shfl_up(x, off, kWave);
            if (lane >= off) x += y;
        }
        if (lane < ck.nrows) args.xs[size_t(bh) * N + ts + lane] = x - dm;
    }

    // dFq = 2^Lambda_i (diag(1/d) dOut S_prev^T + dden z_prev^T) + B Fk
    f32x4_t dfq[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) dfq[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks) {
        const F8<E> a = frag_row(ck.sDn, LV, i0 + l16, 32 * ks + 8 * g4);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) dfq[dt] = mma(a, frag_row(ck.sS, LV, 16 * dt + l16, 32 * ks + 8 * g4), dfq[dt]);
    }
    {
        float yq[4] = {0.f, 0.f, 0.f, 0.f};            // Fq_i . (carried-state part of dFq_i)
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const float zd = ck.sZ[16 * dt + l16];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = dfq[dt][r] * inv[r] + dd[r] * zd;
                dfq[dt][r] = GATED ? x * fast_exp2(lam_r[r]) : x;
                if constexpr (GATED) yq[r] += X::to_f32(ck.sQ[(i0 + 4 * g4 + r) * LQ + 16 * dt + l16]) * dfq[dt][r];
            }
        }
        if constexpr (GATED) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float s = sum16(yq[r]);
                const int i = i0 + 4 * g4 + r;
                if (l16 == 0 && ts + i < N) args.yq[size_t(bh) * N + ts + i] = s;
            }
        }
    }
    for (int ks = 0; ks <= (w >> 1); ++ks) {
        const F8<E> a = frag_row(ck.sA, LA, i0 + l16, 32 * ks + 8 * g4);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) dfq[dt] = mma(a, frag_col(ck.sK, LQ, 32 * ks + 8 * g4, 16 * dt, l16), dfq[dt]);
    }

    // dq = dFq * phi'(q), written to LDS once every read of phi(K) is done
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dfq[dt][r] *= dphi_of(X::to_f32(ck.sQ[(i0 + 4 * g4 + r) * LQ + 16 * dt + l16]));

    // this wave's rows of dOut become 2^Lambda_i dnum_i and its rows of V become
    // 2^(Lambda_last - Lambda_j) v_j (every other read of both is done)
    const float lam_last = ck.lam(C - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * g4 + r;
        const float f = GATED ? fast_exp2(lam_r[r]) : 1.0f;
        const float fv = GATED ? fast_exp2(fminf(lam_last - lam_r[r], 0.0f)) : 1.0f;
#pragma unroll
        for (int et = 0; et < NE; ++et) {
            E& x = ck.sDn[i * LV + 16 * et + l16];
            x = X::from_f32(X::to_f32(x) * (f * inv[r]));
            if constexpr (GATED) {
                E& y = ck.sV[i * LV + 16 * et + l16];
                y = X::from_f32(X::to_f32(y) * fv);
            }
        }
        if (l16 == 0) ck.sDd[i] = dd[r] * f;
    }
    __syncthreads();
    // The chunk's adjoint total dR_c = Fq^T (2^Lambda dNum), dr_c = Fq^T (2^Lambda dden),
    // into the run's with the decay 2^logp from the run's start; and the state carried
    // across the chunk: S <- 2^Lambda_last S + Fk^T (2^(Lambda_last - Lambda_j) V), z alike.
    {
        const float fp = GATED ? fast_exp2(logp) : 1.0f, fc = GATED ? fast_exp2(lam_last) : 1.0f;
#pragma unroll
        for (int u = 0; u < B::kStateUnits; ++u) {
            const int t = w + 4 * u, a = t / NE, b = t % NE;
            const f32x4_t dr = ck.tile_tn(ck.sQ, LQ, a, ck.sDn, LV, b);
            const f32x4_t ds = ck.tile_tn(ck.sK, LQ, a, ck.sV, LV, b);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                racc[u][k] += fp * dr[k];
                sacc[u][k] = fc * sacc[u][k] + ds[k];
            }
        }
        // the z parts, Fq^T (2^Lambda dden) and Fk^T 2^(Lambda_last - Lambda_j): every
        // thread sums a slice of the rows of one column, into sA (free in this phase)
        float* part = reinterpret_cast<float*>(ck.sA);
        {
            const int d = ck.tid % D, i0p = (ck.tid / D) * kRowsPer;
            float sr = 0.0f, sz = 0.0f;
#pragma unroll
            for (int ii = 0; ii < kRowsPer; ++ii) {
                const int i = i0p + ii;
                sr += X::to_f32(ck.sQ[i * LQ + d]) * ck.sDd[i];
                const float fk = X::to_f32(ck.sK[i * LQ + d]);
                sz += GATED ? fk * fast_exp2(fminf(lam_last - ck.lam(i), 0.0f)) : fk;
            }
            part[ck.tid] = sr;
            part[kThreads + ck.tid] = sz;
        }
        __syncthreads();
        if (ck.tid < D) {
            float sr = 0.0f, sz = 0.0f;
#pragma unroll
            for (int p = 0; p < kParts; ++p) {
                sr += part[p * D + ck.tid];
                sz += part[kThreads + p * D + ck.tid];
            }
            rzacc += fp * sr;
            zacc = fc * zacc + sz;
        }
        logp += lam_last;
    }
    // phi(K) is no longer read: it takes dq for the coalesced store
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) ck.sK[(i0 + 4 * g4 + r) * LQ + 16 * dt + l16] = X::from_f32(dfq[dt][r]);
    __syncthreads();
    ck.template store_out<D>(reinterpret_cast<E*>(args.dq) + size_t(bh) * N * D, ck.sK, LQ);
    __syncthreads();                  // every read of this chunk's tiles is done
    }

    // the run's adjoint total at its reversed slot
    const size_t rslot = size_t(bh) * (args.NR + 1) + (args.NR - 1 - ck.run);
    ck.put_slot(args.rst + rslot * (D * DV), racc);
    if (ck.tid < D) args.rzt[rslot * D + ck.tid] = rzacc;
    if (GATED && ck.tid == 0) args.rlg[rslot] = logp;
}

// ------------------------------------------------------------ dk / dv pass ----

template <typename E, int D, int DV, bool GATED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BwdShape<E, D, DV>::kWaves,
                                                                           BwdShape<E, D, DV>::kWaves)))
void bwd_dkv_kernel(BwdArgs args) {
    using B = BwdChunk<E, D, DV, GATED>;
    using X = Elem<E>;
    constexpr int C = B::C, LQ = B::LQ, LV = B::LV, LA = B::LA;
    constexpr int ND = D / 16, NE = DV / 16, NI = C / 16;
    constexpr int kParts = kThreads / D, kRowsPer = C / kParts;   // column sums: threads per column, rows each
    extern __shared__ __align__(16) unsigned char smem[];
    B ck;
    ck.init(smem, args.N, args.NC, args.LC);
    const int w = ck.w, bh = ck.bh;
    const int N = args.N, NC = args.NC;
    const E* qb = reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D;
    const E* kb = reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D;
    const E* vb = reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV;
    const E* dob = reinterpret_cast<const E*>(args.dout) + size_t(bh) * N * DV;
    static_assert(D <= kThreads && C <= kThreads, "one thread per state row and per token");

    // R, r: the adjoint of the state after the current chunk, carried backwards through
    // the run in fp32 (accumulator-layout pieces, r[tid] for tid < D), from the scanned
    // slot after the run (zero after the last run).
    const bool last_run = ck.run == args.NR - 1;
    f32x4_t racc[B::kStateUnits];
    float rzacc = 0.0f;
    if (!last_run) {
        const size_t rsl = size_t(bh) * (args.NR + 1) + (args.NR - 2 - ck.run);
        ck.load_slot(racc, args.rst + rsl * (D * DV));
        if (ck.tid < D) rzacc = args.rzt[rsl * D + ck.tid];
    } else {
#pragma unroll
        for (int u = 0; u < B::kStateUnits; ++u) racc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // tb: the pairs across the boundary after the current chunk (keys up to it, queries
    // after it), <R, S> + <r, z> with S, z the state after the chunk; at the run's end from
    // the forward slot after the run, then back chunk by chunk (W_c = tb - K_c, and the
    // boundary in front of the chunk carries W_c + Y_c).
    float tb = 0.0f;
    if constexpr (GATED) {
        float wp = 0.0f;
        if (!last_run) {
            const size_t fsl = size_t(bh) * args.NR + ck.run;
            f32x4_t sf[B::kStateUnits];
            ck.load_slot(sf, args.fst + fsl * (D * DV));
#pragma unroll
            for (int u = 0; u < B::kStateUnits; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) wp += racc[u][k] * sf[u][k];
            if (ck.tid < D) wp += rzacc * args.fzt[fsl * D + ck.tid];
        }
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) wp += __shfl_xor(wp, off, kWave);
        if (ck.lane == 0) ck.sRow[ck.w] = wp;
        __syncthreads();
        tb = ck.sRow[0] + ck.sRow[1] + ck.sRow[2] + ck.sRow[3];
        __syncthreads();
    }

    // staging registers, loaded one chunk ahead of the products (the run is walked
    // backwards)
    f32x4_t sq[B::template kRowUnits<D>], sk[B::template kRowUnits<D>];
    f32x4_t sv[B::template kRowUnits<DV>], so[B::template kRowUnits<DV>];
    float sdd = 0.0f, sinv = 0.0f, syq = 0.0f, sg = 1.0f;
    auto issue = [&](int cn) {
        const int tn = cn * C, nn = min(C, N - tn);
        ck.template load_rows<D>(sq, qb, tn, nn);
        ck.template load_rows<D>(sk, kb, tn, nn);
        ck.template load_rows<DV>(sv, vb, tn, nn);
        ck.template load_rows<DV>(so, dob, tn, nn);
        if (ck.tid < C) {
            const size_t t = size_t(bh) * N + tn + min(ck.tid, nn - 1);
            sdd = args.dden[t];
            sinv = args.inv[t];
            if constexpr (GATED) syq = args.yq[t];
        }
        if constexpr (GATED) sg = ck.load_gate(args.g + size_t(bh) * N, tn, nn);
    };
    if constexpr (B::Sh::kAhead) issue(ck.c_end - 1);
    for (int c = ck.c_end - 1; c >= ck.c_first; --c) {
    ck.refresh();
    const int lane = ck.lane, l16 = ck.l16, g4 = ck.g4;
    ck.set_chunk(c);
    const int ts = ck.ts;
    if constexpr (!B::Sh::kAhead) issue(c);
    ck.template store_rows<D, true>(ck.sQ, LQ, sq);
    ck.template store_rows<D, true>(ck.sK, LQ, sk);
    ck.template store_rows<DV, false>(ck.sV, LV, sv);
    ck.template store_rows<DV, false>(ck.sDn, LV, so);
    if (ck.tid < C) {
        ck.sDd[ck.tid] = ck.tid < ck.nrows ? sdd : 0.0f;
        ck.sInv[ck.tid] = ck.tid < ck.nrows ? sinv : 0.0f;
    }
    ck.store_slot(racc);
    if (ck.tid < D) ck.sZ[ck.tid] = rzacc;
    if constexpr (GATED) {
        // Y_c = sum of yq over the chunk's queries (wave 0: one lane per token)
        if (ck.w == 0) {
            float y = lane < ck.nrows ? syq : 0.0f;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) y += __shfl_xor(y, off, kWave);
            if (lane == 0) ck.sRow[0] = y;
        }
    }
    ck.stage_lambda(sg);
    __syncthreads();
    if (B::Sh::kAhead && c > ck.c_first) issue(c - 1);

    const int j0 = 16 * w;            // this wave's key rows
    float lam_r[4], tail[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        lam_r[r] = ck.lam(j0 + 4 * g4 + r);
        tail[r] = GATED ? fast_exp2(fminf(ck.lam(C - 1) - lam_r[r], 0.0f)) : 1.0f;   // 2^(Lambda_last - Lambda_j)
    }

    // A^T diag(1/d) = Fk Fq^T diag(1/d) and B^T = V dOut^T diag(1/d) + 1 dden^T, both
    // decayed and masked (i >= j)
    f32x4_t bt[NI];
    {
        f32x4_t at[NI];
#pragma unroll
        for (int it = 0; it < NI; ++it) {
            at[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            bt[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const F8<E> a = frag_row(ck.sK, LQ, j0 + l16, 32 * ks + 8 * g4);
#pragma unroll
            for (int it = 0; it < NI; ++it)
                if (it >= w) at[it] = mma(a, frag_row(ck.sQ, LQ, 16 * it + l16, 32 * ks + 8 * g4), at[it]);
        }
#pragma unroll
        for (int ks = 0; ks < DV / 32; ++ks) {
            const F8<E> a = frag_row(ck.sV, LV, j0 + l16, 32 * ks + 8 * g4);
#pragma unroll
            for (int it = 0; it < NI; ++it)
                if (it >= w) bt[it] = mma(a, frag_row(ck.sDn, LV, 16 * it + l16, 32 * ks + 8 * g4), bt[it]);
        }
#pragma unroll
        for (int it = 0; it < NI; ++it) {
            const int i = 16 * it + l16;
            const float li = ck.lam(i);
            const float ddi = ck.sDd[i], invi = ck.sInv[i];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = j0 + 4 * g4 + r;
                const bool keep = it >= w && i >= j;
                const float f = GATED ? fast_exp2(fminf(li - lam_r[r], 0.0f)) : 1.0f;
                ck.sA[j * LA + i] = X::from_f32(keep ? at[it][r] * (f * invi) : 0.0f);
                bt[it][r] = keep ? (bt[it][r] * invi + ddi) * f : 0.0f;
            }
        }
    }
    __syncthreads();

    // dV = 2^(Lambda_last - Lambda_j) Fk R + (A^T diag(1/d)) dOut
    f32x4_t dv[NE];
    {
#pragma unroll
        for (int et = 0; et < NE; ++et) dv[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const F8<E> a = frag_row(ck.sK, LQ, j0 + l16, 32 * ks + 8 * g4);
#pragma unroll
            for (int et = 0; et < NE; ++et) dv[et] = mma(a, frag_col(ck.sS, LV, 32 * ks + 8 * g4, 16 * et, l16), dv[et]);
        }
        if constexpr (GATED) {
#pragma unroll
            for (int et = 0; et < NE; ++et)
#pragma unroll
                for (int r = 0; r < 4; ++r) dv[et][r] *= tail[r];
        }
        for (int ks = w >> 1; ks < C / 32; ++ks) {
            const F8<E> a = frag_row(ck.sA, LA, j0 + l16, 32 * ks + 8 * g4);
#pragma unroll
            for (int et = 0; et < NE; ++et) dv[et] = mma(a, frag_col(ck.sDn, LV, 32 * ks + 8 * g4, 16 * et, l16), dv[et]);
        }
    }
    __syncthreads();
    // B^T over this wave's rows into sA (every read of A^T finished before the barrier);
    // dOut, dden are not read again as they are: their rows become 2^Lambda_i dnum_i and
    // 2^Lambda_i dden_i for the chunk's adjoint total
#pragma unroll
    for (int it = 0; it < NI; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) ck.sA[(j0 + 4 * g4 + r) * LA + 16 * it + l16] = X::from_f32(bt[it][r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = j0 + 4 * g4 + r;
        const float f = (GATED ? fast_exp2(lam_r[r]) : 1.0f) * ck.sInv[i];
#pragma unroll
        for (int et = 0; et < NE; ++et) {
            E& x = ck.sDn[i * LV + 16 * et + l16];
            x = X::from_f32(X::to_f32(x) * f);
        }
    }
    if (GATED && ck.tid < C) ck.sDd[ck.tid] *= fast_exp2(ck.lam(ck.tid));
    __syncthreads();

    // dFk = 2^(Lambda_last - Lambda_j) (V R^T + 1 r^T) + B^T Fq
    f32x4_t dfk[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) dfk[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DV / 32; ++ks) {
        const F8<E> a = frag_row(ck.sV, LV, j0 + l16, 32 * ks + 8 * g4);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) dfk[dt] = mma(a, frag_row(ck.sS, LV, 16 * dt + l16, 32 * ks + 8 * g4), dfk[dt]);
    }
    {
        float zk[4] = {0.f, 0.f, 0.f, 0.f};            // Fk_j . (carried-state part of dFk_j)
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const float rd = ck.sZ[16 * dt + l16];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dfk[dt][r] = (dfk[dt][r] + rd) * tail[r];
                if constexpr (GATED) zk[r] += X::to_f32(ck.sK[(j0 + 4 * g4 + r) * LQ + 16 * dt + l16]) * dfk[dt][r];
            }
        }
        if constexpr (GATED) {
            float kw = 0.0f;                           // K_c: this wave's part of sum_j zk_j
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float s = sum16(zk[r]);
                const int j = j0 + 4 * g4 + r;
                if (l16 == 0 && ts + j < N) args.zk[size_t(bh) * N + ts + j] = s;
                kw += s;
            }
            kw += __shfl_xor(kw, 16, kWave);
            kw += __shfl_xor(kw, 32, kWave);
            if (lane == 0) ck.sRow[1 + w] = kw;
        }
    }
    for (int ks = w >> 1; ks < C / 32; ++ks) {
        const F8<E> a = frag_row(ck.sA, LA, j0 + l16, 32 * ks + 8 * g4);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) dfk[dt] = mma(a, frag_col(ck.sQ, LQ, 32 * ks + 8 * g4, 16 * dt, l16), dfk[dt]);
    }
    // the adjoint carried across the chunk: R <- 2^Lambda_last R + Fq^T (2^Lambda dNum),
    // r <- 2^Lambda_last r + Fq^T (2^Lambda dden)
    const float fc = GATED ? fast_exp2(ck.lam(C - 1)) : 1.0f;
    {
#pragma unroll
        for (int u = 0; u < B::kStateUnits; ++u) {
            const int t = w + 4 * u, a = t / NE, b = t % NE;
            const f32x4_t dr = ck.tile_tn(ck.sQ, LQ, a, ck.sDn, LV, b);
#pragma unroll
            for (int k = 0; k < 4; ++k) racc[u][k] = fc * racc[u][k] + dr[k];
        }
        // the z part Fq^T (2^Lambda dden): every thread sums a slice of the rows of one
        // column, into sCol
        const int d = ck.tid % D, i0p = (ck.tid / D) * kRowsPer;
        float sr = 0.0f;
#pragma unroll
        for (int ii = 0; ii < kRowsPer; ++ii) sr += X::to_f32(ck.sQ[(i0p + ii) * LQ + d]) * ck.sDd[i0p + ii];
        ck.sCol[ck.tid] = sr;
    }
    // dk = dFk * phi'(k) and dv through the now free phi(K) and V tiles, stored coalesced
    __syncthreads();
    if (ck.tid < D) {
        float sr = 0.0f;
#pragma unroll
        for (int p = 0; p < kParts; ++p) sr += ck.sCol[p * D + ck.tid];
        rzacc = fc * rzacc + sr;
    }
    if constexpr (GATED) {
        // W_c = tb - K_c: keys in front of the chunk against queries after it
        const float wcv = tb - (ck.sRow[1] + ck.sRow[2] + ck.sRow[3] + ck.sRow[4]);
        if (ck.tid == 0) args.wc[size_t(bh) * NC + c] = wcv;
        tb = wcv + ck.sRow[0];
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
        {
            E& x = ck.sK[(j0 + 4 * g4 + r) * LQ + 16 * dt + l16];      // phi(k), read before it takes dk
            x = X::from_f32(dfk[dt][r] * dphi_of(X::to_f32(x)));
        }
#pragma unroll
    for (int et = 0; et < NE; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r) ck.sV[(j0 + 4 * g4 + r) * LV + 16 * et + l16] = X::from_f32(dv[et][r]);
    __syncthreads();
    ck.template store_out<D>(reinterpret_cast<E*>(args.dk) + size_t(bh) * N * D, ck.sK, LQ);
    ck.template store_out<DV>(reinterpret_cast<E*>(args.dv) + size_t(bh) * N * DV, ck.sV, LV);
    __syncthreads();                  // every read of this chunk's tiles is done
    }
}

// --------------------------------------------------------------- gate pass ----

// dg_l = (X_l + Y_l + Z_l + W_c) / g_l for token l of chunk c, one wave per chunk and
// one lane per token: Y_l = sum_{i >= l} yq_i and Z_l = sum_{j < l} zk_j within the chunk.
static __global__ __launch_bounds__(kThreads) void bwd_dg_kernel(const float* g, const float* xs, const float* yq,
                                                                const float* zk, const float* wc, float* dg, int N,
                                                                int NC, int nwork) {
    constexpr int C = kBwdChunk;
    static_assert(C == kWave, "one lane per token of a chunk");
    const int item = blockIdx.x * (kThreads / kWave) + int(threadIdx.x) / kWave;   // (head, chunk)
    if (item >= nwork) return;
    const int lane = threadIdx.x % kWave;
    const int bh = item / NC, c = item % NC;
    const int t = c * C + lane;
    const bool in = t < N;
    const size_t at = size_t(bh) * N + (in ? t : 0);
    const float x = in ? xs[at] : 0.0f, y = in ? yq[at] : 0.0f, z = in ? zk[at] : 0.0f;
    float ysuf = y, zpre = z;                     // inclusive suffix of y, inclusive prefix of z
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float a = __shfl_down(ysuf, off, kWave);
        const float b = __shfl_up(zpre, off, kWave);
        if (lane + off < kWave) ysuf += a;
        if (lane >= off) zpre += b;
    }
    if (in) dg[at] = (x + ysuf + (zpre - z) + wc[size_t(bh) * NC + c]) / g[at];
}

}  // namespace linattn
