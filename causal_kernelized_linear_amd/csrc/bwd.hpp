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
//
// Precision (bf16 where the LDS holds the extra tiles, BwdShape::kSplit).  Operands that
// are not exact bf16 inputs go to the MFMA products as two bf16 parts, x = hi + lo with
// hi = bf16(x), lo = bf16(x - hi), and a product takes hi hi + lo hi + hi lo: the
// features phi(Q), phi(K) in every product, the staged state (S in the dq pass, R in the
// dk/dv pass), the scaled rows of the state steps, and A and B where the denominators
// can be small (the sequence's first chunk; every chunk when gated).  The totals walk
// that gives the states in front of the runs splits phi(K) the same way.  Rounded once,
// each of these alone leaves a gradient row error of 5e-3 to 8e-3 at 4096 tokens (a CPU
// model of the passes), which add up to 1.2e-2; split, dq and dk come to about 4e-3.
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
// adjoint totals in reverse order.
//
// Layout.  The chunk's rows (phi(Q), phi(K), V, dOut) and one state are staged in LDS as
// row-major tiles; an operand whose contraction index runs down a tile's rows is read
// with ds_read_b64_tr_b16 (bf16) or element by element (fp32).  The [C][C] score tiles
// never go to LDS: each wave computes them transposed (lane l16 owning one of its own
// rows, four consecutive partners per lane group), which is exactly the operand layout of
// the 16x16x16 MFMA that consumes them; the outputs come out transposed the same way and
// go to memory as four consecutive columns per lane.  Sums that would take a loop over
// the chunk (den's z part, the z vectors of the state steps) ride on the 16-byte pad
// group of each row as two extra columns, an fp32 value split into a bf16 high and low
// part, so they come out of the MFMA products that run anyway.
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
    float* fst;          // [BH][FS][D*Dv] accumulator layout: slot t < FS-1 holds the state after
                         // part t % FP of run t / FP (the state after run r: slot (r+1) FP - 1)
    float* fzt;          // [BH][FS][D]
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
    int FP;              // parts each run's forward total is walked in (by separate workgroups)
    int FS;              // forward state slots per head, (NR - 1) FP + 1
    float eps;
    int normalize;
};

constexpr int kBwdChunk = kBwdChunkHost;

template <typename E, int D, int DV>
struct BwdShape {
    static constexpr int C = kBwdChunk;
    static constexpr int PAD = 16 / int(sizeof(E));   // one 16-byte group per row
    static constexpr int LQ = D + PAD;                 // phi(Q), phi(K) [C][D]
    static constexpr int LV = DV + PAD;                // V, dOut [C][Dv]; S_prev / R [D][Dv]
    static constexpr size_t kOffQ = 0;
    static constexpr size_t kOffK = kOffQ + size_t(C) * LQ * sizeof(E);
    static constexpr size_t kOffV = kOffK + size_t(C) * LQ * sizeof(E);
    static constexpr size_t kOffDn = kOffV + size_t(C) * LV * sizeof(E);
    static constexpr size_t kOffS = kOffDn + size_t(C) * LV * sizeof(E);
    static constexpr size_t kOffLam = kOffS + size_t(D) * LV * sizeof(E);
    static constexpr size_t kOffDd = kOffLam + size_t(C) * 4;
    static constexpr size_t kOffInv = kOffDd + size_t(C) * 4;
    static constexpr size_t kOffCol = kOffInv + size_t(C) * 4;     // [4][C] per-wave column sums of P
    static constexpr size_t kOffRow = kOffCol + size_t(4) * C * 4;  // [C] row sums of P
    static constexpr size_t kOffZ = kOffRow + size_t(C) * 4;
    // bf16 where the LDS allows (bwd_split): the low parts of phi(Q), phi(K) and of the
    // staged state, each operand x going to the products as bf16(x) and bf16(x - bf16(x))
    static constexpr bool kSplit = bwd_split(int(sizeof(E)), D, DV);
    static constexpr size_t kOffQlo = kOffZ + size_t(D) * 4;
    static constexpr size_t kOffKlo = kOffQlo + (kSplit ? size_t(C) * LQ * sizeof(E) : 0);
    static constexpr size_t kOffSlo = kOffKlo + (kSplit ? size_t(C) * LQ * sizeof(E) : 0);
    static constexpr size_t kBytes = kOffSlo + (kSplit ? size_t(D) * LV * sizeof(E) : 0);
    static_assert(kBytes == bwd_lds_bytes(int(sizeof(E)), D, DV), "host LDS formula out of step");
    static_assert(PAD >= 2, "the pad group carries two extra columns");
    // An extra 16-column operand block at column Dv reads the pad group and then, past it,
    // the start of the next row (or, for a tile's last row, the next region: the next
    // tile, or the fp32 vectors after S); those columns only feed output rows or columns
    // that are thrown away.  Every tile is followed by at least that much LDS.
    static_assert(kOffLam + size_t(16) * 4 <= kBytes, "room behind S for the extra block");
    // workgroups (so waves per SIMD) the LDS allows: the register target of both kernels,
    // so the compiler does not squeeze the accumulators for an occupancy out of reach
    static constexpr int kWaves = int(kMaxLds / kBytes) < 1 ? 1 : int(kMaxLds / kBytes);
    // 16-byte pieces per thread of a state in accumulator layout, and of one chunk's four
    // row tiles.  Loading the next chunk's rows during this chunk's products keeps them
    // live across the products, beside the two carried states: done where all of it stays
    // within 32 pieces (128 registers) and at most two workgroups share a CU; at three,
    // the other workgroups hide the loads as well and the registers are better spent
    // (measured equal or faster without).
    static constexpr int kStateUnits = D * DV / 4 / kThreads;
    static constexpr int kRowPieces = (2 * C * D + 2 * C * DV) * int(sizeof(E)) / 16 / kThreads;
    static constexpr bool kAhead = kWaves <= 2 && kRowPieces + 2 * kStateUnits <= 32;
    // Whether the lane indices are made opaque once per chunk (BwdChunk::refresh): with
    // the larger tiles, addresses hoisted out of the chunk loop spill; at D = Dv = 64 bf16
    // they fit (three workgroups per CU before the split operands' tiles, two with them,
    // 218-230 VGPRs) and save VALU instructions (train_bf16 backward 4% faster).
    static constexpr bool kOpaqueLanes = !(sizeof(E) == 2 && D == 64 && DV == 64) && kWaves < 3;
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
typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i16x4_t tr_read(const uint16_t* t, int ld, int k0, int n0, int l16) {
    typedef __attribute__((address_space(3))) i16x4_t* lds_ptr_t;
    const uint16_t* p = t + (k0 + (l16 >> 2)) * ld + n0 + 4 * (l16 & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr_t)(const_cast<uint16_t*>(p)));
}

__device__ __forceinline__ F8<uint16_t> frag_col(const uint16_t* t, int ld, int k0, int n0, int l16) {
    const i16x4_t a = tr_read(t, ld, k0, n0, l16), b = tr_read(t, ld, k0 + 4, n0, l16);
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

// The same with four contraction slots, for the 16x16x16 product: slot e of lane l holds
// t[k0 + e][n0 + l % 16].
__device__ __forceinline__ F4<uint16_t> frag4_col(const uint16_t* t, int ld, int k0, int n0, int l16) {
    return __builtin_bit_cast(F4<uint16_t>, tr_read(t, ld, k0, n0, l16));
}

__device__ __forceinline__ F4<float> frag4_col(const float* t, int ld, int k0, int n0, int l16) {
    F4<float> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f.x[e] = t[(k0 + e) * ld + n0 + l16];
    return f;
}

// One 16x16 output tile step over 16 values of the contraction index: lane l supplies
// row l % 16 of A and column l % 16 of B with the four slots of lane group l / 16
// (contraction index 4 (l / 16) + slot); the accumulator layout is mma's.  bf16: one
// v_mfma_f32_16x16x16_bf16; float: four v_mfma_f32_16x16x4_f32, slot s feeding step s.
__device__ __forceinline__ f32x4_t mma4(const F4<uint16_t>& a, const F4<uint16_t>& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b),
                                                     c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mma4(const F4<float>& a, const F4<float>& b, f32x4_t c) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x[s], b.x[s], c, 0, 0, 0);
    return c;
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

// Column 0 plus column 1 of an accumulator row, in lanes l16 = 0 and 1 (the high and low
// parts of a split value).
__device__ __forceinline__ float pair01(float x) { return x + dpp_move<0xB1>(x); }

// Sum over the four lane groups (every lane getting the sum for its l16).
__device__ __forceinline__ float sum_groups(float x) {
    x += __shfl_xor(x, 16, kWave);
    x += __shfl_xor(x, 32, kWave);
    return x;
}

// The derivative of elu + 1 from its value: phi'(x) = 1 above zero, where phi(x) = x + 1 > 1,
// and exp(x) = phi(x) at or below zero, so phi'(x) = min(phi(x), 1).  Taken from the staged
// features (in the input precision), it adds one rounding of the size of the output's own.
__device__ __forceinline__ float dphi_of(float f) { return fminf(f, 1.0f); }

template <typename E>
__device__ __forceinline__ F4<E> pack4(const f32x4_t& c) {
    F4<E> f;
#pragma unroll
    for (int r = 0; r < 4; ++r) f.x[r] = Elem<E>::from_f32(c[r]);
    return f;
}

template <typename E>
__device__ __forceinline__ f32x4_t unpack4(const F4<E>& f) {
    f32x4_t c;
#pragma unroll
    for (int r = 0; r < 4; ++r) c[r] = Elem<E>::to_f32(f.x[r]);
    return c;
}

// A 16-byte pad group holding x split as (high, low) in operand precision, then zeros.
template <typename E>
__device__ __forceinline__ f32x4_t split_pad(float x) {
    using X = Elem<E>;
    F8<E> o{};
    constexpr int EPG = 16 / int(sizeof(E));
    E h = X::from_f32(x);
    E lo = X::from_f32(x - X::to_f32(h));
    if constexpr (EPG == 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o.x[e] = E(0);
        o.x[0] = h;
        o.x[1] = lo;
        return __builtin_bit_cast(f32x4_t, o);
    } else {
        return f32x4_t{X::to_f32(h), X::to_f32(lo), 0.0f, 0.0f};
    }
}

// The per-workgroup machinery shared by both gradient kernels.
template <typename E, int D, int DV, bool GATED>
struct BwdChunk {
    using Sh = BwdShape<E, D, DV>;
    using X = Elem<E>;
    static constexpr int C = Sh::C, LQ = Sh::LQ, LV = Sh::LV;
    static constexpr int EPG = 16 / int(sizeof(E));       // elements per 16-byte group
    static constexpr int KZ = D / 64;                      // 16-row z tiles per wave (tiles w, w + 4, ...)

    E* sQ;
    E* sK;
    E* sV;
    E* sDn;
    E* sS;
    E* sQlo;       // split operands (Sh::kSplit): low parts of phi(Q), phi(K) and the state
    E* sKlo;
    E* sSlo;
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
        sQlo = reinterpret_cast<E*>(smem + Sh::kOffQlo);
        sKlo = reinterpret_cast<E*>(smem + Sh::kOffKlo);
        sSlo = reinterpret_cast<E*>(smem + Sh::kOffSlo);
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

    // The lane indices made opaque at the top of every chunk (where the shape asks for
    // it): the compiler then rebuilds the many LDS addresses derived from them inside the
    // chunk loop instead of hoisting them all out of it and holding them in registers
    // across the products.
    __device__ __forceinline__ void refresh() {
        if constexpr (Sh::kOpaqueLanes) asm volatile("" : "+v"(tid), "+v"(lane), "+v"(l16), "+v"(g4));
    }

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
    // chunk's end become zero.  LO (bf16 phi only): the low parts phi - bf16(phi) into
    // `lo`, laid out like the tile.
    template <int W, bool PHI, bool LO = false>
    __device__ __forceinline__ void store_rows(E* tile, int ld, const f32x4_t (&r)[kRowUnits<W>], E* lo = nullptr) const {
        static_assert(!LO || (PHI && sizeof(E) == 2), "low parts: bf16 features only");
        constexpr int G = W * int(sizeof(E)) / 16;
#pragma unroll
        for (int u = 0; u < kRowUnits<W>; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = (idx % G) * EPG;
            f32x4_t out = {0.f, 0.f, 0.f, 0.f}, out_lo = {0.f, 0.f, 0.f, 0.f};
            if (row < nrows) {
                if constexpr (sizeof(E) == 2) {
                    const F8<E> in = __builtin_bit_cast(F8<E>, r[u]);
                    F8<E> o, ol;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if constexpr (PHI) {
                            const float f = phi(X::to_f32(in.x[e]));
                            o.x[e] = X::from_f32(f);
                            if constexpr (LO) ol.x[e] = X::from_f32(f - X::to_f32(o.x[e]));
                        } else {
                            o.x[e] = in.x[e];
                        }
                    }
                    out = __builtin_bit_cast(f32x4_t, o);
                    if constexpr (LO) out_lo = __builtin_bit_cast(f32x4_t, ol);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = PHI ? phi(r[u][e]) : r[u][e];
                }
            }
            *reinterpret_cast<f32x4_t*>(tile + row * ld + col) = out;
            if constexpr (LO) *reinterpret_cast<f32x4_t*>(lo + row * ld + col) = out_lo;
        }
    }

    // Four consecutive staged features (element offset `at` of a phi tile), with their low
    // parts added back where the operands are split.
    __device__ __forceinline__ f32x4_t feat4(const E* hi, const E* lo, int at) const {
        f32x4_t f = unpack4(lds_f4(hi + at));
        if constexpr (Sh::kSplit) f += unpack4(lds_f4(lo + at));
        return f;
    }

    // The pad group of row `row` of a tile with `ld` = width + PAD.
    __device__ __forceinline__ f32x4_t* pad_of(E* tile, int ld, int width, int row) const {
        return reinterpret_cast<f32x4_t*>(tile + row * ld + width);
    }

    // A state slot in accumulator layout: D * Dv / 4 16-byte pieces per workgroup.
    static constexpr int kStateUnits = Sh::kStateUnits;

    __device__ __forceinline__ void load_slot(f32x4_t (&r)[kStateUnits], const float* slot) const {
#pragma unroll
        for (int u = 0; u < kStateUnits; ++u) r[u] = *reinterpret_cast<const f32x4_t*>(slot + 4 * (tid + u * kThreads));
    }

    // ... into sS (row-major [D][Dv], operand precision); split (Sh::kSplit), the low
    // parts into sSlo.
    __device__ __forceinline__ void store_slot(const f32x4_t (&r)[kStateUnits]) const {
#pragma unroll
        for (int u = 0; u < kStateUnits; ++u) {
            const int q4 = tid + u * kThreads;
            const int t = q4 / kWave, ln = q4 % kWave;
            const int a = t / (DV / 16), b = t % (DV / 16);
            const int d = 16 * a + 4 * (ln >> 4), e = 16 * b + (ln & 15);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const E h = X::from_f32(r[u][k]);
                sS[(d + k) * LV + e] = h;
                if constexpr (Sh::kSplit) sSlo[(d + k) * LV + e] = X::from_f32(r[u][k] - X::to_f32(h));
            }
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

    // A [D] vector in the z-holder lanes: lane l16 = 0 of group g4 in wave w holds entries
    // 16 (w + 4 t) + 4 g4 + r of tile t < KZ (zero elsewhere).
    __device__ __forceinline__ void load_zvec(float (&z)[KZ][4], const float* src) const {
#pragma unroll
        for (int t = 0; t < KZ; ++t) {
            const f32x4_t v = (src && l16 == 0) ? *reinterpret_cast<const f32x4_t*>(src + 16 * (w + 4 * t) + 4 * g4)
                                                : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) z[t][r] = v[r];
        }
    }

    __device__ __forceinline__ void put_zvec(float* dst, const float (&z)[KZ][4]) const {
        if (l16 == 0) {
#pragma unroll
            for (int t = 0; t < KZ; ++t)
                *reinterpret_cast<f32x4_t*>(dst + 16 * (w + 4 * t) + 4 * g4) = f32x4_t{z[t][0], z[t][1], z[t][2], z[t][3]};
        }
    }

    // One 16x16 state tile, contraction over the chunk's rows: lhs^T rhs for the tile's
    // rows a and columns b of two row-major tiles (this lane's accumulator piece).
    __device__ __forceinline__ f32x4_t tile_tn(const E* lhs, int ldl, int a, const E* rhs, int ldr, int b,
                                               f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f}) const {
#pragma unroll
        for (int ks = 0; ks < C / 32; ++ks)
            acc = mma(frag_col(lhs, ldl, 32 * ks + 8 * g4, 16 * a, l16), frag_col(rhs, ldr, 32 * ks + 8 * g4, 16 * b, l16),
                      acc);
        return acc;
    }

    // The state steps' products with split operands (Sh::kSplit): lhs^T rhs with the
    // low parts lhs_lo of lhs and, unless null, rhs_lo of rhs (hi hi + lo hi + hi lo).
    // rhs_lo has no pad group: for the extra column block (b = DV / 16) it is skipped.
    __device__ __forceinline__ f32x4_t tile_tn_split(const E* lhs, const E* lhs_lo, int ldl, int a, const E* rhs,
                                                     const E* rhs_lo, int ldr, int b) const {
        if constexpr (!Sh::kSplit) {
            return tile_tn(lhs, ldl, a, rhs, ldr, b);
        } else {
            const bool rlo = rhs_lo != nullptr && b < DV / 16;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C / 32; ++ks) {
                const int k0 = 32 * ks + 8 * g4;
                const F8<E> l = frag_col(lhs, ldl, k0, 16 * a, l16), r = frag_col(rhs, ldr, k0, 16 * b, l16);
                acc = mma(l, r, acc);
                acc = mma(frag_col(lhs_lo, ldl, k0, 16 * a, l16), r, acc);
                if (rlo) acc = mma(l, frag_col(rhs_lo, ldr, k0, 16 * b, l16), acc);
            }
            return acc;
        }
    }

    // Rows of dOut scaled by 2^Lambda_i / d_i and their pad groups set to the split
    // 2^Lambda_i dden_i (sDd holds dden_i, times 2^Lambda_i if DD_DECAYED), for the
    // chunk's adjoint total; with V, rows scaled by 2^(Lambda_last - Lambda_j) and the pad
    // to the split factor, for the state step.
    // Split (Sh::kSplit): the low parts of the scaled dOut rows go to dn_lo and those of
    // the scaled V rows (gated, WITH_V) to v_lo, both laid out like sDn (no pad group).
    template <bool WITH_V, bool DD_DECAYED>
    __device__ __forceinline__ void scale_rows(E* dn_lo = nullptr, E* v_lo = nullptr) const {
        constexpr int G = DV * int(sizeof(E)) / 16 + 1;    // groups per row, pad included
        const float lam_last = lam(C - 1);
        for (int idx = tid; idx < C * G; idx += kThreads) {
            const int row = idx / G, gi = idx % G;
            const float fl = GATED ? fast_exp2(lam(row)) : 1.0f;
            if (gi < G - 1) {
                f32x4_t* p = reinterpret_cast<f32x4_t*>(sDn + row * LV + gi * EPG);
                if constexpr (Sh::kSplit)
                    *p = scale16(*p, fl * sInv[row], reinterpret_cast<f32x4_t*>(dn_lo + row * LV + gi * EPG));
                else
                    *p = scale16(*p, fl * sInv[row]);
            } else {
                *pad_of(sDn, LV, DV, row) = split_pad<E>(DD_DECAYED ? sDd[row] : sDd[row] * fl);
            }
            if constexpr (WITH_V && GATED) {
                const float fv = fast_exp2(fminf(lam_last - lam(row), 0.0f));
                if (gi < G - 1) {
                    f32x4_t* p = reinterpret_cast<f32x4_t*>(sV + row * LV + gi * EPG);
                    if constexpr (Sh::kSplit)
                        *p = scale16(*p, fv, reinterpret_cast<f32x4_t*>(v_lo + row * LV + gi * EPG));
                    else
                        *p = scale16(*p, fv);
                } else {
                    *pad_of(sV, LV, DV, row) = split_pad<E>(row < nrows ? fv : 0.0f);
                }
            }
        }
    }

    // 16 bytes of elements times f, rounded to the operand type; with lo (bf16), the
    // rounding's remainder bf16(x f - bf16(x f)) goes there.
    static __device__ __forceinline__ f32x4_t scale16(f32x4_t v, float f, f32x4_t* lo = nullptr) {
        if constexpr (sizeof(E) == 2) {
            F8<E> x = __builtin_bit_cast(F8<E>, v), xl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y = X::to_f32(x.x[e]) * f;
                x.x[e] = X::from_f32(y);
                xl.x[e] = X::from_f32(y - X::to_f32(x.x[e]));
            }
            if (lo != nullptr) *lo = __builtin_bit_cast(f32x4_t, xl);
            return __builtin_bit_cast(f32x4_t, x);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= f;
            return v;
        }
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
                sLam[lane] = wave_incl_scan(lane < nrows ? fast_log2(gv) : 0.0f);
            }
        }
    }

    __device__ __forceinline__ float lam(int i) const {
        if constexpr (GATED) return sLam[i];
        return 0.0f;
    }

    // Lambda of rows i .. i + 3 (i a multiple of 4).
    __device__ __forceinline__ f32x4_t lam4(int i) const {
        if constexpr (GATED) return *reinterpret_cast<const f32x4_t*>(sLam + i);
        return f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
};

// Four consecutive elements out to memory (8 bytes bf16, 16 bytes fp32).
template <typename E>
__device__ __forceinline__ void store4(E* p, const f32x4_t& v) {
    *reinterpret_cast<F4<E>*>(p) = pack4<E>(v);
}

// ----------------------------------------------------------------- dq pass ----

template <typename E, int D, int DV, bool GATED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BwdShape<E, D, DV>::kWaves,
                                                                           BwdShape<E, D, DV>::kWaves)))
void bwd_dq_kernel(BwdArgs args) {
    using B = BwdChunk<E, D, DV, GATED>;
    using X = Elem<E>;
    constexpr int C = B::C, LQ = B::LQ, LV = B::LV, KZ = B::KZ;
    constexpr int ND = D / 16, NE = DV / 16, NJ = C / 16;
    constexpr bool kSplit = B::Sh::kSplit;
    extern __shared__ __align__(16) unsigned char smem[];
    B ck;
    ck.init(smem, args.N, args.NC, args.LC);
    const int w = ck.w, bh = ck.bh;
    const int N = args.N;
    const E* qb = reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D;
    const E* kb = reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D;
    const E* vb = reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV;
    const E* dob = reinterpret_cast<const E*>(args.dout) + size_t(bh) * N * DV;
    E* dqb = reinterpret_cast<E*>(args.dq) + size_t(bh) * N * D;

    // The state in front of the current chunk, carried through the run in fp32 (this
    // thread's accumulator-layout pieces; z in the z-holder lanes): from the scanned slot
    // in front of the run, or S0 / z0 for the first run.
    f32x4_t sacc[B::kStateUnits];
    float zv[KZ][4];
    if (ck.run > 0) {
        const size_t fslot = size_t(bh) * args.FS + (size_t(ck.run) * args.FP - 1);
        ck.load_slot(sacc, args.fst + fslot * (D * DV));
        ck.load_zvec(zv, args.fzt + fslot * D);
    } else {
        ck.load_user(sacc, args.s0 ? args.s0 + size_t(bh) * D * DV : nullptr);
        ck.load_zvec(zv, args.z0 ? args.z0 + size_t(bh) * D : nullptr);
    }
    // The run's adjoint total (what its queries pass to the state in front of it): the sum
    // over its chunks of the chunk's adjoint total times the decay from the run's start to
    // the chunk's start, 2^logp.
    f32x4_t racc[B::kStateUnits];
#pragma unroll
    for (int u = 0; u < B::kStateUnits; ++u) racc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float rzv[KZ][4] = {};
    float logp = 0.0f;

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
    ck.template store_rows<D, true, kSplit>(ck.sQ, LQ, sq, ck.sQlo);
    ck.template store_rows<D, true, kSplit>(ck.sK, LQ, sk, ck.sKlo);
    ck.template store_rows<DV, false>(ck.sV, LV, sv);
    ck.template store_rows<DV, false>(ck.sDn, LV, so);
    ck.store_slot(sacc);
    if (l16 == 0) {
        // z_prev into sZ and, split, into the state's pad columns (den's z part)
#pragma unroll
        for (int t = 0; t < KZ; ++t) {
            const int d0 = 16 * (w + 4 * t) + 4 * g4;
            *reinterpret_cast<f32x4_t*>(ck.sZ + d0) = f32x4_t{zv[t][0], zv[t][1], zv[t][2], zv[t][3]};
#pragma unroll
            for (int r = 0; r < 4; ++r) *ck.pad_of(ck.sS, LV, DV, d0 + r) = split_pad<E>(zv[t][r]);
        }
    }
    if (ck.tid < C) {
        // V's pad: a column of ones (the row sums of A come out of A V), then zeros
        *ck.pad_of(ck.sV, LV, DV, ck.tid) = split_pad<E>(ck.tid < ck.nrows ? 1.0f : 0.0f);
    }
    ck.stage_lambda(sg);
    __syncthreads();
    if (B::Sh::kAhead && c + 1 < ck.c_end) issue(c + 1);

    // This lane's query row of the wave's transposed tiles, and its decay.
    const int i0 = 16 * w, il = i0 + l16;
    const float lam_i = ck.lam(il), f_i = GATED ? fast_exp2(lam_i) : 1.0f;

    // A, transposed: lane (l16, g4) holds query il against keys 16 jt + 4 g4 + r.  sc keeps
    // the undecayed fp32 scores for the pair sums of d log g.
    f32x4_t sc[NJ];
    F4<E> pa[NJ], pa_lo[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) sc[jt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        const F8<E> bq = frag_row(ck.sQ, LQ, il, 32 * ks + 8 * g4);
        F8<E> bql;
        if constexpr (kSplit) bql = frag_row(ck.sQlo, LQ, il, 32 * ks + 8 * g4);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt)
            if (jt <= w) {
                const F8<E> kf = frag_row(ck.sK, LQ, 16 * jt + l16, 32 * ks + 8 * g4);
                sc[jt] = mma(kf, bq, sc[jt]);
                if constexpr (kSplit) {
                    sc[jt] = mma(kf, bql, sc[jt]);
                    sc[jt] = mma(frag_row(ck.sKlo, LQ, 16 * jt + l16, 32 * ks + 8 * g4), bq, sc[jt]);
                }
            }
    }
    // where the denominators can be small (the sequence's first chunk, with no state in
    // front; every chunk when gated, whose decay keeps the state short) the products also
    // take the low parts of A and B
    const bool first = kSplit && (GATED || c == 0);
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        const f32x4_t lj = ck.lam4(16 * jt + 4 * g4);
        f32x4_t x;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * jt + 4 * g4 + r;
            x[r] = (jt <= w && j <= il) ? sc[jt][r] : 0.0f;
            if constexpr (GATED) x[r] *= fast_exp2(fminf(lam_i - lj[r], 0.0f));
        }
        pa[jt] = pack4<E>(x);
        if constexpr (kSplit) pa_lo[jt] = pack4<E>(x - unpack4(pa[jt]));
    }

    // num^T[e][i] = 2^Lambda_i (S^T Fq^T)[e][i] + (V^T A^T)[e][i], with one extra block of
    // rows e = Dv, Dv + 1 holding den's parts (S's pad: z split; V's pad: 1, 0)
    f32x4_t nt[NE + 1];
#pragma unroll
    for (int et = 0; et <= NE; ++et) nt[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        const F8<E> bq = frag_row(ck.sQ, LQ, il, 32 * ks + 8 * g4);
        F8<E> bql;
        if constexpr (kSplit) bql = frag_row(ck.sQlo, LQ, il, 32 * ks + 8 * g4);
#pragma unroll
        for (int et = 0; et <= NE; ++et) {
            const F8<E> sf = frag_col(ck.sS, LV, 32 * ks + 8 * g4, 16 * et, l16);
            nt[et] = mma(sf, bq, nt[et]);
            if constexpr (kSplit) {
                // S Fq_lo (z's split pad included) and S_lo Fq (S_lo has no pad group:
                // the extra block skips it)
                nt[et] = mma(sf, bql, nt[et]);
                if (et < NE) nt[et] = mma(frag_col(ck.sSlo, LV, 32 * ks + 8 * g4, 16 * et, l16), bq, nt[et]);
            }
        }
    }
    if constexpr (GATED) {
#pragma unroll
        for (int et = 0; et <= NE; ++et)
#pragma unroll
            for (int r = 0; r < 4; ++r) nt[et][r] *= f_i;
    }
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
        if (jt <= w) {
#pragma unroll
            for (int et = 0; et <= NE; ++et) {
                const F4<E> vf = frag4_col(ck.sV, LV, 16 * jt + 4 * g4, 16 * et, l16);
                nt[et] = mma4(vf, pa[jt], nt[et]);
                if constexpr (kSplit) {
                    if (first) nt[et] = mma4(vf, pa_lo[jt], nt[et]);
                }
            }
        }

    // den (in lanes g4 = 0: rows Dv and Dv + 1 of the extra block), 1/d and
    // dden = -(dout . num) / d^2 in fp32; dnum = dout / d stays implicit
    const float den = __shfl(nt[NE][0] + nt[NE][1], l16, kWave);
    const float inv = args.normalize ? 1.0f / fmaxf(den, args.eps) : 1.0f;
    float dd;
    {
        float dsum = 0.0f;
#pragma unroll
        for (int et = 0; et < NE; ++et) {
            const F4<E> o4 = lds_f4(ck.sDn + il * LV + 16 * et + 4 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) dsum += X::to_f32(o4.x[r]) * nt[et][r];
        }
        dsum = sum_groups(dsum);
        dd = (args.normalize && den >= args.eps) ? -dsum * inv * inv : 0.0f;
        if (g4 == 0) {
            if (ts + il < N) {
                args.dden[size_t(bh) * N + ts + il] = dd;
                args.inv[size_t(bh) * N + ts + il] = inv;
            }
            ck.sInv[il] = inv;
            ck.sDd[il] = dd * f_i;
        }
    }

    // B, transposed like A: ((dout_i . v_j) / d_i + dden_i) decayed and masked; with it the
    // pair terms P_ij = (Fq_i . Fk_j) B_ij in fp32, summed by row (j < i) and by column
    F4<E> pb[NJ], pb_lo[NJ];
    float prow = 0.0f;
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        f32x4_t bt = {0.f, 0.f, 0.f, 0.f};
        if (jt <= w) {
#pragma unroll
            for (int ks = 0; ks < DV / 32; ++ks)
                bt = mma(frag_row(ck.sV, LV, 16 * jt + l16, 32 * ks + 8 * g4), frag_row(ck.sDn, LV, il, 32 * ks + 8 * g4),
                         bt);
        }
        const f32x4_t lj = ck.lam4(16 * jt + 4 * g4);
        f32x4_t x, pc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * jt + 4 * g4 + r;
            x[r] = (jt <= w && j <= il) ? bt[r] * inv + dd : 0.0f;
            if constexpr (GATED) {
                x[r] *= fast_exp2(fminf(lam_i - lj[r], 0.0f));
                const float p = (jt <= w && j < il) ? sc[jt][r] * x[r] : 0.0f;
                prow += p;
                pc[r] = sum16(p);
            }
        }
        pb[jt] = pack4<E>(x);
        if constexpr (kSplit) pb_lo[jt] = pack4<E>(x - unpack4(pb[jt]));
        if constexpr (GATED) {
            if (l16 == 0) *reinterpret_cast<f32x4_t*>(ck.sCol + w * C + 16 * jt + 4 * g4) = pc;
        }
    }
    if constexpr (GATED) {
        prow = sum_groups(prow);
        if (g4 == 0) ck.sRow[il] = prow;
    }

    // dFq^T[d][i] = 2^Lambda_i ((S dOut^T)[d][i] / d_i + z_d dden_i) + (Fk^T B^T)[d][i]
    f32x4_t ft[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
        ft[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DV / 32; ++ks) {
            const F8<E> bo = frag_row(ck.sDn, LV, il, 32 * ks + 8 * g4);
            ft[dt] = mma(frag_row(ck.sS, LV, 16 * dt + l16, 32 * ks + 8 * g4), bo, ft[dt]);
            if constexpr (kSplit) ft[dt] = mma(frag_row(ck.sSlo, LV, 16 * dt + l16, 32 * ks + 8 * g4), bo, ft[dt]);
        }
    }
    {
        float yq = 0.0f;                              // Fq_i . (carried-state part of dFq_i)
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const f32x4_t z4 = *reinterpret_cast<const f32x4_t*>(ck.sZ + 16 * dt + 4 * g4);
            const F4<E> q4 = lds_f4(ck.sQ + il * LQ + 16 * dt + 4 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ft[dt][r] = (ft[dt][r] * inv + dd * z4[r]) * f_i;
                if constexpr (GATED) yq += X::to_f32(q4.x[r]) * ft[dt][r];
            }
        }
        if constexpr (GATED) {
            yq = sum_groups(yq);
            if (g4 == 0 && ts + il < N) args.yq[size_t(bh) * N + ts + il] = yq;
        }
    }
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
        if (jt <= w) {
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const F4<E> kf = frag4_col(ck.sK, LQ, 16 * jt + 4 * g4, 16 * dt, l16);
                ft[dt] = mma4(kf, pb[jt], ft[dt]);
                if constexpr (kSplit) {
                    ft[dt] = mma4(frag4_col(ck.sKlo, LQ, 16 * jt + 4 * g4, 16 * dt, l16), pb[jt], ft[dt]);
                    if (first) ft[dt] = mma4(kf, pb_lo[jt], ft[dt]);
                }
            }
        }
    // dq = dFq * phi'(q): four consecutive columns of row il per lane
    if (ts + il < N) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const f32x4_t f4 = ck.feat4(ck.sQ, ck.sQlo, il * LQ + 16 * dt + 4 * g4);
            f32x4_t o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = ft[dt][r] * dphi_of(f4[r]);
            store4<E>(dqb + size_t(ts + il) * D + 16 * dt + 4 * g4, o);
        }
    }
    __syncthreads();
    // X_l = sum_{m < l} (col_m - row_m): the pairs inside the chunk with j < l <= i
    if (GATED && w == 0) {
        const float dm = ck.sCol[lane] + ck.sCol[C + lane] + ck.sCol[2 * C + lane] + ck.sCol[3 * C + lane] -
                         ck.sRow[lane];
        const float x = wave_incl_scan(dm);
        if (lane < ck.nrows) args.xs[size_t(bh) * N + ts + lane] = x - dm;
    }
    // rows of dOut become 2^Lambda_i dnum_i (pad: 2^Lambda_i dden_i split), rows of V
    // 2^(Lambda_last - Lambda_j) v_j (pad: the factor split, for z's step).  Split: their
    // low parts go where the state's tiles were (read for the last time above).
    E* const dn_lo = kSplit ? ck.sSlo : nullptr;
    E* const v_lo = kSplit && GATED ? ck.sS : nullptr;
    ck.template scale_rows<true, true>(dn_lo, v_lo);
    __syncthreads();
    // The chunk's adjoint total dR_c = Fq^T (2^Lambda dNum), dr_c = Fq^T (2^Lambda dden),
    // into the run's with the decay 2^logp from the run's start; and the state carried
    // across the chunk: S <- 2^Lambda_last S + Fk^T (2^(Lambda_last - Lambda_j) V), z alike.
    // The z parts are the extra column block (pad columns 0 + 1) of the same products.
    {
        const float lam_last = ck.lam(C - 1);
        const float fp = GATED ? fast_exp2(logp) : 1.0f, fc = GATED ? fast_exp2(lam_last) : 1.0f;
#pragma unroll
        for (int u = 0; u < B::kStateUnits; ++u) {
            const int t = w + 4 * u, a = t / NE, b = t % NE;
            const f32x4_t dr = ck.tile_tn_split(ck.sQ, ck.sQlo, LQ, a, ck.sDn, dn_lo, LV, b);
            const f32x4_t ds = ck.tile_tn_split(ck.sK, ck.sKlo, LQ, a, ck.sV, v_lo, LV, b);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                racc[u][k] += fp * dr[k];
                sacc[u][k] = fc * sacc[u][k] + ds[k];
            }
        }
#pragma unroll
        for (int t = 0; t < KZ; ++t) {
            const f32x4_t dr = ck.tile_tn_split(ck.sQ, ck.sQlo, LQ, w + 4 * t, ck.sDn, nullptr, LV, NE);
            const f32x4_t ds = ck.tile_tn_split(ck.sK, ck.sKlo, LQ, w + 4 * t, ck.sV, nullptr, LV, NE);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                rzv[t][r] += fp * pair01(dr[r]);
                zv[t][r] = fc * zv[t][r] + pair01(ds[r]);
            }
        }
        logp += lam_last;
    }
    __syncthreads();                  // every read of this chunk's tiles is done
    }

    // the run's adjoint total at its reversed slot
    const size_t rslot = size_t(bh) * (args.NR + 1) + (args.NR - 1 - ck.run);
    ck.put_slot(args.rst + rslot * (D * DV), racc);
    ck.put_zvec(args.rzt + rslot * D, rzv);
    if (GATED && ck.tid == 0) args.rlg[rslot] = logp;
}

// ------------------------------------------------------------ dk / dv pass ----

template <typename E, int D, int DV, bool GATED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BwdShape<E, D, DV>::kWaves,
                                                                           BwdShape<E, D, DV>::kWaves)))
void bwd_dkv_kernel(BwdArgs args) {
    using B = BwdChunk<E, D, DV, GATED>;
    using X = Elem<E>;
    constexpr int C = B::C, LQ = B::LQ, LV = B::LV, KZ = B::KZ;
    constexpr int ND = D / 16, NE = DV / 16, NI = C / 16;
    constexpr bool kSplit = B::Sh::kSplit;
    extern __shared__ __align__(16) unsigned char smem[];
    B ck;
    ck.init(smem, args.N, args.NC, args.LC);
    const int w = ck.w, bh = ck.bh;
    const int N = args.N, NC = args.NC;
    const E* qb = reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D;
    const E* kb = reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D;
    const E* vb = reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV;
    const E* dob = reinterpret_cast<const E*>(args.dout) + size_t(bh) * N * DV;
    E* dkb = reinterpret_cast<E*>(args.dk) + size_t(bh) * N * D;
    E* dvb = reinterpret_cast<E*>(args.dv) + size_t(bh) * N * DV;
    static_assert(C <= kThreads, "one thread per token");

    // R, r: the adjoint of the state after the current chunk, carried backwards through
    // the run in fp32 (accumulator-layout pieces; r in the z-holder lanes), from the
    // scanned slot after the run (zero after the last run).
    const bool last_run = ck.run == args.NR - 1;
    f32x4_t racc[B::kStateUnits];
    float rzv[KZ][4];
    size_t rsl = 0;
    if (!last_run) {
        rsl = size_t(bh) * (args.NR + 1) + (args.NR - 2 - ck.run);
        ck.load_slot(racc, args.rst + rsl * (D * DV));
    } else {
#pragma unroll
        for (int u = 0; u < B::kStateUnits; ++u) racc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    ck.load_zvec(rzv, last_run ? nullptr : args.rzt + rsl * D);
    // tb: the pairs across the boundary after the current chunk (keys up to it, queries
    // after it), <R, S> + <r, z> with S, z the state after the chunk; at the run's end from
    // the forward slot after the run, then back chunk by chunk (W_c = tb - K_c, and the
    // boundary in front of the chunk carries W_c + Y_c).
    float tb = 0.0f;
    if constexpr (GATED) {
        float wp = 0.0f;
        if (!last_run) {
            const size_t fsl = size_t(bh) * args.FS + (size_t(ck.run + 1) * args.FP - 1);
            f32x4_t sf[B::kStateUnits];
            ck.load_slot(sf, args.fst + fsl * (D * DV));
            float fz[KZ][4];
            ck.load_zvec(fz, args.fzt + fsl * D);
#pragma unroll
            for (int u = 0; u < B::kStateUnits; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) wp += racc[u][k] * sf[u][k];
#pragma unroll
            for (int t = 0; t < KZ; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) wp += rzv[t][r] * fz[t][r];
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
    ck.template store_rows<D, true, kSplit>(ck.sQ, LQ, sq, ck.sQlo);
    ck.template store_rows<D, true, kSplit>(ck.sK, LQ, sk, ck.sKlo);
    ck.template store_rows<DV, false>(ck.sV, LV, sv);
    ck.template store_rows<DV, false>(ck.sDn, LV, so);
    if (ck.tid < C) {
        ck.sDd[ck.tid] = ck.tid < ck.nrows ? sdd : 0.0f;
        ck.sInv[ck.tid] = ck.tid < ck.nrows ? sinv : 0.0f;
    }
    ck.store_slot(racc);
    ck.put_zvec(ck.sZ, rzv);
    if constexpr (GATED) {
        // Y_c = sum of yq over the chunk's queries (wave 0: one lane per token)
        if (ck.w == 0) {
            const float y = wave_incl_scan(lane < ck.nrows ? syq : 0.0f);
            if (lane == kWave - 1) ck.sRow[0] = y;
        }
    }
    ck.stage_lambda(sg);
    __syncthreads();
    if (B::Sh::kAhead && c > ck.c_first) issue(c - 1);

    // This lane's key row of the wave's transposed tiles, and its decay to the chunk's end.
    const int j0 = 16 * w, jl = j0 + l16;
    const float lam_j = ck.lam(jl);
    const float tail = GATED ? fast_exp2(fminf(ck.lam(C - 1) - lam_j, 0.0f)) : 1.0f;   // 2^(Lambda_last - Lambda_j)

    // A diag(1/d) and B, transposed: lane (l16, g4) holds key jl against queries
    // 16 it + 4 g4 + r (it >= w), decayed and masked (i >= j):
    //   pa = (Fq_i . Fk_j) 2^(Lambda_i - Lambda_j) / d_i,  pb = ((dout_i . v_j) / d_i + dden_i) 2^(...)
    // Each is consumed (and dv stored) before the other is formed, to keep registers low.
    const bool valid = ts + jl < N;
    // the low parts of B where the dq pass takes them
    const bool first = kSplit && (GATED || c == 0);
    {
        F4<E> pa[NI];
#pragma unroll
        for (int it = 0; it < NI; ++it) {
            f32x4_t at = {0.f, 0.f, 0.f, 0.f};
            if (it >= w) {
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
                    at = mma(frag_row(ck.sQ, LQ, 16 * it + l16, 32 * ks + 8 * g4), frag_row(ck.sK, LQ, jl, 32 * ks + 8 * g4),
                             at);
            }
            const int i4 = 16 * it + 4 * g4;
            const f32x4_t li = ck.lam4(i4);
            const f32x4_t iv = *reinterpret_cast<const f32x4_t*>(ck.sInv + i4);
            f32x4_t xa;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool keep = it >= w && i4 + r >= jl;
                const float f = GATED ? fast_exp2(fminf(li[r] - lam_j, 0.0f)) : 1.0f;
                xa[r] = keep ? at[r] * (f * iv[r]) : 0.0f;
            }
            pa[it] = pack4<E>(xa);
        }
        // dV^T[e][j] = 2^(Lambda_last - Lambda_j) (R^T Fk^T)[e][j] + (dOut^T (A diag(1/d)))[e][j]
        f32x4_t dvt[NE];
#pragma unroll
        for (int et = 0; et < NE; ++et) {
            dvt[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const F8<E> bk = frag_row(ck.sK, LQ, jl, 32 * ks + 8 * g4);
                dvt[et] = mma(frag_col(ck.sS, LV, 32 * ks + 8 * g4, 16 * et, l16), bk, dvt[et]);
                if constexpr (kSplit) dvt[et] = mma(frag_col(ck.sSlo, LV, 32 * ks + 8 * g4, 16 * et, l16), bk, dvt[et]);
            }
            if constexpr (GATED) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dvt[et][r] *= tail;
            }
        }
#pragma unroll
        for (int it = 0; it < NI; ++it)
            if (it >= w) {
#pragma unroll
                for (int et = 0; et < NE; ++et)
                    dvt[et] = mma4(frag4_col(ck.sDn, LV, 16 * it + 4 * g4, 16 * et, l16), pa[it], dvt[et]);
            }
        // dv: four consecutive columns of row jl per lane
        if (valid) {
#pragma unroll
            for (int et = 0; et < NE; ++et) store4<E>(dvb + size_t(ts + jl) * DV + 16 * et + 4 * g4, dvt[et]);
        }
    }
    F4<E> pb[NI], pb_lo[NI];
#pragma unroll
    for (int it = 0; it < NI; ++it) {
        f32x4_t bt = {0.f, 0.f, 0.f, 0.f};
        if (it >= w) {
#pragma unroll
            for (int ks = 0; ks < DV / 32; ++ks)
                bt = mma(frag_row(ck.sDn, LV, 16 * it + l16, 32 * ks + 8 * g4), frag_row(ck.sV, LV, jl, 32 * ks + 8 * g4),
                         bt);
        }
        const int i4 = 16 * it + 4 * g4;
        const f32x4_t li = ck.lam4(i4);
        const f32x4_t iv = *reinterpret_cast<const f32x4_t*>(ck.sInv + i4);
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(ck.sDd + i4);
        f32x4_t xb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool keep = it >= w && i4 + r >= jl;
            const float f = GATED ? fast_exp2(fminf(li[r] - lam_j, 0.0f)) : 1.0f;
            xb[r] = keep ? (bt[r] * iv[r] + d4[r]) * f : 0.0f;
        }
        pb[it] = pack4<E>(xb);
        if constexpr (kSplit) pb_lo[it] = pack4<E>(xb - unpack4(pb[it]));
    }

    // dFk^T[d][j] = 2^(Lambda_last - Lambda_j) ((R V^T)[d][j] + r_d) + (Fq^T B)[d][j]
    f32x4_t fk[ND];
    {
        float zk = 0.0f;                              // Fk_j . (carried-state part of dFk_j)
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            fk[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DV / 32; ++ks) {
                const F8<E> bv = frag_row(ck.sV, LV, jl, 32 * ks + 8 * g4);
                fk[dt] = mma(frag_row(ck.sS, LV, 16 * dt + l16, 32 * ks + 8 * g4), bv, fk[dt]);
                if constexpr (kSplit) fk[dt] = mma(frag_row(ck.sSlo, LV, 16 * dt + l16, 32 * ks + 8 * g4), bv, fk[dt]);
            }
            const f32x4_t r4 = *reinterpret_cast<const f32x4_t*>(ck.sZ + 16 * dt + 4 * g4);
            const F4<E> k4 = lds_f4(ck.sK + jl * LQ + 16 * dt + 4 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                fk[dt][r] = (fk[dt][r] + r4[r]) * tail;
                if constexpr (GATED) zk += X::to_f32(k4.x[r]) * fk[dt][r];
            }
        }
        if constexpr (GATED) {
            zk = sum_groups(zk);
            if (g4 == 0 && valid) args.zk[size_t(bh) * N + ts + jl] = zk;
            const float kw = sum16(valid ? zk : 0.0f);     // K_c: this wave's part of sum_j zk_j
            if (lane == 0) ck.sRow[1 + w] = kw;
        }
    }
#pragma unroll
    for (int it = 0; it < NI; ++it)
        if (it >= w) {
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const F4<E> qf = frag4_col(ck.sQ, LQ, 16 * it + 4 * g4, 16 * dt, l16);
                fk[dt] = mma4(qf, pb[it], fk[dt]);
                if constexpr (kSplit) {
                    fk[dt] = mma4(frag4_col(ck.sQlo, LQ, 16 * it + 4 * g4, 16 * dt, l16), pb[it], fk[dt]);
                    if (first) fk[dt] = mma4(qf, pb_lo[it], fk[dt]);
                }
            }
        }
    // dk = dFk * phi'(k): four consecutive columns of row jl per lane
    if (valid) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const f32x4_t f4 = ck.feat4(ck.sK, ck.sKlo, jl * LQ + 16 * dt + 4 * g4);
            f32x4_t o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = fk[dt][r] * dphi_of(f4[r]);
            store4<E>(dkb + size_t(ts + jl) * D + 16 * dt + 4 * g4, o);
        }
    }
    __syncthreads();
    if constexpr (GATED) {
        // W_c = tb - K_c: keys in front of the chunk against queries after it
        const float wcv = tb - (ck.sRow[1] + ck.sRow[2] + ck.sRow[3] + ck.sRow[4]);
        if (ck.tid == 0) args.wc[size_t(bh) * NC + c] = wcv;
        tb = wcv + ck.sRow[0];
    }
    // rows of dOut become 2^Lambda_i dnum_i (pad: 2^Lambda_i dden_i split); split, their
    // low parts go where R's were (read for the last time above)
    E* const dn_lo = kSplit ? ck.sSlo : nullptr;
    ck.template scale_rows<false, false>(dn_lo);
    __syncthreads();
    // the adjoint carried across the chunk: R <- 2^Lambda_last R + Fq^T (2^Lambda dNum),
    // r <- 2^Lambda_last r + Fq^T (2^Lambda dden) (the extra column block)
    {
        const float fc = GATED ? fast_exp2(ck.lam(C - 1)) : 1.0f;
#pragma unroll
        for (int u = 0; u < B::kStateUnits; ++u) {
            const int t = w + 4 * u, a = t / NE, b = t % NE;
            const f32x4_t dr = ck.tile_tn_split(ck.sQ, ck.sQlo, LQ, a, ck.sDn, dn_lo, LV, b);
#pragma unroll
            for (int k = 0; k < 4; ++k) racc[u][k] = fc * racc[u][k] + dr[k];
        }
#pragma unroll
        for (int t = 0; t < KZ; ++t) {
            const f32x4_t dr = ck.tile_tn_split(ck.sQ, ck.sQlo, LQ, w + 4 * t, ck.sDn, nullptr, LV, NE);
#pragma unroll
            for (int r = 0; r < 4; ++r) rzv[t][r] = fc * rzv[t][r] + pair01(dr[r]);
        }
    }
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
