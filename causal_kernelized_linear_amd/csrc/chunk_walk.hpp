// Chunked forward of causal kernelized linear attention for gfx950.
//
// The sequence of every (batch, head) is cut into nseg segments of L chunks of CH
// tokens.  One forward is:
//
//   1. walk<TOTALS>  one workgroup per (head, segment, part) for every segment but
//      the last, each segment cut into `tparts` parts of ceil(L / tparts) chunks:
//      walks the part's chunks and accumulates its own total
//          T = sum_j w_j phi(k_j) v_j^T,  t = sum_j w_j phi(k_j)
//      (w_j = product of the gates after j inside the part; 1 ungated) and, gated,
//      the log2 of the part's total decay.  Reads K and V only.
//   2. the state in front of each segment,
//          P_0 = S0,  P_{s+1} = Gamma_s P_s + T_s      (fp32, over the parts in order),
//      either summed by each output workgroup itself from the totals in front of
//      it (few, small states, one part per segment) or by scan_kernel, in place,
//      beforehand.
//   3. walk<OUTPUT>  one workgroup per (head, segment): starts from P_s and walks the
//      segment's chunks carrying S and z in registers.  Per chunk it forms the masked
//      quadratic part on MFMA, adds the carried-state part, divides by the clamped
//      denominator, stores O, and folds the chunk into the state.  The last
//      segment's workgroup leaves S_N, z_N in the workspace for final_kernel when the
//      caller asks for them.
//
// This is the chunked parallel form of the aiwiki.thehackersbrain.dev page (the
// chunked listing: quadratic inside a chunk, recurrent across chunks, and the
// closing paragraph on the O(c^2) / O(d^2) balance), with the state pass split
// into segment totals plus a prefix so every workgroup of the walk is independent.
//
// Chunk algebra for a chunk [s, s + CH) with Fq = phi(Q_c), Fk = phi(K_c):
//     A     = tril(Fq Fk^T)                  (diagonal kept)
//     num   = Fq S_prev + A V_c,   den = Fq z_prev + A 1,   O_c = num / max(den, eps)
//     (O_c = num in the normaliser-free mode of retention)
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
//     query row of O^T, so the divide stays in the lane.
//   * the denominator rides on the same MFMAs as one more 16-row output tile: its
//     A operand has ones in rows 0, 4, 8, 12 against A^T (the row sums of A, over
//     exactly the rounded values the numerator uses) and z split into a high and a
//     low part in rows 4g and 4g+1 against Fq^T, so every lane group ends up holding
//     its queries' denominators in its first two accumulator slots.
//   * query strips of 16 rows are dealt to waves in pairs (w, 7-w) so every wave
//     gets the same number of causal tiles; only the diagonal key block is masked.
//   * the [D, Dv] state lives in MFMA accumulators (fp32) spread over the waves,
//     wave w owning the d-tiles [w D/64, (w+1) D/64) for every dv; z rides along as
//     one more tile per d-tile whose B operand is a column of ones.  The operand copy
//     S^T (input precision) and z are re-staged in LDS once per chunk.
//   * the fold's key-major Fk operand comes from the row-major Fk tile through
//     ds_read_b64_tr_b16 in the bf16 output walks (gated: with a decayed copy of V^T
//     and the keys' decays as z's operand); the fp32 walks and the totals walk stage a
//     transposed copy of Fk (decayed when gated) instead.
//   * loads are branch-free: rows past the end are clamped to the last row; in a
//     chunk that crosses the end their features are zeroed.  The next chunk's K and V
//     are in flight while this chunk's products run, and its Q while this chunk's
//     state is folded.
//   * column parts (VS > 1): the value columns are cut into VS parts of DV columns
//     (rows of v, o, S0 and S_N are DV * VS wide), and each part is walked by its own
//     workgroups with its own [D, DV] slice of S.  Every column of o depends on S's
//     own columns only, so the parts never exchange anything; each recomputes phi(Q),
//     phi(K), A and z.  Blocks i and i + 8 of the grid walk the two parts of one
//     (head, segment), so both sit on the same XCD (workgroups are dealt to the eight
//     XCDs round-robin) and read Q and K through one L2.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {

struct WalkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;      // gated only
    void* o;             // OUTPUT only
    float* st;           // [BH][nslots][D*Dv] accumulator layout: slot t < (nseg-1) tparts holds
                         // the total of part t % tparts of segment t / tparts (after the scan:
                         // the state after it); slot (nseg-1) tparts receives S_N
    float* zt;           // [BH][nslots][D], alike
    float* lg;           // [BH][nslots] log2 of each part's total decay (gated)
    const float* s0;     // [BH][D][Dv] initial state or NULL (caller layout)
    const float* z0;     // [BH][D] or NULL
    int N;
    int BH;              // heads (B * H)
    int nseg;            // segments per sequence
    int L;               // chunks per segment
    int tparts;          // parts of a segment walked by separate totals workgroups (1: direct prefix)
    int nslots;          // workspace slots per head: (nseg - 1) * tparts + 1
    int direct;          // 1: the output walk sums the totals in front of its segment itself
    int want_final;      // 1: the last segment's output walk leaves S_N, z_N in slot nslots - 1
    float eps;
    int normalize;       // 1: o = num / max(den, eps); 0: o = num (the denominator is not used)
    float fshift;        // RELU walks only: the shift of relu(x) + shift
    const float* W;      // FAVOR walks only: the projections [H][D][D] (fp32), one set per head
    int H;               // FAVOR walks only: heads per batch (W's head is bh % H)
    int stream_kv = 0;   // totals walk: K and V loaded non-temporally (the output walk's reads
                         // of them will not find them in the caches anyway)
};

// Column part and item (head * segments + segment) of a walk workgroup.  With VS parts,
// groups of 8 consecutive blocks take 8 consecutive items, one group per part in turn,
// so the parts of an item are 8 blocks apart (the same XCD) and dispatched together.
// GROUP (one part, a grid of whole groups of 8): blocks are dealt to the 8 XCDs in turn,
// so block b takes item (b mod 8) (grid / 8) + b / 8 and each XCD runs a run of
// consecutive items, whole heads: every later segment of a head reads the totals in front
// of it through one L2 (the direct prefix).
// item >= items: a padding block of the last group, which does nothing.
template <int VS, bool GROUP = false>
__device__ __forceinline__ void walk_block(int items, int& item, int& part) {
    if constexpr (VS == 1) {
        const unsigned g = gridDim.x;
        item = GROUP && g % 8 == 0 ? int((blockIdx.x % 8) * (g / 8) + blockIdx.x / 8) : int(blockIdx.x);
        part = 0;
    } else {
        const int lo = blockIdx.x % 8, hi = blockIdx.x / 8;
        part = hi % VS;
        item = (hi / VS) * 8 + lo;
    }
    (void)items;
}

// Blocks of a walk launch over `items` (head, segment) pairs and VS column parts (GROUP:
// whole groups of 8, as walk_block's GROUP mapping needs).
__host__ __device__ constexpr unsigned walk_grid(unsigned items, int VS, bool group = false) {
    return VS == 1 && !group ? items : (items + 7) / 8 * 8 * unsigned(VS);
}

template <typename E, int D, int DV, int CH, bool GATED, bool OUT>
struct WalkShape {
    static_assert(CH >= 32 && CH <= 256 && (CH & (CH - 1)) == 0, "chunk must be a power of two in [32, 256]");
    static constexpr bool kBf16 = sizeof(E) == 2;
    static constexpr bool kRowK = OUT;                         // row-major Fk tile
    static constexpr bool kKT = !OUT || !kBf16;                // transposed (decayed) Fk^T tile
    // the gated bf16 output walk folds with the decay on V: S += Fk^T (2^(L_last - L) V),
    // from a decayed copy of V^T ([Dv] rows instead of Fk^T's [D])
    static constexpr bool kVD = OUT && GATED && kBf16;
    static constexpr int LKT = CH + (CH >= 128 ? 16 : 0);  // row stride of Fk^T [D][CH] and V^T [Dv][CH]
    static constexpr int LS = D;                      // row stride of S^T [Dv][D] (groups swizzled)
    static constexpr int LZ = D + 8;                  // row stride of the split z rows
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

    // LDS carve-up, in bytes from the base.
    static constexpr size_t kOffK = 0;
    static constexpr size_t kOffKt = kOffK + (kRowK ? size_t(CH) * D * sizeof(E) : 0);
    static constexpr size_t kOffVt = kOffKt + (kKT ? size_t(D) * LKT * sizeof(E) : 0);
    static constexpr size_t kOffVd = kOffVt + size_t(DV) * LKT * sizeof(E);
    static constexpr size_t kOffSt = kOffVd + (kVD ? size_t(DV) * LKT * sizeof(E) : 0);
    static constexpr size_t kOffZb = kOffSt + (OUT ? size_t(DV) * LS * sizeof(E) : 0);
    // Lambda: one row for the workgroup, or (kLamPerWave) one per wave
    static constexpr bool kLamPerWave = walk_lambda_per_wave(int(sizeof(E)), D, DV, CH, GATED, OUT);
    static constexpr size_t kOffLam = kOffZb + (OUT ? size_t(4) * LZ * sizeof(E) : 0);
    static constexpr size_t kOffDec = kOffLam + size_t(CH) * 4 * (kLamPerWave ? 4 : 1);   // kVD: each key's decay (bf16)
    static constexpr size_t kOffO = kOffDec + (kVD ? size_t(CH) * sizeof(E) : 0);
    static constexpr int kOBlock = 16 * 128;          // per wave: 16 rows x 128 bytes of o
    static constexpr size_t kBytes = kOffO + (OUT ? size_t(kThreads / kWave) * kOBlock : 0);
    static_assert(kBytes == walk_lds_bytes(int(sizeof(E)), D, DV, CH, GATED, OUT), "host LDS formula out of step");
    // waves per SIMD the kernel is compiled for (amdgpu_waves_per_eu): a fixed target keeps
    // the compiler from squeezing registers for an occupancy the shape cannot reach, which
    // would make it wait for the next chunk's loads early
    static constexpr int kWaves = walk_waves(int(sizeof(E)), D, DV, CH, GATED, OUT);
    // chunks whose loads are in flight ahead of the one being processed (walk_depth)
    static constexpr int kDepth = walk_depth(int(sizeof(E)), D, DV, CH, GATED, OUT);
};

// Query strip handled by wave w in its m-th slot, or -1.
template <int NSTRIP>
__host__ __device__ constexpr int strip_of(int w, int m) {
    const int pair = m >> 1;
    const int s = (m & 1) ? (pair * 8 + 7 - w) : (pair * 8 + w);
    return s < NSTRIP ? s : -1;
}

// LDS layouts follow how gfx950 serves LDS, as measured with its bank-conflict counter:
// 64 banks of 4 bytes for reads, a 16-byte read serving in one cycle the 16 lanes of a
// 32-lane half whose lane bits 2..4 have the same parity, an 8-byte read (or transpose
// read) 32 consecutive lanes; writes 128 bytes per cycle over 32 banks, 8 consecutive
// lanes of a 16-byte write or 16 of an 8-byte one.  Every tile below is row-major with
// its 8-element (16-byte) groups permuted per row as group ^ h(row); the h and the row
// padding of each tile were found by searching that model over all of the tile's
// accesses at every built shape.
//
// Row-major phi(K) tile [rows][W], no padding, h from row bits 1, 3 (W = 64) or 0, 1, 3
// (W = 128): its staging writes, A^T operand reads (16 rows in the key order of the
// transposed products) and transpose reads (4 rows x 4 columns per 16 lanes) are all
// conflict-free.
template <int W>
__device__ __forceinline__ int tile_off(int row, int col) {
    int h;
    if constexpr (W == 64)
        h = (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
    else
        h = ((row & 1) << 1) | (((row >> 1) & 1) << 2) | (((row >> 3) & 1) << 3);
    return row * W + ((((col >> 3) ^ h) & (W / 8 - 1)) << 3) + (col & 7);
}

// S^T tile [Dv][D], no padding, h from row bits 0, 1, 3: the operand reads (rows in the
// output tiles' dv order, out_dv) are conflict-free; the 8-byte staging writes (once per
// chunk) take two cycles.
template <int D>
__device__ __forceinline__ int st_off(int row, int col) {
    const int h = (row & 3) | (((row >> 3) & 1) << 2) | (D == 128 ? ((row & 1) << 3) : 0);
    return row * D + ((((col >> 3) ^ h) & (D / 8 - 1)) << 3) + (col & 7);
}

// Row m of O^T tile u holds dv = out_dv(u, m): tiles 2t and 2t+1 together hold the 8
// consecutive dv 32t + 8(m/4) .. + 7 in lane group m/4, so each lane writes its output
// row as 16-byte pieces.
__device__ __forceinline__ int out_dv(int u, int m) { return 32 * (u >> 1) + 8 * (m >> 2) + 4 * (u & 1) + (m & 3); }

// Key-major bf16 operand from a row-major tile_off<W> tile: slot e of lane l holds
// tile[k0 + e][m0 + l % 16] (k0 includes the lane group's offset).  Each
// ds_read_b64_tr_b16 gives every lane of a 16-lane block four rows of one column
// when block lane j points at row k0 + j / 4, columns m0 + 4 (j % 4) .. + 3.
template <int W>
__device__ __forceinline__ F8<uint16_t> tr_operand(const uint16_t* tile, int k0, int m0, int l16) {
    typedef short i16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4_t* lds_ptr_t;
    const int r = k0 + (l16 >> 2), c = m0 + 4 * (l16 & 3);
    const i16x4_t a =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr_t)(const_cast<uint16_t*>(tile + tile_off<W>(r, c))));
    const i16x4_t b =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr_t)(const_cast<uint16_t*>(tile + tile_off<W>(r + 4, c))));
    F8<uint16_t> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f.x[e] = uint16_t(a[e]);
        f.x[4 + e] = uint16_t(b[e]);
    }
    return f;
}

// One head's output rows as a buffer resource: stores past its end (rows past N) are
// dropped by the hardware, so the tail needs no branch.  Byte offsets are 32-bit; the
// library keeps every head's output below 2 GiB.  The stores are non-temporal at device
// scope (cache policy bits nt and sc1, aux = 18) and write whole 128-byte lines
// (store_strip): o is written once and never read back, and its write-back then happens
// inside this walk instead of running beside the next kernel.  With plain stores the
// totals walk that follows took 29.4 us instead of 24.8; nt alone gave the output walk
// 52.2 us, nt with sc1 49.8-50.7 (bf16, B=8 H=16 N=4096 D=Dv=64, 128-token chunks,
// event-timed at steady clocks).
typedef int v4i_t __attribute__((ext_vector_type(4)));
// The 16-byte groups of one F8<E> (one for bf16, two for fp32), as bits.
template <typename E>
struct Groups16 {
    v4i_t g[sizeof(F8<E>) / 16];
};
struct OutRsrc {
    static constexpr int kNonTemporal = 18;
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ void init(void* base, unsigned bytes) {
        r = __builtin_amdgcn_make_buffer_rsrc(base, 0, int(bytes), 0x00020000);
    }
    __device__ __forceinline__ void store(const v4i_t& v, int off) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNonTemporal);
    }
};

// The per-thread machinery of one workgroup walking chunks of one head.
// OUT: the workgroup forms outputs (row-major Fk, S^T and the split z in LDS).
// IDENT: q and k already hold the features (another map applied beforehand), so the
// walker uses them as they are instead of applying elu + 1.  RELU: the features are
// relu(x) + fshift, applied while staging like elu + 1.  SPLITK (totals walk, bf16): each
// element of Fk^T goes to LDS as a high and a low part, hi = bf16(f), lo = bf16(f - hi),
// the low parts in a tile of their own after the shape's tiles, and the fold takes both,
// so the totals carry the features to about 16 bits instead of 8.  FAVOR (bf16,
// ungated, D features from D input dimensions): the features are FAVOR+'s positive random
// features, exp(w_m . x - |x|^2 / 2) / sqrt(D), projected on the MFMA while staging (W
// split into bf16 high and low parts in LDS after the shape's tiles, favor_lds_bytes).
template <typename E, int D, int DV, int CH, bool GATED, bool OUT, bool IDENT = false, bool RELU = false, int VS = 1,
          bool SPLITK = false, bool FAVOR = false>
struct ChunkWalker {
    using Sh = WalkShape<E, D, DV, CH, GATED, OUT>;
    static_assert(!SPLITK || (Sh::kKT && !OUT && sizeof(E) == 2), "split features: bf16 totals walk only");
    static_assert(!FAVOR || (sizeof(E) == 2 && !GATED && !IDENT && !RELU && VS == 1 && !SPLITK),
                  "in-walk FAVOR+ features: bf16, ungated");
    static constexpr int LW = D + 8;        // row stride of W's split tiles
    using X = Elem<E>;
    static constexpr int LKT = Sh::LKT, LS = Sh::LS;
    static constexpr int DVF = DV * VS;     // row length of v and o (all column parts)
    float fshift = 0.0f;

    __device__ __forceinline__ float feat(float x) const {
        if constexpr (IDENT) return x;
        else if constexpr (RELU) return fmaxf(x, 0.0f) + fshift;
        else return phi(x);
    }

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
    E* sKtLo;      // SPLITK: low parts of Fk^T, laid out like sKt
    E* sVd;        // kVD: decayed V^T, laid out like sVt
    E* sDec;       // kVD: the keys' decays 2^(L_last - L_j), for z's fold
    E* sWh;        // FAVOR: W's high and low parts [D][LW], after the shape's tiles
    E* sWl;
    E* sVt;
    E* sSt;
    E* sZb;        // [4][LZ]: z high part, z low part, two zero rows
    float* sLam;
    unsigned char* sO;   // this wave's 16 x 128-byte block of o (output walk)
    int tid, w, lane, l16, g4;
    int N;
    int last;      // last row the loads may touch: the end of the walked range (clamped to N - 1)
    int stream_kv = 0;   // totals walk: K and V loaded non-temporally (WalkArgs::stream_kv)
    const E* qb;
    const E* kb;
    const E* vb;
    const float* gb;

    // Fk^T and V^T rows are [CH] keys in groups of 8 (16 bytes), padded by 16 elements
    // from CH = 128 up; group j of row r sits at slot j ^ h(r).  The MFMA operand reads
    // (16 consecutive rows for the fold, rows in out_dv order for A V, one group per lane
    // group) are conflict-free at every shape; the transposed staging writes (4-key
    // quads) take at most two cycles per 128 bytes at 64-row tiles, four at 128-row tiles
    // below CH = 128.
    static __device__ __forceinline__ int tidx(int row, int group) {
        int h;
        if constexpr (CH == 32)
            h = ((row >> 5) & 1) | (((row >> 3) & 1) << 1);
        else if constexpr (CH == 64)
            h = ((row >> 5) & 1) | (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
        else
            h = ((row >> 3) & 7) | (((row >> 3) & 1) << 3);
        return row * LKT + (((group ^ h) & (CH / 8 - 1)) << 3);
    }
    // Rows of phi(K) held by staging unit kq, slot r: four consecutive keys when a
    // transposed copy is written (one 8-byte quad per feature), else the strided rows
    // kq, kq + CH/4, ... that tile_off serves without bank conflicts.
    static constexpr bool kStridedK = !Sh::kKT;
    static __device__ __forceinline__ int krow_of(int kq, int r) { return kStridedK ? kq + (CH / 4) * r : 4 * kq + r; }

    __device__ __forceinline__ void init(unsigned char* smem, int N_, const E* q, const E* k, const E* v,
                                         const float* g) {
        sK = reinterpret_cast<E*>(smem + Sh::kOffK);
        sKt = reinterpret_cast<E*>(smem + Sh::kOffKt);
        sVd = reinterpret_cast<E*>(smem + Sh::kOffVd);
        sDec = reinterpret_cast<E*>(smem + Sh::kOffDec);
        sVt = reinterpret_cast<E*>(smem + Sh::kOffVt);
        sSt = reinterpret_cast<E*>(smem + Sh::kOffSt);
        sZb = reinterpret_cast<E*>(smem + Sh::kOffZb);
        sKtLo = reinterpret_cast<E*>(smem + Sh::kBytes);
        sWh = reinterpret_cast<E*>(smem + Sh::kBytes);
        sWl = sWh + D * LW;
        tid = threadIdx.x;
        w = __builtin_amdgcn_readfirstlane(tid / kWave);
        sLam = reinterpret_cast<float*>(smem + Sh::kOffLam) + (Sh::kLamPerWave ? w * CH : 0);
        sO = smem + Sh::kOffO + size_t(w) * Sh::kOBlock;
        lane = tid % kWave;
        l16 = lane & 15;
        g4 = lane >> 4;
        N = N_;
        last = N_ - 1;
        qb = q;
        kb = k;
        vb = v;
        gb = g;
    }

    // Global -> registers for the chunk starting at token ts.  Rows past `last` are
    // clamped to it (always in bounds: the prefetch behind the walk's last chunk rereads
    // one cached row); stage() zeroes the features of rows past N.
    // PARTS selects K (1), V (2) or both (3; the split walk divides them between its two
    // kinds of wave).
    // The output walks read every row for the last time, so their loads are non-temporal;
    // the totals walk's are where stream_kv says so.
    template <int PARTS = 3>
    __device__ __forceinline__ void load(Regs& R, int ts) const {
        if (OUT || stream_kv)
            load_kv<PARTS, true>(R, ts);
        else
            load_kv<PARTS, false>(R, ts);
        if constexpr (GATED) {
            // every wave loads the gates (cached; every wave, or wave 0, scans them), so the
            // loads sit behind no branch
#pragma unroll
            for (int i = 0; i < Sh::GPT; ++i) {
                const int j = lane * Sh::GPT + i;
                const float gv = gb[min(ts + j, last)];
                R.rg[i] = (j < CH && ts + j < N) ? gv : 1.0f;
            }
        }
    }
    template <int PARTS, bool NT>
    __device__ __forceinline__ void load_kv(Regs& R, int ts) const {
#pragma unroll
        for (int it = 0; it < Sh::KPT; ++it) {
            if (!(PARTS & 1)) break;
            const int u = tid + it * kThreads;
            const int cg = u % (D / 8), kq = (u / (D / 8)) % (CH / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = min(ts + krow_of(kq, r), last);
                R.rk[it][r] = global_f8<NT>(kb + size_t(row) * D + 8 * cg);
            }
        }
#pragma unroll
        for (int it = 0; it < Sh::VPT; ++it) {
            if (!(PARTS & 2)) break;
            const int u = tid + it * kThreads;
            const int cg = u % (DV / 8), kq = (u / (DV / 8)) % (CH / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = min(ts + 4 * kq + r, last);
                R.rv[it][r] = global_f8<NT>(vb + size_t(row) * DVF + 8 * cg);
            }
        }
    }

    __device__ __forceinline__ void load_q(QRegs& Q, int ts) const {
#pragma unroll
        for (int m = 0; m < Sh::MAXS; ++m) {
            const int s = max(strip_of<Sh::NSTRIP>(w, m), 0);
            const int row = min(ts + 16 * s + l16, last);
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks)
                Q.rq[m][ks] = global_f8<true>(qb + size_t(row) * D + 32 * ks + 8 * g4);
        }
    }

    // Lambda_j = inclusive sum of log2 g over the chunk, into sLam: by wave 0 for the
    // workgroup, or (kLamPerWave) by every wave into its own row, which only it reads, so
    // that no barrier follows (every wave holds the chunk's gates).
    __device__ __forceinline__ void lambda(const Regs& R) const {
        if (!Sh::kLamPerWave && w != 0) return;
        float loc[Sh::GPT];
        float run = 0.0f;
#pragma unroll
        for (int i = 0; i < Sh::GPT; ++i) {
            run += fast_log2(R.rg[i]);
            loc[i] = run;
        }
        const float excl = wave_incl_scan(run) - run;
#pragma unroll
        for (int i = 0; i < Sh::GPT; ++i) {
            const int j = lane * Sh::GPT + i;
            if (j < CH) sLam[j] = excl + loc[i];
        }
    }

    // phi(K) -> Fk (row-major) and/or Fk^T (decayed when gated); V -> V^T (and, kVD, its
    // decayed copy and the keys' decays).  TAIL: the chunk crosses the end of the
    // sequence, so rows past N get zero features.
    template <bool TAIL, int PARTS = 3>
    __device__ __forceinline__ void stage(const Regs& R, int ts, float lam_last) const {
        if constexpr (FAVOR) {
            if constexpr ((PARTS & 1) != 0) stage_favor_k<TAIL>(R, ts);
        }
#pragma unroll
        for (int it = 0; it < Sh::KPT; ++it) {
            const int u = tid + it * kThreads;
            if (!FAVOR && (PARTS & 1) && u < Sh::NKU) {
                const int cg = u % (D / 8), kq = u / (D / 8);
                E fr[4][8];
                float ff[4][8];      // SPLITK: the features before rounding
#pragma unroll
                for (int r = 0; r < 4; ++r) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float f = feat(X::to_f32(R.rk[it][r].x[e]));
                        ff[r][e] = TAIL ? (ts + krow_of(kq, r) < N ? f : 0.0f) : f;
                        fr[r][e] = X::from_f32(ff[r][e]);
                    }
                    if constexpr (Sh::kRowK) {
                        F8<E> t;
#pragma unroll
                        for (int e = 0; e < 8; ++e) t.x[e] = fr[r][e];
                        *reinterpret_cast<F8<E>*>(sK + tile_off<D>(krow_of(kq, r), 8 * cg)) = t;
                    }
                }
                if constexpr (Sh::kKT) {
                    float dec[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        dec[r] = GATED ? fast_exp2(fminf(lam_last - sLam[4 * kq + r], 0.0f)) : 1.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        F4<E> t, tl;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if constexpr (SPLITK) {
                                const float fv = GATED ? ff[r][e] * dec[r] : ff[r][e];
                                t.x[r] = X::from_f32(fv);
                                tl.x[r] = X::from_f32(fv - X::to_f32(t.x[r]));
                            } else {
                                t.x[r] = GATED ? X::from_f32(X::to_f32(fr[r][e]) * dec[r]) : fr[r][e];
                            }
                        }
                        const int at = tidx(8 * cg + e, kq >> 1) + 4 * (kq & 1);
                        *reinterpret_cast<F4<E>*>(sKt + at) = t;
                        if constexpr (SPLITK) *reinterpret_cast<F4<E>*>(sKtLo + at) = tl;
                    }
                }
            }
        }
#pragma unroll
        for (int it = 0; it < Sh::VPT; ++it) {
            const int u = tid + it * kThreads;
            if ((PARTS & 2) && u < Sh::NVU) {
                const int cg = u % (DV / 8), kq = u / (DV / 8);
                float dec[4];
                if constexpr (Sh::kVD) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) dec[r] = fast_exp2(fminf(lam_last - sLam[4 * kq + r], 0.0f));
                    if (cg == 0) {
                        F4<E> d4;
#pragma unroll
                        for (int r = 0; r < 4; ++r) d4.x[r] = X::from_f32(dec[r]);
                        *reinterpret_cast<F4<E>*>(sDec + 4 * kq) = d4;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    F4<E> t, td;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        t.x[r] = R.rv[it][r].x[e];
                        if constexpr (Sh::kVD) td.x[r] = X::from_f32(X::to_f32(t.x[r]) * dec[r]);
                    }
                    const int at = tidx(8 * cg + e, kq >> 1) + 4 * (kq & 1);
                    *reinterpret_cast<F4<E>*>(sVt + at) = t;
                    if constexpr (Sh::kVD) *reinterpret_cast<F4<E>*>(sVd + at) = td;
                }
            }
        }
    }

    __device__ __forceinline__ void phi_q(const QRegs& Q, F8<E> (&fq)[Sh::MAXS][D / 32]) const {
        if constexpr (FAVOR) {
            favor_q(Q, fq);
        } else {
#pragma unroll
            for (int m = 0; m < Sh::MAXS; ++m)
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) fq[m][ks].x[e] = X::from_f32(feat(X::to_f32(Q.rq[m][ks].x[e])));
        }
    }

    // ---- FAVOR+ features (FAVOR walks) ----
    //
    // W of this head, split (hi = bf16(w), lo = bf16(w - hi)), into sWh / sWl; once per
    // workgroup, before the first chunk is staged (whose barriers order it).
    __device__ __forceinline__ void stage_w(const float* Wb) const {
        if constexpr (FAVOR) {
            for (int u = tid; u < D * D / 4; u += kThreads) {
                const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(Wb + 4 * u);
                const int m = (4 * u) / D, d = (4 * u) % D;
                F4<E> h, l;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h.x[e] = X::from_f32(w4[e]);
                    l.x[e] = X::from_f32(w4[e] - X::to_f32(h.x[e]));
                }
                *reinterpret_cast<F4<E>*>(sWh + m * LW + d) = h;
                *reinterpret_cast<F4<E>*>(sWl + m * LW + d) = l;
            }
        }
    }

    // exp(y - h) / sqrt(D) for a projection y and a half squared norm h.
    static __device__ __forceinline__ float favor_feat(float y, float h) {
        return fast_exp2((y - h) * kLog2e) * __builtin_amdgcn_rsqf(float(D));
    }

    // The chunk's keys: the raw rows go to LDS where their features will be (the
    // row-major phi(K) tile, or in the totals walk the transposed one's space, laid out
    // row-major by tile_off) with each row's |k|^2 / 2 in sLam; after a barrier every
    // wave projects its 16-row blocks of keys on the MFMA (W hi and lo against the
    // exact bf16 rows) and forms the features; after a second barrier (every raw row
    // read) they go to the tile the walk reads: phi(K) row-major (output walk) or phi(K)^T
    // (totals walk).  Rows past N (TAIL) get zero features.
    template <bool TAIL>
    __device__ __forceinline__ void stage_favor_k(const Regs& R, int ts) const {
        E* const raw = OUT ? sK : sKt;
        float* const sNrm = sLam;
#pragma unroll
        for (int it = 0; it < Sh::KPT; ++it) {
            const int u = tid + it * kThreads;
            const int cg = u % (D / 8), kq = (u / (D / 8)) % (CH / 4);
            float sq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = krow_of(kq, r);
                if (u < Sh::NKU) *reinterpret_cast<F8<E>*>(raw + tile_off<D>(row, 8 * cg)) = R.rk[it][r];
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = X::to_f32(R.rk[it][r].x[e]);
                    acc += x * x;
                }
                sq[r] = lane_group_sum<D / 8>(acc);
            }
            if (u < Sh::NKU && cg == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sNrm[krow_of(kq, r)] = 0.5f * sq[r];
            }
        }
        __syncthreads();
        // wave w: key blocks w, w + 4, ... (CH / 64 of them), all D / 16 feature tiles.
        // The wave first reads the raw rows of its blocks into registers, then takes W's
        // operands one feature tile at a time and applies each to all of its blocks.
        // Output walk: a wave reads the raw rows of its own blocks only and writes their
        // features over them (its LDS accesses complete in order), so each feature tile
        // goes out as soon as it is formed.  Totals walk: the transposed features land on
        // other waves' raw rows, so they wait in registers for a barrier.
        constexpr int NJB = CH / 64, NMT = D / 16, KS = D / 32;
        static_assert(NJB >= 1, "chunks of at least 64 tokens");
        F8<E> xf[NJB][KS];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) xf[jb][ks] = lds_f8(raw + tile_off<D>(16 * (w + 4 * jb) + l16, 32 * ks + 8 * g4));
        float h[NJB];              // output walk: the norm term of key 16 (w + 4 jb) + l16
        f32x4_t h4[NJB];           // totals walk: of keys 16 (w + 4 jb) + 4 g4 + r
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            const int j0 = 16 * (w + 4 * jb);
            if constexpr (OUT)
                h[jb] = sNrm[j0 + l16];
            else
                h4[jb] = *reinterpret_cast<const f32x4_t*>(sNrm + j0 + 4 * g4);
        }
        __builtin_amdgcn_wave_barrier();
        F4<E> fv[OUT ? 1 : NJB][NMT];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            f32x4_t y[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) y[jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const F8<E> wh = lds_f8(sWh + (16 * mt + l16) * LW + 32 * ks + 8 * g4);
                const F8<E> wl = lds_f8(sWl + (16 * mt + l16) * LW + 32 * ks + 8 * g4);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    if constexpr (OUT) {
                        // y[m][j]: lane holds features 16 mt + 4 g4 + r of key j0 + l16
                        y[jb] = mma(wh, xf[jb][ks], y[jb]);
                        y[jb] = mma(wl, xf[jb][ks], y[jb]);
                    } else {
                        // y[j][m]: lane holds keys j0 + 4 g4 + r against feature 16 mt + l16
                        y[jb] = mma(xf[jb][ks], wh, y[jb]);
                        y[jb] = mma(xf[jb][ks], wl, y[jb]);
                    }
                }
            }
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int j0 = 16 * (w + 4 * jb);
                if constexpr (OUT) {
                    const int j = j0 + l16;
                    const bool in = !TAIL || ts + j < N;
#pragma unroll
                    for (int r = 0; r < 4; ++r) fv[0][mt].x[r] = X::from_f32(in ? favor_feat(y[jb][r], h[jb]) : 0.0f);
                    *reinterpret_cast<F4<E>*>(sK + tile_off<D>(j, 16 * mt + 4 * g4)) = fv[0][mt];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool in = !TAIL || ts + j0 + 4 * g4 + r < N;
                        fv[jb][mt].x[r] = X::from_f32(in ? favor_feat(y[jb][r], h4[jb][r]) : 0.0f);
                    }
                }
            }
        }
        if constexpr (!OUT) {
            __syncthreads();
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int kq0 = 4 * (w + 4 * jb) + g4;      // keys 4 kq0 .. 4 kq0 + 3
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt)
                    *reinterpret_cast<F4<E>*>(sKt + tidx(16 * mt + l16, kq0 >> 1) + 4 * (kq0 & 1)) = fv[jb][mt];
            }
        }
    }

    // This wave's query strips: the projection W q on the MFMA (W's parts against the
    // exact bf16 rows in registers: lane (l16, g4) gets features 16 mt + 4 g4 + r of
    // query l16), |q|^2 / 2 summed over the four lane groups, the features, and their
    // regrouping into the operand layout (features 32 ks + 8 g4 .. + 7 of query l16)
    // through the wave's 16-row block of LDS, 64 features at a time.
    __device__ __forceinline__ void favor_q(const QRegs& Q, F8<E> (&fq)[Sh::MAXS][D / 32]) const {
        constexpr int MS = Sh::MAXS, KS = D / 32;
        E* const blk = reinterpret_cast<E*>(sO);          // 16 rows x 64 features
        float h[MS];
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            float sq = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = X::to_f32(Q.rq[m][ks].x[e]);
                    sq += x * x;
                }
            sq += __shfl_xor(sq, 16, kWave);
            sq += __shfl_xor(sq, 32, kWave);
            h[m] = 0.5f * sq;
        }
        // each of W's operands is read once and applied to every strip of the wave; the
        // strips' features go through the block one strip at a time
#pragma unroll
        for (int half = 0; half < D / 64; ++half) {
            F4<E> f[MS][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int mt = 4 * half + t;
                f32x4_t y[MS];
#pragma unroll
                for (int m = 0; m < MS; ++m) y[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const F8<E> wh = lds_f8(sWh + (16 * mt + l16) * LW + 32 * ks + 8 * g4);
                    const F8<E> wl = lds_f8(sWl + (16 * mt + l16) * LW + 32 * ks + 8 * g4);
#pragma unroll
                    for (int m = 0; m < MS; ++m) {
                        y[m] = mma(wh, Q.rq[m][ks], y[m]);
                        y[m] = mma(wl, Q.rq[m][ks], y[m]);
                    }
                }
#pragma unroll
                for (int m = 0; m < MS; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) f[m][t].x[r] = X::from_f32(favor_feat(y[m][r], h[m]));
            }
#pragma unroll
            for (int m = 0; m < MS; ++m) {
#pragma unroll
                for (int t = 0; t < 4; ++t) *reinterpret_cast<F4<E>*>(blk + l16 * 64 + 16 * t + 4 * g4) = f[m][t];
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) fq[m][2 * half + kk] = lds_f8(blk + l16 * 64 + 32 * kk + 8 * g4);
                __builtin_amdgcn_wave_barrier();
            }
        }
    }

    // The two zero rows of the split-z operand; written once, before the first barrier.
    __device__ __forceinline__ void clear_zb() const {
        constexpr int NU = 2 * Sh::LZ * int(sizeof(E)) / 16;
        if (tid < NU)
            *reinterpret_cast<F8<uint16_t>*>(reinterpret_cast<unsigned char*>(sZb + 2 * Sh::LZ) + 16 * tid) =
                zero8<uint16_t>();
    }

    // S^T (operand precision) and z = z_hi + z_lo (operand precision each) into LDS for
    // the carried-state part.
    __device__ __forceinline__ void stage_state(const f32x4_t (&sacc)[Sh::TPW], const f32x4_t (&zacc)[Sh::ZT]) const {
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i) {
            const int a = w * Sh::ZT + i;
#pragma unroll
            for (int b = 0; b < Sh::NB; ++b) {
                F4<E> t;
#pragma unroll
                for (int r = 0; r < 4; ++r) t.x[r] = X::from_f32(sacc[i * Sh::NB + b][r]);
                *reinterpret_cast<F4<E>*>(sSt + st_off<D>(16 * b + l16, 16 * a + 4 * g4)) = t;
            }
            if (l16 == 0) {
                F4<E> hi, lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hi.x[r] = X::from_f32(zacc[i][r]);
                    lo.x[r] = X::from_f32(zacc[i][r] - X::to_f32(hi.x[r]));
                }
                *reinterpret_cast<F4<E>*>(sZb + 16 * a + 4 * g4) = hi;
                *reinterpret_cast<F4<E>*>(sZb + Sh::LZ + 16 * a + 4 * g4) = lo;
            }
        }
    }

    // State fold: S = 2^lam_last S + Fk^T V (Fk^T decayed when gated, or V in the gated
    // bf16 output walk), z alike.
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
            const E* const vsrc = Sh::kVD ? sVd : sVt;
            // z's B operand: a column of ones, or (kVD) of the keys' decays
            F8<E> zb = ones;
            if constexpr (Sh::kVD) {
                const F8<E> d8 = lds_f8(sDec + 32 * kbk + 8 * g4);
#pragma unroll
                for (int e = 0; e < 8; ++e) zb.x[e] = l16 == 0 ? d8.x[e] : X::from_f32(0.0f);
            }
#pragma unroll
            for (int b = 0; b < Sh::NB; ++b) vf[b] = lds_f8(vsrc + tidx(16 * b + l16, 4 * kbk + g4));
#pragma unroll
            for (int i = 0; i < Sh::ZT; ++i) {
                const int a = w * Sh::ZT + i;
                F8<E> ka;
                if constexpr (Sh::kKT)
                    ka = lds_f8(sKt + tidx(16 * a + l16, 4 * kbk + g4));
                else
                    ka = tr_operand<D>(sK, 32 * kbk + 8 * g4, 16 * a, l16);
#pragma unroll
                for (int b = 0; b < Sh::NB; ++b) sacc[i * Sh::NB + b] = mma(ka, vf[b], sacc[i * Sh::NB + b]);
                zacc[i] = mma(ka, zb, zacc[i]);
                if constexpr (SPLITK) {
                    const F8<E> kl = lds_f8(sKtLo + tidx(16 * a + l16, 4 * kbk + g4));
#pragma unroll
                    for (int b = 0; b < Sh::NB; ++b) sacc[i * Sh::NB + b] = mma(kl, vf[b], sacc[i * Sh::NB + b]);
                    zacc[i] = mma(kl, ones, zacc[i]);
                }
            }
        }
    }

    // Walk chunks c0 .. c0+nch-1 of the head, folding each into (sacc, zacc); with OUT
    // also form and store the outputs (S^T and z must then already be staged in LDS).
    // One register set: K and V of the next chunk are loaded right after this chunk is
    // staged, Q of the next chunk once this chunk's outputs no longer need it.  Those
    // loads are issued on every chunk, the last included (they then reread the range's
    // last row), so the wait counts the compiler derives stay exact and nothing waits
    // for a prefetch before its data is used.  (A second register set, loading two
    // chunks ahead, made the totals walk slower.)  The last chunk is folded only when
    // fold_last is set.  prologue() runs once the first chunk's loads are in flight (the
    // output walk forms the state in front of its segment there).
    //
    // With a prefetch depth of two (Sh::kDepth, for shapes that run one workgroup per
    // compute unit and have the registers) two register sets alternate: the loads of
    // chunk n + 2 go out while chunk n is processed, so twice the bytes are in flight.
    template <typename Prologue>
    __device__ __forceinline__ void walk(int c0, int nch, f32x4_t (&sacc)[Sh::TPW], f32x4_t (&zacc)[Sh::ZT],
                                         float& lg_total, const OutRsrc& ob, float eps, int norm, bool fold_last,
                                         Prologue&& prologue) {
        last = min(N, (c0 + max(nch, 1)) * CH) - 1;
        if constexpr (Sh::kDepth == 1) {
            Regs R;
            QRegs qr;
            load(R, c0 * CH);
            if constexpr (OUT) load_q(qr, c0 * CH);
            prologue();
            for (int n = 0; n < nch; ++n) step(R, qr, c0, n, nch, sacc, zacc, lg_total, ob, eps, norm, fold_last);
        } else {
            static_assert(Sh::kDepth == 2, "prefetch depth 1 or 2");
            Regs R0, R1;
            QRegs q0, q1;
            load(R0, c0 * CH);
            if constexpr (OUT) load_q(q0, c0 * CH);
            load(R1, (c0 + 1) * CH);
            if constexpr (OUT) load_q(q1, (c0 + 1) * CH);
            prologue();
            for (int n = 0; n < nch; n += 2) {
                step(R0, q0, c0, n, nch, sacc, zacc, lg_total, ob, eps, norm, fold_last);
                if (n + 1 < nch) step(R1, q1, c0, n + 1, nch, sacc, zacc, lg_total, ob, eps, norm, fold_last);
            }
        }
    }

    // Chunk c0 + n, whose K, V (R) and Q (qr) are loaded; R and qr are then reloaded with
    // chunk c0 + n + kDepth (rows past the walked range reread its last row).
    __device__ __forceinline__ void step(Regs& R, QRegs& qr, int c0, int n, int nch, f32x4_t (&sacc)[Sh::TPW],
                                         f32x4_t (&zacc)[Sh::ZT], float& lg_total, const OutRsrc& ob, float eps,
                                         int norm, bool fold_last) {
        const int ts = (c0 + n) * CH;
        if constexpr (GATED) {
            lambda(R);
            if constexpr (Sh::kLamPerWave)
                __builtin_amdgcn_wave_barrier();   // the wave's own row, read by its other lanes
            else
                __syncthreads();
        }
        const float lam_last = GATED ? sLam[CH - 1] : 0.0f;
        if (ts + CH <= N)
            stage<false>(R, ts, lam_last);
        else
            stage<true>(R, ts, lam_last);
        F8<E> fq[Sh::MAXS][D / 32];
        if constexpr (OUT) phi_q(qr, fq);
        load(R, ts + Sh::kDepth * CH);
        __syncthreads();
        if constexpr (OUT) {
            outputs(fq, ts, ob, eps, norm);
            load_q(qr, ts + Sh::kDepth * CH);
        }
        const bool more = n + 1 < nch;
        if (more || fold_last) fold(sacc, zacc, lam_last);
        lg_total += lam_last;
        __syncthreads();
        if (OUT && more) stage_state(sacc, zacc);
    }

    // One query strip of o out to memory: rows row0 .. row0 + 15, the lane holding row
    // l16's columns 32t + 8g4 .. 32t + 8g4 + 7 in outv[t].  A store of those directly
    // writes half of each of 16 rows' 128-byte lines per instruction; here each 128-byte
    // column block goes through this wave's LDS block first (16-byte group j of row r at
    // slot j ^ (r & 7): conflict-free writes of 8 rows per cycle and reads of whole rows)
    // and is read back so that each store instruction writes 8 whole rows' lines.  The
    // wave's LDS operations complete in order, so only the compiler has to be kept from
    // moving them (wave_barrier).  Rows past N fall outside the output resource and are
    // dropped by the hardware.
    __device__ __forceinline__ void store_strip(const F8<E> (&outv)[DV / 32], int row0, const OutRsrc& ob) const {
        constexpr int RB = DV * int(sizeof(E));   // bytes per row of this column part of o
        constexpr int RBF = DVF * int(sizeof(E)); // bytes from one row of o to the next
        constexpr int GPT = int(sizeof(E)) / 2;   // 16-byte groups per lane in each outv[t]
        static_assert(sizeof(F8<E>) == 16 * GPT, "outv[t] is GPT 16-byte groups");
#pragma unroll
        for (int c = 0; c < RB / 128; ++c) {
#pragma unroll
            for (int t = 0; t < DV / 32; ++t) {
                // group 4 GPT t + GPT g4 + h of the row: column block (4 GPT t) / 8 for every g4
                if ((4 * GPT * t) / 8 != c) continue;
                const Groups16<E> grp = __builtin_bit_cast(Groups16<E>, outv[t]);
#pragma unroll
                for (int h = 0; h < GPT; ++h) {
                    const int j = (4 * GPT * t) % 8 + GPT * g4 + h;
                    *reinterpret_cast<v4i_t*>(sO + 128 * l16 + ((j ^ (l16 & 7)) << 4)) = grp.g[h];
                }
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 8 * i + (lane >> 3), j = lane & 7;
                const v4i_t x = *reinterpret_cast<const v4i_t*>(sO + 128 * r + ((j ^ (r & 7)) << 4));
                ob.store(x, (row0 + r) * RBF + 128 * c + 16 * j);
            }
            __builtin_amdgcn_wave_barrier();
        }
    }

    // Outputs of the chunk starting at ts for the query strips of wave WV (the variant
    // used once D * Dv reaches 128 x 128, with one strip per wave).  The wave is a compile-time constant here, so its strips, their key-block counts and their
    // diagonal blocks are too: the loops below unroll into straight-line code in which
    // the strips' independent MFMA chains interleave.  Every S^T, phi(K) and V^T operand
    // is read from LDS once per wave and used for all strips that need it.
    //   carried part:  O^T += S^T Fq^T,  den += (z_hi, z_lo)^T Fq^T
    //   causal part, per 32-key block p:  A^T = Fk Fq^T (two 16-key tiles whose rows are
    //   ordered so lane group g holds keys 8g..8g+7), decay and, on the diagonal block
    //   only, the causal mask; then O^T += V^T A^T and den += ones A^T.
    template <int WV>
    __device__ __forceinline__ void outputs_w(const F8<E> (&fq)[Sh::MAXS][D / 32], int ts, const OutRsrc& ob,
                                              float eps, int norm) const {
        constexpr int MS = Sh::MAXS, NT = DV / 16, KS = D / 32, MAXP = (Sh::NSTRIP + 1) / 2;
        F8<E> ones_a;                  // rows 0, 4, 8, 12 of the denominator's A operand
#pragma unroll
        for (int e = 0; e < 8; ++e) ones_a.x[e] = X::from_f32((l16 & 3) == 0 ? 1.0f : 0.0f);
        const E* zrow = sZb + (l16 & 3) * Sh::LZ;   // z_hi, z_lo, 0, 0 by row mod 4
        auto strip = [](int m) { return strip_of<Sh::NSTRIP>(WV, m); };
        auto npairs = [&](int m) { return strip(m) < 0 ? 0 : strip(m) / 2 + 1; };
        f32x4_t acc[MS][NT];
        f32x4_t accd[MS];
        float lam_q[MS];
#pragma unroll
        for (int m = 0; m < MS; ++m) {
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            accd[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            lam_q[m] = 0.0f;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const F8<E> sop = lds_f8(sSt + st_off<D>(out_dv(t, l16), 32 * ks + 8 * g4));
#pragma unroll
                for (int m = 0; m < MS; ++m)
                    if (strip(m) >= 0) acc[m][t] = mma(sop, fq[m][ks], acc[m][t]);
            }
            const F8<E> zop = lds_f8(zrow + 32 * ks + 8 * g4);
#pragma unroll
            for (int m = 0; m < MS; ++m)
                if (strip(m) >= 0) accd[m] = mma(zop, fq[m][ks], accd[m]);
        }
        if constexpr (GATED) {
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                if (strip(m) < 0) continue;
                lam_q[m] = sLam[16 * strip(m) + l16];
                const float sc = fast_exp2(lam_q[m]);
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[m][t] *= sc;
                accd[m] *= sc;
            }
        }
        const int krow = 8 * (l16 >> 2) + (l16 & 3);
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            bool any = false;
#pragma unroll
            for (int m = 0; m < MS; ++m) any = any || p < npairs(m);
            if (!any) continue;
            F8<E> k0[KS], k1[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                k0[ks] = lds_f8(sK + tile_off<D>(32 * p + krow, 32 * ks + 8 * g4));
                k1[ks] = lds_f8(sK + tile_off<D>(32 * p + krow + 4, 32 * ks + 8 * g4));
            }
            f32x4_t l0 = {0.f, 0.f, 0.f, 0.f}, l1 = {0.f, 0.f, 0.f, 0.f};
            if constexpr (GATED) {
                l0 = *reinterpret_cast<const f32x4_t*>(sLam + 32 * p + 8 * g4);
                l1 = *reinterpret_cast<const f32x4_t*>(sLam + 32 * p + 8 * g4 + 4);
            }
            F8<E> bA[MS];
#pragma unroll
            for (int m = 0; m < MS; ++m) {
                if (p >= npairs(m)) continue;
                f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    a0 = mma(k0[ks], fq[m][ks], a0);
                    a1 = mma(k1[ks], fq[m][ks], a1);
                }
                const bool diag = p == npairs(m) - 1;
                const int qi = 16 * strip(m) + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x0 = a0[r], x1 = a1[r];
                    if constexpr (GATED) {
                        x0 *= fast_exp2(fminf(lam_q[m] - l0[r], 0.0f));
                        x1 *= fast_exp2(fminf(lam_q[m] - l1[r], 0.0f));
                    }
                    if (diag) {
                        const int kk = 32 * p + 8 * g4 + r;
                        x0 = kk <= qi ? x0 : 0.0f;
                        x1 = kk + 4 <= qi ? x1 : 0.0f;
                    }
                    bA[m].x[r] = X::from_f32(x0);
                    bA[m].x[4 + r] = X::from_f32(x1);
                }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const F8<E> vop = lds_f8(sVt + tidx(out_dv(t, l16), 4 * p + g4));
#pragma unroll
                for (int m = 0; m < MS; ++m)
                    if (p < npairs(m)) acc[m][t] = mma(vop, bA[m], acc[m][t]);
            }
#pragma unroll
            for (int m = 0; m < MS; ++m)
                if (p < npairs(m)) accd[m] = mma(ones_a, bA[m], accd[m]);
        }
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            if (strip(m) < 0) continue;
            const float inv = norm ? __builtin_amdgcn_rcpf(fmaxf(accd[m][0] + accd[m][1], eps)) : 1.0f;
            F8<E> outv[NT / 2];
#pragma unroll
            for (int t = 0; t < NT / 2; ++t) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    outv[t].x[r] = X::from_f32(acc[m][2 * t][r] * inv);
                    outv[t].x[4 + r] = X::from_f32(acc[m][2 * t + 1][r] * inv);
                }
            }
            store_strip(outv, ts + 16 * strip(m), ob);
        }
    }

    // One 32-key block p of the causal part for query strip s (query row qi of this
    // lane), for the strip-by-strip variant below: A^T tiles, decay and mask (DIAG: the
    // block holding the diagonal), then O^T += V^T A^T and den += ones A^T.
    template <bool DIAG>
    __device__ __forceinline__ void pair(int p, int qi, float lam_q, const F8<E> (&fqm)[D / 32], const F8<E>& ones_a,
                                         f32x4_t (&acc)[DV / 16], f32x4_t& accd) const {
        // Row m of the first A^T tile is key 8(m/4) + m%4 of the block and row m of the
        // second is that key + 4, so lane group g holds keys 8g..8g+7 of the block.
        const int krow = 8 * (l16 >> 2) + (l16 & 3);
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            a0 = mma(lds_f8(sK + tile_off<D>(32 * p + krow, 32 * ks + 8 * g4)), fqm[ks], a0);
            a1 = mma(lds_f8(sK + tile_off<D>(32 * p + krow + 4, 32 * ks + 8 * g4)), fqm[ks], a1);
        }
        f32x4_t l0 = {0.f, 0.f, 0.f, 0.f}, l1 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (GATED) {
            l0 = *reinterpret_cast<const f32x4_t*>(sLam + 32 * p + 8 * g4);
            l1 = *reinterpret_cast<const f32x4_t*>(sLam + 32 * p + 8 * g4 + 4);
        }
        F8<E> bA;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x0 = a0[r], x1 = a1[r];
            if constexpr (GATED) {
                x0 *= fast_exp2(fminf(lam_q - l0[r], 0.0f));
                x1 *= fast_exp2(fminf(lam_q - l1[r], 0.0f));
            }
            if constexpr (DIAG) {
                const int k0 = 32 * p + 8 * g4 + r;
                x0 = k0 <= qi ? x0 : 0.0f;
                x1 = k0 + 4 <= qi ? x1 : 0.0f;
            }
            bA.x[r] = X::from_f32(x0);
            bA.x[4 + r] = X::from_f32(x1);
        }
#pragma unroll
        for (int t = 0; t < DV / 16; ++t) acc[t] = mma(lds_f8(sVt + tidx(out_dv(t, l16), 4 * p + g4)), bA, acc[t]);
        accd = mma(ones_a, bA, accd);
    }
    // Outputs strip by strip with a runtime block loop: fewer live registers; the
    // faster variant while the operand tiles are small (D * Dv below 128 x 128), and the
    // one that fits the registers when a wave holds several strips of 128 x 128 tiles.
    __device__ __forceinline__ void outputs_seq(const F8<E> (&fq)[Sh::MAXS][D / 32], int ts, const OutRsrc& ob,
                                                float eps, int norm) const {
        F8<E> ones_a;                  // rows 0, 4, 8, 12 of the denominator's A operand
#pragma unroll
        for (int e = 0; e < 8; ++e) ones_a.x[e] = X::from_f32((l16 & 3) == 0 ? 1.0f : 0.0f);
        const E* zrow = sZb + (l16 & 3) * Sh::LZ;   // z_hi, z_lo, 0, 0 by row mod 4
#pragma unroll
        for (int m = 0; m < Sh::MAXS; ++m) {
            const int s = strip_of<Sh::NSTRIP>(w, m);
            if (s < 0) continue;
            const int qi = 16 * s + l16;
            f32x4_t acc[DV / 16];
#pragma unroll
            for (int t = 0; t < DV / 16; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            f32x4_t accd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
                for (int t = 0; t < DV / 16; ++t)
                    acc[t] = mma(lds_f8(sSt + st_off<D>(out_dv(t, l16), 32 * ks + 8 * g4)), fq[m][ks], acc[t]);
                accd = mma(lds_f8(zrow + 32 * ks + 8 * g4), fq[m][ks], accd);
            }
            float lam_q = 0.0f;
            if constexpr (GATED) {
                lam_q = sLam[qi];
                const float sc = fast_exp2(lam_q);
#pragma unroll
                for (int t = 0; t < DV / 16; ++t) acc[t] *= sc;
                accd *= sc;
            }
            const int npairs = s / 2 + 1;
            for (int p = 0; p + 1 < npairs; ++p) pair<false>(p, qi, lam_q, fq[m], ones_a, acc, accd);
            pair<true>(npairs - 1, qi, lam_q, fq[m], ones_a, acc, accd);
            const float inv = norm ? __builtin_amdgcn_rcpf(fmaxf(accd[0] + accd[1], eps)) : 1.0f;
            F8<E> outv[DV / 32];
#pragma unroll
            for (int t = 0; t < DV / 32; ++t) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    outv[t].x[r] = X::from_f32(acc[2 * t][r] * inv);
                    outv[t].x[4 + r] = X::from_f32(acc[2 * t + 1][r] * inv);
                }
            }
            store_strip(outv, ts + 16 * s, ob);
        }
    }

    // Outputs of the chunk starting at ts for this wave's query strips (w is uniform).
    __device__ __forceinline__ void outputs(const F8<E> (&fq)[Sh::MAXS][D / 32], int ts, const OutRsrc& ob,
                                            float eps, int norm) const {
        if constexpr (D * DV < 128 * 128 || Sh::MAXS > 1) {
            outputs_seq(fq, ts, ob, eps, norm);
        } else {
            switch (w) {
                case 0: outputs_w<0>(fq, ts, ob, eps, norm); break;
                case 1: outputs_w<1>(fq, ts, ob, eps, norm); break;
                case 2: outputs_w<2>(fq, ts, ob, eps, norm); break;
                default: outputs_w<3>(fq, ts, ob, eps, norm); break;
            }
        }
    }
};

// Accumulator-layout element r of state tile j of wave w, lane (l16, g4):
// S[16a + 4 g4 + r][16b + l16] with a = w ZT + j / NB, b = j % NB; z tile i of wave w
// holds z[16(w ZT + i) + 4 g4 + r] in its l16 == 0 lanes (zero elsewhere).
// The state in front of segment `seg` of head bh (column part `part`), in the
// accumulator layout of wave w's tiles: S0 (or zero) plus, with the direct prefix, the
// totals of the segments in front, decayed; else the scanned slot in front of it.
template <typename Sh, bool GATED, int DV, int VS>
__device__ __forceinline__ void segment_prefix(const WalkArgs& args, int bh, int part, int seg, size_t slot0, int w,
                                               int lane, int l16, int g4, f32x4_t (&sacc)[Sh::TPW],
                                               f32x4_t (&zacc)[Sh::ZT]) {
    constexpr int D = Sh::NA * 16, DVF = DV * VS;
    auto st_at = [&](int s, int j) {
        return args.st + (slot0 + s) * (D * DV) + ((w * Sh::TPW + j) * kWave + lane) * 4;
    };
    auto zt_at = [&](int s, int i) { return args.zt + (slot0 + s) * D + 16 * (w * Sh::ZT + i) + 4 * g4; };
    auto get4 = [](const float* p) { return *reinterpret_cast<const f32x4_t*>(p); };
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    if (args.direct || seg == 0) {
        if (args.s0) {
            const float* s0b = args.s0 + size_t(bh) * D * DVF + part * DV;
#pragma unroll
            for (int j = 0; j < Sh::TPW; ++j) {
                const int u = w * Sh::TPW + j;
                const int a = u / Sh::NB, b = u % Sh::NB;
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[j][r] = s0b[size_t(16 * a + 4 * g4 + r) * DVF + 16 * b + l16];
            }
        }
        if (args.z0) {
            const float* z0b = args.z0 + size_t(bh) * D;
#pragma unroll
            for (int i = 0; i < Sh::ZT; ++i) {
                const f32x4_t zv = get4(z0b + 16 * (w * Sh::ZT + i) + 4 * g4);
                zacc[i] = l16 == 0 ? zv : zero4;
            }
        }
        if (args.direct) {
            const float* lgb = args.lg + slot0;
#pragma unroll 2
            for (int s = 0; s < seg * args.tparts; ++s) {   // every part of every segment in front
                const float f = GATED ? fast_exp2(lgb[s]) : 1.0f;
#pragma unroll
                for (int j = 0; j < Sh::TPW; ++j) sacc[j] = f * sacc[j] + get4(st_at(s, j));
#pragma unroll
                for (int i = 0; i < Sh::ZT; ++i) {
                    const f32x4_t zv = get4(zt_at(s, i));
                    zacc[i] = f * zacc[i] + (l16 == 0 ? zv : zero4);
                }
            }
        }
    } else {
        const int pre = seg * args.tparts - 1;     // the scanned slot in front of the segment
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j) sacc[j] = get4(st_at(pre, j));
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i) {
            const f32x4_t zv = get4(zt_at(pre, i));
            zacc[i] = l16 == 0 ? zv : zero4;
        }
    }
}

// Waves per SIMD a walk kernel is compiled for: the shape's, or with FAVOR's W tiles in
// the LDS as many workgroups as then fit.
template <typename Sh>
constexpr int walk_kernel_waves(bool favor) {
    if (!favor) return Sh::kWaves;
    const int lds = int(kMaxLds / (Sh::kBytes + favor_lds_bytes(Sh::NA * 16)));
    const int v = lds < Sh::kWaves ? lds : Sh::kWaves;
    return v < 1 ? 1 : v;
}

// VS column parts of DV columns each (VS = 1: the whole of Dv = DV).  The workspace
// slots are per (head, column part): slot (bh * VS + part) * nslots + t holds that
// part's [D, DV] slice of the state and its own copy of z.
template <typename E, int D, int DV, int CH, bool GATED, bool OUTPUT, bool IDENT = false, bool RELU = false,
          int VS = 1, bool SPLITK = false, bool FAVOR = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    walk_kernel_waves<WalkShape<E, D, DV, CH, GATED, OUTPUT>>(FAVOR),
    walk_kernel_waves<WalkShape<E, D, DV, CH, GATED, OUTPUT>>(FAVOR)))) void walk_kernel(WalkArgs args) {
    using Sh = WalkShape<E, D, DV, CH, GATED, OUTPUT>;
    using W = ChunkWalker<E, D, DV, CH, GATED, OUTPUT, IDENT, RELU, VS, SPLITK, FAVOR>;
    constexpr int DVF = DV * VS;
    extern __shared__ __align__(16) unsigned char smem[];

    // the totals skip the last segment and cut the others into tparts parts
    const int nsw = OUTPUT ? args.nseg : (args.nseg - 1) * args.tparts;
    int item, part;
    walk_block<VS, OUTPUT>(args.BH * nsw, item, part);
    if (item >= args.BH * nsw) return;                      // padding block (uniform over the workgroup)
    const int sub = item % nsw;                             // segment (output) or totals slot
    const int bh = item / nsw;
    const int seg = OUTPUT ? sub : sub / args.tparts;
    const int N = args.N;
    const int nchunks_total = (N + CH - 1) / CH;
    int c0 = seg * args.L, nch = min(args.L, nchunks_total - c0);
    if constexpr (!OUTPUT) {
        // part sub % tparts of the segment; a part past the segment's chunks is empty
        const int lp = (args.L + args.tparts - 1) / args.tparts;
        const int end = c0 + nch;
        c0 += (sub % args.tparts) * lp;
        nch = max(0, min(lp, end - c0));
        c0 = min(c0, end);
    }

    W wk;
    if constexpr (RELU) wk.fshift = args.fshift;
    wk.init(smem, N, reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D,
            reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D,
            reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DVF + part * DV,
            GATED ? args.g + size_t(bh) * N : nullptr);
    wk.stream_kv = __builtin_amdgcn_readfirstlane(args.stream_kv);
    const int w = wk.w, lane = wk.lane, l16 = wk.l16, g4 = wk.g4;
    if constexpr (FAVOR) wk.stage_w(args.W + size_t(bh % args.H) * D * D);
    OutRsrc ob;
    if constexpr (OUTPUT)
        ob.init(reinterpret_cast<E*>(args.o) + size_t(bh) * N * DVF + part * DV,
                unsigned(N) * DVF * sizeof(E) - unsigned(part * DV * sizeof(E)));
    const size_t slot0 = (size_t(bh) * VS + part) * args.nslots;
    auto st_at = [&](int s, int j) {
        return args.st + (slot0 + s) * (D * DV) + ((w * Sh::TPW + j) * kWave + lane) * 4;
    };
    auto zt_at = [&](int s, int i) { return args.zt + (slot0 + s) * D + 16 * (w * Sh::ZT + i) + 4 * g4; };
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};

    f32x4_t sacc[Sh::TPW];
    f32x4_t zacc[Sh::ZT];
#pragma unroll
    for (int j = 0; j < Sh::TPW; ++j) sacc[j] = zero4;
#pragma unroll
    for (int i = 0; i < Sh::ZT; ++i) zacc[i] = zero4;
    const bool final_seg = seg == args.nseg - 1;

    // P_seg (output walk): from S0 and the totals in front (direct) or from the scanned
    // slot, formed while the first chunk's loads are in flight.
    auto prologue = [&]() {
        if constexpr (OUTPUT) {
            segment_prefix<Sh, GATED, DV, VS>(args, bh, part, seg, slot0, w, lane, l16, g4, sacc, zacc);
            wk.clear_zb();
            wk.stage_state(sacc, zacc);
        }
    };
    float lg_total = 0.0f;
    const bool keep = !OUTPUT || (final_seg && args.want_final);

    wk.walk(c0, nch, sacc, zacc, lg_total, ob, args.eps, args.normalize, keep, prologue);

    if (keep) {
        const int slot = OUTPUT ? args.nslots - 1 : sub;
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j) *reinterpret_cast<f32x4_t*>(st_at(slot, j)) = sacc[j];
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i)
            if (l16 == 0) *reinterpret_cast<f32x4_t*>(zt_at(slot, i)) = zacc[i];
        if (!OUTPUT && GATED && wk.tid == 0) args.lg[slot0 + slot] = lg_total;
    }
}

// The output walk with its work split between two kinds of wave (bf16, ungated): 8 waves
// in one workgroup per CU, two per SIMD.  At D = Dv = 128 and 64-token chunks the 4-wave
// walk would hold one workgroup per CU; at D = Dv = 64 and 128-token chunks it holds two,
// but one workgroup per CU halves the segments, and with them the keys and values the
// totals walk reads.  Waves 0-3 (output waves) take the chunk's 16-query strips, one each
// at 64 tokens, strips w and 7 - w at 128 (the same causal work per wave): they load Q,
// apply phi and form the strips' outputs from S^T, phi(K) and V^T in LDS.  Waves 4-7 (state waves) hold the carried state in their accumulators as
// the 4-wave walk does: they load K and V, stage phi(K) and V^T, fold the chunk into the
// state and stage S^T and z for the next chunk.  Both keep the loads of two chunks in
// flight.  Every tile the two kinds share has two LDS buffers, so that the kinds meet at
// one barrier per chunk: while the output waves form chunk n's outputs from buffer
// n mod 2, the state waves fold chunk n from the same buffer and stage chunk n + 1 (its
// phi(K), V^T and the state in front of it) into the other.  One SIMD runs an output
// wave and a state wave side by side, so that the VALU, LDS and MFMA work and the waits
// of the two overlap, and either kind's lighter phase fills the other's heavier one.
constexpr int kSplitThreads = 2 * kThreads;

template <typename E, int D, int DV, int CH, bool RELU = false>
struct SplitShape {
    using W = ChunkWalker<E, D, DV, CH, false, true, false, RELU>;
    using Sh = typename W::Sh;
    // Its own carve-up: each tile's two buffers side by side, so that one register holds
    // a lane's address in both (the second is the first plus an instruction's immediate
    // offset, under 64 KiB).
    static constexpr size_t kK = size_t(CH) * D * sizeof(E);
    static constexpr size_t kVt = size_t(DV) * Sh::LKT * sizeof(E);
    static constexpr size_t kSt = size_t(DV) * Sh::LS * sizeof(E);
    static constexpr size_t kZb = size_t(4) * Sh::LZ * sizeof(E);
    static constexpr size_t kOffK = 0;
    static constexpr size_t kOffVt = kOffK + 2 * kK;
    static constexpr size_t kOffSt = kOffVt + 2 * kVt;
    static constexpr size_t kOffZb = kOffSt + 2 * kSt;
    static constexpr size_t kOffLam = kOffZb + 2 * kZb;
    static constexpr size_t kOffO = kOffLam + size_t(CH) * 4;
    static constexpr size_t kBytes = kOffO + size_t(kThreads / kWave) * Sh::kOBlock;
    static_assert(kK < 65536 && kVt < 65536 && kSt < 65536 && kZb < 65536, "buffer pairs within an immediate offset");
    static_assert((Sh::MAXS == 1 && Sh::NSTRIP == 4) || (Sh::MAXS == 2 && Sh::NSTRIP == 8),
                  "one query strip per output wave, or two (strips w and 7 - w: equal causal work)");
    static_assert(Sh::kRowK && !Sh::kKT && !Sh::kVD, "the walk stages the row-major phi(K) tile and V^T only");
    static_assert(kBytes == split_walk_lds_bytes(int(sizeof(E)), D, DV, CH), "host LDS formula out of step");
};

template <typename E, int D, int DV, int CH, bool RELU = false>
__global__ __launch_bounds__(kSplitThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void walk_split_kernel(
    WalkArgs args) {
    using SS = SplitShape<E, D, DV, CH, RELU>;
    using W = typename SS::W;
    using Sh = typename SS::Sh;
    extern __shared__ __align__(16) unsigned char smem[];

    const int item = blockIdx.x;
    const int seg = item % args.nseg;
    const int bh = item / args.nseg;
    const int N = args.N;
    const int nchunks_total = (N + CH - 1) / CH;
    const int c0 = seg * args.L, nch = min(args.L, nchunks_total - c0);

    // the 4-wave walker's members, renumbered within each kind of wave
    W wk;
    if constexpr (RELU) wk.fshift = args.fshift;
    wk.init(smem, N, reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D,
            reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D,
            reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV, nullptr);
    const bool state_wave = threadIdx.x >= kThreads;       // uniform over each wave
    wk.tid = threadIdx.x % kThreads;
    wk.w = __builtin_amdgcn_readfirstlane(wk.tid / kWave);
    wk.sO = smem + SS::kOffO + size_t(wk.w) * Sh::kOBlock;
    wk.sLam = reinterpret_cast<float*>(smem + SS::kOffLam);
    wk.last = min(N, (c0 + max(nch, 1)) * CH) - 1;
    E* const k_buf[2] = {reinterpret_cast<E*>(smem + SS::kOffK), reinterpret_cast<E*>(smem + SS::kOffK + SS::kK)};
    E* const vt_buf[2] = {reinterpret_cast<E*>(smem + SS::kOffVt), reinterpret_cast<E*>(smem + SS::kOffVt + SS::kVt)};
    E* const st_buf[2] = {reinterpret_cast<E*>(smem + SS::kOffSt), reinterpret_cast<E*>(smem + SS::kOffSt + SS::kSt)};
    E* const zb_buf[2] = {reinterpret_cast<E*>(smem + SS::kOffZb), reinterpret_cast<E*>(smem + SS::kOffZb + SS::kZb)};
    wk.sK = k_buf[0];
    wk.sVt = vt_buf[0];
    wk.sSt = st_buf[0];
    wk.sZb = zb_buf[0];
    const int w = wk.w, lane = wk.lane, l16 = wk.l16, g4 = wk.g4;

    OutRsrc ob;
    ob.init(reinterpret_cast<E*>(args.o) + size_t(bh) * N * DV, unsigned(N) * DV * sizeof(E));
    const size_t slot0 = size_t(bh) * args.nslots;
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    const bool keep = seg == args.nseg - 1 && args.want_final;

    // Each kind of wave runs its own loop, so that neither holds the other's registers;
    // both meet at one barrier before the first chunk and one after each chunk (nch is
    // uniform over the workgroup, and the kind of wave is uniform over each wave).
    if (state_wave) {
        f32x4_t sacc[Sh::TPW];
        f32x4_t zacc[Sh::ZT];
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j) sacc[j] = zero4;
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i) zacc[i] = zero4;
        // two register sets of K and V: the loads of chunks n + 2 and n + 3 are in flight
        // while chunk n + 1 is staged (three sets would spill)
        typename W::Regs R0, R1;
        wk.load(R0, c0 * CH);
        wk.load(R1, (c0 + 1) * CH);
        segment_prefix<Sh, false, DV, 1>(args, bh, 0, seg, slot0, w, lane, l16, g4, sacc, zacc);
        auto stage_chunk = [&](typename W::Regs& R, int n) {
            const int ts = (c0 + n) * CH;
            wk.sK = k_buf[n & 1];
            wk.sVt = vt_buf[n & 1];
            if (ts + CH <= N)
                wk.template stage<false>(R, ts, 0.0f);
            else
                wk.template stage<true>(R, ts, 0.0f);
            wk.load(R, ts + 2 * CH);
        };
        // chunk 0 and the state in front of it into the first buffers
        wk.sZb = zb_buf[0];
        wk.clear_zb();
        wk.stage_state(sacc, zacc);
        if (nch > 0) stage_chunk(R0, 0);
        __syncthreads();
        // chunk n: stage chunk n + 1 (R_next) into the other buffers, fold chunk n from
        // buffer n & 1 and stage the state after it beside chunk n + 1
        auto step = [&](typename W::Regs& R_next, int n) {
            const bool more = n + 1 < nch;
            if (more) stage_chunk(R_next, n + 1);
            wk.sK = k_buf[n & 1];
            wk.sVt = vt_buf[n & 1];
            if (more || keep) wk.fold(sacc, zacc, 0.0f);
            if (more) {
                wk.sSt = st_buf[(n + 1) & 1];
                wk.sZb = zb_buf[(n + 1) & 1];
                wk.stage_state(sacc, zacc);
            }
            __syncthreads();
        };
        for (int n = 0; n < nch; n += 2) {
            step(R1, n);
            if (n + 1 < nch) step(R0, n + 1);
        }
        if (keep) {
            const size_t slot = slot0 + args.nslots - 1;
#pragma unroll
            for (int j = 0; j < Sh::TPW; ++j)
                *reinterpret_cast<f32x4_t*>(args.st + slot * (D * DV) + ((w * Sh::TPW + j) * kWave + lane) * 4) =
                    sacc[j];
#pragma unroll
            for (int i = 0; i < Sh::ZT; ++i)
                if (l16 == 0)
                    *reinterpret_cast<f32x4_t*>(args.zt + slot * D + 16 * (w * Sh::ZT + i) + 4 * g4) = zacc[i];
        }
    } else {
        // two register sets of Q, as for K and V
        typename W::QRegs q0, q1;
        wk.load_q(q0, c0 * CH);
        wk.load_q(q1, (c0 + 1) * CH);
        wk.sZb = zb_buf[1];
        wk.clear_zb();
        __syncthreads();
        auto step = [&](typename W::QRegs& qr, int n) {
            const int ts = (c0 + n) * CH;
            F8<E> fq[Sh::MAXS][D / 32];
            wk.phi_q(qr, fq);
            wk.load_q(qr, ts + 2 * CH);
            wk.sSt = st_buf[n & 1];
            wk.sZb = zb_buf[n & 1];
            wk.sK = k_buf[n & 1];
            wk.sVt = vt_buf[n & 1];
            // at D = Dv = 64 the per-wave straight-line form (both strips' operands read
            // once); at 128 x 128 the strip with a runtime key-block loop, since the
            // straight-line form holds more operands than two waves per SIMD leave
            // registers for
            if constexpr (D * DV < 128 * 128) {
                switch (w) {
                    case 0: wk.template outputs_w<0>(fq, ts, ob, args.eps, args.normalize); break;
                    case 1: wk.template outputs_w<1>(fq, ts, ob, args.eps, args.normalize); break;
                    case 2: wk.template outputs_w<2>(fq, ts, ob, args.eps, args.normalize); break;
                    default: wk.template outputs_w<3>(fq, ts, ob, args.eps, args.normalize); break;
                }
            } else {
                wk.outputs_seq(fq, ts, ob, args.eps, args.normalize);
            }
            __syncthreads();
        };
        for (int n = 0; n < nch; n += 2) {
            step(q0, n);
            if (n + 1 < nch) step(q1, n + 1);
        }
    }
}

// In place over the first nscan of each head's nslots slots: slot s becomes
// P_{s+1} = 2^lg_s P_s + T_s with P_0 = S0 (fp32), one thread per state element.  Only
// the slots that a reader takes are written back: every keep-th (s + 1 a multiple of
// keep; keep = the parts per segment, whose prefixes are read only at segment starts).
// Element e < D*Dv is in accumulator layout: tile u = e / 256 (a = u / (Dv/16),
// b = u % (Dv/16)), lane = (e / 4) % 64, r = e % 4, which is S[16a + 4(lane/16) + r][16b + lane%16].
// With VS column parts the slots are per (head, part), vbh = bh * VS + part, each a
// [D][DV] slice whose initial value is columns part * DV .. of the caller's S0 rows.
template <int D, int DV, bool GATED, int VS = 1>
__global__ __launch_bounds__(kThreads) void scan_kernel(float* st, float* zt, const float* lg, const float* s0,
                                                       const float* z0, int nslots, int nscan, int keep) {
    constexpr int NS = D * DV;
    constexpr int NBLK = (NS + D + kThreads - 1) / kThreads;   // workgroups per head and part
    const int e = (blockIdx.x % NBLK) * kThreads + threadIdx.x;
    const int vbh = blockIdx.x / NBLK;
    const int bh = vbh / VS, part = vbh % VS;
    if (e >= NS + D) return;
    float* base;
    size_t stride;
    size_t uidx;      // index into the caller's [D][Dv] or [D] layout
    const float* init;
    if (e < NS) {
        const int u = e / 256, lane = (e / 4) % 64, r = e % 4;
        const int a = u / (DV / 16), b = u % (DV / 16);
        const int d = 16 * a + 4 * (lane / 16) + r, dv = 16 * b + lane % 16;
        uidx = size_t(bh) * NS * VS + size_t(d) * DV * VS + part * DV + dv;
        base = st + size_t(vbh) * nslots * NS + e;
        stride = NS;
        init = s0;
    } else {
        const int d = e - NS;
        uidx = size_t(bh) * D + d;
        base = zt + size_t(vbh) * nslots * D + d;
        stride = D;
        init = z0;
    }
    const float* lgb = GATED ? lg + size_t(vbh) * nslots : nullptr;
    const int n = nscan;
    float acc = init ? init[uidx] : 0.0f;
    constexpr int U = 8;                         // loads in flight per thread
    for (int s0i = 0; s0i < n; s0i += U) {
        float t[U], f[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int s = min(s0i + i, n - 1);
            t[i] = base[size_t(s) * stride];
            f[i] = GATED ? fast_exp2(lgb[s]) : 1.0f;
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (s0i + i < n) {
                acc = f[i] * acc + t[i];
                if ((s0i + i + 1) % keep == 0) base[size_t(s0i + i) * stride] = acc;
            }
        }
    }
}

// One state slot (accumulator layout; nslots per head) into the caller's [D][Dv] and [D]
// layouts: S_N, z_N from the forward's last slot.  A launch of its own, so s_out may
// alias s0 (every read of s0 is done by then).
// With VS column parts, slot vbh = bh * VS + part fills columns part * DV .. of S_N's
// rows, and part 0's copy of z gives z_N.
template <int D, int DV, int VS = 1>
__global__ __launch_bounds__(kThreads) void final_kernel(const float* st, const float* zt, int nslots, int which,
                                                        float* s_out, float* z_out) {
    constexpr int NS = D * DV;
    constexpr int NBLK = (NS + D + kThreads - 1) / kThreads;
    const int e = (blockIdx.x % NBLK) * kThreads + threadIdx.x;
    const int vbh = blockIdx.x / NBLK;
    const int bh = vbh / VS, part = vbh % VS;
    if (e >= NS + D) return;
    const size_t slot = size_t(vbh) * nslots + which;
    if (e < NS) {
        if (!s_out) return;
        const int u = e / 256, lane = (e / 4) % 64, r = e % 4;
        const int a = u / (DV / 16), b = u % (DV / 16);
        const int d = 16 * a + 4 * (lane / 16) + r, dv = 16 * b + lane % 16;
        s_out[size_t(bh) * NS * VS + size_t(d) * DV * VS + part * DV + dv] = st[slot * NS + e];
    } else {
        if (!z_out || part != 0) return;
        z_out[size_t(bh) * D + (e - NS)] = zt[slot * D + (e - NS)];
    }
}

}  // namespace linattn
