// Host-side launch interface between the C ABI (api.hip) and the kernel
// instantiations (fwd_*.hip, decode.hip).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace linattn {

struct FwdLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* g;          // NULL: ungated
    void* o;
    const float* s0;
    const float* z0;
    float* s_out;
    float* z_out;
    void* ws;                // caller's workspace, carved by fwd_workspace_layout
    int BH, N, D, Dv, chunk, nseg, L;
    float eps;
    int normalize;           // 1: o = num / max(den, eps); 0: o = num
    hipStream_t stream;
    hipEvent_t prof[4];      // measurement hook: all NULL when unused
    float fshift = 0.0f;     // the walk under relu(x) + fshift features only
    int vsplit = 1;          // column parts of Dv walked by separate workgroups (walk_vsplit)
    int tparts = 1;          // parts of a segment walked by separate totals workgroups
    const float* W = nullptr;    // FAVOR walks: the projections [H][D][D] fp32
    int H = 1;
};

// Chunk sizes with kernel instantiations.
inline bool chunk_is_built(int chunk) { return chunk == 32 || chunk == 64 || chunk == 128 || chunk == 256; }

// Dynamic LDS bytes of a walk kernel for (element size, D, Dv, chunk, gated; out: the
// output walk, else the totals walk).  WalkShape<...>::kBytes is checked against it.
// The output walk always stages the row-major Fk tile, S^T and the split z rows; the
// transposed Fk^T copy is staged by the totals walk and, in fp32, by the output walk
// too; the gated bf16 output walk stages a decayed copy of V^T instead.
constexpr size_t kMaxLds = 160 * 1024;   // LDS per compute unit on gfx950
constexpr size_t kLastLevelCache = size_t(256) << 20;   // MI355X's memory-side cache

// Whether the forward's totals walk loads K and V non-temporally: when K and V together
// exceed the last-level cache, the output walk that reads them again cannot find them
// there, and the totals walk's loads need not displace anything for it.
constexpr bool totals_stream_kv(long BH, long N, int D, int Dv, int esize) {
    return size_t(BH) * size_t(N) * size_t(D + Dv) * size_t(esize) > kLastLevelCache;
}

// The walk's tiles with one row of chunk-local log2 decays (Lambda) for the workgroup.
constexpr size_t walk_lds_bytes_shared_lambda(int esize, int D, int Dv, int chunk, bool gated, bool out = true) {
    const size_t es = size_t(esize), lkt = size_t(chunk) + (chunk >= 128 ? 16 : 0);
    const bool kt = !out || esize != 2;
    const bool vd = out && gated && esize == 2;
    // the output walk also holds one 16-row x 128-byte block of o for each of its four waves
    return (out ? size_t(chunk) * D * es : 0) + (kt ? size_t(D) * lkt * es : 0) + size_t(Dv) * lkt * es +
           (vd ? size_t(Dv) * lkt * es + size_t(chunk) * es : 0) +
           (out ? size_t(Dv) * D * es + size_t(4) * (D + 8) * es : 0) + size_t(chunk) * 4 +
           (out ? size_t(4) * 16 * 128 : 0);
}

// Whether each wave of a gated walk forms and keeps its own row of Lambda (no barrier
// between the gates' scan and its first use): wherever the three more rows fit the LDS.
constexpr bool walk_lambda_per_wave(int esize, int D, int Dv, int chunk, bool gated, bool out = true) {
    return gated && walk_lds_bytes_shared_lambda(esize, D, Dv, chunk, gated, out) + size_t(3) * chunk * 4 <= kMaxLds;
}

// Dynamic LDS bytes of a walk kernel (WalkShape<...>::kBytes is checked against it).
constexpr size_t walk_lds_bytes(int esize, int D, int Dv, int chunk, bool gated, bool out = true) {
    return walk_lds_bytes_shared_lambda(esize, D, Dv, chunk, gated, out) +
           (walk_lambda_per_wave(esize, D, Dv, chunk, gated, out) ? size_t(3) * chunk * 4 : 0);
}

// Whether the output walk of a shape runs as the split 8-wave walk (walk_split_kernel),
// one workgroup per CU: bf16, ungated, features elu + 1 or relu + shift, Dv uncut, and
// D = Dv = 128 with 64-token chunks or D = Dv = 64 with 128-token chunks.
constexpr bool walk_split(int esize, int D, int Dv, int chunk, bool gated) {
    return esize == 2 && !gated && ((D == 128 && Dv == 128 && chunk == 64) || (D == 64 && Dv == 64 && chunk == 128));
}

// LDS the FAVOR walks add after the shape's tiles: W's high and low parts, [D][D + 8]
// bf16 each.
constexpr size_t favor_lds_bytes(int D) { return size_t(2) * D * (D + 8) * 2; }

// Its LDS: the 4-wave output walk's tiles plus a second S^T and split-z buffer, a second
// phi(K) tile and a second V^T tile.
constexpr size_t split_walk_lds_bytes(int esize, int D, int Dv, int chunk) {
    return walk_lds_bytes(esize, D, Dv, chunk, false, true) + size_t(Dv) * D * esize + size_t(4) * (D + 8) * esize +
           size_t(chunk) * D * esize + size_t(Dv) * (chunk + (chunk >= 128 ? 16 : 0)) * esize;
}

// Waves per SIMD a walk kernel is compiled for (one wave of every workgroup sits on each
// SIMD, so this is also its workgroups per compute unit): what its LDS allows, capped by
// the register budget its shape can live with.  The plan sizes one round of the output
// walk with it, and the totals walk's parts (totals_parts) fill one round of its own.
// The totals walk holds no outputs and fits two waves at every shape but the gated one
// at D = Dv = 128 from 128-token chunks (at D = Dv = 128, chunk 64: one wave gave 220 us
// for the long-context totals, two with twice the workgroups 166 us).
constexpr int walk_waves(int esize, int D, int Dv, int chunk, bool gated, bool out) {
    const int lds = int(kMaxLds / walk_lds_bytes(esize, D, Dv, chunk, gated, out));
    const int work = D * Dv * (esize == 2 ? 1 : 2) * (chunk > 128 ? 2 : 1);   // grows with the live tiles
    int regs = out || (gated && work >= 128 * 128 && chunk >= 128) ? 1 : 2;
    if (work <= 64 * 64) regs = out ? 2 : 3;
    else if (work <= 2 * 64 * 64) regs = out ? 1 : 2;
    const int v = lds < regs ? lds : regs;
    return v < 1 ? 1 : v;
}

// Column parts the forward cuts the value dimension into (each part walked by its own
// workgroups with a [D, Dv / parts] slice of the state): 1 when the full-width tiles fit
// the LDS, else 2 when Dv = 128 and the 64-column tiles do, else 0 (not supported).
constexpr int walk_vsplit(int esize, int D, int Dv, int chunk, bool gated) {
    if (walk_lds_bytes(esize, D, Dv, chunk, gated) <= kMaxLds) return 1;
    if (Dv == 128 && walk_lds_bytes(esize, D, 64, chunk, gated) <= kMaxLds) return 2;
    return 0;
}

// Prefetch depth of a walk kernel: chunks whose K, V (and Q) loads are in flight ahead
// of the chunk being processed.  Two for the ungated 128 x 128 output walks of chunks up
// to 64 tokens: one workgroup per compute unit leaves them only their own loads to hide
// HBM latency, and a second register set fits (the gated output walk would spill; the
// totals walk would drop to one wave per SIMD).
constexpr int walk_depth(int esize, int D, int Dv, int chunk, bool gated, bool out) {
    return out && esize == 2 && !gated && D * Dv >= 128 * 128 && chunk <= 64 ? 2 : 1;
}

inline size_t round_up256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the forward: per-segment states [BH][nseg][D*Dv], z [BH][nseg][D], log2
// decays [BH][nseg] (float), each region 256-byte aligned.
inline size_t fwd_workspace_layout(size_t slots, int D, int Dv, size_t* off_zt, size_t* off_lg) {
    const size_t st = round_up256(slots * size_t(D) * Dv * 4);
    const size_t zt = round_up256(slots * size_t(D) * 4);
    if (off_zt) *off_zt = st;
    if (off_lg) *off_lg = st + zt;
    return st + zt + round_up256(slots * 4);
}

// The output walk sums the totals in front of its segment itself when they are few
// and small (at most seven 64 x 64 states, with one part per segment; totals_parts keeps
// the parts within the same budget); otherwise a scan launch does it first.
inline bool prefix_direct(int nseg, int D, int Dv) { return size_t(nseg - 1) * D * Dv <= size_t(7) * 64 * 64; }

// Parts each segment's total is cut into, where the totals walk's (nseg - 1) segments
// per head alone can leave compute units idle: as many as fill one round of that walk
// with a scanned prefix, half of one with the direct prefix (whose output walk reads
// every part in front of its segment, within the direct prefix's budget), at most one
// per chunk.
inline int totals_parts(long heads, int nseg, int L, int D, int Dv, long round) {
    if (nseg <= 1) return 1;
    long p = round / (heads * long(nseg - 1));
    if (p < 1) p = 1;
    if (p > L) p = L;
    if (prefix_direct(nseg, D, Dv)) {
        // parts only where the segments alone would fill less than half a round, and then
        // as many as fill half of it: the output walk sums every part in front of its
        // segment (train_bf16: three parts 73-75 us, six 75-77 us), at most seven 64 x 64
        // states in all
        if (heads * long(nseg - 1) * 2 > round) return 1;
        p = round / (2 * heads * long(nseg - 1));
        if (p > L) p = L;
        const long cap = long(7) * 64 * 64 / (long(nseg - 1) * D * Dv);
        if (p > cap) p = cap < 1 ? 1 : cap;
    }
    // no empty parts: as many as parts of ceil(L / p) chunks take
    const long lp = (L + p - 1) / p;
    return int((L + lp - 1) / lp);
}

// Dynamic LDS bytes of a gradient kernel: phi(Q), phi(K) [C][D], V, dOut [C][Dv] and one
// state [D][Dv], each row padded by 16 bytes, plus the chunk's decays, dden, 1/d, the
// column and row sums of its pair terms and one fp32 [D] vector.  BwdShape<...>::kBytes
// is checked against it.
constexpr int kBwdChunkHost = 64;
constexpr size_t bwd_base_lds_bytes(int esize, int D, int Dv) {
    const size_t es = size_t(esize), pad = 16 / es, C = kBwdChunkHost;
    return (2 * C * (D + pad) + 2 * C * (Dv + pad) + size_t(D) * (Dv + pad)) * es + (8 * C + D) * 4;
}
// The low parts of phi(Q), phi(K) and of one state (bf16 operands split in two), where
// they fit beside the rest: every bf16 shape but D = Dv = 128.
constexpr size_t bwd_split_lds_bytes(int esize, int D, int Dv) {
    const size_t es = size_t(esize), pad = 16 / es, C = kBwdChunkHost;
    return (2 * C * (D + pad) + size_t(D) * (Dv + pad)) * es;
}
constexpr bool bwd_split(int esize, int D, int Dv) {
    return esize == 2 && bwd_base_lds_bytes(esize, D, Dv) + bwd_split_lds_bytes(esize, D, Dv) <= kMaxLds;
}
constexpr size_t bwd_lds_bytes(int esize, int D, int Dv) {
    return bwd_base_lds_bytes(esize, D, Dv) + (bwd_split(esize, D, Dv) ? bwd_split_lds_bytes(esize, D, Dv) : 0);
}

// Chunks per run of the passes that walk runs of chunks (the gradients' dq and dk/dv
// passes, the per-dimension decay's totals and outputs).  A workgroup walks a run and
// carries the states through it in registers, so the state traffic (a [D][Dv] fp32 slot
// read or written per run) falls with the run's length.  The runs per head are as many
// as one round of `per_cu` workgroups per compute unit holds, so the grid fills the
// device once, and the run is the chunks shared out over them (at most kBwdMaxRun).
constexpr int kBwdMaxRun = 16;
inline int bwd_chunks_per_group(long BH, int NC, int per_cu, int cus) {
    const long resident = long(cus) * long(per_cu < 1 ? 1 : per_cu);
    long runs = resident / BH;
    if (runs < 1) runs = 1;
    if (runs > NC) runs = NC;
    long run = (NC + runs - 1) / runs;
    if (run > kBwdMaxRun) run = kBwdMaxRun;
    return run < 1 ? 1 : int(run);
}

// Workspace of the backward: the state in front of every run and the runs' adjoint
// totals with their reverse scan (sized for runs of one chunk, NC and NC + 1 slots per
// head, so the size does not depend on the device), then five fp32 [BH][N] rows (1/d,
// dden and the three per-token pair sums of d log g) and one [BH][NC] row.
struct BwdLayout {
    size_t fwd, fzt, flg, rev, rzt, rlg, inv, dden, xs, yq, zk, wc, bytes;
};

inline BwdLayout bwd_workspace_layout(size_t BH, int N, int D, int Dv) {
    BwdLayout L;
    const size_t nc = (size_t(N) + kBwdChunkHost - 1) / kBwdChunkHost;
    size_t oz = 0, ol = 0;
    const size_t fb = fwd_workspace_layout(BH * nc, D, Dv, &oz, &ol);
    L.fwd = 0; L.fzt = oz; L.flg = ol;
    const size_t rb = fwd_workspace_layout(BH * (nc + 1), D, Dv, &oz, &ol);
    L.rev = fb; L.rzt = fb + oz; L.rlg = fb + ol;
    const size_t row = round_up256(BH * size_t(N) * 4);
    L.inv = fb + rb;
    L.dden = L.inv + row;
    L.xs = L.dden + row;
    L.yq = L.xs + row;
    L.zk = L.yq + row;
    L.wc = L.zk + row;
    L.bytes = L.wc + round_up256(BH * nc * 4);
    return L;
}

struct BwdLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* g;          // NULL: ungated
    const void* dout;
    const float* s0;
    const float* z0;
    void* dq;
    void* dk;
    void* dv;
    float* dg;               // NULL: not written (or ungated)
    float* ds0;              // NULL: not written
    float* dz0;              // NULL: not written
    void* ws;
    int BH, N, D, Dv;
    float eps;
    int normalize;
    int cus;                 // compute units of the device (sizes the runs)
    int run;                 // chunks per run; 0: chosen from the device's size
    hipStream_t stream;
};

// Dynamic LDS bytes of the per-dimension-decay kernels: phi(Q), phi(K) [C][D], V [C][Dv]
// and S_prev [D][Dv] (rows padded by 16 bytes), the decays [C][D + 4] and one [D] vector
// in fp32.  VdShape<...>::kBytes is checked against it.
constexpr size_t vd_lds_bytes(int esize, int D, int Dv) {
    const size_t es = size_t(esize), pad = 16 / es, C = kBwdChunkHost;
    return (2 * C * (D + pad) + C * (Dv + pad) + size_t(D) * (Dv + pad)) * es + C * (size_t(D) + 4) * 4 +
           size_t(D) * 4;
}

// Workspace of the per-dimension-decay forward, sized for runs of one chunk (the run
// length is chosen at launch): the state after every 64-token chunk
// [BH][NC][D*Dv], its z [BH][NC][D] and each chunk's log2 decay per dimension [BH][NC][D].
struct VdLayout {
    size_t st, zt, lg, bytes;
};

inline VdLayout vd_workspace_layout(size_t BH, int N, int D, int Dv) {
    VdLayout L;
    const size_t nc = (size_t(N) + kBwdChunkHost - 1) / kBwdChunkHost;
    size_t oz = 0, ol = 0;
    const size_t fb = fwd_workspace_layout(BH * nc, D, Dv, &oz, &ol);
    L.st = 0;
    L.zt = oz;
    L.lg = fb;
    L.bytes = fb + round_up256(BH * nc * size_t(D) * 4);
    return L;
}

struct VdLaunch {
    const void* q;
    const void* k;
    const void* v;
    const float* a;
    void* o;
    const float* s0;
    const float* z0;
    float* s_out;
    float* z_out;
    void* ws;
    int BH, N, D, Dv;
    float eps;
    int normalize;
    int cus;                 // compute units of the device (sizes the runs)
    hipStream_t stream;
};

hipError_t launch_vd_bf16(const VdLaunch& p);
hipError_t launch_vd_f32(const VdLaunch& p);

// A forward under another feature map.  Kind 1, relu + shift: the walk applies it while
// staging q and k.  Kind 2, FAVOR+ with W [H][M][D]: the features of q and k are written
// to the head of the workspace, then the walk of `fwd` runs over them with M state rows.
struct FeatLaunch {
    FwdLaunch fwd;           // q, k: the inputs; ws: the whole workspace; D: their width
    int kind;
    float shift;
    const float* W;
    int H, M, es;
    int BH, N, D;
    hipStream_t stream;
};

hipError_t launch_feature_fwd(const FeatLaunch& p);

hipError_t launch_fwd_bf16(const FwdLaunch& p);
hipError_t launch_fwd_f32(const FwdLaunch& p);
hipError_t launch_bwd_bf16(const BwdLaunch& p);
hipError_t launch_bwd_f32(const BwdLaunch& p);
hipError_t launch_decode(int dtype, const void* q, const void* k, const void* v, float* S, float* z, void* o,
                         int BH, int D, int Dv, float eps, const float* g, const float* ga, int normalize,
                         hipStream_t stream);

}  // namespace linattn
