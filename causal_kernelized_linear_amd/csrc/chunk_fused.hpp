// Single-pass chunked forward for gfx950: every workgroup walks one segment of one
// head twice, and the segments of a head hand their states to each other through
// global memory with a decoupled look-back, so no separate state pass or scan launch
// is needed and K and V come from HBM only once (the second walk finds them in the
// cache hierarchy).
//
// Per workgroup:
//   1. take a dispatch ticket (atomic counter); ticket t is segment t % nseg of head
//      t / nseg, so a segment's predecessors always hold smaller tickets and are
//      already running or done: every wait below is on work that can finish.
//   2. pass 1: walk the segment's chunks folding phi(K)^T V and phi(K)^T 1 into the
//      segment total T (and, gated, the log2 of its total decay); publish T as the
//      "aggregate" record and raise the segment's flag to 1.
//   3. look-back: walk predecessors j = s-1, s-2, ... adding their published records
//      (scaled by the decay between them and this segment) until one has its
//      "inclusive" record (flag 2) or the sequence start is reached (then S0, z0):
//      this gives P_s, the state in front of the segment.
//   4. publish the inclusive record Gamma_s P_s + T and raise the flag to 2.
//   5. pass 2: walk the segment's chunks from P_s forming the outputs (the same
//      per-chunk work as the three-launch path's output walk).
//
// Publication follows the HIP memory model at agent scope: every wave waits for its
// record stores before the workgroup barrier, thread 0 then stores the flag with
// release semantics, and the reader's thread 0 loads the flag and fences with acquire
// semantics before the barrier after which its workgroup reads the record.  Records are written once per launch and are 256-byte aligned, so
// no cache line is shared between records.  A wait that exceeds a bound of several
// tenths of a second gives up and poisons the segment's outputs with NaN, so the kernel
// always terminates.
//
// The flags and the ticket counter are cleared by a small kernel launched just before;
// the final state S_N, z_N is copied out by a third small kernel after, so no segment
// overwrites S0 while another may still read it (s_out may alias s0).
#pragma once

#include "chunk_walk.hpp"

namespace linattn {

struct FusedArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    void* o;
    const float* s0;
    const float* z0;
    float* rec;          // [BH][nseg][2][REC]: aggregate (0) and inclusive (1) records
    int* flags;          // [BH*nseg] segment flags, then the ticket counter
    int N;
    int nseg;
    int L;
    float eps;
};

// Record: [0, D*Dv) state in accumulator layout, [D*Dv, D*Dv + D) z, [D*Dv + D] log2
// of the segment's total decay; padded to a multiple of 64 floats (256 bytes).
template <int D, int DV>
struct Rec {
    static constexpr int kZ = D * DV;
    static constexpr int kLg = D * DV + D;
    static constexpr int kFloats = ((D * DV + D + 1 + 63) / 64) * 64;
};

constexpr int kSpinLimit = 1 << 22;

static __global__ __launch_bounds__(kThreads) void fused_clear_kernel(int* flags, int n) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) flags[i] = 0;
}

// Copies the inclusive record of every head's last segment into s_out / z_out.
template <int D, int DV>
__global__ __launch_bounds__(kThreads) void fused_final_kernel(const float* rec, int nseg, float* s_out,
                                                              float* z_out) {
    constexpr int NS = D * DV;
    constexpr int NBLK = (NS + D + kThreads - 1) / kThreads;
    const int e = (blockIdx.x % NBLK) * kThreads + threadIdx.x;
    const int bh = blockIdx.x / NBLK;
    if (e >= NS + D) return;
    const float* ri = rec + ((size_t(bh) * nseg + (nseg - 1)) * 2 + 1) * Rec<D, DV>::kFloats;
    if (e < NS) {
        if (!s_out) return;
        const int u = e / 256, lane = (e / 4) % 64, r = e % 4;
        const int a = u / (DV / 16), b = u % (DV / 16);
        const int d = 16 * a + 4 * (lane / 16) + r, dv = 16 * b + lane % 16;
        s_out[size_t(bh) * NS + size_t(d) * DV + dv] = ri[e];
    } else {
        if (!z_out) return;
        z_out[size_t(bh) * D + (e - NS)] = ri[e];
    }
}

template <typename E, int D, int DV, int CH, bool GATED>
__global__ __launch_bounds__(kThreads) void fused_kernel(FusedArgs args) {
    using Sh = WalkShape<E, D, DV, CH>;
    using W = ChunkWalker<E, D, DV, CH, GATED, true>;
    using R = Rec<D, DV>;
    extern __shared__ __align__(16) unsigned char smem[];
    int* s_int = reinterpret_cast<int*>(smem + Sh::bytes(true));

    const int tid = threadIdx.x;
    if (tid == 0) s_int[0] = atomicAdd(args.flags + size_t(gridDim.x), 1);
    __syncthreads();
    const int ticket = s_int[0];
    const int seg = ticket % args.nseg;
    const int bh = ticket / args.nseg;
    const int N = args.N;
    const int nchunks_total = (N + CH - 1) / CH;
    const int c0 = seg * args.L;
    const int nch = min(args.L, nchunks_total - c0);

    W wk;
    wk.init(smem, N, reinterpret_cast<const E*>(args.q) + size_t(bh) * N * D,
            reinterpret_cast<const E*>(args.k) + size_t(bh) * N * D,
            reinterpret_cast<const E*>(args.v) + size_t(bh) * N * DV, GATED ? args.g + size_t(bh) * N : nullptr);
    const int w = wk.w, lane = wk.lane, l16 = wk.l16, g4 = wk.g4;
    E* ob = reinterpret_cast<E*>(args.o) + size_t(bh) * N * DV;
    int* flag = args.flags + size_t(bh) * args.nseg;
    float* rec_head = args.rec + size_t(bh) * args.nseg * 2 * R::kFloats;

    // ---- pass 1: segment total ------------------------------------------------
    f32x4_t sacc[Sh::TPW];
    f32x4_t zacc[Sh::ZT];
#pragma unroll
    for (int j = 0; j < Sh::TPW; ++j) sacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < Sh::ZT; ++i) zacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float lg_total = 0.0f;
    wk.template walk<false, true>(c0, nch, sacc, zacc, lg_total, nullptr, args.eps);

    auto put4 = [&](float* dst, const f32x4_t& x) { *reinterpret_cast<f32x4_t*>(dst) = x; };
    auto write_record = [&](float* dst, const f32x4_t (&s)[Sh::TPW], const f32x4_t (&z)[Sh::ZT]) {
#pragma unroll
        for (int j = 0; j < Sh::TPW; ++j) put4(dst + ((w * Sh::TPW + j) * kWave + lane) * 4, s[j]);
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i)
            if (l16 == 0) put4(dst + R::kZ + 16 * (w * Sh::ZT + i) + 4 * g4, z[i]);
    };
    // Every wave waits until its record stores have reached its XCD's L2; after the
    // barrier, thread 0's release store of the flag writes that L2 back (one
    // write-back per publication) before the flag becomes visible.
    auto publish = [&](int value) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) __hip_atomic_store(flag + seg, value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto get4 = [&](const float* src) -> f32x4_t { return *reinterpret_cast<const f32x4_t*>(src); };

    float* rec_agg = rec_head + size_t(seg) * 2 * R::kFloats;
    float* rec_inc = rec_agg + R::kFloats;
    write_record(rec_agg, sacc, zacc);
    if (tid == 0) rec_agg[R::kLg] = lg_total;
    publish(1);

    // ---- look-back: state in front of the segment -----------------------------
    f32x4_t P[Sh::TPW];
    f32x4_t Pz[Sh::ZT];
#pragma unroll
    for (int j = 0; j < Sh::TPW; ++j) P[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < Sh::ZT; ++i) Pz[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float run = 0.0f;            // log2 decay from the records added so far to this segment
    bool ok = true;
    int j = seg - 1;
    while (j >= 0) {
        if (tid == 0) {
            int f;
            int spins = 0;
            while ((f = __hip_atomic_load(flag + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > kSpinLimit) {
                    f = -1;
                    break;
                }
            }
            s_int[1] = f;
            // acquire: stale cache lines of the record are dropped before any wave of
            // this workgroup (same CU, same L2) reads it after the barrier below
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        const int f = s_int[1];
        __syncthreads();
        if (f < 0) {
            ok = false;
            break;
        }
        const float* src = rec_head + (size_t(j) * 2 + (f == 2 ? 1 : 0)) * R::kFloats;
        const float sc = GATED ? fast_exp2(run) : 1.0f;
#pragma unroll
        for (int jj = 0; jj < Sh::TPW; ++jj)
            P[jj] += sc * get4(src + ((w * Sh::TPW + jj) * kWave + lane) * 4);
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i) {
            const f32x4_t zv = get4(src + R::kZ + 16 * (w * Sh::ZT + i) + 4 * g4);
            if (l16 == 0) Pz[i] += sc * zv;
        }
        if (f == 2) break;
        if constexpr (GATED) run += src[R::kLg];
        --j;
    }
    if (ok && j < 0) {
        const float sc = GATED ? fast_exp2(run) : 1.0f;
        if (args.s0) {
            const float* s0b = args.s0 + size_t(bh) * D * DV;
#pragma unroll
            for (int jj = 0; jj < Sh::TPW; ++jj) {
                const int u = w * Sh::TPW + jj;
                const int a = u / Sh::NB, b = u % Sh::NB;
#pragma unroll
                for (int r = 0; r < 4; ++r) P[jj][r] += sc * s0b[size_t(16 * a + 4 * g4 + r) * DV + 16 * b + l16];
            }
        }
        if (args.z0 && l16 == 0) {
            const float* z0b = args.z0 + size_t(bh) * D;
#pragma unroll
            for (int i = 0; i < Sh::ZT; ++i) Pz[i] += sc * *reinterpret_cast<const f32x4_t*>(z0b + 16 * (w * Sh::ZT + i) + 4 * g4);
        }
    }
    if (!ok) {
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int jj = 0; jj < Sh::TPW; ++jj) P[jj] = f32x4_t{nan, nan, nan, nan};
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i) Pz[i] = f32x4_t{nan, nan, nan, nan};
    }

    // ---- inclusive record: Gamma_s P + T ------------------------------------------
    {
        const float gs = GATED ? fast_exp2(lg_total) : 1.0f;
#pragma unroll
        for (int jj = 0; jj < Sh::TPW; ++jj) sacc[jj] += gs * P[jj];
#pragma unroll
        for (int i = 0; i < Sh::ZT; ++i) zacc[i] += gs * Pz[i];
        write_record(rec_inc, sacc, zacc);
        publish(2);
    }

    // ---- pass 2: outputs from P ---------------------------------------------------
#pragma unroll
    for (int jj = 0; jj < Sh::TPW; ++jj) sacc[jj] = P[jj];
#pragma unroll
    for (int i = 0; i < Sh::ZT; ++i) zacc[i] = Pz[i];
    wk.stage_state(sacc, zacc);
    float lg_unused = 0.0f;
    wk.template walk<true, false>(c0, nch, sacc, zacc, lg_unused, ob, args.eps);
}

}  // namespace linattn
