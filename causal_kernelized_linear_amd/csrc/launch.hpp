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
    void* ws;                // caller's workspace, carved by the dispatch (see fwd_workspace_bytes)
    int BH, N, D, Dv, chunk, nseg, L;
    float eps;
    hipStream_t stream;
    hipEvent_t prof[4];      // measurement hook: all NULL when unused
    int algo;                // 1: three launches, 2: single pass with look-back
};

// Chunk sizes with kernel instantiations.
inline bool chunk_is_built(int chunk) { return chunk == 32 || chunk == 64 || chunk == 128 || chunk == 256; }

// Dynamic LDS bytes of the output walk for (element size, D, Dv, chunk); the
// same formula as WalkShape::bytes(true).
inline size_t walk_lds_bytes(int esize, int D, int Dv, int chunk) {
    const int pe = 16 / esize;
    return size_t(chunk) * (D + pe) * esize + size_t(D) * (chunk + pe) * esize + size_t(Dv) * (chunk + pe) * esize +
           size_t(Dv) * (D + pe) * esize + size_t(D) * 4 + size_t(chunk) * 4;
}

constexpr size_t kMaxLds = 160 * 1024;   // LDS per compute unit on gfx950

inline size_t round_up256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the three-launch path: totals/prefixes [BH][nseg][D*Dv], z [BH][nseg][D],
// log2 decays [BH][nseg].
inline size_t three_pass_bytes(size_t heads, int D, int Dv, size_t* off_zt, size_t* off_lg) {
    const size_t st = round_up256(heads * size_t(D) * Dv * 4);
    const size_t zt = round_up256(heads * size_t(D) * 4);
    if (off_zt) *off_zt = st;
    if (off_lg) *off_lg = st + zt;
    return st + zt + round_up256(heads * 4);
}

// Workspace of the single-pass path: two records per segment, then the flags and
// the ticket counter.
inline size_t fused_record_floats(int D, int Dv) { return size_t((D * Dv + D + 1 + 63) / 64) * 64; }
inline size_t fused_bytes(size_t heads, int D, int Dv, size_t* off_flags) {
    const size_t rec = round_up256(heads * 2 * fused_record_floats(D, Dv) * 4);
    if (off_flags) *off_flags = rec;
    return rec + round_up256((heads + 1) * 4);
}

inline size_t fwd_workspace_bytes(size_t heads, int D, int Dv) {
    const size_t a = three_pass_bytes(heads, D, Dv, nullptr, nullptr);
    const size_t b = fused_bytes(heads, D, Dv, nullptr);
    return a > b ? a : b;
}

hipError_t launch_fwd_bf16(const FwdLaunch& p);
hipError_t launch_fwd_f32(const FwdLaunch& p);
hipError_t launch_decode(int dtype, const void* q, const void* k, const void* v, float* S, float* z, void* o,
                         int BH, int D, int Dv, float eps, hipStream_t stream);

}  // namespace linattn
