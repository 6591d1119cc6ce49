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
    float* ws_st;            // [BH][nseg][D*Dv]
    float* ws_zt;            // [BH][nseg][D]
    float* ws_lg;            // [BH][nseg]
    int BH, N, D, Dv, chunk, nseg, L;
    float eps;
    hipStream_t stream;
    hipEvent_t prof[4];      // measurement hook: all NULL when unused
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

hipError_t launch_fwd_bf16(const FwdLaunch& p);
hipError_t launch_fwd_f32(const FwdLaunch& p);
hipError_t launch_decode(int dtype, const void* q, const void* k, const void* v, float* S, float* z, void* o,
                         int BH, int D, int Dv, float eps, hipStream_t stream);

}  // namespace linattn
