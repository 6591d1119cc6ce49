// Feature maps other than elu + 1:
//   relu   phi(x) = max(x, 0) + shift   (the F.relu(x) + eps alternative of the
//          anandmoghan-problems page, "Key Functions & Tricks"), applied by the chunked
//          walk itself while it stages q and k (its RELU form);
//   favor  phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m), the positive random features of
//          Performer's FAVOR+ (aicassindra.com page, "Performer: unbiased softmax by
//          positive random features"), for the m rows w_r of a per-head W [H][m][D],
//          written by a pass of their own; the walk then takes them as they are (its
//          IDENT form).
// The FAVOR+ projection is an fp32 MFMA product: rounding W or x to bf16 would put an
// error of about 2^-9 |w| |x| into the exponent.
#include "chunk_walk.hpp"
#include "fwd_dispatch.hpp"

namespace linattn {

// One workgroup per (head, 64 rows): the rows' FAVOR+ features into f [BH][N][M].
template <typename E, int D, int M>
__global__ __launch_bounds__(kThreads) void feature_kernel(const E* __restrict__ x, const float* __restrict__ W,
                                                           E* __restrict__ f, int N, int H) {
    using X = Elem<E>;
    constexpr int C = 64, LX = D + 4;
    const int nch = (N + C - 1) / C;
    const int c = blockIdx.x % nch, bh = blockIdx.x / nch, ts = c * C, nrows = min(C, N - ts);
    const int tid = threadIdx.x;
    const E* xb = x + size_t(bh) * N * D;
    E* fb = f + size_t(bh) * N * M;
    {
        extern __shared__ __align__(16) unsigned char smem[];
        float* sX = reinterpret_cast<float*>(smem);            // [C][LX]
        float* sW = sX + C * LX;                                 // [M][LX]
        float* sN = sW + M * LX;                                 // [C] |x|^2 / 2
        const float* Wh = W + size_t(bh % H) * M * D;
        // every load first: x in 16-byte units (rows clamped), W in fp32 quads
        constexpr int EPG = 16 / int(sizeof(E)), G = D / EPG, UX = C * G / kThreads, UW = M * D / 4 / kThreads;
        f32x4_t rx[UX], rw[UW];
#pragma unroll
        for (int u = 0; u < UX; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = (idx % G) * EPG;
            rx[u] = *reinterpret_cast<const f32x4_t*>(xb + size_t(ts + min(row, nrows - 1)) * D + col);
        }
#pragma unroll
        for (int u = 0; u < UW; ++u) rw[u] = *reinterpret_cast<const f32x4_t*>(Wh + 4 * (tid + u * kThreads));
#pragma unroll
        for (int u = 0; u < UX; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = (idx % G) * EPG;
            if constexpr (sizeof(E) == 2) {
                const F8<E> in = __builtin_bit_cast(F8<E>, rx[u]);
#pragma unroll
                for (int e = 0; e < 8; ++e) sX[row * LX + col + e] = row < nrows ? X::to_f32(in.x[e]) : 0.0f;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) sX[row * LX + col + e] = row < nrows ? rx[u][e] : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < UW; ++u) {
            const int i = 4 * (tid + u * kThreads);
            *reinterpret_cast<f32x4_t*>(sW + (i / D) * LX + i % D) = rw[u];
        }
        __syncthreads();
        if (tid < C) {
            float s = 0.0f;
            for (int d = 0; d < D; ++d) s += sX[tid * LX + d] * sX[tid * LX + d];
            sN[tid] = 0.5f * s;
        }
        __syncthreads();
        const int w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
        const int l16 = lane & 15, g4 = lane >> 4;
        constexpr int NR = M / 16;
        f32x4_t acc[NR];
#pragma unroll
        for (int t = 0; t < NR; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const F8<float> a = lds_f8(sX + (16 * w + l16) * LX + 32 * ks + 8 * g4);
#pragma unroll
            for (int t = 0; t < NR; ++t) acc[t] = mma(a, lds_f8(sW + (16 * t + l16) * LX + 32 * ks + 8 * g4), acc[t]);
        }
        const float rs = 1.0f / sqrtf(float(M));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * g4 + r;
            if (i < nrows) {
                const float h = sN[i];
#pragma unroll
                for (int t = 0; t < NR; ++t)
                    fb[size_t(ts + i) * M + 16 * t + l16] = X::from_f32(fast_exp2((acc[t][r] - h) * kLog2e) * rs);
            }
        }
    }
}

template <int D, int M>
constexpr size_t feature_lds_bytes() {
    return (size_t(64) * (D + 4) + size_t(M) * (D + 4) + 64) * 4;
}

template <typename E, int D, int M>
static hipError_t run_features(const FeatLaunch& p, const void* x, void* f) {
    const int nch = (p.N + 63) / 64;
    const dim3 grid(unsigned(p.BH) * unsigned(nch)), block(kThreads);
    constexpr size_t lds = feature_lds_bytes<D, M>();
    static bool attr = false;
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(feature_kernel<E, D, M>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL((feature_kernel<E, D, M>), grid, block, lds, p.stream, static_cast<const E*>(x), p.W,
                       static_cast<E*>(f), p.N, p.H);
    return hipGetLastError();
}

// The walk over the features: state rows M, chunk 64 or 128.
template <typename E, int M, int DV>
static hipError_t run_feature_walks(const FwdLaunch& p) {
    const bool gated = p.g != nullptr;
    switch (p.chunk) {
        case 64: return gated ? run_fwd<E, M, DV, 64, true, true>(p) : run_fwd<E, M, DV, 64, false, true>(p);
        case 128: return gated ? run_fwd<E, M, DV, 128, true, true>(p) : run_fwd<E, M, DV, 128, false, true>(p);
        default: return hipErrorInvalidValue;
    }
}

// The walk under relu + shift features, over q and k as given.
template <typename E, int D, int DV>
static hipError_t run_relu_walks(const FwdLaunch& p) {
    const bool gated = p.g != nullptr;
    switch (p.chunk) {
        case 64: return gated ? run_fwd<E, D, DV, 64, true, false, true>(p) : run_fwd<E, D, DV, 64, false, false, true>(p);
        case 128: return gated ? run_fwd<E, D, DV, 128, true, false, true>(p) : run_fwd<E, D, DV, 128, false, false, true>(p);
        default: return hipErrorInvalidValue;
    }
}

template <typename E>
static hipError_t run_feature_fwd(const FeatLaunch& p) {
    if (p.kind == 1) {
        FwdLaunch w = p.fwd;
        w.fshift = p.shift;
        if (p.M != p.D) return hipErrorInvalidValue;
        if (p.D == 64 && w.Dv == 64) return run_relu_walks<E, 64, 64>(w);
        if (p.D == 64 && w.Dv == 128) return run_relu_walks<E, 64, 128>(w);
        if (p.D == 128 && w.Dv == 64) return run_relu_walks<E, 128, 64>(w);
        if (p.D == 128 && w.Dv == 128) return run_relu_walks<E, 128, 128>(w);
        return hipErrorInvalidValue;
    }
    char* ws = static_cast<char*>(p.fwd.ws);
    const size_t fbytes = round_up256(size_t(p.BH) * p.N * p.M * sizeof(E));
    void* fq = ws;
    void* fk = ws + fbytes;
    hipError_t e = hipSuccess;
#define LINATTN_FEAT(DD, MM)                                                             \
    if (p.D == DD && p.M == MM) {                                                        \
        e = run_features<E, DD, MM>(p, p.fwd.q, fq);                                     \
        if (e == hipSuccess) e = run_features<E, DD, MM>(p, p.fwd.k, fk);                \
    } else
    LINATTN_FEAT(64, 64) LINATTN_FEAT(64, 128) LINATTN_FEAT(128, 64) LINATTN_FEAT(128, 128) { return hipErrorInvalidValue; }
#undef LINATTN_FEAT
    if (e != hipSuccess) return e;
    FwdLaunch w = p.fwd;
    w.q = fq;
    w.k = fk;
    w.D = p.M;
    w.ws = ws + 2 * fbytes;
    if (p.M == 64 && w.Dv == 64) return run_feature_walks<E, 64, 64>(w);
    if (p.M == 64 && w.Dv == 128) return run_feature_walks<E, 64, 128>(w);
    if (p.M == 128 && w.Dv == 64) return run_feature_walks<E, 128, 64>(w);
    if (p.M == 128 && w.Dv == 128) return run_feature_walks<E, 128, 128>(w);
    return hipErrorInvalidValue;
}

hipError_t launch_feature_fwd(const FeatLaunch& p) {
    return p.es == 2 ? run_feature_fwd<uint16_t>(p) : run_feature_fwd<float>(p);
}

}  // namespace linattn
