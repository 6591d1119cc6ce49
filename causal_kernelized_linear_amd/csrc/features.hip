// Feature maps other than elu + 1:
//   relu   phi(x) = max(x, 0) + shift   (the F.relu(x) + eps alternative of the
//          anandmoghan-problems page, "Key Functions & Tricks"), applied by the chunked
//          walk itself while it stages q and k (its RELU form);
//   favor  phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m), the positive random features of
//          Performer's FAVOR+ (aicassindra.com page, "Performer: unbiased softmax by
//          positive random features"), for the m rows w_r of a per-head W [H][m][D]:
//          for bf16 inputs, no gate and m = D = 64 formed by the walk itself while it stages
//          k and q (its FAVOR form); otherwise written by a pass of their own, which the
//          walk then takes as they are (its IDENT form).
// The FAVOR+ projection w_r . x keeps fp32 accuracy on the bf16 MFMA: every fp32 operand
// is split into a bf16 high part and a bf16 low part (the high part's rounding error),
// and w . x = x_hi . w_hi + x_hi . w_lo + x_lo . w_hi, dropping x_lo . w_lo (about 2^-16
// of the product); a bf16 input has no low part.  Each partial product of two bf16
// values is exact in the fp32 accumulator.  Rounding W or x to bf16 alone would put an
// error of about 2^-9 |w| |x| into the exponent.
#include "bwd.hpp"          // MFMA fragment helpers and lane sums
#include "chunk_walk.hpp"
#include "fwd_dispatch.hpp"

namespace linattn {

// LDS of the feature pass: x (high and, for fp32 inputs, low parts) [64][D] and W's high
// and low parts [M][D], bf16 rows padded by 16 bytes, and |x|^2 / 2 per row.
template <typename E, int D, int M>
struct FeatShape {
    static constexpr int C = 64, LX = D + 8;
    static constexpr bool kSplitX = sizeof(E) == 4;
    static constexpr size_t kOffXh = 0;
    static constexpr size_t kOffXl = kOffXh + size_t(C) * LX * 2;
    static constexpr size_t kOffWh = kOffXl + (kSplitX ? size_t(C) * LX * 2 : 0);
    static constexpr size_t kOffWl = kOffWh + size_t(M) * LX * 2;
    static constexpr size_t kOffN = kOffWl + size_t(M) * LX * 2;
    static constexpr size_t kBytes = kOffN + size_t(C) * 4;
};

// Sum over G consecutive lanes (G in {8, 16, 32}, aligned), every lane getting it.
template <int G>
__device__ __forceinline__ float sum_lanes(float x) {
    static_assert(G == 8 || G == 16 || G == 32, "lane group");
    if constexpr (G == 8) {
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
        return x;
    } else {
        x = sum16(x);
        if constexpr (G == 32) x += __shfl_xor(x, 16, kWave);
        return x;
    }
}

// A value split into bf16 high and low parts.
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
    using B = Elem<uint16_t>;
    hi = B::from_f32(v);
    lo = B::from_f32(v - B::to_f32(hi));
}

// One workgroup per (tensor, head, kFeatBlocks blocks of 64 rows), q and k in one launch
// (blocks 2i and 2i + 1 take the same rows of q and of k): the rows' FAVOR+ features into
// fq or fk [BH][N][M].  W's split is staged once per workgroup and serves all its
// blocks; each block's rows are loaded while the block before it is projected.
constexpr int kFeatBlocks = 4;

template <typename E, int D, int M>
__global__ __launch_bounds__(kThreads) void feature_kernel(const E* __restrict__ xq, const E* __restrict__ xk,
                                                           const float* __restrict__ W, E* __restrict__ fq,
                                                           E* __restrict__ fk, int N, int H) {
    using Sh = FeatShape<E, D, M>;
    using X = Elem<E>;
    constexpr int C = Sh::C, LX = Sh::LX, NR = M / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* sXh = reinterpret_cast<uint16_t*>(smem + Sh::kOffXh);
    uint16_t* sXl = reinterpret_cast<uint16_t*>(smem + Sh::kOffXl);
    uint16_t* sWh = reinterpret_cast<uint16_t*>(smem + Sh::kOffWh);
    uint16_t* sWl = reinterpret_cast<uint16_t*>(smem + Sh::kOffWl);
    float* sN = reinterpret_cast<float*>(smem + Sh::kOffN);
    const int nsup = (N + C * kFeatBlocks - 1) / (C * kFeatBlocks);
    const int which = blockIdx.x & 1, item = blockIdx.x >> 1;
    const int sup = item % nsup, bh = item / nsup;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int l16 = lane & 15, g4 = lane >> 4;
    const E* xb = (which ? xk : xq) + size_t(bh) * N * D;
    E* fb = (which ? fk : fq) + size_t(bh) * N * M;
    const float* Wh = W + size_t(bh % H) * M * D;

    constexpr int EPG = 16 / int(sizeof(E)), G = D / EPG, UX = C * G / kThreads, UW = M * D / 4 / kThreads;
    // a block's x in 16-byte units (rows clamped); the first block's go out before W's
    f32x4_t rx[UX];
    auto load_block = [&](int ts_, int nrows_) {
#pragma unroll
        for (int u = 0; u < UX; ++u) {
            const int idx = tid + u * kThreads, row = idx / G, col = (idx % G) * EPG;
            rx[u] = *reinterpret_cast<const f32x4_t*>(xb + size_t(ts_ + min(row, nrows_ - 1)) * D + col);
        }
    };
    {
        const int ts0 = sup * kFeatBlocks * C;
        if (ts0 < N) load_block(ts0, min(C, N - ts0));
    }
    // W's high and low parts, once
    {
        f32x4_t rw[UW];
#pragma unroll
        for (int u = 0; u < UW; ++u) rw[u] = *reinterpret_cast<const f32x4_t*>(Wh + 4 * (tid + u * kThreads));
#pragma unroll
        for (int u = 0; u < UW; ++u) {
            const int i = 4 * (tid + u * kThreads), m = i / D, d = i % D;
            F4<uint16_t> oh, ol;
#pragma unroll
            for (int e = 0; e < 4; ++e) split_bf16(rw[u][e], oh.x[e], ol.x[e]);
            *reinterpret_cast<F4<uint16_t>*>(sWh + m * LX + d) = oh;
            *reinterpret_cast<F4<uint16_t>*>(sWl + m * LX + d) = ol;
        }
    }
    for (int blk = 0; blk < kFeatBlocks; ++blk) {
    const int ts = (sup * kFeatBlocks + blk) * C;
    if (ts >= N) break;                                       // uniform over the workgroup
    const int nrows = min(C, N - ts);

    // x into LDS (split when fp32), and each row's |x|^2 / 2 summed over the G lanes that
    // hold it (rows past the end are zero)
#pragma unroll
    for (int u = 0; u < UX; ++u) {
        const int idx = tid + u * kThreads, row = idx / G, col = (idx % G) * EPG;
        const bool in = row < nrows;
        float sq = 0.0f;
        if constexpr (sizeof(E) == 2) {
            const F8<uint16_t> v = __builtin_bit_cast(F8<uint16_t>, rx[u]);
            F8<uint16_t> o;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = in ? X::to_f32(v.x[e]) : 0.0f;
                o.x[e] = in ? v.x[e] : uint16_t(0);
                sq += xv * xv;
            }
            *reinterpret_cast<F8<uint16_t>*>(sXh + row * LX + col) = o;
        } else {
            F4<uint16_t> oh, ol;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xv = in ? rx[u][e] : 0.0f;
                split_bf16(xv, oh.x[e], ol.x[e]);
                sq += xv * xv;
            }
            *reinterpret_cast<F4<uint16_t>*>(sXh + row * LX + col) = oh;
            *reinterpret_cast<F4<uint16_t>*>(sXl + row * LX + col) = ol;
        }
        sq = sum_lanes<G>(sq);
        if (idx % G == 0) sN[row] = 0.5f * sq;
    }
    // the next block's rows, in flight during this block's products and stores
    if (blk + 1 < kFeatBlocks && ts + C < N) load_block(ts + C, min(C, N - ts - C));
    __syncthreads();

    // (W x)^T: lane (l16, g4) holds row i = 16 w + l16 against features 16 t + 4 g4 + r
    f32x4_t acc[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        const int k0 = 32 * ks + 8 * g4;
        const F8<uint16_t> bh_ = frag_row(sXh, LX, 16 * w + l16, k0);
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            const F8<uint16_t> ah = frag_row(sWh, LX, 16 * t + l16, k0);
            acc[t] = mma(ah, bh_, acc[t]);
            acc[t] = mma(frag_row(sWl, LX, 16 * t + l16, k0), bh_, acc[t]);
            if constexpr (Sh::kSplitX) acc[t] = mma(ah, frag_row(sXl, LX, 16 * w + l16, k0), acc[t]);
        }
    }
    // features exp(w . x - |x|^2 / 2) / sqrt(M): four consecutive per lane
    const int i = 16 * w + l16;
    if (i < nrows) {
        const float h = sN[i], rs = 1.0f / sqrtf(float(M));
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            f32x4_t o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = fast_exp2((acc[t][r] - h) * kLog2e) * rs;
            *reinterpret_cast<F4<E>*>(fb + size_t(ts + i) * M + 16 * t + 4 * g4) = pack4<E>(o);
        }
    }
    __syncthreads();                  // the block's x and |x|^2 are read: the next may overwrite
    }
}

template <typename E, int D, int M>
static hipError_t run_features(const FeatLaunch& p, void* fq, void* fk) {
    const int nsup = (p.N + 64 * kFeatBlocks - 1) / (64 * kFeatBlocks);
    const dim3 grid(2u * unsigned(p.BH) * unsigned(nsup)), block(kThreads);
    constexpr size_t lds = FeatShape<E, D, M>::kBytes;
    static bool attr = false;
    if (!attr) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(feature_kernel<E, D, M>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL((feature_kernel<E, D, M>), grid, block, lds, p.stream, static_cast<const E*>(p.fwd.q),
                       static_cast<const E*>(p.fwd.k), p.W, static_cast<E*>(fq), static_cast<E*>(fk), p.N, p.H);
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

// The walk forming FAVOR+ features itself (bf16, ungated, M = D): no feature pass.
template <int D, int DV>
static hipError_t run_favor_walks(const FwdLaunch& p) {
    switch (p.chunk) {
        case 64: return run_fwd<uint16_t, D, DV, 64, false, false, false, 1, true>(p);
        case 128: return run_fwd<uint16_t, D, DV, 128, false, false, false, 1, true>(p);
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
    if constexpr (sizeof(E) == 2) {
        // bf16, ungated, M = D = 64: the walks project and exponentiate while staging
        // (at D = 128 W's tiles leave too little LDS and too few registers)
        if (p.fwd.g == nullptr && p.M == p.D && p.D == 64 && (p.fwd.chunk == 64 || p.fwd.chunk == 128)) {
            FwdLaunch w = p.fwd;
            w.W = p.W;
            w.H = p.H;
            w.ws = ws + 2 * fbytes;
            if (w.Dv == 64) return run_favor_walks<64, 64>(w);
            if (w.Dv == 128) return run_favor_walks<64, 128>(w);
        }
    }
    void* fq = ws;
    void* fk = ws + fbytes;
    hipError_t e = hipSuccess;
#define LINATTN_FEAT(DD, MM)                                                             \
    if (p.D == DD && p.M == MM) {                                                        \
        e = run_features<E, DD, MM>(p, fq, fk);                                          \
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
