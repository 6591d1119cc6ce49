// Template dispatch of the chunked forward over (D, Dv, chunk, gated) for one
// element type; included once per element type so the instantiations compile in
// parallel translation units.
#pragma once

#include "chunk_fused.hpp"
#include "chunk_walk.hpp"
#include "launch.hpp"

namespace linattn {

template <typename E, int D, int DV, int CH, bool GATED>
hipError_t run_fwd_three_pass(const FwdLaunch& p) {
    using Sh = WalkShape<E, D, DV, CH>;
    size_t off_zt = 0, off_lg = 0;
    three_pass_bytes(size_t(p.BH) * p.nseg, D, DV, &off_zt, &off_lg);
    char* wsb = static_cast<char*>(p.ws);
    WalkArgs a;
    a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.o = p.o;
    a.st = reinterpret_cast<float*>(wsb);
    a.zt = reinterpret_cast<float*>(wsb + off_zt);
    a.lg = reinterpret_cast<float*>(wsb + off_lg);
    a.N = p.N; a.nseg = p.nseg; a.L = p.L; a.eps = p.eps;
    auto* k_tot = walk_kernel<E, D, DV, CH, GATED, false>;
    auto* k_out = walk_kernel<E, D, DV, CH, GATED, true>;
    static bool attrs_set = false;         // benign race: idempotent attribute set
    if (!attrs_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_tot),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(Sh::bytes(false)));
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_out), hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(Sh::bytes(true)));
        if (e != hipSuccess) return e;
        attrs_set = true;
    }
    const unsigned nwg = unsigned(p.BH) * unsigned(p.nseg);
    auto mark = [&](int i) { if (p.prof[i]) (void)hipEventRecord(p.prof[i], p.stream); };
    mark(0);
    hipLaunchKernelGGL(k_tot, dim3(nwg), dim3(kThreads), Sh::bytes(false), p.stream, a);
    mark(1);
    constexpr int NBLK = (D * DV + D + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((scan_kernel<D, DV, GATED>), dim3(unsigned(p.BH) * NBLK), dim3(kThreads), 0, p.stream,
                       a.st, a.zt, a.lg, p.s0, p.z0, p.s_out, p.z_out, p.nseg);
    mark(2);
    hipLaunchKernelGGL(k_out, dim3(nwg), dim3(kThreads), Sh::bytes(true), p.stream, a);
    mark(3);
    return hipGetLastError();
}

template <typename E, int D, int DV, int CH, bool GATED>
hipError_t run_fwd_fused(const FwdLaunch& p) {
    using Sh = WalkShape<E, D, DV, CH>;
    const size_t heads = size_t(p.BH) * p.nseg;
    size_t off_flags = 0;
    fused_bytes(heads, D, DV, &off_flags);
    char* wsb = static_cast<char*>(p.ws);
    FusedArgs a;
    a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.o = p.o;
    a.s0 = p.s0; a.z0 = p.z0;
    a.rec = reinterpret_cast<float*>(wsb);
    a.flags = reinterpret_cast<int*>(wsb + off_flags);
    a.N = p.N; a.nseg = p.nseg; a.L = p.L; a.eps = p.eps;
    auto* k_fused = fused_kernel<E, D, DV, CH, GATED>;
    const size_t lds = Sh::bytes(true) + 16;
    static bool attrs_set = false;         // benign race: idempotent attribute set
    if (!attrs_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_fused),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
        attrs_set = true;
    }
    auto mark = [&](int i) { if (p.prof[i]) (void)hipEventRecord(p.prof[i], p.stream); };
    mark(0);
    const int nflags = int(heads) + 1;
    hipLaunchKernelGGL(fused_clear_kernel, dim3((nflags + kThreads - 1) / kThreads), dim3(kThreads), 0, p.stream,
                       a.flags, nflags);
    mark(1);
    hipLaunchKernelGGL(k_fused, dim3(unsigned(heads)), dim3(kThreads), lds, p.stream, a);
    mark(2);
    if (p.s_out || p.z_out) {
        constexpr int NBLK = (D * DV + D + kThreads - 1) / kThreads;
        hipLaunchKernelGGL((fused_final_kernel<D, DV>), dim3(unsigned(p.BH) * NBLK), dim3(kThreads), 0, p.stream,
                           a.rec, p.nseg, p.s_out, p.z_out);
    }
    mark(3);
    return hipGetLastError();
}

template <typename E, int D, int DV, int CH, bool GATED>
hipError_t run_fwd(const FwdLaunch& p) {
    using Sh = WalkShape<E, D, DV, CH>;
    if constexpr (Sh::bytes(true) + 16 > kMaxLds) {
        return hipErrorInvalidValue;           // rejected earlier by the ABI's support check
    } else {
        return p.algo == 2 ? run_fwd_fused<E, D, DV, CH, GATED>(p) : run_fwd_three_pass<E, D, DV, CH, GATED>(p);
    }
}

template <typename E, int D, int DV>
hipError_t run_fwd_chunk(const FwdLaunch& p) {
    const bool gated = p.g != nullptr;
    switch (p.chunk) {
        case 32:  return gated ? run_fwd<E, D, DV, 32, true>(p) : run_fwd<E, D, DV, 32, false>(p);
        case 64:  return gated ? run_fwd<E, D, DV, 64, true>(p) : run_fwd<E, D, DV, 64, false>(p);
        case 128: return gated ? run_fwd<E, D, DV, 128, true>(p) : run_fwd<E, D, DV, 128, false>(p);
        case 256: return gated ? run_fwd<E, D, DV, 256, true>(p) : run_fwd<E, D, DV, 256, false>(p);
        default:  return hipErrorInvalidValue;
    }
}

template <typename E>
hipError_t run_fwd_typed(const FwdLaunch& p) {
    if (p.D == 64 && p.Dv == 64) return run_fwd_chunk<E, 64, 64>(p);
    if (p.D == 64 && p.Dv == 128) return run_fwd_chunk<E, 64, 128>(p);
    if (p.D == 128 && p.Dv == 64) return run_fwd_chunk<E, 128, 64>(p);
    if (p.D == 128 && p.Dv == 128) return run_fwd_chunk<E, 128, 128>(p);
    return hipErrorInvalidValue;
}

}  // namespace linattn
