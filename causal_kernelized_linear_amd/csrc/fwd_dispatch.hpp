// Template dispatch of the chunked forward over (D, Dv, chunk, gated) for one
// element type; included once per element type so the instantiations compile in
// parallel translation units.
#pragma once

#include "chunk_walk.hpp"
#include "launch.hpp"

namespace linattn {

// DV is the width of one column part; VS parts make up the caller's Dv = DV * VS.
template <typename E, int D, int DV, int CH, bool GATED, bool IDENT = false, bool RELU = false, int VS = 1,
          bool FAVOR = false>
hipError_t run_fwd_walks(const FwdLaunch& p) {
    using ShT = WalkShape<E, D, DV, CH, GATED, false>;
    using ShO = WalkShape<E, D, DV, CH, GATED, true>;
    const int tparts = p.tparts;
    const int nslots = (p.nseg - 1) * tparts + 1;
    size_t off_zt = 0, off_lg = 0;
    fwd_workspace_layout(size_t(p.BH) * VS * nslots, D, DV, &off_zt, &off_lg);
    char* wsb = static_cast<char*>(p.ws);
    WalkArgs a;
    a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.o = p.o;
    a.st = reinterpret_cast<float*>(wsb);
    a.zt = reinterpret_cast<float*>(wsb + off_zt);
    a.lg = reinterpret_cast<float*>(wsb + off_lg);
    a.s0 = p.s0; a.z0 = p.z0;
    a.N = p.N; a.BH = p.BH; a.nseg = p.nseg; a.L = p.L; a.tparts = tparts; a.nslots = nslots;
    a.eps = p.eps; a.normalize = p.normalize;
    a.fshift = p.fshift;
    a.W = p.W;
    a.H = p.H;
    a.direct = prefix_direct(p.nseg, D, DV) ? 1 : 0;
    a.want_final = (p.s_out || p.z_out) ? 1 : 0;
    a.stream_kv = totals_stream_kv(p.BH, p.N, D, DV * VS, int(sizeof(E))) ? 1 : 0;
    auto* k_tot = walk_kernel<E, D, DV, CH, GATED, false, IDENT, RELU, VS, false, FAVOR>;
    // the output walk: the split 8-wave walk where its shape has one, else the 4-wave one
    constexpr bool kSplit = walk_split(int(sizeof(E)), D, DV, CH, GATED) && VS == 1 && !IDENT && !FAVOR;
    auto* k_out = [] {
        if constexpr (kSplit)
            return walk_split_kernel<E, D, DV, CH, RELU>;
        else
            return walk_kernel<E, D, DV, CH, GATED, true, IDENT, RELU, VS, false, FAVOR>;
    }();
    constexpr size_t kFavorBytes = FAVOR ? favor_lds_bytes(D) : 0;
    constexpr size_t kTotBytes = ShT::kBytes + kFavorBytes;
    constexpr size_t kOutBytes = kSplit ? split_walk_lds_bytes(int(sizeof(E)), D, DV, CH) : ShO::kBytes + kFavorBytes;
    constexpr unsigned kOutThreads = kSplit ? kSplitThreads : kThreads;
    static bool attrs_set = false;         // benign race: idempotent attribute set
    if (!attrs_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_tot),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(kTotBytes));
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_out), hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(kOutBytes));
        if (e != hipSuccess) return e;
        attrs_set = true;
    }
    constexpr int NBLK = (D * DV + D + kThreads - 1) / kThreads;
    const unsigned vheads = unsigned(p.BH) * VS;
    auto mark = [&](int i) { if (p.prof[i]) (void)hipEventRecord(p.prof[i], p.stream); };
    mark(0);
    if (p.nseg > 1)
        hipLaunchKernelGGL(k_tot, dim3(walk_grid(unsigned(p.BH) * unsigned((p.nseg - 1) * tparts), VS)),
                           dim3(kThreads), kTotBytes, p.stream, a);
    mark(1);
    if (p.nseg > 1 && !a.direct)
        hipLaunchKernelGGL((scan_kernel<D, DV, GATED, VS>), dim3(vheads * NBLK), dim3(kThreads), 0, p.stream, a.st,
                           a.zt, a.lg, p.s0, p.z0, nslots, nslots - 1, tparts);
    mark(2);
    hipLaunchKernelGGL(k_out, dim3(walk_grid(unsigned(p.BH) * unsigned(p.nseg), VS, !kSplit)), dim3(kOutThreads), kOutBytes,
                       p.stream, a);
    if (a.want_final)
        hipLaunchKernelGGL((final_kernel<D, DV, VS>), dim3(vheads * NBLK), dim3(kThreads), 0, p.stream, a.st, a.zt,
                           nslots, nslots - 1, p.s_out, p.z_out);
    mark(3);
    return hipGetLastError();
}

template <typename E, int D, int DV, int CH, bool GATED, bool IDENT = false, bool RELU = false, int VS = 1,
          bool FAVOR = false>
hipError_t run_fwd(const FwdLaunch& p) {
    if constexpr (WalkShape<E, D, DV, CH, GATED, true>::kBytes + (FAVOR ? favor_lds_bytes(D) : 0) > kMaxLds) {
        return hipErrorInvalidValue;           // rejected earlier by the ABI's support check
    } else {
        return run_fwd_walks<E, D, DV, CH, GATED, IDENT, RELU, VS, FAVOR>(p);
    }
}

template <typename E, int D, int DV, int VS = 1>
hipError_t run_fwd_chunk(const FwdLaunch& p) {
    const bool gated = p.g != nullptr;
    switch (p.chunk) {
        case 32:  return gated ? run_fwd<E, D, DV, 32, true, false, false, VS>(p)
                               : run_fwd<E, D, DV, 32, false, false, false, VS>(p);
        case 64:  return gated ? run_fwd<E, D, DV, 64, true, false, false, VS>(p)
                               : run_fwd<E, D, DV, 64, false, false, false, VS>(p);
        case 128: return gated ? run_fwd<E, D, DV, 128, true, false, false, VS>(p)
                               : run_fwd<E, D, DV, 128, false, false, false, VS>(p);
        case 256: return gated ? run_fwd<E, D, DV, 256, true, false, false, VS>(p)
                               : run_fwd<E, D, DV, 256, false, false, false, VS>(p);
        default:  return hipErrorInvalidValue;
    }
}

// p.vsplit column parts (walk_vsplit): 2 walks Dv = 128 as two parts of 64 columns.
template <typename E>
hipError_t run_fwd_typed(const FwdLaunch& p) {
    if (p.vsplit == 2) {
        if (p.D == 64 && p.Dv == 128) return run_fwd_chunk<E, 64, 64, 2>(p);
        if (p.D == 128 && p.Dv == 128) return run_fwd_chunk<E, 128, 64, 2>(p);
        return hipErrorInvalidValue;
    }
    if (p.vsplit != 1) return hipErrorInvalidValue;
    if (p.D == 64 && p.Dv == 64) return run_fwd_chunk<E, 64, 64>(p);
    if (p.D == 64 && p.Dv == 128) return run_fwd_chunk<E, 64, 128>(p);
    if (p.D == 128 && p.Dv == 64) return run_fwd_chunk<E, 128, 64>(p);
    if (p.D == 128 && p.Dv == 128) return run_fwd_chunk<E, 128, 128>(p);
    return hipErrorInvalidValue;
}

}  // namespace linattn
