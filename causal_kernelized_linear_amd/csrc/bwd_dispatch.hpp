// Template dispatch of the backward over (D, Dv, gated) for one element type; included
// once per element type so the instantiations compile in parallel translation units.
#pragma once

#include "bwd.hpp"
#include "chunk_walk.hpp"
#include "launch.hpp"

namespace linattn {

template <typename Kern>
static hipError_t set_lds(Kern* k, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               int(bytes));
}

template <typename E, int D, int DV, bool GATED>
hipError_t run_bwd(const BwdLaunch& p) {
    using Sh = BwdShape<E, D, DV>;
    using ShT = WalkShape<E, D, DV, kBwdChunk, GATED, false>;
    if constexpr (Sh::kBytes > kMaxLds) {
        return hipErrorInvalidValue;           // rejected earlier by the ABI's support check
    } else {
        constexpr int C = kBwdChunk;
        const int NC = (p.N + C - 1) / C;
        const BwdLayout lay = bwd_workspace_layout(size_t(p.BH), p.N, D, DV);
        char* ws = static_cast<char*>(p.ws);
        // the totals walk with the features split like the gradient passes' operands
        constexpr bool kSplitK = Sh::kSplit;
        constexpr size_t kTotBytes = ShT::kBytes + (kSplitK ? size_t(D) * ShT::LKT * sizeof(E) : 0);
        auto* k_tot = walk_kernel<E, D, DV, C, GATED, false, false, false, 1, kSplitK>;
        auto* k_dq = bwd_dq_kernel<E, D, DV, GATED>;
        auto* k_dkv = bwd_dkv_kernel<E, D, DV, GATED>;
        static bool attrs_set = false;         // benign race: idempotent attribute set
        if (!attrs_set) {
            hipError_t e = set_lds(k_tot, kTotBytes);
            if (e == hipSuccess) e = set_lds(k_dq, Sh::kBytes);
            if (e == hipSuccess) e = set_lds(k_dkv, Sh::kBytes);
            if (e != hipSuccess) return e;
            attrs_set = true;
        }
        BwdArgs a;
        a.q = p.q; a.k = p.k; a.v = p.v; a.g = p.g; a.dout = p.dout; a.s0 = p.s0; a.z0 = p.z0;
        a.dq = p.dq; a.dk = p.dk; a.dv = p.dv;
        a.fst = reinterpret_cast<float*>(ws + lay.fwd);
        a.fzt = reinterpret_cast<float*>(ws + lay.fzt);
        a.rst = reinterpret_cast<float*>(ws + lay.rev);
        a.rzt = reinterpret_cast<float*>(ws + lay.rzt);
        a.rlg = reinterpret_cast<float*>(ws + lay.rlg);
        a.inv = reinterpret_cast<float*>(ws + lay.inv);
        a.dden = reinterpret_cast<float*>(ws + lay.dden);
        a.xs = reinterpret_cast<float*>(ws + lay.xs);
        a.yq = reinterpret_cast<float*>(ws + lay.yq);
        a.zk = reinterpret_cast<float*>(ws + lay.zk);
        a.wc = reinterpret_cast<float*>(ws + lay.wc);
        a.N = p.N; a.NC = NC; a.eps = p.eps; a.normalize = p.normalize;
        // as many workgroups per CU as the LDS holds (two at D = Dv = 64 bf16, with the
        // split operands' tiles): measured faster than fewer, longer runs
        a.LC = p.run > 0 ? (p.run < NC ? p.run : NC) : bwd_chunks_per_group(p.BH, NC, Sh::kWaves, p.cus);
        const int NR = (NC + a.LC - 1) / a.LC;
        a.NR = NR;
        // each run's forward total in as many parts as fill one round of the totals walk
        // (its runs alone can leave compute units idle), at most one per chunk; the slots
        // then number (NR - 1) FP + 1 <= NC per head, within the workspace
        {
            const long waves = walk_waves(int(sizeof(E)), D, DV, C, GATED, false);
            const long fit = long(kMaxLds / kTotBytes);
            const long round = long(p.cus) * (waves < fit ? waves : fit);
            long fp = NR > 1 ? round / (long(p.BH) * (NR - 1)) : 1;
            if (fp > a.LC) fp = a.LC;
            a.FP = fp < 1 ? 1 : int(fp);
        }
        a.FS = (NR - 1) * a.FP + 1;
        constexpr int NBLK = (D * DV + D + kThreads - 1) / kThreads;
        const unsigned BH = unsigned(p.BH);
        // the state in front of every run: the forward's totals walk with one run per
        // segment (in FP parts), then its scan over the parts (which starts from S0, z0)
        if (NR > 1) {
            WalkArgs w;
            w.q = p.q; w.k = p.k; w.v = p.v; w.g = p.g; w.o = nullptr;
            w.st = a.fst; w.zt = a.fzt; w.lg = reinterpret_cast<float*>(ws + lay.flg);
            w.s0 = p.s0; w.z0 = p.z0;
            w.N = p.N; w.BH = p.BH; w.nseg = NR; w.L = a.LC; w.tparts = a.FP; w.nslots = a.FS; w.direct = 0; w.want_final = 0; w.eps = p.eps; w.normalize = 1;
            hipLaunchKernelGGL(k_tot, dim3(BH * unsigned((NR - 1) * a.FP)), dim3(kThreads), kTotBytes, p.stream, w);
            hipLaunchKernelGGL((scan_kernel<D, DV, GATED>), dim3(BH * NBLK), dim3(kThreads), 0, p.stream, a.fst, a.fzt,
                               w.lg, p.s0, p.z0, a.FS, a.FS - 1, a.FP);
        }
        hipLaunchKernelGGL(k_dq, dim3(BH * unsigned(NR)), dim3(kThreads), Sh::kBytes, p.stream, a);
        // adjoint states: the scan over the runs' adjoint totals, last run first
        hipLaunchKernelGGL((scan_kernel<D, DV, GATED>), dim3(BH * NBLK), dim3(kThreads), 0, p.stream, a.rst, a.rzt,
                           a.rlg, static_cast<const float*>(nullptr), static_cast<const float*>(nullptr), NR + 1, NR, 1);
        hipLaunchKernelGGL(k_dkv, dim3(BH * unsigned(NR)), dim3(kThreads), Sh::kBytes, p.stream, a);
        if (GATED && p.dg) {
            const int nwork = p.BH * NC, per = kThreads / kWave;
            hipLaunchKernelGGL(bwd_dg_kernel, dim3(unsigned((nwork + per - 1) / per)), dim3(kThreads), 0, p.stream, p.g,
                               a.xs, a.yq, a.zk, a.wc, p.dg, p.N, NC, nwork);
        }
        if (p.ds0 || p.dz0)
            hipLaunchKernelGGL((final_kernel<D, DV>), dim3(BH * NBLK), dim3(kThreads), 0, p.stream, a.rst, a.rzt,
                               NR + 1, NR - 1, p.ds0, p.dz0);
        return hipGetLastError();
    }
}

template <typename E, int D, int DV>
hipError_t run_bwd_gate(const BwdLaunch& p) {
    return p.g ? run_bwd<E, D, DV, true>(p) : run_bwd<E, D, DV, false>(p);
}

template <typename E>
hipError_t run_bwd_typed(const BwdLaunch& p) {
    if (p.D == 64 && p.Dv == 64) return run_bwd_gate<E, 64, 64>(p);
    if (p.D == 64 && p.Dv == 128) return run_bwd_gate<E, 64, 128>(p);
    if (p.D == 128 && p.Dv == 64) return run_bwd_gate<E, 128, 64>(p);
    if (p.D == 128 && p.Dv == 128) return run_bwd_gate<E, 128, 128>(p);
    return hipErrorInvalidValue;
}

}  // namespace linattn
