// Dispatch of the per-dimension-decay forward for both element types.
#include "bwd_dispatch.hpp"
#include "vdecay.hpp"

namespace linattn {

template <typename E, int D, int DV>
static hipError_t run_vd(const VdLaunch& p) {
    using Sh = VdShape<E, D, DV>;
    if constexpr (Sh::kBytes > kMaxLds) {
        return hipErrorInvalidValue;           // rejected earlier by the ABI's support check
    } else {
        constexpr int C = kBwdChunk;
        const int NC = (p.N + C - 1) / C;
        const VdLayout lay = vd_workspace_layout(size_t(p.BH), p.N, D, DV);
        char* ws = static_cast<char*>(p.ws);
        auto* k_tot = vd_totals_kernel<E, D, DV>;
        auto* k_out = vd_out_kernel<E, D, DV>;
        static bool attrs_set = false;         // benign race: idempotent attribute set
        if (!attrs_set) {
            hipError_t e = set_lds(k_tot, Sh::kBytes);
            if (e == hipSuccess) e = set_lds(k_out, Sh::kBytes);
            if (e != hipSuccess) return e;
            attrs_set = true;
        }
        VdArgs a;
        a.q = p.q; a.k = p.k; a.v = p.v; a.a = p.a; a.o = p.o; a.s0 = p.s0; a.z0 = p.z0;
        a.st = reinterpret_cast<float*>(ws + lay.st);
        a.zt = reinterpret_cast<float*>(ws + lay.zt);
        a.lg = reinterpret_cast<float*>(ws + lay.lg);
        a.N = p.N; a.NC = NC; a.eps = p.eps; a.normalize = p.normalize;
        const bool want_final = p.s_out || p.z_out;
        a.LC = bwd_chunks_per_group(p.BH, NC, Sh::kWaves, p.cus);
        a.NR = (NC + a.LC - 1) / a.LC;
        a.NT = want_final ? a.NR : a.NR - 1;
        const unsigned BH = unsigned(p.BH);
        constexpr int NBLK = (D * DV + D + kThreads - 1) / kThreads;
        // run totals, their scan (the state after every run, from S0), outputs
        if (a.NT > 0) {
            hipLaunchKernelGGL(k_tot, dim3(BH * unsigned(a.NT)), dim3(kThreads), Sh::kBytes, p.stream, a);
            hipLaunchKernelGGL((vd_scan_kernel<D, DV>), dim3(BH * NBLK), dim3(kThreads), 0, p.stream, a.st, a.zt, a.lg,
                               p.s0, p.z0, a.NT, a.NR);
        }
        hipLaunchKernelGGL(k_out, dim3(BH * unsigned(a.NR)), dim3(kThreads), Sh::kBytes, p.stream, a);
        if (want_final)
            hipLaunchKernelGGL((final_kernel<D, DV>), dim3(BH * NBLK), dim3(kThreads), 0, p.stream, a.st, a.zt, a.NR,
                               a.NR - 1, p.s_out, p.z_out);
        return hipGetLastError();
    }
}

template <typename E>
static hipError_t run_vd_typed(const VdLaunch& p) {
    if (p.D == 64 && p.Dv == 64) return run_vd<E, 64, 64>(p);
    if (p.D == 64 && p.Dv == 128) return run_vd<E, 64, 128>(p);
    if (p.D == 128 && p.Dv == 64) return run_vd<E, 128, 64>(p);
    if (p.D == 128 && p.Dv == 128) return run_vd<E, 128, 128>(p);
    return hipErrorInvalidValue;
}

hipError_t launch_vd_bf16(const VdLaunch& p) { return run_vd_typed<uint16_t>(p); }
hipError_t launch_vd_f32(const VdLaunch& p) { return run_vd_typed<float>(p); }

}  // namespace linattn
