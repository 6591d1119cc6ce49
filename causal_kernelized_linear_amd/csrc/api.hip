// C ABI of the library: argument checks, segment planning, workspace carving and
// dispatch to the kernel instantiations.  The contract is documented in
// include/linattn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <utility>

#include "../../include/linattn.h"
#include "launch.hpp"

namespace {

using linattn::FwdLaunch;

// Compute units of the current device (cached per ordinal); 256, an MI355X's count,
// when no device answers.
int device_cus() {
    static std::mutex mu;
    static int cus[256];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) {
        (void)hipGetLastError();
        return 256;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cus[dev] = n;
    }
    return cus[dev];
}

// Workgroups of one round of the output walk: compute units times the workgroups each
// holds at once.  Each head's sequence is split into nseg segments of L chunks so that
// B*H*nseg reaches this count when the sequence is long enough: every workgroup is then
// resident from the start, and the per-workgroup set-up (the state in front of the
// segment, the first loads) is paid once.
// vs: the column parts of Dv the walk is cut into (walk_vsplit), each with its own
// workgroups.
// split: the features allow the split output walk (elu + 1, relu + shift).
long target_workgroups(int esize, int D, int Dv, int chunk, bool gated, int vs = 1, bool split = true) {
    // the split output walk: one 8-wave workgroup per compute unit
    if (split && vs == 1 && linattn::walk_split(esize, D, Dv, chunk, gated)) return long(device_cus());
    return long(device_cus()) * linattn::walk_waves(esize, D, Dv / vs, chunk, gated, true);
}

// The largest target over the element types and both forwards (for the feature maps'
// walk, which is never cut into column parts): the workspace size does not depend on them.
long max_target_workgroups(int D, int Dv, int chunk) {
    long t = 0;
    for (int es : {2, 4})
        for (bool gated : {false, true}) {
            const long x = target_workgroups(es, D, Dv, chunk, gated, 1, false);
            t = x > t ? x : t;
        }
    return t;
}

struct Plan {
    int nseg = 0;
    int L = 0;
    int vs = 1;
    int tparts = 1;
    size_t bytes = 0;
};

// Each of the B*H*vs (head, column part) pairs is cut into nseg segments so that their
// count reaches the target, and each segment's total into tparts parts so that the
// totals walk fills `totals_round` workgroups.  nseg grows with the target (never
// shrinks), so the workspace sized for the largest target serves every smaller one.
Plan make_plan(long BH, int N, int D, int Dv, int chunk, long target, int vs = 1, long totals_round = 0) {
    Plan p;
    const long heads = BH * vs;
    const long nc = (long(N) + chunk - 1) / chunk;
    long nseg = (target + heads - 1) / heads;
    if (nseg < 1) nseg = 1;
    if (nseg > nc) nseg = nc;
    const long L = (nc + nseg - 1) / nseg;
    nseg = (nc + L - 1) / L;
    p.nseg = int(nseg);
    p.L = int(L);
    p.vs = vs;
    p.tparts = linattn::totals_parts(heads, p.nseg, p.L, D, Dv / vs, totals_round);
    const size_t nslots = size_t(p.nseg - 1) * size_t(p.tparts) + 1;
    p.bytes = linattn::fwd_workspace_layout(size_t(heads) * nslots, D, Dv / vs, nullptr, nullptr);
    return p;
}

// The plan of the chunked or gated forward (vs = 0: the shape is not supported).
Plan fwd_plan(int esize, long BH, int N, int D, int Dv, int chunk, bool gated) {
    const int vs = linattn::walk_vsplit(esize, D, Dv, chunk, gated);
    if (vs == 0) {
        Plan p;
        p.vs = 0;
        return p;
    }
    const long totals_round = long(device_cus()) * linattn::walk_waves(esize, D, Dv / vs, chunk, gated, false);
    return make_plan(BH, N, D, Dv, chunk, target_workgroups(esize, D, Dv, chunk, gated, vs), vs, totals_round);
}

// The plan of the walks under other feature maps (state rows M): relu + shift walks q
// and k as given, so it takes the chunked forward's plan, split walk included; FAVOR+
// keeps the 4-wave walks' plan with one part per segment total.
Plan feature_plan(int esize, bool gated, long BH, int N, int M, int Dv, int chunk, bool relu) {
    const long round = relu ? long(device_cus()) * linattn::walk_waves(esize, M, Dv, chunk, gated, false) : 0;
    return make_plan(BH, N, M, Dv, chunk, target_workgroups(esize, M, Dv, chunk, gated, 1, relu), 1, round);
}

// Workspace bytes that serve the forward of this shape whatever its element type and
// gating: the largest of their plans.
size_t fwd_workspace_bytes(long BH, int N, int D, int Dv, int chunk) {
    size_t b = 0;
    for (int es : {2, 4})
        for (bool gated : {false, true}) {
            const Plan p = fwd_plan(es, BH, N, D, Dv, chunk, gated);
            if (p.vs != 0 && p.bytes > b) b = p.bytes;
        }
    if (b == 0)   // no element type supports the shape: the plan it would have uncut
        b = make_plan(BH, N, D, Dv, chunk, max_target_workgroups(D, Dv, chunk)).bytes;
    return b;
}

// Scratch of linattn_fwd_ex_noalloc: a fixed array in device memory, one copy per device
// (the runtime places it when the library's device code loads there), held until the
// process ends.  Host code never uses the array's name as an address: its device address
// on the current device comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kScratchBytes = LINATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device, or NULL when it cannot be looked up.
void* device_scratch() {
    static std::mutex mu;
    static void* ptrs[256];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

// Measurement hook (linattn_set_profile_events): one-shot, process-wide.
std::mutex g_prof_mu;
hipEvent_t g_prof[4] = {nullptr, nullptr, nullptr, nullptr};

void take_profile_events(hipEvent_t out[4]) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    for (int i = 0; i < 4; ++i) {
        out[i] = g_prof[i];
        g_prof[i] = nullptr;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool dim_ok(int x) { return x == 64 || x == 128; }

size_t esize(linattn_dtype_t dt) { return dt == LINATTN_BF16 ? 2 : 4; }

bool dtype_ok(int dt) { return dt == LINATTN_F32 || dt == LINATTN_BF16; }

bool out_ok(int m) { return m == LINATTN_OUT_NORMALIZED || m == LINATTN_OUT_NUMERATOR; }

// The device must be a gfx950.  Cached per device ordinal.
linattn_status_t check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return LINATTN_ERR_HIP;
    }
    static std::mutex mu;
    static signed char usable[256];    // 0 unknown, 1 usable, -1 not usable
    if (dev >= 256) return LINATTN_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (usable[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return LINATTN_ERR_HIP;
        }
        usable[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    }
    return usable[dev] == 1 ? LINATTN_OK : LINATTN_ERR_HIP;
}

// fixed_scratch: the workspace is the library's own device array (ws and ws_bytes are
// ignored), for linattn_fwd_ex_noalloc.
linattn_status_t fwd_common(const void* q, const void* k, const void* v, const float* g, void* o, const float* s0,
                            const float* z0, float* s_out, float* z_out, int B, int H, int N, int D, int Dv,
                            int chunk, linattn_dtype_t dtype, float eps, linattn_output_t out, void* ws,
                            size_t ws_bytes, void* stream, bool fixed_scratch = false) {
    if (B < 0 || H < 0 || N < 0 || D <= 0 || Dv <= 0 || chunk <= 0) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(dtype) || !out_ok(out) || !(eps > 0.0f) || !std::isfinite(eps)) return LINATTN_ERR_INVALID_ARGUMENT;
    const long BH = long(B) * long(H);
    if (BH == 0 || N == 0) return LINATTN_OK;
    if (BH > (1L << 24) || long(N) * BH > (1L << 40)) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!q || !k || !v || !o) return LINATTN_ERR_INVALID_ARGUMENT;
    for (const void* p : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(g),
                          static_cast<const void*>(s0), static_cast<const void*>(z0),
                          static_cast<const void*>(s_out), static_cast<const void*>(z_out)})
        if (p && !aligned16(p)) return LINATTN_ERR_INVALID_ARGUMENT;
    const size_t es = esize(dtype);
    const size_t nqk = size_t(BH) * N * D * es, nv = size_t(BH) * N * Dv * es, ng = size_t(BH) * N * 4;
    const size_t ns = size_t(BH) * D * Dv * 4, nz = size_t(BH) * D * 4;
    // o is written while other workgroups still read every input and the initial state;
    // the final state is written after every read of the inputs, so s_out / z_out may
    // share memory with s0 / z0 but with nothing else
    if (overlap(o, nv, q, nqk) || overlap(o, nv, k, nqk) || overlap(o, nv, v, nv) || overlap(o, nv, g, ng) ||
        overlap(o, nv, s0, ns) || overlap(o, nv, z0, nz))
        return LINATTN_ERR_INVALID_ARGUMENT;
    for (const auto& fin : {std::make_pair(static_cast<const void*>(s_out), ns),
                            std::make_pair(static_cast<const void*>(z_out), nz)})
        if (overlap(fin.first, fin.second, q, nqk) || overlap(fin.first, fin.second, k, nqk) ||
            overlap(fin.first, fin.second, v, nv) || overlap(fin.first, fin.second, g, ng) ||
            overlap(fin.first, fin.second, o, nv))
            return LINATTN_ERR_INVALID_ARGUMENT;
    if (overlap(s_out, ns, z_out, nz)) return LINATTN_ERR_INVALID_ARGUMENT;
    // outputs are addressed with 32-bit byte offsets per head
    if ((size_t(N) + 256) * size_t(Dv) * es >= (size_t(1) << 31)) return LINATTN_ERR_UNSUPPORTED;
    if (!dim_ok(D) || !dim_ok(Dv) || !linattn::chunk_is_built(chunk)) return LINATTN_ERR_UNSUPPORTED;
    const Plan plan = fwd_plan(int(es), BH, N, D, Dv, chunk, g != nullptr);
    if (plan.vs == 0) return LINATTN_ERR_UNSUPPORTED;
    if (fixed_scratch) {
        if (plan.bytes > kScratchBytes) return LINATTN_ERR_SCRATCH_LIMIT;
        const linattn_status_t dst = check_device();
        if (dst != LINATTN_OK) return dst;
        ws = device_scratch();
        if (!ws) return LINATTN_ERR_HIP;
        ws_bytes = kScratchBytes;
    }
    if (ws_bytes < plan.bytes || !ws || !aligned16(ws)) return LINATTN_ERR_WORKSPACE;
    if (overlap(ws, plan.bytes, q, nqk) || overlap(ws, plan.bytes, k, nqk) || overlap(ws, plan.bytes, v, nv) ||
        overlap(ws, plan.bytes, o, nv) || overlap(ws, plan.bytes, g, ng) ||
        overlap(ws, plan.bytes, s0, ns) || overlap(ws, plan.bytes, s_out, ns) || overlap(ws, plan.bytes, z0, nz) ||
        overlap(ws, plan.bytes, z_out, nz))
        return LINATTN_ERR_WORKSPACE;
    const linattn_status_t dst = check_device();
    if (dst != LINATTN_OK) return dst;

    FwdLaunch L;
    L.prof[0] = L.prof[1] = L.prof[2] = L.prof[3] = nullptr;
    L.q = q; L.k = k; L.v = v; L.g = g; L.o = o;
    L.s0 = s0; L.z0 = z0; L.s_out = s_out; L.z_out = z_out;
    L.ws = ws;
    L.BH = int(BH); L.N = N; L.D = D; L.Dv = Dv; L.chunk = chunk;
    L.nseg = plan.nseg; L.L = plan.L; L.vsplit = plan.vs; L.tparts = plan.tparts; L.eps = eps;
    L.normalize = out == LINATTN_OUT_NORMALIZED ? 1 : 0;
    L.stream = static_cast<hipStream_t>(stream);
    take_profile_events(L.prof);
    (void)hipGetLastError();   // start from a clean error state
    const hipError_t e = dtype == LINATTN_BF16 ? linattn::launch_fwd_bf16(L) : linattn::launch_fwd_f32(L);
    return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

linattn_status_t decode_common(const void* q, const void* k, const void* v, const float* g, const float* ga, float* S,
                               float* z, void* o, int B, int H, int D, int Dv, linattn_dtype_t dtype, float eps,
                               linattn_output_t out, void* stream) {
    if (B < 0 || H < 0 || D <= 0 || Dv <= 0) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(dtype) || !out_ok(out) || !(eps > 0.0f) || !std::isfinite(eps)) return LINATTN_ERR_INVALID_ARGUMENT;
    const long BH = long(B) * long(H);
    if (BH == 0) return LINATTN_OK;
    if (BH > (1L << 31) - 1) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!q || !k || !v || !S || !o || (!z && out == LINATTN_OUT_NORMALIZED)) return LINATTN_ERR_INVALID_ARGUMENT;
    for (const void* p : {q, k, v, static_cast<const void*>(g), static_cast<const void*>(ga),
                          static_cast<const void*>(S), static_cast<const void*>(z), static_cast<const void*>(o)})
        if (p && !aligned16(p)) return LINATTN_ERR_INVALID_ARGUMENT;
    const size_t es = esize(dtype);
    const size_t no = size_t(BH) * Dv * es, ns = size_t(BH) * D * Dv * 4, nz = size_t(BH) * D * 4,
                 ng = size_t(BH) * 4;
    if (overlap(o, no, q, size_t(BH) * D * es) || overlap(o, no, k, size_t(BH) * D * es) || overlap(o, no, v, no) ||
        overlap(o, no, S, ns) || overlap(o, no, z, nz) || overlap(S, ns, z, nz) || overlap(g, ng, S, ns) ||
        overlap(g, ng, z, nz) || overlap(g, ng, o, no) || overlap(ga, nz, S, ns) || overlap(ga, nz, z, nz) ||
        overlap(ga, nz, o, no))
        return LINATTN_ERR_INVALID_ARGUMENT;
    if (!dim_ok(D) || !dim_ok(Dv)) return LINATTN_ERR_UNSUPPORTED;
    const linattn_status_t dst = check_device();
    if (dst != LINATTN_OK) return dst;
    (void)hipGetLastError();
    const hipError_t e = linattn::launch_decode(int(dtype), q, k, v, S, z, o, int(BH), D, Dv, eps, g, ga,
                                                out == LINATTN_OUT_NORMALIZED ? 1 : 0,
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

linattn_status_t bwd_common(const void* q, const void* k, const void* v, const float* g, const void* dout,
                            const float* s0, const float* z0, void* dq, void* dk, void* dv, float* dg, float* ds0,
                            float* dz0, int B, int H, int N, int D, int Dv, linattn_dtype_t dtype, float eps,
                            linattn_output_t out, int run, void* ws, size_t ws_bytes, void* stream) {
    if (B < 0 || H < 0 || N < 0 || D <= 0 || Dv <= 0 || run < 0) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(dtype) || !out_ok(out) || !(eps > 0.0f) || !std::isfinite(eps)) return LINATTN_ERR_INVALID_ARGUMENT;
    const long BH = long(B) * long(H);
    if (BH == 0 || N == 0) return LINATTN_OK;
    if (BH > (1L << 24) || long(N) * BH > (1L << 40)) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return LINATTN_ERR_INVALID_ARGUMENT;
    for (const void* p : {q, k, v, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                          static_cast<const void*>(dv), static_cast<const void*>(g), static_cast<const void*>(s0),
                          static_cast<const void*>(z0), static_cast<const void*>(dg), static_cast<const void*>(ds0),
                          static_cast<const void*>(dz0)})
        if (p && !aligned16(p)) return LINATTN_ERR_INVALID_ARGUMENT;
    const size_t es = esize(dtype);
    const size_t nqk = size_t(BH) * N * D * es, nv = size_t(BH) * N * Dv * es, ng = size_t(BH) * N * 4;
    const size_t ns = size_t(BH) * D * Dv * 4, nz = size_t(BH) * D * 4;
    struct Buf { const void* p; size_t n; };
    const Buf ins[] = {{q, nqk}, {k, nqk}, {v, nv}, {g, ng}, {dout, nv}, {s0, ns}, {z0, nz}};
    const Buf outs[] = {{dq, nqk}, {dk, nqk}, {dv, nv}, {g ? dg : nullptr, ng}, {ds0, ns}, {dz0, nz}};
    for (const Buf& o : outs) {
        for (const Buf& i : ins)
            if (overlap(o.p, o.n, i.p, i.n)) return LINATTN_ERR_INVALID_ARGUMENT;
        for (const Buf& o2 : outs)
            if (&o2 != &o && overlap(o.p, o.n, o2.p, o2.n)) return LINATTN_ERR_INVALID_ARGUMENT;
    }
    if ((size_t(N) + 256) * size_t(Dv > D ? Dv : D) * es >= (size_t(1) << 31)) return LINATTN_ERR_UNSUPPORTED;
    if (!dim_ok(D) || !dim_ok(Dv) || linattn::bwd_lds_bytes(int(es), D, Dv) > linattn::kMaxLds)
        return LINATTN_ERR_UNSUPPORTED;
    const linattn::BwdLayout lay = linattn::bwd_workspace_layout(size_t(BH), N, D, Dv);
    if (ws_bytes < lay.bytes || !ws || !aligned16(ws)) return LINATTN_ERR_WORKSPACE;
    for (const Buf& b : ins)
        if (overlap(ws, lay.bytes, b.p, b.n)) return LINATTN_ERR_WORKSPACE;
    for (const Buf& b : outs)
        if (overlap(ws, lay.bytes, b.p, b.n)) return LINATTN_ERR_WORKSPACE;
    const linattn_status_t dst = check_device();
    if (dst != LINATTN_OK) return dst;

    linattn::BwdLaunch L;
    L.q = q; L.k = k; L.v = v; L.g = g; L.dout = dout; L.s0 = s0; L.z0 = z0;
    L.dq = dq; L.dk = dk; L.dv = dv; L.dg = g ? dg : nullptr; L.ds0 = ds0; L.dz0 = dz0;
    L.ws = ws;
    L.BH = int(BH); L.N = N; L.D = D; L.Dv = Dv;
    L.eps = eps;
    L.normalize = out == LINATTN_OUT_NORMALIZED ? 1 : 0;
    L.cus = device_cus();
    L.run = run;
    L.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const hipError_t e = dtype == LINATTN_BF16 ? linattn::launch_bwd_bf16(L) : linattn::launch_bwd_f32(L);
    return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

linattn_status_t vd_common(const void* q, const void* k, const void* v, const float* a, void* o, const float* s0,
                           const float* z0, float* s_out, float* z_out, int B, int H, int N, int D, int Dv,
                           linattn_dtype_t dtype, float eps, linattn_output_t out, void* ws, size_t ws_bytes,
                           void* stream) {
    if (B < 0 || H < 0 || N < 0 || D <= 0 || Dv <= 0) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(dtype) || !out_ok(out) || !(eps > 0.0f) || !std::isfinite(eps)) return LINATTN_ERR_INVALID_ARGUMENT;
    const long BH = long(B) * long(H);
    if (BH == 0 || N == 0) return LINATTN_OK;
    if (BH > (1L << 24) || long(N) * BH > (1L << 40)) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!q || !k || !v || !a || !o) return LINATTN_ERR_INVALID_ARGUMENT;
    for (const void* p : {q, k, v, static_cast<const void*>(a), static_cast<const void*>(o),
                          static_cast<const void*>(s0), static_cast<const void*>(z0), static_cast<const void*>(s_out),
                          static_cast<const void*>(z_out)})
        if (p && !aligned16(p)) return LINATTN_ERR_INVALID_ARGUMENT;
    const size_t es = esize(dtype);
    const size_t nqk = size_t(BH) * N * D * es, nv = size_t(BH) * N * Dv * es, na = size_t(BH) * N * D * 4;
    const size_t ns = size_t(BH) * D * Dv * 4, nz = size_t(BH) * D * 4;
    if (overlap(o, nv, q, nqk) || overlap(o, nv, k, nqk) || overlap(o, nv, v, nv) || overlap(o, nv, a, na) ||
        overlap(s_out, ns, o, nv) || overlap(z_out, nz, o, nv) || overlap(s_out, ns, a, na) ||
        overlap(z_out, nz, a, na))
        return LINATTN_ERR_INVALID_ARGUMENT;
    if ((size_t(N) + 256) * size_t(Dv > D ? Dv : D) * 4 >= (size_t(1) << 31)) return LINATTN_ERR_UNSUPPORTED;
    if (!dim_ok(D) || !dim_ok(Dv) || linattn::vd_lds_bytes(int(es), D, Dv) > linattn::kMaxLds)
        return LINATTN_ERR_UNSUPPORTED;
    const linattn::VdLayout lay = linattn::vd_workspace_layout(size_t(BH), N, D, Dv);
    if (ws_bytes < lay.bytes || !ws || !aligned16(ws)) return LINATTN_ERR_WORKSPACE;
    for (const auto& b : {std::make_pair(static_cast<const void*>(q), nqk), std::make_pair(static_cast<const void*>(k), nqk),
                          std::make_pair(static_cast<const void*>(v), nv), std::make_pair(static_cast<const void*>(a), na),
                          std::make_pair(static_cast<const void*>(o), nv), std::make_pair(static_cast<const void*>(s0), ns),
                          std::make_pair(static_cast<const void*>(z0), nz),
                          std::make_pair(static_cast<const void*>(s_out), ns),
                          std::make_pair(static_cast<const void*>(z_out), nz)})
        if (overlap(ws, lay.bytes, b.first, b.second)) return LINATTN_ERR_WORKSPACE;
    const linattn_status_t dst = check_device();
    if (dst != LINATTN_OK) return dst;
    linattn::VdLaunch L;
    L.q = q; L.k = k; L.v = v; L.a = a; L.o = o; L.s0 = s0; L.z0 = z0; L.s_out = s_out; L.z_out = z_out;
    L.ws = ws;
    L.BH = int(BH); L.N = N; L.D = D; L.Dv = Dv; L.eps = eps;
    L.normalize = out == LINATTN_OUT_NORMALIZED ? 1 : 0;
    L.cus = device_cus();
    L.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const hipError_t e = dtype == LINATTN_BF16 ? linattn::launch_vd_bf16(L) : linattn::launch_vd_f32(L);
    return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

size_t feature_bytes(long BH, int N, int M, size_t es) { return linattn::round_up256(size_t(BH) * N * M * es); }

linattn_status_t feat_common(const void* q, const void* k, const void* v, const float* g, void* o, const float* s0,
                             const float* z0, float* s_out, float* z_out, int B, int H, int N, int D, int Dv,
                             int chunk, linattn_dtype_t dtype, float eps, linattn_output_t out, int feature,
                             float shift, const float* W, int M, void* ws, size_t ws_bytes, void* stream) {
    if (B < 0 || H < 0 || N < 0 || D <= 0 || Dv <= 0 || chunk <= 0 || M <= 0) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!dtype_ok(dtype) || !out_ok(out) || !(eps > 0.0f) || !std::isfinite(eps) || !std::isfinite(shift))
        return LINATTN_ERR_INVALID_ARGUMENT;
    if (feature != LINATTN_FEATURE_RELU && feature != LINATTN_FEATURE_FAVOR) return LINATTN_ERR_INVALID_ARGUMENT;
    if ((feature == LINATTN_FEATURE_RELU) != (W == nullptr)) return LINATTN_ERR_INVALID_ARGUMENT;
    if (feature == LINATTN_FEATURE_RELU && M != D) return LINATTN_ERR_INVALID_ARGUMENT;
    const long BH = long(B) * long(H);
    if (BH == 0 || N == 0) return LINATTN_OK;
    if (BH > (1L << 24) || long(N) * BH > (1L << 40)) return LINATTN_ERR_INVALID_ARGUMENT;
    if (!q || !k || !v || !o) return LINATTN_ERR_INVALID_ARGUMENT;
    for (const void* p : {q, k, v, static_cast<const void*>(g), static_cast<const void*>(o),
                          static_cast<const void*>(s0), static_cast<const void*>(z0), static_cast<const void*>(s_out),
                          static_cast<const void*>(z_out), static_cast<const void*>(W)})
        if (p && !aligned16(p)) return LINATTN_ERR_INVALID_ARGUMENT;
    const size_t es = esize(dtype);
    const size_t nqk = size_t(BH) * N * D * es, nv = size_t(BH) * N * Dv * es, nw = size_t(H) * M * D * 4;
    const size_t ns = size_t(BH) * M * Dv * 4, nz = size_t(BH) * M * 4;
    if (overlap(o, nv, q, nqk) || overlap(o, nv, k, nqk) || overlap(o, nv, v, nv) ||
        overlap(o, nv, g, size_t(BH) * N * 4) || overlap(o, nv, W, nw))
        return LINATTN_ERR_INVALID_ARGUMENT;
    if ((size_t(N) + 256) * size_t(Dv > M ? Dv : M) * es >= (size_t(1) << 31)) return LINATTN_ERR_UNSUPPORTED;
    if (!dim_ok(D) || !dim_ok(Dv) || !dim_ok(M) || (chunk != 64 && chunk != 128) ||
        linattn::walk_lds_bytes(int(es), M, Dv, chunk, g != nullptr) > linattn::kMaxLds ||
        (feature == LINATTN_FEATURE_FAVOR && (size_t(64) * (D + 4) + size_t(M) * (D + 4) + 64) * 4 > linattn::kMaxLds))
        return LINATTN_ERR_UNSUPPORTED;
    const Plan plan = feature_plan(int(es), g != nullptr, BH, N, M, Dv, chunk, feature == LINATTN_FEATURE_RELU);
    const size_t fb = feature_bytes(BH, N, M, es);
    const size_t need = 2 * fb + plan.bytes;
    if (ws_bytes < need || !ws || !aligned16(ws)) return LINATTN_ERR_WORKSPACE;
    for (const auto& b : {std::make_pair(static_cast<const void*>(q), nqk), std::make_pair(static_cast<const void*>(k), nqk),
                          std::make_pair(static_cast<const void*>(v), nv), std::make_pair(static_cast<const void*>(o), nv),
                          std::make_pair(static_cast<const void*>(g), size_t(BH) * N * 4),
                          std::make_pair(static_cast<const void*>(W), nw),
                          std::make_pair(static_cast<const void*>(s0), ns), std::make_pair(static_cast<const void*>(z0), nz),
                          std::make_pair(static_cast<const void*>(s_out), ns),
                          std::make_pair(static_cast<const void*>(z_out), nz)})
        if (overlap(ws, need, b.first, b.second)) return LINATTN_ERR_WORKSPACE;
    const linattn_status_t dst = check_device();
    if (dst != LINATTN_OK) return dst;
    linattn::FeatLaunch L;
    FwdLaunch& F = L.fwd;
    F.prof[0] = F.prof[1] = F.prof[2] = F.prof[3] = nullptr;
    F.q = q; F.k = k; F.v = v; F.g = g; F.o = o;
    F.s0 = s0; F.z0 = z0; F.s_out = s_out; F.z_out = z_out;
    F.ws = ws;
    F.BH = int(BH); F.N = N; F.D = D; F.Dv = Dv; F.chunk = chunk;
    F.nseg = plan.nseg; F.L = plan.L; F.tparts = plan.tparts; F.eps = eps;
    F.normalize = out == LINATTN_OUT_NORMALIZED ? 1 : 0;
    F.stream = static_cast<hipStream_t>(stream);
    L.kind = feature; L.shift = shift; L.W = W; L.H = H; L.M = M; L.es = int(es);
    L.BH = int(BH); L.N = N; L.D = D; L.stream = F.stream;
    (void)hipGetLastError();
    const hipError_t e = linattn::launch_feature_fwd(L);
    return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

}  // namespace

extern "C" {

size_t linattn_fwd_features_workspace_size(int B, int H, int N, int D, int Dv, int chunk, int M,
                                           linattn_dtype_t dtype) {
    if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || Dv <= 0 || chunk <= 0 || M <= 0 || !dtype_ok(dtype)) return 0;
    const long BH = long(B) * long(H);
    const size_t es = esize(dtype);
    // the largest of the feature maps' plans over gating (relu + shift may take the split
    // walk's plan: fewer segments, but their totals in parts)
    size_t b = make_plan(BH, N, M, Dv, chunk, max_target_workgroups(M, Dv, chunk)).bytes;
    for (bool gated : {false, true}) {
        const size_t r = feature_plan(int(es), gated, BH, N, M, Dv, chunk, true).bytes;
        b = r > b ? r : b;
    }
    return 2 * feature_bytes(BH, N, M, es) + b;
}

linattn_status_t linattn_fwd_features(const void* q, const void* k, const void* v, const float* g, void* o,
                                      const float* s0, const float* z0, float* s_out, float* z_out, int B, int H,
                                      int N, int D, int Dv, int chunk, linattn_dtype_t dtype, float eps,
                                      linattn_output_t out, linattn_feature_t feature, float shift, const float* W,
                                      int M, void* workspace, size_t workspace_bytes, void* stream) {
    try {
        return feat_common(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, out, int(feature),
                           shift, W, M, workspace, workspace_bytes, stream);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

size_t linattn_bwd_workspace_size(int B, int H, int N, int D, int Dv, linattn_dtype_t dtype) {
    if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || Dv <= 0 || !dtype_ok(dtype)) return 0;
    return linattn::bwd_workspace_layout(size_t(B) * size_t(H), N, D, Dv).bytes;
}

linattn_status_t linattn_bwd(const void* q, const void* k, const void* v, const float* g, const void* dout,
                             const float* s0, const float* z0, void* dq, void* dk, void* dv, float* dg, float* ds0,
                             float* dz0, int B, int H, int N, int D, int Dv, linattn_dtype_t dtype, float eps,
                             linattn_output_t out, int run, void* workspace, size_t workspace_bytes, void* stream) {
    try {
        return bwd_common(q, k, v, g, dout, s0, z0, dq, dk, dv, dg, ds0, dz0, B, H, N, D, Dv, dtype, eps, out, run,
                          workspace, workspace_bytes, stream);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

size_t linattn_fwd_workspace_size(int B, int H, int N, int D, int Dv, int chunk) {
    if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || Dv <= 0 || chunk <= 0) return 0;
    return fwd_workspace_bytes(long(B) * long(H), N, D, Dv, chunk);
}

linattn_status_t linattn_fwd_chunked(const void* q, const void* k, const void* v, void* o, const float* s0,
                                     const float* z0, float* s_out, float* z_out, int B, int H, int N, int D, int Dv,
                                     int chunk, linattn_dtype_t dtype, float eps, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    try {
        return fwd_common(q, k, v, nullptr, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps,
                          LINATTN_OUT_NORMALIZED, workspace, workspace_bytes, stream);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

linattn_status_t linattn_fwd_gated(const void* q, const void* k, const void* v, const float* g, void* o,
                                   const float* s0, const float* z0, float* s_out, float* z_out, int B, int H, int N,
                                   int D, int Dv, int chunk, linattn_dtype_t dtype, float eps, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    try {
        if (!g && long(B) * long(H) * long(N) > 0) return LINATTN_ERR_INVALID_ARGUMENT;
        return fwd_common(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps,
                          LINATTN_OUT_NORMALIZED, workspace, workspace_bytes, stream);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

linattn_status_t linattn_fwd_ex(const void* q, const void* k, const void* v, const float* g, void* o, const float* s0,
                                const float* z0, float* s_out, float* z_out, int B, int H, int N, int D, int Dv,
                                int chunk, linattn_dtype_t dtype, float eps, linattn_output_t out, void* workspace,
                                size_t workspace_bytes, void* stream) {
    try {
        return fwd_common(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, out, workspace,
                          workspace_bytes, stream);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

linattn_status_t linattn_fwd_ex_noalloc(const void* q, const void* k, const void* v, const float* g, void* o,
                                        const float* s0, const float* z0, float* s_out, float* z_out, int B, int H,
                                        int N, int D, int Dv, int chunk, linattn_dtype_t dtype, float eps,
                                        linattn_output_t out, void* stream) {
    try {
        return fwd_common(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, out, nullptr, 0,
                          stream, true);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

linattn_status_t linattn_decode_step(const void* q, const void* k, const void* v, float* S, float* z, void* o, int B,
                                     int H, int D, int Dv, linattn_dtype_t dtype, float eps, void* stream) {
    try {
        return decode_common(q, k, v, nullptr, nullptr, S, z, o, B, H, D, Dv, dtype, eps, LINATTN_OUT_NORMALIZED,
                             stream);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

linattn_status_t linattn_decode_step_ex(const void* q, const void* k, const void* v, const float* g, float* S,
                                        float* z, void* o, int B, int H, int D, int Dv, linattn_dtype_t dtype,
                                        float eps, linattn_output_t out, void* stream) {
    try {
        return decode_common(q, k, v, g, nullptr, S, z, o, B, H, D, Dv, dtype, eps, out, stream);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

linattn_status_t linattn_decode_step_vdecay(const void* q, const void* k, const void* v, const float* a, float* S,
                                            float* z, void* o, int B, int H, int D, int Dv, linattn_dtype_t dtype,
                                            float eps, linattn_output_t out, void* stream) {
    try {
        if (!a && long(B) * long(H) > 0) return LINATTN_ERR_INVALID_ARGUMENT;
        return decode_common(q, k, v, nullptr, a, S, z, o, B, H, D, Dv, dtype, eps, out, stream);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

size_t linattn_fwd_vdecay_workspace_size(int B, int H, int N, int D, int Dv) {
    if (B <= 0 || H <= 0 || N <= 0 || D <= 0 || Dv <= 0) return 0;
    return linattn::vd_workspace_layout(size_t(B) * size_t(H), N, D, Dv).bytes;
}

linattn_status_t linattn_fwd_vdecay(const void* q, const void* k, const void* v, const float* a, void* o,
                                    const float* s0, const float* z0, float* s_out, float* z_out, int B, int H, int N,
                                    int D, int Dv, linattn_dtype_t dtype, float eps, linattn_output_t out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    try {
        return vd_common(q, k, v, a, o, s0, z0, s_out, z_out, B, H, N, D, Dv, dtype, eps, out, workspace,
                         workspace_bytes, stream);
    } catch (...) {
        return LINATTN_ERR_HIP;
    }
}

linattn_status_t linattn_set_profile_events(void* ev0, void* ev1, void* ev2, void* ev3) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof[0] = static_cast<hipEvent_t>(ev0);
    g_prof[1] = static_cast<hipEvent_t>(ev1);
    g_prof[2] = static_cast<hipEvent_t>(ev2);
    g_prof[3] = static_cast<hipEvent_t>(ev3);
    return LINATTN_OK;
}

const char* linattn_status_string(linattn_status_t status) {
    switch (status) {
        case LINATTN_OK: return "ok";
        case LINATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LINATTN_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case LINATTN_ERR_WORKSPACE: return "workspace missing, too small, misaligned or overlapping";
        case LINATTN_ERR_HIP: return "HIP error or no usable gfx950 device";
        case LINATTN_ERR_SCRATCH_LIMIT:
            return "problem needs more scratch than the fixed device array of linattn_fwd_ex_noalloc holds";
        default: return "unknown status";
    }
}

}  // extern "C"
