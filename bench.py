"""Benchmark of the causal kernelized linear attention hot path on one MI355X.

One step = one chunked forward (phi, per-segment state totals, the prefix that
carries the state across segments, the masked intra-chunk products, the
carried-state term and the divide) over the
training-shaped workload B=8, H=16, N=4096, D=Dv=64, bf16, chunk 128, with the
inputs already resident in HBM.  Input sets are rotated so no step starts with
its inputs warm in the 256 MB Infinity Cache.  The scalar-gated forward
(B=4, H=16, N=8192, D=Dv=64, chunk 128), the long-context forward
(B=1, H=32, N=65536, D=Dv=128, chunk sweep), the decode step (B=256, H=32,
D=Dv=128, fp32 state), its gated form, the normaliser-free output mode of the
gated forward and of the gated decode, the backward of the training-shaped and
gated forwards, the per-dimension decay (forward and decode) and the ReLU and FAVOR+
feature maps are timed in the same run and reported in extra fields.

Prints ONE JSON line.  ms_per_step and value come from a timed pass bracketed by
two hipEvents only.  Per-kernel durations come from a second timed pass of the same
length with hipEvents recorded on the launch stream around each kernel (the
library's measurement hook); those markers sit between dependent launches and add a
few microseconds each, so they never enter the headline.  A third pass brackets
only the output walk (one event before it, one after); the roofline object prices
that kernel time against MI355X's 8 TB/s.  Its traffic figure comes from the
committed rocprofv3 counter summary and is null once the kernel sources have
changed.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
# the forward's steps between the measurement hook's four events: segment totals, the
# scan over segments (skipped when the output walk sums the prefix itself), output walk
PHASES = ("walk_totals", "scan", "walk_output")
DOMINANT = ("walk_output", "walk_kernel<bf16,64,64,{c},ungated,output>")
KERNEL_SOURCES = os.path.join(ROOT, "causal_kernelized_linear_amd", "csrc")
COUNTERS = os.path.join(ROOT, "profiles", "counters_walk_output_train_bf16.json")
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "causal linear-attn fwd tokens/s + % bf16 MFMA peak; decode GB/s % HBM peak"


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        import torch
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(h.value)
        self.pool.extend(out)
        return out

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, a, b):
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(f.value)

    def close(self):
        for h in self.pool:
            self.hip.hipEventDestroy(h)
        self.pool = []


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def fwd_units(w):
    return w.B * w.H * w.N


def fwd_bytes_per_unit(w):
    es = 4 if w.dtype == "f32" else 2
    b = (2 * w.D + w.Dv) * es + w.Dv * es
    if w.kind == "gated":
        b += 4
    return b


def fwd_flops_per_unit(w, chunk):
    return 4 * w.D * w.Dv + (chunk + 1) * (w.D + w.Dv)


def time_forward(w, chunk, steps, warmup, ev, rotate_bytes=600e6, normalize=True):
    """Time `steps` forwards of workload w; returns a dict of timings (ms).

    Two timed passes of `steps` forwards each.  The first is bracketed by two hipEvents
    only: it gives ms_per_step.  The second also records the library's four per-launch
    events on every forward (the measurement hook), which gives the per-kernel times;
    those event records sit between dependent launches and lengthen the step, so the
    headline figure never comes from the second pass."""
    import torch
    from causal_kernelized_linear_amd import binding, workloads

    dev = torch.device("cuda:0")
    base = workloads.make_inputs(w)
    sets = [{n: t.to(dev) for n, t in base.items()}]
    per_set = sum(t.numel() * t.element_size() for t in sets[0].values())
    nsets = max(2, min(6, int(rotate_bytes // max(per_set, 1)) + 1))
    for _ in range(nsets - 1):
        sets.append({n: t.clone() for n, t in sets[0].items()})
    outs = [torch.empty(w.B, w.H, w.N, w.Dv, dtype=w.torch_dtype, device=dev) for _ in range(nsets)]
    ws = torch.empty(max(binding.workspace_bytes(w.B, w.H, w.N, w.D, w.Dv, chunk), 1), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(i):
        s = sets[i % nsets]
        if not normalize:
            binding.fwd(s["q"], s["k"], s["v"], g=s.get("g"), chunk=chunk, out=outs[i % nsets], workspace=ws,
                        normalize=False)
        elif w.kind == "gated":
            binding.fwd_gated(s["q"], s["k"], s["v"], s["g"], chunk=chunk, out=outs[i % nsets], workspace=ws)
        else:
            binding.fwd_chunked(s["q"], s["k"], s["v"], chunk=chunk, out=outs[i % nsets], workspace=ws)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    # pass 1: the whole forward, no per-launch events
    t0, t1 = ev.create(2)
    wall0 = time.perf_counter()
    ev.record(t0, stream)
    for i in range(steps):
        call(i)
    ev.record(t1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev.ms(t0, t1)
    # pass 2: the same forwards with the per-launch events
    evs = [ev.create(4) for _ in range(steps)]
    u0, u1 = ev.create(2)
    ev.record(u0, stream)
    for i in range(steps):
        binding.linattn_set_profile_events(*evs[i])
        call(i)
    ev.record(u1, stream)
    torch.cuda.synchronize()
    names = PHASES
    per = {nm: [ev.ms(e[i], e[i + 1]) for e in evs] for i, nm in enumerate(names)}
    # pass 3: only the output walk bracketed (one event before it, one after)
    ows = [ev.create(2) for _ in range(steps)]
    for i in range(steps):
        binding.linattn_set_profile_events(0, 0, ows[i][0], ows[i][1])
        call(i)
    torch.cuda.synchronize()
    out_only = [ev.ms(a, b) for a, b in ows]
    res = {
        "ms_per_step": total_ms / steps,
        "wall_ms_per_step": 1e3 * wall / steps,
        "ms_per_step_with_launch_events": ev.ms(u0, u1) / steps,
        "kernel_ms": {nm: sum(v) / steps for nm, v in per.items()},
        "kernel_ms_median": {nm: _median(v) for nm, v in per.items()},
        "walk_output_ms_alone": sum(out_only) / steps,
        "input_sets": nsets,
    }
    del sets, outs, ws
    torch.cuda.empty_cache()
    return res


def time_decode(w, steps, warmup, ev, normalize=True):
    """Per-step time of the decode step (gated when the workload carries g); in the
    normaliser-free mode z is not passed, so the step moves no z bytes."""
    import torch
    from causal_kernelized_linear_amd import binding, workloads

    dev = torch.device("cuda:0")
    base = workloads.make_inputs(w)
    nsets = 2                                  # 2 x 516 MiB of state: never warm in the 256 MB cache
    sets = [{n: t.to(dev) for n, t in base.items()}]
    sets.append({n: t.clone() for n, t in sets[0].items()})
    outs = [torch.empty(w.B, w.H, w.Dv, dtype=w.torch_dtype, device=dev) for _ in range(nsets)]
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(i):
        s = sets[i % nsets]
        binding.decode_step(s["q"], s["k"], s["v"], s["S"], s["z"] if normalize else None, out=outs[i % nsets],
                            g=s.get("g"), normalize=normalize, a=s.get("a"))

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    evs = [ev.create(2) for _ in range(steps)]
    for i in range(steps):
        ev.record(evs[i][0], stream)
        call(i)
        ev.record(evs[i][1], stream)
    torch.cuda.synchronize()
    ks = [ev.ms(a, b) for a, b in evs]
    del sets, outs
    torch.cuda.empty_cache()
    return {"ms_per_step": sum(ks) / steps, "ms_median": _median(ks)}


BWD_CHUNK = 64                  # the backward's own chunk


def bwd_bytes_per_unit(w):
    """q, k, v, dout read once and dq, dk, dv written once (plus g read and dg written)."""
    es = 4 if w.dtype == "f32" else 2
    b = 2 * (2 * w.D + w.Dv) * es + w.Dv * es
    if w.kind == "gated":
        b += 8
    return b


def bwd_flops_per_unit(w):
    """Products per token-head of the chunked backward, recompute included: six state-sized
    products (the chunk totals, Fq S_prev, dOut S_prev^T, the adjoint fold, Fk R, V R^T)
    of 2 D Dv each, and the causal halves of eight chunk products (A and B in both
    kernels, A V, B Fk, A^T dOut, B^T Fq)."""
    return 12 * w.D * w.Dv + 4 * (BWD_CHUNK + 1) * (w.D + w.Dv)


def time_backward(w, steps, warmup, ev):
    """Per-step time of linattn_bwd on workload w (inputs and outputs preallocated)."""
    import torch
    from causal_kernelized_linear_amd import binding, workloads

    dev = torch.device("cuda:0")
    base = workloads.make_inputs(w, with_grad=True)
    sets = [{n: t.to(dev) for n, t in base.items()}]
    sets.append({n: t.clone() for n, t in sets[0].items()})
    grads = [{"dq": torch.empty_like(s["q"]), "dk": torch.empty_like(s["k"]), "dv": torch.empty_like(s["v"]),
              "dg": torch.empty_like(s["g"]) if "g" in s else None} for s in sets]
    dt = binding.BF16 if w.dtype == "bf16" else binding.F32
    ws = torch.empty(binding.linattn_bwd_workspace_size(w.B, w.H, w.N, w.D, w.Dv, dt), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(i):
        s = sets[i % 2]
        binding.bwd(s["q"], s["k"], s["v"], s["dout"], g=s.get("g"), workspace=ws, grads=grads[i % 2])

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0, t1 = ev.create(2)
    ev.record(t0, stream)
    for i in range(steps):
        call(i)
    ev.record(t1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    del sets, grads, ws
    torch.cuda.empty_cache()
    return {"ms_per_step": ms}


def vd_bytes_per_unit(w):
    """q, k, v and the per-dimension decay read once, o written once."""
    es = 4 if w.dtype == "f32" else 2
    return (2 * w.D + w.Dv) * es + 4 * w.D + w.Dv * es


def time_vdecay(w, steps, warmup, ev):
    """Per-step time of linattn_fwd_vdecay on workload w (two input sets rotated)."""
    import torch
    from causal_kernelized_linear_amd import binding, workloads

    dev = torch.device("cuda:0")
    base = workloads.make_inputs(w)
    sets = [{n: t.to(dev) for n, t in base.items()}]
    sets.append({n: t.clone() for n, t in sets[0].items()})
    outs = [torch.empty(w.B, w.H, w.N, w.Dv, dtype=w.torch_dtype, device=dev) for _ in range(2)]
    ws = torch.empty(binding.linattn_fwd_vdecay_workspace_size(w.B, w.H, w.N, w.D, w.Dv), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(i):
        s = sets[i % 2]
        binding.fwd_vdecay(s["q"], s["k"], s["v"], s["a"], out=outs[i % 2], workspace=ws)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0, t1 = ev.create(2)
    ev.record(t0, stream)
    for i in range(steps):
        call(i)
    ev.record(t1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    del sets, outs, ws
    torch.cuda.empty_cache()
    return {"ms_per_step": ms}


def time_features(w, feature, steps, warmup, ev, M=64):
    """Per-step time of linattn_fwd_features on workload w (two input sets rotated)."""
    import torch
    from causal_kernelized_linear_amd import binding, workloads

    dev = torch.device("cuda:0")
    base = workloads.make_inputs(w)
    sets = [{n: t.to(dev) for n, t in base.items()}]
    sets.append({n: t.clone() for n, t in sets[0].items()})
    W = workloads.favor_projection(w.seed, w.H, M, w.D).to(dev) if feature == "favor" else None
    m = M if feature == "favor" else w.D
    dt = binding.BF16 if w.dtype == "bf16" else binding.F32
    ws = torch.empty(binding.linattn_fwd_features_workspace_size(w.B, w.H, w.N, w.D, w.Dv, w.chunks[0], m, dt),
                     dtype=torch.uint8, device=dev)
    outs = [torch.empty(w.B, w.H, w.N, w.Dv, dtype=w.torch_dtype, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream(dev).cuda_stream

    def call(i):
        s = sets[i % 2]
        binding.fwd_features(s["q"], s["k"], s["v"], feature, shift=0.05, W=W, chunk=w.chunks[0], out=outs[i % 2],
                             workspace=ws)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    t0, t1 = ev.create(2)
    ev.record(t0, stream)
    for i in range(steps):
        call(i)
    ev.record(t1, stream)
    torch.cuda.synchronize()
    ms = ev.ms(t0, t1) / steps
    del sets, outs, ws
    torch.cuda.empty_cache()
    return {"ms_per_step": ms}


def decode_bytes(w, with_z=True):
    """S (and z) read and written once, q, k, v read, o written, plus the gate when gated."""
    es = 4 if w.dtype == "f32" else 2
    per_head = 2 * (w.D * w.Dv + (w.D if with_z else 0)) * 4 + (2 * w.D + w.Dv) * es + w.Dv * es
    if w.kind == "decode_gated":
        per_head += 4
    if w.kind == "decode_vdecay":
        per_head += 4 * w.D
    return per_head * w.B * w.H


# the files the dominant kernel (the bf16 output walk) is built from
DOMINANT_SOURCES = ("chunk_walk.hpp", "device_common.hpp", "fwd_bf16.hip", "fwd_dispatch.hpp", "launch.hpp")


def source_digest():
    """sha256 over the dominant kernel's sources, to tell whether stored counters still apply."""
    import hashlib
    h = hashlib.sha256()
    for name in DOMINANT_SOURCES:
        with open(os.path.join(KERNEL_SOURCES, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(kernel_name):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary, scaled by its copy-kernel calibration; None when the kernel sources changed
    since the counters were taken."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_sha256") != source_digest() or c.get("kernel") != kernel_name:
        return None
    return 1024.0 * (c["fetch_kib"] * c["fetch_factor"] + c["write_kib"] * c["write_factor"])


def cpu_baseline(w, seconds_hint=10.0):
    """The fp64 oracle, as it stands, on a bounded sample of workload w (all heads,
    the first tokens), on the host cores; returns tokens/s scaled to the workload."""
    import numpy as np
    from causal_kernelized_linear_amd import workloads
    import oracle

    ntok = w.N
    inp = workloads.make_inputs(w, N=ntok)
    q, k, v = (workloads.to_f64(inp[n]) for n in ("q", "k", "v"))
    t = time.perf_counter()
    oracle.causal_linear_attention(q, k, v)
    dt = time.perf_counter() - t
    # B*ntok token positions (every head) in dt seconds
    return {
        "value": w.B * ntok / dt,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"fp64 NumPy recurrence over the whole workload ({w.B}x{w.H} heads, {ntok} tokens), "
                  f"{dt:.1f} s, one thread (elementwise NumPy and einsum), "
                  f"host has {os.cpu_count()} cpus, affinity {len(os.sched_getaffinity(0))}",
        "seconds": dt,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The device needs tens of milliseconds of sustained work to reach its steady clocks:
    # after 10 warmup steps (about 1 ms) train_bf16 measured 85-87 us per step, after 1000
    # (about 80 ms) 71-72 us, run after run on one device.
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--chunk", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="time only the headline workload")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (calibrates rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from causal_kernelized_linear_amd import binding, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    binding.lib()
    ev = HipEvents()
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    w = workloads.WORKLOADS["train_bf16"]
    chunk = args.chunk
    r = time_forward(w, chunk, args.steps, args.warmup, ev)
    units = fwd_units(w)
    tok_s = w.B * w.N / (r["ms_per_step"] * 1e-3)
    bpu = fwd_bytes_per_unit(w)
    fpu = fwd_flops_per_unit(w, chunk)
    dom, dom_name = DOMINANT
    dom_name = dom_name.format(c=chunk)
    t_out = r["walk_output_ms_alone"] * 1e-3
    achieved = bpu * units / t_out / 1e9
    step_s = r["ms_per_step"] * 1e-3
    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "train_bf16: causal linear attention forward B=8 H=16 N=4096 D=Dv=64 bf16, "
                               "fp32 state, chunk %d, eps 1e-6" % chunk,
                   "B": w.B, "H": w.H, "N": w.N, "D": w.D, "Dv": w.Dv, "chunk": chunk},
        "roofline": {
            "bound": "hbm",
            "kernel": dom_name,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": stored_traffic(dom_name),
            "algorithmic_bytes_per_launch": bpu * units,
            "kernel_ms": r["walk_output_ms_alone"],
            "kernel_ms_note": "hipEvents before and after the output walk only (third timed pass)",
        },
        "forward": {
            "kernel_ms": r["kernel_ms"],
            "kernel_ms_median": r["kernel_ms_median"],
            "wall_ms_per_step": r["wall_ms_per_step"],
            "ms_per_step_with_launch_events": r["ms_per_step_with_launch_events"],
            "algorithmic_GBps": bpu * units / step_s / 1e9,
            "hbm_frac": bpu * units / step_s / 1e9 / HBM_PEAK_GBS,
            "useful_TFLOPs": fpu * units / step_s / 1e12,
            "mfma_bf16_frac": fpu * units / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "input_sets_rotated": r["input_sets"],
        },
    }

    if not args.no_extra:
        extra_steps = max(5, min(args.steps, 20))
        extra_warm = max(2, min(args.warmup, 200))     # each leg follows host-side set-up
        wg = workloads.WORKLOADS["gated_bf16"]
        rg = time_forward(wg, 128, extra_steps, extra_warm, ev)
        ug = fwd_units(wg)
        sg = rg["ms_per_step"] * 1e-3
        line["gated"] = {
            "workload": "gated_bf16: B=4 H=16 N=8192 D=Dv=64 bf16, scalar gate, chunk 128",
            "tokens_per_s": wg.B * wg.N / sg, "ms_per_step": rg["ms_per_step"], "kernel_ms": rg["kernel_ms"],
            "algorithmic_GBps": fwd_bytes_per_unit(wg) * ug / sg / 1e9,
            "hbm_frac": fwd_bytes_per_unit(wg) * ug / sg / 1e9 / HBM_PEAK_GBS,
            "useful_TFLOPs": fwd_flops_per_unit(wg, 128) * ug / sg / 1e12,
            "mfma_bf16_frac": fwd_flops_per_unit(wg, 128) * ug / sg / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        }
        wd = workloads.WORKLOADS["decode_bf16"]
        rd = time_decode(wd, extra_steps, extra_warm, ev)
        sd = rd["ms_per_step"] * 1e-3
        line["decode"] = {
            "workload": "decode_bf16: B=256 H=32 D=Dv=128, fp32 state, one token",
            "GBps": decode_bytes(wd) / sd / 1e9, "hbm_frac": decode_bytes(wd) / sd / 1e9 / HBM_PEAK_GBS,
            "tokens_per_s": wd.B / sd, "ms_per_step": rd["ms_per_step"], "ms_median": rd["ms_median"],
            "bytes_per_step": decode_bytes(wd),
        }
        rn = time_forward(wg, 128, extra_steps, extra_warm, ev, normalize=False)
        sn = rn["ms_per_step"] * 1e-3
        line["gated_numerator"] = {
            "workload": "gated_bf16 in the normaliser-free output mode (o = phi(q)^T S)",
            "tokens_per_s": wg.B * wg.N / sn, "ms_per_step": rn["ms_per_step"], "kernel_ms": rn["kernel_ms"],
            "algorithmic_GBps": fwd_bytes_per_unit(wg) * ug / sn / 1e9,
            "hbm_frac": fwd_bytes_per_unit(wg) * ug / sn / 1e9 / HBM_PEAK_GBS,
        }
        wdg = workloads.WORKLOADS["decode_gated_bf16"]
        for key, norm in (("decode_gated", True), ("decode_gated_numerator", False)):
            rdg = time_decode(wdg, extra_steps, extra_warm, ev, normalize=norm)
            sdg = rdg["ms_per_step"] * 1e-3
            nbytes = decode_bytes(wdg, with_z=norm)
            line[key] = {
                "workload": "decode_gated_bf16: B=256 H=32 D=Dv=128, fp32 state, one token, gate per head"
                            + ("" if norm else "; normaliser-free, no z"),
                "GBps": nbytes / sdg / 1e9, "hbm_frac": nbytes / sdg / 1e9 / HBM_PEAK_GBS,
                "tokens_per_s": wdg.B / sdg, "ms_per_step": rdg["ms_per_step"], "ms_median": rdg["ms_median"],
                "bytes_per_step": nbytes,
            }
        for key, wname in (("backward", "train_bf16"), ("backward_gated", "gated_bf16")):
            wb = workloads.WORKLOADS[wname]
            rb = time_backward(wb, extra_steps, extra_warm, ev)
            sb = rb["ms_per_step"] * 1e-3
            ub = fwd_units(wb)
            line[key] = {
                "workload": f"{wname} backward: dq, dk, dv" + (", dg" if wb.kind == "gated" else "") +
                            f" for sum(dout * o), chunk {BWD_CHUNK}",
                "tokens_per_s": wb.B * wb.N / sb, "ms_per_step": rb["ms_per_step"],
                "algorithmic_GBps": bwd_bytes_per_unit(wb) * ub / sb / 1e9,
                "hbm_frac": bwd_bytes_per_unit(wb) * ub / sb / 1e9 / HBM_PEAK_GBS,
                "useful_TFLOPs": bwd_flops_per_unit(wb) * ub / sb / 1e12,
                "mfma_bf16_frac": bwd_flops_per_unit(wb) * ub / sb / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            }
        wvd = workloads.WORKLOADS["vdecay_bf16"]
        rvd = time_vdecay(wvd, extra_steps, extra_warm, ev)
        svd = rvd["ms_per_step"] * 1e-3
        uvd = fwd_units(wvd)
        line["vdecay"] = {
            "workload": "vdecay_bf16: B=4 H=16 N=8192 D=Dv=64 bf16, per-dimension decay a [B,H,N,D] fp32, chunk 64",
            "tokens_per_s": wvd.B * wvd.N / svd, "ms_per_step": rvd["ms_per_step"],
            "algorithmic_GBps": vd_bytes_per_unit(wvd) * uvd / svd / 1e9,
            "hbm_frac": vd_bytes_per_unit(wvd) * uvd / svd / 1e9 / HBM_PEAK_GBS,
        }
        wdv = workloads.WORKLOADS["decode_vdecay_bf16"]
        rdv = time_decode(wdv, extra_steps, extra_warm, ev)
        sdv = rdv["ms_per_step"] * 1e-3
        line["decode_vdecay"] = {
            "workload": "decode_vdecay_bf16: B=256 H=32 D=Dv=128, fp32 state, one token, decay per dimension",
            "GBps": decode_bytes(wdv) / sdv / 1e9, "hbm_frac": decode_bytes(wdv) / sdv / 1e9 / HBM_PEAK_GBS,
            "tokens_per_s": wdv.B / sdv, "ms_per_step": rdv["ms_per_step"], "bytes_per_step": decode_bytes(wdv),
        }
        for key, wname, feat in (("features_relu", "train_bf16", "relu"), ("features_favor", "favor_bf16", "favor")):
            wf = workloads.WORKLOADS[wname]
            rf = time_features(wf, feat, extra_steps, extra_warm, ev)
            sf = rf["ms_per_step"] * 1e-3
            uf = fwd_units(wf)
            line[key] = {
                "workload": f"{wname} forward under " + ("relu(x) + 0.05" if feat == "relu" else
                                                         "FAVOR+ with 64 random features per head") + ", chunk 128",
                "tokens_per_s": wf.B * wf.N / sf, "ms_per_step": rf["ms_per_step"],
                "algorithmic_GBps": fwd_bytes_per_unit(wf) * uf / sf / 1e9,
                "hbm_frac": fwd_bytes_per_unit(wf) * uf / sf / 1e9 / HBM_PEAK_GBS,
            }
        wl = workloads.WORKLOADS["longctx_bf16"]
        sweep = {}
        for c in wl.chunks:
            try:
                rl = time_forward(wl, c, max(3, extra_steps // 2), extra_warm, ev, rotate_bytes=2.5e9)
            except RuntimeError as e:
                sweep[str(c)] = {"status": str(e)}
                continue
            ul = fwd_units(wl)
            sl = rl["ms_per_step"] * 1e-3
            sweep[str(c)] = {
                "tokens_per_s": wl.B * wl.N / sl, "ms_per_step": rl["ms_per_step"], "kernel_ms": rl["kernel_ms"],
                "algorithmic_GBps": fwd_bytes_per_unit(wl) * ul / sl / 1e9,
                "hbm_frac": fwd_bytes_per_unit(wl) * ul / sl / 1e9 / HBM_PEAK_GBS,
                "useful_TFLOPs": fwd_flops_per_unit(wl, c) * ul / sl / 1e12,
                "mfma_bf16_frac": fwd_flops_per_unit(wl, c) * ul / sl / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            }
        line["longctx_chunk_sweep"] = {"workload": "longctx_bf16: B=1 H=32 N=65536 D=Dv=128 bf16", **sweep}

    if not args.no_cpu_baseline:
        cb = cpu_baseline(w)
        line["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
    ev.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
