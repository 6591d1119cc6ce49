"""Benchmark of the causal kernelized linear attention hot path on one MI355X.

One step = one chunked forward (phi, the per-segment state totals, the prefix that
carries the state across segments, the masked intra-chunk products, the
carried-state term and the divide) over the long-context workload B=1, H=32,
N=65536, D=Dv=128, bf16 inputs 0.5 N(0,1), fp32 state, chunk 64 (--chunk), with the
inputs already resident in HBM.  Input sets are rotated so no step starts with its
inputs warm in the 256 MB Infinity Cache.  The headline is timed last, after the other
legs have brought the device to its steady clocks.  Timed in the same run and reported
in extra fields: the chunk sweep 64/128/256 of that workload, the training-shaped
forward (B=8, H=16, N=4096, D=Dv=64, chunk 128), the fp32 parity workload (B=1, H=2,
N=512, D=Dv=64, chunk 64), the scalar-gated forward (B=4, H=16, N=8192, D=Dv=64, chunk
128), the decode step (B=256, H=32, D=Dv=128, fp32 state), its gated form, the
normaliser-free output mode, the backward of the training-shaped and gated forwards,
the per-dimension decay (forward and decode) and the ReLU and FAVOR+ feature maps.

Prints ONE JSON line.  ms_per_step and value come from a timed pass bracketed by
two hipEvents only.  Per-kernel durations come from a second timed pass of the same
length with hipEvents recorded on the launch stream around each kernel (the
library's measurement hook); those markers sit between dependent launches and add a
few microseconds each, so they never enter the headline.  A third pass brackets
only the output walk (one event before it, one after); the roofline object prices
that kernel time against MI355X's 8 TB/s.  Its traffic figure comes from the
committed rocprofv3 counter summary and is null once the kernel sources have
changed.  The oracle baseline (cpu_baseline) runs before the GPU is touched, on a
bounded sample of the headline workload, pooled over the host cores.

--only selects legs (for profiling runs); --no-extra times the headline alone.
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
KERNEL_SOURCES = os.path.join(ROOT, "causal_kernelized_linear_amd", "csrc")
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


def device_input_sets(w, rotate_bytes=600e6):
    """Workload w's inputs on the GPU: enough copies to rotate through more than
    `rotate_bytes`, so no step starts with its inputs warm in the 256 MB Infinity Cache."""
    import torch
    from causal_kernelized_linear_amd import workloads

    dev = torch.device("cuda:0")
    base = workloads.make_inputs(w)
    sets = [{n: t.to(dev) for n, t in base.items()}]
    per_set = sum(t.numel() * t.element_size() for t in sets[0].values())
    nsets = max(2, min(6, int(rotate_bytes // max(per_set, 1)) + 1))
    for _ in range(nsets - 1):
        sets.append({n: t.clone() for n, t in sets[0].items()})
    return sets


def warm_up(call, warmup, ev, stream, settle_ms=0.0):
    """Untimed warmup: `warmup` calls, then (settle_ms > 0) more, until the device has run
    at least settle_ms of them back to back.  Its clocks reach their steady state only
    after tens of milliseconds of sustained work, and the host-side set-up before each
    leg lets them fall; settle_ms is used for the legs beside the headline, whose own
    warmup is exactly --warmup steps."""
    import torch

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    if settle_ms <= 0.0:
        return
    done_ms, n = 0.0, warmup
    a, b = ev.create(2)
    batch = 8
    while done_ms < settle_ms and n < warmup + 100000:
        ev.record(a, stream)
        for j in range(batch):
            call(n + j)
        ev.record(b, stream)
        torch.cuda.synchronize()
        took = ev.ms(a, b)
        done_ms += took
        n += batch
        per = max(took / batch, 1e-3)
        batch = max(1, min(4096, int((settle_ms - done_ms) / per) + 1))


def time_forward(w, chunk, steps, warmup, ev, rotate_bytes=600e6, normalize=True, sets=None, settle_ms=0.0):
    """Time `steps` forwards of workload w; returns a dict of timings (ms).

    Two timed passes of `steps` forwards each.  The first is bracketed by two hipEvents
    only: it gives ms_per_step.  The second also records the library's four per-launch
    events on every forward (the measurement hook), which gives the per-kernel times;
    those event records sit between dependent launches and lengthen the step, so the
    headline figure never comes from the second pass.  `sets`: input sets already on the
    device (device_input_sets), else drawn here."""
    import torch
    from causal_kernelized_linear_amd import binding

    dev = torch.device("cuda:0")
    if sets is None:
        sets = device_input_sets(w, rotate_bytes)
    nsets = len(sets)
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

    warm_up(call, warmup, ev, stream, settle_ms)
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


def time_decode(w, steps, warmup, ev, normalize=True, settle_ms=0.0):
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

    warm_up(call, warmup, ev, stream, settle_ms)
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


def time_backward(w, steps, warmup, ev, settle_ms=0.0):
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

    warm_up(call, warmup, ev, stream, settle_ms)
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


def time_vdecay(w, steps, warmup, ev, settle_ms=0.0):
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

    warm_up(call, warmup, ev, stream, settle_ms)
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


def time_features(w, feature, steps, warmup, ev, M=64, settle_ms=0.0):
    """Per-step time of linattn_fwd_features on workload w (two input sets rotated)."""
    import torch
    from causal_kernelized_linear_amd import binding, workloads

    dev = torch.device("cuda:0")
    base = workloads.make_inputs(w)
    sets = [{n: t.to(dev) for n, t in base.items()}]
    sets.append({n: t.clone() for n, t in sets[0].items()})
    W = workloads.favor_projection(w.seed, w.H, M, w.D, orthogonal=True).to(dev) if feature == "favor" else None
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

    warm_up(call, warmup, ev, stream, settle_ms)
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


# the files the dominant kernel (the bf16 output walk) and its launch plan are built from
DOMINANT_SOURCES = ("chunk_walk.hpp", "device_common.hpp", "fwd_bf16.hip", "fwd_dispatch.hpp", "launch.hpp",
                    "api.hip")


def source_digest():
    """sha256 over the dominant kernel's sources, to tell whether stored counters still apply."""
    import hashlib
    h = hashlib.sha256()
    for name in DOMINANT_SOURCES:
        with open(os.path.join(KERNEL_SOURCES, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def output_walk_name(w, chunk):
    """The output walk kernel of forward workload w at this chunk, as the counter summaries
    name it: the split 8-wave walk at D = Dv = 128 and chunk 64 and at D = Dv = 64 and
    chunk 128 (ungated bf16), the walk over two column parts of 64 where the full tiles
    exceed the LDS (chunk 256 at D = Dv = 128)."""
    if w.dtype == "bf16" and w.kind == "fwd":
        if w.D == 128 and w.Dv == 128 and chunk == 64:
            return "walk_split_kernel<bf16,128,128,64>"
        if w.D == 64 and w.Dv == 64 and chunk == 128:
            return "walk_split_kernel<bf16,64,64,128>"
        if w.D == 128 and w.Dv == 128 and chunk == 256:
            return "walk_kernel<bf16,128,64,256,ungated,output,parts2>"
    return f"walk_kernel<{w.dtype},{w.D},{w.Dv},{chunk},{'gated' if w.kind == 'gated' else 'ungated'},output>"


def counters_path(workload, chunk):
    return os.path.join(ROOT, "profiles", f"counters_walk_output_{workload}_c{chunk}.json")


def stored_traffic(kernel_name, workload, chunk):
    """HBM bytes per launch of the output walk from the committed rocprofv3 counter summary
    of this workload and chunk, scaled by its copy-kernel calibration; None when there is
    none or the kernel sources changed since the counters were taken."""
    try:
        with open(counters_path(workload, chunk)) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_sha256") != source_digest() or c.get("kernel") != kernel_name:
        return None
    return 1024.0 * (c["fetch_kib"] * c["fetch_factor"] + c["write_kib"] * c["write_factor"])


# ---------------------------------------------------------------- oracle baseline ----

_CPU_INPUTS = {}


def _one_thread():
    """Pool initializer: every worker keeps to one thread."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _oracle_heads(heads):
    """The oracle over some (b, h) heads of the inputs the parent drew before forking."""
    import numpy as np
    import oracle
    q, k, v = (_CPU_INPUTS[n] for n in ("q", "k", "v"))
    pick = lambda a: np.stack([a[b, h] for b, h in heads])[None]
    o, _, _ = oracle.causal_linear_attention(pick(q), pick(k), pick(v))
    return float(o[0, :, -1].sum())


def cpu_baseline(w, ntok):
    """The fp64 oracle, as it stands, on a bounded sample of workload w: every head, the
    first `ntok` tokens (drawn with the workload's seed at that length).  The heads are
    dealt to a fork pool of one worker per host core this process may run on (at most 16,
    the host share of one GPU), each kept to one thread.  Returns tokens/s of the sample
    (B * ntok tokens over the wall time, all heads) and the core count used."""
    import multiprocessing as mp
    from causal_kernelized_linear_amd import workloads

    inp = workloads.make_inputs(w, N=ntok)
    for n in ("q", "k", "v"):
        _CPU_INPUTS[n] = workloads.to_f64(inp[n])
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    cores = max(1, min(len(os.sched_getaffinity(0)), 16, len(heads)))
    groups = [heads[i::cores] for i in range(cores)]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores, initializer=_one_thread) as pool:
        t = time.perf_counter()
        pool.map(_oracle_heads, groups, chunksize=1)
        dt = time.perf_counter() - t
    _CPU_INPUTS.clear()
    return {
        "value": w.B * ntok / dt,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{w.name}: fp64 NumPy recurrence over all {w.B}x{w.H} heads and the first {ntok} of "
                  f"{w.N} tokens, the heads dealt to {cores} single-threaded worker processes; "
                  f"{dt:.2f} s wall (host: {os.cpu_count()} cpus, affinity {len(os.sched_getaffinity(0))})",
        "seconds": dt,
    }


# ------------------------------------------------------------------------- legs ----

LEGS = ("longctx", "sweep", "train", "fp32", "gated", "gated_numerator", "decode", "decode_gated", "backward",
        "vdecay", "decode_vdecay", "features")


def fwd_leg(w, chunk, r):
    """Rates of one timed forward leg (r from time_forward) against both peaks, and the
    output walk's own HBM rate from its event-bracketed time."""
    units = fwd_units(w)
    bpu, fpu = fwd_bytes_per_unit(w), fwd_flops_per_unit(w, chunk)
    step_s = r["ms_per_step"] * 1e-3
    out_s = r["walk_output_ms_alone"] * 1e-3
    return {
        "tokens_per_s": w.B * w.N / step_s, "ms_per_step": r["ms_per_step"],
        "kernel_ms": r["kernel_ms"], "kernel_ms_median": r["kernel_ms_median"],
        "walk_output_ms_alone": r["walk_output_ms_alone"],
        "walk_output_hbm_frac": bpu * units / out_s / 1e9 / HBM_PEAK_GBS,
        "algorithmic_GBps": bpu * units / step_s / 1e9,
        "hbm_frac": bpu * units / step_s / 1e9 / HBM_PEAK_GBS,
        "useful_TFLOPs": fpu * units / step_s / 1e12,
        "mfma_bf16_frac": fpu * units / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "input_sets_rotated": r["input_sets"],
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The device needs tens of milliseconds of sustained work to reach its steady clocks
    # (train_bf16: 85-87 us per step after 10 warmup steps, 71-72 us after 1000).
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--chunk", type=int, default=64, help="chunk of the long-context headline")
    ap.add_argument("--only", default="", help="comma-separated legs to run (default: all): " + ", ".join(LEGS))
    ap.add_argument("--cpu-tokens", type=int, default=16384,
                    help="tokens per head of the oracle's bounded sample of the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="time only the headline workload")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (calibrates rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    legs = [x for x in args.only.split(",") if x] or (["longctx"] if args.no_extra else list(LEGS))
    for x in legs:
        if x not in LEGS:
            print(f"unknown leg {x!r}; legs: {', '.join(LEGS)}", file=sys.stderr)
            sys.exit(2)

    from causal_kernelized_linear_amd import workloads
    wl = workloads.WORKLOADS["longctx_bf16"]
    # the oracle baseline runs first, in worker processes forked before this process
    # touches the GPU
    cb = None
    if "longctx" in legs and not args.no_cpu_baseline:
        cb = cpu_baseline(wl, min(args.cpu_tokens, wl.N))

    import torch
    from causal_kernelized_linear_amd import binding

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

    extra_steps = max(5, min(args.steps, 20))
    # each extra leg follows host-side set-up (its inputs drawn on the CPU, seconds during
    # which the device idles and its clocks fall): its warmup runs at least 100 steps and
    # 50 ms of them back to back, whatever --warmup the headline is given
    extra_warm = 100
    extra_settle_ms = 50.0
    chunk = args.chunk
    # the headline's inputs go to the device first, so that its warmup follows the other
    # legs' GPU work directly, with no host-side set-up in between
    head_sets = device_input_sets(wl, rotate_bytes=2.5e9) if ("longctx" in legs or "sweep" in legs) else None
    line = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}

    if "train" in legs:
        wt = workloads.WORKLOADS["train_bf16"]
        rt = time_forward(wt, 128, args.steps, extra_warm, ev, settle_ms=extra_settle_ms)
        line["train"] = {"workload": "train_bf16: B=8 H=16 N=4096 D=Dv=64 bf16, fp32 state, chunk 128",
                         **fwd_leg(wt, 128, rt),
                         "walk_output_traffic": stored_traffic(output_walk_name(wt, 128), wt.name, 128)}

    if "fp32" in legs:
        wf = workloads.WORKLOADS["fp32_small"]
        rf = time_forward(wf, 64, extra_steps, extra_warm, ev, settle_ms=extra_settle_ms)
        line["fp32_small"] = {"workload": "fp32_small: B=1 H=2 N=512 D=Dv=64 fp32, chunk 64 (launch-bound)",
                              "tokens_per_s": wf.B * wf.N / (rf["ms_per_step"] * 1e-3),
                              "ms_per_step": rf["ms_per_step"], "kernel_ms": rf["kernel_ms"]}

    wg = workloads.WORKLOADS["gated_bf16"]
    if "gated" in legs:
        rg = time_forward(wg, 128, extra_steps, extra_warm, ev, settle_ms=extra_settle_ms)
        line["gated"] = {"workload": "gated_bf16: B=4 H=16 N=8192 D=Dv=64 bf16, scalar gate, chunk 128",
                         **fwd_leg(wg, 128, rg)}

    if "decode" in legs:
        wd = workloads.WORKLOADS["decode_bf16"]
        rd = time_decode(wd, extra_steps, extra_warm, ev, settle_ms=extra_settle_ms)
        sd = rd["ms_per_step"] * 1e-3
        line["decode"] = {
            "workload": "decode_bf16: B=256 H=32 D=Dv=128, fp32 state, one token",
            "GBps": decode_bytes(wd) / sd / 1e9, "hbm_frac": decode_bytes(wd) / sd / 1e9 / HBM_PEAK_GBS,
            "tokens_per_s": wd.B / sd, "ms_per_step": rd["ms_per_step"], "ms_median": rd["ms_median"],
            "bytes_per_step": decode_bytes(wd),
        }

    if "gated_numerator" in legs:
        rn = time_forward(wg, 128, extra_steps, extra_warm, ev, normalize=False, settle_ms=extra_settle_ms)
        sn = rn["ms_per_step"] * 1e-3
        ug = fwd_units(wg)
        line["gated_numerator"] = {
            "workload": "gated_bf16 in the normaliser-free output mode (o = phi(q)^T S)",
            "tokens_per_s": wg.B * wg.N / sn, "ms_per_step": rn["ms_per_step"], "kernel_ms": rn["kernel_ms"],
            "algorithmic_GBps": fwd_bytes_per_unit(wg) * ug / sn / 1e9,
            "hbm_frac": fwd_bytes_per_unit(wg) * ug / sn / 1e9 / HBM_PEAK_GBS,
        }

    if "decode_gated" in legs:
        wdg = workloads.WORKLOADS["decode_gated_bf16"]
        for key, norm in (("decode_gated", True), ("decode_gated_numerator", False)):
            rdg = time_decode(wdg, extra_steps, extra_warm, ev, normalize=norm, settle_ms=extra_settle_ms)
            sdg = rdg["ms_per_step"] * 1e-3
            nbytes = decode_bytes(wdg, with_z=norm)
            line[key] = {
                "workload": "decode_gated_bf16: B=256 H=32 D=Dv=128, fp32 state, one token, gate per head"
                            + ("" if norm else "; normaliser-free, no z"),
                "GBps": nbytes / sdg / 1e9, "hbm_frac": nbytes / sdg / 1e9 / HBM_PEAK_GBS,
                "tokens_per_s": wdg.B / sdg, "ms_per_step": rdg["ms_per_step"], "ms_median": rdg["ms_median"],
                "bytes_per_step": nbytes,
            }

    if "backward" in legs:
        for key, wname in (("backward", "train_bf16"), ("backward_gated", "gated_bf16")):
            wb = workloads.WORKLOADS[wname]
            rb = time_backward(wb, extra_steps, extra_warm, ev, settle_ms=extra_settle_ms)
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

    if "vdecay" in legs:
        wvd = workloads.WORKLOADS["vdecay_bf16"]
        rvd = time_vdecay(wvd, extra_steps, extra_warm, ev, settle_ms=extra_settle_ms)
        svd = rvd["ms_per_step"] * 1e-3
        uvd = fwd_units(wvd)
        line["vdecay"] = {
            "workload": "vdecay_bf16: B=4 H=16 N=8192 D=Dv=64 bf16, per-dimension decay a [B,H,N,D] fp32, chunk 64",
            "tokens_per_s": wvd.B * wvd.N / svd, "ms_per_step": rvd["ms_per_step"],
            "algorithmic_GBps": vd_bytes_per_unit(wvd) * uvd / svd / 1e9,
            "hbm_frac": vd_bytes_per_unit(wvd) * uvd / svd / 1e9 / HBM_PEAK_GBS,
        }

    if "decode_vdecay" in legs:
        wdv = workloads.WORKLOADS["decode_vdecay_bf16"]
        rdv = time_decode(wdv, extra_steps, extra_warm, ev, settle_ms=extra_settle_ms)
        sdv = rdv["ms_per_step"] * 1e-3
        line["decode_vdecay"] = {
            "workload": "decode_vdecay_bf16: B=256 H=32 D=Dv=128, fp32 state, one token, decay per dimension",
            "GBps": decode_bytes(wdv) / sdv / 1e9, "hbm_frac": decode_bytes(wdv) / sdv / 1e9 / HBM_PEAK_GBS,
            "tokens_per_s": wdv.B / sdv, "ms_per_step": rdv["ms_per_step"], "bytes_per_step": decode_bytes(wdv),
        }

    if "features" in legs:
        for key, wname, feat in (("features_relu", "train_bf16", "relu"), ("features_favor", "favor_bf16", "favor")):
            wf = workloads.WORKLOADS[wname]
            rf = time_features(wf, feat, extra_steps, extra_warm, ev, settle_ms=extra_settle_ms)
            sf = rf["ms_per_step"] * 1e-3
            uf = fwd_units(wf)
            line[key] = {
                "workload": f"{wname} forward under " + ("relu(x) + 0.05" if feat == "relu" else
                                                         "FAVOR+ with 64 orthogonal random features per head") +
                            ", chunk 128",
                "tokens_per_s": wf.B * wf.N / sf, "ms_per_step": rf["ms_per_step"],
                "algorithmic_GBps": fwd_bytes_per_unit(wf) * uf / sf / 1e9,
                "hbm_frac": fwd_bytes_per_unit(wf) * uf / sf / 1e9 / HBM_PEAK_GBS,
            }

    # the chunk sweep on the headline's own inputs, chunk 64 last, then the headline: the
    # headline's warmup follows the same kernels with no host-side work in between
    if "sweep" in legs:
        sweep = {}
        for c in sorted(wl.chunks, reverse=True):
            rl = time_forward(wl, c, max(3, extra_steps // 2), extra_warm, ev, rotate_bytes=2.5e9, sets=head_sets,
                              settle_ms=extra_settle_ms)
            sweep[str(c)] = fwd_leg(wl, c, rl)
        line["longctx_chunk_sweep"] = {"workload": "longctx_bf16: B=1 H=32 N=65536 D=Dv=128 bf16",
                                       **{str(c): sweep[str(c)] for c in wl.chunks}}

    # the headline last: the legs above have brought the device to its steady clocks
    if "longctx" in legs:
        r = time_forward(wl, chunk, args.steps, args.warmup, ev, sets=head_sets)
        head_sets = None
        units = fwd_units(wl)
        bpu = fwd_bytes_per_unit(wl)
        dom_name = output_walk_name(wl, chunk)
        achieved = bpu * units / (r["walk_output_ms_alone"] * 1e-3) / 1e9
        line.update({
            "value": wl.B * wl.N / (r["ms_per_step"] * 1e-3),
            "ms_per_step": r["ms_per_step"],
            "config": {"workload": "longctx_bf16: causal linear attention forward B=1 H=32 N=65536 D=Dv=128 bf16 "
                                   "(0.5 N(0,1) inputs), fp32 state, chunk %d, eps 1e-6" % chunk,
                       "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D, "Dv": wl.Dv, "chunk": chunk},
            "roofline": {
                "bound": "hbm",
                "kernel": dom_name,
                "achieved": achieved,
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": stored_traffic(dom_name, wl.name, chunk),
                "algorithmic_bytes_per_launch": bpu * units,
                "kernel_ms": r["walk_output_ms_alone"],
                "kernel_ms_note": "hipEvents on the launch stream before and after the output walk only "
                                  "(third timed pass)",
            },
            "forward": fwd_leg(wl, chunk, r),
        })
        line["forward"]["wall_ms_per_step"] = r["wall_ms_per_step"]
        line["forward"]["ms_per_step_with_launch_events"] = r["ms_per_step_with_launch_events"]

    if cb is not None:
        line["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        line["cpu_baseline"]["gpu_speedup"] = line["value"] / cb["value"]
    ev.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
