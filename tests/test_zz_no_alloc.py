"""GPU check of linattn_fwd_ex_noalloc, the forward for callers that cannot allocate.

It must give exactly what linattn_fwd_ex gives with a caller-allocated workspace (the
same kernels on the same plan), call after call on the shared fixed scratch: two calls
in a row, the second on a smaller problem than the first, each compared with the
workspace entry point on the same inputs.
"""
import pytest
import torch

from causal_kernelized_linear_amd import binding, workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CALLS = [
    # (seed, B, H, N, D, Dv, dtype, chunk, gated, normalize): the first call needs the
    # larger scratch (64 segments per head, the scanned prefix), the second less
    [(71, 1, 4, 16384, 128, 128, "bf16", 64, False, True), (72, 2, 2, 700, 64, 64, "bf16", 128, True, True)],
    [(73, 2, 16, 4096, 64, 64, "bf16", 128, True, False), (74, 1, 3, 333, 64, 128, "f32", 128, False, True)],
    [(75, 1, 8, 8192, 128, 128, "bf16", 256, False, True), (76, 1, 1, 100, 128, 128, "bf16", 256, False, True)],
]


def _say(msg):
    print(msg, flush=True)


def _run(case, noalloc):
    seed, B, H, N, D, Dv, dt, chunk, gated, normalize = case
    inp = workloads.random_inputs(seed, B, H, N, D, Dv, dtype=dt, gated=gated, g_low=0.9, with_state=True,
                                  state_scale=5.0)
    x = {n: t.to(DEV) for n, t in inp.items()}
    o = torch.empty(B, H, N, Dv, dtype=x["q"].dtype, device=DEV)
    s_out = torch.empty(B, H, D, Dv, dtype=torch.float32, device=DEV)
    z_out = torch.empty(B, H, D, dtype=torch.float32, device=DEV)
    ptrs = [x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["g"].data_ptr() if gated else 0, o.data_ptr(),
            x["s0"].data_ptr(), x["z0"].data_ptr(), s_out.data_ptr(), z_out.data_ptr()]
    dtc = binding.BF16 if dt == "bf16" else binding.F32
    mode = binding.OUT_NORMALIZED if normalize else binding.OUT_NUMERATOR
    stream = torch.cuda.current_stream().cuda_stream
    if noalloc:
        code = binding.linattn_fwd_ex_noalloc(*ptrs, B, H, N, D, Dv, chunk, dtc, 1e-6, mode, stream)
    else:
        ws = torch.empty(binding.linattn_fwd_workspace_size(B, H, N, D, Dv, chunk), dtype=torch.uint8, device=DEV)
        code = binding.linattn_fwd_ex(*ptrs, B, H, N, D, Dv, chunk, dtc, 1e-6, mode, ws.data_ptr(), ws.numel(),
                                      stream)
    assert code == 0, binding.linattn_status_string(code)
    torch.cuda.synchronize()
    return o, s_out, z_out


@pytest.mark.parametrize("calls", CALLS, ids=["large_then_small", "gated_numerator_then_f32", "chunk256"])
def test_noalloc_equals_workspace_entry(calls):
    for case in calls:
        _say(f"noalloc {case}")
        got = _run(case, True)
        ref = _run(case, False)
        for a, b, name in zip(got, ref, ("o", "s_out", "z_out")):
            assert torch.equal(a, b), (case, name, (a.float() - b.float()).abs().max().item())


def test_noalloc_replayed_from_a_graph():
    """The entry point for callers that cannot allocate, captured once into a HIP graph
    (after one eager call has done the library's per-device set-up) and replayed three
    times, with eager calls between the replays that reuse the shared scratch for another
    problem: every replay matches the eager result on the same inputs."""
    case = (81, 2, 4, 3000, 64, 64, "bf16", 128, True, True)
    other = (82, 1, 8, 8192, 128, 128, "bf16", 64, False, True)
    seed, B, H, N, D, Dv, dt, chunk, gated, normalize = case
    inp = workloads.random_inputs(seed, B, H, N, D, Dv, dtype=dt, gated=gated, g_low=0.9, with_state=True,
                                  state_scale=5.0)
    x = {n: t.to(DEV) for n, t in inp.items()}
    o = torch.empty(B, H, N, Dv, dtype=x["q"].dtype, device=DEV)
    s_out = torch.empty(B, H, D, Dv, dtype=torch.float32, device=DEV)
    z_out = torch.empty(B, H, D, dtype=torch.float32, device=DEV)
    ptrs = [x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["g"].data_ptr(), o.data_ptr(),
            x["s0"].data_ptr(), x["z0"].data_ptr(), s_out.data_ptr(), z_out.data_ptr()]

    def call(stream):
        return binding.linattn_fwd_ex_noalloc(*ptrs, B, H, N, D, Dv, chunk, binding.BF16, 1e-6, binding.OUT_NORMALIZED,
                                              stream)

    _say(f"graph: eager call {case}")
    assert call(torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    want = [t.clone() for t in (o, s_out, z_out)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        code = call(torch.cuda.current_stream().cuda_stream)
    assert code == 0, binding.linattn_status_string(code)
    for rep in range(3):
        _say(f"graph: replay {rep} after an eager call on {other}")
        for t in (o, s_out, z_out):
            t.fill_(float("nan"))
        _run(other, True)                       # the shared scratch now holds another problem
        graph.replay()
        torch.cuda.synchronize()
        for a, b, name in zip((o, s_out, z_out), want, ("o", "s_out", "z_out")):
            assert torch.equal(a, b), (rep, name)
