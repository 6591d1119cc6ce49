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
