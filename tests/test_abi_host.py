"""Host-side checks of the C ABI (no kernel is launched; runs without a GPU).

The library must load, export every entry point declared in include/linattn.h,
and reject bad arguments with the documented status codes before touching any
device memory.  The pointer values used here are fake but aligned and disjoint.
Every test that passes them runs only where no GPU is visible (``fake_ptrs``):
a call that passed validation would otherwise launch kernels on addresses that do
not exist.  Calls are built to fail validation anyway; the ones that pass it (to
reach the device check) are in ``test_no_device_is_reported_not_crashed``.
"""
import os
import re
import subprocess

import pytest
import torch

from causal_kernelized_linear_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4

# fake, 16-byte aligned, disjoint device addresses (never dereferenced)
Q, K, V, O, G, S0, Z0, SO, ZO, WS = (0x10_0000_0000 * (i + 1) for i in range(10))

# counting devices does not initialise the GPU runtime
fake_ptrs = pytest.mark.skipif(torch.cuda.device_count() > 0,
                               reason="fake device pointers are passed only where no GPU is visible")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(linattn_[a-z_0-9]+)\s*\(", text))
                  - {"linattn_status_t", "linattn_dtype_t", "linattn_output_t"})


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert set(syms) == set(binding.EXPORTS), syms
    lib = binding.lib()
    for s in syms:
        assert getattr(lib, s) is not None
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    for s in syms:
        assert re.search(rf"\bT {s}\b", out), s


def test_status_strings():
    for code in range(6):
        assert isinstance(binding.linattn_status_string(code), str)
    assert "scratch" in binding.linattn_status_string(5)
    assert binding.linattn_status_string(0) == "ok"
    assert binding.linattn_status_string(99) == "unknown status"


def test_workspace_size():
    ws = binding.linattn_fwd_workspace_size
    assert ws(0, 1, 128, 64, 64, 128) == 0
    assert ws(1, 1, 0, 64, 64, 128) == 0
    assert ws(1, 1, 128, 64, 64, -1) == 0
    a = ws(8, 16, 4096, 64, 64, 128)
    assert a > 0 and a % 256 == 0
    # at least one fp32 state per head, at most one per chunk per head
    assert 8 * 16 * 64 * 64 * 4 <= a <= 8 * 16 * 32 * (64 * 64 + 64 + 1) * 4 + 3 * 256


def fwd(q=Q, k=K, v=V, o=O, s0=0, z0=0, so=0, zo=0, B=1, H=2, N=256, D=64, Dv=64, chunk=128, dt=1, eps=1e-6,
        ws=WS, wsb=1 << 30, gated=False, g=G, out=None):
    if out is not None:
        return binding.linattn_fwd_ex(q, k, v, g if gated else 0, o, s0, z0, so, zo, B, H, N, D, Dv, chunk, dt, eps,
                                      out, ws, wsb, 0)
    if gated:
        return binding.linattn_fwd_gated(q, k, v, g, o, s0, z0, so, zo, B, H, N, D, Dv, chunk, dt, eps, ws, wsb, 0)
    return binding.linattn_fwd_chunked(q, k, v, o, s0, z0, so, zo, B, H, N, D, Dv, chunk, dt, eps, ws, wsb, 0)


@fake_ptrs
@pytest.mark.parametrize("gated", [False, True])
def test_fwd_rejects_bad_arguments(gated):
    assert fwd(B=-1, gated=gated) == INVALID
    assert fwd(D=0, gated=gated) == INVALID
    assert fwd(chunk=0, gated=gated) == INVALID
    assert fwd(eps=0.0, gated=gated) == INVALID
    assert fwd(eps=-1e-6, gated=gated) == INVALID
    assert fwd(eps=float("nan"), gated=gated) == INVALID
    assert fwd(dt=7, gated=gated) == INVALID
    assert fwd(q=0, gated=gated) == INVALID
    assert fwd(o=0, gated=gated) == INVALID
    assert fwd(v=V + 8, gated=gated) == INVALID                 # misaligned
    assert fwd(o=Q + 64, gated=gated) == INVALID                # o overlaps q
    assert fwd(s0=O + 64, gated=gated) == INVALID               # o overlaps s0
    assert fwd(z0=O + 64, gated=gated) == INVALID               # o overlaps z0
    assert fwd(so=O + 64, gated=gated) == INVALID               # s_out overlaps o
    assert fwd(zo=O + 64, gated=gated) == INVALID               # z_out overlaps o
    assert fwd(so=Q + 64, gated=gated) == INVALID               # s_out overlaps q
    assert fwd(zo=K, gated=gated) == INVALID                    # z_out overlaps k
    assert fwd(so=V + 16, gated=gated) == INVALID               # s_out overlaps v
    assert fwd(so=SO, zo=SO + 64, gated=gated) == INVALID       # s_out overlaps z_out
    if gated:
        assert fwd(zo=G, gated=gated) == INVALID                # z_out overlaps g
    assert fwd(D=96, gated=gated) == UNSUPPORTED
    assert fwd(Dv=32, gated=gated) == UNSUPPORTED
    assert fwd(chunk=100, gated=gated) == UNSUPPORTED
    assert fwd(chunk=16, gated=gated) == UNSUPPORTED
    assert fwd(chunk=512, gated=gated) == UNSUPPORTED
    # 256 tokens at D = 128 pass the support checks (the value columns in two parts at
    # Dv = 128) and stop at the device check, with no GPU here
    assert fwd(D=128, Dv=128, chunk=256, gated=gated) == HIP
    assert fwd(D=128, Dv=64, chunk=256, gated=gated) == HIP
    assert fwd(dt=0, D=128, Dv=128, chunk=128, gated=gated) == UNSUPPORTED
    assert fwd(dt=0, D=128, Dv=64, chunk=128, gated=gated) == UNSUPPORTED
    assert fwd(dt=0, D=64, Dv=64, chunk=256, gated=gated) == UNSUPPORTED
    assert fwd(ws=0, gated=gated) == WORKSPACE
    assert fwd(wsb=16, gated=gated) == WORKSPACE
    assert fwd(ws=WS + 4, gated=gated) == WORKSPACE
    assert fwd(ws=Q, gated=gated) == WORKSPACE                  # workspace overlaps q
    # empty problems succeed without touching anything
    assert fwd(B=0, q=0, k=0, v=0, o=0, ws=0, wsb=0, gated=gated) == OK
    assert fwd(N=0, q=0, k=0, v=0, o=0, ws=0, wsb=0, gated=gated) == OK


def test_profile_hook_arguments():
    assert binding.linattn_set_profile_events(0, 0, 0, 0) == OK
    # any subset of handles may be given; disarm again before anything could record them
    assert binding.linattn_set_profile_events(16, 0, 0, 0) == OK
    assert binding.linattn_set_profile_events(0, 0, 0, 0) == OK


@fake_ptrs
def test_gated_requires_gate():
    assert fwd(gated=True, g=0) == INVALID


@fake_ptrs
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("out", [0, 1])
def test_fwd_ex_checks_like_the_fixed_forwards(gated, out):
    assert fwd(gated=gated, out=out, B=-1) == INVALID
    assert fwd(gated=gated, out=out, eps=0.0) == INVALID
    assert fwd(gated=gated, out=out, o=Q + 64) == INVALID
    if gated:
        assert fwd(gated=gated, out=out, g=O + 32) == INVALID          # g overlaps o (ungated, g is not read)
    assert fwd(gated=gated, out=out, D=96) == UNSUPPORTED
    assert fwd(gated=gated, out=out, ws=0) == WORKSPACE
    assert fwd(gated=gated, out=out, B=0, q=0, k=0, v=0, o=0, ws=0, wsb=0) == OK


def fwd_noalloc(q=Q, k=K, v=V, g=0, o=O, s0=0, z0=0, so=0, zo=0, B=1, H=2, N=256, D=64, Dv=64, chunk=128, dt=1,
                eps=1e-6, out=0):
    return binding.linattn_fwd_ex_noalloc(q, k, v, g, o, s0, z0, so, zo, B, H, N, D, Dv, chunk, dt, eps, out, 0)


@fake_ptrs
def test_fwd_noalloc_checks_like_fwd_ex():
    assert fwd_noalloc(B=-1) == INVALID
    assert fwd_noalloc(eps=0.0) == INVALID
    assert fwd_noalloc(out=2) == INVALID
    assert fwd_noalloc(o=Q + 64) == INVALID
    assert fwd_noalloc(g=O + 32) == INVALID                    # g overlaps o
    assert fwd_noalloc(so=O) == INVALID                        # s_out overlaps o
    assert fwd_noalloc(D=96) == UNSUPPORTED
    assert fwd_noalloc(dt=0, D=128, Dv=128, chunk=128) == UNSUPPORTED
    assert fwd_noalloc(B=0, q=0, k=0, v=0, o=0) == OK


@fake_ptrs
def test_fwd_noalloc_rejects_shapes_beyond_its_scratch():
    # one state slot of 64 KiB per head: 1024 heads need 64 MiB, beyond the fixed 32 MiB
    assert binding.linattn_fwd_workspace_size(1024, 1, 64, 128, 128, 64) > binding.NOALLOC_SCRATCH_BYTES
    assert fwd_noalloc(B=1024, H=1, N=64, D=128, Dv=128, chunk=64) == 5
    # the long-context shape fits at every chunk
    for chunk in (64, 128, 256):
        assert binding.linattn_fwd_workspace_size(1, 32, 65536, 128, 128, chunk) <= binding.NOALLOC_SCRATCH_BYTES


@fake_ptrs
def test_fwd_ex_rejects_unknown_output_mode():
    assert fwd(out=2) == INVALID
    assert fwd(out=-1) == INVALID
    assert fwd(out=2, gated=True) == INVALID


def decode(q=Q, k=K, v=V, S=S0, z=Z0, o=O, B=4, H=2, D=128, Dv=128, dt=1, eps=1e-6):
    return binding.linattn_decode_step(q, k, v, S, z, o, B, H, D, Dv, dt, eps, 0)


def decode_ex(q=Q, k=K, v=V, g=G, S=S0, z=Z0, o=O, B=4, H=2, D=128, Dv=128, dt=1, eps=1e-6, out=0):
    return binding.linattn_decode_step_ex(q, k, v, g, S, z, o, B, H, D, Dv, dt, eps, out, 0)


@fake_ptrs
def test_decode_ex_rejects_bad_arguments():
    assert decode_ex(out=2) == INVALID
    assert decode_ex(z=0, out=0) == INVALID                     # the normalised output needs z
    assert decode_ex(g=G + 4) == INVALID                        # misaligned gate
    assert decode_ex(g=S0 + 16) == INVALID                      # gate overlaps S
    assert decode_ex(g=O) == INVALID                            # gate overlaps o
    assert decode_ex(S=0) == INVALID
    assert decode_ex(D=96) == UNSUPPORTED
    assert decode_ex(B=0, q=0) == OK


@fake_ptrs
def test_decode_rejects_bad_arguments():
    assert decode(B=-1) == INVALID
    assert decode(S=0) == INVALID
    assert decode(eps=0.0) == INVALID
    assert decode(dt=3) == INVALID
    assert decode(z=Z0 + 4) == INVALID
    assert decode(o=S0) == INVALID                              # o overlaps S
    assert decode(z=S0 + 16) == INVALID                         # z overlaps S
    assert decode(D=96) == UNSUPPORTED
    assert decode(B=0, q=0) == OK


DO, DQ, DK, DV, DG = (0x10_0000_0000 * (i + 11) for i in range(5))


def bwd(q=Q, k=K, v=V, g=G, do=DO, dq=DQ, dk=DK, dv=DV, dg=DG, B=2, H=2, N=256, D=64, Dv=64, dt=1, eps=1e-6, out=0,
        run=0, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = binding.linattn_bwd_workspace_size(B, H, N, D, Dv, dt)
    return binding.linattn_bwd(q, k, v, g, do, S0, Z0, dq, dk, dv, dg, 0, 0, B, H, N, D, Dv, dt, eps, out, run, WS,
                               ws_bytes, 0)


@fake_ptrs
def test_bwd_rejects_bad_arguments():
    assert bwd(run=-1) == INVALID
    assert bwd(eps=0.0) == INVALID
    assert bwd(out=2) == INVALID
    assert bwd(dq=Q) == INVALID                                 # dq overlaps q
    assert bwd(dg=DQ + 16) == INVALID                           # dg overlaps dq
    assert bwd(dk=DK + 4) == INVALID                            # misaligned
    assert bwd(D=96) == UNSUPPORTED
    assert bwd(ws_bytes=binding.linattn_bwd_workspace_size(2, 2, 256, 64, 64, 1) - 1) == WORKSPACE
    assert bwd(B=0, q=0) == OK


def test_bwd_workspace_size():
    ws = binding.linattn_bwd_workspace_size
    assert ws(0, 1, 128, 64, 64, 1) == 0
    a = ws(8, 16, 4096, 64, 64, 1)
    # a state slot per chunk and per head (an upper bound for any run length), twice
    assert a % 256 == 0 and a >= 2 * 8 * 16 * 64 * 64 * 64 * 4


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful where no GPU is present")
def test_no_device_is_reported_not_crashed():
    assert fwd() == HIP
    assert fwd(out=1, gated=True) == HIP
    assert fwd_noalloc() == HIP
    assert decode() == HIP
    assert decode_ex(g=0, z=0, out=1) == HIP                    # valid: numerator mode needs no z
    assert bwd(run=3) == HIP
