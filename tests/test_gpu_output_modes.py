"""GPU parity of the gated decode step and the normaliser-free output mode.

The normaliser-free mode returns o = phi(q)^T S, retention's output, with no
phi(q)^T z denominator (aicassindra.com page, "RetNet and gated linear
attention"; learn.pranaymahendrakar.com page, "Implementation reality").  The
gated decode step is the recurrent form of the gated forward, one token at a
time.  Expected values come from the oracle with the same flags.
"""
import numpy as np
import pytest
import torch

import oracle
from causal_kernelized_linear_amd import binding, workloads
from parity import TOL, matrix_rel_err, rowwise_rel_err, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


def _dev(t):
    return None if t is None else t.to(DEV)


def fwd_ex(inp, chunk, out_mode, s0=None, z0=None):
    """linattn_fwd_ex through the raw C entry point; returns (o, S_N, z_N)."""
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    g = _dev(inp.get("g"))
    s0, z0 = _dev(s0), _dev(z0)
    B, H, N, D = q.shape
    Dv = v.shape[-1]
    o = torch.empty(B, H, N, Dv, dtype=q.dtype, device=DEV)
    S = torch.empty(B, H, D, Dv, dtype=torch.float32, device=DEV)
    z = torch.empty(B, H, D, dtype=torch.float32, device=DEV)
    nb = binding.linattn_fwd_workspace_size(B, H, N, D, Dv, chunk)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
    p = lambda t: 0 if t is None else t.data_ptr()          # noqa: E731
    dt = binding.BF16 if q.dtype == torch.bfloat16 else binding.F32
    code = binding.linattn_fwd_ex(p(q), p(k), p(v), p(g), p(o), p(s0), p(z0), p(S), p(z), B, H, N, D, Dv, chunk, dt,
                                  1e-6, out_mode, p(ws), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert code == 0, binding.linattn_status_string(code)
    torch.cuda.synchronize()
    return o, S, z


def oracle_run(inp, normalize, s0=None, z0=None, heads=None):
    def pick(t):
        if t is None:
            return None
        a = to64(t)
        return a if heads is None else np.stack([a[b, h] for b, h in heads])[None]
    return oracle.causal_linear_attention(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), g=pick(inp.get("g")),
                                          s0=pick(s0), z0=pick(z0), normalize=normalize)


def sel(t, heads):
    a = to64(t)
    return np.stack([a[b, h] for b, h in heads])[None]


CASES = [
    # (B, H, N, D, Dv, dtype, chunk)
    (1, 2, 512, 64, 64, "f32", 64),
    (1, 1, 97, 64, 128, "f32", 64),
    (2, 1, 200, 128, 128, "f32", 32),
    (2, 2, 640, 64, 64, "bf16", 128),
    (1, 2, 777, 128, 128, "bf16", 128),
    (1, 2, 333, 128, 64, "bf16", 64),
    (2, 1, 515, 64, 128, "bf16", 256),
    (1, 1, 1, 64, 64, "bf16", 128),
    (3, 1, 2049, 64, 64, "bf16", 256),
]


@pytest.mark.parametrize("gated", [False, True], ids=["ungated", "gated"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}D{}Dv{}{}c{}".format(*c))
def test_numerator_mode_against_oracle(case, gated):
    B, H, N, D, Dv, dt, chunk = case
    _say(f"numerator mode {case} gated={gated}")
    inp = workloads.random_inputs(31 + N + D, B, H, N, D, Dv, dtype=dt, gated=gated, g_low=0.8, with_state=True,
                                  state_scale=5.0)
    o, S, z = fwd_ex(inp, chunk, binding.OUT_NUMERATOR, s0=inp["s0"], z0=inp["z0"])
    o_ref, S_ref, z_ref = oracle_run(inp, False, s0=inp["s0"], z0=inp["z0"])
    tol = TOL[dt]
    assert rowwise_rel_err(to64(o), o_ref) <= tol
    assert matrix_rel_err(to64(S), S_ref) <= tol
    assert matrix_rel_err(to64(z), z_ref) <= tol
    # the state walk does not depend on the output mode
    on, Sn, zn = fwd_ex(inp, chunk, binding.OUT_NORMALIZED, s0=inp["s0"], z0=inp["z0"])
    assert torch.equal(S, Sn) and torch.equal(z, zn)


@pytest.mark.parametrize("gated", [False, True], ids=["ungated", "gated"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fwd_ex_normalized_is_the_fixed_forward(dt, gated):
    inp = workloads.random_inputs(8, 2, 2, 700, 64, 64, dtype=dt, gated=gated)
    _say(f"fwd_ex normalised vs fixed entry dt={dt} gated={gated}")
    o, S, z = fwd_ex(inp, 64, binding.OUT_NORMALIZED)
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    if gated:
        o2, S2, z2 = binding.fwd_gated(q, k, v, _dev(inp["g"]), chunk=64, return_state=True)
    else:
        o2, S2, z2 = binding.fwd_chunked(q, k, v, chunk=64, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2) and torch.equal(z, z2)


def test_numerator_constant_gate_closed_form():
    # q = k = 0 gives phi(q).phi(k) = D; with v constant c and a constant gate gamma,
    # o_i = D c (1 - gamma^(i+1)) / (1 - gamma) (retention's fixed decay).
    B, H, N, D, Dv, gamma = 1, 2, 300, 64, 64, 0.95
    c = torch.linspace(-1.0, 1.0, Dv)
    inp = {"q": torch.zeros(B, H, N, D), "k": torch.zeros(B, H, N, D),
           "v": c.expand(B, H, N, Dv).contiguous(), "g": torch.full((B, H, N), gamma)}
    _say("numerator closed form")
    o, _, _ = fwd_ex(inp, 64, binding.OUT_NUMERATOR)
    i = np.arange(N, dtype=np.float64)[:, None]
    want = D * c.double().numpy()[None, :] * (1 - gamma ** (i + 1)) / (1 - gamma)
    assert rowwise_rel_err(to64(o)[0, 0], want) <= TOL["f32"]
    assert rowwise_rel_err(to64(o)[0, 1], want) <= TOL["f32"]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("mode", ["gated", "numerator", "gated_numerator"])
def test_decode_ex_small(mode, dims, dt):
    D, Dv = dims
    B, H = 3, 5
    gen = torch.Generator().manual_seed(D + 3 * Dv + len(mode))
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    q = torch.randn(B, H, D, generator=gen).to(tdt)
    k = torch.randn(B, H, D, generator=gen).to(tdt)
    v = torch.randn(B, H, Dv, generator=gen).to(tdt)
    S = torch.randn(B, H, D, Dv, generator=gen) * 30
    z = torch.randn(B, H, D, generator=gen).abs() * 30
    g = (0.5 + 0.5 * torch.rand(B, H, generator=gen)) if "gated" in mode else None
    normalize = "numerator" not in mode
    _say(f"decode_ex {mode} dims={dims} dt={dt}")
    o_ref, S_ref, z_ref = oracle.decode_step(to64(q), to64(k), to64(v), to64(S), to64(z),
                                             g=None if g is None else to64(g), normalize=normalize)
    Sd, zd = S.to(DEV), z.to(DEV)
    o = binding.decode_step(q.to(DEV), k.to(DEV), v.to(DEV), Sd, zd, g=_dev(g), normalize=normalize)
    torch.cuda.synchronize()
    assert rowwise_rel_err(to64(o), o_ref) <= TOL[dt]
    assert matrix_rel_err(to64(Sd), S_ref) <= 1e-6
    assert matrix_rel_err(to64(zd), z_ref) <= 1e-6
    if not normalize:
        # without a denominator z is optional: the same step with no z gives the same o and S
        Sn = S.to(DEV)
        o2 = binding.decode_step(q.to(DEV), k.to(DEV), v.to(DEV), Sn, None, g=_dev(g), normalize=False)
        torch.cuda.synchronize()
        assert torch.equal(o2, o) and torch.equal(Sn, Sd)


def test_decode_ex_defaults_are_the_fixed_decode():
    B, H, D, Dv = 4, 3, 128, 64
    gen = torch.Generator().manual_seed(5)
    q, k = (torch.randn(B, H, D, generator=gen).to(torch.bfloat16).to(DEV) for _ in range(2))
    v = torch.randn(B, H, Dv, generator=gen).to(torch.bfloat16).to(DEV)
    S = (torch.randn(B, H, D, Dv, generator=gen) * 10).to(DEV)
    z = (torch.randn(B, H, D, generator=gen).abs() * 10).to(DEV)
    S1, z1, S2, z2 = S.clone(), z.clone(), S.clone(), z.clone()
    o1 = binding.decode_step(q, k, v, S1, z1)
    o2 = torch.empty_like(o1)
    st = torch.cuda.current_stream().cuda_stream
    code = binding.linattn_decode_step_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), 0, S2.data_ptr(), z2.data_ptr(),
                                          o2.data_ptr(), B, H, D, Dv, binding.BF16, 1e-6, binding.OUT_NORMALIZED, st)
    assert code == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(z1, z2)


@pytest.mark.parametrize("normalize", [True, False], ids=["normalized", "numerator"])
def test_gated_prefill_then_gated_decode(normalize):
    B, H, N, D, Dv = 1, 2, 257, 128, 128
    inp = workloads.random_inputs(78, B, H, N + 1, D, Dv, dtype="bf16", gated=True, g_low=0.85)
    pre = {n: t[:, :, :N] for n, t in inp.items()}
    _say(f"gated prefill then decode normalize={normalize}")
    _, S, z = fwd_ex(pre, 128, binding.OUT_NORMALIZED if normalize else binding.OUT_NUMERATOR)
    o = binding.decode_step(inp["q"][:, :, N].contiguous().to(DEV), inp["k"][:, :, N].contiguous().to(DEV),
                            inp["v"][:, :, N].contiguous().to(DEV), S, z, g=inp["g"][:, :, N].contiguous().to(DEV),
                            normalize=normalize)
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = oracle_run(inp, normalize)
    assert rowwise_rel_err(to64(o), o_ref[:, :, N]) <= TOL["bf16"]
    assert matrix_rel_err(to64(S), S_ref) <= TOL["bf16"]


def _heads(B, H, n, seed):
    rng = np.random.default_rng(seed)
    idx = rng.choice(B * H, size=min(n, B * H), replace=False)
    return [(int(i) // H, int(i) % H) for i in sorted(idx)]


def test_workload_gated_numerator_sampled_heads():
    w = workloads.WORKLOADS["gated_bf16"]
    inp = workloads.make_inputs(w)
    heads = _heads(w.B, w.H, 4, 15)
    _say(f"gated_bf16 numerator mode, oracle on heads {heads}")
    o, S, z = fwd_ex(inp, w.chunks[0], binding.OUT_NUMERATOR)
    o_ref, S_ref, _ = oracle_run(inp, False, heads=heads)
    assert rowwise_rel_err(sel(o, heads), o_ref) <= TOL["bf16"]
    assert matrix_rel_err(sel(S, heads), S_ref) <= TOL["bf16"]
    assert torch.isfinite(o).all().item()


@pytest.mark.parametrize("normalize", [True, False], ids=["normalized", "numerator"])
def test_workload_decode_gated_sampled_heads(normalize):
    w = workloads.WORKLOADS["decode_gated_bf16"]
    inp = workloads.make_inputs(w)
    heads = _heads(w.B, w.H, 64, 17)
    _say(f"decode_gated_bf16 full size normalize={normalize}")
    q, k, v, g = (inp[n].to(DEV) for n in ("q", "k", "v", "g"))
    S, z = inp["S"].to(DEV), inp["z"].to(DEV)
    o = binding.decode_step(q, k, v, S, z, g=g, normalize=normalize)
    torch.cuda.synchronize()
    pick = lambda n: sel(inp[n], heads)[0]                   # noqa: E731
    gsel = np.array([to64(inp["g"])[b, h] for b, h in heads])
    o_ref, S_ref, z_ref = oracle.decode_step(pick("q"), pick("k"), pick("v"), pick("S"), pick("z"), g=gsel,
                                             normalize=normalize)
    assert rowwise_rel_err(sel(o, heads)[0], o_ref) <= TOL["bf16"]
    assert matrix_rel_err(sel(S, heads), S_ref[None]) <= 1e-6
    assert matrix_rel_err(sel(z, heads), z_ref[None]) <= 1e-6
