"""GPU parity of the per-dimension decay (gated linear attention's Diag(alpha_t)):
linattn_fwd_vdecay and linattn_decode_step_vdecay against the fp64 oracle with the same
decay (aicassindra.com page, "RetNet and gated linear attention")."""
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


def decay(seed, shape, low):
    gen = torch.Generator().manual_seed(seed)
    return low + (1.0 - low) * torch.rand(*shape, generator=gen, dtype=torch.float32)


def oracle_run(inp, a, normalize=True, s0=None, z0=None, heads=None):
    def pick(t):
        if t is None:
            return None
        x = to64(t)
        return x if heads is None else np.stack([x[b, h] for b, h in heads])[None]
    return oracle.causal_linear_attention(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), s0=pick(s0), z0=pick(z0),
                                          normalize=normalize, a=pick(a))


CASES = [
    # (B, H, N, D, Dv, dtype)
    (1, 2, 256, 64, 64, "f32"),
    (1, 1, 97, 64, 128, "f32"),
    (2, 1, 150, 64, 64, "f32"),
    (2, 2, 640, 64, 64, "bf16"),
    (1, 2, 333, 128, 128, "bf16"),
    (1, 2, 200, 64, 128, "bf16"),
    (1, 1, 1, 64, 64, "bf16"),
    (3, 1, 1025, 64, 64, "bf16"),
    (1, 2, 150, 128, 64, "f32"),
]


@pytest.mark.parametrize("normalize", [True, False], ids=["normalized", "numerator"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}D{}Dv{}{}".format(*c))
def test_vdecay_small_against_oracle(case, normalize):
    B, H, N, D, Dv, dt = case
    _say(f"vdecay {case} normalize={normalize}")
    inp = workloads.random_inputs(91 + N + D, B, H, N, D, Dv, dtype=dt, with_state=True, state_scale=5.0)
    a = decay(N + D, (B, H, N, D), 0.5)
    o, S, z = binding.fwd_vdecay(*(_dev(inp[n]) for n in ("q", "k", "v")), _dev(a), s0=_dev(inp["s0"]),
                                 z0=_dev(inp["z0"]), return_state=True, normalize=normalize)
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = oracle_run(inp, a, normalize, s0=inp["s0"], z0=inp["z0"])
    tol = TOL[dt]
    assert rowwise_rel_err(to64(o), o_ref) <= tol
    assert matrix_rel_err(to64(S), S_ref) <= tol
    assert matrix_rel_err(to64(z), z_ref) <= tol


def test_vdecay_unsupported_raises():
    inp = workloads.random_inputs(3, 1, 1, 64, 128, 128, dtype="f32")
    a = decay(4, (1, 1, 64, 128), 0.5)
    with pytest.raises(RuntimeError, match="unsupported"):
        binding.fwd_vdecay(*(_dev(inp[n]) for n in ("q", "k", "v")), _dev(a))


def test_vdecay_strong_decay_range():
    # decays down to 2^-8 per token: the rescaled block operands stay finite
    B, H, N, D, Dv = 1, 2, 300, 64, 64
    inp = workloads.random_inputs(17, B, H, N, D, Dv, dtype="bf16")
    a = decay(18, (B, H, N, D), 2.0 ** -8)
    _say("vdecay strong decay")
    o = binding.fwd_vdecay(*(_dev(inp[n]) for n in ("q", "k", "v")), _dev(a))
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item()
    o_ref, _, _ = oracle_run(inp, a)
    assert rowwise_rel_err(to64(o), o_ref) <= TOL["bf16"]


def test_vdecay_equal_dims_is_the_scalar_gate():
    B, H, N, D, Dv = 1, 2, 500, 64, 64
    inp = workloads.random_inputs(19, B, H, N, D, Dv, dtype="f32", gated=True, g_low=0.8)
    a = inp["g"][..., None].expand(B, H, N, D).contiguous()
    _say("vdecay with equal dimensions vs the gated forward")
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    o1 = binding.fwd_vdecay(q, k, v, _dev(a))
    o2 = binding.fwd_gated(q, k, v, _dev(inp["g"]), chunk=64)
    torch.cuda.synchronize()
    assert rowwise_rel_err(to64(o1), to64(o2)) <= TOL["f32"]


@pytest.mark.parametrize("normalize", [True, False], ids=["normalized", "numerator"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_vdecay_small(dims, dt, normalize):
    D, Dv = dims
    B, H = 3, 5
    gen = torch.Generator().manual_seed(D + 5 * Dv)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    q = torch.randn(B, H, D, generator=gen).to(tdt)
    k = torch.randn(B, H, D, generator=gen).to(tdt)
    v = torch.randn(B, H, Dv, generator=gen).to(tdt)
    S = torch.randn(B, H, D, Dv, generator=gen) * 30
    z = torch.randn(B, H, D, generator=gen).abs() * 30
    a = decay(D + Dv, (B, H, D), 0.3)
    _say(f"decode vdecay dims={dims} dt={dt} normalize={normalize}")
    o_ref, S_ref, z_ref = oracle.decode_step(to64(q), to64(k), to64(v), to64(S), to64(z), a=to64(a), normalize=normalize)
    Sd, zd = S.to(DEV), z.to(DEV)
    o = binding.decode_step(q.to(DEV), k.to(DEV), v.to(DEV), Sd, zd, a=a.to(DEV), normalize=normalize)
    torch.cuda.synchronize()
    assert rowwise_rel_err(to64(o), o_ref) <= TOL[dt]
    assert matrix_rel_err(to64(Sd), S_ref) <= 1e-6
    assert matrix_rel_err(to64(zd), z_ref) <= 1e-6


def test_vdecay_prefill_then_decode():
    B, H, N, D, Dv = 1, 2, 257, 128, 128
    inp = workloads.random_inputs(79, B, H, N + 1, D, Dv, dtype="bf16")
    a = decay(80, (B, H, N + 1, D), 0.7)
    _say("vdecay prefill then decode")
    _, S, z = binding.fwd_vdecay(*(_dev(inp[n][:, :, :N]) for n in ("q", "k", "v")), _dev(a[:, :, :N].contiguous()),
                                 return_state=True)
    o = binding.decode_step(*(inp[n][:, :, N].contiguous().to(DEV) for n in ("q", "k", "v")), S, z,
                            a=a[:, :, N].contiguous().to(DEV))
    torch.cuda.synchronize()
    o_ref, _, _ = oracle_run(inp, a)
    assert rowwise_rel_err(to64(o), o_ref[:, :, N]) <= TOL["bf16"]


def _heads(B, H, n, seed):
    rng = np.random.default_rng(seed)
    idx = rng.choice(B * H, size=min(n, B * H), replace=False)
    return [(int(i) // H, int(i) % H) for i in sorted(idx)]


def test_vdecay_workload_sampled_heads():
    w = workloads.WORKLOADS["vdecay_bf16"]
    inp = workloads.make_inputs(w)
    heads = _heads(w.B, w.H, 4, 21)
    _say(f"vdecay_bf16 full size, oracle on heads {heads}")
    o, S, z = binding.fwd_vdecay(*(_dev(inp[n]) for n in ("q", "k", "v", "a")), return_state=True)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = oracle_run(inp, inp["a"], heads=heads)
    sel = lambda t: np.stack([to64(t)[b, h] for b, h in heads])[None]     # noqa: E731
    assert rowwise_rel_err(sel(o), o_ref) <= TOL["bf16"]
    assert matrix_rel_err(sel(S), S_ref) <= TOL["bf16"]
    assert torch.isfinite(o).all().item()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_vdecay_runs_sampled_heads(dt):
    """128 heads of 596 tokens: on a 256-CU device the launch walks each head in several
    runs of chunks (the last run and chunk ragged), carrying the state through each run;
    outputs, final state and z against the oracle on sampled heads."""
    B, H, N, D, Dv = 2, 64, 596, 64, 64
    inp = workloads.random_inputs(777, B, H, N, D, Dv, dtype=dt, with_state=True, state_scale=5.0)
    a = decay(778, (B, H, N, D), 0.5)
    heads = _heads(B, H, 4, 23)
    _say(f"vdecay runs {dt}, oracle on heads {heads}")
    o, S, z = binding.fwd_vdecay(*(_dev(inp[n]) for n in ("q", "k", "v")), _dev(a), s0=_dev(inp["s0"]),
                                 z0=_dev(inp["z0"]), return_state=True)
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = oracle_run(inp, a, s0=inp["s0"], z0=inp["z0"], heads=heads)
    sel = lambda t: np.stack([to64(t)[b, h] for b, h in heads])[None]     # noqa: E731
    assert rowwise_rel_err(sel(o), o_ref) <= TOL[dt]
    assert matrix_rel_err(sel(S), S_ref) <= TOL[dt]
    assert matrix_rel_err(sel(z), z_ref) <= TOL[dt]


def test_decode_vdecay_workload_sampled_heads():
    w = workloads.WORKLOADS["decode_vdecay_bf16"]
    inp = workloads.make_inputs(w)
    heads = _heads(w.B, w.H, 64, 23)
    _say("decode_vdecay_bf16 full size")
    S, z = inp["S"].to(DEV), inp["z"].to(DEV)
    o = binding.decode_step(*(inp[n].to(DEV) for n in ("q", "k", "v")), S, z, a=inp["a"].to(DEV))
    torch.cuda.synchronize()
    pick = lambda n: np.stack([to64(inp[n])[b, h] for b, h in heads])      # noqa: E731
    o_ref, S_ref, _ = oracle.decode_step(pick("q"), pick("k"), pick("v"), pick("S"), pick("z"), a=pick("a"))
    got = lambda t: np.stack([to64(t)[b, h] for b, h in heads])            # noqa: E731
    assert rowwise_rel_err(got(o), o_ref) <= TOL["bf16"]
    assert matrix_rel_err(got(S)[None], S_ref[None]) <= 1e-6
