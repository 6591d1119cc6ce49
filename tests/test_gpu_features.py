"""GPU parity of the other feature maps (linattn_fwd_features): ReLU plus a shift and
FAVOR+ random features, against the oracle with the same map (anandmoghan-problems page,
"Key Functions & Tricks"; aicassindra.com page, "Performer")."""
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


def spec(feature, shift, W):
    return ("relu", shift) if feature == "relu" else ("favor", to64(W))


CASES = [
    # (B, H, N, D, Dv, M, dtype, chunk, feature)
    (1, 2, 300, 64, 64, 64, "f32", 64, "relu"),
    (2, 2, 640, 64, 64, 64, "bf16", 128, "relu"),
    (1, 2, 333, 128, 128, 128, "bf16", 64, "relu"),
    (1, 2, 300, 64, 64, 64, "f32", 64, "favor"),
    (1, 2, 257, 64, 64, 128, "bf16", 64, "favor"),
    (2, 2, 640, 64, 64, 64, "bf16", 128, "favor"),
    (1, 2, 200, 128, 64, 64, "bf16", 128, "favor"),
    (1, 1, 1, 64, 64, 64, "bf16", 64, "favor"),
    # bf16, M = D = 64: ungated, the walk forms the features while staging (ragged tails,
    # several segments, Dv = 128)
    (1, 3, 64 * 5 + 17, 64, 128, 64, "bf16", 128, "favor"),
    (2, 1, 64 * 9 + 40, 64, 64, 64, "bf16", 64, "favor"),
]


@pytest.mark.parametrize("normalize", [True, False], ids=["normalized", "numerator"])
@pytest.mark.parametrize("gated", [False, True], ids=["ungated", "gated"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}N{}D{}Dv{}M{}{}c{}{}".format(*c))
def test_features_small_against_oracle(case, gated, normalize):
    B, H, N, D, Dv, M, dt, chunk, feature = case
    _say(f"features {case} gated={gated} normalize={normalize}")
    scale = 1.0 if feature == "relu" else D ** -0.25
    inp = workloads.random_inputs(7 + N + M, B, H, N, D, Dv, dtype=dt, scale=scale, gated=gated, g_low=0.8,
                                  with_state=True, state_scale=2.0)
    s0 = inp["s0"] if M == D else torch.randn(B, H, M, Dv, generator=torch.Generator().manual_seed(1)) * 2.0
    z0 = inp["z0"] if M == D else torch.rand(B, H, M, generator=torch.Generator().manual_seed(2)) * 2.0
    W = workloads.favor_projection(N + D, H, M, D) if feature == "favor" else None
    o, S, z = binding.fwd_features(*(_dev(inp[n]) for n in ("q", "k", "v")), feature, shift=0.05, W=_dev(W),
                                   g=_dev(inp.get("g")), chunk=chunk, s0=_dev(s0), z0=_dev(z0), return_state=True,
                                   normalize=normalize)
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = oracle.causal_linear_attention(
        to64(inp["q"]), to64(inp["k"]), to64(inp["v"]), g=None if not gated else to64(inp["g"]), s0=to64(s0),
        z0=to64(z0), normalize=normalize, feature=spec(feature, 0.05, W))
    tol = TOL[dt]
    assert rowwise_rel_err(to64(o), o_ref) <= tol
    assert matrix_rel_err(to64(S), S_ref) <= tol
    assert matrix_rel_err(to64(z), z_ref) <= tol


@pytest.mark.parametrize("feature", ["relu", "favor"])
def test_features_decode_step(feature):
    B, H, D, Dv, M = 3, 4, 64, 64, 128 if feature == "favor" else 64
    gen = torch.Generator().manual_seed(3)
    q = (torch.randn(B, H, D, generator=gen) * 0.35).to(torch.bfloat16)
    k = (torch.randn(B, H, D, generator=gen) * 0.35).to(torch.bfloat16)
    v = torch.randn(B, H, Dv, generator=gen).to(torch.bfloat16)
    S = torch.randn(B, H, M, Dv, generator=gen) * 10
    z = torch.rand(B, H, M, generator=gen) * 10
    W = workloads.favor_projection(4, H, M, D) if feature == "favor" else None
    _say(f"features decode {feature}")
    o_ref, S_ref, z_ref = oracle.decode_step(to64(q), to64(k), to64(v), to64(S), to64(z), feature=spec(feature, 0.05, W))
    Sd, zd = S.to(DEV), z.to(DEV)
    o = binding.decode_step_features(q.to(DEV), k.to(DEV), v.to(DEV), Sd, zd, feature, shift=0.05, W=_dev(W))
    torch.cuda.synchronize()
    assert rowwise_rel_err(to64(o), o_ref) <= TOL["bf16"]
    assert matrix_rel_err(to64(Sd), S_ref) <= TOL["bf16"]
    assert matrix_rel_err(to64(zd), z_ref) <= TOL["bf16"]


def test_features_reject_bad_arguments():
    inp = workloads.random_inputs(5, 1, 1, 64, 64, 64, dtype="bf16")
    q, k, v = (_dev(inp[n]) for n in ("q", "k", "v"))
    with pytest.raises(RuntimeError, match="unsupported"):
        binding.fwd_features(q, k, v, "relu", chunk=32)
    with pytest.raises(RuntimeError, match="unsupported"):
        binding.fwd_features(q, k, v, "favor", W=_dev(workloads.favor_projection(1, 1, 96, 64)))


def _heads(B, H, n, seed):
    rng = np.random.default_rng(seed)
    idx = rng.choice(B * H, size=min(n, B * H), replace=False)
    return [(int(i) // H, int(i) % H) for i in sorted(idx)]


@pytest.mark.parametrize("feature", ["relu", "favor"])
def test_features_workload_sampled_heads(feature):
    w = workloads.WORKLOADS["train_bf16" if feature == "relu" else "favor_bf16"]
    inp = workloads.make_inputs(w)
    W = workloads.favor_projection(w.seed, w.H, 64, w.D) if feature == "favor" else None
    heads = _heads(w.B, w.H, 3, 29)
    _say(f"{w.name} with {feature} features, oracle on heads {heads}")
    o = binding.fwd_features(*(_dev(inp[n]) for n in ("q", "k", "v")), feature, shift=0.05, W=_dev(W), chunk=128)
    torch.cuda.synchronize()
    pick = lambda t: np.stack([to64(t)[b, h] for b, h in heads])[None]    # noqa: E731
    Wsel = None if W is None else to64(W)[[h for _, h in heads]]
    o_ref, _, _ = oracle.causal_linear_attention(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]),
                                                 feature=("relu", 0.05) if W is None else ("favor", Wsel))
    assert rowwise_rel_err(pick(o), o_ref) <= TOL["bf16"]
    assert torch.isfinite(o).all().item()


def test_favor_in_walk_many_heads():
    # FAVOR+ on 128 heads of D = Dv = M = 64 at chunk 128, the walks forming the features
    # while staging: several segments per head whose totals the output walk sums itself,
    # with an initial state, a ragged tail and the final state returned
    B, H, N, D, Dv, chunk = 8, 16, 128 * 7 + 77, 64, 64, 128
    inp = workloads.random_inputs(63, B, H, N, D, Dv, dtype="bf16", scale=D ** -0.25, with_state=True,
                                  state_scale=2.0)
    W = workloads.favor_projection(63, H, D, D)
    heads = _heads(B, H, 4, 63)
    _say(f"favor in-walk features, 128 heads, oracle on heads {heads}")
    o, S, z = binding.fwd_features(*(_dev(inp[n]) for n in ("q", "k", "v")), "favor", W=_dev(W), chunk=chunk,
                                   s0=_dev(inp["s0"]), z0=_dev(inp["z0"]), return_state=True)
    torch.cuda.synchronize()
    pick = lambda t: np.stack([to64(t)[b, h] for b, h in heads])[None]    # noqa: E731
    o_ref, S_ref, z_ref = oracle.causal_linear_attention(
        pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), s0=pick(inp["s0"]), z0=pick(inp["z0"]),
        feature=("favor", to64(W)[[h for _, h in heads]]))
    assert rowwise_rel_err(pick(o), o_ref) <= TOL["bf16"]
    assert matrix_rel_err(pick(S), S_ref) <= TOL["bf16"]
    assert matrix_rel_err(pick(z), z_ref) <= TOL["bf16"]


@pytest.mark.parametrize("gated", [False, True], ids=["ungated", "gated"])
@pytest.mark.parametrize("chunk", [64, 128])
@pytest.mark.parametrize("M", [64, 128])
def test_features_orthogonal_favor(M, chunk, gated):
    # the page's orthogonal projections (aicassindra.com page, "Performer"): blocks of D
    # orthogonal rows, two blocks when M = 2 D (ungated with M = D: features formed in
    # the walk; otherwise by the feature pass)
    B, H, N, D, Dv = 2, 2, 700, 64, 64
    inp = workloads.random_inputs(91 + M, B, H, N, D, Dv, dtype="bf16", scale=D ** -0.25, gated=gated, g_low=0.9)
    W = workloads.favor_projection(92 + M, H, M, D, orthogonal=True)
    _say(f"orthogonal favor M={M} chunk={chunk} gated={gated}")
    g = inp.get("g")
    o, S, z = binding.fwd_features(*(_dev(inp[n]) for n in ("q", "k", "v")), "favor", W=_dev(W), g=_dev(g),
                                   chunk=chunk, return_state=True)
    torch.cuda.synchronize()
    o_ref, S_ref, z_ref = oracle.causal_linear_attention(to64(inp["q"]), to64(inp["k"]), to64(inp["v"]),
                                                         g=None if g is None else to64(g),
                                                         feature=("favor", to64(W)))
    assert rowwise_rel_err(to64(o), o_ref) <= TOL["bf16"]
    assert matrix_rel_err(to64(S), S_ref) <= TOL["bf16"]
    assert matrix_rel_err(to64(z), z_ref) <= TOL["bf16"]
