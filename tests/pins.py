"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes an oracle module (anything exposing ``phi``,
``causal_linear_attention`` and ``decode_step``) and raises on a mismatch.
``test_oracle.py`` runs them on the real oracle; ``test_oracle_mutants.py``
runs them on copies of the oracle with planted mistakes and expects each
mistake to be caught by at least one pin.

Nothing here retypes the oracle's recurrence: the references are the pages'
worked examples (``golden/``), hand-derived values, closed forms, and a brute
force pairwise sum that uses torch's own ``elu`` for the feature map.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def elu1(x):
    """elu(x) + 1 through torch's library elu, in float64 (independent of the oracle's phi)."""
    return torch.nn.functional.elu(torch.as_tensor(np.asarray(x, dtype=np.float64))).numpy() + 1.0


def pairwise(q, k, v, g=None, eps=1e-6, normalize=True):
    """Brute force: W_ij = phi(q_i).phi(k_j) * prod_{l=j+1..i} g_l for j <= i, O = W V / max(W 1, eps),
    or O = W V alone when ``normalize`` is False (the parallel form of retention on the
    aicassindra.com page, "RetNet and gated linear attention": a decay-masked score
    matrix times V, with no denominator).

    The explicit masked kernel-score form (learn.pranaymahendrakar.com page,
    Developer level, part 3 of linear_attention.py; anandmoghan-problems page,
    "Key Functions & Tricks", the equivalence check), with the decay weights of
    the same page's "Try it yourself" exercise.  Pure loops over (i, j): tiny
    inputs only.  Inputs [..., N, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    fq, fk = elu1(q), elu1(k)
    lead = q.shape[:-2]
    n = q.shape[-2]
    o = np.zeros(lead + (n, v.shape[-1]))
    for idx in np.ndindex(*lead):
        for i in range(n):
            num = np.zeros(v.shape[-1])
            den = 0.0
            for j in range(i + 1):
                w = float(np.dot(fq[idx + (i,)], fk[idx + (j,)]))
                if g is not None:
                    for l in range(j + 1, i + 1):
                        w *= float(g[idx + (l,)])
                num += w * v[idx + (j,)]
                den += w
            o[idx + (i,)] = num / max(den, eps) if normalize else num
    return o


def _rng_inputs(seed, lead, n, d, dv, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=lead + (n, d)) * scale
    k = rng.normal(size=lead + (n, d)) * scale
    v = rng.normal(size=lead + (n, dv))
    return q, k, v


# ---------------------------------------------------------------- pins ----

def pin_phi_values(orc):
    """phi = elu + 1: closed-form values on both branches, continuity at 0, positivity."""
    x = np.array([-700.0, -30.0, -2.0, -1.0, -1e-12, 0.0, 1e-12, 0.5, 1.0, 3.0])
    got = orc.phi(x)
    want = np.array([math.exp(-700.0), math.exp(-30.0), math.exp(-2.0), math.exp(-1.0),
                     math.exp(-1e-12), 1.0, 1.0 + 1e-12, 1.5, 2.0, 4.0])
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)
    assert np.all(got > 0)
    y = np.linspace(-20, 20, 4001)
    # torch's elu is expm1(x) on the negative side, so elu + 1 loses ~1e-16 absolute there
    np.testing.assert_allclose(orc.phi(y), elu1(y), rtol=1e-14, atol=2e-16)


def pin_hand_example(orc):
    """Hand-worked exact example, ungated and gated, including the final state."""
    gd = golden("hand_example.json")
    q, k, v = (np.array(gd[n], dtype=np.float64) for n in ("q", "k", "v"))
    o, S, z = orc.causal_linear_attention(q, k, v)
    np.testing.assert_allclose(o, gd["o_ungated"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(S, gd["S_N_ungated"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(z, gd["z_N_ungated"], rtol=1e-14, atol=0)
    o, S, z = orc.causal_linear_attention(q, k, v, g=np.array(gd["g"]))
    np.testing.assert_allclose(o, gd["o_gated"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(S, gd["S_N_gated"], rtol=1e-14, atol=0)
    np.testing.assert_allclose(z, gd["z_N_gated"], rtol=1e-14, atol=0)


def pin_eps_clamp(orc):
    """Denominator below eps: the clamp reading gives 0.5 * v0 (golden/eps_clamp.json)."""
    gd = golden("eps_clamp.json")
    o, _, _ = orc.causal_linear_attention(np.array(gd["q"]), np.array(gd["k"]), np.array(gd["v"]),
                                          eps=gd["eps"])
    np.testing.assert_allclose(o, gd["o"], rtol=1e-12, atol=0)


def pin_first_output_is_v0(orc):
    """Output 0 equals v_0 for any q_0 (anandmoghan-problems page, step 6)."""
    for seed, (d, dv) in enumerate([(3, 2), (4, 4), (8, 6), (1, 5)]):
        q, k, v = _rng_inputs(100 + seed, (2, 3), 5, d, dv)
        o, _, _ = orc.causal_linear_attention(q, k, v)
        np.testing.assert_allclose(o[..., 0, :], v[..., 0, :], rtol=1e-13, atol=1e-15)
        g = np.random.default_rng(seed).uniform(0.3, 1.0, size=(2, 3, 5))
        o, _, _ = orc.causal_linear_attention(q, k, v, g=g)
        np.testing.assert_allclose(o[..., 0, :], v[..., 0, :], rtol=1e-13, atol=1e-15)


def pin_pairwise_bruteforce(orc):
    """Recurrence equals the brute-force masked pairwise form on tiny inputs, ungated and gated."""
    for seed, (n, d, dv) in enumerate([(6, 3, 2), (9, 4, 4), (7, 8, 6), (5, 2, 7)]):
        q, k, v = _rng_inputs(200 + seed, (2,), n, d, dv, scale=1.5)
        o, _, _ = orc.causal_linear_attention(q, k, v)
        np.testing.assert_allclose(o, pairwise(q, k, v), rtol=1e-12, atol=1e-14)
        g = np.random.default_rng(300 + seed).uniform(0.2, 1.0, size=(2, n))
        o, _, _ = orc.causal_linear_attention(q, k, v, g=g)
        np.testing.assert_allclose(o, pairwise(q, k, v, g=g), rtol=1e-12, atol=1e-14)


def pin_p4_noncausal_example(orc):
    """mlblogg.com worked example: the non-causal output for query i equals the causal
    recurrence's last row when every query is q_i (the last row sees every key);
    it must match the pairwise-normalised reference to atol 1e-10, shape (12, 6)."""
    gd = golden("p4_worked_example.json")
    rng = np.random.default_rng(gd["seed"])
    q, k = rng.normal(size=tuple(gd["qk_size"]))
    v = rng.normal(size=tuple(gd["v_size"]))
    fq, fk = elu1(q), elu1(k)
    scores = fq @ fk.T
    reference = (scores @ v) / scores.sum(-1, keepdims=True)
    n = q.shape[0]
    qq = np.broadcast_to(q[:, None, :], (n, n, q.shape[1]))            # batch i: every query is q_i
    kk = np.broadcast_to(k[None], (n,) + k.shape)
    vv = np.broadcast_to(v[None], (n,) + v.shape)
    o, _, _ = orc.causal_linear_attention(qq, kk, vv)
    out = o[:, -1, :]
    assert list(out.shape) == gd["printed_shape"]
    np.testing.assert_allclose(out, reference, atol=gd["atol"], rtol=0)


def pin_p2_worked_example(orc):
    """learn.pranaymahendrakar.com Developer script (seed 0, N=8, d=4): the fp64 oracle sits
    within the page's 1e-4 of the fp32 masked quadratic form, and within 1e-5 (the order of
    the printed max difference, 4.8e-7, which is fp32 noise)."""
    gd = golden("p2_worked_example.json")
    torch.manual_seed(gd["seed"])
    N, d = gd["N"], gd["d"]
    Q, K, V = torch.randn(N, d), torch.randn(N, d), torch.randn(N, d)
    fq = torch.nn.functional.elu(Q) + 1
    fk = torch.nn.functional.elu(K) + 1
    left = (fq @ fk.T) @ V
    right = fq @ (fk.T @ V)
    assert torch.allclose(left, right, atol=gd["associative_atol"]) == gd["printed_associative"]
    w = (fq @ fk.T) * torch.tril(torch.ones(N, N))
    quad = (w @ V) / (w.sum(-1, keepdim=True) + 1e-6)
    o, S, _ = orc.causal_linear_attention(Q.double().numpy(), K.double().numpy(), V.double().numpy())
    diff = np.abs(o - quad.double().numpy()).max()
    assert (diff <= gd["recurrent_vs_quadratic_atol"]) == gd["printed_recurrent_matches_quadratic"]
    assert diff <= 1e-5, diff
    assert S.size == gd["printed_state_numbers"]


def pin_doctest_shapes(orc):
    """anandmoghan-problems doctest: q, k (1,4,3), v (1,4,2) -> output (1,4,2)."""
    gd = golden("p3_doctest.json")
    rng = np.random.default_rng(3)
    q = rng.normal(size=gd["q_shape"])
    k = rng.normal(size=gd["k_shape"])
    v = rng.normal(size=gd["v_shape"])
    o, S, z = orc.causal_linear_attention(q, k, v)
    assert list(o.shape) == gd["out_shape"]
    assert S.shape == (1, 3, 2) and z.shape == (1, 3)


def pin_convex_hull(orc):
    """Non-negative weights: every output coordinate lies between the min and max of the
    values seen so far (aiwiki.thehackersbrain.dev page, opening section)."""
    q, k, v = _rng_inputs(400, (3,), 40, 6, 5, scale=2.0)
    g = np.random.default_rng(401).uniform(0.5, 1.0, size=(3, 40))
    for gg in (None, g):
        o, _, _ = orc.causal_linear_attention(q, k, v, g=gg)
        lo = np.minimum.accumulate(v, axis=-2)
        hi = np.maximum.accumulate(v, axis=-2)
        assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def pin_closed_forms(orc):
    """Constant V gives O = V; constant K gives the prefix mean of V whatever Q is
    (and with a constant gate gamma, the normalised exponential moving average);
    the output is affine-equivariant in V."""
    rng = np.random.default_rng(500)
    n, d, dv = 12, 5, 3
    q = rng.normal(size=(2, n, d)) * 2
    k = rng.normal(size=(2, n, d))
    c = rng.normal(size=(2, 1, dv))
    o, _, _ = orc.causal_linear_attention(q, k, np.broadcast_to(c, (2, n, dv)))
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=1e-13, atol=1e-14)
    kc = np.broadcast_to(rng.normal(size=(2, 1, d)), (2, n, d))
    v = rng.normal(size=(2, n, dv))
    o, _, _ = orc.causal_linear_attention(q, kc, v)
    mean = np.cumsum(v, axis=-2) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, mean, rtol=1e-12, atol=1e-13)
    gamma = 0.7
    o, _, _ = orc.causal_linear_attention(q, kc, v, g=np.full((2, n), gamma))
    want = np.zeros_like(v)
    for i in range(n):
        w = gamma ** (i - np.arange(i + 1))
        want[:, i] = (w[None, :, None] * v[:, : i + 1]).sum(1) / w.sum()
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-13)
    alpha, beta = -1.7, 0.3
    o1, _, _ = orc.causal_linear_attention(q, k, v)
    o2, _, _ = orc.causal_linear_attention(q, k, alpha * v + beta)
    np.testing.assert_allclose(o2, alpha * o1 + beta, rtol=1e-12, atol=1e-12)


def pin_unit_gate_is_ungated(orc):
    """g == 1 reproduces the ungated result exactly."""
    q, k, v = _rng_inputs(600, (2, 2), 17, 4, 3)
    a = orc.causal_linear_attention(q, k, v)
    b = orc.causal_linear_attention(q, k, v, g=np.ones((2, 2, 17)))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def pin_resume(orc):
    """The state is a checkpoint: running N1 tokens, then N2 tokens from (S_N1, z_N1),
    equals one run over N1 + N2 tokens, ungated and gated."""
    q, k, v = _rng_inputs(700, (2,), 30, 4, 6)
    g = np.random.default_rng(701).uniform(0.6, 1.0, size=(2, 30))
    for gg in (None, g):
        o, S, z = orc.causal_linear_attention(q, k, v, g=gg)
        g1 = None if gg is None else gg[..., :11]
        g2 = None if gg is None else gg[..., 11:]
        o1, S1, z1 = orc.causal_linear_attention(q[..., :11, :], k[..., :11, :], v[..., :11, :], g=g1)
        o2, S2, z2 = orc.causal_linear_attention(q[..., 11:, :], k[..., 11:, :], v[..., 11:, :], g=g2,
                                                 s0=S1, z0=z1)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=-2), o, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(S2, S, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(z2, z, rtol=1e-13, atol=1e-13)


def pin_decode_composition(orc):
    """A decode step from the state after N tokens equals row N of the run over N + 1 tokens,
    and its state update is S + phi(k) v^T exactly (elementwise)."""
    q, k, v = _rng_inputs(800, (3,), 10, 5, 4)
    g = np.random.default_rng(801).uniform(0.5, 1.0, size=(3, 10))
    for gg in (None, g):
        o, S, z = orc.causal_linear_attention(q, k, v, g=gg)
        _, S9, z9 = orc.causal_linear_attention(q[..., :9, :], k[..., :9, :], v[..., :9, :],
                                                g=None if gg is None else gg[..., :9])
        od, Sd, zd = orc.decode_step(q[..., 9, :], k[..., 9, :], v[..., 9, :], S9, z9,
                                     g=None if gg is None else gg[..., 9])
        np.testing.assert_allclose(od, o[..., 9, :], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(Sd, S, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(zd, z, rtol=1e-13, atol=1e-13)
    S0 = np.abs(np.random.default_rng(802).normal(size=(3, 5, 4))) * 1000
    z0 = np.abs(np.random.default_rng(803).normal(size=(3, 5))) * 1000
    _, Sd, zd = orc.decode_step(q[..., 0, :], k[..., 0, :], v[..., 0, :], S0, z0)
    fk = elu1(k[..., 0, :])
    np.testing.assert_allclose(Sd, S0 + fk[..., :, None] * v[..., 0, None, :], rtol=1e-15, atol=1e-13)
    np.testing.assert_allclose(zd, z0 + fk, rtol=1e-15, atol=1e-13)


def pin_numerator_mode(orc):
    """Normaliser-free output (retention: aicassindra.com page, "RetNet and gated linear
    attention"; learn.pranaymahendrakar.com page, "Implementation reality").

    * brute force: o = W V with the decay-weighted scores, ungated and gated;
    * closed form: q = k = 0 makes phi(q).phi(k) = D, so with V constant c, a constant
      gate gamma and an initial state S0, o_i = gamma^(i+1) 1^T S0 + D c (1 - gamma^(i+1)) / (1 - gamma),
      and gamma = 1 gives 1^T S0 + D c (i + 1);
    * the state it returns is the normalised mode's, and a decode step in this mode
      continues a run in this mode."""
    for seed, (n, d, dv) in enumerate([(6, 3, 2), (9, 4, 4), (7, 8, 6)]):
        q, k, v = _rng_inputs(900 + seed, (2,), n, d, dv, scale=1.5)
        o, _, _ = orc.causal_linear_attention(q, k, v, normalize=False)
        np.testing.assert_allclose(o, pairwise(q, k, v, normalize=False), rtol=1e-12, atol=1e-13)
        g = np.random.default_rng(950 + seed).uniform(0.2, 1.0, size=(2, n))
        o, _, _ = orc.causal_linear_attention(q, k, v, g=g, normalize=False)
        np.testing.assert_allclose(o, pairwise(q, k, v, g=g, normalize=False), rtol=1e-12, atol=1e-13)
    n, d, dv = 14, 6, 3
    rng = np.random.default_rng(990)
    c = rng.normal(size=(2, 1, dv))
    S0 = rng.normal(size=(2, d, dv))
    zero = np.zeros((2, n, d))
    i = np.arange(n)[None, :, None]
    for gamma in (1.0, 0.8):
        g = np.full((2, n), gamma)
        o, _, _ = orc.causal_linear_attention(zero, zero, np.broadcast_to(c, (2, n, dv)), g=g, s0=S0,
                                              z0=np.ones((2, d)), normalize=False)
        geo = (i + 1.0) if gamma == 1.0 else (1 - gamma ** (i + 1.0)) / (1 - gamma)
        want = gamma ** (i + 1.0) * S0.sum(1)[:, None, :] + d * c * geo
        np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-13)
    q, k, v = _rng_inputs(995, (3,), 10, 5, 4)
    g = np.random.default_rng(996).uniform(0.5, 1.0, size=(3, 10))
    on, Sn, zn = orc.causal_linear_attention(q, k, v, g=g)
    o, S, z = orc.causal_linear_attention(q, k, v, g=g, normalize=False)
    np.testing.assert_array_equal(S, Sn)
    np.testing.assert_array_equal(z, zn)
    _, S9, z9 = orc.causal_linear_attention(q[..., :9, :], k[..., :9, :], v[..., :9, :], g=g[..., :9],
                                            normalize=False)
    od, Sd, zd = orc.decode_step(q[..., 9, :], k[..., 9, :], v[..., 9, :], S9, z9, g=g[..., 9], normalize=False)
    np.testing.assert_allclose(od, o[..., 9, :], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Sd, S, rtol=1e-13, atol=1e-13)


def _pairwise_vector(q, k, v, a, normalize=True, eps=1e-6):
    """Brute force with per-dimension decay: A_ij = sum_d phi(q_i)[d] phi(k_j)[d] prod_{l=j+1..i} a_l[d]
    for j <= i; O = A V / max(A 1, eps) (or A V).  Pure loops, tiny inputs only."""
    fq, fk = elu1(q), elu1(k)
    lead = q.shape[:-2]
    n = q.shape[-2]
    o = np.zeros(lead + (n, v.shape[-1]))
    for idx in np.ndindex(*lead):
        for i in range(n):
            num = np.zeros(v.shape[-1])
            den = 0.0
            for j in range(i + 1):
                w = fq[idx + (i,)] * fk[idx + (j,)]
                for l in range(j + 1, i + 1):
                    w = w * a[idx + (l,)]
                wsum = float(w.sum())
                num += wsum * v[idx + (j,)]
                den += wsum
            o[idx + (i,)] = num / max(den, eps) if normalize else num
    return o


def pin_vector_decay(orc):
    """Per-dimension decay (gated linear attention's Diag(alpha_t), aicassindra.com page):
    * the per-dimension decay-weighted pairwise form, both output modes, D != Dv;
    * a decay equal in every dimension is the scalar gate;
    * closed form: q = k = 0 and a constant decay gamma_d per dimension, V constant c,
      no normaliser: o_i = c sum_d (1 - gamma_d^(i+1)) / (1 - gamma_d);
    * a decode step with this token's decay continues the run."""
    for seed, (n, d, dv) in enumerate([(6, 3, 2), (8, 4, 5)]):
        q, k, v = _rng_inputs(1600 + seed, (2,), n, d, dv, scale=1.5)
        a = np.random.default_rng(1650 + seed).uniform(0.3, 1.0, size=(2, n, d))
        for normalize in (True, False):
            o, _, _ = orc.causal_linear_attention(q, k, v, a=a, normalize=normalize)
            np.testing.assert_allclose(o, _pairwise_vector(q, k, v, a, normalize), rtol=1e-12, atol=1e-13)
    q, k, v = _rng_inputs(1700, (2, 2), 11, 4, 3)
    g = np.random.default_rng(1701).uniform(0.5, 1.0, size=(2, 2, 11))
    x = orc.causal_linear_attention(q, k, v, g=g)
    y = orc.causal_linear_attention(q, k, v, a=np.repeat(g[..., None], 4, -1))
    for p_, r_ in zip(x, y):
        np.testing.assert_allclose(r_, p_, rtol=1e-13, atol=1e-14)
    n, d, dv = 12, 4, 3
    gam = np.array([0.5, 0.8, 0.95, 1.0])
    c = np.random.default_rng(1702).normal(size=(1, 1, dv))
    zero = np.zeros((1, n, d))
    o, _, _ = orc.causal_linear_attention(zero, zero, np.broadcast_to(c, (1, n, dv)),
                                          a=np.broadcast_to(gam, (1, n, d)), normalize=False)
    i = np.arange(n, dtype=np.float64)[:, None]
    geo = np.where(gam < 1.0, (1 - gam[None, :] ** (i + 1)) / np.where(gam < 1.0, 1 - gam[None, :], 1.0), i + 1)
    np.testing.assert_allclose(o[0], c[0] * geo.sum(-1, keepdims=True), rtol=1e-13, atol=1e-13)
    q, k, v = _rng_inputs(1703, (3,), 10, 5, 4)
    a = np.random.default_rng(1704).uniform(0.5, 1.0, size=(3, 10, 5))
    o, S, z = orc.causal_linear_attention(q, k, v, a=a)
    _, S9, z9 = orc.causal_linear_attention(q[..., :9, :], k[..., :9, :], v[..., :9, :], a=a[..., :9, :])
    od, Sd, zd = orc.decode_step(q[..., 9, :], k[..., 9, :], v[..., 9, :], S9, z9, a=a[..., 9, :])
    np.testing.assert_allclose(od, o[..., 9, :], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sd, S, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(zd, z, rtol=1e-13, atol=1e-13)


def pin_relu_features(orc):
    """ReLU plus a shift (anandmoghan-problems page, "Key Functions & Tricks"): the masked
    pairwise form with torch's relu, both output modes; q = k = 0 makes every weight
    D shift^2, so the normalised output is the prefix mean of V."""
    shift = 0.05
    q, k, v = _rng_inputs(1800, (2,), 9, 4, 3, scale=1.5)
    fq = torch.relu(torch.as_tensor(q)).numpy() + shift
    fk = torch.relu(torch.as_tensor(k)).numpy() + shift
    for normalize in (True, False):
        o, _, _ = orc.causal_linear_attention(q, k, v, feature=("relu", shift), normalize=normalize)
        w = np.tril(np.einsum("bid,bjd->bij", fq, fk))
        want = w @ v
        if normalize:
            want = want / np.maximum(w.sum(-1, keepdims=True), 1e-6)
        np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-13)
    zero = np.zeros((2, 9, 4))
    o, _, _ = orc.causal_linear_attention(zero, zero, v, feature=("relu", shift))
    np.testing.assert_allclose(o, np.cumsum(v, axis=-2) / np.arange(1, 10)[:, None], rtol=1e-12, atol=1e-13)


def pin_favor_features(orc):
    """FAVOR+ (aicassindra.com page, "Performer"): the features' expected inner product is
    exp(q . k) over Gaussian projections (Monte Carlo over 4000 draws of 8 features,
    within 5 standard errors), and with many features the causal attention they give
    approaches causal softmax attention, o_i = sum_{j<=i} exp(q_i.k_j) v_j / sum exp(q_i.k_j),
    written out directly."""
    rng = np.random.default_rng(1900)
    d = 4
    q1 = rng.normal(size=(1, 1, d)) * 0.4
    k1 = rng.normal(size=(1, 1, d)) * 0.4
    est = []
    for r in range(4000):
        W = np.random.default_rng(10_000 + r).normal(size=(1, 8, d))
        fq, fk = orc.favor_features(q1, W), orc.favor_features(k1, W)
        est.append(float((fq * fk).sum()))
    est = np.array(est)
    target = float(np.exp((q1 * k1).sum()))
    se = est.std() / np.sqrt(len(est))
    assert abs(est.mean() - target) < 5 * se, (est.mean(), target, se)
    n, h = 7, 2
    q = rng.normal(size=(1, h, n, d)) * 0.3
    k = rng.normal(size=(1, h, n, d)) * 0.3
    v = rng.normal(size=(1, h, n, 3))
    W = np.random.default_rng(1901).normal(size=(h, 20000, d))
    o, S, z = orc.causal_linear_attention(q, k, v, feature=("favor", W))
    assert S.shape == (1, h, 20000, 3) and z.shape == (1, h, 20000)
    sm = np.zeros_like(o)
    for hh in range(h):
        for i in range(n):
            wts = np.exp(np.array([q[0, hh, i] @ k[0, hh, j] for j in range(i + 1)]))
            sm[0, hh, i] = (wts[:, None] * v[0, hh, : i + 1]).sum(0) / wts.sum()
    np.testing.assert_allclose(o, sm, atol=0.05)
    # a decode step with the same features continues a run (favor and relu)
    W = np.random.default_rng(1902).normal(size=(h, 6, d))
    for feat in (("favor", W), ("relu", 0.1)):
        o, S, z = orc.causal_linear_attention(q, k, v, feature=feat)
        _, S6, z6 = orc.causal_linear_attention(q[..., :6, :], k[..., :6, :], v[..., :6, :], feature=feat)
        od, Sd, zd = orc.decode_step(q[..., 6, :], k[..., 6, :], v[..., 6, :], S6, z6, feature=feat)
        np.testing.assert_allclose(od, o[..., 6, :], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Sd, S, rtol=1e-12, atol=1e-13)


ALL_PINS = [
    pin_phi_values,
    pin_hand_example,
    pin_eps_clamp,
    pin_first_output_is_v0,
    pin_pairwise_bruteforce,
    pin_p4_noncausal_example,
    pin_p2_worked_example,
    pin_doctest_shapes,
    pin_convex_hull,
    pin_closed_forms,
    pin_unit_gate_is_ungated,
    pin_resume,
    pin_decode_composition,
    pin_numerator_mode,
    pin_vector_decay,
    pin_relu_features,
    pin_favor_features,
]
