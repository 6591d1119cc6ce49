"""Pins for the backward oracle (oracle/backward.py).

Each ``pin_*`` takes a module exposing ``causal_linear_attention_bwd`` and raises on a
mismatch.  The references are independent of the reverse walk being checked:

* central finite differences of the forward oracle (pinned on its own in pins.py);
* torch autograd through the explicit decay-weighted pairwise form, which never
  forms a state (learn.pranaymahendrakar.com page, Developer level, the masked
  kernel-score form; "Try it yourself" for the decay weights);
* closed forms for q = k = 0 (phi = 1) under a constant gate;
* invariants of the normalised output: shifting every v by c shifts every o by c,
  so sum_j dv_j = sum_i do_i; scaling phi(q_i) leaves o_i unchanged, so
  phi(q_i) . dphi(q_i) = 0 where the clamp is inactive.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.recurrence as fwd_oracle


def _inputs(seed, lead, n, d, dv, gated=True, state=True):
    rng = np.random.default_rng(seed)
    out = {
        "q": rng.normal(size=lead + (n, d)),
        "k": rng.normal(size=lead + (n, d)),
        "v": rng.normal(size=lead + (n, dv)),
        "do": rng.normal(size=lead + (n, dv)),
        "g": rng.uniform(0.5, 1.0, size=lead + (n,)) if gated else None,
        "s0": rng.normal(size=lead + (d, dv)) if state else None,
        "z0": np.abs(rng.normal(size=lead + (d,))) if state else None,
    }
    return out


def _loss(x, normalize, eps=1e-6):
    o, _, _ = fwd_oracle.causal_linear_attention(x["q"], x["k"], x["v"], g=x["g"], s0=x["s0"], z0=x["z0"], eps=eps,
                                                 normalize=normalize)
    return float((o * x["do"]).sum())


def pin_bwd_finite_differences(orc):
    """Every gradient against central differences of the forward oracle (fp64, h = 1e-6),
    gated with an initial state, both output modes, on tiny inputs; the second case puts
    some denominators below the clamp (very negative queries make phi(q) tiny)."""
    cases = [(1100, None), (1101, -16.0)]       # -16: den_2 = 7e-7 < eps, den_3 = 2e-6
    for seed, qshift in cases:
        for normalize in (True, False):
            x = _inputs(seed, (2,), 6, 3, 2)
            if qshift is not None:
                x["q"][0, 2:4] += qshift
                x["z0"] = x["z0"] * 1e-3
            got = orc.causal_linear_attention_bwd(x["q"], x["k"], x["v"], x["do"], g=x["g"], s0=x["s0"], z0=x["z0"],
                                                  normalize=normalize)
            for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("s0", "ds0"), ("z0", "dz0")):
                base = x[name]
                fd = np.zeros_like(base)
                for idx in np.ndindex(*base.shape):
                    h = 1e-6 * max(1.0, abs(base[idx]))
                    xp = dict(x)
                    xp[name] = base.copy()
                    xp[name][idx] += h
                    lp = _loss(xp, normalize)
                    xp[name][idx] -= 2 * h
                    lm = _loss(xp, normalize)
                    fd[idx] = (lp - lm) / (2 * h)
                np.testing.assert_allclose(got[gname], fd, rtol=2e-6, atol=2e-7 * max(1.0, np.abs(fd).max()),
                                           err_msg=f"{gname} normalize={normalize} seed={seed}")


def _pairwise_torch(q, k, v, g, normalize, eps=1e-6):
    """o_i = sum_{j<=i} w_ij v_j / max(sum_{j<=i} w_ij, eps), w_ij = phi(q_i).phi(k_j) prod_{l=j+1..i} g_l,
    written with dense masked matrices (no state); phi through torch's elu."""
    fq = torch.nn.functional.elu(q) + 1
    fk = torch.nn.functional.elu(k) + 1
    n = q.shape[-2]
    scores = fq @ fk.transpose(-1, -2)
    mask = torch.tril(torch.ones(n, n, dtype=torch.float64))
    if g is not None:
        lg = torch.cumsum(torch.log(g), dim=-1)                       # sum_{l<=i} log g_l
        decay = torch.exp((lg[..., :, None] - lg[..., None, :]).clamp(max=0.0)) * mask
        w = scores * decay
    else:
        w = scores * mask
    num = w @ v
    if not normalize:
        return num
    return num / torch.clamp(w.sum(-1, keepdim=True), min=eps)


def pin_bwd_autograd_pairwise(orc):
    """dq, dk, dv, dg equal torch autograd through the pairwise form, ungated and gated,
    both output modes (no initial state: the pairwise form has none)."""
    for gated in (False, True):
        for normalize in (True, False):
            x = _inputs(1200 + gated, (2, 2), 37, 4, 3, gated=gated, state=False)
            ts = {n: torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v")}
            tg = torch.tensor(x["g"], requires_grad=True) if gated else None
            o = _pairwise_torch(ts["q"], ts["k"], ts["v"], tg, normalize)
            (o * torch.tensor(x["do"])).sum().backward()
            got = orc.causal_linear_attention_bwd(x["q"], x["k"], x["v"], x["do"], g=x["g"], normalize=normalize)
            for n in ("q", "k", "v"):
                ref = ts[n].grad.numpy()
                np.testing.assert_allclose(got["d" + n], ref, rtol=1e-9, atol=1e-11 * max(1.0, np.abs(ref).max()))
            if gated:
                ref = tg.grad.numpy()
                np.testing.assert_allclose(got["dg"], ref, rtol=1e-9, atol=1e-11 * max(1.0, np.abs(ref).max()))


def pin_bwd_closed_forms(orc):
    """q = k = 0 (phi = 1, phi'(0) = 1), a constant gate gamma, no normaliser:
    o_i = D sum_{j<=i} gamma^(i-j) v_j, so dv_j = D sum_{i>=j} gamma^(i-j) do_i, and every
    component of dq_i is sum_{j<=i} gamma^(i-j) v_j . do_i, every component of dk_j is
    sum_{i>=j} gamma^(i-j) do_i . v_j."""
    n, d, dv, gamma = 9, 4, 3, 0.75
    rng = np.random.default_rng(1300)
    v = rng.normal(size=(2, n, dv))
    do = rng.normal(size=(2, n, dv))
    zero = np.zeros((2, n, d))
    got = orc.causal_linear_attention_bwd(zero, zero, v, do, g=np.full((2, n), gamma), normalize=False)
    lag = np.arange(n)[:, None] - np.arange(n)[None, :]             # i - j
    w = np.where(lag >= 0, gamma ** np.maximum(lag, 0).astype(np.float64), 0.0)
    np.testing.assert_allclose(got["dv"], d * np.einsum("ij,bie->bje", w, do), rtol=1e-13, atol=1e-13)
    vdo = np.einsum("bie,bje->bij", do, v)                        # do_i . v_j
    dq = (w[None] * vdo).sum(-1)
    dk = (w[None] * vdo).sum(-2)
    np.testing.assert_allclose(got["dq"], np.repeat(dq[..., None], d, -1), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(got["dk"], np.repeat(dk[..., None], d, -1), rtol=1e-13, atol=1e-13)


def pin_bwd_invariants(orc):
    """Normalised output: sum_j dv_j = sum_i do_i (shift invariance), phi(q_i) . dphi(q_i) = 0
    (scale invariance of each row, clamp inactive), dg_0 = 0 without an initial state, and
    g = 1 gives the ungated gradients."""
    x = _inputs(1400, (3,), 25, 5, 4, gated=True, state=False)
    got = orc.causal_linear_attention_bwd(x["q"], x["k"], x["v"], x["do"], g=x["g"])
    np.testing.assert_allclose(got["dv"].sum(-2), x["do"].sum(-2), rtol=1e-11, atol=1e-11)
    fq = fwd_oracle.phi(x["q"])
    dfq = got["dq"] / np.where(x["q"] > 0, 1.0, np.exp(np.minimum(x["q"], 0.0)))
    np.testing.assert_allclose((fq * dfq).sum(-1), 0.0, atol=1e-10 * np.abs(fq * dfq).max())
    np.testing.assert_array_equal(got["dg"][..., 0], 0.0)
    a = orc.causal_linear_attention_bwd(x["q"], x["k"], x["v"], x["do"])
    b = orc.causal_linear_attention_bwd(x["q"], x["k"], x["v"], x["do"], g=np.ones_like(x["g"]))
    for n in ("dq", "dk", "dv", "ds0", "dz0"):
        np.testing.assert_allclose(a[n], b[n], rtol=1e-13, atol=1e-14)


def pin_bwd_block_independent(orc):
    """The checkpoint spacing is bookkeeping: block 1, 7 and 256 give the same gradients."""
    x = _inputs(1500, (2,), 30, 3, 3)
    ref = orc.causal_linear_attention_bwd(x["q"], x["k"], x["v"], x["do"], g=x["g"], s0=x["s0"], z0=x["z0"])
    for block in (1, 7):
        got = orc.causal_linear_attention_bwd(x["q"], x["k"], x["v"], x["do"], g=x["g"], s0=x["s0"], z0=x["z0"],
                                              block=block)
        for n in ref:
            np.testing.assert_allclose(got[n], ref[n], rtol=1e-12, atol=1e-13)


ALL_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_autograd_pairwise,
    pin_bwd_closed_forms,
    pin_bwd_invariants,
    pin_bwd_block_independent,
]
