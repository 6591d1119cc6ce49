"""Plain fp64 CPU oracle of the gradients of causal kernelized linear attention.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call it.  It shares no code with the HIP path.

The pages give the forward only; they call the chunked form the training path
(aiwiki.thehackersbrain.dev page, closing paragraph of the chunked listing;
learn.pranaymahendrakar.com page, "Implementation reality": never train with the
sequential recurrence).  The gradients here are the plain definition: reverse-mode
differentiation, token by token, of the recurrence that ``recurrence.py`` runs
forwards (learn.pranaymahendrakar.com page, Researcher level, "Derivation", with
the scalar decay of "Try it yourself"):

    S_t = g_t S_{t-1} + phi(k_t) v_t^T,   z_t = g_t z_{t-1} + phi(k_t)
    num_t = S_t^T phi(q_t),   den_t = phi(q_t) . z_t
    o_t = num_t / max(den_t, eps)          (or o_t = num_t without the normaliser)

for the loss L = sum_t do_t . o_t, i.e. given the upstream gradient do.  Walking
t from N-1 down to 0 with the adjoints dS, dz of the state after token t
(zero after the last token):

    d      = max(den_t, eps)
    dnum   = do_t / d
    dden   = -(do_t . num_t) / d^2 where den_t >= eps, else 0 (the clamp passes no
             gradient below eps; at equality it passes, as torch's clamp does)
    dS    += phi(q_t) dnum^T,     dz += dden phi(q_t)
    dphi(q_t) = S_t dnum + dden z_t
    dphi(k_t) = dS v_t + dz
    dv_t      = dS^T phi(k_t)
    dg_t      = <dS, S_{t-1}> + <dz, z_{t-1}>
    dS, dz   *= g_t                     (the adjoint of the state after token t-1)

and at the end dS0 = dS, dz0 = dz.  Finally dq = dphi(q) * phi'(q) and
dk = dphi(k) * phi'(k), with phi'(x) = 1 for x > 0 and exp(x) for x <= 0.

States are kept at checkpoints every ``block`` tokens and recomputed inside a
block during the backward walk, so memory stays at O(N/block + block) states.
"""
from __future__ import annotations

import numpy as np

from .recurrence import EPS, phi


def dphi(x):
    """Derivative of elu(x) + 1 (alpha = 1): 1 above zero, exp(x) at or below it."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def causal_linear_attention_bwd(q, k, v, do, g=None, s0=None, z0=None, eps=EPS, normalize=True, block=256):
    """Gradients of sum(do * o) for o = causal_linear_attention(q, k, v, g, s0, z0, eps, normalize).

    q, k: [..., N, D]; v, do: [..., N, Dv]; g: [..., N] or None; s0: [..., D, Dv] or None;
    z0: [..., D] or None.  Returns a dict with dq, dk, dv (like q, k, v), dg (like g, or
    None), ds0 [..., D, Dv] and dz0 [..., D] (the gradients of the initial state, zeros
    included), all float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lead = q.shape[:-2]
    n, d = q.shape[-2], q.shape[-1]
    dv_ = v.shape[-1]
    gated = g is not None
    if gated:
        g = np.asarray(g, dtype=np.float64)
    S = np.zeros(lead + (d, dv_)) if s0 is None else np.array(s0, dtype=np.float64, copy=True)
    z = np.zeros(lead + (d,)) if z0 is None else np.array(z0, dtype=np.float64, copy=True)
    fq, fk = phi(q), phi(k)

    def step(S, z, t):
        if gated:
            S = g[..., t, None, None] * S
            z = g[..., t, None] * z
        return S + fk[..., t, :, None] * v[..., t, None, :], z + fk[..., t, :]

    # forward walk, keeping the state in front of every block
    starts = list(range(0, n, block))
    ckpt = []
    for b0 in starts:
        ckpt.append((S.copy(), z.copy()))
        for t in range(b0, min(n, b0 + block)):
            S, z = step(S, z, t)

    dfq = np.zeros_like(fq)
    dfk = np.zeros_like(fk)
    dv = np.zeros_like(v)
    dg = np.zeros_like(g) if gated else None
    dS = np.zeros(lead + (d, dv_))
    dz = np.zeros(lead + (d,))
    for bi in range(len(starts) - 1, -1, -1):
        b0, b1 = starts[bi], min(n, starts[bi] + block)
        Sb, zb = ckpt[bi]
        before = [(Sb, zb)]                      # before[i]: the state in front of token b0 + i
        for t in range(b0, b1):
            before.append(step(*before[-1], t))
        for t in range(b1 - 1, b0 - 1, -1):
            S_prev, z_prev = before[t - b0]
            S_t, z_t = before[t - b0 + 1]
            num = np.einsum("...d,...de->...e", fq[..., t, :], S_t)
            den = np.einsum("...d,...d->...", fq[..., t, :], z_t)
            if normalize:
                dd = np.maximum(den, eps)
                dnum = do[..., t, :] / dd[..., None]
                dden = np.where(den >= eps, -np.einsum("...e,...e->...", do[..., t, :], num) / dd ** 2, 0.0)
            else:
                dnum = do[..., t, :]
                dden = np.zeros(den.shape)
            dS = dS + fq[..., t, :, None] * dnum[..., None, :]
            dz = dz + dden[..., None] * fq[..., t, :]
            dfq[..., t, :] = np.einsum("...de,...e->...d", S_t, dnum) + dden[..., None] * z_t
            dfk[..., t, :] = np.einsum("...de,...e->...d", dS, v[..., t, :]) + dz
            dv[..., t, :] = np.einsum("...de,...d->...e", dS, fk[..., t, :])
            if gated:
                dg[..., t] = np.einsum("...de,...de->...", dS, S_prev) + np.einsum("...d,...d->...", dz, z_prev)
                dS = g[..., t, None, None] * dS
                dz = g[..., t, None] * dz
    return {"dq": dfq * dphi(q), "dk": dfk * dphi(k), "dv": dv, "dg": dg, "ds0": dS, "dz0": dz}
