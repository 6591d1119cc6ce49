"""fp64 model of the chunked parallel form (test infrastructure only).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.  This is not the
parity reference (that is ``recurrence.causal_linear_attention``); it is the
chunk algebra written out plainly so the tests can show, on the CPU, that the
chunked form reaches the recurrence's result for any chunk size, ragged tails,
gating and an initial state.

Ungated, following the chunked code of the aiwiki.thehackersbrain.dev page
(the ``linear_attention_chunked`` listing and the closing paragraph: quadratic
inside a chunk, recurrent across chunks).  For a chunk of rows [s, e) with
Fq = phi(Q_c), Fk = phi(K_c):
    A     = tril(Fq Fk^T)                       (causal mask, diagonal kept)
    num   = Fq S_prev + A V_c
    den   = Fq z_prev + A 1
    O_c   = num / max(den, eps)
    S_next = S_prev + Fk^T V_c,   z_next = z_prev + Fk^T 1

Gated, the "weighted quadratic form" that the learn.pranaymahendrakar.com page
("Try it yourself") asks for, with a chunk-local inclusive log-decay
L_i = sum_{l=s..i} log g_l:
    A_ij  = Fq_i . Fk_j * exp(L_i - L_j)   for j <= i, else 0
    num_i = exp(L_i) Fq_i S_prev + sum_j A_ij v_j
    den_i = exp(L_i) Fq_i . z_prev + sum_j A_ij
    S_next = exp(L_last) S_prev + sum_j exp(L_last - L_j) Fk_j v_j^T   (same for z)
Every decay factor used is exp of a non-positive number, so nothing overflows.

``normalize=False`` returns num alone, as the recurrence does.

Per-dimension decay a [..., N, D] (gated linear attention), with the chunk-local
inclusive L_i[d] = sum_{l=s..i} log a_l[d]:
    A_ij  = sum_d Fq_i[d] Fk_j[d] exp(L_i[d] - L_j[d])   for j <= i
    num_i = (Fq_i * exp(L_i)) S_prev + sum_j A_ij v_j,  den alike with z_prev
    S_next = Diag(exp(L_last)) S_prev + (Fk * exp(L_last - L))^T V_c   (z alike)
"""
from __future__ import annotations

import numpy as np

from .recurrence import EPS, phi


def chunked_linear_attention(q, k, v, chunk, g=None, s0=None, z0=None, eps=EPS, normalize=True, a=None):
    """Chunked form over [..., N, D] inputs.  Returns (o, S_N, z_N) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    n, d = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    S = np.zeros(lead + (d, dv)) if s0 is None else np.array(s0, dtype=np.float64, copy=True)
    z = np.zeros(lead + (d,)) if z0 is None else np.array(z0, dtype=np.float64, copy=True)
    fq_all, fk_all = phi(q), phi(k)
    o = np.zeros(lead + (n, dv))
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        fq, fk, vc = fq_all[..., s:e, :], fk_all[..., s:e, :], v[..., s:e, :]
        c = e - s
        tril = np.tril(np.ones((c, c)))
        scores = fq @ np.swapaxes(fk, -1, -2)
        if a is not None:
            lam = np.cumsum(np.log(np.asarray(a, dtype=np.float64)[..., s:e, :]), axis=-2)    # [.., c, D]
            diff = lam[..., :, None, :] - lam[..., None, :, :]                             # [.., i, j, D]
            w = np.exp(np.minimum(diff, 0.0)) * tril[..., None]
            A = np.einsum("...id,...jd,...ijd->...ij", fq, fk, w)
            fqd = fq * np.exp(lam)
            num = fqd @ S + A @ vc
            den = fqd @ z[..., :, None] + A.sum(-1, keepdims=True)
            fkd = fk * np.exp(lam[..., -1:, :] - lam)
            last = np.exp(lam[..., -1, :])
            S = last[..., :, None] * S + np.swapaxes(fkd, -1, -2) @ vc
            z = last * z + fkd.sum(-2)
        elif g is None:
            A = scores * tril
            num = fq @ S + A @ vc
            den = fq @ z[..., :, None] + A.sum(-1, keepdims=True)
            S = S + np.swapaxes(fk, -1, -2) @ vc
            z = z + fk.sum(-2)
        else:
            lam = np.cumsum(np.log(np.asarray(g, dtype=np.float64)[..., s:e]), axis=-1)
            diff = lam[..., :, None] - lam[..., None, :]
            decay = np.where(tril > 0, np.exp(np.minimum(diff, 0.0)), 0.0)
            A = scores * decay
            row = np.exp(lam)[..., :, None]
            num = row * (fq @ S) + A @ vc
            den = row * (fq @ z[..., :, None]) + A.sum(-1, keepdims=True)
            tail = np.exp(lam[..., -1:] - lam)                   # exp(L_last - L_j)
            fkd = fk * tail[..., :, None]
            last = np.exp(lam[..., -1])
            S = last[..., None, None] * S + np.swapaxes(fkd, -1, -2) @ vc
            z = last[..., None] * z + fkd.sum(-2)
        o[..., s:e, :] = num / np.maximum(den, eps) if normalize else num
    return o, S, z
