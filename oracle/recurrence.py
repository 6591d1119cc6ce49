"""Plain fp64 CPU oracle: causal kernelized linear attention as a token-by-token recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module; the
product path (the HIP library and its Python binding) never does.  It shares no
code with the HIP path.

What it computes (all arithmetic in float64, inputs widened exactly):

* phi(x) = elu(x) + 1 with alpha = 1, i.e. x + 1 for x > 0 and exp(x) for
  x <= 0.  The map is the one of "Transformers are RNNs" named on the
  learn.pranaymahendrakar.com page (Researcher level, "Derivation") and on the
  aicassindra.com page ("Linear Transformer: elu+1 ...").  The exp branch is
  evaluated on min(x, 0) so the unused branch cannot overflow, as the
  mlblogg.com page does in "An implementation you can check".

* Other feature maps, by ``feature``: ``("relu", shift)`` gives max(x, 0) + shift (the
  "F.relu(x) + eps" alternative the anandmoghan-problems page names under "Key Functions
  & Tricks"); ``("favor", W)`` gives Performer's positive random features
  phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m) for the m rows w_r of W [H, m, D] (one
  set per head; aicassindra.com page, "Performer: unbiased softmax by positive random
  features", whose expected inner product is exp(q . k)).  The state is then
  [m, Dv] and z [m].

* The causal recurrence of the learn.pranaymahendrakar.com page (Researcher
  level, "Derivation", the display equations for S_i, z_i and o_i):
      S_i = S_{i-1} + phi(k_i) v_i^T,   z_i = z_{i-1} + phi(k_i),
      o_i = S_i^T phi(q_i) / (z_i^T phi(q_i)).
  The current token is added to the state before the query reads it (the
  mlblogg.com page, "The causal recurrence"; step 3 before step 4 of the
  anandmoghan-problems page, "Step-by-Step Approach").  No 1/sqrt(d) scaling:
  that belongs to the softmax similarity only.

* The denominator is clamped, o_i = num_i / max(den_i, eps) with eps = 1e-6,
  as the chunked code of the aiwiki.thehackersbrain.dev page divides by
  ``clamp(min=1e-6)``.  (Other pages add eps instead; the clamp is the reading
  taken.)

* The gated recurrence with a scalar gate per head and token:
      S_t = g_t S_{t-1} + phi(k_t) v_t^T,   z_t = g_t z_{t-1} + phi(k_t).
  The decay form of S is the one on the aiwiki.thehackersbrain.dev page ("What
  is actually lost", with G_t a scalar) and the learn.pranaymahendrakar.com
  page ("Try it yourself", "Why plain linear attention underperforms"); the
  same gate also decays z, which keeps o_i a normalised average with weights
  prod_{l=j+1..i} g_l phi(q_i).phi(k_j).

* The vector-valued (per key dimension) decay of gated linear attention:
      S_t = Diag(a_t) S_{t-1} + phi(k_t) v_t^T,   z_t = a_t * z_{t-1} + phi(k_t),
  a_t in (0, 1]^D per head and token (aicassindra.com page, "RetNet and gated linear
  attention": S_i = Diag(alpha_i) S_{i-1} + k_i v_i^T; aiwiki.thehackersbrain.dev page,
  "What is actually lost": the decay G_t multiplies S_{t-1} elementwise, here with
  G_t[d, e] = a_t[d]).  z takes the same decay, as it does under the scalar gate.  A
  scalar gate and a vector decay may both be given; they multiply.

* An optional initial state (S0, z0) replaces the zero state, so a sequence
  can be resumed from a saved state; the final state (S_N, z_N) is returned.

* ``normalize=False`` returns the numerator alone, o_i = S_i^T phi(q_i): the
  output of retention, which has no phi(q)^T z denominator and leaves the
  scaling to a normalisation layer after the attention (aicassindra.com page,
  "RetNet and gated linear attention"; learn.pranaymahendrakar.com page,
  "Implementation reality": modern variants drop the normaliser).  The state
  recurrence is unchanged, z included, so a run can switch modes on a resumed
  state; eps is not used.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def phi(x):
    """elu(x) + 1 with alpha = 1, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def relu_features(x, shift):
    """max(x, 0) + shift, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + shift


def favor_features(x, W):
    """exp(W x - |x|^2 / 2) / sqrt(m) for x [..., H, D] and W [H, m, D] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    proj = np.einsum("...hd,hmd->...hm", x, W)
    return np.exp(proj - 0.5 * np.sum(x * x, axis=-1, keepdims=True)) / np.sqrt(W.shape[-2])


def feature_map(feature):
    """The map x [..., D] -> [..., m] that ``feature`` names (None: elu + 1)."""
    if feature is None:
        return phi
    kind = feature[0]
    if kind == "relu":
        return lambda x: relu_features(x, feature[1])
    if kind == "favor":
        return lambda x: favor_features(x, feature[1])
    raise ValueError(f"unknown feature map {kind!r}")


def causal_linear_attention(q, k, v, g=None, s0=None, z0=None, eps=EPS, normalize=True, a=None, feature=None):
    """Causal kernelized linear attention, one token at a time.

    q, k: [..., N, D]; v: [..., N, Dv]; g: [..., N] or None;
    s0: [..., D, Dv] or None; z0: [..., D] or None (None means zeros).
    normalize: divide by max(phi(q)^T z, eps) (True) or return the numerator.
    a: [..., N, m] per-dimension decay or None.
    feature: None (elu + 1), ("relu", shift) or ("favor", W [H, m, D]); with FAVOR+ the
    leading dimensions must end in H.
    Leading dimensions (batch, heads) are independent and are vectorised.
    Returns (o [..., N, Dv], S_N [..., D, Dv], z_N [..., D]), all float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lead = q.shape[:-2]
    n = q.shape[-2]
    dv = v.shape[-1]
    fmap = feature_map(feature)
    d = np.asarray(fmap(q[..., :1, :][..., 0, :])).shape[-1]     # feature width m
    if s0 is None:
        S = np.zeros(lead + (d, dv))
    else:
        S = np.array(s0, dtype=np.float64, copy=True)
    if z0 is None:
        z = np.zeros(lead + (d,))
    else:
        z = np.array(z0, dtype=np.float64, copy=True)
    if g is not None:
        g = np.asarray(g, dtype=np.float64)
    if a is not None:
        a = np.asarray(a, dtype=np.float64)
    o = np.zeros(lead + (n, dv))
    for t in range(n):
        fq = fmap(q[..., t, :])
        fk = fmap(k[..., t, :])
        if g is not None:
            gt = g[..., t]
            S = gt[..., None, None] * S
            z = gt[..., None] * z
        if a is not None:
            at = a[..., t, :]
            S = at[..., :, None] * S
            z = at * z
        S = S + fk[..., :, None] * v[..., t, None, :]
        z = z + fk
        num = np.einsum("...d,...de->...e", fq, S)
        den = np.einsum("...d,...d->...", fq, z)
        o[..., t, :] = num / np.maximum(den, eps)[..., None] if normalize else num
    return o, S, z


def decode_step(q, k, v, S, z, g=None, eps=EPS, normalize=True, a=None, feature=None):
    """One recurrent decode step from a stored state.

    q, k: [..., D]; v: [..., Dv]; S: [..., D, Dv]; z: [..., D]; g: [...] or None;
    a: [..., D] or None.
    The new token is folded into the state first, then read, exactly as one
    iteration of ``causal_linear_attention``.  Returns (o, S', z').
    """
    q = np.asarray(q, dtype=np.float64)[..., None, :]
    k = np.asarray(k, dtype=np.float64)[..., None, :]
    v = np.asarray(v, dtype=np.float64)[..., None, :]
    gg = None if g is None else np.asarray(g, dtype=np.float64)[..., None]
    aa = None if a is None else np.asarray(a, dtype=np.float64)[..., None, :]
    o, S1, z1 = causal_linear_attention(q, k, v, g=gg, s0=S, z0=z, eps=eps, normalize=normalize, a=aa,
                                        feature=feature)
    return o[..., 0, :], S1, z1
