"""The chunk algebra (oracle/chunked.py) reaches the recurrence's result (CPU only).

Chunk size 1 is the recurrence itself; a chunk at least as long as the sequence
is the masked quadratic form; everything between, ragged tails, gating and an
initial state must agree to fp64 rounding."""
import numpy as np
import pytest

import oracle


def _inputs(seed, lead, n, d, dv):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=lead + (n, d))
    k = rng.normal(size=lead + (n, d))
    v = rng.normal(size=lead + (n, dv))
    g = rng.uniform(0.5, 1.0, size=lead + (n,))
    s0 = rng.normal(size=lead + (d, dv))
    z0 = np.abs(rng.normal(size=lead + (d,)))
    return q, k, v, g, s0, z0


@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 100, 128, 1000])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("normalize", [True, False])
def test_chunked_equals_recurrence(chunk, gated, with_state, normalize):
    q, k, v, g, s0, z0 = _inputs(chunk * 7 + gated, (2, 2), 100, 8, 6)
    kw = dict(g=g if gated else None, s0=s0 if with_state else None, z0=z0 if with_state else None,
              normalize=normalize)
    o_r, S_r, z_r = oracle.causal_linear_attention(q, k, v, **kw)
    o_c, S_c, z_c = oracle.chunked_linear_attention(q, k, v, chunk, **kw)
    np.testing.assert_allclose(o_c, o_r, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S_c, S_r, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(z_c, z_r, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("chunk", [1, 16, 64, 100])
@pytest.mark.parametrize("normalize", [True, False])
def test_chunked_vector_decay_equals_recurrence(chunk, normalize):
    q, k, v, _, s0, z0 = _inputs(chunk + 5, (2,), 90, 6, 5)
    a = np.random.default_rng(chunk).uniform(0.4, 1.0, size=(2, 90, 6))
    kw = dict(a=a, s0=s0, z0=z0, normalize=normalize)
    o_r, S_r, z_r = oracle.causal_linear_attention(q, k, v, **kw)
    o_c, S_c, z_c = oracle.chunked_linear_attention(q, k, v, chunk, **kw)
    np.testing.assert_allclose(o_c, o_r, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S_c, S_r, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(z_c, z_r, rtol=1e-11, atol=1e-11)


def test_chunked_long_decay_does_not_overflow():
    # 0.05 ** 300 underflows; chunk-local decays must keep every factor <= 1.
    q, k, v, _, _, _ = _inputs(11, (1,), 300, 4, 4)
    g = np.full((1, 300), 0.05)
    o_r, _, _ = oracle.causal_linear_attention(q, k, v, g=g)
    o_c, _, _ = oracle.chunked_linear_attention(q, k, v, 128, g=g)
    assert np.all(np.isfinite(o_c))
    np.testing.assert_allclose(o_c, o_r, rtol=1e-10, atol=1e-12)
