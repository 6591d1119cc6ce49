"""Error metric and helpers for GPU-vs-oracle parity tests.

Metric (row-wise relative error): the maximum over output rows r = (b, h, t) of
max|o_gpu[r] - o_ref[r]| / max|o_ref[r]|.  Outputs are normalised averages of
signed values, so single entries can sit near zero while the row does not;
the row's own scale is the meaningful denominator.  States use the same metric
per (b, h) matrix.  Tolerances: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs with
fp32 state.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rowwise_rel_err(got, ref, axis=-1):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    num = np.abs(got - ref).max(axis=axis)
    den = np.maximum(np.abs(ref).max(axis=axis), 1e-30)
    return float((num / den).max())


def grad_rel_err(got, ref, floor=1e-2):
    """Row-wise relative error of a gradient [B, H, N, X]: max|diff| over a row divided by
    the row's max|ref|, floored at `floor` times the largest such row scale of the same
    (b, h).  Some gradient rows are exactly zero by structure (dq of the first token
    when nothing precedes it: o_0 = v_0 whatever q_0 is), so their own scale cannot be
    the denominator."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.maximum(den, np.maximum(floor * den.max(axis=-1, keepdims=True), 1e-30))
    return float((num / den).max())


def matrix_rel_err(got, ref):
    """Per leading index (b, h): max|diff| / max|ref| over the trailing matrix dims."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    g = got.reshape(got.shape[0], got.shape[1], -1)
    r = ref.reshape(ref.shape[0], ref.shape[1], -1)
    return rowwise_rel_err(g, r, axis=-1)


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()
