"""The seeded input generators: properties the pages fix for the random inputs they
describe (no attention arithmetic here beyond the oracle's own feature map)."""
import numpy as np
import torch

import oracle
from causal_kernelized_linear_amd import workloads


def test_orthogonal_favor_rows():
    # aicassindra.com page, "Performer": the projections w_r are made orthogonal.  Within
    # each block of D rows the directions are orthonormal; blocks and heads differ.
    H, M, D = 3, 20, 8
    W = workloads.favor_projection(5, H, M, D, orthogonal=True).double()
    assert W.shape == (H, M, D) and W.dtype == torch.float64
    for h in range(H):
        for b0 in range(0, M, D):
            blk = W[h, b0:b0 + D]
            gram = blk @ blk.T
            off = gram - torch.diag(torch.diagonal(gram))
            assert off.abs().max().item() < 1e-5 * gram.abs().max().item()
    assert not torch.allclose(W[0], W[1])
    # the default stays independent Gaussian rows, drawn as before
    g = torch.Generator().manual_seed(5)
    assert torch.equal(workloads.favor_projection(5, H, M, D), torch.randn(H, M, D, generator=g))


def test_orthogonal_favor_rows_have_gaussian_lengths():
    # each row keeps the length of an N(0, I_D) draw: E|w|^2 = D (6000 rows, 5 standard errors)
    W = workloads.favor_projection(6, 50, 120, 16, orthogonal=True).double()
    sq = (W ** 2).sum(-1).flatten()
    assert abs(sq.mean().item() - 16) < 5 * sq.std().item() / np.sqrt(sq.numel())


def test_orthogonal_features_estimate_exp_dot():
    # with orthogonal rows the FAVOR+ features still estimate exp(q.k) without bias (the
    # page's claim for the positive random features; Monte Carlo over 3000 draws of one
    # block of 4 orthogonal rows, within 5 standard errors)
    rng = np.random.default_rng(77)
    d = 4
    q = rng.normal(size=(1, 1, d)) * 0.4
    k = rng.normal(size=(1, 1, d)) * 0.4
    est = []
    for r in range(3000):
        W = workloads.favor_projection(20_000 + r, 1, d, d, orthogonal=True).double().numpy()
        est.append(float((oracle.favor_features(q, W) * oracle.favor_features(k, W)).sum()))
    est = np.array(est)
    target = float(np.exp((q * k).sum()))
    assert abs(est.mean() - target) < 5 * est.std() / np.sqrt(len(est)), (est.mean(), target)
