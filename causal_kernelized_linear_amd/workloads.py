"""Seeded synthetic inputs for causal kernelized linear attention.

This module only draws random numbers: it holds none of the attention
arithmetic, so both the CPU oracle's tests and the HIP path can take their
inputs from it.  Every draw comes from one ``torch.Generator('cpu')`` seeded
per workload, in the fixed order Q, K, V, then the gate g or the decode state
(S, z).  Low-precision tensors are made with ``.to(torch.bfloat16)``, which
rounds to nearest even; the oracle later receives exactly those rounded values
widened to float64.

The named workloads follow the shapes and value distributions of the
workloads the pages discuss: head dimension 64 or 128 (the 32-head, 128-wide
linear heads of the hybrid stacks on the learn.pranaymahendrakar.com page,
"What modern variants change"), chunks of 64-256 (page 1 closing paragraph,
page 2 "Implementation reality"), and decay gates close to one (page 2 "Try it
yourself").  No dataset is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                     # "fwd", "gated", "vdecay", "decode", "decode_gated" or "decode_vdecay"
    B: int
    H: int
    N: int                        # tokens (1 for a decode step)
    D: int
    Dv: int
    dtype: str                    # "f32" or "bf16": dtype of q, k, v and o
    chunks: tuple = (128,)
    seed: int = 0
    scale: float = 1.0            # multiplies N(0,1) draws of q, k, v (in fp32, before rounding)
    eps: float = 1e-6
    note: str = ""

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "fp32_small": Workload("fp32_small", "fwd", 1, 2, 512, 64, 64, "f32", (64,), 1001,
                           note="fp32 parity case, oracle finishes in seconds"),
    "train_bf16": Workload("train_bf16", "fwd", 8, 16, 4096, 64, 64, "bf16", (128,), 1002,
                           note="training-shaped layer"),
    "longctx_bf16": Workload("longctx_bf16", "fwd", 1, 32, 65536, 128, 128, "bf16", (64, 128, 256), 1003,
                             scale=0.5, note="long context, chunk sweep"),
    "decode_bf16": Workload("decode_bf16", "decode", 256, 32, 1, 128, 128, "bf16", (1,), 1004,
                            note="one recurrent step for 256 sequences, fp32 state"),
    "gated_bf16": Workload("gated_bf16", "gated", 4, 16, 8192, 64, 64, "bf16", (128,), 1005,
                           note="scalar gate per head per token"),
    "decode_gated_bf16": Workload("decode_gated_bf16", "decode_gated", 256, 32, 1, 128, 128, "bf16", (1,), 1006,
                                  note="one gated recurrent step: the decode form of the gated forward"),
    "vdecay_bf16": Workload("vdecay_bf16", "vdecay", 4, 16, 8192, 64, 64, "bf16", (64,), 1007,
                            note="per-dimension decay per head and token (gated linear attention)"),
    "favor_bf16": Workload("favor_bf16", "fwd", 8, 16, 4096, 64, 64, "bf16", (128,), 1009, scale=64 ** -0.25,
                           note="FAVOR+ random features (64 orthogonal rows per head) on training-shaped inputs scaled by D^-1/4"),
    "decode_vdecay_bf16": Workload("decode_vdecay_bf16", "decode_vdecay", 256, 32, 1, 128, 128, "bf16", (1,), 1008,
                                   note="one recurrent step under a per-dimension decay"),
}


def _randn(gen, shape, scale=1.0):
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x


def make_inputs(w: Workload, B=None, H=None, N=None, with_grad=False):
    """Draw the inputs of workload ``w`` (optionally with B, H or N overridden).

    Returns a dict of CPU tensors in their stored dtypes:
      fwd:    q, k [B,H,N,D]; v [B,H,N,Dv]
      gated:  the same plus g [B,H,N] float32, g = 0.9 + 0.1*sigmoid(N(0,1))
      decode: q, k [B,H,D]; v [B,H,Dv]; S [B,H,D,Dv] and z [B,H,D] float32,
              each 1000*|N(0,1)| (a state after about 1000 tokens)
      decode_gated: the same plus this token's gate g [B,H] float32, drawn last as
              0.9 + 0.1*sigmoid(N(0,1)) like the gated forward's gates
      vdecay: the forward's q, k, v plus a per-dimension decay a [B,H,N,D] float32,
              0.9 + 0.1*sigmoid(N(0,1)) elementwise
      decode_vdecay: the decode inputs plus this token's decay a [B,H,D], drawn alike
    With ``with_grad`` (forward kinds) an upstream gradient dout [B,H,N,Dv] ~ N(0,1) in
    the input dtype is drawn after everything else, for the backward.
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    gen = torch.Generator(device="cpu").manual_seed(w.seed)
    dt = w.torch_dtype
    if w.kind in ("decode", "decode_gated", "decode_vdecay"):
        q = _randn(gen, (B, H, w.D), w.scale).to(dt)
        k = _randn(gen, (B, H, w.D), w.scale).to(dt)
        v = _randn(gen, (B, H, w.Dv), w.scale).to(dt)
        S = _randn(gen, (B, H, w.D, w.Dv)).abs_().mul_(1000.0)
        z = _randn(gen, (B, H, w.D)).abs_().mul_(1000.0)
        out = {"q": q, "k": k, "v": v, "S": S, "z": z}
        if w.kind == "decode_gated":
            out["g"] = 0.9 + 0.1 * torch.sigmoid(_randn(gen, (B, H)))
        if w.kind == "decode_vdecay":
            out["a"] = 0.9 + 0.1 * torch.sigmoid(_randn(gen, (B, H, w.D)))
        return out
    q = _randn(gen, (B, H, N, w.D), w.scale).to(dt)
    k = _randn(gen, (B, H, N, w.D), w.scale).to(dt)
    v = _randn(gen, (B, H, N, w.Dv), w.scale).to(dt)
    out = {"q": q, "k": k, "v": v}
    if w.kind == "gated":
        out["g"] = 0.9 + 0.1 * torch.sigmoid(_randn(gen, (B, H, N)))
    if w.kind == "vdecay":
        out["a"] = 0.9 + 0.1 * torch.sigmoid(_randn(gen, (B, H, N, w.D)))
    if with_grad:
        out["dout"] = _randn(gen, (B, H, N, w.Dv)).to(dt)
    return out


def favor_projection(seed, H, M, D, orthogonal=False):
    """Per-head FAVOR+ projections W [H, M, D], float32.

    Default: independent N(0, I_D) rows.  ``orthogonal=True``: the orthogonal random
    features of Performer (aicassindra.com page, "Performer": the projections w_r are
    made orthogonal).  Rows come in blocks of D; within a block their directions are the
    orthonormal columns of the QR factor of a D x D Gaussian draw (signs fixed by R's
    diagonal, so the basis is uniformly random), and each row is given the length of an
    independent N(0, I_D) draw, so every single row is still distributed as N(0, I_D).
    Blocks, and heads, are independent; the last block is cut to M rows."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    if not orthogonal:
        return torch.randn(H, M, D, generator=gen, dtype=torch.float32)
    nblk = (M + D - 1) // D
    W = torch.empty(H, nblk * D, D, dtype=torch.float64)
    for h in range(H):
        for b in range(nblk):
            G = torch.randn(D, D, generator=gen, dtype=torch.float64)
            Qf, R = torch.linalg.qr(G)
            Qf = Qf * torch.sign(torch.diagonal(R))[None, :]
            lengths = torch.randn(D, D, generator=gen, dtype=torch.float64).norm(dim=1)
            W[h, b * D:(b + 1) * D] = Qf.T * lengths[:, None]
    return W[:, :M].to(torch.float32).contiguous()


def random_inputs(seed, B, H, N, D, Dv, dtype="bf16", scale=1.0, gated=False,
                  g_low=0.9, with_state=False, state_scale=1.0, with_grad=False):
    """Small ad-hoc seeded inputs for edge-case tests (ragged N, odd shapes).

    g (if requested) is drawn uniformly in [g_low, 1].  With ``with_state`` an
    initial state s0 = state_scale*|N(0,1)|-ish is drawn too (s0 may have either
    sign; z0 is kept non-negative as a sum of positive features would be); with
    ``with_grad`` an upstream gradient dout ~ N(0,1) is drawn last.
    """
    gen = torch.Generator(device="cpu").manual_seed(seed)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = _randn(gen, (B, H, N, D), scale).to(dt)
    k = _randn(gen, (B, H, N, D), scale).to(dt)
    v = _randn(gen, (B, H, N, Dv), scale).to(dt)
    out = {"q": q, "k": k, "v": v}
    if gated:
        u = torch.rand(B, H, N, generator=gen, dtype=torch.float32)
        out["g"] = g_low + (1.0 - g_low) * u
    if with_state:
        out["s0"] = _randn(gen, (B, H, D, Dv)) * state_scale
        out["z0"] = _randn(gen, (B, H, D)).abs_() * state_scale
    if with_grad:
        out["dout"] = _randn(gen, (B, H, N, Dv)).to(dt)
    return out


def to_f64(t) -> np.ndarray:
    """Exact widening of a stored tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
