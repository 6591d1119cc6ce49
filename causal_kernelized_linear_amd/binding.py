"""ctypes binding of ``liblinattn.so`` (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only turns torch tensors into device pointers, picks the current HIP stream,
allocates the caller-side workspace and output tensors with torch, and raises
``RuntimeError`` carrying the library's status string on any failure.  There is
no fallback: if the library is missing, every call raises.

Function names match the C ABI (include/linattn.h):
    linattn_fwd_chunked, linattn_fwd_gated, linattn_fwd_ex, linattn_fwd_ex_noalloc, linattn_decode_step,
    linattn_decode_step_ex, linattn_fwd_workspace_size, linattn_bwd,
    linattn_bwd_workspace_size, linattn_fwd_vdecay, linattn_fwd_vdecay_workspace_size,
    linattn_decode_step_vdecay, linattn_fwd_features, linattn_fwd_features_workspace_size,
    linattn_status_string
plus the tensor-level helpers fwd_chunked, fwd_gated, fwd, fwd_vdecay, fwd_features,
decode_step_features, bwd and decode_step.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinattn.so")

F32, BF16 = 0, 1
OUT_NORMALIZED, OUT_NUMERATOR = 0, 1
FEATURE_RELU, FEATURE_FAVOR = 1, 2
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "hip", 5: "scratch limit"}
NOALLOC_SCRATCH_BYTES = 32 << 20     # LINATTN_NOALLOC_SCRATCH_BYTES

_lock = threading.Lock()
_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

EXPORTS = {
    "linattn_fwd_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "linattn_fwd_chunked": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _sz, _p]),
    "linattn_fwd_gated": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _sz, _p]),
    "linattn_fwd_ex": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _p, _sz, _p]),
    "linattn_fwd_ex_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _p]),
    "linattn_decode_step": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p]),
    "linattn_decode_step_ex": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p]),
    "linattn_bwd_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "linattn_fwd_vdecay_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "linattn_fwd_features_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "linattn_fwd_features": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _f, _p, _i,
                                  _p, _sz, _p]),
    "linattn_fwd_vdecay": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p, _sz, _p]),
    "linattn_decode_step_vdecay": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p]),
    "linattn_bwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _i, _p,
                         _sz, _p]),
    "linattn_status_string": (ctypes.c_char_p, [_i]),
    "linattn_set_profile_events": (_i, [_p, _p, _p, _p]),
}


def lib():
    """Load the library once; raise if it was not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m causal_kernelized_linear_amd.build`")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in EXPORTS.items():
                fn = getattr(h, name)
                fn.restype = res
                fn.argtypes = args
            _lib = h
        return _lib


def linattn_status_string(code: int) -> str:
    return lib().linattn_status_string(int(code)).decode()


def _check(code: int, what: str):
    if code != 0:
        raise RuntimeError(f"{what}: {linattn_status_string(code)} (status {code})")


def linattn_fwd_workspace_size(B, H, N, D, Dv, chunk) -> int:
    return int(lib().linattn_fwd_workspace_size(B, H, N, D, Dv, chunk))


def linattn_fwd_chunked(q, k, v, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, ws, ws_bytes,
                        stream) -> int:
    """Raw C call with integer pointers (0 = NULL); returns the status code."""
    return int(lib().linattn_fwd_chunked(q, k, v, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, ws,
                                         ws_bytes, stream))


def linattn_fwd_gated(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, ws, ws_bytes,
                      stream) -> int:
    return int(lib().linattn_fwd_gated(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, ws,
                                       ws_bytes, stream))


def linattn_fwd_ex(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, out, ws, ws_bytes,
                   stream) -> int:
    return int(lib().linattn_fwd_ex(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, out, ws,
                                    ws_bytes, stream))


def linattn_fwd_ex_noalloc(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, out,
                           stream) -> int:
    return int(lib().linattn_fwd_ex_noalloc(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps,
                                            out, stream))


def linattn_decode_step(q, k, v, S, z, o, B, H, D, Dv, dtype, eps, stream) -> int:
    return int(lib().linattn_decode_step(q, k, v, S, z, o, B, H, D, Dv, dtype, eps, stream))


def linattn_decode_step_ex(q, k, v, g, S, z, o, B, H, D, Dv, dtype, eps, out, stream) -> int:
    return int(lib().linattn_decode_step_ex(q, k, v, g, S, z, o, B, H, D, Dv, dtype, eps, out, stream))


def linattn_bwd_workspace_size(B, H, N, D, Dv, dtype) -> int:
    return int(lib().linattn_bwd_workspace_size(B, H, N, D, Dv, dtype))


def linattn_bwd(q, k, v, g, dout, s0, z0, dq, dk, dv, dg, ds0, dz0, B, H, N, D, Dv, dtype, eps, out, run, ws,
                ws_bytes, stream) -> int:
    return int(lib().linattn_bwd(q, k, v, g, dout, s0, z0, dq, dk, dv, dg, ds0, dz0, B, H, N, D, Dv, dtype, eps, out,
                                 run, ws, ws_bytes, stream))


def linattn_fwd_vdecay_workspace_size(B, H, N, D, Dv) -> int:
    return int(lib().linattn_fwd_vdecay_workspace_size(B, H, N, D, Dv))


def linattn_fwd_vdecay(q, k, v, a, o, s0, z0, s_out, z_out, B, H, N, D, Dv, dtype, eps, out, ws, ws_bytes,
                       stream) -> int:
    return int(lib().linattn_fwd_vdecay(q, k, v, a, o, s0, z0, s_out, z_out, B, H, N, D, Dv, dtype, eps, out, ws,
                                        ws_bytes, stream))


def linattn_decode_step_vdecay(q, k, v, a, S, z, o, B, H, D, Dv, dtype, eps, out, stream) -> int:
    return int(lib().linattn_decode_step_vdecay(q, k, v, a, S, z, o, B, H, D, Dv, dtype, eps, out, stream))


def linattn_fwd_features_workspace_size(B, H, N, D, Dv, chunk, M, dtype) -> int:
    return int(lib().linattn_fwd_features_workspace_size(B, H, N, D, Dv, chunk, M, dtype))


def linattn_fwd_features(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, out, feature, shift,
                         W, M, ws, ws_bytes, stream) -> int:
    return int(lib().linattn_fwd_features(q, k, v, g, o, s0, z0, s_out, z_out, B, H, N, D, Dv, chunk, dtype, eps, out,
                                          feature, shift, W, M, ws, ws_bytes, stream))


def linattn_set_profile_events(ev0, ev1, ev2, ev3) -> int:
    """Arm the measurement hook with raw hipEvent_t handles (ints; 0 is not recorded, all 0 disarms)."""
    return int(lib().linattn_set_profile_events(ev0, ev1, ev2, ev3))


# ------------------------------------------------------------ tensor level ----

def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _need(t, name, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def workspace_bytes(B, H, N, D, Dv, chunk) -> int:
    return linattn_fwd_workspace_size(B, H, N, D, Dv, chunk)


def _fwd(q, k, v, g, chunk, eps, s0, z0, return_state, out, workspace, normalize=True):
    dt = _dtype_code(q)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype, dev)
    for t, n in ((g, "g"), (s0, "s0"), (z0, "z0")):
        _need(t, n, torch.float32, dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, D]")
    B, H, N, D = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("k must match q, and v must be [B, H, N, Dv]")
    if g is not None and tuple(g.shape) != (B, H, N):
        raise ValueError("g must be [B, H, N]")
    if s0 is not None and tuple(s0.shape) != (B, H, D, Dv):
        raise ValueError("s0 must be [B, H, D, Dv]")
    if z0 is not None and tuple(z0.shape) != (B, H, D):
        raise ValueError("z0 must be [B, H, D]")
    o = torch.empty(B, H, N, Dv, dtype=q.dtype, device=dev) if out is None else out
    s_out = z_out = None
    if return_state:
        s_out = torch.empty(B, H, D, Dv, dtype=torch.float32, device=dev)
        z_out = torch.empty(B, H, D, dtype=torch.float32, device=dev)
    nbytes = linattn_fwd_workspace_size(B, H, N, D, Dv, chunk)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small")
    wsb = workspace.numel() * workspace.element_size()
    st = _stream(dev)
    if not normalize:
        code = linattn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), _ptr(s0), _ptr(z0), _ptr(s_out),
                              _ptr(z_out), B, H, N, D, Dv, chunk, dt, eps, OUT_NUMERATOR, _ptr(workspace), wsb, st)
        _check(code, "linattn_fwd_ex")
    elif g is None:
        code = linattn_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(s0), _ptr(z0), _ptr(s_out),
                                   _ptr(z_out), B, H, N, D, Dv, chunk, dt, eps, _ptr(workspace), wsb, st)
        _check(code, "linattn_fwd_chunked")
    else:
        code = linattn_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), _ptr(s0), _ptr(z0), _ptr(s_out),
                                 _ptr(z_out), B, H, N, D, Dv, chunk, dt, eps, _ptr(workspace), wsb, st)
        _check(code, "linattn_fwd_gated")
    if return_state:
        return o, s_out, z_out
    return o


def fwd_chunked(q, k, v, chunk=128, eps=1e-6, s0=None, z0=None, return_state=False, out=None, workspace=None):
    """Causal kernelized linear attention forward, chunked.  q, k [B,H,N,D]; v [B,H,N,Dv]
    (bf16 or fp32, on the GPU).  Returns o (and S_N, z_N when return_state)."""
    return _fwd(q, k, v, None, chunk, eps, s0, z0, return_state, out, workspace)


def fwd_gated(q, k, v, g, chunk=128, eps=1e-6, s0=None, z0=None, return_state=False, out=None, workspace=None):
    """Scalar-gated forward; g [B,H,N] float32 in (0, 1]."""
    if g is None:
        raise ValueError("fwd_gated needs g")
    return _fwd(q, k, v, g, chunk, eps, s0, z0, return_state, out, workspace)


def fwd(q, k, v, g=None, chunk=128, eps=1e-6, s0=None, z0=None, return_state=False, out=None, workspace=None,
        normalize=True):
    """The general forward (linattn_fwd_ex): optional gate g [B,H,N] float32, and
    ``normalize=False`` for the normaliser-free output o = phi(q)^T S."""
    return _fwd(q, k, v, g, chunk, eps, s0, z0, return_state, out, workspace, normalize)


def fwd_vdecay(q, k, v, a, eps=1e-6, s0=None, z0=None, return_state=False, out=None, workspace=None, normalize=True):
    """Per-dimension decay forward (linattn_fwd_vdecay): a [B,H,N,D] float32 in [2^-8, 1]."""
    dt = _dtype_code(q)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype, dev)
    for t, n in ((a, "a"), (s0, "s0"), (z0, "z0")):
        _need(t, n, torch.float32, dev)
    if q.dim() != 4 or a is None or tuple(a.shape) != tuple(q.shape):
        raise ValueError("q must be [B, H, N, D] and a of the same shape")
    B, H, N, D = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("k must match q, and v must be [B, H, N, Dv]")
    o = torch.empty(B, H, N, Dv, dtype=q.dtype, device=dev) if out is None else out
    s_out = z_out = None
    if return_state:
        s_out = torch.empty(B, H, D, Dv, dtype=torch.float32, device=dev)
        z_out = torch.empty(B, H, D, dtype=torch.float32, device=dev)
    nbytes = linattn_fwd_vdecay_workspace_size(B, H, N, D, Dv)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small")
    code = linattn_fwd_vdecay(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(o), _ptr(s0), _ptr(z0), _ptr(s_out),
                              _ptr(z_out), B, H, N, D, Dv, dt, eps, OUT_NORMALIZED if normalize else OUT_NUMERATOR,
                              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(code, "linattn_fwd_vdecay")
    if return_state:
        return o, s_out, z_out
    return o


def fwd_features(q, k, v, feature, shift=0.0, W=None, g=None, chunk=128, eps=1e-6, s0=None, z0=None,
                 return_state=False, out=None, workspace=None, normalize=True, s_out=None, z_out=None):
    """Forward under another feature map (linattn_fwd_features): feature "relu" (max(x, 0) +
    shift) or "favor" (W [H, M, D] float32 random features).  The state has M rows."""
    dt = _dtype_code(q)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype, dev)
    for t, n in ((g, "g"), (s0, "s0"), (z0, "z0"), (W, "W"), (s_out, "s_out"), (z_out, "z_out")):
        _need(t, n, torch.float32, dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, D]")
    B, H, N, D = q.shape
    Dv = v.shape[-1]
    kind = {"relu": FEATURE_RELU, "favor": FEATURE_FAVOR}[feature]
    if kind == FEATURE_FAVOR and (W is None or W.dim() != 3 or W.shape[0] != H or W.shape[2] != D):
        raise ValueError("favor needs W [H, M, D]")
    M = W.shape[1] if kind == FEATURE_FAVOR else D
    o = torch.empty(B, H, N, Dv, dtype=q.dtype, device=dev) if out is None else out
    if return_state and s_out is None:
        s_out = torch.empty(B, H, M, Dv, dtype=torch.float32, device=dev)
        z_out = torch.empty(B, H, M, dtype=torch.float32, device=dev)
    nbytes = linattn_fwd_features_workspace_size(B, H, N, D, Dv, chunk, M, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small")
    code = linattn_fwd_features(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), _ptr(s0), _ptr(z0), _ptr(s_out),
                                _ptr(z_out), B, H, N, D, Dv, chunk, dt, eps,
                                OUT_NORMALIZED if normalize else OUT_NUMERATOR, kind, shift,
                                _ptr(W) if kind == FEATURE_FAVOR else 0, M, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev))
    _check(code, "linattn_fwd_features")
    if return_state:
        return o, s_out, z_out
    return o


def decode_step_features(q, k, v, S, z, feature, shift=0.0, W=None, g=None, eps=1e-6, normalize=True):
    """One decode step under another feature map: linattn_fwd_features over one token with
    the state (S [B,H,M,Dv], z [B,H,M]) as both its initial and its final state, updated
    in place.  q, k [B,H,D], v [B,H,Dv]; g [B,H] or None.  Returns o [B,H,Dv]."""
    o = fwd_features(q.unsqueeze(2), k.unsqueeze(2), v.unsqueeze(2), feature, shift=shift, W=W,
                     g=None if g is None else g.unsqueeze(2).contiguous(), chunk=64, eps=eps, s0=S, z0=z, s_out=S,
                     z_out=z, normalize=normalize)
    return o[:, :, 0]


def bwd(q, k, v, dout, g=None, s0=None, z0=None, eps=1e-6, normalize=True, state_grads=False, workspace=None,
        grads=None, run=0):
    """Gradients of sum(dout * o) for o = fwd(q, k, v, g, s0=s0, z0=z0, eps=eps, normalize=normalize).
    Returns a dict with dq, dk, dv, dg (None when ungated) and, with ``state_grads``, ds0
    and dz0.  ``grads`` may hold preallocated dq, dk, dv, dg tensors; ``run`` is the
    chunks per run (0: the library's choice)."""
    dt = _dtype_code(q)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, n, q.dtype, dev)
    for t, n in ((g, "g"), (s0, "s0"), (z0, "z0")):
        _need(t, n, torch.float32, dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, D]")
    B, H, N, D = q.shape
    Dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or dout.shape != v.shape:
        raise ValueError("k must match q; v and dout must be [B, H, N, Dv]")
    if g is not None and tuple(g.shape) != (B, H, N):
        raise ValueError("g must be [B, H, N]")
    grads = dict(grads or {})
    dq = grads.get("dq") if grads.get("dq") is not None else torch.empty_like(q)
    dk = grads.get("dk") if grads.get("dk") is not None else torch.empty_like(k)
    dv = grads.get("dv") if grads.get("dv") is not None else torch.empty_like(v)
    dg = None
    if g is not None:
        dg = grads.get("dg") if grads.get("dg") is not None else torch.empty_like(g)
    ds0 = dz0 = None
    if state_grads:
        ds0 = torch.empty(B, H, D, Dv, dtype=torch.float32, device=dev)
        dz0 = torch.empty(B, H, D, dtype=torch.float32, device=dev)
    nbytes = linattn_bwd_workspace_size(B, H, N, D, Dv, dt)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small")
    code = linattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dout), _ptr(s0), _ptr(z0), _ptr(dq), _ptr(dk), _ptr(dv),
                       _ptr(dg), _ptr(ds0), _ptr(dz0), B, H, N, D, Dv, dt, eps,
                       OUT_NORMALIZED if normalize else OUT_NUMERATOR, int(run), _ptr(workspace),
                       workspace.numel() * workspace.element_size(), _stream(dev))
    _check(code, "linattn_bwd")
    return {"dq": dq, "dk": dk, "dv": dv, "dg": dg, "ds0": ds0, "dz0": dz0}


def decode_step(q, k, v, S, z, eps=1e-6, out=None, g=None, normalize=True, a=None):
    """One decode step: q, k [B,H,D], v [B,H,Dv]; S [B,H,D,Dv] and z [B,H,D] (float32)
    are updated in place.  g [B,H] float32 gates the state first (S <- g S + ...), or a
    [B,H,D] float32 decays each of its rows (S <- Diag(a) S + ...); with
    ``normalize=False`` the output is the numerator and z may be None.  Returns o [B,H,Dv]."""
    dt = _dtype_code(q)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, n, q.dtype, dev)
    _need(S, "S", torch.float32, dev)
    _need(z, "z", torch.float32, dev)
    _need(g, "g", torch.float32, dev)
    if q.dim() != 3:
        raise ValueError("q must be [B, H, D]")
    B, H, D = q.shape
    Dv = v.shape[-1]
    if tuple(S.shape) != (B, H, D, Dv) or k.shape != q.shape or (z is not None and tuple(z.shape) != (B, H, D)):
        raise ValueError("shape mismatch")
    if g is not None and tuple(g.shape) != (B, H):
        raise ValueError("g must be [B, H]")
    _need(a, "a", torch.float32, dev)
    if a is not None and (tuple(a.shape) != (B, H, D) or g is not None):
        raise ValueError("a must be [B, H, D], and not given with g")
    if z is None and normalize:
        raise ValueError("the normalised output needs z")
    o = torch.empty(B, H, Dv, dtype=q.dtype, device=dev) if out is None else out
    if a is not None:
        code = linattn_decode_step_vdecay(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(S), _ptr(z), _ptr(o), B, H, D, Dv,
                                          dt, eps, OUT_NORMALIZED if normalize else OUT_NUMERATOR, _stream(dev))
        _check(code, "linattn_decode_step_vdecay")
    elif g is None and normalize:
        code = linattn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z), _ptr(o), B, H, D, Dv, dt, eps,
                                   _stream(dev))
        _check(code, "linattn_decode_step")
    else:
        code = linattn_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S), _ptr(z), _ptr(o), B, H, D, Dv, dt,
                                      eps, OUT_NORMALIZED if normalize else OUT_NUMERATOR, _stream(dev))
        _check(code, "linattn_decode_step_ex")
    return o
