"""Causal linear attention (elu+1 kernel, per-head decay, gated delta rule)
on MI355X: a thin Python binding over the C-ABI library liblinattn.so.

Only argument marshalling happens here; every step of the computation runs
in the HIP kernels behind include/linattn.h.  PyTorch supplies device memory
and the current stream.  There is no fallback: if the library is missing or
a tensor is not on a GPU, the call raises.

    o, S, z = prefill(q, k, v, gamma=gamma, eps=1e-6)       # LINEAR, elu+1
    o, S, _ = prefill(q, k, v, rule="delta", g=g)             # gated delta
    o, S, _ = prefill(q, k, v, rule="delta", g=g, alpha=a)    # with decay
    o = decode_step(q1, k1, v1, S, z)                         # in place on S, z
    o, S, z = prefill(q, k, v, conv_weight=W, conv_cache=C)   # short conv; C in place
    o = decode_step(q1, k1, v1, S, z, conv_weight=W, conv_cache=C)
    o, S, z = prefill(q, k, v, den_out=den)                   # keep den for training
    dq, dk, dv, dS0, dz0 = backward(q, k, v, o, den, do)      # gradients
    dq, dk, dv, dg, da, dS0 = delta_backward(q, k, v, g, do, alpha=a)
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import LinattnError, LibraryMissing  # noqa: F401

__all__ = ["prefill", "decode_step", "backward", "delta_backward",
           "delta_backward_workspace_size", "state_init",
           "workspace_size",
           "LinattnError", "LibraryMissing"]

_RULES = {"linear": _lib.LA_RULE_LINEAR, "delta": _lib.LA_RULE_DELTA}
_FMAPS = {"elu1": _lib.LA_FMAP_ELU1, "identity": _lib.LA_FMAP_IDENTITY}
_DTYPES = {torch.float32: _lib.LA_F32, torch.bfloat16: _lib.LA_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_gpu(*ts):
    for t in ts:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError("liblinattn works on GPU tensors only")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _need_f32(*ts):
    for t in ts:
        if t is not None and t.dtype != torch.float32:
            raise ValueError("gamma, g, alpha, states must be float32")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _conv_check(conv_weight, conv_cache, q, H, d, dv, cache_lead):
    """Shapes of the short-convolution filters [H, w, 2d+dv] and the conv
    cache [*cache_lead, w-1, 2d+dv]; returns w (0 without filters)."""
    if conv_weight is None:
        if conv_cache is not None:
            raise ValueError("conv_cache needs conv_weight")
        return 0
    if conv_weight.dim() != 3 or tuple(conv_weight.shape[::2]) != (H, 2 * d + dv):
        raise ValueError(f"conv_weight must be [H, w, 2d+dv] = [{H}, w, {2 * d + dv}]")
    w = conv_weight.shape[1]
    if conv_cache is not None:
        want = (*cache_lead, w - 1, 2 * d + dv)
        if tuple(conv_cache.shape) != want or conv_cache.dtype != q.dtype:
            raise ValueError(f"conv_cache must be {list(want)} of dtype {q.dtype}")
    return w


def _prefill_args(q, k, v, rule, fmap, gamma, g, eps, alpha=None):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,N,d] and v [B,H,N,dv]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, H, N, d = q.shape
    a = _lib.PrefillArgs()
    a.B, a.H, a.N, a.d, a.dv = B, H, N, d, v.shape[3]
    a.dtype = _DTYPES[q.dtype]
    a.rule = _RULES[rule]
    a.fmap = _FMAPS[fmap]
    a.gamma = _ptr(gamma)
    a.g = _ptr(g)
    a.alpha = _ptr(alpha)
    a.eps = float(eps)
    return a


def workspace_size(q, k, v, *, rule="linear", fmap=None, gamma=None, g=None,
                   eps=1e-6, alpha=None, conv_weight=None, den_out=None):
    """Workspace bytes la_prefill needs for these tensors (current device);
    den_out: the denominators tensor the call will write, if any."""
    if fmap is None:
        fmap = "elu1" if rule == "linear" else "identity"
    a = _prefill_args(q, k, v, rule, fmap, gamma, g, eps, alpha)
    if conv_weight is not None:
        a.conv_weight, a.conv_width = _ptr(conv_weight), conv_weight.shape[1]
    a.den_out = _ptr(den_out)
    n = _lib.load().la_prefill_workspace_size(ctypes.byref(a))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes")
    return int(n)


def prefill(q, k, v, *, rule="linear", fmap=None, gamma=None, g=None, eps=1e-6,
            S_in=None, z_in=None, S_out=None, z_out=None, return_state=True,
            o=None, workspace=None, alpha=None, conv_weight=None, conv_cache=None,
            conv_cache_out=None, den_out=None, noalloc=False):
    """Chunked prefill over [B,H,N,*] sequences (see la_prefill).

    rule "linear": fmap defaults to "elu1"; gamma [H] fp32 or None; eps >= 0;
                   or, instead of gamma, alpha [B,H,N,d] fp32: a decay per key
                   channel and token in (0, 1] (taken as 2^-15 below it).  Optionally a short causal
                   convolution of q, k, v: conv_weight [H, w, 2d+dv] fp32
                   (w <= 4) and conv_cache [B,H,w-1,2d+dv] (dtype of q), read
                   as the tokens before the sequence and overwritten in place
                   with the last w-1 tokens (None: zeros before, not kept),
                   or, with conv_cache_out, written there instead.
                   den_out [B,H,N] fp32 receives each token's denominator
                   (the input of backward()).
    rule "delta":  fmap "identity"; g [B,H,N] fp32 required; alpha [B,H,N]
                   fp32 state decay in (0, 1] or None.
    noalloc=True calls la_prefill_noalloc: the library's static device
    scratch replaces the workspace (none may be passed), so the call itself
    allocates nothing beyond the outputs made here when not given.
    Returns (o, S_out, z_out); the states are None unless requested
    (return_state) or passed in.  z_out is always None for "delta".
    """
    if fmap is None:
        fmap = "elu1" if rule == "linear" else "identity"
    _need_gpu(q, k, v, gamma, g, alpha, S_in, z_in, S_out, z_out, o, workspace,
              conv_weight, conv_cache, conv_cache_out, den_out)
    _need_f32(gamma, g, alpha, S_in, z_in, S_out, z_out, conv_weight, den_out)
    if den_out is not None and tuple(den_out.shape) != tuple(q.shape[:3]):
        raise ValueError("den_out must be [B,H,N]")
    if alpha is not None:
        want = q.shape if rule == "linear" else q.shape[:3]
        if tuple(alpha.shape) != tuple(want):
            raise ValueError(f"alpha must be {list(want)} for rule {rule!r}")
    a = _prefill_args(q, k, v, rule, fmap, gamma, g, eps, alpha)
    B, H, N, d = q.shape
    dv = v.shape[3]
    w = _conv_check(conv_weight, conv_cache, q, H, d, dv, (B, H))
    if conv_cache_out is not None:
        _conv_check(conv_weight, conv_cache_out, q, H, d, dv, (B, H))
    if w:
        a.conv_weight, a.conv_width = _ptr(conv_weight), w
        a.conv_in = _ptr(conv_cache)
        a.conv_out = _ptr(conv_cache if conv_cache_out is None else conv_cache_out)
    if o is None:
        o = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    if return_state and S_out is None:
        S_out = torch.empty((B, H, d, dv), dtype=torch.float32, device=q.device)
    if return_state and z_out is None and rule == "linear":
        z_out = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    a.S_in, a.z_in = _ptr(S_in), _ptr(z_in)
    a.S_out, a.z_out = _ptr(S_out), _ptr(z_out)
    a.q, a.k, a.v, a.o = _ptr(q), _ptr(k), _ptr(v), _ptr(o)
    a.den_out = _ptr(den_out)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        _lib.check(lib.la_prefill_noalloc(ctypes.byref(a), _stream()), "la_prefill_noalloc")
        return o, S_out, z_out
    need = lib.la_prefill_workspace_size(ctypes.byref(a))
    if need == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes")
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    _lib.check(lib.la_prefill(ctypes.byref(a), _stream()), "la_prefill")
    return o, S_out, z_out


def _conv_grads(a, conv_weight, conv_cache, dconv_cache_out, conv_cache_grad, q, H, d, dv,
                lead):
    """Fill the convolution fields of backward arguments; returns (dW, dC)."""
    w = _conv_check(conv_weight, conv_cache, q, H, d, dv, lead)
    if dconv_cache_out is not None:
        _conv_check(conv_weight, dconv_cache_out, q, H, d, dv, lead)
    if not w:
        return None, None
    dW = torch.empty_like(conv_weight)
    dC = None
    if conv_cache_grad and w > 1:
        dC = torch.empty((*lead, w - 1, 2 * d + dv), dtype=q.dtype, device=q.device)
    a.conv_weight, a.conv_width, a.conv_in = _ptr(conv_weight), w, _ptr(conv_cache)
    a.grad_conv_out, a.grad_conv_weight, a.grad_conv_in = _ptr(dconv_cache_out), _ptr(dW), \
        _ptr(dC)
    return dW, dC


def backward(q, k, v, o, den, do, *, fmap="elu1", gamma=None, S_in=None, z_in=None,
             dS_out=None, dz_out=None, state_grad=True, workspace=None,
             fwd_workspace=None, conv_weight=None, conv_cache=None, dconv_cache_out=None,
             conv_cache_grad=True, alpha=None):
    """Gradients of a LINEAR prefill (see la_backward): q, k [B,H,N,d], v, o,
    do [B,H,N,dv] (dtype of q), den [B,H,N] fp32 from prefill(den_out=...);
    gamma, S_in, z_in as in the forward; dS_out [B,H,d,dv], dz_out [B,H,d]
    the gradient with respect to the final state, or None.
    fwd_workspace: the workspace the forward prefill ran with (prefill's
    workspace=, same inputs), whose segment states are then reused.
    conv_weight, conv_cache: the forward's short convolution (q, k, v raw);
    dconv_cache_out: dL/d(the conv cache it returned), or None.
    alpha: the forward's per-key-channel decay [B,H,N,d] fp32 (instead of
    gamma), or None.
    Returns (dq, dk, dv, dS_in, dz_in); the last two are None unless
    state_grad; with a convolution also (dconv_weight, dconv_cache) (the
    latter None unless conv_cache_grad and w > 1); with alpha, dalpha
    [B,H,N,d] fp32 last."""
    _need_gpu(q, k, v, o, den, do, gamma, S_in, z_in, dS_out, dz_out, workspace, fwd_workspace,
              conv_weight, conv_cache, dconv_cache_out, alpha)
    _need_f32(den, gamma, S_in, z_in, dS_out, dz_out, conv_weight, alpha)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,N,d] and v [B,H,N,dv]")
    if o.shape != v.shape or do.shape != v.shape or tuple(den.shape) != tuple(q.shape[:3]):
        raise ValueError("o, do must be [B,H,N,dv] and den [B,H,N]")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == do.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v, o, do must share dtype float32 or bfloat16")
    B, H, N, d = q.shape
    dv = v.shape[3]
    a = _lib.BackwardArgs()
    a.B, a.H, a.N, a.d, a.dv = B, H, N, d, dv
    a.dtype = _DTYPES[q.dtype]
    a.fmap = _FMAPS[fmap]
    dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dS_in = dz_in = None
    if state_grad:
        dS_in = torch.empty((B, H, d, dv), dtype=torch.float32, device=q.device)
        dz_in = torch.empty((B, H, d), dtype=torch.float32, device=q.device)
    a.q, a.k, a.v, a.o, a.den, a.grad_o = (_ptr(t) for t in (q, k, v, o, den, do))
    a.gamma, a.S_in, a.z_in = _ptr(gamma), _ptr(S_in), _ptr(z_in)
    a.grad_S_out, a.grad_z_out = _ptr(dS_out), _ptr(dz_out)
    a.grad_q, a.grad_k, a.grad_v = _ptr(dq), _ptr(dk), _ptr(dvv)
    a.grad_S_in, a.grad_z_in = _ptr(dS_in), _ptr(dz_in)
    dal = None
    if alpha is not None:
        if tuple(alpha.shape) != tuple(q.shape):
            raise ValueError("alpha must be [B,H,N,d]")
        dal = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        a.alpha, a.grad_alpha = _ptr(alpha), _ptr(dal)
    dW, dC = _conv_grads(a, conv_weight, conv_cache, dconv_cache_out, conv_cache_grad, q, H, d,
                         dv, (B, H))
    if fwd_workspace is not None:
        a.fwd_workspace = _ptr(fwd_workspace)
        a.fwd_workspace_bytes = fwd_workspace.numel() * fwd_workspace.element_size()
    lib = _lib.load()
    need = lib.la_backward_workspace_size(ctypes.byref(a))
    if need == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes")
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    _lib.check(lib.la_backward(ctypes.byref(a), _stream()), "la_backward")
    out = (dq, dk, dvv, dS_in, dz_in)
    if conv_weight is not None:
        out += (dW, dC)
    return out + (dal,) if alpha is not None else out


def delta_backward_workspace_size(q, k, v, conv_weight=None):
    """Workspace bytes la_delta_backward needs for these tensors."""
    B, H, N, d = q.shape
    a = _lib.DeltaBackwardArgs()
    a.B, a.H, a.N, a.d, a.dv = B, H, N, d, v.shape[3]
    a.dtype = _DTYPES[q.dtype]
    if conv_weight is not None:
        a.conv_weight, a.conv_width = _ptr(conv_weight), conv_weight.shape[1]
        a.grad_conv_weight = a.conv_weight  # (only whether it is set is read)
    n = _lib.load().la_delta_backward_workspace_size(ctypes.byref(a))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes")
    return int(n)


def delta_backward(q, k, v, g, do, *, alpha=None, S_in=None, dS_out=None, state_grad=True,
                   workspace=None, conv_weight=None, conv_cache=None, dconv_cache_out=None,
                   conv_cache_grad=True):
    """Gradients of a gated-delta prefill (see la_delta_backward): q, k
    [B,H,N,d], v, do [B,H,N,dv] (bf16), g and alpha [B,H,N] fp32 (alpha
    None: no decay), S_in [B,H,d,dv] the forward's initial state, dS_out
    the gradient with respect to the final state (or None); conv_weight,
    conv_cache, dconv_cache_out as in backward().
    Returns (dq, dk, dv, dg, dalpha, dS_in); dalpha is None without a decay,
    dS_in None unless state_grad; with a convolution also (dconv_weight,
    dconv_cache)."""
    _need_gpu(q, k, v, g, do, alpha, S_in, dS_out, workspace, conv_weight, conv_cache,
              dconv_cache_out)
    _need_f32(g, alpha, S_in, dS_out, conv_weight)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,H,N,d] and v [B,H,N,dv]")
    if do.shape != v.shape or tuple(g.shape) != tuple(q.shape[:3]):
        raise ValueError("do must be [B,H,N,dv] and g [B,H,N]")
    if alpha is not None and tuple(alpha.shape) != tuple(q.shape[:3]):
        raise ValueError("alpha must be [B,H,N]")
    if not (q.dtype == k.dtype == v.dtype == do.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v, do must share dtype float32 or bfloat16")
    B, H, N, d = q.shape
    dv = v.shape[3]
    a = _lib.DeltaBackwardArgs()
    a.B, a.H, a.N, a.d, a.dv = B, H, N, d, dv
    a.dtype = _DTYPES[q.dtype]
    dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    da = None if alpha is None else torch.empty_like(dg)
    dS_in = torch.empty((B, H, d, dv), dtype=torch.float32, device=q.device) if state_grad \
        else None
    a.q, a.k, a.v, a.g, a.alpha, a.S_in = (_ptr(t) for t in (q, k, v, g, alpha, S_in))
    a.grad_o, a.grad_S_out = _ptr(do), _ptr(dS_out)
    a.grad_q, a.grad_k, a.grad_v, a.grad_g = _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(dg)
    a.grad_alpha, a.grad_S_in = _ptr(da), _ptr(dS_in)
    dW, dC = _conv_grads(a, conv_weight, conv_cache, dconv_cache_out, conv_cache_grad, q, H, d,
                         dv, (B, H))
    lib = _lib.load()
    need = lib.la_delta_backward_workspace_size(ctypes.byref(a))
    if need == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes")
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    _lib.check(lib.la_delta_backward(ctypes.byref(a), _stream()), "la_delta_backward")
    if conv_weight is not None:
        return dq, dk, dvv, dg, da, dS_in, dW, dC
    return dq, dk, dvv, dg, da, dS_in


def decode_step(q, k, v, S, z=None, *, rule="linear", fmap=None, gamma=None,
                g=None, eps=1e-6, o=None, alpha=None, conv_weight=None, conv_cache=None):
    """One token per sequence: q, k [B,H,d], v [B,H,dv]; S [B,H,d,dv] (and z
    [B,H,d] for "linear") are updated in place; "delta" takes g [B,H] and
    an optional decay alpha [B,H]; "linear" an optional per-channel decay
    alpha [B,H,d] instead of gamma, and an optional short convolution
    (conv_weight [H, w, 2d+dv], conv_cache [B,H,w-1,2d+dv] shifted in
    place).  Returns o [B,H,dv]."""
    if fmap is None:
        fmap = "elu1" if rule == "linear" else "identity"
    _need_gpu(q, k, v, S, z, gamma, g, alpha, o, conv_weight, conv_cache)
    _need_f32(S, z, gamma, g, alpha, conv_weight)
    if q.dim() != 3 or k.shape != q.shape or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B,H,d] and v [B,H,dv]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, H, d = q.shape
    dv = v.shape[2]
    if S.shape != (B, H, d, dv) or (z is not None and z.shape != (B, H, d)):
        raise ValueError("state shape mismatch")
    if alpha is not None:
        want = (B, H, d) if rule == "linear" else (B, H)
        if tuple(alpha.shape) != want:
            raise ValueError(f"alpha must be {list(want)} for rule {rule!r}")
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    a = _lib.DecodeArgs()
    a.B, a.H, a.d, a.dv = B, H, d, dv
    a.dtype = _DTYPES[q.dtype]
    a.rule = _RULES[rule]
    a.fmap = _FMAPS[fmap]
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.gamma, a.g, a.alpha = _ptr(gamma), _ptr(g), _ptr(alpha)
    a.eps = float(eps)
    a.S, a.z, a.o = _ptr(S), _ptr(z), _ptr(o)
    w = _conv_check(conv_weight, conv_cache, q, H, d, dv, (B, H))
    if w:
        a.conv_weight, a.conv_width, a.conv_cache = _ptr(conv_weight), w, _ptr(conv_cache)
    _lib.check(_lib.load().la_decode_step(ctypes.byref(a), _stream()),
               "la_decode_step")
    return o


def state_init(S, z=None):
    """Zero a state in place on the current stream (fill kernel)."""
    _need_gpu(S, z)
    _need_f32(S, z)
    B, H, d, dv = S.shape
    _lib.check(_lib.load().la_state_init(_ptr(S), _ptr(z), B, H, d, dv, _stream()),
               "la_state_init")
    return S, z
