"""Plain fp64 CPU oracle for causal linear attention and the gated delta rule.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the test suite, the package smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP
library and imports nothing from it.

Everything here is deliberately slow and literal: a Python loop over tokens,
each step written as the pages write the recurrence, in float64 NumPy.
Inputs are upcast exactly (bf16 and fp32 values are representable in fp64),
so the oracle evaluates the method on the very values the GPU consumes.

Sources (cited by page title and section):
  [WILA]  "What Is Linear Attention?" (xutianle.me): section 2 (kernel trick,
          S and z), section 4 (causal recurrence), 5.1 (gamma decay),
          5.2 (delta rule), 5.3 (gate), 5.4 (short convolution, conv
          cache).
  [EAV]   "Efficient attention variants" (bailixisu.com): section 4 (kernel
          form, elu+1), section 5 (causal prefix form, write-then-read),
          5.1 (hand-worked example), 7.1 (RetNet decay), 7.3 (DeltaNet),
          7.4 (Gated DeltaNet: scalar decay before the delta correction),
          section 10 (NumPy self-check: dense vs recurrent).
  [LIO3]  "LLM inference optimisation (3): Linear Attention" (wangyu.me):
          'recurrent form of the summary', 'implementation', 'delta rule'
          (with its gating variant).
  [TAR]   "Transformers Are RNNs" (myhz0606.com): epsilon in the
          denominator, multiplicative causal mask.

Readings where the pages disagree:
  * The state is read AFTER the current token is written (token attends to
    itself), as [WILA] section 4 and [EAV] section 5 state.
  * eps is added to the denominator: o = phi(q).S / (phi(q).z + eps).
  * gamma decays both S and z.
  * The delta rule uses the raw k and q (no feature map, no normaliser), the
    prediction is S^T k with S stored [r, dv], the gate scales the write, and
    the output is read from the updated state: o_t = S_t^T q_t.
  * The optional decay alpha_t of the delta rule is a scalar per token and
    head, applied to the old state before the prediction ([EAV] 7.4 warns
    that the error must be taken on the decayed state).
  * The short convolution of [WILA] 5.4 is depthwise (one filter per head
    and channel), causal, over the w most recent tokens including the
    current one, with no bias and no activation; it is applied to the raw
    q, k and v before the feature map, and its cache holds the last w-1
    raw tokens.

Parity pins live in tests/test_oracle.py; every function below is pinned
there against printed values, closed forms or brute force.
"""
from __future__ import annotations

import numpy as np

FMAP_IDENTITY = "identity"
FMAP_ELU1 = "elu1"


def _f64(x):
    """Exact upcast of a NumPy / torch (CPU) array to float64."""
    if hasattr(x, "detach"):  # torch tensor: go through float32 exactly
        x = x.detach().to("cpu")
        import torch

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def phi_elu1(x):
    """elu(x) + 1 with alpha = 1.

    [EAV] section 4 names elu(x)+1 as the positive feature map of the Linear
    Transformer; its section-10 program evaluates it as max(x,0) +
    exp(min(x,0)) so that no large positive exponent is formed.  For x > 0
    this is x + 1, for x <= 0 it is e^x (so phi(0) = 1).
    """
    x = _f64(x)
    return np.maximum(x, 0.0) + np.exp(np.minimum(x, 0.0))


def feature_map(x, fmap):
    """phi applied elementwise.  IDENTITY means the inputs already are the
    non-negative features ([EAV] 5.1 gives its example features directly)."""
    if fmap == FMAP_ELU1:
        return phi_elu1(x)
    if fmap == FMAP_IDENTITY:
        return _f64(x)
    raise ValueError(f"unknown feature map {fmap!r}")


def _gamma_heads(gamma, H):
    """Per-head decay as a float64 vector of length H (None means 1)."""
    if gamma is None:
        return np.ones(H, dtype=np.float64)
    g = _f64(gamma).reshape(-1)
    if g.shape[0] != H:
        raise ValueError("gamma must have one value per head")
    return g


# ---------------------------------------------------------------------------
# LINEAR rule (elu+1 kernel, optional per-head decay, eps-stabilised normaliser)
# ---------------------------------------------------------------------------

def _row_decay(dec, S):
    """A decay as one factor per state row: [...] (per head) is broadcast
    over the r rows; [..., r] (per key channel) is used as is."""
    return dec[..., None] if dec.ndim == S.ndim - 2 else dec


def linear_step(S, z, fq, fk, v, gamma_bh, eps):
    """One token of causal linear attention, on features already mapped.

    S: [..., r, dv], z: [..., r], fq, fk: [..., r], v: [..., dv],
    gamma_bh: [...] (decay per leading index) or [..., r] (one decay per key
    channel, GLA).  Returns (o, S_new, z_new).

    State update ([WILA] section 4 with the decay of 5.1, applied to S and z):
        S_t = gamma * S_{t-1} + phi(k_t) v_t^T
        z_t = gamma * z_{t-1} + phi(k_t)
    With a per-channel decay alpha_t ([EAV] 7.2, GLA: each entry keeps its
    own state row, broadcast along the value axis) gamma becomes diag(alpha_t)
    on the rows of S and elementwise on z.
    Read after the write ([EAV] section 5: write first, then read, so the
    token attends to itself), with eps in the denominator ([TAR]):
        o_t = phi(q_t)^T S_t / (phi(q_t) . z_t + eps)
    """
    dec = _row_decay(gamma_bh, S)
    S_new = dec[..., :, None] * S + fk[..., :, None] * v[..., None, :]
    z_new = dec * z + fk
    num = np.einsum("...r,...rd->...d", fq, S_new)
    den = np.einsum("...r,...r->...", fq, z_new) + eps
    return num / den[..., None], S_new, z_new


def linear_prefill(q, k, v, *, gamma=None, eps=1e-6, fmap=FMAP_ELU1,
                   S0=None, z0=None, alpha=None):
    """Causal linear attention over a whole sequence, token by token.

    q, k: [B, H, N, d]; v: [B, H, N, dv]; gamma: [H] or None; alpha: [B, H,
    N, d] per-channel decay or None (not together with gamma); S0: [B, H, d,
    dv] or None (zero state); z0: [B, H, d] or None.
    Returns (o [B, H, N, dv], S_N [B, H, d, dv], z_N [B, H, d]) in float64.
    """
    if alpha is not None and gamma is not None:
        raise ValueError("gamma and alpha are alternatives")
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    fq, fk = feature_map(q, fmap), feature_map(k, fmap)
    gam = np.broadcast_to(_gamma_heads(gamma, H)[None, :], (B, H))
    S = np.zeros((B, H, d, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros((B, H, d)) if z0 is None else _f64(z0).copy()
    o = np.empty((B, H, N, dv))
    al = None if alpha is None else _f64(alpha)
    for t in range(N):
        o[:, :, t], S, z = linear_step(S, z, fq[:, :, t], fk[:, :, t],
                                       v[:, :, t], gam if al is None else al[:, :, t],
                                       eps)
    return o, S, z


def linear_decode_step(q, k, v, S, z, *, gamma=None, eps=1e-6, fmap=FMAP_ELU1,
                       alpha=None):
    """One decode step against a persistent state: the same token body as
    the prefill ([LIO3] 'recurrent form': read once, add once per token).

    q, k: [B, H, d]; v: [B, H, dv]; S: [B, H, d, dv]; z: [B, H, d];
    alpha: [B, H, d] per-channel decay or None (not together with gamma).
    Returns (o [B, H, dv], S_new, z_new); the inputs are not modified.
    """
    if alpha is not None and gamma is not None:
        raise ValueError("gamma and alpha are alternatives")
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H = q.shape[:2]
    gam = np.broadcast_to(_gamma_heads(gamma, H)[None, :], (B, H))
    if alpha is not None:
        gam = _f64(alpha)
    return linear_step(_f64(S), _f64(z), feature_map(q, fmap),
                       feature_map(k, fmap), v, gam, eps)


def linear_quadratic(q, k, v, *, gamma=None, eps=1e-6, fmap=FMAP_ELU1):
    """The O(N^2) masked matrix form, zero initial state.

    A = (phi(Q) phi(K)^T) (.) D with D_ij = gamma^(i-j) for j <= i and 0
    otherwise (the multiplicative causal mask of [TAR], with the unrolled
    RetNet decay of [EAV] 7.1); O = (A V) / (A 1 + eps), as in the dense
    function of [EAV] section 10 (which has no eps).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, _ = q.shape
    gam = _gamma_heads(gamma, H)
    fq, fk = feature_map(q, fmap), feature_map(k, fmap)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    lag = np.where(i >= j, i - j, 0)
    D = np.where(i >= j, gam[:, None, None] ** lag[None], 0.0)  # [H, N, N]
    A = np.matmul(fq, np.swapaxes(fk, -1, -2)) * D[None]
    return np.matmul(A, v) / (A.sum(axis=-1, keepdims=True) + eps)


# ---------------------------------------------------------------------------
# Backward pass of the LINEAR rule (training)
# ---------------------------------------------------------------------------

def phi_elu1_grad(x):
    """Derivative of elu(x)+1: 1 above zero, e^x at or below (1 at 0 from
    both sides)."""
    x = _f64(x)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def feature_map_grad(x, fmap):
    if fmap == FMAP_ELU1:
        return phi_elu1_grad(x)
    if fmap == FMAP_IDENTITY:
        return np.ones_like(_f64(x))
    raise ValueError(f"unknown feature map {fmap!r}")


def linear_denominators(q, k, *, gamma=None, eps=1e-6, fmap=FMAP_ELU1, z0=None, alpha=None):
    """den_t = phi(q_t) . z_t + eps of every token (what the output of the
    LINEAR rule divides by), with z_t = gamma z_(t-1) + phi(k_t), or with a
    per-channel decay z_t = alpha_t * z_(t-1) + phi(k_t).
    q, k: [B, H, N, d]; alpha [B, H, N, d] or None.  Returns [B, H, N] in
    float64."""
    if alpha is not None and gamma is not None:
        raise ValueError("gamma and alpha are alternatives")
    q, k = _f64(q), _f64(k)
    B, H, N, d = q.shape
    fq, fk = feature_map(q, fmap), feature_map(k, fmap)
    gam = np.broadcast_to(_gamma_heads(gamma, H)[None, :], (B, H))
    al = None if alpha is None else _f64(alpha)
    z = np.zeros((B, H, d)) if z0 is None else _f64(z0).copy()
    den = np.empty((B, H, N))
    for t in range(N):
        z = (gam[..., None] if al is None else al[:, :, t]) * z + fk[:, :, t]
        den[:, :, t] = np.einsum("...r,...r->...", fq[:, :, t], z) + eps
    return den


def linear_backward(q, k, v, do, *, gamma=None, eps=1e-6, fmap=FMAP_ELU1,
                    S0=None, z0=None, dS_N=None, dz_N=None, alpha=None):
    """Gradients of the LINEAR rule's prefill, token by token in reverse.

    The pages motivate parallel training ([WILA] 8, [EAV] 8 and 10) but give
    no gradient formulas; this is reverse-mode differentiation of the
    recurrence of linear_step, written out.  With S_t, z_t the state after
    token t, den_t = phi(q_t).z_t + eps and g_t = dL/do_t:
        dnum_t = g_t / den_t,   dden_t = -(g_t . o_t) / den_t
        dphi(q_t) = S_t dnum_t + z_t dden_t
    and, with the adjoints Sh_t = dL/dS_t, zh_t = dL/dz_t (all later tokens
    and the final-state gradient included),
        Sh_t = phi(q_t) dnum_t^T + gamma Sh_(t+1),   zh_t = phi(q_t) dden_t + gamma zh_(t+1)
        dphi(k_t) = Sh_t v_t + zh_t,   dv_t = Sh_t^T phi(k_t)
        dS_in = gamma Sh_0 (the gradient of the initial state; tokens count
        from 0), dz_in likewise,
    then dq = dphi(q) * phi'(q), dk = dphi(k) * phi'(k).  With a per-channel
    decay alpha_t ([EAV] 7.2, GLA) in place of gamma, S_t = diag(alpha_t)
    S_(t-1) + phi(k_t) v_t^T: the adjoint is carried back through
    diag(alpha_t) instead of gamma, and
        dalpha_t[f] = sum_c Sh_t[f, c] S_(t-1)[f, c] + zh_t[f] z_(t-1)[f]
    (S_(-1) = S0: the state the decay multiplies).

    q, k: [B, H, N, d]; v, do: [B, H, N, dv]; gamma [H] or None; alpha [B, H,
    N, d] or None (not together with gamma); S0, z0 the initial state or
    None; dS_N [B, H, d, dv], dz_N [B, H, d] the gradient of the loss with
    respect to the final state, or None.
    Returns (dq, dk, dv, dS_0, dz_0), and dalpha [B, H, N, d] after them when
    alpha is given, in float64.
    """
    if alpha is not None and gamma is not None:
        raise ValueError("gamma and alpha are alternatives")
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    dv_ = v.shape[-1]
    fq, fk = feature_map(q, fmap), feature_map(k, fmap)
    gam = np.broadcast_to(_gamma_heads(gamma, H)[None, :], (B, H))
    al = None if alpha is None else _f64(alpha)
    S = np.zeros((B, H, d, dv_)) if S0 is None else _f64(S0).copy()
    z = np.zeros((B, H, d)) if z0 is None else _f64(z0).copy()
    Ss, zs = [S], [z]  # the state before token 0, then after every token
    for t in range(N):  # forward pass, keeping every state
        _, S, z = linear_step(S, z, fq[:, :, t], fk[:, :, t], v[:, :, t],
                              gam if al is None else al[:, :, t], eps)
        Ss.append(S)
        zs.append(z)
    Sh = np.zeros((B, H, d, dv_)) if dS_N is None else _f64(dS_N).copy()
    zh = np.zeros((B, H, d)) if dz_N is None else _f64(dz_N).copy()
    dfq = np.empty((B, H, N, d))
    dfk = np.empty((B, H, N, d))
    dvv = np.empty((B, H, N, dv_))
    dal = None if al is None else np.empty((B, H, N, d))
    for t in range(N - 1, -1, -1):
        St, zt, fqt = Ss[t + 1], zs[t + 1], fq[:, :, t]
        num = np.einsum("...r,...rd->...d", fqt, St)
        den = np.einsum("...r,...r->...", fqt, zt) + eps
        g = do[:, :, t]
        dnum = g / den[..., None]
        dden = -np.einsum("...d,...d->...", g, num) / den ** 2
        dfq[:, :, t] = np.einsum("...rd,...d->...r", St, dnum) + zt * dden[..., None]
        Sh = Sh + fqt[..., :, None] * dnum[..., None, :]
        zh = zh + fqt * dden[..., None]
        dfk[:, :, t] = np.einsum("...rd,...d->...r", Sh, v[:, :, t]) + zh
        dvv[:, :, t] = np.einsum("...rd,...r->...d", Sh, fk[:, :, t])
        if al is None:
            Sh = gam[..., None, None] * Sh
            zh = gam[..., None] * zh
        else:
            dal[:, :, t] = np.einsum("...rd,...rd->...r", Sh, Ss[t]) + zh * zs[t]
            Sh = al[:, :, t][..., None] * Sh
            zh = al[:, :, t] * zh
    out = (dfq * feature_map_grad(q, fmap), dfk * feature_map_grad(k, fmap), dvv, Sh, zh)
    return out if al is None else out + (dal,)


# ---------------------------------------------------------------------------
# Short causal convolution before the attention ([WILA] 5.4)
# ---------------------------------------------------------------------------

def short_conv(x, weight, cache=None):
    """Depthwise causal convolution along the token axis.

    [WILA] 5.4 adds a short convolution over a window of the last w tokens in
    front of the linear state, and splits the inference cache into the
    recurrent state and a conv cache of the most recent tokens.  Read here as
    one length-w filter per head and channel, tap w-1 on the current token
    and tap j on the token w-1-j places back:
        y_t[c] = sum_{j=0..w-1} weight[h, j, c] * x_{t-(w-1)+j}[c]
    Tokens before the sequence come from the cache (oldest first), or are
    zero without one.

    x: [B, H, N, c]; weight: [H, w, c]; cache: [B, H, w-1, c] or None.
    Returns (y [B, H, N, c], cache after the last token [B, H, w-1, c]: the
    last w-1 raw tokens of cache followed by x), in float64.
    """
    x, W = _f64(x), _f64(weight)
    B, H, N, c = x.shape
    w = W.shape[1]
    hist = np.zeros((B, H, w - 1, c)) if cache is None else _f64(cache).copy()
    y = np.empty((B, H, N, c))
    for t in range(N):
        window = np.concatenate([hist, x[:, :, t:t + 1]], axis=2)  # oldest first
        y[:, :, t] = np.sum(window * W[None], axis=2)
        hist = window[:, :, 1:]
    return y, hist


def _conv_split(a, d):
    """Channels [q | k | v] of a conv weight or cache: d, d and the rest."""
    a = _f64(a)
    return a[..., :d], a[..., d:2 * d], a[..., 2 * d:]


def linear_prefill_conv(q, k, v, conv_weight, *, conv_cache=None, **kw):
    """Short convolution of q, k and v ([WILA] 5.4), then linear_prefill.

    conv_weight: [H, w, 2d + dv], channels [q | k | v]; conv_cache:
    [B, H, w-1, 2d + dv] raw tokens before the sequence, or None (zeros).
    Other keywords as linear_prefill.  Returns (o, S_N, z_N, conv cache
    after the last token [B, H, w-1, 2d + dv]).
    """
    d = q.shape[-1]
    wq, wk, wv = _conv_split(conv_weight, d)
    cq = ck = cv = None
    if conv_cache is not None:
        cq, ck, cv = _conv_split(conv_cache, d)
    yq, hq = short_conv(q, wq, cq)
    yk, hk = short_conv(k, wk, ck)
    yv, hv = short_conv(v, wv, cv)
    o, S, z = linear_prefill(yq, yk, yv, **kw)
    return o, S, z, np.concatenate([hq, hk, hv], axis=-1)


def linear_decode_step_conv(q, k, v, S, z, conv_weight, conv_cache, **kw):
    """One decode step with the short convolution: the new token joins the
    conv cache's window, the convolved q, k, v go through
    linear_decode_step.  q, k: [B, H, d]; v: [B, H, dv]; conv_cache:
    [B, H, w-1, 2d + dv].  Returns (o, S_new, z_new, conv cache after the
    token); the inputs are not modified."""
    d = q.shape[-1]
    wq, wk, wv = _conv_split(conv_weight, d)
    cq, ck, cv = _conv_split(conv_cache, d)
    yq, hq = short_conv(_f64(q)[:, :, None], wq, cq)
    yk, hk = short_conv(_f64(k)[:, :, None], wk, ck)
    yv, hv = short_conv(_f64(v)[:, :, None], wv, cv)
    o, S_new, z_new = linear_decode_step(yq[:, :, 0], yk[:, :, 0], yv[:, :, 0], S, z, **kw)
    return o, S_new, z_new, np.concatenate([hq, hk, hv], axis=-1)


def short_conv_backward(x, weight, dy, cache=None, dcache_out=None):
    """Gradients of short_conv: reverse mode of its two results, the outputs
    y_t[c] = sum_j weight[h, j, c] x~_(t+j)[c] over the sequence x~ = [cache |
    x] (cache rows oldest first, zeros without one) and the returned cache,
    the last w-1 rows of x~.  The pages give the convolution but no gradient
    formulas ([WILA] 5.4); this is the chain rule written out.

    dy: dL/dy [B, H, N, c]; dcache_out: dL/d(returned cache) [B, H, w-1, c]
    or None.  Returns (dx [B, H, N, c], dweight [H, w, c] (summed over the
    batch), dcache [B, H, w-1, c]) in float64.
    """
    x, W, dy = _f64(x), _f64(weight), _f64(dy)
    B, H, N, c = x.shape
    w = W.shape[1]
    hist = np.zeros((B, H, w - 1, c)) if cache is None else _f64(cache)
    full = np.concatenate([hist, x], axis=2)  # row r is token r - (w-1)
    dfull = np.zeros_like(full)
    dW = np.zeros((H, w, c))
    for t in range(N):
        for j in range(w):  # y_t reads full row t + j with tap j
            dfull[:, :, t + j] += W[None, :, j] * dy[:, :, t]
            dW[:, j] += np.sum(dy[:, :, t] * full[:, :, t + j], axis=0)
    if dcache_out is not None and w > 1:
        dfull[:, :, full.shape[2] - (w - 1):] += _f64(dcache_out)
    return dfull[:, :, w - 1:], dW, dfull[:, :, :w - 1]


def _conv_backward_qkv(q, k, v, W, cache, dy, dcache_out):
    """short_conv_backward on the channels [q | k | v]: (dq, dk, dv, dW, dcache)."""
    d = q.shape[-1]
    ws = _conv_split(W, d)
    cs = (None,) * 3 if cache is None else _conv_split(cache, d)
    dco = (None,) * 3 if dcache_out is None else _conv_split(dcache_out, d)
    out = [short_conv_backward(x, wx, g, cx, gx)
           for x, wx, g, cx, gx in zip((q, k, v), ws, dy, cs, dco)]
    return (out[0][0], out[1][0], out[2][0],
            np.concatenate([o[1] for o in out], axis=-1),
            np.concatenate([o[2] for o in out], axis=-1))


def linear_backward_conv(q, k, v, do, conv_weight, *, conv_cache=None, dconv_cache_out=None,
                         **kw):
    """Gradients of linear_prefill_conv: linear_backward on the convolved q,
    k, v, then the convolution's chain rule.  dconv_cache_out: dL/d(the conv
    cache it returns) or None.  Other keywords as linear_backward.  Returns
    (dq, dk, dv, dconv_weight [H, w, 2d+dv], dconv_cache [B, H, w-1, 2d+dv],
    dS_0, dz_0), and dalpha after them with a per-channel decay, in
    float64."""
    d = q.shape[-1]
    wq, wk, wv = _conv_split(conv_weight, d)
    cq = ck = cv = None
    if conv_cache is not None:
        cq, ck, cv = _conv_split(conv_cache, d)
    yq, _ = short_conv(q, wq, cq)
    yk, _ = short_conv(k, wk, ck)
    yv, _ = short_conv(v, wv, cv)
    gq, gk, gv, dS0, dz0, *dal = linear_backward(yq, yk, yv, do, **kw)
    dq, dk, dv, dW, dC = _conv_backward_qkv(q, k, v, conv_weight, conv_cache, (gq, gk, gv),
                                            dconv_cache_out)
    return (dq, dk, dv, dW, dC, dS0, dz0, *dal)


# ---------------------------------------------------------------------------
# Gated DELTA rule (raw q, k; no normaliser)
# ---------------------------------------------------------------------------

def delta_step(S, q, k, v, g, alpha=None):
    """One token of the gated delta rule.

    [WILA] 5.2-5.3: predict what the state already returns for this key,
    write only the residual, scaled by the write gate g_t:
        v_hat_t = S_{t-1}^T k_t            (S stored [r, dv])
        S_t     = S_{t-1} + g_t k_t (v_t - v_hat_t)^T
    The output is read from the updated state: o_t = S_t^T q_t.
    With a scalar decay alpha_t ([EAV] 7.4, Gated DeltaNet; [LIO3] 'delta
    rule', gating): the old state is decayed first and the prediction is
    taken from the decayed state,
        S_t = alpha_t S_{t-1} + g_t k_t (v_t - alpha_t S_{t-1}^T k_t)^T.
    alpha None means alpha_t = 1 (the plain gated delta rule).
    S: [..., d, dv]; q, k: [..., d]; v: [..., dv]; g, alpha: [...].
    """
    if alpha is not None:
        S = alpha[..., None, None] * S
    v_hat = np.einsum("...rd,...r->...d", S, k)
    S_new = S + g[..., None, None] * k[..., :, None] * (v - v_hat)[..., None, :]
    o = np.einsum("...rd,...r->...d", S_new, q)
    return o, S_new


def delta_prefill(q, k, v, g, *, S0=None, alpha=None):
    """Gated delta rule over a whole sequence, token by token.

    q, k: [B, H, N, d]; v: [B, H, N, dv]; g: [B, H, N]; alpha: [B, H, N] or
    None (no decay); S0: [B, H, d, dv] or None.  Returns (o [B, H, N, dv],
    S_N [B, H, d, dv]) in float64.
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    al = None if alpha is None else _f64(alpha)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, d, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((B, H, N, dv))
    for t in range(N):
        o[:, :, t], S = delta_step(S, q[:, :, t], k[:, :, t], v[:, :, t],
                                   g[:, :, t], None if al is None else al[:, :, t])
    return o, S


def delta_decode_step(q, k, v, g, S, alpha=None):
    """One decode step of the gated delta rule against a persistent state.

    q, k: [B, H, d]; v: [B, H, dv]; g, alpha: [B, H] (alpha None: no decay);
    S: [B, H, d, dv].  Returns (o [B, H, dv], S_new); S is not modified.
    """
    return delta_step(_f64(S), _f64(q), _f64(k), _f64(v), _f64(g),
                      None if alpha is None else _f64(alpha))


def delta_prefill_conv(q, k, v, g, conv_weight, *, conv_cache=None, S0=None, alpha=None):
    """Short convolution of q, k and v ([WILA] 5.4, which adds it in front of
    the linear layer beside Gamma, Delta and Gate), then delta_prefill on the
    convolved q, k, v.  The pages give no normalisation after the
    convolution, so none is applied: the rule sees the filters' outputs.

    conv_weight: [H, w, 2d + dv], channels [q | k | v]; conv_cache:
    [B, H, w-1, 2d + dv] raw tokens before the sequence, or None (zeros).
    Returns (o, S_N, conv cache after the last token [B, H, w-1, 2d + dv]).
    """
    d = q.shape[-1]
    wq, wk, wv = _conv_split(conv_weight, d)
    cq = ck = cv = None
    if conv_cache is not None:
        cq, ck, cv = _conv_split(conv_cache, d)
    yq, hq = short_conv(q, wq, cq)
    yk, hk = short_conv(k, wk, ck)
    yv, hv = short_conv(v, wv, cv)
    o, S = delta_prefill(yq, yk, yv, g, S0=S0, alpha=alpha)
    return o, S, np.concatenate([hq, hk, hv], axis=-1)


def delta_decode_step_conv(q, k, v, g, S, conv_weight, conv_cache, alpha=None):
    """One decode step of the gated delta rule behind the short convolution:
    the token joins the conv cache's window, the convolved q, k, v go through
    delta_decode_step.  q, k: [B, H, d]; v: [B, H, dv]; g, alpha: [B, H];
    conv_cache: [B, H, w-1, 2d + dv].  Returns (o, S_new, conv cache after
    the token); the inputs are not modified."""
    d = q.shape[-1]
    wq, wk, wv = _conv_split(conv_weight, d)
    cq, ck, cv = _conv_split(conv_cache, d)
    yq, hq = short_conv(_f64(q)[:, :, None], wq, cq)
    yk, hk = short_conv(_f64(k)[:, :, None], wk, ck)
    yv, hv = short_conv(_f64(v)[:, :, None], wv, cv)
    o, S_new = delta_decode_step(yq[:, :, 0], yk[:, :, 0], yv[:, :, 0], g, S, alpha=alpha)
    return o, S_new, np.concatenate([hq, hk, hv], axis=-1)


def delta_backward(q, k, v, g, do, *, alpha=None, S0=None, dS_N=None):
    """Gradients of the gated delta rule's prefill, token by token in reverse.

    The pages motivate parallel training ([WILA] 8, [EAV] 8 and 10) but give
    no gradient formulas; this is reverse-mode differentiation of delta_step,
    written out.  With a = alpha_t (1 without a decay), the forward step is
        S_t = a (I - g_t k_t k_t^T) S_{t-1} + g_t k_t v_t^T,   o_t = S_t^T q_t.
    With the adjoint Sh_t = dL/dS_t (all later tokens and the final-state
    gradient included), the residual u_t = v_t - a S_{t-1}^T k_t and
    w_t = Sh_t^T k_t:
        Sh_t   = q_t do_t^T + a_(t+1) (I - g_(t+1) k_(t+1) k_(t+1)^T) Sh_(t+1)
        dq_t   = S_t do_t
        dv_t   = g_t w_t
        dg_t   = w_t . u_t
        dk_t   = g_t Sh_t u_t - a g_t S_{t-1} w_t
        dalpha_t = <Sh_t, S_{t-1}> - g_t (S_{t-1}^T k_t) . w_t
    and the initial-state gradient is what the adjoint becomes before token
    0, a_0 (I - g_0 k_0 k_0^T) Sh_0.

    q, k: [B, H, N, d]; v, do: [B, H, N, dv]; g: [B, H, N]; alpha: [B, H, N]
    or None; S0: [B, H, d, dv] or None (zeros); dS_N: [B, H, d, dv] (the
    gradient with respect to the final state) or None (zero).
    Returns (dq, dk, dv, dg, dalpha, dS_0) in float64; dalpha is None
    without a decay.
    """
    q, k, v, g, do = _f64(q), _f64(k), _f64(v), _f64(g), _f64(do)
    al = None if alpha is None else _f64(alpha)
    B, H, N, d = q.shape
    dv_ = v.shape[-1]
    S = np.zeros((B, H, d, dv_)) if S0 is None else _f64(S0).copy()
    states = [S]  # states[t] = S_{t-1}, the state token t starts from
    for t in range(N):
        _, S = delta_step(S, q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t],
                          None if al is None else al[:, :, t])
        states.append(S)
    Sh = np.zeros((B, H, d, dv_)) if dS_N is None else _f64(dS_N).copy()
    dq = np.empty((B, H, N, d))
    dk = np.empty((B, H, N, d))
    dvv = np.empty((B, H, N, dv_))
    dg = np.empty((B, H, N))
    da = None if al is None else np.empty((B, H, N))
    for t in range(N - 1, -1, -1):
        qt, kt, vt, gt = q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t]
        a = np.ones((B, H)) if al is None else al[:, :, t]
        S_prev, S_t = states[t], states[t + 1]
        Sh = Sh + qt[..., :, None] * do[:, :, t][..., None, :]
        dq[:, :, t] = np.einsum("...rd,...d->...r", S_t, do[:, :, t])
        pred = np.einsum("...rd,...r->...d", S_prev, kt)  # S_{t-1}^T k_t
        u = vt - a[..., None] * pred
        w = np.einsum("...rd,...r->...d", Sh, kt)
        dvv[:, :, t] = gt[..., None] * w
        dg[:, :, t] = np.einsum("...d,...d->...", w, u)
        dk[:, :, t] = (gt[..., None] * np.einsum("...rd,...d->...r", Sh, u)
                       - (a * gt)[..., None] * np.einsum("...rd,...d->...r", S_prev, w))
        if da is not None:
            da[:, :, t] = (np.einsum("...rd,...rd->...", Sh, S_prev)
                           - gt * np.einsum("...d,...d->...", pred, w))
        Sh = a[..., None, None] * (Sh - gt[..., None, None] * kt[..., :, None] * w[..., None, :])
    return dq, dk, dvv, dg, da, Sh


def delta_backward_conv(q, k, v, g, do, conv_weight, *, conv_cache=None, dconv_cache_out=None,
                        alpha=None, S0=None, dS_N=None):
    """Gradients of delta_prefill_conv: delta_backward on the convolved q, k,
    v, then the convolution's chain rule.  Returns (dq, dk, dv, dg, dalpha,
    dconv_weight [H, w, 2d+dv], dconv_cache [B, H, w-1, 2d+dv], dS_0)."""
    d = q.shape[-1]
    wq, wk, wv = _conv_split(conv_weight, d)
    cq = ck = cv = None
    if conv_cache is not None:
        cq, ck, cv = _conv_split(conv_cache, d)
    yq, _ = short_conv(q, wq, cq)
    yk, _ = short_conv(k, wk, ck)
    yv, _ = short_conv(v, wv, cv)
    gq, gk, gv, dg, dal, dS0 = delta_backward(yq, yk, yv, g, do, alpha=alpha, S0=S0, dS_N=dS_N)
    dq, dk, dv, dW, dC = _conv_backward_qkv(q, k, v, conv_weight, conv_cache, (gq, gk, gv),
                                            dconv_cache_out)
    return dq, dk, dv, dg, dal, dW, dC, dS0
