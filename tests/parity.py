"""Comparison helpers for the GPU-vs-oracle parity tests.

Error metric (one reading, stated once): for outputs, the largest over
output rows (one token of one head, length dv) of
    max_c |o_gpu - o_ref| / max_c |o_ref|;
for states, the same over (b, h) blocks of S (d x dv) and z (d).  Rows whose
reference is exactly zero are compared absolutely.  Elementwise relative
error is not used: outputs are weighted averages of zero-mean values and
single elements can sit arbitrarily close to zero.  Where a whole row is a
sum that can cancel (a weighted average over 2 or 3 values per row, a
gradient made of terms of both signs) the row is judged against the sum of
its terms' magnitudes instead (assert_terms_close, assert_grad_close): the
rounding error of a sum is bounded by a multiple of that, not of the sum.
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def row_rel_err(got, ref, axes=(-1,)):
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows = all axes but
    `axes`)."""
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    diff = np.abs(g - r).max(axis=axes)
    scale = np.abs(r).max(axis=axes)
    scale = np.where(scale > 0, scale, 1.0)
    return float((diff / scale).max())


def assert_close(got, ref, tol, what="", axes=(-1,)):
    """Row-relative parity at `tol` (the plain metric above)."""
    e = row_rel_err(got, ref, axes)
    print(f"[parity] {what}: {e:.3e} (tol {tol:.0e})", flush=True)
    assert e <= tol, f"{what}: max row-relative error {e:.3e} > {tol:.1e}"
    return e


def assert_terms_close(got, ref, scale, tol, what=""):
    """Rows of a sum that can cancel: max over rows of max_c |got - ref| /
    max_c scale, with `scale` the per-element sum of the magnitudes of the
    terms (e.g. linear_output_scale)."""
    g, r, sc = f64(got), f64(ref), f64(scale)
    assert g.shape == r.shape == sc.shape, (g.shape, r.shape, sc.shape)
    if not np.all(np.isfinite(g)):
        e = float("inf")
    else:
        s = sc.max(axis=-1)
        e = float((np.abs(g - r).max(axis=-1) / np.where(s > 0, s, 1.0)).max())
    print(f"[parity] {what}: {e:.3e} (tol {tol:.0e}, vs |terms|)", flush=True)
    assert e <= tol, f"{what}: max error {e:.3e} of the terms' magnitude > {tol:.1e}"
    return e


def linear_output_scale(q, k, v, *, gamma=None, eps=1e-6, fmap="elu1", S0=None, z0=None):
    """Per-element sums of |terms| of the LINEAR rule's output o_t = num_t /
    den_t (fp64): (sum_j gamma^(t-j) (phi(q_t).phi(k_j)) |v_j| + gamma^(t+1)
    |phi(q_t)^T S0|) / den_t + |o_t|, the last term for the denominator's
    own rounding."""
    import oracle
    q, k, v = f64(q), f64(k), f64(v)
    B, H, N, d = q.shape
    fq, fk = oracle.feature_map(q, fmap), oracle.feature_map(k, fmap)
    gam = np.ones(H) if gamma is None else f64(gamma)
    o, _, _ = oracle.linear_prefill(q, k, v, gamma=gamma, eps=eps, fmap=fmap, S0=S0, z0=z0)
    den = oracle.linear_denominators(q, k, gamma=gamma, eps=eps, fmap=fmap, z0=z0)
    t = np.arange(N)
    lag = t[:, None] - t[None, :]
    sc = np.zeros_like(o)
    for b in range(B):
        for h in range(H):
            D = np.where(lag >= 0, gam[h] ** np.maximum(lag, 0), 0.0)
            A = (fq[b, h] @ fk[b, h].T) * D
            num = A @ np.abs(v[b, h])
            if S0 is not None:
                num += (gam[h] ** (t + 1.0))[:, None] * np.abs(fq[b, h] @ f64(S0)[b, h])
            sc[b, h] = num / den[b, h][:, None] + np.abs(o[b, h])
    return sc


def cpu(t):
    return None if t is None else t.detach().to("cpu")


def assert_grad_close(got, ref, scale, tol, what=""):
    """Gradients: max over rows of max_c |got - ref| / max_c scale, where
    `scale` holds, per element, the sum of the absolute values of the terms
    whose sum is the gradient (an element's rounding error is bounded by a
    multiple of that sum, not of the sum itself, which can cancel to nearly
    zero: with the normaliser, dq and dk are small differences of large
    terms)."""
    g, r, sc = f64(got), f64(ref), f64(scale)
    assert g.shape == r.shape == sc.shape, (g.shape, r.shape, sc.shape)
    if g.size == 0:
        e = 0.0
    elif not np.all(np.isfinite(g)):
        e = float("inf")
    else:
        diff = np.abs(g - r).max(axis=-1)
        s = sc.max(axis=-1)
        e = float((diff / np.where(s > 0, s, 1.0)).max())
    print(f"[parity] {what}: {e:.3e} (tol {tol:.0e}, vs |terms|)", flush=True)
    assert e <= tol, f"{what}: max error {e:.3e} of the terms' magnitude > {tol:.1e}"
    return e


def linear_grad_scales(q, k, v, do, o, den, *, gamma=None, fmap="elu1", S0=None, z0=None,
                       dS_N=None, dz_N=None):
    """Per-element sums of |terms| of dq, dk, dv, dS_in, dz_in for the LINEAR
    rule (fp64, from the oracle's o and den), over the whole sequence as one
    block, with |dA_tj| taken term by term (|g_t|.|v_j| + |g_t.o_t|) / den_t:
        dq_t ~ sum_j D_tj |dA_tj| |phi(k_j)| + gamma^(t+1) (|g_t| |S0| + |g.o| |z0|) / den_t
        dk_j ~ sum_t D_tj |dA_tj| |phi(q_t)| + gamma^(N-1-j) (|dS_N| |v_j| + |dz_N|)
        dv_j ~ sum_t D_tj A_tj |g_t| / den_t + gamma^(N-1-j) |dS_N|^T |phi(k_j)|
        dS_in ~ sum_t gamma^(t+1) |phi(q_t)| |g_t|^T / den_t + gamma^N |dS_N|
    Returns (sq, sk, sv, sS, sz) with the shapes of the gradients."""
    import oracle
    q, k, v, do, o, den = (f64(x) for x in (q, k, v, do, o, den))
    B, H, N, d = q.shape
    dv = v.shape[-1]
    fq, fk = oracle.feature_map(q, fmap), oracle.feature_map(k, fmap)
    gam = np.ones(H) if gamma is None else f64(gamma)
    t = np.arange(N)
    lag = t[:, None] - t[None, :]
    sq, sk = np.zeros_like(q), np.zeros_like(k)
    sv = np.zeros_like(v)
    sS = np.zeros((B, H, d, dv))
    sz = np.zeros((B, H, d))
    for b in range(B):
        for h in range(H):
            D = np.where(lag >= 0, gam[h] ** np.maximum(lag, 0), 0.0)
            g, rd = do[b, h], 1.0 / den[b, h]
            go = np.abs(np.sum(g * o[b, h], -1))
            dA = ((np.abs(g) @ np.abs(v[b, h]).T) + go[:, None]) * rd[:, None] * D
            A = (fq[b, h] @ fk[b, h].T) * D
            sq[b, h] = dA @ np.abs(fk[b, h])
            sk[b, h] = dA.T @ np.abs(fq[b, h])
            sv[b, h] = np.abs(A).T @ (np.abs(g) * rd[:, None])
            w = gam[h] ** (t + 1.0)
            sS[b, h] = (np.abs(fq[b, h]) * (w * rd)[:, None]).T @ np.abs(g)
            sz[b, h] = (np.abs(fq[b, h]) * (w * rd * go)[:, None]).sum(0)
            if S0 is not None:
                sq[b, h] += (w * rd)[:, None] * (np.abs(g) @ np.abs(f64(S0)[b, h]).T
                                                 + go[:, None] * np.abs(f64(z0)[b, h])[None, :])
            wl = gam[h] ** (N - 1.0 - t)
            if dS_N is not None:
                dS, dz = np.abs(f64(dS_N)[b, h]), np.abs(f64(dz_N)[b, h])
                sk[b, h] += wl[:, None] * (np.abs(v[b, h]) @ dS.T + dz[None, :])
                sv[b, h] += wl[:, None] * (np.abs(fk[b, h]) @ dS)
                sS[b, h] += gam[h] ** N * dS
                sz[b, h] += gam[h] ** N * dz
    return sq, sk, sv, sS, sz


def gla_grad_scales(q, k, v, do, o, den, alpha, *, fmap="elu1", S0=None, z0=None, dS_N=None,
                    dz_N=None):
    """Per-element sums of |terms| of dq, dk, dv, dS_in, dz_in and dalpha
    for the LINEAR rule with a per-channel decay alpha (fp64, from the
    oracle's o and den): every gradient is a sum of products of nonnegative
    magnitudes, so the same recurrences run on magnitudes give those sums:
        |S|_t = alpha_t |S|_(t-1) + |phi(k_t)| [|v_t| | 1]^T   ([S | z], from |S0|, |z0|)
        |Sh|_t = phi(q_t) |dn_t|^T + alpha_(t+1) |Sh|_(t+1)     (from |dS_N|, |dz_N|)
    with |dn_t| = [|g_t| | |g_t . o_t|] / den_t; then dq_t ~ |S|_t |dn_t|,
    dk_t ~ |Sh|_t [|v_t| | 1], dv_t ~ |Sh|_t^T |phi(k_t)|, d(S, z)_in ~
    alpha_0 |Sh|_0, dalpha_t ~ sum_c |Sh|_t |S|_(t-1)."""
    import oracle
    q, k, v, do, o, den, al = (f64(x) for x in (q, k, v, do, o, den, alpha))
    B, H, N, d = q.shape
    dv = v.shape[-1]
    fq, fk = np.abs(oracle.feature_map(q, fmap)), np.abs(oracle.feature_map(k, fmap))
    vp = np.concatenate([np.abs(v), np.ones((B, H, N, 1))], -1)
    dn = np.concatenate([np.abs(do), np.abs(np.sum(do * o, -1, keepdims=True))], -1) / \
        den[..., None]
    S = np.zeros((B, H, d, dv + 1))
    if S0 is not None:
        S[..., :dv] = np.abs(f64(S0))
    if z0 is not None:
        S[..., dv] = np.abs(f64(z0))
    Ss = [S]
    sq = np.empty((B, H, N, d))
    for t in range(N):
        S = al[:, :, t, :, None] * S + fk[:, :, t, :, None] * vp[:, :, t, None, :]
        Ss.append(S)
        sq[:, :, t] = np.einsum("bhfc,bhc->bhf", S, dn[:, :, t])
    Sh = np.zeros((B, H, d, dv + 1))
    if dS_N is not None:
        Sh[..., :dv] = np.abs(f64(dS_N))
    if dz_N is not None:
        Sh[..., dv] = np.abs(f64(dz_N))
    sk, sa = np.empty((B, H, N, d)), np.empty((B, H, N, d))
    sv = np.empty((B, H, N, dv))
    for t in range(N - 1, -1, -1):
        Sh = Sh + fq[:, :, t, :, None] * dn[:, :, t, None, :]
        sk[:, :, t] = np.einsum("bhfc,bhc->bhf", Sh, vp[:, :, t])
        sv[:, :, t] = np.einsum("bhfc,bhf->bhc", Sh[..., :dv], fk[:, :, t])
        sa[:, :, t] = np.sum(Sh * Ss[t], -1)
        Sh = al[:, :, t, :, None] * Sh
    return sq, sk, sv, Sh[..., :dv], Sh[..., dv], sa


def _delta_states(q, k, v, g, alpha, S0):
    """The states of the gated delta rule before every token and after the
    last (fp64, from the oracle's step), [B, H, N + 1, d, dv]."""
    import oracle
    q, k, v, g = f64(q), f64(k), f64(v), f64(g)
    al = None if alpha is None else f64(alpha)
    B, H, N, d = q.shape
    out = np.empty((B, H, N + 1, d, v.shape[-1]))
    out[:, :, 0] = 0.0 if S0 is None else f64(S0)
    for t in range(N):
        _, out[:, :, t + 1] = oracle.delta_step(out[:, :, t], q[:, :, t], k[:, :, t], v[:, :, t],
                                                g[:, :, t], None if al is None else al[:, :, t])
    return out


def delta_output_scale(q, k, v, g, alpha=None, S0=None):
    """Per-element |terms| of the gated delta rule's output o_t = S_t^T q_t:
    |S_t|^T |q_t|."""
    st = _delta_states(q, k, v, g, alpha, S0)
    return np.einsum("bhtrd,bhtr->bhtd", np.abs(st[:, :, 1:]), np.abs(f64(q)))


def delta_grad_scales(q, k, v, g, do, alpha=None, S0=None, dS_N=None):
    """Per-element |terms| of the gated delta rule's gradients (fp64), from
    the states S_(t-1), S_t and the adjoint Sh_t = dL/dS_t (a = alpha_t,
    u_t = v_t - a S_(t-1)^T k_t, w_t = Sh_t^T k_t):
        dq_t ~ |S_t| |do_t|,   dv_t ~ g_t |Sh_t|^T |k_t|,   dg_t ~ |w_t| . |u_t|,
        dk_t ~ g_t (|Sh_t| |u_t| + a |S_(t-1)| |w_t|),
        dalpha_t ~ <|Sh_t|, |S_(t-1)|> + g_t |S_(t-1)^T k_t| . |w_t|,
        dS_in ~ |Sh_0| + g_0 |k_0| |k_0|^T |Sh_0|  (times a_0).
    Returns (sq, sk, sv, sg, salpha, sS) shaped as the gradients."""
    q, k, v, g, do = f64(q), f64(k), f64(v), f64(g), f64(do)
    B, H, N, d = q.shape
    dv = v.shape[-1]
    al = np.ones((B, H, N)) if alpha is None else f64(alpha)
    st = _delta_states(q, k, v, g, alpha, S0)
    Sh = np.zeros((B, H, d, dv)) if dS_N is None else f64(dS_N).copy()
    sq, sk, sv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    sg, sa = np.zeros((B, H, N)), np.zeros((B, H, N))
    for t in range(N - 1, -1, -1):
        Sh = Sh + q[:, :, t, :, None] * do[:, :, t, None, :]
        kt, gt, at, Sp = k[:, :, t], g[:, :, t], al[:, :, t], st[:, :, t]
        pred = np.einsum("bhrd,bhr->bhd", Sp, kt)
        u = v[:, :, t] - at[..., None] * pred
        w = np.einsum("bhrd,bhr->bhd", Sh, kt)
        aSh, aSp = np.abs(Sh), np.abs(Sp)
        sq[:, :, t] = np.einsum("bhrd,bhd->bhr", np.abs(st[:, :, t + 1]), np.abs(do[:, :, t]))
        sv[:, :, t] = gt[..., None] * np.einsum("bhrd,bhr->bhd", aSh, np.abs(kt))
        sg[:, :, t] = np.einsum("bhd,bhd->bh", np.abs(w), np.abs(u))
        sk[:, :, t] = gt[..., None] * (np.einsum("bhrd,bhd->bhr", aSh, np.abs(u))
                                       + at[..., None] * np.einsum("bhrd,bhd->bhr", aSp,
                                                                   np.abs(w)))
        sa[:, :, t] = np.einsum("bhrd,bhrd->bh", aSh, aSp) + \
            gt * np.einsum("bhd,bhd->bh", np.abs(pred), np.abs(w))
        proj = np.einsum("bhr,bhrd->bhd", kt, Sh)
        if t == 0:  # the initial-state gradient's terms: a_0 (|Sh_0| + g_0 |k_0| |k_0|^T |Sh_0|)
            sS = at[..., None, None] * (aSh + gt[..., None, None] * np.abs(kt)[..., :, None] *
                                        np.einsum("bhr,bhrd->bhd", np.abs(kt), aSh)[..., None, :])
        Sh = at[..., None, None] * (Sh - gt[..., None, None] * kt[..., :, None] * proj[..., None, :])
    if N == 0:
        sS = np.abs(Sh)
    return sq, sk, sv, sg, sa, sS
