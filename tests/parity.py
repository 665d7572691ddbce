"""Comparison helpers for the GPU-vs-oracle parity tests.

Error metric (one reading, stated once): for outputs, the largest over
output rows (one token of one head, length dv) of
    max_c |o_gpu - o_ref| / max_c |o_ref|;
for states, the same over (b, h) blocks of S (d x dv) and z (d).  Rows whose
reference is exactly zero are compared absolutely.  Elementwise relative
error is not used: outputs are weighted averages of zero-mean values and
single elements can sit arbitrarily close to zero.  For the same reason a
row's scale is floored at a quarter of the median row norm of the tensor:
with a very small dv (2 or 3 values per row) a whole row of a weighted
average can cancel to near zero while the bf16 rounding of the weights
stays proportional to the values being averaged.  With dv >= 16 the floor
does not bind in practice.
"""
import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def row_rel_err(got, ref, axes=(-1,), floor=True):
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows = all axes but
    `axes`); with `floor`, a row's scale is at least a quarter of the median
    row scale (see the module docstring), without it the plain metric."""
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    diff = np.abs(g - r).max(axis=axes)
    scale = np.abs(r).max(axis=axes)
    if floor:
        scale = np.maximum(scale, 0.25 * np.median(scale))
    scale = np.where(scale > 0, scale, 1.0)
    return float((diff / scale).max())


def assert_close(got, ref, tol, what="", axes=(-1,), floor=True):
    """Row-relative parity at `tol`.  floor=False judges every row by its own
    scale only (the floor is not applied at all)."""
    e = row_rel_err(got, ref, axes, floor)
    print(f"[parity] {what}: {e:.3e} (tol {tol:.0e}{'' if floor else ', no floor'})",
          flush=True)
    assert e <= tol, f"{what}: max row-relative error {e:.3e} > {tol:.1e}"
    return e


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
