"""Pins for the fp64 oracle: each check compares the oracle with something
other than itself -- a value the pages print, a closed form, a library
routine, finite differences, or brute force on tiny inputs.

Every pin is a function of the oracle module, so tests/test_oracle.py runs
them on the real oracle and tests/test_oracle_mutations.py runs them on
deliberately broken copies to show that each plausible mistake is caught.
"""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bh(x):
    """Add leading batch and head axes of size 1."""
    return np.asarray(x, dtype=np.float64)[None, None]


# --- feature map -----------------------------------------------------------

def pin_phi_closed_form(orc):
    """elu(x)+1 with alpha = 1: x+1 above zero, e^x at or below zero,
    phi(0) = 1 (Efficient attention variants, section 4 and section 10)."""
    xs = [-30.0, -2.5, -1.0, -1e-3, 0.0, 1e-3, 0.5, 3.0, 1000.0]
    got = orc.phi_elu1(np.array(xs))
    want = [x + 1.0 if x > 0 else math.exp(x) for x in xs]
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)
    assert got[4] == 1.0


def pin_phi_matches_torch(orc):
    """Against a library routine: torch.nn.functional.elu (alpha=1) + 1."""
    import torch

    x = np.random.default_rng(7).normal(scale=3.0, size=4096)
    ref = (torch.nn.functional.elu(torch.from_numpy(x)) + 1.0).numpy()
    # torch forms expm1(x) + 1, which loses relative (not absolute) precision
    # for very negative x, hence the absolute floor.
    np.testing.assert_allclose(orc.phi_elu1(x), ref, rtol=1e-14, atol=1e-15)


# --- LINEAR rule -----------------------------------------------------------

def _handworked_inputs():
    g = _golden("handworked_example.json")
    fk = np.array(g["phi_k"], dtype=np.float64)
    v = np.array(g["v"], dtype=np.float64)
    # The page gives only phi(q3); the same query feature is used at every
    # position (a reading: the other two outputs are then derived by hand).
    fq = np.tile(np.array(g["phi_q3"], dtype=np.float64), (3, 1))
    return g, fq, fk, v


def pin_handworked_example(orc):
    """The printed example: three keys with similarities 1, 2, 3 to phi(q3),
    weights 1/6, 2/6, 3/6, output [10/6, 7/6]."""
    g, fq, fk, v = _handworked_inputs()
    o, S, z = orc.linear_prefill(_bh(fq), _bh(fk), _bh(v), eps=0.0,
                                 fmap=orc.FMAP_IDENTITY)
    np.testing.assert_allclose(o[0, 0, 2], g["o3"], rtol=1e-15)
    # the same value through the quadratic form, and its normalised weights
    oq = orc.linear_quadratic(_bh(fq), _bh(fk), _bh(v), eps=0.0,
                              fmap=orc.FMAP_IDENTITY)
    np.testing.assert_allclose(oq[0, 0, 2], g["o3"], rtol=1e-15)
    sims = fk @ np.array(g["phi_q3"], dtype=np.float64)
    np.testing.assert_allclose(sims, g["similarities_q3"])
    np.testing.assert_allclose(sims / sims.sum(), g["weights_q3"], rtol=1e-15)
    # With eps = 1e-6 the printed row moves by eps / den = 1e-6 / 6.
    o_eps, _, _ = orc.linear_prefill(_bh(fq), _bh(fk), _bh(v), eps=1e-6,
                                     fmap=orc.FMAP_IDENTITY)
    np.testing.assert_allclose(o_eps[0, 0, 2], g["o3"], rtol=2e-7)


def pin_handworked_derived_rows(orc):
    """Rows 1 and 2 worked out by hand from the same table (query feature
    [1,2] everywhere): o1 = v1 = [1,0]; o2 = (1*v1 + 2*v2)/3 = [1/3, 4/3].
    The final state is sum_j phi(k_j) v_j^T = [[4,1],[3,3]], z = [2,2]."""
    _, fq, fk, v = _handworked_inputs()
    o, S, z = orc.linear_prefill(_bh(fq), _bh(fk), _bh(v), eps=0.0,
                                 fmap=orc.FMAP_IDENTITY)
    np.testing.assert_allclose(o[0, 0, 0], [1.0, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 1], [1 / 3, 4 / 3], rtol=1e-15)
    np.testing.assert_allclose(S[0, 0], [[4, 1], [3, 3]], rtol=0, atol=0)
    np.testing.assert_allclose(z[0, 0], [2, 2], rtol=0, atol=0)


def _selfcheck_inputs():
    p = _golden("printed_values.json")["dense_vs_recurrent_selfcheck"]
    rng = np.random.default_rng(p["seed"])
    q = rng.normal(size=(p["N"], p["d"]))
    k = rng.normal(size=(p["N"], p["d"]))
    v = rng.normal(size=(p["N"], p["dv"]))
    return p, q, k, v


def _brute_linear(q, k, v, gamma, eps, phi):
    """The definition written out per output: o_i is the similarity-weighted
    average of v_j over j <= i, similarity gamma^(i-j) phi(q_i).phi(k_j),
    with eps added to the weight sum.  Pure Python loops, tiny inputs."""
    N, dv = v.shape
    out = np.zeros((N, dv))
    for i in range(N):
        num = [0.0] * dv
        den = 0.0
        for j in range(i + 1):
            s = sum(phi(q[i, a]) * phi(k[j, a]) for a in range(q.shape[1]))
            s *= gamma ** (i - j)
            den += s
            for c in range(dv):
                num[c] += s * v[j, c]
        out[i] = [x / (den + eps) for x in num]
    return out


def pin_selfcheck_dense_vs_recurrent(orc):
    """The page's own NumPy check: recurrence == masked quadratic form on
    N=17, d=4, dv=3 normal inputs from seed 42, to 1e-12 (printed max
    difference 4.44e-16)."""
    p, q, k, v = _selfcheck_inputs()
    rec, _, _ = orc.linear_prefill(_bh(q), _bh(k), _bh(v), eps=0.0)
    den = orc.linear_quadratic(_bh(q), _bh(k), _bh(v), eps=0.0)
    np.testing.assert_allclose(den, rec, rtol=p["rtol"], atol=p["atol"])
    assert np.max(np.abs(den - rec)) < 1e3 * p["printed_max_abs_error"]


def pin_brute_force_linear(orc):
    """Recurrence against the definition written out by brute force, with a
    per-head decay and eps, on tiny inputs with d != dv."""
    rng = np.random.default_rng(11)
    H, N, d, dv = 2, 9, 3, 5
    q = rng.normal(size=(1, H, N, d))
    k = rng.normal(size=(1, H, N, d))
    v = rng.normal(size=(1, H, N, dv))
    gam = np.array([1.0, 0.8])
    eps = 0.25
    o, _, _ = orc.linear_prefill(q, k, v, gamma=gam, eps=eps)
    phi = lambda x: x + 1.0 if x > 0 else math.exp(x)  # noqa: E731
    for h in range(H):
        ref = _brute_linear(q[0, h], k[0, h], v[0, h], gam[h], eps, phi)
        np.testing.assert_allclose(o[0, h], ref, rtol=1e-12, atol=1e-14)
    oq = orc.linear_quadratic(q, k, v, gamma=gam, eps=eps)
    np.testing.assert_allclose(oq, o, rtol=1e-12, atol=1e-14)


def pin_no_future_leakage(orc):
    """Changing k and v from token 8 on leaves outputs 0..7 unchanged and
    changes later outputs (Efficient attention variants, section 10)."""
    p, q, k, v = _selfcheck_inputs()
    t0 = p["perturb_from"]
    k2, v2 = k.copy(), v.copy()
    k2[t0:] += p["k_shift"]
    v2[t0:] += p["v_shift"]
    a, _, _ = orc.linear_prefill(_bh(q), _bh(k), _bh(v), eps=0.0)
    b, _, _ = orc.linear_prefill(_bh(q), _bh(k2), _bh(v2), eps=0.0)
    np.testing.assert_allclose(a[..., :t0, :], b[..., :t0, :], rtol=0,
                               atol=1e-12)
    assert np.all(np.abs(a[..., t0:, :] - b[..., t0:, :]).max(axis=-1) > 1e-3)


def pin_final_state_closed_form(orc):
    """At the end of the sequence S = phi(K)^T W V and z = phi(K)^T w with
    w_j = gamma^(N-1-j) (w = 1 without decay), computed with a library
    matmul; and the last output equals the non-causal reassociated form
    phi(q_N) (phi(K)^T V) / (phi(q_N) . sum_j phi(k_j))."""
    rng = np.random.default_rng(3)
    H, N, d, dv = 3, 40, 6, 4
    q = rng.normal(size=(2, H, N, d))
    k = rng.normal(size=(2, H, N, d))
    v = rng.normal(size=(2, H, N, dv))
    gam = np.array([1.0, 0.97, 0.5])
    o, S, z = orc.linear_prefill(q, k, v, gamma=gam, eps=0.0)
    fk = np.maximum(k, 0) + np.exp(np.minimum(k, 0))
    fq = np.maximum(q, 0) + np.exp(np.minimum(q, 0))
    for h in range(H):
        w = gam[h] ** np.arange(N - 1, -1, -1)
        for b in range(2):
            np.testing.assert_allclose(S[b, h], fk[b, h].T @ (w[:, None] * v[b, h]),
                                       rtol=1e-12)
            np.testing.assert_allclose(z[b, h], fk[b, h].T @ w, rtol=1e-12)
    # gamma = 1 head: the last row is the non-causal formula's last row
    St = fk[:, 0].transpose(0, 2, 1) @ v[:, 0]
    last = np.einsum("br,brd->bd", fq[:, 0, -1], St) / np.einsum(
        "br,br->b", fq[:, 0, -1], fk[:, 0].sum(axis=1))[:, None]
    np.testing.assert_allclose(o[:, 0, -1], last, rtol=1e-12)


def pin_gamma_one_is_plain(orc):
    """A decay of exactly 1 is the plain prefix sum."""
    rng = np.random.default_rng(5)
    q, k = rng.normal(size=(2, 1, 2, 12, 4))
    v = rng.normal(size=(1, 2, 12, 3))
    a = orc.linear_prefill(q, k, v, gamma=np.ones(2), eps=1e-6)
    b = orc.linear_prefill(q, k, v, gamma=None, eps=1e-6)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def pin_decay_printed_value(orc):
    """gamma = 0.99: a record written once weighs ~0.366 after 100 further
    steps (printed to three digits); S and z both decay."""
    p = _golden("printed_values.json")["decay_after_100_steps"]
    n = p["steps"] + 1
    k = np.zeros((1, 1, n, 1))
    v = np.zeros((1, 1, n, 1))
    k[0, 0, 0, 0] = 1.0
    v[0, 0, 0, 0] = 1.0
    q = np.ones((1, 1, n, 1))
    _, S, z = orc.linear_prefill(q, k, v, gamma=np.array([p["gamma"]]),
                                 eps=0.0, fmap=orc.FMAP_IDENTITY)
    half_ulp = 0.5 * 10.0 ** (-p["printed_digits"])
    assert abs(S[0, 0, 0, 0] - p["printed"]) <= half_ulp
    assert abs(z[0, 0, 0] - p["printed"]) <= half_ulp
    assert abs(S[0, 0, 0, 0] - 0.99 ** 100) < 1e-15


def pin_duplicate_key_linear(orc):
    """One unit key written with 2 then 5: unnormalised read 7, normalised
    read 3.5 (Efficient attention variants, section 7.3)."""
    p = _golden("printed_values.json")["duplicate_unit_key"]
    e1 = np.array([1.0, 0.0])
    k = np.stack([e1, e1])[None, None]
    v = np.array(p["values"], dtype=np.float64).reshape(1, 1, 2, 1)
    o, S, z = orc.linear_prefill(k, k, v, eps=0.0, fmap=orc.FMAP_IDENTITY)
    assert e1 @ S[0, 0, :, 0] == p["additive_read"]
    assert o[0, 0, 1, 0] == p["normalised_read"]


def pin_chunk_split_and_decode(orc):
    """Splitting the sequence and carrying (S, z) gives the same result, and
    a decode step after a prefill equals the next row of a longer prefill."""
    rng = np.random.default_rng(9)
    q = rng.normal(size=(2, 3, 20, 5))
    k = rng.normal(size=(2, 3, 20, 5))
    v = rng.normal(size=(2, 3, 20, 2))
    gam = np.array([0.9, 1.0, 0.6])
    o, S, z = orc.linear_prefill(q, k, v, gamma=gam, eps=1e-3)
    o1, S1, z1 = orc.linear_prefill(q[:, :, :7], k[:, :, :7], v[:, :, :7],
                                    gamma=gam, eps=1e-3)
    o2, S2, z2 = orc.linear_prefill(q[:, :, 7:19], k[:, :, 7:19], v[:, :, 7:19],
                                    gamma=gam, eps=1e-3, S0=S1, z0=z1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o[:, :, :19],
                               rtol=1e-12)
    od, Sd, zd = orc.linear_decode_step(q[:, :, 19], k[:, :, 19], v[:, :, 19],
                                        S2, z2, gamma=gam, eps=1e-3)
    np.testing.assert_allclose(od, o[:, :, 19], rtol=1e-12)
    np.testing.assert_allclose(Sd, S, rtol=1e-12)
    np.testing.assert_allclose(zd, z, rtol=1e-12)


# --- gated DELTA rule ------------------------------------------------------

def pin_duplicate_key_delta(orc):
    """Delta update with step 1 on a unit key written with 2 then 5 reads 5;
    a direction orthogonal to the key is untouched (section 7.3)."""
    p = _golden("printed_values.json")["duplicate_unit_key"]
    e1, e2 = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    S0 = np.array([[0.0], [4.0]])[None, None]  # something stored along e2
    k = np.stack([e1, e1])[None, None]
    v = np.array(p["values"], dtype=np.float64).reshape(1, 1, 2, 1)
    g = np.ones((1, 1, 2))
    o, S = orc.delta_prefill(k, k, v, g, S0=S0)
    assert e1 @ S[0, 0, :, 0] == p["delta_read"]
    assert o[0, 0, 1, 0] == p["delta_read"]
    assert e2 @ S[0, 0, :, 0] == 4.0


def pin_delta_gate_zero(orc):
    """g = 0 never writes: S stays S0 and every output is S0^T q_t; from a
    zero state every output is zero."""
    rng = np.random.default_rng(12)
    q = rng.normal(size=(1, 2, 10, 4))
    k = rng.normal(size=(1, 2, 10, 4))
    v = rng.normal(size=(1, 2, 10, 3))
    S0 = rng.normal(size=(1, 2, 4, 3))
    g = np.zeros((1, 2, 10))
    o, S = orc.delta_prefill(q, k, v, g, S0=S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, np.matmul(q, S0), rtol=1e-14)
    o0, S0b = orc.delta_prefill(q, k, v, g)
    assert not np.any(o0) and not np.any(S0b)


def pin_delta_first_token(orc):
    """From a zero state the first output is g (k . q) v (closed form)."""
    rng = np.random.default_rng(13)
    q, k = rng.normal(size=(2, 1, 1, 1, 6))
    v = rng.normal(size=(1, 1, 1, 4))
    g = np.array([[[0.3]]])
    o, _ = orc.delta_prefill(q, k, v, g)
    np.testing.assert_allclose(o[0, 0, 0], 0.3 * float(k[0, 0, 0] @ q[0, 0, 0])
                               * v[0, 0, 0], rtol=1e-14)


def pin_delta_gradient_step(orc):
    """One delta step is one gradient step of size g on the loss
    L(S) = 1/2 ||S^T k - v||^2 (section 7.3); the gradient is taken by
    central finite differences, independently of any formula."""
    rng = np.random.default_rng(14)
    d, dv = 5, 3
    S = rng.normal(size=(d, dv))
    k = rng.normal(size=d)
    v = rng.normal(size=dv)
    q = rng.normal(size=d)
    g = 0.37

    def loss(M):
        r = M.T @ k - v
        return 0.5 * float(r @ r)

    grad = np.zeros_like(S)
    h = 1e-5
    for a in range(d):
        for c in range(dv):
            Sp, Sm = S.copy(), S.copy()
            Sp[a, c] += h
            Sm[a, c] -= h
            grad[a, c] = (loss(Sp) - loss(Sm)) / (2 * h)
    _, S_new = orc.delta_decode_step(q[None, None], k[None, None],
                                     v[None, None], np.array([[g]]),
                                     S[None, None])
    np.testing.assert_allclose(S_new[0, 0], S - g * grad, rtol=1e-7, atol=1e-8)


def pin_delta_brute_force(orc):
    """Sequence against explicit matrix products S <- (I - g k k^T) S + g k v^T
    and o = S^T q on tiny inputs with d != dv."""
    rng = np.random.default_rng(15)
    N, d, dv = 11, 4, 6
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(N, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.normal(size=(N, dv))
    g = 1 / (1 + np.exp(-rng.normal(size=N)))
    S0 = rng.normal(size=(d, dv))
    S = S0.copy()
    ref = np.zeros((N, dv))
    eye = np.eye(d)
    for t in range(N):
        S = (eye - g[t] * np.outer(k[t], k[t])) @ S + g[t] * np.outer(k[t], v[t])
        ref[t] = S.T @ q[t]
    o, Sf = orc.delta_prefill(_bh(q), _bh(k), _bh(v), _bh(g), S0=_bh(S0))
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sf[0, 0], S, rtol=1e-12, atol=1e-13)


def pin_delta_split_and_decode(orc):
    """Sequence split with carried state, and decode after prefill."""
    rng = np.random.default_rng(16)
    q = rng.normal(size=(1, 2, 15, 4))
    k = rng.normal(size=(1, 2, 15, 4))
    v = rng.normal(size=(1, 2, 15, 5))
    g = rng.uniform(size=(1, 2, 15))
    o, S = orc.delta_prefill(q, k, v, g)
    o1, S1 = orc.delta_prefill(q[:, :, :6], k[:, :, :6], v[:, :, :6], g[:, :, :6])
    o2, S2 = orc.delta_prefill(q[:, :, 6:14], k[:, :, 6:14], v[:, :, 6:14],
                               g[:, :, 6:14], S0=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o[:, :, :14],
                               rtol=1e-12)
    od, Sd = orc.delta_decode_step(q[:, :, 14], k[:, :, 14], v[:, :, 14],
                                   g[:, :, 14], S2)
    np.testing.assert_allclose(od, o[:, :, 14], rtol=1e-12)
    np.testing.assert_allclose(Sd, S, rtol=1e-12)


# --- gated delta rule with a scalar decay (Gated DeltaNet) -----------------

def pin_gdn_matrix_form(orc):
    """Efficient attention variants 7.4 writes the decayed rule as
    S_t = alpha_t (I - g_t k_t k_t^T) S_{t-1} + g_t k_t v_t^T; explicit matrix
    products on tiny inputs (d != dv, alpha well away from 1) must match,
    outputs read from the updated state."""
    rng = np.random.default_rng(21)
    N, d, dv = 12, 4, 5
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(N, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.normal(size=(N, dv))
    g = 1 / (1 + np.exp(-rng.normal(size=N)))
    al = rng.uniform(0.3, 0.95, size=N)
    S0 = rng.normal(size=(d, dv))
    S = S0.copy()
    ref = np.zeros((N, dv))
    eye = np.eye(d)
    for t in range(N):
        S = al[t] * (eye - g[t] * np.outer(k[t], k[t])) @ S + g[t] * np.outer(k[t], v[t])
        ref[t] = S.T @ q[t]
    o, Sf = orc.delta_prefill(_bh(q), _bh(k), _bh(v), _bh(g), S0=_bh(S0), alpha=_bh(al))
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sf[0, 0], S, rtol=1e-12, atol=1e-13)


def pin_gdn_pure_decay(orc):
    """With g = 0 nothing is written: S_t = (alpha_1 ... alpha_t) S_0, so
    o_t = (prod alpha) S_0^T q_t (closed form)."""
    rng = np.random.default_rng(22)
    N, d, dv = 9, 3, 4
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(N, d))
    v = rng.normal(size=(N, dv))
    al = rng.uniform(0.5, 1.0, size=N)
    S0 = rng.normal(size=(d, dv))
    o, Sf = orc.delta_prefill(_bh(q), _bh(k), _bh(v), _bh(np.zeros(N)), S0=_bh(S0),
                              alpha=_bh(al))
    cum = np.cumprod(al)
    np.testing.assert_allclose(o[0, 0], cum[:, None] * (q @ S0), rtol=1e-13)
    np.testing.assert_allclose(Sf[0, 0], cum[-1] * S0, rtol=1e-13)


def pin_gdn_unit_key_overwrite(orc):
    """A unit key with g = 1 replaces what the decayed state holds for that
    key (the error is taken on the decayed state, Efficient attention
    variants 7.4): row 0 of S_t becomes v_t, the other rows only decay."""
    d, dv = 3, 2
    S0 = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    k = np.array([[1.0, 0.0, 0.0], [1.0, 0.0, 0.0]])
    v = np.array([[7.0, -1.0], [0.5, 8.0]])
    al = np.array([0.5, 0.25])
    o, Sf = orc.delta_prefill(_bh(k), _bh(k), _bh(v), _bh(np.ones(2)), S0=_bh(S0),
                              alpha=_bh(al))
    want = np.array([[0.5, 8.0], [3.0 * 0.125, 4.0 * 0.125], [5.0 * 0.125, 6.0 * 0.125]])
    np.testing.assert_allclose(Sf[0, 0], want, rtol=1e-15)
    np.testing.assert_allclose(o[0, 0], v, rtol=1e-15)  # q = e_1 reads row 0


def pin_gdn_alpha_one_and_split(orc):
    """alpha = 1 is the plain gated delta rule; with decay, a split sequence
    with carried state and a decode step after prefill give the same
    outputs and state."""
    rng = np.random.default_rng(23)
    q = rng.normal(size=(1, 2, 13, 4))
    k = rng.normal(size=(1, 2, 13, 4))
    v = rng.normal(size=(1, 2, 13, 3))
    g = rng.uniform(size=(1, 2, 13))
    al = rng.uniform(0.6, 1.0, size=(1, 2, 13))
    o_plain, S_plain = orc.delta_prefill(q, k, v, g)
    o_one, S_one = orc.delta_prefill(q, k, v, g, alpha=np.ones((1, 2, 13)))
    np.testing.assert_allclose(o_one, o_plain, rtol=1e-14)
    np.testing.assert_allclose(S_one, S_plain, rtol=1e-14)
    o, S = orc.delta_prefill(q, k, v, g, alpha=al)
    o1, S1 = orc.delta_prefill(q[:, :, :5], k[:, :, :5], v[:, :, :5], g[:, :, :5],
                               alpha=al[:, :, :5])
    o2, S2 = orc.delta_prefill(q[:, :, 5:12], k[:, :, 5:12], v[:, :, 5:12], g[:, :, 5:12],
                               S0=S1, alpha=al[:, :, 5:12])
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o[:, :, :12], rtol=1e-12)
    od, Sd = orc.delta_decode_step(q[:, :, 12], k[:, :, 12], v[:, :, 12], g[:, :, 12], S2,
                                   alpha=al[:, :, 12])
    np.testing.assert_allclose(od, o[:, :, 12], rtol=1e-12)
    np.testing.assert_allclose(Sd, S, rtol=1e-12)


# --- linear rule with a per-channel decay (GLA) ----------------------------

def pin_gla_quadratic_form(orc):
    """Unrolling S_t = diag(alpha_t) S_{t-1} + phi(k_t) v_t^T gives the score
    A_ti = sum_f phi(q_t)_f phi(k_i)_f prod_{m=i+1..t} alpha_m,f for i <= t
    (Efficient attention variants 7.2: each key channel keeps its own row);
    brute force on tiny inputs with d != dv, from a nonzero initial state."""
    rng = np.random.default_rng(31)
    N, d, dv, eps = 9, 3, 5, 1e-3
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(N, d))
    v = rng.normal(size=(N, dv))
    al = rng.uniform(0.4, 1.0, size=(N, d))
    S0 = rng.uniform(0.0, 1.0, size=(d, dv))
    z0 = rng.uniform(0.5, 1.0, size=d)
    fq, fk = orc.phi_elu1(q), orc.phi_elu1(k)
    ref = np.zeros((N, dv))
    for t in range(N):
        dec0 = np.prod(al[:t + 1], axis=0)          # decay of the initial state
        num = (fq[t] * dec0) @ S0
        den = (fq[t] * dec0) @ z0
        for i in range(t + 1):
            a = np.sum(fq[t] * fk[i] * np.prod(al[i + 1:t + 1], axis=0))
            num = num + a * v[i]
            den = den + a
        ref[t] = num / (den + eps)
    o, _, _ = orc.linear_prefill(_bh(q), _bh(k), _bh(v), eps=eps, S0=_bh(S0), z0=_bh(z0),
                                 alpha=_bh(al))
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-12, atol=1e-14)


def pin_gla_one_hot_keys(orc):
    """Identity features and one-hot keys: each state row only decays by its
    own channel's alpha and receives the values written to it (closed form
    per row), z likewise."""
    d, dv = 3, 2
    k = np.array([[1, 0, 0], [0, 0, 1], [1, 0, 0], [0, 1, 0]], dtype=np.float64)
    v = np.array([[1.0, 2.0], [3.0, -1.0], [0.5, 0.25], [4.0, 4.0]])
    al = np.array([[0.5, 0.9, 0.8], [0.25, 0.5, 0.5], [1.0, 0.75, 0.5], [0.5, 0.5, 0.25]])
    S0 = np.ones((d, dv))
    _, S, z = orc.linear_prefill(_bh(k), _bh(k), _bh(v), fmap=orc.FMAP_IDENTITY, S0=_bh(S0),
                                 z0=_bh(np.ones(d)), alpha=_bh(al))
    want_S = np.empty((d, dv))
    want_z = np.empty(d)
    for f in range(d):
        row, zz = S0[f].copy(), 1.0
        for t in range(4):
            row = al[t, f] * row + k[t, f] * v[t]
            zz = al[t, f] * zz + k[t, f]
        want_S[f], want_z[f] = row, zz
    np.testing.assert_allclose(S[0, 0], want_S, rtol=1e-15)
    np.testing.assert_allclose(z[0, 0], want_z, rtol=1e-15)
    assert abs(S[0, 0][1, 0] - (0.9 * 0.5 * 0.75 * 1.0 * 0.5 + 4.0)) < 1e-15


def pin_gla_uniform_is_gamma_and_split(orc):
    """A per-channel decay equal to gamma_h on every channel and token is the
    per-head decay; with varying alpha, a split sequence with carried state
    and a decode step after prefill give the same result."""
    rng = np.random.default_rng(32)
    B, H, N, d, dv = 1, 2, 11, 4, 3
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    v = rng.normal(size=(B, H, N, dv))
    gamma = np.array([0.9, 0.6])
    al_u = np.broadcast_to(gamma[None, :, None, None], (B, H, N, d)).copy()
    og, Sg, zg = orc.linear_prefill(q, k, v, gamma=gamma)
    oa, Sa, za = orc.linear_prefill(q, k, v, alpha=al_u)
    np.testing.assert_allclose(oa, og, rtol=1e-14)
    np.testing.assert_allclose(Sa, Sg, rtol=1e-14)
    al = rng.uniform(0.5, 1.0, size=(B, H, N, d))
    o, S, z = orc.linear_prefill(q, k, v, alpha=al)
    o1, S1, z1 = orc.linear_prefill(q[:, :, :4], k[:, :, :4], v[:, :, :4], alpha=al[:, :, :4])
    o2, S2, z2 = orc.linear_prefill(q[:, :, 4:10], k[:, :, 4:10], v[:, :, 4:10], S0=S1, z0=z1,
                                    alpha=al[:, :, 4:10])
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o[:, :, :10], rtol=1e-12)
    od, Sd, zd = orc.linear_decode_step(q[:, :, 10], k[:, :, 10], v[:, :, 10], S2, z2,
                                        alpha=al[:, :, 10])
    np.testing.assert_allclose(od, o[:, :, 10], rtol=1e-12)
    np.testing.assert_allclose(Sd, S, rtol=1e-12)
    np.testing.assert_allclose(zd, z, rtol=1e-12)


# --- short causal convolution (What Is Linear Attention? 5.4) ---------------

def _correlate_conv(x, W, cache):
    """Per head and channel: numpy's 'valid' correlation of the cache
    followed by the sequence with the filter (tap w-1 on the current token).
    x: [H, N, c], W: [H, w, c], cache: [H, w-1, c]."""
    H, N, c = x.shape
    full = np.concatenate([cache, x], axis=1)
    y = np.empty((H, N, c))
    for h in range(H):
        for ch in range(c):
            y[h, :, ch] = np.correlate(full[h, :, ch], W[h, :, ch], mode="valid")
    return y, full[:, full.shape[1] - (W.shape[1] - 1):]


def pin_conv_matches_numpy_correlate(orc):
    """The depthwise causal convolution equals numpy's correlation of the
    cached tokens followed by the sequence, per channel; the new cache is
    the last w-1 raw tokens; widths 1..4, sequences shorter than the cache."""
    rng = np.random.default_rng(41)
    for w in (1, 2, 3, 4):
        for N in (1, 2, 7):
            H, c = 2, 3
            x = rng.normal(size=(1, H, N, c))
            W = rng.normal(size=(H, w, c))
            cache = rng.normal(size=(1, H, w - 1, c))
            y, hist = orc.short_conv(x, W, cache)
            ry, rh = _correlate_conv(x[0], W, cache[0])
            np.testing.assert_allclose(y[0], ry, rtol=1e-13, atol=1e-14)
            np.testing.assert_array_equal(hist[0], rh)
            y0, _ = orc.short_conv(x, W)  # no cache: zeros before the sequence
            ry0, _ = _correlate_conv(x[0], W, np.zeros_like(cache[0]))
            np.testing.assert_allclose(y0[0], ry0, rtol=1e-13, atol=1e-14)


def pin_conv_then_attention_brute_force(orc):
    """linear_prefill_conv on channels [q | k | v] (distinct filters, d != dv)
    equals the O(N^2) masked form on inputs convolved by numpy's correlation,
    and returns the raw last tokens as the cache."""
    rng = np.random.default_rng(42)
    H, N, d, dv, w, eps = 2, 9, 3, 4, 4, 1e-3
    q = rng.normal(size=(1, H, N, d))
    k = rng.normal(size=(1, H, N, d))
    v = rng.normal(size=(1, H, N, dv))
    W = rng.normal(size=(H, w, 2 * d + dv))
    cache = rng.normal(size=(1, H, w - 1, 2 * d + dv))
    o, _, _, hist = orc.linear_prefill_conv(q, k, v, W, conv_cache=cache, eps=eps)
    cq, _ = _correlate_conv(q[0], W[..., :d], cache[0][..., :d])
    ck, _ = _correlate_conv(k[0], W[..., d:2 * d], cache[0][..., d:2 * d])
    cv, _ = _correlate_conv(v[0], W[..., 2 * d:], cache[0][..., 2 * d:])
    fq, fk = orc.phi_elu1(cq), orc.phi_elu1(ck)
    ref = np.empty((H, N, dv))
    for h in range(H):
        for t in range(N):
            a = np.array([fq[h, t] @ fk[h, i] for i in range(t + 1)])
            ref[h, t] = (a @ cv[h, :t + 1]) / (a.sum() + eps)
    np.testing.assert_allclose(o[0], ref, rtol=1e-11, atol=1e-13)
    raw = np.concatenate([q, k, v], axis=-1)[0]
    np.testing.assert_array_equal(hist[0], raw[:, N - (w - 1):])


def pin_conv_identity_and_shift_filters(orc):
    """The unit filter on the current token leaves q, k, v unchanged; the
    unit filter on the oldest tap delays the sequence by w-1 tokens, the
    cache supplying the first ones."""
    rng = np.random.default_rng(43)
    B, H, N, d, dv, w = 1, 2, 6, 3, 2, 3
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    v = rng.normal(size=(B, H, N, dv))
    cache = rng.normal(size=(B, H, w - 1, 2 * d + dv))
    ident = np.zeros((H, w, 2 * d + dv))
    ident[:, w - 1] = 1.0
    o, S, z, _ = orc.linear_prefill_conv(q, k, v, ident, conv_cache=cache, gamma=[0.9, 0.8])
    o0, S0, z0 = orc.linear_prefill(q, k, v, gamma=[0.9, 0.8])
    np.testing.assert_allclose(o, o0, rtol=1e-14)
    np.testing.assert_allclose(S, S0, rtol=1e-14)
    shift = np.zeros((H, w, 2 * d + dv))
    shift[:, 0] = 1.0
    o, _, _, _ = orc.linear_prefill_conv(q, k, v, shift, conv_cache=cache)
    full = np.concatenate([cache, np.concatenate([q, k, v], axis=-1)], axis=2)[:, :, :N]
    o1, _, _ = orc.linear_prefill(full[..., :d], full[..., d:2 * d], full[..., 2 * d:])
    np.testing.assert_allclose(o, o1, rtol=1e-14)


def pin_conv_split_and_decode(orc):
    """Prefill in pieces (one shorter than the conv window) carrying S, z and
    the conv cache, then decode steps, equals one prefill of the whole
    sequence."""
    rng = np.random.default_rng(44)
    B, H, N, d, dv, w = 2, 1, 12, 3, 2, 4
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    v = rng.normal(size=(B, H, N, dv))
    W = rng.normal(size=(H, w, 2 * d + dv))
    al = rng.uniform(0.5, 1.0, size=(B, H, N, d))
    o, S, z, C = orc.linear_prefill_conv(q, k, v, W, alpha=al)
    parts, S1, z1, C1 = [], None, None, None
    for a, b in ((0, 5), (5, 7), (7, 10)):
        oi, S1, z1, C1 = orc.linear_prefill_conv(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], W,
                                                 conv_cache=C1, S0=S1, z0=z1,
                                                 alpha=al[:, :, a:b])
        parts.append(oi)
    np.testing.assert_allclose(np.concatenate(parts, axis=2), o[:, :, :10], rtol=1e-12)
    for t in (10, 11):
        od, S1, z1, C1 = orc.linear_decode_step_conv(q[:, :, t], k[:, :, t], v[:, :, t], S1,
                                                     z1, W, C1, alpha=al[:, :, t])
        np.testing.assert_allclose(od, o[:, :, t], rtol=1e-12)
    np.testing.assert_allclose(S1, S, rtol=1e-12)
    np.testing.assert_allclose(z1, z, rtol=1e-12)
    np.testing.assert_array_equal(C1, C)


def pin_conv_then_delta_brute_force(orc):
    """delta_prefill_conv (distinct filters, d != dv, with a decay) equals
    explicit matrix products S <- alpha (I - g k k^T) S + g k v^T, o = S^T q
    on inputs convolved by numpy's correlation, and returns the raw last
    tokens as the cache."""
    rng = np.random.default_rng(45)
    H, N, d, dv, w = 2, 9, 3, 4, 3
    q = rng.normal(size=(1, H, N, d))
    k = rng.normal(size=(1, H, N, d))
    v = rng.normal(size=(1, H, N, dv))
    g = rng.uniform(0.1, 0.9, size=(1, H, N))
    al = rng.uniform(0.6, 1.0, size=(1, H, N))
    W = rng.normal(size=(H, w, 2 * d + dv)) * 0.6
    cache = rng.normal(size=(1, H, w - 1, 2 * d + dv))
    S0 = rng.normal(size=(1, H, d, dv))
    o, S, hist = orc.delta_prefill_conv(q, k, v, g, W, conv_cache=cache, S0=S0, alpha=al)
    cq, _ = _correlate_conv(q[0], W[..., :d], cache[0][..., :d])
    ck, _ = _correlate_conv(k[0], W[..., d:2 * d], cache[0][..., d:2 * d])
    cv, _ = _correlate_conv(v[0], W[..., 2 * d:], cache[0][..., 2 * d:])
    eye = np.eye(d)
    for h in range(H):
        Sh = S0[0, h].copy()
        for t in range(N):
            kk = ck[h, t]
            Sh = al[0, h, t] * (eye - g[0, h, t] * np.outer(kk, kk)) @ Sh + \
                g[0, h, t] * np.outer(kk, cv[h, t])
            np.testing.assert_allclose(o[0, h, t], Sh.T @ cq[h, t], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(S[0, h], Sh, rtol=1e-11, atol=1e-12)
    raw = np.concatenate([q, k, v], axis=-1)[0]
    np.testing.assert_array_equal(hist[0], raw[:, N - (w - 1):])


def pin_conv_delta_identity_split_and_decode(orc):
    """The unit filter on the current token gives delta_prefill itself; with
    a general filter, prefill in pieces (one shorter than the conv window)
    carrying S and the conv cache, then decode steps, equals one prefill."""
    rng = np.random.default_rng(46)
    B, H, N, d, dv, w = 2, 1, 12, 3, 2, 4
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    v = rng.normal(size=(B, H, N, dv))
    g = rng.uniform(size=(B, H, N))
    al = rng.uniform(0.5, 1.0, size=(B, H, N))
    ident = np.zeros((H, w, 2 * d + dv))
    ident[:, w - 1] = 1.0
    cache = rng.normal(size=(B, H, w - 1, 2 * d + dv))
    o, S, _ = orc.delta_prefill_conv(q, k, v, g, ident, conv_cache=cache, alpha=al)
    o0, S0 = orc.delta_prefill(q, k, v, g, alpha=al)
    np.testing.assert_allclose(o, o0, rtol=1e-14)
    np.testing.assert_allclose(S, S0, rtol=1e-14)
    W = rng.normal(size=(H, w, 2 * d + dv)) * 0.5
    o, S, C = orc.delta_prefill_conv(q, k, v, g, W, alpha=al)
    parts, S1, C1 = [], None, None
    for a, b in ((0, 5), (5, 7), (7, 10)):
        oi, S1, C1 = orc.delta_prefill_conv(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b],
                                            g[:, :, a:b], W, conv_cache=C1, S0=S1,
                                            alpha=al[:, :, a:b])
        parts.append(oi)
    np.testing.assert_allclose(np.concatenate(parts, axis=2), o[:, :, :10], rtol=1e-12)
    for t in (10, 11):
        od, S1, C1 = orc.delta_decode_step_conv(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t],
                                                S1, W, C1, alpha=al[:, :, t])
        np.testing.assert_allclose(od, o[:, :, t], rtol=1e-12)
    np.testing.assert_allclose(S1, S, rtol=1e-12)
    np.testing.assert_array_equal(C1, C)


# --- backward of the LINEAR rule (derived; the pages give no formulas) ------

def _torch_linear_loss(q, k, v, do, gamma, eps, S0, z0, dS, dz, elu):
    """Loss sum(o * do) + sum(S_N * dS) + sum(z_N * dz) of the recurrence,
    built from torch ops so that autograd differentiates it."""
    import torch
    phi = (lambda x: torch.nn.functional.elu(x) + 1.0) if elu else (lambda x: x)
    fq, fk = phi(q), phi(k)
    S, z = S0, z0
    loss = 0.0
    for t in range(q.shape[-2]):
        S = gamma[:, None, None] * S + fk[:, t, :, None] * v[:, t, None, :]
        z = gamma[:, None] * z + fk[:, t]
        num = torch.einsum("hr,hrd->hd", fq[:, t], S)
        den = (fq[:, t] * z).sum(-1) + eps
        loss = loss + ((num / den[:, None]) * do[:, t]).sum()
    return loss + (S * dS).sum() + (z * dz).sum()


def pin_backward_matches_autograd(orc):
    """dq, dk, dv and the initial-state gradients equal torch autograd's
    through the recurrence, with decay, eps, an initial state, a final-state
    gradient, d != dv, for both feature maps."""
    import torch
    rng = np.random.default_rng(51)
    H, N, d, dv, eps = 2, 9, 3, 4, 1e-2
    for elu in (True, False):
        q = rng.normal(size=(H, N, d)) * (1.0 if elu else 0.0) + (0.0 if elu else 1.0)
        k = rng.normal(size=(H, N, d)) * (1.0 if elu else 0.0) + (0.0 if elu else 1.0)
        if not elu:  # non-negative features for the identity map
            q, k = rng.uniform(0.1, 1.0, size=(H, N, d)), rng.uniform(0.1, 1.0, size=(H, N, d))
        v = rng.normal(size=(H, N, dv))
        do = rng.normal(size=(H, N, dv))
        S0 = rng.normal(size=(H, d, dv)) * 0.3
        z0 = rng.uniform(0.5, 1.0, size=(H, d))
        dS = rng.normal(size=(H, d, dv))
        dz = rng.normal(size=(H, d))
        gamma = np.array([0.9, 0.7])
        T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
        tq, tk, tv, tS0, tz0 = T(q), T(k), T(v), T(S0), T(z0)
        loss = _torch_linear_loss(tq, tk, tv, torch.tensor(do), torch.tensor(gamma), eps, tS0,
                                  tz0, torch.tensor(dS), torch.tensor(dz), elu)
        loss.backward()
        fmap = orc.FMAP_ELU1 if elu else orc.FMAP_IDENTITY
        got = orc.linear_backward(q[None], k[None], v[None], do[None], gamma=gamma, eps=eps,
                                  fmap=fmap, S0=S0[None], z0=z0[None], dS_N=dS[None],
                                  dz_N=dz[None])
        for g, t in zip(got, (tq, tk, tv, tS0, tz0)):
            np.testing.assert_allclose(g[0], t.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_backward_finite_differences(orc):
    """Central differences of the oracle's own forward (loss sum(o * do))
    agree with the backward on every entry of q, k and v."""
    rng = np.random.default_rng(52)
    B, H, N, d, dv, eps, h = 1, 1, 5, 3, 2, 1e-3, 1e-6
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    v = rng.normal(size=(B, H, N, dv))
    do = rng.normal(size=(B, H, N, dv))
    gamma = [0.8]
    dq, dk, dvv, _, _ = orc.linear_backward(q, k, v, do, gamma=gamma, eps=eps)

    def loss(q_, k_, v_):
        o, _, _ = orc.linear_prefill(q_, k_, v_, gamma=gamma, eps=eps)
        return float(np.sum(o * do))
    for x, g in ((q, dq), (k, dk), (v, dvv)):
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if a is x else a for a in (q, k, v)]
            args_m = [xm if a is x else a for a in (q, k, v)]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def _torch_gla_loss(q, k, v, do, alpha, eps, S0, z0, dS, dz, elu):
    """As _torch_linear_loss with a per-channel decay alpha [H, N, d]:
    S_t = diag(alpha_t) S_(t-1) + phi(k_t) v_t^T, z_t = alpha_t z_(t-1) + phi(k_t)."""
    import torch
    phi = (lambda x: torch.nn.functional.elu(x) + 1.0) if elu else (lambda x: x)
    fq, fk = phi(q), phi(k)
    S, z = S0, z0
    loss = 0.0
    for t in range(q.shape[-2]):
        S = alpha[:, t, :, None] * S + fk[:, t, :, None] * v[:, t, None, :]
        z = alpha[:, t] * z + fk[:, t]
        num = torch.einsum("hr,hrd->hd", fq[:, t], S)
        den = (fq[:, t] * z).sum(-1) + eps
        loss = loss + ((num / den[:, None]) * do[:, t]).sum()
    return loss + (S * dS).sum() + (z * dz).sum()


def pin_gla_backward_matches_autograd(orc):
    """With a per-channel decay: dq, dk, dv, the initial-state gradients and
    dalpha equal torch autograd's through the recurrence (both feature maps,
    an initial state, a final-state gradient, d != dv)."""
    import torch
    rng = np.random.default_rng(54)
    H, N, d, dv, eps = 2, 8, 3, 4, 1e-2
    for elu in (True, False):
        if elu:
            q, k = rng.normal(size=(H, N, d)), rng.normal(size=(H, N, d))
        else:
            q, k = rng.uniform(0.1, 1.0, size=(H, N, d)), rng.uniform(0.1, 1.0, size=(H, N, d))
        v = rng.normal(size=(H, N, dv))
        do = rng.normal(size=(H, N, dv))
        al = rng.uniform(0.3, 1.0, size=(H, N, d))
        S0 = rng.normal(size=(H, d, dv)) * 0.3
        z0 = rng.uniform(0.5, 1.0, size=(H, d))
        dS = rng.normal(size=(H, d, dv))
        dz = rng.normal(size=(H, d))
        T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
        tq, tk, tv, tal, tS0, tz0 = T(q), T(k), T(v), T(al), T(S0), T(z0)
        loss = _torch_gla_loss(tq, tk, tv, torch.tensor(do), tal, eps, tS0, tz0,
                               torch.tensor(dS), torch.tensor(dz), elu)
        loss.backward()
        fmap = orc.FMAP_ELU1 if elu else orc.FMAP_IDENTITY
        got = orc.linear_backward(q[None], k[None], v[None], do[None], alpha=al[None], eps=eps,
                                  fmap=fmap, S0=S0[None], z0=z0[None], dS_N=dS[None],
                                  dz_N=dz[None])
        assert len(got) == 6
        for g, t in zip(got, (tq, tk, tv, tS0, tz0, tal)):
            np.testing.assert_allclose(g[0], t.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_gla_backward_finite_differences(orc):
    """Central differences of the oracle's own forward with a per-channel
    decay (loss sum(o * do) + final-state terms) agree with the backward on
    every entry of alpha, q, k and v."""
    rng = np.random.default_rng(55)
    B, H, N, d, dv, eps, h = 1, 1, 5, 3, 2, 1e-3, 1e-6
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    v = rng.normal(size=(B, H, N, dv))
    do = rng.normal(size=(B, H, N, dv))
    al = rng.uniform(0.2, 1.0, size=(B, H, N, d))
    dS = rng.normal(size=(B, H, d, dv))
    dz = rng.normal(size=(B, H, d))
    dq, dk, dvv, _, _, dal = orc.linear_backward(q, k, v, do, alpha=al, eps=eps, dS_N=dS,
                                                 dz_N=dz)

    def loss(q_, k_, v_, a_):
        o, S, z = orc.linear_prefill(q_, k_, v_, alpha=a_, eps=eps)
        return float(np.sum(o * do) + np.sum(S * dS) + np.sum(z * dz))
    args = (q, k, v, al)
    for i, g in enumerate((dq, dk, dvv, dal)):
        x = args[i]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = (loss(*[xp if j == i else a for j, a in enumerate(args)])
                       - loss(*[xm if j == i else a for j, a in enumerate(args)])) / (2 * h)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def pin_gla_backward_uniform_is_gamma(orc):
    """alpha_t = gamma (every token and channel) gives the per-head rule's
    gradients, and the sum of dalpha over tokens and channels is dL/dgamma
    (a central difference of the per-head forward in gamma)."""
    rng = np.random.default_rng(56)
    B, H, N, d, dv, eps, h = 1, 2, 7, 3, 4, 1e-2, 1e-6
    q = rng.normal(size=(B, H, N, d))
    k = rng.normal(size=(B, H, N, d))
    v = rng.normal(size=(B, H, N, dv))
    do = rng.normal(size=(B, H, N, dv))
    S0 = rng.normal(size=(B, H, d, dv)) * 0.3
    z0 = rng.uniform(0.5, 1.0, size=(B, H, d))
    gamma = np.array([0.85, 0.6])
    al = np.broadcast_to(gamma[None, :, None, None], (B, H, N, d)).copy()
    kw = dict(eps=eps, S0=S0, z0=z0)
    want = orc.linear_backward(q, k, v, do, gamma=gamma, **kw)
    got = orc.linear_backward(q, k, v, do, alpha=al, **kw)
    for g, w in zip(got[:5], want):
        np.testing.assert_allclose(g, w, rtol=1e-12, atol=1e-14)
    for hh in range(H):
        def loss(gv):
            gg = gamma.copy()
            gg[hh] = gv
            o, _, _ = orc.linear_prefill(q, k, v, gamma=gg, **kw)
            return float(np.sum(o * do))
        fd = (loss(gamma[hh] + h) - loss(gamma[hh] - h)) / (2 * h)
        np.testing.assert_allclose(got[5][0, hh].sum(), fd, rtol=1e-6, atol=1e-9)


def pin_gla_denominators_brute_force(orc):
    """With a per-channel decay: den_t = sum_f phi(q_t)_f (sum_{j<=t}
    prod_{j<s<=t} alpha_s[f] phi(k_j)_f + prod_{s<=t} alpha_s[f] z0_f) + eps,
    by explicit loops over tokens and channels."""
    rng = np.random.default_rng(57)
    N, d, eps = 6, 3, 1e-2
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(N, d))
    al = rng.uniform(0.3, 1.0, size=(N, d))
    z0 = rng.uniform(0.1, 1.0, size=d)
    fq, fk = orc.phi_elu1(q), orc.phi_elu1(k)
    den = orc.linear_denominators(_bh(q), _bh(k), alpha=_bh(al), eps=eps, z0=_bh(z0))[0, 0]
    for t in range(N):
        want = eps
        for f in range(d):
            zf = z0[f] * np.prod(al[:t + 1, f])
            for j in range(t + 1):
                zf += np.prod(al[j + 1:t + 1, f]) * fk[j, f]
            want += fq[t, f] * zf
        assert abs(den[t] - want) < 1e-12 * want


def pin_denominators_brute_force(orc):
    """den_t = sum_{j<=t} gamma^(t-j) phi(q_t).phi(k_j) + gamma^(t+1) phi(q_t).z0
    + eps, by explicit double loop; and den_t o_t equals the numerator of
    the quadratic form."""
    rng = np.random.default_rng(53)
    N, d, dv, eps, g = 7, 3, 2, 1e-2, 0.85
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(N, d))
    v = rng.normal(size=(N, dv))
    z0 = rng.uniform(0.1, 1.0, size=d)
    fq, fk = orc.phi_elu1(q), orc.phi_elu1(k)
    den = orc.linear_denominators(_bh(q), _bh(k), gamma=[g], eps=eps, z0=_bh(z0))[0, 0]
    for t in range(N):
        want = eps + g ** (t + 1) * fq[t] @ z0
        for j in range(t + 1):
            want += g ** (t - j) * fq[t] @ fk[j]
        assert abs(den[t] - want) < 1e-12 * want
    o, _, _ = orc.linear_prefill(_bh(q), _bh(k), _bh(v), gamma=[g], eps=eps)
    den0 = orc.linear_denominators(_bh(q), _bh(k), gamma=[g], eps=eps)[0, 0]
    for t in range(N):
        num = sum(g ** (t - j) * (fq[t] @ fk[j]) * v[j] for j in range(t + 1))
        np.testing.assert_allclose(o[0, 0, t] * den0[t], num, rtol=1e-12, atol=1e-14)


# --- backward of the gated DELTA rule (derived; the pages give no formulas) --

def _torch_delta_loss(q, k, v, g, al, S0, do, dS):
    """Loss sum(o * do) + sum(S_N * dS) of the gated delta recurrence written
    with explicit matrices, S_t = a (I - g k k^T) S_{t-1} + g k v^T,
    o_t = S_t^T q_t, in torch ops so that autograd differentiates it."""
    import torch
    H, N, d = q.shape
    eye = torch.eye(d, dtype=torch.float64)
    S, loss = S0, 0.0
    for t in range(N):
        kt = k[:, t]
        A = al[:, t, None, None] * (eye - g[:, t, None, None] * kt[:, :, None] * kt[:, None, :])
        S = A @ S + g[:, t, None, None] * kt[:, :, None] * v[:, t, None, :]
        loss = loss + (torch.einsum("hrd,hr->hd", S, q[:, t]) * do[:, t]).sum()
    return loss + (S * dS).sum()


def pin_delta_backward_matches_autograd(orc):
    """dq, dk, dv, dg, dalpha and the initial-state gradient of the gated
    delta rule equal torch autograd's through the explicit-matrix recurrence,
    with and without the decay, an initial state, a final-state gradient and
    d != dv."""
    import torch
    rng = np.random.default_rng(61)
    H, N, d, dv = 2, 8, 3, 4
    for decay in (False, True):
        q = rng.normal(size=(H, N, d))
        k = rng.normal(size=(H, N, d)) * 0.6
        v = rng.normal(size=(H, N, dv))
        g = rng.uniform(0.1, 0.9, size=(H, N))
        al = rng.uniform(0.6, 1.0, size=(H, N)) if decay else np.ones((H, N))
        do = rng.normal(size=(H, N, dv))
        S0 = rng.normal(size=(H, d, dv)) * 0.5
        dS = rng.normal(size=(H, d, dv))
        T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
        tq, tk, tv, tg, ta, tS0 = T(q), T(k), T(v), T(g), T(al), T(S0)
        _torch_delta_loss(tq, tk, tv, tg, ta, tS0, torch.tensor(do), torch.tensor(dS)).backward()
        got = orc.delta_backward(q[None], k[None], v[None], g[None], do[None],
                                 alpha=al[None] if decay else None, S0=S0[None],
                                 dS_N=dS[None])
        want = [tq, tk, tv, tg, ta if decay else None, tS0]
        for name, x, t in zip(("dq", "dk", "dv", "dg", "dalpha", "dS0"), got, want):
            if t is None:
                assert x is None, name
                continue
            np.testing.assert_allclose(x[0], t.grad.numpy(), rtol=1e-10, atol=1e-12,
                                       err_msg=name)


def pin_delta_backward_finite_differences(orc):
    """Central differences of the oracle's own forward (loss sum(o * do) +
    sum(S_N * dS)) agree with the backward on every entry of q, k, v, g,
    alpha and the initial state."""
    rng = np.random.default_rng(62)
    B, H, N, d, dv, h = 1, 1, 5, 3, 2, 1e-6
    x = {"q": rng.normal(size=(B, H, N, d)), "k": rng.normal(size=(B, H, N, d)) * 0.6,
         "v": rng.normal(size=(B, H, N, dv)), "g": rng.uniform(0.1, 0.9, size=(B, H, N)),
         "alpha": rng.uniform(0.6, 1.0, size=(B, H, N)),
         "S0": rng.normal(size=(B, H, d, dv)) * 0.5}
    do = rng.normal(size=(B, H, N, dv))
    dS = rng.normal(size=(B, H, d, dv))
    grads = dict(zip(("q", "k", "v", "g", "alpha", "S0"),
                     orc.delta_backward(x["q"], x["k"], x["v"], x["g"], do, alpha=x["alpha"],
                                        S0=x["S0"], dS_N=dS)))

    def loss(y):
        o, S = orc.delta_prefill(y["q"], y["k"], y["v"], y["g"], S0=y["S0"], alpha=y["alpha"])
        return float(np.sum(o * do) + np.sum(S * dS))
    for name in x:
        fd = np.empty_like(x[name])
        for idx in np.ndindex(x[name].shape):
            yp, ym = dict(x), dict(x)
            yp[name], ym[name] = x[name].copy(), x[name].copy()
            yp[name][idx] += h
            ym[name][idx] -= h
            fd[idx] = (loss(yp) - loss(ym)) / (2 * h)
        np.testing.assert_allclose(grads[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def _torch_conv(x, W, cache):
    """The short convolution as explicit tap sums over [cache | x] in torch
    ops (x [H, N, c], W [H, w, c], cache [H, w-1, c]); returns (y, the last
    w-1 rows of [cache | x])."""
    import torch
    full = torch.cat([cache, x], dim=1)
    w, N = W.shape[1], x.shape[1]
    y = sum(W[:, j, None, :] * full[:, j:j + N, :] for j in range(w))
    return y, full[:, full.shape[1] - (w - 1):]


def _conv_grads_case(rng, H, N, d, dv, w):
    q = rng.normal(size=(H, N, d))
    k = rng.normal(size=(H, N, d)) * 0.6
    v = rng.normal(size=(H, N, dv))
    W = rng.normal(size=(H, w, 2 * d + dv)) * 0.5
    W[:, w - 1] += 1.0
    C = rng.normal(size=(H, w - 1, 2 * d + dv)) * 0.5
    dC = rng.normal(size=(H, w - 1, 2 * d + dv))
    do = rng.normal(size=(H, N, dv))
    return q, k, v, W, C, dC, do


def pin_conv_backward_matches_autograd(orc):
    """linear_backward_conv and delta_backward_conv equal torch autograd's
    gradients through explicit tap sums and the recurrences (inputs, filters,
    conv cache, initial state; with a final-state gradient and a gradient on
    the returned conv cache), widths 1..4."""
    import torch
    rng = np.random.default_rng(71)
    H, N, d, dv = 2, 7, 3, 4
    T = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)  # noqa: E731
    for w in (1, 2, 4):
        q, k, v, W, C, dC, do = _conv_grads_case(rng, H, N, d, dv, w)
        # LINEAR (elu+1, decay, eps)
        S0 = rng.normal(size=(H, d, dv)) * 0.3
        z0 = rng.uniform(0.5, 1.0, size=(H, d))
        dS, dz = rng.normal(size=(H, d, dv)), rng.normal(size=(H, d))
        gamma, eps = np.array([0.9, 0.7]), 1e-2
        tq, tk, tv, tW, tC, tS0, tz0 = T(q), T(k), T(v), T(W), T(C), T(S0), T(z0)
        x = torch.cat([tq, tk, tv], dim=-1)
        y, cout = _torch_conv(x, tW, tC)
        loss = _torch_linear_loss(y[..., :d], y[..., d:2 * d], y[..., 2 * d:], torch.tensor(do),
                                  torch.tensor(gamma), eps, tS0, tz0, torch.tensor(dS),
                                  torch.tensor(dz), True)
        (loss + (cout * torch.tensor(dC)).sum()).backward()
        got = orc.linear_backward_conv(q[None], k[None], v[None], do[None], W,
                                       conv_cache=C[None], dconv_cache_out=dC[None],
                                       gamma=gamma, eps=eps, S0=S0[None], z0=z0[None],
                                       dS_N=dS[None], dz_N=dz[None])
        want = (tq.grad, tk.grad, tv.grad, tW.grad, tC.grad, tS0.grad, tz0.grad)
        for name, gx, t in zip(("dq", "dk", "dv", "dW", "dC", "dS0", "dz0"), got, want):
            gx = gx if name == "dW" else gx[0]
            np.testing.assert_allclose(gx, t.numpy(), rtol=1e-10, atol=1e-12,
                                       err_msg=f"linear w={w} {name}")
        # DELTA with a decay
        g = rng.uniform(0.1, 0.9, size=(H, N))
        al = rng.uniform(0.6, 1.0, size=(H, N))
        tq, tk, tv, tW, tC, tS0 = T(q), T(k * 0.5), T(v), T(W), T(C), T(S0)
        x = torch.cat([tq, tk, tv], dim=-1)
        y, cout = _torch_conv(x, tW, tC)
        loss = _torch_delta_loss(y[..., :d], y[..., d:2 * d], y[..., 2 * d:], torch.tensor(g),
                                 torch.tensor(al), tS0, torch.tensor(do), torch.tensor(dS))
        (loss + (cout * torch.tensor(dC)).sum()).backward()
        got = orc.delta_backward_conv(q[None], (k * 0.5)[None], v[None], g[None], do[None], W,
                                      conv_cache=C[None], dconv_cache_out=dC[None],
                                      alpha=al[None], S0=S0[None], dS_N=dS[None])
        want = (tq.grad, tk.grad, tv.grad, None, None, tW.grad, tC.grad, tS0.grad)
        for name, gx, t in zip(("dq", "dk", "dv", "dg", "dal", "dW", "dC", "dS0"), got, want):
            if t is None:
                continue
            gx = gx if name == "dW" else gx[0]
            np.testing.assert_allclose(gx, t.numpy(), rtol=1e-10, atol=1e-12,
                                       err_msg=f"delta w={w} {name}")


def pin_conv_backward_finite_differences(orc):
    """The filter and conv-cache gradients of linear_backward_conv against
    central differences of linear_prefill_conv's loss sum(o * do)."""
    rng = np.random.default_rng(72)
    H, N, d, dv, w = 1, 6, 2, 3, 3
    q, k, v, W, C, _, do = _conv_grads_case(rng, H, N, d, dv, w)
    q, k, v, C, do = q[None], k[None], v[None], C[None], do[None]
    loss = lambda W_, C_: np.sum(orc.linear_prefill_conv(q, k, v, W_, conv_cache=C_)[0] * do)  # noqa: E731
    _, _, _, dW, dC, _, _ = orc.linear_backward_conv(q, k, v, do, W, conv_cache=C)
    h = 1e-6
    for idx in ((0, 0, 0), (0, 1, 2), (0, 2, 5), (0, 2, 6)):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += h
        Wm[idx] -= h
        np.testing.assert_allclose(dW[idx], (loss(Wp, C) - loss(Wm, C)) / (2 * h), rtol=1e-6,
                                   atol=1e-8)
    for idx in ((0, 0, 0, 1), (0, 0, 1, 4), (0, 0, 1, 6)):
        Cp, Cm = C.copy(), C.copy()
        Cp[idx] += h
        Cm[idx] -= h
        np.testing.assert_allclose(dC[idx], (loss(W, Cp) - loss(W, Cm)) / (2 * h), rtol=1e-6,
                                   atol=1e-8)


def pin_delta_backward_gate_zero(orc):
    """With g = 0 the state never changes (S_t = S0, no decay), so
    o_t = S0^T q_t: dq_t = S0 do_t, dk = dv = 0, dS0 = sum_t q_t do_t^T, and
    dg_t = (Sh_t^T k_t) . (v_t - S0^T k_t) with Sh_t = sum_(s>=t) q_s do_s^T."""
    rng = np.random.default_rng(63)
    N, d, dv = 6, 3, 4
    q, k, v = rng.normal(size=(N, d)), rng.normal(size=(N, d)), rng.normal(size=(N, dv))
    do = rng.normal(size=(N, dv))
    S0 = rng.normal(size=(d, dv))
    dq, dk, dvv, dg, da, dS0 = orc.delta_backward(_bh(q), _bh(k), _bh(v), _bh(np.zeros(N)),
                                                   _bh(do), S0=_bh(S0))
    assert da is None
    np.testing.assert_allclose(dq[0, 0], do @ S0.T, rtol=1e-12, atol=1e-14)
    assert not dk.any() and not dvv.any()
    np.testing.assert_allclose(dS0[0, 0], q.T @ do, rtol=1e-12, atol=1e-14)
    for t in range(N):
        Sh = q[t:].T @ do[t:]
        want = (Sh.T @ k[t]) @ (v[t] - S0.T @ k[t])
        np.testing.assert_allclose(dg[0, 0, t], want, rtol=1e-12, atol=1e-14)


ALL_PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]
