"""Plant plausible mistakes in a private copy of the oracle and check that
the pins catch every one of them (CPU only).  The real oracle module is not
touched: each mutant is a freshly loaded copy of oracle/la_oracle.py."""
import importlib.util
import os

import numpy as np
import pytest

from oracle_pins import ALL_PINS

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(
    os.path.abspath(__file__))), "oracle", "la_oracle.py")


def _fresh():
    spec = importlib.util.spec_from_file_location("la_oracle_mutant", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _rows(gam, S):
    return gam[..., None] if gam.ndim == S.ndim - 2 else gam


def _read_before_write(m):
    def step(S, z, fq, fk, v, gam, eps):
        num = np.einsum("...r,...rd->...d", fq, S)
        den = np.einsum("...r,...r->...", fq, z) + eps
        S2 = _rows(gam, S)[..., :, None] * S + fk[..., :, None] * v[..., None, :]
        z2 = _rows(gam, S) * z + fk
        return num / den[..., None], S2, z2
    m.linear_step = step


def _z_not_decayed(m):
    orig = m.linear_step
    def step(S, z, fq, fk, v, gam, eps):
        o, S2, _ = orig(S, z, fq, fk, v, gam, eps)
        z2 = z + fk
        num = np.einsum("...r,...rd->...d", fq, S2)
        return num / (np.einsum("...r,...r->...", fq, z2) + eps)[..., None], S2, z2
    m.linear_step = step


def _eps_outside(m):
    orig = m.linear_step
    def step(S, z, fq, fk, v, gam, eps):
        o, S2, z2 = orig(S, z, fq, fk, v, gam, 0.0)
        return o + eps, S2, z2
    m.linear_step = step


def _no_plus_one(m):
    m.phi_elu1 = lambda x: np.where(m._f64(x) > 0, m._f64(x), np.exp(m._f64(x)) - 1)


def _exp_everywhere(m):
    m.phi_elu1 = lambda x: np.exp(m._f64(x))


def _decay_off_by_one(m):
    orig = m.linear_step
    def step(S, z, fq, fk, v, gam, eps):
        return orig(S, z, fq, _rows(gam, S) * fk, v, gam, eps)
    m.linear_step = step


def _outer_transposed(m):
    def step(S, z, fq, fk, v, gam, eps):
        d, dv = S.shape[-2:]
        upd = (v[..., :, None] * fk[..., None, :])
        upd = upd.reshape(upd.shape[:-2] + (d, dv)) if upd.size == S.size else upd
        S2 = _rows(gam, S)[..., :, None] * S + upd
        z2 = _rows(gam, S) * z + fk
        num = np.einsum("...r,...rd->...d", fq, S2)
        return num / (np.einsum("...r,...r->...", fq, z2) + eps)[..., None], S2, z2
    m.linear_step = step


def _quadratic_strict_mask(m):
    orig = m.linear_quadratic
    def quad(q, k, v, *, gamma=None, eps=1e-6, fmap=m.FMAP_ELU1):
        qq = m._f64(q)
        qq = np.concatenate([np.zeros_like(qq[..., :1, :]) - 50, qq[..., :-1, :]], axis=-2)
        return orig(q, k, v, gamma=gamma, eps=eps, fmap=fmap) * 0 + orig(
            qq, k, v, gamma=gamma, eps=eps, fmap=fmap)
    m.linear_quadratic = quad


def _decayed(S, alpha):
    return S if alpha is None else alpha[..., None, None] * S


def _delta_not_transposed(m):
    def step(S, q, k, v, g, alpha=None):
        S = _decayed(S, alpha)
        d, dv = S.shape[-2:]
        if d == dv:
            v_hat = np.einsum("...rd,...d->...r", S, k)
        else:
            v_hat = np.einsum("...rd,...r->...d", S, k)[..., ::-1]
        S2 = S + g[..., None, None] * k[..., :, None] * (v - v_hat)[..., None, :]
        return np.einsum("...rd,...r->...d", S2, q), S2
    m.delta_step = step


def _delta_wrong_sign(m):
    def step(S, q, k, v, g, alpha=None):
        S = _decayed(S, alpha)
        v_hat = np.einsum("...rd,...r->...d", S, k)
        S2 = S + g[..., None, None] * k[..., :, None] * (v + v_hat)[..., None, :]
        return np.einsum("...rd,...r->...d", S2, q), S2
    m.delta_step = step


def _delta_output_before_update(m):
    def step(S, q, k, v, g, alpha=None):
        S = _decayed(S, alpha)
        v_hat = np.einsum("...rd,...r->...d", S, k)
        S2 = S + g[..., None, None] * k[..., :, None] * (v - v_hat)[..., None, :]
        return np.einsum("...rd,...r->...d", S, q), S2
    m.delta_step = step


def _delta_gate_on_value_only(m):
    def step(S, q, k, v, g, alpha=None):
        S = _decayed(S, alpha)
        v_hat = np.einsum("...rd,...r->...d", S, k)
        S2 = S + k[..., :, None] * (g[..., None] * v - v_hat)[..., None, :]
        return np.einsum("...rd,...r->...d", S2, q), S2
    m.delta_step = step


def _delta_dropped_correction(m):
    def step(S, q, k, v, g, alpha=None):
        S = _decayed(S, alpha)
        S2 = S + g[..., None, None] * k[..., :, None] * v[..., None, :]
        return np.einsum("...rd,...r->...d", S2, q), S2
    m.delta_step = step


def _gdn_error_on_undecayed_state(m):
    def step(S, q, k, v, g, alpha=None):
        v_hat = np.einsum("...rd,...r->...d", S, k)
        S2 = _decayed(S, alpha) + g[..., None, None] * k[..., :, None] * (v - v_hat)[..., None, :]
        return np.einsum("...rd,...r->...d", S2, q), S2
    m.delta_step = step


def _gdn_decay_after_write(m):
    def step(S, q, k, v, g, alpha=None):
        v_hat = np.einsum("...rd,...r->...d", S, k)
        S2 = _decayed(S + g[..., None, None] * k[..., :, None] * (v - v_hat)[..., None, :], alpha)
        return np.einsum("...rd,...r->...d", S2, q), S2
    m.delta_step = step


def _gdn_decay_on_write_too(m):
    def step(S, q, k, v, g, alpha=None):
        S = _decayed(S, alpha)
        v_hat = np.einsum("...rd,...r->...d", S, k)
        S2 = S + _decayed(g[..., None, None] * k[..., :, None] * (v - v_hat)[..., None, :],
                          alpha)
        return np.einsum("...rd,...r->...d", S2, q), S2
    m.delta_step = step


def _gla_decay_on_value_axis(m):
    def step(S, z, fq, fk, v, gam, eps):
        if gam.ndim == S.ndim - 1 and S.shape[-1] != S.shape[-2]:
            dv = S.shape[-1]
            g = np.resize(gam, gam.shape[:-1] + (dv,))
            S2 = g[..., None, :] * S + fk[..., :, None] * v[..., None, :]
        else:
            S2 = _rows(gam, S)[..., :, None] * S + fk[..., :, None] * v[..., None, :]
        z2 = _rows(gam, S) * z + fk
        num = np.einsum("...r,...rd->...d", fq, S2)
        den = np.einsum("...r,...r->...", fq, z2) + eps
        return num / den[..., None], S2, z2
    m.linear_step = step


def _gla_decay_after_write(m):
    def step(S, z, fq, fk, v, gam, eps):
        r = _rows(gam, S)
        S2 = r[..., :, None] * (S + fk[..., :, None] * v[..., None, :])
        z2 = r * (z + fk)
        num = np.einsum("...r,...rd->...d", fq, S2)
        den = np.einsum("...r,...r->...", fq, z2) + eps
        return num / den[..., None], S2, z2
    m.linear_step = step


def _conv_taps_reversed(m):
    orig = m.short_conv
    m.short_conv = lambda x, W, cache=None: orig(x, m._f64(W)[:, ::-1], cache)


def _conv_cache_newest_first(m):
    orig = m.short_conv
    def conv(x, W, cache=None):
        return orig(x, W, None if cache is None else m._f64(cache)[:, :, ::-1])
    m.short_conv = conv


def _conv_cache_ignored(m):
    orig = m.short_conv
    def conv(x, W, cache=None):
        y, _ = orig(x, W, None)
        _, hist = orig(x, W, cache)
        return y, hist
    m.short_conv = conv


def _conv_excludes_current_token(m):
    def conv(x, W, cache=None):
        x, W = m._f64(x), m._f64(W)
        B, H, N, c = x.shape
        w = W.shape[1]
        hist = np.zeros((B, H, w, c))
        if cache is not None:
            hist[:, :, 1:] = m._f64(cache)
        y = np.empty((B, H, N, c))
        for t in range(N):
            y[:, :, t] = np.sum(hist * W[None], axis=2)
            hist = np.concatenate([hist[:, :, 1:], x[:, :, t:t + 1]], axis=2)
        return y, hist[:, :, 1:]
    m.short_conv = conv


def _conv_qk_filters_swapped(m):
    orig = m._conv_split
    def split(a, d):
        a0, a1, a2 = orig(a, d)
        return a1, a0, a2
    m._conv_split = split


def _patched(old, new):
    """A mutant made by editing one line of the oracle's source text."""
    def mutate(m):
        src = open(ORACLE_SRC).read()
        assert src.count(old) == 1, old
        exec(compile(src.replace(old, new), ORACLE_SRC, "exec"), m.__dict__)
    mutate.__name__ = "_patch"
    return mutate


_bwd_dden_dropped = _patched(
    'dden = -np.einsum("...d,...d->...", g, num) / den ** 2', "dden = 0.0 * den")
_bwd_dden_sign = _patched(
    'dden = -np.einsum("...d,...d->...", g, num) / den ** 2',
    'dden = np.einsum("...d,...d->...", g, num) / den ** 2')
_bwd_phi_grad_one = _patched("        return phi_elu1_grad(x)\n",
                             "        return np.ones_like(_f64(x))\n")
_bwd_adjoint_not_decayed = _patched("Sh = gam[..., None, None] * Sh", "Sh = 1.0 * Sh")
_bwd_dv_from_query = _patched('np.einsum("...rd,...r->...d", Sh, fk[:, :, t])',
                              'np.einsum("...rd,...r->...d", Sh, fq[:, :, t])')
_bwd_dk_without_z = _patched("v[:, :, t]) + zh", "v[:, :, t])")
for _n in ("_bwd_dden_dropped", "_bwd_dden_sign", "_bwd_phi_grad_one",
           "_bwd_adjoint_not_decayed", "_bwd_dv_from_query", "_bwd_dk_without_z"):
    globals()[_n].__name__ = _n


_dbwd_dk_no_state_term = _patched(
    """                       - (a * gt)[..., None] * np.einsum("...rd,...d->...r", S_prev, w))""",
    """                       - 0.0 * np.einsum("...rd,...d->...r", S_prev, w))""")
_dbwd_adjoint_not_decayed = _patched(
    "Sh = a[..., None, None] * (Sh - gt", "Sh = (Sh - gt")
_dbwd_adjoint_no_projection = _patched(
    "(Sh - gt[..., None, None] * kt[..., :, None] * w[..., None, :])", "(Sh)")
_dbwd_dv_without_gate = _patched("dvv[:, :, t] = gt[..., None] * w", "dvv[:, :, t] = w")
_dbwd_dq_from_previous_state = _patched(
    'dq[:, :, t] = np.einsum("...rd,...d->...r", S_t, do[:, :, t])',
    'dq[:, :, t] = np.einsum("...rd,...d->...r", S_prev, do[:, :, t])')
_dbwd_residual_undecayed = _patched("u = vt - a[..., None] * pred", "u = vt - pred")
_dbwd_dalpha_no_gate_term = _patched(
    "                           - gt * np.einsum(\"...d,...d->...\", pred, w))",
    "                           - 0.0 * gt)")
for _n in ("_dbwd_dk_no_state_term", "_dbwd_adjoint_not_decayed", "_dbwd_adjoint_no_projection",
           "_dbwd_dv_without_gate", "_dbwd_dq_from_previous_state", "_dbwd_residual_undecayed",
           "_dbwd_dalpha_no_gate_term"):
    globals()[_n].__name__ = _n


_dconv_raw_values = _patched("o, S = delta_prefill(yq, yk, yv, g, S0=S0, alpha=alpha)",
                             "o, S = delta_prefill(yq, yk, _f64(v), g, S0=S0, alpha=alpha)")
_dconv_decode_raw_query = _patched("o, S_new = delta_decode_step(yq[:, :, 0],",
                                   "o, S_new = delta_decode_step(_f64(q),")
_dconv_decode_cache_kept = _patched("return o, S_new, np.concatenate([hq, hk, hv], axis=-1)",
                                    "return o, S_new, _f64(conv_cache)")
for _n in ("_dconv_raw_values", "_dconv_decode_raw_query", "_dconv_decode_cache_kept"):
    globals()[_n].__name__ = _n


_cbwd_tap_mirrored = _patched("dfull[:, :, t + j] += W[None, :, j] * dy[:, :, t]",
                              "dfull[:, :, t + j] += W[None, :, w - 1 - j] * dy[:, :, t]")
_cbwd_weight_from_output = _patched(
    "dW[:, j] += np.sum(dy[:, :, t] * full[:, :, t + j], axis=0)",
    "dW[:, j] += np.sum(dy[:, :, t] * full[:, :, t + w - 1], axis=0)")
_cbwd_cache_grad_dropped = _patched(
    "        dfull[:, :, full.shape[2] - (w - 1):] += _f64(dcache_out)\n",
    "        pass\n")
for _n in ("_cbwd_tap_mirrored", "_cbwd_weight_from_output", "_cbwd_cache_grad_dropped"):
    globals()[_n].__name__ = _n

# backward with a per-channel decay
_gbwd_dalpha_after_state = _patched(
    'dal[:, :, t] = np.einsum("...rd,...rd->...r", Sh, Ss[t]) + zh * zs[t]',
    'dal[:, :, t] = np.einsum("...rd,...rd->...r", Sh, Ss[t + 1]) + zh * zs[t + 1]')
_gbwd_dalpha_no_z = _patched(
    'dal[:, :, t] = np.einsum("...rd,...rd->...r", Sh, Ss[t]) + zh * zs[t]',
    'dal[:, :, t] = np.einsum("...rd,...rd->...r", Sh, Ss[t])')
_gbwd_adjoint_next_decay = _patched(
    "Sh = al[:, :, t][..., None] * Sh", "Sh = al[:, :, min(t + 1, N - 1)][..., None] * Sh")
_gbwd_den_undecayed = _patched(
    "z = (gam[..., None] if al is None else al[:, :, t]) * z + fk[:, :, t]",
    "z = (gam[..., None] if al is None else 1.0) * z + fk[:, :, t]")
for _n in ("_gbwd_dalpha_after_state", "_gbwd_dalpha_no_z", "_gbwd_adjoint_next_decay",
           "_gbwd_den_undecayed"):
    globals()[_n].__name__ = _n


MUTANTS = [_read_before_write, _z_not_decayed, _eps_outside, _no_plus_one,
           _exp_everywhere, _decay_off_by_one, _outer_transposed,
           _quadratic_strict_mask, _delta_not_transposed, _delta_wrong_sign,
           _delta_output_before_update, _delta_gate_on_value_only,
           _delta_dropped_correction, _gdn_error_on_undecayed_state,
           _gdn_decay_after_write, _gdn_decay_on_write_too, _gla_decay_on_value_axis,
           _gla_decay_after_write, _conv_taps_reversed, _conv_cache_newest_first,
           _conv_cache_ignored, _conv_excludes_current_token, _conv_qk_filters_swapped,
           _bwd_dden_dropped, _bwd_dden_sign, _bwd_phi_grad_one, _bwd_adjoint_not_decayed,
           _bwd_dv_from_query, _bwd_dk_without_z, _dbwd_dk_no_state_term,
           _dbwd_adjoint_not_decayed, _dbwd_adjoint_no_projection, _dbwd_dv_without_gate,
           _dbwd_dq_from_previous_state, _dbwd_residual_undecayed, _dbwd_dalpha_no_gate_term,
           _dconv_raw_values, _dconv_decode_raw_query, _dconv_decode_cache_kept,
           _cbwd_tap_mirrored, _cbwd_weight_from_output, _cbwd_cache_grad_dropped,
           _gbwd_dalpha_after_state, _gbwd_dalpha_no_z, _gbwd_adjoint_next_decay,
           _gbwd_den_undecayed]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__.strip("_"))
def test_pins_catch_mutant(mutate):
    mod = _fresh()
    mutate(mod)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except AssertionError:  # a wrong value; any other error is a harness bug
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {mutate.__name__}"
