"""Planted mistakes in the oracle must each fail at least one pin.

Every mutation replaces one piece of oracle/wkv7_oracle.py (on the CPU, via
monkeypatch) with a plausible slip; the test passes only if some pin in
tests/oracle_pins.py then raises.
"""
import numpy as np
import pytest

from oracle import wkv7_oracle as O
from tests import oracle_pins as P


def _mm(S, x):
    return np.matmul(S, x[..., :, None])[..., 0]


def _tr(S):
    return np.swapaxes(S, -1, -2)


MUTATIONS = {
    # removal projection
    "removal_transposed": ("_removal", lambda S, a: _mm(_tr(S), a)),
    "removal_dropped": ("_removal", lambda S, a: np.zeros(S.shape[:-1])),
    # state transition
    "b_term_dropped": ("_transition", lambda S, w, sa, b, v, k: S * w[..., None, :] + v[..., :, None] * k[..., None, :]),
    "b_term_sign": ("_transition", lambda S, w, sa, b, v, k:
                    S * w[..., None, :] - sa[..., :, None] * b[..., None, :] + v[..., :, None] * k[..., None, :]),
    "b_term_outer_swapped": ("_transition", lambda S, w, sa, b, v, k:
                             S * w[..., None, :] + b[..., :, None] * sa[..., None, :] + v[..., :, None] * k[..., None, :]),
    "decay_on_rows": ("_transition", lambda S, w, sa, b, v, k:
                      S * w[..., :, None] + sa[..., :, None] * b[..., None, :] + v[..., :, None] * k[..., None, :]),
    "kv_outer_swapped": ("_transition", lambda S, w, sa, b, v, k:
                         S * w[..., None, :] + sa[..., :, None] * b[..., None, :] + k[..., :, None] * v[..., None, :]),
    "decay_dropped": ("_transition", lambda S, w, sa, b, v, k:
                      S + sa[..., :, None] * b[..., None, :] + v[..., :, None] * k[..., None, :]),
    "decay_after_add": ("_transition", lambda S, w, sa, b, v, k:
                        (S + sa[..., :, None] * b[..., None, :] + v[..., :, None] * k[..., None, :]) * w[..., None, :]),
    # readout
    "readout_transposed": ("_readout", lambda S, r: _mm(_tr(S), r)),
    "readout_before_update": ("_step", lambda S, r, w, k, v, a, b:
                              (O._transition(S, w, O._removal(S, a), b, v, k), O._readout(S, r))),
    # epilogue
    "epilogue_scale_dropped": ("_epilogue", lambda y, r, k, v, rk, ys:
                               y + (np.sum(r * k * rk, axis=-1)[..., None] * v if rk is not None else 0.0)),
    "epilogue_bonus_on_r": ("_epilogue", lambda y, r, k, v, rk, ys:
                            y * ys + (np.sum(r * k * rk, axis=-1)[..., None] * r if rk is not None else 0.0)),
    "epilogue_rk_dropped": ("_epilogue", lambda y, r, k, v, rk, ys:
                            y * ys + (np.sum(r * k, axis=-1)[..., None] * v if rk is not None else 0.0)),
    # log-decay conversion
    "logneglog_sign": ("decay_from_logneglog", lambda x: np.exp(-np.exp(-x))),
    "logneglog_single_exp": ("decay_from_logneglog", lambda x: np.exp(x)),
    # kernel vectors from k
    "kk_unnormalised": ("kernel_vectors_from_k", lambda k, w, al: (k * (1 - w + al), -k, k * al)),
    "kk_key_factor_dropped": ("kernel_vectors_from_k", lambda k, w, al: (
        k, -k / np.linalg.norm(k, axis=-1, keepdims=True), al * k / np.linalg.norm(k, axis=-1, keepdims=True))),
    "kk_key_factor_sign": ("kernel_vectors_from_k", lambda k, w, al: (
        k * (1 + w - al), -k / np.linalg.norm(k, axis=-1, keepdims=True),
        al * k / np.linalg.norm(k, axis=-1, keepdims=True))),
    "kk_b_without_alpha": ("kernel_vectors_from_k", lambda k, w, al: (
        k * (1 - w + al), -k / np.linalg.norm(k, axis=-1, keepdims=True), k / np.linalg.norm(k, axis=-1, keepdims=True))),
    "kk_a_sign": ("kernel_vectors_from_k", lambda k, w, al: (
        k * (1 - w + al), k / np.linalg.norm(k, axis=-1, keepdims=True),
        al * k / np.linalg.norm(k, axis=-1, keepdims=True))),
    # attention mask
    "mask_state_ignored": ("_masked", lambda m, So, Sn, y: (Sn, np.where(m[:, None, None], y, 0.0))),
    "mask_output_kept": ("_masked", lambda m, So, Sn, y: (np.where(m[:, None, None, None], Sn, So), y)),
    # backward
    "bwd_dr_from_previous_state": ("_bwd_token", lambda U, Sp, Sc, r, w, k, v, a, b, dyc: _patch(
        _ORIG_BWD(U, Sp, Sc, r, w, k, v, a, b, dyc), 0, np.einsum("...ij,...i->...j", Sp, dyc))),
    "bwd_dw_dropped": ("_bwd_token", lambda U, Sp, Sc, r, w, k, v, a, b, dyc: _patch(
        _ORIG_BWD(U, Sp, Sc, r, w, k, v, a, b, dyc), 1, np.zeros_like(w))),
    "bwd_dk_transposed": ("_bwd_token", lambda U, Sp, Sc, r, w, k, v, a, b, dyc: _patch(
        _ORIG_BWD(U, Sp, Sc, r, w, k, v, a, b, dyc), 2,
        np.einsum("...ij,...j->...i", U + dyc[..., :, None] * r[..., None, :], v))),
    "bwd_db_from_updated_state": ("_bwd_token", lambda U, Sp, Sc, r, w, k, v, a, b, dyc: _patch(
        _ORIG_BWD(U, Sp, Sc, r, w, k, v, a, b, dyc), 5,
        np.einsum("...ij,...i->...j", U + dyc[..., :, None] * r[..., None, :],
                  np.einsum("...ij,...j->...i", Sc, a)))),
    "bwd_state_through_G_not_transpose": ("_bwd_token", lambda U, Sp, Sc, r, w, k, v, a, b, dyc: (
        _with_U(_ORIG_BWD(U, Sp, Sc, r, w, k, v, a, b, dyc), U + dyc[..., :, None] * r[..., None, :], w, a, b))),
    "bwd_readout_before_update": ("_bwd_token", lambda U, Sp, Sc, r, w, k, v, a, b, dyc: (
        _ORIG_BWD(U, Sp, Sc, r, w, k, v, a, b, np.zeros_like(dyc))[0] + dyc[..., :, None] * r[..., None, :],
        _ORIG_BWD(U, Sp, Sc, r, w, k, v, a, b, dyc)[1])),
    "bwd_epilogue_dbeta_on_r": ("_bwd_epilogue", lambda dy, r, k, v, rk: (
        np.sum(dy * r, axis=-1)[..., None] * k * rk, np.sum(dy * v, axis=-1)[..., None] * r * rk,
        np.sum(r * k * rk, axis=-1)[..., None] * dy, np.sum(dy * v, axis=-1)[..., None] * r * k)),
    "bwd_epilogue_dv_dropped": ("_bwd_epilogue", lambda dy, r, k, v, rk: (
        np.sum(dy * v, axis=-1)[..., None] * k * rk, np.sum(dy * v, axis=-1)[..., None] * r * rk,
        0.0 * dy, np.sum(dy * v, axis=-1)[..., None] * r * k)),
    # grouped KV heads
    "gqa_interleaved": ("_expand_kv", lambda x, H: np.tile(x, (1,) * (x.ndim - 2) + (H // x.shape[-2], 1))),
}


_ORIG_BWD = O._bwd_token


def _patch(res, i, value):
    U_prev, grads = res
    grads = list(grads)
    grads[i] = value
    return U_prev, tuple(grads)


def _with_U(res, U, w, a, b):
    """Replace U_prev by U (diag(w) + a b^T), the step's own matrix instead of its transpose."""
    Ua = np.einsum("...ij,...j->...i", U, a)
    return U * w[..., None, :] + Ua[..., :, None] * b[..., None, :], res[1]


def _any_pin_fails():
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
        except (ValueError, IndexError, np.linalg.LinAlgError):
            failed.append(pin.__name__ + " (error)")
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = _any_pin_fails()
    assert failed, f"planted mistake {name!r} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    assert _any_pin_fails() == []
