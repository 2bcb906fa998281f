"""fp64 CPU oracle for the RWKV-4 WKV operator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only the tests and the benchmark's CPU-baseline leg use it.  It shares no
code with the HIP library.

What it computes, per batch b and channel c, over tokens t = 1 .. T (the SSM
note "RWKV: state-space based sequence model", time-mixing section, the WKV
operator):

  wkv_t = (sum_{i<t} e^{-(t-1-i) w + k_i} v_i + e^{u + k_t} v_t)
        / (sum_{i<t} e^{-(t-1-i) w + k_i}     + e^{u + k_t})

with a per-channel decay rate w and bonus u.  An initial state (a_0, b_0) (the
numerator and denominator sums before token 1, as in the note's recurrent form
a_t = e^{-w} a_{t-1} + e^{k_t} v_t, b_t = e^{-w} b_{t-1} + e^{k_t}) enters as
e^{-(t-1) w} a_0 and e^{-(t-1) w} b_0.  The oracle evaluates the sums as
written, token by token; it returns y = wkv and the final (a_T, b_T).

Pinned by tests/test_wkv4_pins.py: a hand-worked example, the note's recurrent
form, the causal softmax it reduces to at w = u = 0, invariance under
k -> k + c, constant v, and the large-w limit.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = ["as_f64", "wkv4_forward"]


def as_f64(x: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """Widen to float64; uint16 arrays are bf16 bit patterns."""
    if x is None:
        return None
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _past_weights(t: int, w, ek):
    """Weights e^{-(t-1-i) w + k_i} of the tokens i < t (0-based) seen from token t: [B, t, C]."""
    lag = (t - 1 - np.arange(t))[None, :, None]
    return np.exp(-lag * w[None, None, :]) * ek[:, :t]


def _state_decay(n: int, w):
    """e^{-n w}: the initial state seen n tokens later."""
    return np.exp(-n * w)[None, :]


def wkv4_forward(w, u, k, v, state0: Optional[Tuple[np.ndarray, np.ndarray]] = None):
    """w, u: [C]; k, v: [B, T, C]; state0: (a_0, b_0) each [B, C] or None (zeros).
    Returns y [B, T, C] and (a_T, b_T), all float64."""
    w, u, k, v = (as_f64(x) for x in (w, u, k, v))
    B, T, C = k.shape
    a0 = np.zeros((B, C)) if state0 is None else as_f64(state0[0])
    b0 = np.zeros((B, C)) if state0 is None else as_f64(state0[1])
    y = np.empty((B, T, C))
    ek = np.exp(k)
    for t in range(T):
        wt = _past_weights(t, w, ek)
        # the initial state is the sum before token 1: at token t (0-based) it has decayed t times
        carry = _state_decay(t, w)
        num = np.sum(wt * v[:, :t], axis=1) + carry * a0 + np.exp(u + k[:, t]) * v[:, t]
        den = np.sum(wt, axis=1) + carry * b0 + np.exp(u + k[:, t])
        y[:, t] = num / den
    wT = _past_weights(T, w, ek)
    a_T = np.sum(wT * v, axis=1) + _state_decay(T, w) * a0
    b_T = np.sum(wT, axis=1) + _state_decay(T, w) * b0
    return y, (a_T, b_T)
