"""Pins for the RWKV-4 WKV oracle (oracle/wkv4_oracle.py): each checks it
against something other than itself."""
import json
import os

import numpy as np

from oracle import wkv4_oracle as O4

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(x, y, tol, what):
    x, y = np.asarray(x, float), np.asarray(y, float)
    err = float(np.max(np.abs(x - y))) if x.size else 0.0
    scale = max(1.0, float(np.max(np.abs(y)))) if y.size else 1.0
    assert err <= tol * scale, f"{what}: max abs diff {err:.3e}"


def _rand(seed, B=2, T=7, C=3):
    rng = np.random.default_rng(seed)
    w = rng.uniform(0.05, 2.0, C)
    u = rng.standard_normal(C)
    k = rng.standard_normal((B, T, C))
    v = rng.standard_normal((B, T, C))
    a0 = rng.uniform(0.0, 2.0, (B, C)) * rng.standard_normal((B, C))
    b0 = rng.uniform(0.5, 2.0, (B, C))
    return w, u, k, v, (a0, b0)


def pin_wkv4_hand_example():
    """Three hand-worked tokens (tests/golden/wkv4_hand_example.json)."""
    with open(os.path.join(GOLDEN, "wkv4_hand_example.json")) as f:
        g = json.load(f)
    y, (a, b) = O4.wkv4_forward(np.array(g["w"]), np.array(g["u"]), np.array(g["k"]), np.array(g["v"]))
    _close(y, g["expected_y"], 1e-14, "hand y")
    _close(a, g["expected_a"], 1e-14, "hand a")
    _close(b, g["expected_b"], 1e-14, "hand b")


def pin_wkv4_recurrent_form():
    """The note's recurrent form: wkv_t = (a_{t-1} + e^{u+k_t} v_t) / (b_{t-1} + e^{u+k_t}),
    a_t = e^{-w} a_{t-1} + e^{k_t} v_t, b_t likewise, from a nonzero initial state."""
    w, u, k, v, st = _rand(40)
    y, (aT, bT) = O4.wkv4_forward(w, u, k, v, st)
    a, b = st[0].copy(), st[1].copy()
    for t in range(k.shape[1]):
        e = np.exp(u + k[:, t])
        _close(y[:, t], (a + e * v[:, t]) / (b + e), 1e-12, f"recurrent wkv t={t}")
        a = np.exp(-w) * a + np.exp(k[:, t]) * v[:, t]
        b = np.exp(-w) * b + np.exp(k[:, t])
    _close(aT, a, 1e-12, "recurrent a_T")
    _close(bT, b, 1e-12, "recurrent b_T")


def pin_wkv4_causal_softmax():
    """w = 0, u = 0: every past token and the current one weigh e^{k_i}, so wkv_t is
    the causal softmax average sum_{i<=t} softmax(k_{<=t})_i v_i."""
    _, _, k, v, _ = _rand(41)
    C = k.shape[2]
    y, _ = O4.wkv4_forward(np.zeros(C), np.zeros(C), k, v)
    for t in range(k.shape[1]):
        p = np.exp(k[:, :t + 1] - k[:, :t + 1].max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        _close(y[:, t], np.sum(p * v[:, :t + 1], axis=1), 1e-12, f"softmax t={t}")


def pin_wkv4_key_shift_and_constant_value():
    """Adding c to every k scales numerator and denominator alike (y unchanged, the
    zero-state sums scale by e^c); a constant v gives y = v."""
    w, u, k, v, _ = _rand(42)
    y1, (a1, b1) = O4.wkv4_forward(w, u, k, v)
    y2, (a2, b2) = O4.wkv4_forward(w, u, k + 30.0, v)
    _close(y2, y1, 1e-12, "k shift y")
    _close(a2 * np.exp(-30.0), a1, 1e-12, "k shift a")
    _close(b2 * np.exp(-30.0), b1, 1e-12, "k shift b")
    y3, _ = O4.wkv4_forward(w, u, k, np.full_like(v, 2.5))
    _close(y3, np.full_like(v, 2.5), 1e-12, "constant v")


def pin_wkv4_large_decay():
    """w -> infinity (here 60): only the previous token survives next to the current
    one, wkv_t = (e^{k_{t-1}} v_{t-1} + e^{u+k_t} v_t) / (e^{k_{t-1}} + e^{u+k_t})."""
    _, u, k, v, _ = _rand(43)
    C = k.shape[2]
    y, _ = O4.wkv4_forward(np.full(C, 60.0), u, k, v)
    for t in range(1, k.shape[1]):
        e0, e1 = np.exp(k[:, t - 1]), np.exp(u + k[:, t])
        _close(y[:, t], (e0 * v[:, t - 1] + e1 * v[:, t]) / (e0 + e1), 1e-12, f"large w t={t}")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
