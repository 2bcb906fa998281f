"""fp64 CPU oracle for the RWKV-7 "Goose" WKV recurrence (generalised delta rule).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module;
only the tests, the package smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library: it decodes bf16 itself and
reads the generator's arrays as plain data.

What it computes (per batch b and head h, state S of shape D_v x D_k,
value rows i, key columns j):

  S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T          (1)
  y_t = S_t r_t                                              (2)

(1) is the full state update of the wiki note "RWKV-7 Goose: Expressive
Dynamic State Evolution", section "generalised delta rule", written with the
kernel's vectors a = -kappa_hat and b = kappa_hat * alpha (the hxa07D article,
section 8, passes -kk and kk*a to the kernel).  (2) reads the state after the
update, as in the youngju.dev RWKV-7 article's time-mix pseudocode, where the
per-token readout einsum follows the state update.

Options, all from the hxa07D article (forward listing):
  * w_mode "logneglog": the w input holds log(-log(decay)) and the decay is
    exp(-exp(w)) (section 3, decay in log space).
  * grouped KV heads: k and v have H_kv heads and head h reads KV head
    h // (H / H_kv), i.e. repeat_kv's contiguous repetition (section 6).
  * epilogue: y_t <- y_scale * y_t + (sum_j r_tj k_tj r_k[h, j]) v_t
    (section 9: scale by head_size^-1/2 plus the r*k*r_k term times v).
  * kk_from_k: the kernel vectors are formed from k and the in-context rate
    alpha, as the forward listing does right before the kernel call (section
    8): kk = normalize(k) per head (L2, floor 1e-12), a = -kk, b = kk * alpha,
    and k itself becomes k * (1 - w + alpha) with w the decay; that modified k
    is also the k of the epilogue's r*k*r_k term.  alpha is passed in the a
    argument.
  * mask [B, T]: the listing passes an attention mask to the kernel without
    defining it; here a masked token (mask == 0) leaves the state unchanged
    and emits y = 0, so padding and variable lengths drop out.

Backward (wkv7_backward): the gradients of L = <dy, y> + <dS_T, S_T> with
respect to every input, by reverse-mode differentiation of (1), (2) and the
epilogue written out token by token (no page gives these formulas).  With
U_t = dL/dS_t, going from t = T down to 1:

  U_t += dy_t r_t^T                               (readout (2) uses S_t)
  dr_t = S_t^T dy_t,  dv_t = U_t k_t,  dk_t = U_t^T v_t
  db_t = U_t^T (S_{t-1} a_t),  da_t = S_{t-1}^T (U_t b_t)
  dw_t[j] = sum_i S_{t-1}[i, j] U_t[i, j]
  U_{t-1} = U_t (diag(w_t) + b_t a_t^T)           (the transpose of the step)

and dS_0 = U_0; dy is first scaled by y_scale, the r*k*r_k term adds its own
direct terms, grouped KV heads sum dk and dv over their group, and in the
log-decay mode dw is carried to x by d decay / dx = -exp(x) decay.

Every function here is pinned by tests/test_oracle_pins.py against things
other than itself: a hand-worked example, closed forms of special cases
(diagonal decay, linear attention / prefix sum), the delta-rule overwrite
invariant, brute-force matrix products, and structural invariants.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = [
    "as_f64", "decay_from_logneglog", "kernel_vectors_from_k", "wkv7_forward", "wkv7_backward",
    "wkv7_brute", "wkv7_unrolled", "wkv7_chunked",
]


def as_f64(x: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """Widen an input to float64.  uint16 arrays are bf16 bit patterns."""
    if x is None:
        return None
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def decay_from_logneglog(x: np.ndarray) -> np.ndarray:
    """decay = exp(-exp(x)) (hxa07D article, section 3)."""
    return np.exp(-np.exp(x))


def _expand_kv(x: np.ndarray, H: int) -> np.ndarray:
    """[.., H_kv, D] -> [.., H, D]: head h uses KV head h // (H / H_kv) (repeat_kv)."""
    H_kv = x.shape[-2]
    if H % H_kv:
        raise ValueError(f"H={H} not a multiple of H_kv={H_kv}")
    return np.repeat(x, H // H_kv, axis=-2)


# --- the three pieces of one step, kept separate so a test can plant mistakes ---

def _removal(S: np.ndarray, a: np.ndarray) -> np.ndarray:
    """sa = S a, per value row: [.., Dv, Dk] x [.., Dk] -> [.., Dv]."""
    return np.matmul(S, a[..., :, None])[..., 0]


def _transition(S, w, sa, b, v, k):
    """S diag(w) + sa b^T + v k^T  (equation (1) with S a precomputed)."""
    return S * w[..., None, :] + sa[..., :, None] * b[..., None, :] + v[..., :, None] * k[..., None, :]


def _readout(S: np.ndarray, r: np.ndarray) -> np.ndarray:
    """y = S r."""
    return np.matmul(S, r[..., :, None])[..., 0]


def _step(S, r, w, k, v, a, b):
    """One token: update (1), then read out (2) from the updated state."""
    S = _transition(S, w, _removal(S, a), b, v, k)
    return S, _readout(S, r)


def _epilogue(y, r, k, v, rk, y_scale):
    """hxa07D output: y_scale * y + (sum_j r_j k_j r_k[h, j]) v; no bonus term without r_k."""
    y = y * y_scale
    if rk is not None:
        y = y + np.sum(r * k * rk, axis=-1)[..., None] * v
    return y


def kernel_vectors_from_k(k, w, alpha):
    """kk = normalize(k) (L2 over the head, floor 1e-12); returns the kernel's
    (k * (1 - w + alpha), a = -kk, b = kk * alpha) for decay w (hxa07D article,
    forward listing, section 8).  k, w, alpha: [..., D] float64."""
    n = np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    kk = k / np.maximum(n, 1e-12)
    return k * (1.0 - w + alpha), -kk, kk * alpha


def _masked(keep, S_old, S_new, y):
    """keep [B] bool: a kept token takes the update and its output; a masked one
    keeps the old state and outputs zero."""
    return (np.where(keep[:, None, None, None], S_new, S_old),
            np.where(keep[:, None, None], y, 0.0))


def wkv7_forward(r, w, k, v, a, b, state0=None, *, w_mode: str = "decay",
                 r_k=None, y_scale: float = 1.0, kk_from_k: bool = False,
                 mask=None) -> Tuple[np.ndarray, np.ndarray]:
    """The recurrence over T tokens, token by token, in float64.

    r, w, a, b: [B, T, H, D]; k, v: [B, T, H_kv, D] (uint16 = bf16 bits, or float).
    state0: [B, H, D, D] or None (zeros).  r_k: [H, D] or None.
    kk_from_k: a holds alpha and b is ignored (see the module notes).
    mask: [B, T] (nonzero = token kept) or None.
    Returns y [B, T, H, D] and the final state [B, H, D, D], both float64.
    """
    r, w, k, v, a = (as_f64(x) for x in (r, w, k, v, a))
    B, T, H, D = r.shape
    k = _expand_kv(k, H)
    v = _expand_kv(v, H)
    if w_mode == "logneglog":
        w = decay_from_logneglog(w)
    elif w_mode != "decay":
        raise ValueError(w_mode)
    if kk_from_k:
        k, a, b = kernel_vectors_from_k(k, w, a)
    else:
        b = as_f64(b)
    keep = None if mask is None else (np.asarray(mask) != 0)
    S = np.zeros((B, H, D, D)) if state0 is None else as_f64(state0).copy()
    rk = None if r_k is None else as_f64(r_k)
    y = np.empty((B, T, H, D))
    for t in range(T):
        S_new, yt = _step(S, r[:, t], w[:, t], k[:, t], v[:, t], a[:, t], b[:, t])
        yt = _epilogue(yt, r[:, t], k[:, t], v[:, t], rk, y_scale)
        if keep is None:
            S, y[:, t] = S_new, yt
        else:
            S, y[:, t] = _masked(keep[:, t], S, S_new, yt)
    return y, S


def wkv7_brute(r, w, k, v, a, b, state0=None):
    """Equation (1) as explicit D x D matrix products, one (b, h) at a time.

    For tiny inputs only.  Builds G_t = diag(w_t) + a_t b_t^T and applies
    S <- S G_t + v_t k_t^T with pure-Python loops over tokens and elements.
    Same argument layout as wkv7_forward (decay mode, no grouping/epilogue).
    """
    r, w, k, v, a, b = (as_f64(x) for x in (r, w, k, v, a, b))
    B, T, H, D = r.shape
    y = np.zeros((B, T, H, D))
    S_out = np.zeros((B, H, D, D))
    for bb in range(B):
        for h in range(H):
            S = [[0.0] * D for _ in range(D)] if state0 is None else \
                [[float(state0[bb, h, i, j]) for j in range(D)] for i in range(D)]
            for t in range(T):
                G = [[(w[bb, t, h, i] if i == j else 0.0) + a[bb, t, h, i] * b[bb, t, h, j]
                      for j in range(D)] for i in range(D)]
                S = [[sum(S[i][m] * G[m][j] for m in range(D)) + v[bb, t, h, i] * k[bb, t, h, j]
                      for j in range(D)] for i in range(D)]
                for i in range(D):
                    y[bb, t, h, i] = sum(S[i][j] * r[bb, t, h, j] for j in range(D))
            S_out[bb, h] = np.array(S)
    return y, S_out


def wkv7_unrolled(r, w, k, v, a, b, state0=None):
    """The recurrence unrolled into products of transition matrices.

    S_t = S_0 P(0, t) + sum_{i <= t} v_i k_i^T P(i, t), with
    P(i, t) = G_{i+1} ... G_t (identity when i = t), G_s = diag(w_s) + a_s b_s^T;
    y_t = S_t r_t.  Every S_t is rebuilt from scratch (no carried state).
    """
    r, w, k, v, a, b = (as_f64(x) for x in (r, w, k, v, a, b))
    B, T, H, D = r.shape
    y = np.zeros((B, T, H, D))
    S_T = np.zeros((B, H, D, D))
    for bb in range(B):
        for h in range(H):
            G = [np.diag(w[bb, s, h]) + np.outer(a[bb, s, h], b[bb, s, h]) for s in range(T)]
            S0 = np.zeros((D, D)) if state0 is None else as_f64(state0)[bb, h]
            for t in range(T):
                P = np.eye(D)
                for s in range(0, t + 1):
                    P = P @ G[s]
                St = S0 @ P
                for i in range(t + 1):
                    Pi = np.eye(D)
                    for s in range(i + 1, t + 1):
                        Pi = Pi @ G[s]
                    St = St + np.outer(v[bb, i, h], k[bb, i, h]) @ Pi
                y[bb, t, h] = St @ r[bb, t, h]
                if t == T - 1:
                    S_T[bb, h] = St
    return y, S_T


def wkv7_chunked(r, w, k, v, a, b, state0=None, *, chunk_len: int = 64):
    """Chunk-parallel form of the same recurrence, in float64.

    The pages state only that the WKV operation parallelises over chunks
    (youngju.dev RWKV-7 article, Q&A 5); this is the algebra used by the HIP
    chunked kernel, kept here so the tests can check it against the
    sequential definition.  Within a chunk of L tokens starting from S0, with
    c_t = sum_{s<=t} log w_s (per key column), E(t, s) = exp(c_t - c_s):

      SA = (I - A_ab)^-1 (At S0^T + A_ak V)   rows sa_t = S_{t-1} a_t
      Y  = Rt S0^T + A_rb SA + A_rk V
      S_L = S0 diag(exp(c_L)) + SA^T Bh + V^T Kh

    where At_t = a_t exp(c_{t-1}), Rt_t = r_t exp(c_t),
    A_ab[t, s] = sum_j a_tj b_sj E(t-1, s)_j  (s < t),  A_ak likewise with k,
    A_rb[t, s] = sum_j r_tj b_sj E(t, s)_j    (s <= t), A_rk likewise with k,
    Bh_s = b_s exp(c_L - c_s), Kh_s = k_s exp(c_L - c_s).
    Decay mode only, no grouping or epilogue.  T must be a multiple of chunk_len.
    """
    r, w, k, v, a, b = (as_f64(x) for x in (r, w, k, v, a, b))
    B, T, H, D = r.shape
    L = chunk_len
    if T % L:
        raise ValueError("T must be a multiple of chunk_len")
    y = np.zeros((B, T, H, D))
    S_T = np.zeros((B, H, D, D))
    for bb in range(B):
        for h in range(H):
            S = np.zeros((D, D)) if state0 is None else as_f64(state0)[bb, h].copy()
            for c0 in range(0, T, L):
                sl = slice(c0, c0 + L)
                R, Wc, K, V, A, Bm = (x[bb, sl, h] for x in (r, w, k, v, a, b))
                c = np.cumsum(np.log(Wc), axis=0)                 # c_t, t = 1..L
                cprev = np.vstack([np.zeros((1, D)), c[:-1]])      # c_{t-1}
                At = A * np.exp(cprev)
                Rt = R * np.exp(c)
                E_prev = np.exp(cprev[:, None, :] - c[None, :, :])  # [t, s, j]
                E_cur = np.exp(c[:, None, :] - c[None, :, :])
                strict = np.tril(np.ones((L, L)), -1)
                incl = np.tril(np.ones((L, L)))
                A_ab = np.einsum("tj,sj,tsj->ts", A, Bm, E_prev) * strict
                A_ak = np.einsum("tj,sj,tsj->ts", A, K, E_prev) * strict
                A_rb = np.einsum("tj,sj,tsj->ts", R, Bm, E_cur) * incl
                A_rk = np.einsum("tj,sj,tsj->ts", R, K, E_cur) * incl
                SA = np.linalg.solve(np.eye(L) - A_ab, At @ S.T + A_ak @ V)
                y[bb, sl, h] = Rt @ S.T + A_rb @ SA + A_rk @ V
                dec = np.exp(c[-1][None, :] - c)                   # exp(c_L - c_s)
                S = S * np.exp(c[-1])[None, :] + SA.T @ (Bm * dec) + V.T @ (K * dec)
            S_T[bb, h] = S
    return y, S_T


# ------------------------------------ backward ------------------------------------

def _bwd_token(U, S_prev, S_cur, r, w, k, v, a, b, dyc):
    """Reverse of one token (update (1), readout (2)).  U = dL/dS_t from the
    later tokens; dyc = the gradient of this token's S_t r_t.  Returns
    dL/dS_{t-1} and the token's (dr, dw, dk, dv, da, db)."""
    U = U + dyc[..., :, None] * r[..., None, :]
    dr = np.einsum("...ij,...i->...j", S_cur, dyc)
    dv = np.einsum("...ij,...j->...i", U, k)
    dk = np.einsum("...ij,...i->...j", U, v)
    sa = np.einsum("...ij,...j->...i", S_prev, a)
    db = np.einsum("...ij,...i->...j", U, sa)
    Ub = np.einsum("...ij,...j->...i", U, b)
    da = np.einsum("...ij,...i->...j", S_prev, Ub)
    dw = np.sum(S_prev * U, axis=-2)
    U_prev = U * w[..., None, :] + Ub[..., :, None] * a[..., None, :]
    return U_prev, (dr, dw, dk, dv, da, db)


def _bwd_epilogue(dy, r, k, v, rk):
    """Direct terms of y += (sum_j r_j k_j rk_j) v: returns (dr, dk, dv, drk)."""
    beta = np.sum(r * k * rk, axis=-1)[..., None]
    dbeta = np.sum(dy * v, axis=-1)[..., None]
    return dbeta * k * rk, dbeta * r * rk, beta * dy, dbeta * r * k


def wkv7_backward(r, w, k, v, a, b, state0, dy, dstate=None, *, w_mode: str = "decay",
                  r_k=None, y_scale: float = 1.0, mask=None, segment: int = 256):
    """Gradients of L = <dy, y> + <dstate, S_T> for the forward wkv7_forward
    computes with the same arguments (kernel vectors given as a, b).

    dy: [B, T, H, D]; dstate: [B, H, D, D] or None (zero).  Returns a dict with
    r, w, a, b [B, T, H, D], k, v [B, T, H_kv, D] (summed over each KV group),
    state0 [B, H, D, D] and r_k [H, D] (None without r_k); dw is with respect to
    the w input in its own mode.  States are kept at every `segment`-th token
    and recomputed in between, so memory stays bounded on long sequences.
    """
    r, w_in, k_kv, v_kv, a, b = (as_f64(x) for x in (r, w, k, v, a, b))
    dy = as_f64(dy)
    B, T, H, D = r.shape
    H_kv = k_kv.shape[-2]
    k = _expand_kv(k_kv, H)
    v = _expand_kv(v_kv, H)
    if w_mode == "logneglog":
        w = decay_from_logneglog(w_in)
    elif w_mode == "decay":
        w = w_in
    else:
        raise ValueError(w_mode)
    keep = np.ones((B, T), dtype=bool) if mask is None else (np.asarray(mask) != 0)
    rk = None if r_k is None else as_f64(r_k)
    S0 = np.zeros((B, H, D, D)) if state0 is None else as_f64(state0).copy()

    def advance(S, t):
        S_new, _ = _step(S, r[:, t], w[:, t], k[:, t], v[:, t], a[:, t], b[:, t])
        return np.where(keep[:, t][:, None, None, None], S_new, S)

    # Forward: checkpoints at t = 0, segment, 2 segment, ...
    ckpt = {}
    S = S0
    for t in range(T):
        if t % segment == 0:
            ckpt[t] = S
        S = advance(S, t)
    S_T = S

    g = {name: np.zeros((B, T, H, D)) for name in ("r", "w", "k", "v", "a", "b")}
    drk = None if rk is None else np.zeros((H, D))
    U = np.zeros((B, H, D, D)) if dstate is None else as_f64(dstate).copy()
    for t0 in reversed(range(0, T, segment)):
        t1 = min(t0 + segment, T)
        states = [ckpt[t0]]                      # states[i] = S_{t0 + i} (before token t0 + i)
        for t in range(t0, t1):
            states.append(advance(states[-1], t))
        for t in reversed(range(t0, t1)):
            m = keep[:, t]
            dyt = np.where(m[:, None, None], dy[:, t], 0.0)
            U_prev, grads = _bwd_token(U, states[t - t0], states[t - t0 + 1], r[:, t], w[:, t], k[:, t],
                                       v[:, t], a[:, t], b[:, t], dyt * y_scale)
            U = np.where(m[:, None, None, None], U_prev, U)
            for name, x in zip(("r", "w", "k", "v", "a", "b"), grads):
                g[name][:, t] = np.where(m[:, None, None], x, 0.0)
            if rk is not None:
                er, ek, ev, erk = _bwd_epilogue(dyt, r[:, t], k[:, t], v[:, t], rk)
                g["r"][:, t] += er
                g["k"][:, t] += ek
                g["v"][:, t] += ev
                drk += erk.sum(axis=0)
    if w_mode == "logneglog":
        g["w"] = g["w"] * w * -np.exp(w_in)
    rep = H // H_kv
    out = {name: g[name] for name in ("r", "w", "a", "b")}
    out["k"] = g["k"].reshape(B, T, H_kv, rep, D).sum(axis=3)
    out["v"] = g["v"].reshape(B, T, H_kv, rep, D).sum(axis=3)
    out["state0"] = U
    out["r_k"] = drk
    out["S_T"] = S_T
    return out
