"""Pins for the fp64 oracle: each function checks the oracle against something
other than itself and raises AssertionError on a mismatch.

They are collected as tests by test_oracle_pins.py and re-run against planted
mistakes by test_oracle_mutations.py, which shows that each plausible slip in
the oracle (a dropped term, a wrong sign, a transposed operand, a wrong
ordering or grouping) fails at least one pin.
"""
import json
import os

import numpy as np

from oracle import wkv7_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_problem(rng, B=1, T=6, H=2, D=3, H_kv=None, s0=True):
    H_kv = H if H_kv is None else H_kv
    r = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H_kv, D))
    v = rng.standard_normal((B, T, H_kv, D))
    w = rng.uniform(0.3, 1.0, (B, T, H, D))
    kap = rng.standard_normal((B, T, H, D))
    kap /= np.linalg.norm(kap, axis=-1, keepdims=True)
    alpha = rng.uniform(0.0, 1.0, (B, T, H, D))
    a, b = -kap, kap * alpha
    S0 = rng.standard_normal((B, H, D, D)) * 0.5 if s0 else None
    return r, w, k, v, a, b, S0


def _close(x, y, tol=1e-12, what=""):
    x, y = np.asarray(x, float), np.asarray(y, float)
    err = np.max(np.abs(x - y)) if x.size else 0.0
    scale = max(1.0, float(np.max(np.abs(y)))) if y.size else 1.0
    assert err <= tol * scale, f"{what}: max abs diff {err:.3e} (scale {scale:.3e})"


def _hand():
    with open(os.path.join(GOLDEN, "hand_example_d2.json")) as f:
        g = json.load(f)
    arr = {k: np.array(g[k], dtype=float) for k in
           ("state0", "w", "a", "b", "k", "v", "r", "r_k", "expected_y", "expected_state",
            "expected_y_epilogue")}
    return g, arr


def pin_hand_example():
    """Hand-worked two-token example (tests/golden/hand_example_d2.json)."""
    g, x = _hand()
    y, S = O.wkv7_forward(x["r"], x["w"], x["k"], x["v"], x["a"], x["b"], x["state0"])
    _close(y, x["expected_y"], 1e-15, "hand y")
    _close(S, x["expected_state"], 1e-15, "hand state")


def pin_hand_epilogue():
    """Same example with the hxa07D epilogue (y_scale = 1/2, r_k = (1, 1/2))."""
    g, x = _hand()
    y, _ = O.wkv7_forward(x["r"], x["w"], x["k"], x["v"], x["a"], x["b"], x["state0"],
                          r_k=x["r_k"], y_scale=g["y_scale"])
    _close(y, x["expected_y_epilogue"], 1e-15, "hand epilogue")


def pin_hand_logneglog():
    """Log-decay input: x = log(log(1/w)) must reproduce the decay-mode example."""
    g, x = _hand()
    lnw = np.log(np.log(1.0 / x["w"]))
    y, S = O.wkv7_forward(x["r"], lnw, x["k"], x["v"], x["a"], x["b"], x["state0"], w_mode="logneglog")
    _close(y, x["expected_y"], 1e-13, "hand logneglog y")
    _close(S, x["expected_state"], 1e-13, "hand logneglog state")


def pin_brute_force():
    """Explicit D x D transition-matrix products on tiny sizes."""
    rng = np.random.default_rng(11)
    r, w, k, v, a, b, S0 = _rand_problem(rng, B=2, T=5, H=2, D=3)
    y, S = O.wkv7_forward(r, w, k, v, a, b, S0)
    yb, Sb = O.wkv7_brute(r, w, k, v, a, b, S0)
    _close(y, yb, 1e-12, "brute y")
    _close(S, Sb, 1e-12, "brute state")


def pin_unrolled_products():
    """Closed product form S_t = S0 prod G + sum v k^T prod G, rebuilt per t."""
    rng = np.random.default_rng(12)
    r, w, k, v, a, b, S0 = _rand_problem(rng, B=1, T=6, H=2, D=4)
    y, S = O.wkv7_forward(r, w, k, v, a, b, S0)
    yu, Su = O.wkv7_unrolled(r, w, k, v, a, b, S0)
    _close(y, yu, 1e-12, "unrolled y")
    _close(S, Su, 1e-12, "unrolled state")


def pin_diagonal_decay_closed_form():
    """a = b = 0, constant per-column decay w: the RWKV-6/RetNet-style decayed sum
    y_t = sum_j r_tj (S0_ij w_j^(t+1) + sum_{s<=t} v_si k_sj w_j^(t-s))."""
    rng = np.random.default_rng(13)
    B, T, H, D = 1, 7, 2, 4
    r, _, k, v, _, _, S0 = _rand_problem(rng, B, T, H, D)
    wc = rng.uniform(0.2, 1.0, (H, D))
    w = np.broadcast_to(wc, (B, T, H, D)).copy()
    z = np.zeros((B, T, H, D))
    y, S = O.wkv7_forward(r, w, k, v, z, z, S0)
    for h in range(H):
        for t in range(T):
            St = S0[0, h] * wc[h] ** (t + 1)
            for s in range(t + 1):
                St = St + np.outer(v[0, s, h], k[0, s, h] * wc[h] ** (t - s))
            _close(y[0, t, h], St @ r[0, t, h], 1e-12, "diag decay y")
        _close(S[0, h], St, 1e-12, "diag decay state")


def pin_varying_decay_columns():
    """a = b = 0, time-varying decay: each key column decays on its own,
    S_T[:, j] = S0[:, j] prod_t w_tj + sum_i v_i k_ij prod_{s > i} w_sj."""
    rng = np.random.default_rng(14)
    B, T, H, D = 2, 6, 1, 3
    r, w, k, v, _, _, S0 = _rand_problem(rng, B, T, H, D)
    z = np.zeros_like(w)
    _, S = O.wkv7_forward(r, w, k, v, z, z, S0)
    for bb in range(B):
        for j in range(D):
            col = S0[bb, 0, :, j] * np.prod(w[bb, :, 0, j])
            for i in range(T):
                col = col + v[bb, i, 0] * k[bb, i, 0, j] * np.prod(w[bb, i + 1:, 0, j])
            _close(S[bb, 0, :, j], col, 1e-12, "column decay")


def pin_linear_attention():
    """w = 1, a = b = 0, S0 = 0: causal linear attention Y = tril(R K^T) V and the
    state is the prefix sum V^T K (youngju.dev article, linear attention)."""
    rng = np.random.default_rng(15)
    B, T, H, D = 1, 9, 3, 5
    r, _, k, v, _, _, _ = _rand_problem(rng, B, T, H, D)
    one, z = np.ones((B, T, H, D)), np.zeros((B, T, H, D))
    y, S = O.wkv7_forward(r, one, k, v, z, z, None)
    for h in range(H):
        R, K, V = r[0, :, h], k[0, :, h], v[0, :, h]
        _close(y[0, :, h], np.tril(R @ K.T) @ V, 1e-12, "linear attention y")
        _close(S[0, h], V.T @ K, 1e-12, "prefix-sum state")


def pin_overwrite_invariant():
    """alpha = 1, w = 1, added key = removal key: the delta rule overwrites the
    value stored under that key, so S_t kappa_t = v_t exactly (wiki note, delta
    rule and value replacement)."""
    rng = np.random.default_rng(16)
    B, T, H, D = 1, 8, 2, 4
    r, _, _, v, _, _, S0 = _rand_problem(rng, B, T, H, D)
    kap = rng.standard_normal((B, T, H, D))
    kap /= np.linalg.norm(kap, axis=-1, keepdims=True)
    one = np.ones((B, T, H, D))
    S = S0.copy()
    for t in range(T):
        _, S = O.wkv7_forward(r[:, t:t + 1], one[:, t:t + 1], kap[:, t:t + 1], v[:, t:t + 1],
                              -kap[:, t:t + 1], kap[:, t:t + 1], S)
        for h in range(H):
            _close(S[0, h] @ kap[0, t, h], v[0, t, h], 1e-12, "overwrite")


def pin_gqa_grouping():
    """H = 4 heads over H_kv = 2 KV heads: heads 0,1 read KV head 0 and heads 2,3
    read KV head 1 (repeat_kv, hxa07D article section 6)."""
    rng = np.random.default_rng(17)
    B, T, H, D = 1, 5, 4, 3
    r, w, k, v, a, b, _ = _rand_problem(rng, B, T, H, D, H_kv=2, s0=False)
    k[:, :, 0] = 0.0
    v[:, :, 0] = 0.0
    y, _ = O.wkv7_forward(r, w, k, v, a, b, None)
    assert np.all(y[:, :, 0:2] == 0.0), "heads 0,1 must see the zeroed KV head 0"
    assert np.all(np.abs(y[:, :, 2:4]) > 0.0), "heads 2,3 must see KV head 1"
    for h in (2, 3):
        sl = slice(h, h + 1)
        yh, _ = O.wkv7_forward(r[:, :, sl], w[:, :, sl], k[:, :, 1:2], v[:, :, 1:2],
                               a[:, :, sl], b[:, :, sl], None)
        _close(y[:, :, sl], yh, 1e-14, "gqa head")


def pin_contraction():
    """alpha = 1 and w <= 1 make G_t symmetric with eigenvalues in [-1, 1], so
    with v = 0 the Frobenius norm of the state never grows."""
    rng = np.random.default_rng(18)
    B, T, H, D = 1, 30, 2, 6
    r, w, _, _, _, _, S0 = _rand_problem(rng, B, T, H, D)
    kap = rng.standard_normal((B, T, H, D))
    kap /= np.linalg.norm(kap, axis=-1, keepdims=True)
    z = np.zeros((B, T, H, D))
    S = S0 * 4.0
    prev = np.linalg.norm(S, axis=(-2, -1))
    shrank = False
    for t in range(T):
        _, S = O.wkv7_forward(r[:, t:t + 1], w[:, t:t + 1], z[:, t:t + 1], z[:, t:t + 1],
                              -kap[:, t:t + 1], kap[:, t:t + 1], S)
        n = np.linalg.norm(S, axis=(-2, -1))
        assert np.all(n <= prev * (1 + 1e-12)), "state norm grew"
        shrank |= bool(np.any(n < prev * 0.999))
        prev = n
    assert shrank


def pin_linearity():
    """y and S_T are jointly linear in (S0, v), and y is linear in r."""
    rng = np.random.default_rng(19)
    r, w, k, v, a, b, S0 = _rand_problem(rng, B=1, T=6, H=2, D=4)
    _, _, _, v2, _, _, S02 = _rand_problem(rng, B=1, T=6, H=2, D=4)
    r2 = rng.standard_normal(r.shape)
    c1, c2 = 0.7, -1.3
    y1, S1 = O.wkv7_forward(r, w, k, v, a, b, S0)
    y2, S2 = O.wkv7_forward(r, w, k, v2, a, b, S02)
    y3, S3 = O.wkv7_forward(r, w, k, c1 * v + c2 * v2, a, b, c1 * S0 + c2 * S02)
    _close(y3, c1 * y1 + c2 * y2, 1e-12, "linear y")
    _close(S3, c1 * S1 + c2 * S2, 1e-12, "linear S")
    y4, _ = O.wkv7_forward(r2, w, k, v, a, b, S0)
    y5, _ = O.wkv7_forward(c1 * r + c2 * r2, w, k, v, a, b, S0)
    _close(y5, c1 * y1 + c2 * y4, 1e-12, "linear in r")


def pin_split_invariance():
    """Carrying the state: forward(T1) then forward(T2) from its state equals forward(T1+T2)."""
    rng = np.random.default_rng(20)
    r, w, k, v, a, b, S0 = _rand_problem(rng, B=2, T=9, H=2, D=3)
    y, S = O.wkv7_forward(r, w, k, v, a, b, S0)
    cut = 4
    ya, Sa = O.wkv7_forward(*(x[:, :cut] for x in (r, w, k, v, a, b)), S0)
    yb, Sb = O.wkv7_forward(*(x[:, cut:] for x in (r, w, k, v, a, b)), Sa)
    _close(np.concatenate([ya, yb], axis=1), y, 1e-13, "split y")
    _close(Sb, S, 1e-13, "split S")


def pin_chunked_matches_sequential():
    """The chunk-parallel algebra equals the sequential recurrence in fp64."""
    rng = np.random.default_rng(21)
    r, w, k, v, a, b, S0 = _rand_problem(rng, B=1, T=24, H=2, D=5)
    w = rng.uniform(0.55, 1.0, w.shape)
    y, S = O.wkv7_forward(r, w, k, v, a, b, S0)
    yc, Sc = O.wkv7_chunked(r, w, k, v, a, b, S0, chunk_len=8)
    _close(yc, y, 1e-11, "chunked y")
    _close(Sc, S, 1e-11, "chunked S")


def _hand_kk():
    with open(os.path.join(GOLDEN, "hand_example_kk_d2.json")) as f:
        g = json.load(f)
    arr = {k: np.array(g[k], dtype=float) for k in
           ("state0", "w", "alpha", "k", "v", "r", "r_k", "expected_y", "expected_state",
            "expected_y_epilogue")}
    return g, arr


def pin_hand_kk_mask():
    """Hand-worked kernel vectors from k, with a masked middle token
    (tests/golden/hand_example_kk_d2.json)."""
    g, x = _hand_kk()
    mask = np.array(g["mask"])
    args = (x["r"], x["w"], x["k"], x["v"], x["alpha"], None, x["state0"])
    y, S = O.wkv7_forward(*args, kk_from_k=True, mask=mask)
    _close(y, x["expected_y"], 1e-14, "hand kk y")
    _close(S, x["expected_state"], 1e-14, "hand kk state")
    y, _ = O.wkv7_forward(*args, kk_from_k=True, mask=mask, r_k=x["r_k"], y_scale=g["y_scale"])
    _close(y, x["expected_y_epilogue"], 1e-14, "hand kk epilogue")


def pin_kk_overwrite_invariant():
    """Kernel vectors from k with alpha = 1 and w = 1: k' = k and the update
    replaces what the state returns for the unit key kk, so S_t kk_t = |k_t| v_t
    (delta rule, wiki note; kk of the hxa07D article, section 8)."""
    rng = np.random.default_rng(22)
    B, T, H, D = 2, 7, 2, 5
    r, _, k, v, _, _, S0 = _rand_problem(rng, B, T, H, D)
    k *= rng.uniform(0.2, 3.0, (B, T, H, 1))
    one = np.ones((B, T, H, D))
    S = S0.copy()
    for t in range(T):
        sl = slice(t, t + 1)
        _, S = O.wkv7_forward(r[:, sl], one[:, sl], k[:, sl], v[:, sl], one[:, sl], None, S,
                              kk_from_k=True)
        n = np.linalg.norm(k[:, t], axis=-1)
        kk = k[:, t] / n[..., None]
        _close(np.einsum("bhij,bhj->bhi", S, kk), n[..., None] * v[:, t], 1e-12, "kk overwrite")


def pin_kk_key_scale():
    """From a zero state, scaling every k by c > 0 scales y and S by c: kk does
    not depend on the length of k and k' is linear in it.  A zero key row gives
    kk = 0 (the 1e-12 floor) and leaves S diag(w) with no NaN."""
    rng = np.random.default_rng(23)
    B, T, H, D = 1, 6, 2, 4
    r, w, k, v, _, _, _ = _rand_problem(rng, B, T, H, D, s0=False)
    alpha = rng.uniform(0.0, 1.0, (B, T, H, D))
    y1, S1 = O.wkv7_forward(r, w, k, v, alpha, None, None, kk_from_k=True)
    y2, S2 = O.wkv7_forward(r, w, 2.5 * k, v, alpha, None, None, kk_from_k=True)
    _close(y2, 2.5 * y1, 1e-12, "kk scale y")
    _close(S2, 2.5 * S1, 1e-12, "kk scale S")
    S0 = rng.standard_normal((B, H, D, D))
    z = np.zeros((B, 1, H, D))
    _, S = O.wkv7_forward(r[:, :1], w[:, :1], z, v[:, :1], alpha[:, :1], None, S0, kk_from_k=True)
    assert np.all(np.isfinite(S))
    _close(S, S0 * w[:, 0][:, :, None, :], 1e-15, "zero key")


def pin_mask_drops_tokens():
    """A masked token is as if it were not in the sequence: the kept tokens'
    outputs and the final state equal those of the sequence with the masked
    tokens removed, and masked positions output zero.  Covers both kernel-vector
    modes, two batch rows with different masks and a fully masked row."""
    rng = np.random.default_rng(24)
    B, T, H, D = 3, 9, 2, 3
    r, w, k, v, a, b, S0 = _rand_problem(rng, B, T, H, D)
    mask = np.ones((B, T), dtype=np.uint8)
    mask[0, [0, 3, 4, 8]] = 0
    mask[1, [5]] = 0
    mask[2, :] = 0
    for kk in (False, True):
        y, S = O.wkv7_forward(r, w, k, v, a, b, S0, kk_from_k=kk, mask=mask)
        for bi in range(B):
            keep = np.flatnonzero(mask[bi])
            assert np.all(y[bi, mask[bi] == 0] == 0.0), "masked output"
            one = lambda x: x[bi:bi + 1][:, keep]
            if keep.size:
                yk, Sk = O.wkv7_forward(one(r), one(w), one(k), one(v), one(a), one(b),
                                        S0[bi:bi + 1], kk_from_k=kk)
                _close(y[bi, keep], yk[0], 1e-13, "mask kept y")
            else:
                Sk = S0[bi:bi + 1]
            _close(S[bi], Sk[0], 1e-13, "mask state")


# ------------------------------- backward -------------------------------

def _bwd_problem(seed, B=2, T=5, H=2, H_kv=1, D=3, logneglog=False):
    rng = np.random.default_rng(seed)
    r, w, k, v, a, b, S0 = _rand_problem(rng, B, T, H, D, H_kv=H_kv)
    if logneglog:
        w = np.log(-np.log(w))
    rk = rng.standard_normal((H, D))
    dy = rng.standard_normal((B, T, H, D))
    dS = rng.standard_normal((B, H, D, D))
    return dict(r=r, w=w, k=k, v=v, a=a, b=b, state0=S0, r_k=rk), dy, dS


_ORDER = ("r", "w", "k", "v", "a", "b", "state0", "r_k")


def _loss(args, dy, dS, **kw):
    y, S = O.wkv7_forward(*(args[n] for n in _ORDER[:7]), r_k=args["r_k"], **kw)
    return float(np.sum(y * dy) + np.sum(S * dS))


def pin_bwd_finite_differences():
    """Every gradient against central differences of the forward oracle's loss
    <dy, y> + <dS, S_T> (fp64, step 1e-6), in both decay modes, with grouped KV
    heads, the epilogue, a masked token and states recomputed from checkpoints."""
    for mode, seed in (("decay", 30), ("logneglog", 31)):
        args, dy, dS = _bwd_problem(seed, logneglog=mode == "logneglog")
        mask = np.ones((2, 5), dtype=np.uint8)
        mask[1, 2] = 0
        kw = dict(w_mode=mode, y_scale=0.7, mask=mask)
        g = O.wkv7_backward(*(args[n] for n in _ORDER[:7]), dy, dS, r_k=args["r_k"], segment=2, **kw)
        h = 1e-6
        for name in _ORDER:
            arr = args[name]
            fd = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                old = arr[idx]
                arr[idx] = old + h
                lp = _loss(args, dy, dS, **kw)
                arr[idx] = old - h
                lm = _loss(args, dy, dS, **kw)
                arr[idx] = old
                fd[idx] = (lp - lm) / (2 * h)
            _close(g[name], fd, 1e-7, f"d{name} vs finite differences ({mode})")


def pin_bwd_linear_attention():
    """a = b = 0, w = 1, S0 = 0: y = tril(R K^T) V and S_T = V^T K, whose gradients
    are dR = tril(dY V^T) K, dK = tril(dY V^T)^T R + V dS, dV = tril(R K^T)^T dY
    + K dS^T and dS0 = dY^T R + dS (linear attention, Goose analysis)."""
    rng = np.random.default_rng(32)
    B, T, H, D = 1, 7, 2, 4
    r, _, k, v, _, _, _ = _rand_problem(rng, B, T, H, D, s0=False)
    z = np.zeros((B, T, H, D))
    one = np.ones((B, T, H, D))
    dy = rng.standard_normal((B, T, H, D))
    dS = rng.standard_normal((B, H, D, D))
    g = O.wkv7_backward(r, one, k, v, z, z, None, dy, dS)
    for h in range(H):
        R, K, V, dY = r[0, :, h], k[0, :, h], v[0, :, h], dy[0, :, h]
        M = np.tril(dY @ V.T)
        _close(g["r"][0, :, h], M @ K, 1e-12, "linear attention dr")
        _close(g["k"][0, :, h], M.T @ R + V @ dS[0, h], 1e-12, "linear attention dk")
        _close(g["v"][0, :, h], np.tril(R @ K.T).T @ dY + K @ dS[0, h].T, 1e-12, "linear attention dv")
        _close(g["state0"][0, h], dY.T @ R + dS[0, h], 1e-12, "linear attention dS0")


def pin_bwd_adjoint():
    """y and S_T are jointly linear in (S0, v), so <dy, y> + <dS, S_T> =
    <dS0, S0> + <dv, v> exactly (with the epilogue, grouped heads and a mask)."""
    args, dy, dS = _bwd_problem(33, T=6, D=4)
    mask = np.ones((2, 6), dtype=np.uint8)
    mask[0, 1] = 0
    kw = dict(w_mode="decay", y_scale=1.3, mask=mask)
    g = O.wkv7_backward(*(args[n] for n in _ORDER[:7]), dy, dS, r_k=args["r_k"], **kw)
    lhs = _loss(args, dy, dS, **kw)
    rhs = np.sum(g["state0"] * args["state0"]) + np.sum(g["v"] * args["v"])
    _close(rhs, lhs, 1e-12, "adjoint identity")


def pin_bwd_homogeneity():
    """y is linear in r, so <dr, r> = <dy, y>; G = diag(w) + a b^T is unchanged by
    a -> c a, b -> b / c, so <da, a> = <db, b>."""
    args, dy, dS = _bwd_problem(34, T=6, D=4)
    g = O.wkv7_backward(*(args[n] for n in _ORDER[:7]), dy, None, r_k=args["r_k"], y_scale=0.6)
    y, _ = O.wkv7_forward(*(args[n] for n in _ORDER[:7]), r_k=args["r_k"], y_scale=0.6)
    _close(np.sum(g["r"] * args["r"]), np.sum(y * dy), 1e-12, "r homogeneity")
    _close(np.sum(g["a"] * args["a"]), np.sum(g["b"] * args["b"]), 1e-12, "a/b rescaling")


def pin_bwd_log_decay_identity():
    """Writing the recurrence with r_t 2^g_t, a_t 2^g_(t-1), b_t 2^-g_t, k_t 2^-g_t
    (g the cumulative log-decay) and S_T = (...) diag(2^g_T), the gradient of each
    log-decay is a suffix sum: dL/dlog w_s = sum_(t>=s) [r dr + a_(t+1) da_(t+1)
    - b db - k dk]_t + diag(S_T^T dS) (one KV head per head, no epilogue)."""
    args, dy, dS = _bwd_problem(35, B=1, T=7, H=2, H_kv=2, D=4)
    g = O.wkv7_backward(*(args[n] for n in _ORDER[:7]), dy, dS, y_scale=0.9)
    r, w, k, a, b = (args[n] for n in ("r", "w", "k", "a", "b"))
    per_t = r * g["r"] - b * g["b"] - k * g["k"]
    per_t[:, :-1] += a[:, 1:] * g["a"][:, 1:]
    S_T = g["S_T"]
    per_t[:, -1] += np.sum(S_T * dS, axis=-2)
    suffix = np.cumsum(per_t[:, ::-1], axis=1)[:, ::-1]
    _close(g["w"] * w, suffix, 1e-12, "log-decay suffix sums")


def pin_bf16_decode():
    """bf16 bit patterns widen exactly: 0x3F80 = 1, 0xC040 = -3, 0x3EAB = 0.333984375."""
    bits = np.array([0x3F80, 0xC040, 0x3EAB, 0x0000], dtype=np.uint16)
    np.testing.assert_array_equal(O.as_f64(bits), [1.0, -3.0, 0.333984375, 0.0])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
