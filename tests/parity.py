"""Comparison rule for GPU results against the fp64 oracle, and helpers that
run the oracle on sampled (batch, head) pairs of a large workload."""
import numpy as np

from oracle import wkv7_oracle as O

# Tolerances on max|x - x_ref| relative to rms(x_ref).
TAU_SCAN = 5e-3      # scan and decode kernels (fp32 state)
TAU_CHUNKED = 1e-2   # chunked kernel: bf16 matrix-core operands, fp32 accumulation
BF16_HALF_ULP = 2.0 ** -8


def rms(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def check(name, got, ref, tau, bf16_out=False):
    """max|got - ref| <= tau * rms(ref), elementwise widened by the bf16
    rounding half-ulp 2^-8 |ref| when `got` was rounded to bf16.
    Returns the normalised error max|got - ref| / rms(ref)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = rms(ref)
    bound = tau * scale + (BF16_HALF_ULP * np.abs(ref) if bf16_out else 0.0)
    diff = np.abs(got - ref)
    bad = diff > bound
    if np.any(bad):
        idx = np.unravel_index(np.argmax(diff - bound), diff.shape)
        raise AssertionError(
            f"{name}: {int(bad.sum())} of {diff.size} elements out of bound; worst at {idx}: "
            f"got {got[idx]:.6g} ref {ref[idx]:.6g} (rms(ref) {scale:.4g}, tau {tau})")
    return float(diff.max() / scale) if scale > 0 else float(diff.max())


def select_pairs(x, wl, pairs):
    """Inputs of the chosen (b, h) pairs stacked along the head axis of a
    single batch: head n of the result is pair n (its KV head already picked,
    so the result has H_kv = H = len(pairs))."""
    rep = wl.H // wl.H_kv
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    hks = hs // rep
    out = {}
    for key in ("r", "w", "a", "b"):
        if x.get(key) is None:
            out[key] = None
            continue
        out[key] = np.ascontiguousarray(np.moveaxis(x[key][bs, :, hs], 0, 1)[None])   # [1, T, n, D]
    for key in ("k", "v"):
        out[key] = np.ascontiguousarray(np.moveaxis(x[key][bs, :, hks], 0, 1)[None])
    out["state0"] = None if x.get("state0") is None else x["state0"][bs, hs][None]   # [1, n, D, D]
    out["r_k"] = None if x.get("r_k") is None else x["r_k"][hs]                       # [n, D]
    return out


def oracle_pairs(x, wl, pairs):
    """Oracle y [n, T, D] and final state [n, D, D] for the chosen (b, h) pairs.
    With a mask, pairs of the same sequence run together under its mask row."""
    kk = getattr(wl, "ab_mode", "given") == "from_k"
    mask = x.get("mask")
    groups = [list(range(len(pairs)))] if mask is None else \
        [[i for i, p in enumerate(pairs) if p[0] == b] for b in sorted({p[0] for p in pairs})]
    y_out = [None] * len(pairs)
    s_out = [None] * len(pairs)
    for idx in groups:
        sel = select_pairs(x, wl, [pairs[i] for i in idx])
        m = None if mask is None else mask[pairs[idx[0]][0]][None]
        y, S = O.wkv7_forward(sel["r"], sel["w"], sel["k"], sel["v"], sel["a"], sel["b"], sel["state0"],
                              w_mode=wl.w_mode, y_scale=wl.y_scale, r_k=sel["r_k"], kk_from_k=kk, mask=m)
        for j, i in enumerate(idx):
            y_out[i] = y[0, :, j]
            s_out[i] = S[0, j]
    return np.stack(y_out), np.stack(s_out)


def sample_pairs(wl, n, seed=0):
    """min(n, B*H) distinct (b, h) pairs, stratified: the flat pair index range
    [0, B*H) is cut into that many equal strata and one pair is drawn from each,
    except that the first stratum gives pair 0 and the last gives pair B*H - 1.
    So the first and the last pair are always in, and the sample spreads over
    every batch and head range (and so over the KV groups) instead of leaning
    to one end."""
    rng = np.random.default_rng(seed)
    total = wl.B * wl.H
    n = min(max(n, 2), total)
    edges = [(i * total) // n for i in range(n + 1)]
    idx = []
    for i in range(n):
        lo, hi = edges[i], edges[i + 1]
        if i == 0:
            idx.append(0)
        elif i == n - 1:
            idx.append(total - 1)
        else:
            idx.append(int(rng.integers(lo, hi)))
    return [(i // wl.H, i % wl.H) for i in idx]


# ---------------- every (batch, head) pair, the oracle in worker processes ----------------
#
# Workers are spawned (fresh interpreters that never touch the GPU), regenerate
# the workload's inputs from its seed, run the oracle on their share of the
# pairs and compare it with the GPU outputs, which they read from shared memory.
# They return sums, so the bound uses the rms over all pairs, as check() does.

_AP = {}


def _ap_init(name, overrides, y_name, y_shape, s_name, s_shape):
    from multiprocessing import shared_memory
    from linear_rnn_sequence_wkv7_amd import inputs as G
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass
    wl = G.workload(name, **overrides)
    _AP["wl"] = wl
    _AP["x"] = G.make_inputs(wl)
    _AP["shm"] = [shared_memory.SharedMemory(name=y_name), shared_memory.SharedMemory(name=s_name)]
    _AP["y"] = np.ndarray(y_shape, dtype=np.float32, buffer=_AP["shm"][0].buf)
    _AP["s"] = np.ndarray(s_shape, dtype=np.float32, buffer=_AP["shm"][1].buf)


def _ap_work(pairs):
    wl, x = _AP["wl"], _AP["x"]
    y_ref, s_ref = oracle_pairs(x, wl, pairs)
    bs = [p[0] for p in pairs]
    hs = [p[1] for p in pairs]
    y = _AP["y"][bs, :, hs].astype(np.float64)
    s = _AP["s"][bs, hs].astype(np.float64)
    finite = bool(np.all(np.isfinite(y)) and np.all(np.isfinite(s)))
    return (float(np.abs(y - y_ref).max()), float(np.sum(y_ref * y_ref)), y_ref.size,
            float(np.abs(s - s_ref).max()), float(np.sum(s_ref * s_ref)), s_ref.size, finite)


def check_all_pairs(name, overrides, y, s, tau, workers=8):
    """GPU y [B, T, H, D] and final state [B, H, D, D] (host float32 arrays) of
    workload `name` (with `overrides`) against the oracle on every (batch, head)
    pair: max|x - x_ref| <= tau * rms(x_ref) over all pairs, for y and the state.
    Returns the two normalised errors."""
    import concurrent.futures as cf
    import multiprocessing as mp
    from multiprocessing import shared_memory
    from linear_rnn_sequence_wkv7_amd import inputs as G
    wl = G.workload(name, **overrides)
    y = np.ascontiguousarray(y, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    assert y.shape == (wl.B, wl.T, wl.H, wl.D) and s.shape == (wl.B, wl.H, wl.D, wl.D)
    shm = [shared_memory.SharedMemory(create=True, size=max(1, y.nbytes)),
           shared_memory.SharedMemory(create=True, size=max(1, s.nbytes))]
    try:
        np.ndarray(y.shape, dtype=np.float32, buffer=shm[0].buf)[...] = y
        np.ndarray(s.shape, dtype=np.float32, buffer=shm[1].buf)[...] = s
        pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
        n = max(1, min(workers, len(pairs)))
        # Pairs of one sequence stay together (a mask row is shared by them).
        shares = [pairs[i::n] for i in range(n)] if wl.mask == "" else \
            [[p for p in pairs if p[0] % n == i] for i in range(n)]
        shares = [sh for sh in shares if sh]
        # A worker that dies (or fails to start) breaks the pool with an error
        # instead of leaving the map waiting.
        with cf.ProcessPoolExecutor(len(shares), mp_context=mp.get_context("spawn"), initializer=_ap_init,
                                    initargs=(name, overrides, shm[0].name, y.shape, shm[1].name, s.shape)) as ex:
            res = list(ex.map(_ap_work, shares))
    finally:
        for m in shm:
            m.close()
            m.unlink()
    assert all(r[6] for r in res), f"{name}: non-finite GPU values"
    out = []
    for i, what in ((0, "y"), (3, "state")):
        err = max(r[i] for r in res)
        scale = float(np.sqrt(sum(r[i + 1] for r in res) / sum(r[i + 2] for r in res)))
        assert err <= tau * scale, f"{name} {what}: max|x - x_ref| {err:.4g} > {tau} * rms {scale:.4g}"
        out.append(err / scale)
    return tuple(out)
