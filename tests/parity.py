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
    """n distinct (b, h) pairs, always including the first and the last."""
    rng = np.random.default_rng(seed)
    total = wl.B * wl.H
    idx = set([0, total - 1])
    idx |= set(rng.choice(total, size=min(n, total), replace=False).tolist())
    idx = sorted(idx)[:max(n, 2)]
    return [(i // wl.H, i % wl.H) for i in idx]
