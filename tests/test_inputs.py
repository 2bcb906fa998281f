"""The seeded input generator (CPU only)."""
import numpy as np
import pytest

from linear_rnn_sequence_wkv7_amd import inputs as G


def test_bf16_round_trip_and_ties():
    x = np.array([1.0, -3.0, 0.1, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 65504.0], dtype=np.float32)
    bits = G.f32_to_bf16_bits(x)
    back = G.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins; 1 + 3*2^-8 rounds up to 1 + 2^-6.
    np.testing.assert_array_equal(back[:2], [1.0, -3.0])
    assert back[3] == 1.0
    assert back[4] == np.float32(1.0 + 2.0 ** -6)
    assert abs(back[2] - 0.1) <= 0.1 * 2.0 ** -8
    rng = np.random.default_rng(0)
    y = rng.standard_normal(100000).astype(np.float32)
    err = np.abs(G.bf16_bits_to_f32(G.f32_to_bf16_bits(y)) - y)
    assert np.all(err <= np.abs(y) * 2.0 ** -8)


def test_deterministic_and_seed_sensitive():
    wl = G.workload("fwd_bf16_b8_t1024_h32_d64", B=1, T=8, H=2)
    x1, x2 = G.make_inputs(wl), G.make_inputs(wl)
    for key in ("r", "w", "k", "v", "a", "b"):
        np.testing.assert_array_equal(x1[key], x2[key])
    x3 = G.make_inputs(wl, seed=wl.seed + 1)
    assert not np.array_equal(x1["r"], x3["r"])


@pytest.mark.parametrize("name", sorted(G.WORKLOADS))
def test_shapes_and_dtypes(name):
    wl = G.WORKLOADS[name]
    small = G.workload(name, B=min(wl.B, 2), T=min(wl.T, 4), steps=min(wl.steps, 2))
    x = G.make_inputs(small)
    lead = (small.steps,) if small.kind == "decode" else ()
    dt = np.uint16 if small.in_dtype == "bf16" else np.float32
    for key in ("r", "w", "a", "b"):
        assert x[key].shape == lead + (small.B, small.T, small.H, small.D) and x[key].dtype == dt
    for key in ("k", "v"):
        assert x[key].shape == lead + (small.B, small.T, small.H_kv, small.D) and x[key].dtype == dt
    if small.s0_std > 0:
        assert x["state0"].shape == (small.B, small.H, small.D, small.D) and x["state0"].dtype == np.float32
    else:
        assert x["state0"] is None
    assert (x["r_k"] is None) == (small.rk_std == 0)


def _f(x):
    return G.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


def test_distributions():
    wl = G.workload("fwd_bf16_b8_t1024_h32_d64", B=2, T=256)
    x = G.make_inputs(wl)
    r, w, a, b = (_f(x[k]).astype(np.float64) for k in ("r", "w", "a", "b"))
    assert abs(r.mean()) < 0.02 and abs(r.std() - 1.0) < 0.02
    # decay range from the -0.5 offset: w in [exp(-exp(-0.5)), 1]
    assert w.min() >= np.exp(-np.exp(-0.5)) * (1 - 2 ** -8) and w.max() <= 1.0
    # a = -kappa with |kappa| = 1 per head; b = kappa * alpha with alpha in (0, 1)
    na = np.linalg.norm(a, axis=-1)
    assert np.allclose(na, 1.0, atol=0.02)
    ratio = np.where(np.abs(a) > 1e-2, -b / np.where(a == 0, 1, a), np.nan)
    ratio = ratio[np.isfinite(ratio)]
    assert ratio.min() > -0.02 and ratio.max() < 1.02


def test_logneglog_and_grouping():
    wl = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", T=16)
    x = G.make_inputs(wl)
    lnw = _f(x["w"]).astype(np.float64)
    assert lnw.max() <= -0.5 + 1e-2                      # -softplus(z) - 0.5 <= -0.5
    decay = np.exp(-np.exp(lnw))
    assert decay.min() >= np.exp(-np.exp(-0.5)) * (1 - 1e-2)
    # removal key is normalise(repeat_kv(k)): heads 4g..4g+3 share KV head g's key
    a = _f(x["a"]).astype(np.float64)
    k = _f(x["k"]).astype(np.float64)
    for h in range(wl.H):
        kh = k[:, :, h // 4]
        kk = kh / np.linalg.norm(kh, axis=-1, keepdims=True)
        assert np.allclose(-a[:, :, h], kk, atol=2e-2)
    assert x["r_k"].shape == (32, 128) and abs(x["r_k"].std() - 0.1) < 0.01


def test_from_k_and_masks():
    base = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", B=3, T=40)
    x = G.make_inputs(G.workload(base.name, B=3, T=40, ab_mode="from_k"))
    alpha = _f(x["a"]).astype(np.float64)
    assert x["b"] is None and alpha.min() > 0.0 and alpha.max() < 1.0
    assert x["mask"] is None
    # The draws before alpha are the same as in the given-a/b mode.
    y = G.make_inputs(base)
    for key in ("r", "k", "v", "w"):
        np.testing.assert_array_equal(x[key], y[key])
    pad = G.make_inputs(G.workload(base.name, B=3, T=40, mask="pad"))["mask"]
    assert pad.shape == (3, 40) and pad.dtype == np.uint8
    assert np.all(pad[0] == 1)
    for row in pad:                       # a kept prefix of at least half the tokens
        n = int(row.sum())
        assert n >= 20 and np.all(row[:n] == 1) and np.all(row[n:] == 0)
    holes = G.make_inputs(G.workload(base.name, B=3, T=4000, H=1, H_kv=1, mask="holes"))["mask"]
    assert abs(1.0 - holes.mean() - 0.125) < 0.01
