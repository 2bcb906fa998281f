"""GPU parity of the two input options of the hxa07D forward (zenn.dev hxa07D
article, section 8): kernel vectors formed from k in the kernel (ab_mode
"from_k": a carries alpha, b is unused) and the attention mask (a masked
token leaves the state unchanged and outputs zero), against the fp64 oracle.
"""
import dataclasses

import numpy as np
import pytest

from linear_rnn_sequence_wkv7_amd import inputs as G
from oracle import wkv7_oracle as O
from tests import parity as P
from tests.gpu_util import announce, dev_inputs, to_dev, to_host, torch

pytestmark = pytest.mark.gpu

TAU = {"scan": P.TAU_SCAN, "chunked": P.TAU_CHUNKED, "two_pass": P.TAU_CHUNKED}


@pytest.fixture(autouse=True)
def _gpu_and_name(request):
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    announce(request.node.nodeid)
    yield


def W():
    from linear_rnn_sequence_wkv7_amd import wkv7
    return wkv7


def make_case(D, B, T, H, H_kv, in_dtype, y_dtype, w_mode, s0, epi, ab_mode, mask, seed):
    return G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", B=B, T=T, H=H, H_kv=H_kv, D=D, in_dtype=in_dtype,
                      y_dtype=y_dtype, w_mode=w_mode, s0_std=s0, rk_std=0.1 if epi else 0.0,
                      y_scale=D ** -0.5 if epi else 1.0, kk_from_k=True, ab_mode=ab_mode, mask=mask,
                      seed=seed)


def edge_mask(m):
    """Sharpen a generated mask: sequence 1 fully masked, sequence 2 has its first
    and last tokens masked (chunk edges), the rest as drawn."""
    m = m.copy()
    if m.shape[0] > 1:
        m[1] = 0
    if m.shape[0] > 2:
        m[2, 0] = 0
        m[2, -1] = 0
    return m


def oracle(wl, x):
    return O.wkv7_forward(x["r"], x["w"], x["k"], x["v"], x["a"], x["b"], x["state0"], w_mode=wl.w_mode,
                          r_k=x["r_k"], y_scale=wl.y_scale, kk_from_k=wl.ab_mode == "from_k",
                          mask=x["mask"])


def run(wl, x, algo):
    d = dev_inputs(x)
    y, s = W().wkv7_forward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"], w_mode=wl.w_mode,
                            y_dtype=wl.y_dtype, algo=algo, y_scale=wl.y_scale, r_k=d["r_k"],
                            ab_mode=wl.ab_mode, mask=d["mask"])
    torch().cuda.synchronize()
    return to_host(y), to_host(s)


def supported(algo, D, ab_mode):
    if algo == "two_pass" and D != 128:
        pytest.skip("the two-pass form exists for D = 128 only")
    return True


SWEEP = [
    # D, B, T, H, H_kv, in, y, w_mode, s0_std, epilogue, ab_mode, mask
    (64, 3, 150, 2, 1, "bf16", "f32", "logneglog", 0.1, True, "from_k", "holes"),
    (64, 3, 150, 2, 2, "bf16", "bf16", "decay", 0.0, False, "given", "holes"),
    (64, 3, 131, 2, 2, "f32", "f32", "decay", 0.1, True, "from_k", "pad"),
    (64, 2, 64, 3, 3, "bf16", "f32", "decay", 0.1, False, "from_k", ""),
    (128, 3, 100, 4, 2, "bf16", "f32", "logneglog", 0.1, True, "from_k", "holes"),
    (128, 3, 100, 2, 2, "bf16", "bf16", "logneglog", 0.0, True, "given", "pad"),
    (128, 3, 70, 2, 2, "f32", "f32", "decay", 0.1, False, "from_k", "pad"),
    (128, 2, 33, 8, 2, "bf16", "f32", "logneglog", 0.1, True, "from_k", ""),
]


@pytest.mark.parametrize("algo", ["scan", "chunked", "two_pass"])
@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "D{}_B{}_T{}_H{}_kv{}_{}_{}_{}_s{}_e{}_{}_{}".format(*c))
def test_mask_and_from_k(case, algo):
    wl = make_case(*case, seed=31 + case[2])
    x = G.make_inputs(wl)
    if x["mask"] is not None:
        x["mask"] = edge_mask(x["mask"])
    if not supported(algo, wl.D, wl.ab_mode):
        with pytest.raises(W().Wkv7Error) as e:
            run(wl, x, algo)
        assert e.value.code == W().WKV7_EUNSUPPORTED
        return
    y_ref, s_ref = oracle(wl, x)
    y, s = run(wl, x, algo)
    P.check("y", y, y_ref, TAU[algo], bf16_out=wl.y_dtype == "bf16")
    P.check("state", s, s_ref, TAU[algo])
    if x["mask"] is not None:
        # Masked tokens output exactly zero; a fully masked sequence keeps its state bit for bit.
        assert np.all(y[x["mask"] == 0] == 0.0)
        s0 = np.zeros_like(s[1]) if x["state0"] is None else x["state0"][1].astype(np.float64)
        np.testing.assert_array_equal(s[1], s0)


@pytest.mark.parametrize("algo", ["scan", "chunked", "two_pass"])
def test_mask_equals_dropping_tokens(algo):
    """Running with a mask equals running the kept tokens alone (per sequence)."""
    supported(algo, 128, "given")
    wl = make_case(128, 2, 96, 2, 2, "bf16", "f32", "decay", 0.1, True, "given", "holes", seed=77)
    x = G.make_inputs(wl)
    y, s = run(wl, x, algo)
    for b in range(wl.B):
        keep = np.flatnonzero(x["mask"][b])
        sub = {k: None if x[k] is None else np.ascontiguousarray(x[k][b:b + 1][:, keep])
               for k in ("r", "w", "k", "v", "a", "b")}
        sub["state0"] = x["state0"][b:b + 1]
        sub["r_k"] = x["r_k"]
        sub["mask"] = None
        wl1 = dataclasses.replace(wl, B=1, T=len(keep), mask="")
        y1, s1 = run(wl1, sub, algo)
        P.check("kept y", y[b:b + 1][:, keep], y1, TAU[algo])
        P.check("state", s[b:b + 1], s1, TAU[algo])


DECODE_SWEEP = [
    # D, B, H, H_kv, in, y, w_mode, s0_std, epilogue, ab_mode
    (64, 6, 5, 5, "bf16", "f32", "decay", 0.1, False, "from_k"),
    (64, 6, 4, 2, "f32", "bf16", "logneglog", 0.1, True, "given"),
    (128, 6, 4, 1, "bf16", "f32", "logneglog", 0.1, True, "from_k"),
    (128, 5, 2, 2, "f32", "f32", "decay", 0.1, False, "from_k"),
]


@pytest.mark.parametrize("case", DECODE_SWEEP, ids=lambda c: "D{}_B{}_H{}_kv{}_{}_{}_{}_s{}_e{}_{}".format(*c))
def test_decode_mask_and_from_k(case):
    D, B, H, H_kv, i_dt, y_dt, wm, s0, epi, ab = case
    wl = make_case(D, B, 1, H, H_kv, i_dt, y_dt, wm, s0, epi, ab, "", seed=41 + B)
    x = G.make_inputs(wl)
    x["mask"] = np.array([[1], [0], [1], [0], [1], [1]][:B], dtype=np.uint8)
    y_ref, s_ref = oracle(wl, x)
    d = dev_inputs(x)
    y, s = W().wkv7_decode_step(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"], w_mode=wm,
                                y_dtype=y_dt, y_scale=wl.y_scale, r_k=d["r_k"], ab_mode=ab, mask=d["mask"])
    torch().cuda.synchronize()
    y, s = to_host(y), to_host(s)
    P.check("decode y", y, y_ref, P.TAU_SCAN, bf16_out=y_dt == "bf16")
    P.check("decode state", s, s_ref, P.TAU_SCAN)
    assert np.all(y[1] == 0.0) and np.all(y[3] == 0.0)
    np.testing.assert_array_equal(s[1], x["state0"][1].astype(np.float64))


@pytest.mark.parametrize("algo", ["scan", "chunked", "two_pass"])
def test_workload_hxa07d_from_k(algo):
    """The hxa07D long-context workload with the kernel vectors formed in the
    kernel, sampled (batch, head) pairs, in the launch configuration the
    benchmark times."""
    wl = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", ab_mode="from_k")
    x = G.make_inputs(wl)
    pairs = P.sample_pairs(wl, 8, seed=wl.seed)
    announce(f"{wl.name} from_k algo={algo} pairs={len(pairs)}")
    y, s = run(wl, x, algo)
    y_ref, s_ref = P.oracle_pairs(x, wl, pairs)
    bs = [p[0] for p in pairs]
    hs = [p[1] for p in pairs]
    e_y = P.check("y", y[bs, :, hs], y_ref, TAU[algo], bf16_out=True)
    e_s = P.check("state", s[bs, hs], s_ref, TAU[algo])
    announce(f"  max err / rms: y {e_y:.3e}  state {e_s:.3e}")


@pytest.mark.parametrize("y_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("algo", ["scan", "chunked"])
def test_workload_fwd_from_k(algo, y_dtype):
    """B8 T1024 H32 D64 with the kernel vectors formed in the kernel (alpha in the a
    slot), 16 sampled sequences, in the launch configuration the benchmark times."""
    wl = G.workload("fwd_bf16_b8_t1024_h32_d64", ab_mode="from_k", y_dtype=y_dtype)
    x = G.make_inputs(wl)
    pairs = P.sample_pairs(wl, 16, seed=wl.seed)
    announce(f"{wl.name} from_k algo={algo} y={y_dtype} pairs={len(pairs)}")
    y, s = run(wl, x, algo)
    y_ref, s_ref = P.oracle_pairs(x, wl, pairs)
    bs = [p[0] for p in pairs]
    hs = [p[1] for p in pairs]
    e_y = P.check("y", y[bs, :, hs], y_ref, TAU[algo], bf16_out=y_dtype == "bf16")
    e_s = P.check("state", s[bs, hs], s_ref, TAU[algo])
    announce(f"  max err / rms: y {e_y:.3e}  state {e_s:.3e}")


@pytest.mark.parametrize("algo", ["scan", "chunked", "two_pass"])
def test_workload_hxa07d_padded(algo):
    """hxa07D shapes with right-padded sequences (mask recipe "pad") at T = 4096."""
    wl = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", T=4096, mask="pad")
    x = G.make_inputs(wl)
    assert x["mask"].sum() < x["mask"].size   # sequence 1 is padded
    pairs = P.sample_pairs(wl, 6, seed=wl.seed)
    y, s = run(wl, x, algo)
    y_ref, s_ref = P.oracle_pairs(x, wl, pairs)
    bs = [p[0] for p in pairs]
    hs = [p[1] for p in pairs]
    P.check("y", y[bs, :, hs], y_ref, TAU[algo], bf16_out=True)
    P.check("state", s[bs, hs], s_ref, TAU[algo])
    assert np.all(y[x["mask"] == 0] == 0.0)
