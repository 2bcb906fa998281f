"""The allocation-free forward entry point (wkv7_forward_noalloc) through the C
ABI: the two-pass form in the library's static device scratch, run in windows
of chunks, against the workspace entry point (wkv7_forward_ws) bit for bit and
against the fp64 oracle to the chunked-path bound."""
import numpy as np
import pytest

from linear_rnn_sequence_wkv7_amd import inputs as G
from tests import parity as P
from tests.gpu_util import announce, dev_inputs, to_host, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_and_name(request):
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    announce(request.node.nodeid)
    yield


def W():
    from linear_rnn_sequence_wkv7_amd import wkv7
    return wkv7


def _window(B, H, nch, with_state_out, D=128):
    """Chunks per (b, h) per window, as the library sizes it."""
    carry = 0 if with_state_out else (B * H * D * D * 4 + 255) // 256 * 256
    return min(nch, (W().NOALLOC_SCRATCH_BYTES - carry) // (B * H * 35584))


def _run_both(wl, x, with_state_out):
    d = dev_inputs(x)
    args = (d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"])
    kw = dict(w_mode=wl.w_mode, y_dtype="f32", y_scale=wl.y_scale, r_k=d["r_k"], ab_mode=wl.ab_mode,
              mask=d["mask"], return_state=with_state_out)
    y_ws, s_ws = W().wkv7_forward(*args, algo="two_pass", **kw)
    y_na, s_na = W().wkv7_forward_noalloc(*args, algo="two_pass", **kw)
    torch().cuda.synchronize()
    return to_host(y_ws), None if s_ws is None else to_host(s_ws), to_host(y_na), \
        None if s_na is None else to_host(s_na)


def test_noalloc_equals_workspace_entry_point_twice():
    """Two calls in a row, the second with a smaller input (and no state_out, so
    the state crosses windows through the scratch's carry area)."""
    # Call 1: hxa07D shapes at T = 4096 (B H = 64, 128 chunks): 5 windows of up to 29 chunks.
    wl = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", T=4096, s0_std=0.1)
    nch = (wl.T + 31) // 32
    win = _window(wl.B, wl.H, nch, True)
    assert 1 <= win < nch
    announce(f"call 1: B{wl.B} T{wl.T} H{wl.H}: {nch} chunks in windows of {win}")
    x = G.make_inputs(wl)
    y_ws, s_ws, y_na, s_na = _run_both(wl, x, True)
    np.testing.assert_array_equal(y_na, y_ws)
    np.testing.assert_array_equal(s_na, s_ws)
    pairs = P.sample_pairs(wl, 8, seed=wl.seed)
    y_ref, s_ref = P.oracle_pairs(x, wl, pairs)
    bs = [p[0] for p in pairs]
    hs = [p[1] for p in pairs]
    e_y = P.check("y", y_na[bs, :, hs], y_ref, P.TAU_CHUNKED)
    e_s = P.check("state", s_na[bs, hs], s_ref, P.TAU_CHUNKED)
    announce(f"  max err / rms vs oracle: y {e_y:.3e}  state {e_s:.3e}")

    # Call 2: smaller (T = 1000, ragged last chunk, grouped KV heads, a mask), no state_out.
    wl2 = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", T=1000, mask="holes")
    nch2 = (wl2.T + 31) // 32
    win2 = _window(wl2.B, wl2.H, nch2, False)
    assert 1 <= win2 < nch2
    announce(f"call 2: B{wl2.B} T{wl2.T} H{wl2.H}, no state_out: {nch2} chunks in windows of {win2}")
    x2 = G.make_inputs(wl2)
    y_ws, _, y_na, s_na = _run_both(wl2, x2, False)
    assert s_na is None
    np.testing.assert_array_equal(y_na, y_ws)
    pairs = P.sample_pairs(wl2, 6, seed=wl2.seed)
    y_ref, _ = P.oracle_pairs(x2, wl2, pairs)
    e_y = P.check("y", y_na[[p[0] for p in pairs], :, [p[1] for p in pairs]], y_ref, P.TAU_CHUNKED)
    announce(f"  max err / rms vs oracle: y {e_y:.3e}")


def test_noalloc_one_window_and_other_algorithms():
    """A call that fits one window, and a D = 64 call (no scratch: the one-pass
    chunked kernel), each equal to the ordinary entry point."""
    wl = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", B=1, T=300, H=4, H_kv=2)
    x = G.make_inputs(wl)
    y_ws, s_ws, y_na, s_na = _run_both(wl, x, True)
    np.testing.assert_array_equal(y_na, y_ws)
    np.testing.assert_array_equal(s_na, s_ws)
    wl64 = G.workload("fwd_bf16_b8_t1024_h32_d64", B=2, T=200, H=4, H_kv=4, s0_std=0.1)
    x64 = G.make_inputs(wl64)
    d = dev_inputs(x64)
    args = (d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"])
    y1, s1 = W().wkv7_forward(*args, y_dtype="f32")
    y2, s2 = W().wkv7_forward_noalloc(*args, y_dtype="f32")
    torch().cuda.synchronize()
    np.testing.assert_array_equal(to_host(y2), to_host(y1))
    np.testing.assert_array_equal(to_host(s2), to_host(s1))
