"""The two-pass D = 128 form gives the same results bit for bit however its
chunks are scheduled: one window with state_out written, one window without it,
in place (state_out == state_in), and the allocation-free entry point's
windows of its static scratch, with the state passed between windows in fp32.
Every chunk is computed by the same instructions in all of them.  The oracle
comparison of these paths is in the parity tests."""
import pytest

from linear_rnn_sequence_wkv7_amd import inputs as G
from tests.gpu_util import announce, dev_inputs, torch

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


CASES = [
    # B, T, H, H_kv, ab_mode, mask
    (2, 4096, 32, 8, "given", ""),
    (1, 2048, 16, 4, "from_k", "holes"),
    (2, 6000, 8, 8, "from_k", "pad"),     # ragged last chunk, uneven windows
    (1, 16384, 4, 1, "given", ""),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_T{}_H{}_kv{}_{}_{}".format(*c))
def test_two_pass_schedules_agree(case):
    B, T, H, H_kv, ab, mask = case
    wl = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", B=B, T=T, H=H, H_kv=H_kv, ab_mode=ab, mask=mask,
                    s0_std=0.1)
    d = dev_inputs(G.make_inputs(wl))
    kw = dict(w_mode=wl.w_mode, y_scale=wl.y_scale, r_k=d["r_k"], ab_mode=ab, mask=d["mask"], algo="two_pass")
    args = [d[n] for n in ("r", "w", "k", "v", "a", "b", "state0")]
    y_st, s_st = W().wkv7_forward(*args, **kw)                       # one window, state written
    y_one, none = W().wkv7_forward(*args, return_state=False, **kw)    # one window, no state_out
    y_na, s_na = W().wkv7_forward_noalloc(*args, **{k: v for k, v in kw.items() if k != "algo"})
    s_in = d["state0"].clone()
    y_ip, s_ip = W().wkv7_forward(*args[:-1], s_in, state_out=s_in, **kw)   # in place
    torch().cuda.synchronize()
    assert none is None
    assert torch().equal(y_st, y_one), "y differs with and without state_out"
    assert torch().equal(y_st, y_na), "one window and the allocation-free windows differ in y"
    assert torch().equal(s_st, s_na), "one window and the allocation-free windows differ in the state"
    assert torch().equal(y_st, y_ip) and torch().equal(s_st, s_ip), "in-place state differs"
    announce(f"  B{B} T{T} H{H}: one window == without state_out == allocation-free windows == in place")


def test_two_pass_follows_the_callers_stream():
    """Work queued before the call on the caller's (non-default) stream is seen
    by both passes, and work queued after it sees the call's outputs (the
    workspace allocated on that stream, too)."""
    t = torch()
    wl = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", B=1, T=4096, H=16, H_kv=4, s0_std=0.1)
    d = dev_inputs(G.make_inputs(wl))
    kw = dict(w_mode=wl.w_mode, y_scale=wl.y_scale, r_k=d["r_k"], algo="two_pass")
    ref_y, ref_s = W().wkv7_forward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"], **kw)
    t.cuda.synchronize()
    st = t.cuda.Stream()
    with t.cuda.stream(st):
        # Inputs produced on the stream just before the call (from zeros), the outputs
        # consumed on it just after.
        v2, s02 = t.zeros_like(d["v"]), t.zeros_like(d["state0"])
        v2.copy_(d["v"])
        s02.copy_(d["state0"])
        y, s = W().wkv7_forward(d["r"], d["w"], d["k"], v2, d["a"], d["b"], s02, **kw)
        y2, s2 = y.clone(), s.clone()
    st.synchronize()
    assert t.equal(y2, ref_y) and t.equal(s2, ref_s)
