"""GPU parity of the RWKV-4 WKV operator (wkv4_forward, through the C ABI)
against the fp64 oracle (oracle/wkv4_oracle.py)."""
import dataclasses

import numpy as np
import pytest

from linear_rnn_sequence_wkv7_amd import inputs as G
from oracle import wkv4_oracle as O4
from tests import parity as P
from tests.gpu_util import announce, to_dev, to_host, torch

pytestmark = pytest.mark.gpu
TAU = P.TAU_SCAN   # fp32 state, one operation per token as in the scan


@pytest.fixture(autouse=True)
def _gpu_and_name(request):
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    announce(request.node.nodeid)
    yield


def W():
    from linear_rnn_sequence_wkv7_amd import wkv7
    return wkv7


def ab_of(state):
    """(A, Bs, P) -> (a, b) in float64."""
    s = np.asarray(state, dtype=np.float64)
    return s[:, 0] * np.exp(s[:, 2]), s[:, 1] * np.exp(s[:, 2])


def run(x, wl, state=None, **kw):
    y, s = W().wkv4_forward(to_dev(x["w"]), to_dev(x["u"]), to_dev(x["k"]), to_dev(x["v"]),
                            to_dev(state if state is not None else x["state"]), y_dtype=wl.y_dtype, **kw)
    torch().cuda.synchronize()
    return to_host(y), to_host(s)


def oracle(x):
    st = None if x["state"] is None else ab_of(x["state"])
    return O4.wkv4_forward(x["w"], x["u"], x["k"], x["v"], st)


SWEEP = [
    # B, T, C, in, y, state, k_offset
    (1, 1, 5, "f32", "f32", False, 0.0),
    (2, 63, 40, "bf16", "f32", True, 0.0),
    (2, 64, 256, "bf16", "bf16", False, 0.0),
    (3, 65, 300, "f32", "bf16", True, 0.0),
    (2, 200, 130, "bf16", "f32", False, 100.0),
    (1, 333, 64, "f32", "f32", True, -60.0),
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "B{}_T{}_C{}_{}_{}_s{}_k{}".format(*c))
def test_wkv4_sweep(case):
    B, T, C, i_dt, y_dt, st, ko = case
    wl = G.Wkv4Workload("t", B=B, T=T, C=C, in_dtype=i_dt, y_dtype=y_dt, seed=61 + T, state=st, k_offset=ko)
    x = G.make_wkv4_inputs(wl)
    y_ref, (a_ref, b_ref) = oracle(x)
    y, s = run(x, wl)
    e = P.check("y", y, y_ref, TAU, bf16_out=y_dt == "bf16")
    a, b = ab_of(s)
    # The state is compared as (a, b) relative to its own scale (a and b grow like e^k).
    P.check("a_T", a / b_ref.max(), a_ref / b_ref.max(), TAU)
    P.check("b_T", b / b_ref.max(), b_ref / b_ref.max(), TAU)
    announce(f"  y err/rms {e:.2e}")


def test_wkv4_lanes_outside_the_fixed_exponent_range():
    """Full chunks run the output pass with one exponent per chunk where every
    token's own terms lie within 2^100 of it, and with the running exponent
    elsewhere.  Channels here mix both forms inside one wave: a k spread of 80
    in one chunk (c = 0 mod 4), u = 45 (c = 1 mod 4), an initial state at
    e^80 (c = 2 mod 4), plain inputs (c = 3 mod 4, of which c = 7 mod 8 grow:
    w = -2, e^128 over a chunk); T = 200 adds a ragged chunk."""
    wl = G.Wkv4Workload("t", B=2, T=200, C=96, in_dtype="f32", y_dtype="f32", seed=17, state=True)
    x = G.make_wkv4_inputs(wl)
    c0, c1, c2 = np.arange(0, 96, 4), np.arange(1, 96, 4), np.arange(2, 96, 4)
    x["k"][:, 70, c0] = 40.0
    x["k"][:, 80, c0] = -40.0
    x["u"][c1] = 45.0
    x["state"][:, 2, c2] = 80.0
    x["w"][7::8] = -2.0
    y_ref, (a_ref, b_ref) = oracle(x)
    y, s = run(x, wl)
    for name, cs in (("spread", c0), ("u", c1), ("state", c2), ("plain", np.arange(3, 96, 8)),
                     ("growing", np.arange(7, 96, 8))):
        P.check(f"y {name}", y[:, :, cs], y_ref[:, :, cs], TAU)
    a, b = ab_of(s)
    for j in range(wl.C):
        sc = b_ref[:, j].max()
        P.check(f"a_T c{j}", a[:, j] / sc, a_ref[:, j] / sc, TAU)
        P.check(f"b_T c{j}", b[:, j] / sc, b_ref[:, j] / sc, TAU)


def test_wkv4_split_and_in_place():
    """Two calls carrying the state (in place) equal one call over both halves."""
    wl = G.Wkv4Workload("t", B=2, T=150, C=96, in_dtype="bf16", y_dtype="f32", seed=7, state=True)
    x = G.make_wkv4_inputs(wl)
    y_ref, _ = oracle(x)
    st = to_dev(x["state"]).clone()
    ys = []
    for sl in (slice(0, 70), slice(70, 150)):
        part = dict(x, k=np.ascontiguousarray(x["k"][:, sl]), v=np.ascontiguousarray(x["v"][:, sl]))
        y, _ = W().wkv4_forward(to_dev(part["w"]), to_dev(part["u"]), to_dev(part["k"]), to_dev(part["v"]), st,
                                y_dtype="f32", state_out=st)
        ys.append(to_host(y))
    torch().cuda.synchronize()
    P.check("y split", np.concatenate(ys, axis=1), y_ref, TAU)


def test_wkv4_zero_tokens():
    wl = G.Wkv4Workload("t", B=2, T=0, C=10, in_dtype="f32", y_dtype="f32", seed=8, state=True)
    x = G.make_wkv4_inputs(wl)
    _, s = run(x, wl)
    np.testing.assert_array_equal(s[:, :2], x["state"][:, :2].astype(np.float64))
    np.testing.assert_allclose(s[:, 2], x["state"][:, 2], rtol=1e-6, atol=1e-6)


def test_wkv4_workload():
    """The bench workload (B8 T4096 C4096, bf16), sampled channels against the oracle."""
    wl = G.WKV4_WORKLOADS["rwkv4_bf16_b8_t4096_c4096"]
    x = G.make_wkv4_inputs(wl)
    y, s = run(x, wl)
    rng = np.random.default_rng(0)
    bs = np.array([0, wl.B - 1] + list(rng.integers(0, wl.B, 4)))
    cs = np.array([0, wl.C - 1] + list(rng.integers(0, wl.C, 4)))
    for b, c in zip(bs, cs):
        sub = {"w": x["w"][c:c + 1], "u": x["u"][c:c + 1], "k": x["k"][b:b + 1, :, c:c + 1],
               "v": x["v"][b:b + 1, :, c:c + 1], "state": None}
        y_ref, (a_ref, b_ref) = oracle(sub)
        P.check(f"y b{b} c{c}", y[b:b + 1, :, c:c + 1], y_ref, TAU, bf16_out=True)
        a, bb = ab_of(s[b:b + 1, :, c:c + 1])
        P.check(f"state b{b} c{c}", np.stack([a, bb]) / b_ref.max(), np.stack([a_ref, b_ref]) / b_ref.max(), TAU)


def test_wkv4_wait_status_reports_exactly_the_waits_that_gave_up():
    """The look-back waits are bounded.  With the default bound none gives up and the
    status is OK with every output finite.  With the smallest bound (two polls) on
    a long sequence, waits may give up: the status must say so exactly when y holds
    NaN (a wait that gives up makes its chunk's y NaN in its channel, and that of
    later chunks that take their incoming state from it), and every finite output
    still matches the default run (to rounding: which earlier chunks' states a
    look-back merges depends on timing)."""
    t = torch()
    g = t.Generator(device="cuda")
    g.manual_seed(11)
    B, T, C = 4, 1 << 15, 1024
    k = t.randn((B, T, C), generator=g, device="cuda").to(t.bfloat16)
    v = t.randn((B, T, C), generator=g, device="cuda").to(t.bfloat16)
    w = t.rand((C,), generator=g, device="cuda") * 0.5
    u = t.randn((C,), generator=g, device="cuda") * 0.5
    ws = t.empty(W().wkv4_workspace_bytes(B, T, C), dtype=t.uint8, device="cuda")
    y0, _ = W().wkv4_forward(w, u, k, v, None, y_dtype="f32", workspace=ws)
    assert W().wkv4_wait_status(k, ws, y_dtype="f32") == W().WKV7_OK
    assert bool(t.isfinite(y0).all())
    gave_up = 0
    for rep in range(3):
        y1, _ = W().wkv4_forward(w, u, k, v, None, y_dtype="f32", workspace=ws, spin_limit=1)
        st = W().wkv4_wait_status(k, ws, y_dtype="f32")
        nan = t.isnan(y1)
        assert (st == W().WKV7_ETIMEOUT) == bool(nan.any()), f"status {st}, NaN {int(nan.sum())}"
        assert t.allclose(y1[~nan], y0[~nan], rtol=1e-5, atol=1e-6)
        gave_up += st == W().WKV7_ETIMEOUT
    announce(f"  smallest bound: {gave_up} of 3 calls had waits that gave up")
