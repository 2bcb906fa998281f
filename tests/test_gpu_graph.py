"""HIP-graph capture of the entry points.  The library only enqueues kernels on
the caller's stream (no allocation, no memset, no synchronisation), so a caller
can capture a sequence of calls once and replay it.  Each captured graph is
replayed several times, with the inputs restored and unrelated eager work run
between the replays, and every replay must reproduce the eager result (bit for
bit where the kernels are deterministic)."""
import dataclasses

import numpy as np
import pytest

from linear_rnn_sequence_wkv7_amd import inputs as G
from tests.gpu_util import announce, dev_inputs, to_dev, to_host, torch

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(autouse=True)
def _gpu_and_name(request):
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    announce(request.node.nodeid)
    yield


def W():
    from linear_rnn_sequence_wkv7_amd import wkv7
    return wkv7


def eager_noise():
    """Unrelated eager work between replays: a forward of another shape."""
    wl = G.workload("fwd_f32_b1_t64_h2_d64", T=40)
    d = dev_inputs(G.make_inputs(wl))
    W().wkv7_forward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"], algo="scan")


def check_replays(graph, reset, outputs, expected, inexact=(), rtol=1e-5):
    for rep in range(REPLAYS):
        reset()
        eager_noise()
        graph.replay()
        torch().cuda.synchronize()
        for name, t in outputs.items():
            got, ref = to_host(t), expected[name]
            if name in inexact:
                np.testing.assert_allclose(got, ref, rtol=rtol, atol=rtol * max(1.0, float(np.abs(ref).max())),
                                           err_msg=f"replay {rep}: {name}")
            else:
                np.testing.assert_array_equal(got, ref, err_msg=f"replay {rep}: {name}")


def test_graph_decode_chain():
    """Eight decode steps on one state (in place) captured as one graph."""
    wl = dataclasses.replace(G.WORKLOADS["decode_bf16_b256_h64_d64_x32"], B=4, H=8, H_kv=8, steps=8)
    x = G.make_inputs(wl)
    steps = [{n: to_dev(x[n][t]) for n in ("r", "w", "k", "v", "a", "b")} for t in range(wl.steps)]
    s0 = to_dev(x["state0"])

    def run(state, ys):
        for t, d in enumerate(steps):
            W().wkv7_decode_step(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], state, y=ys[t], state_out=state)

    st_e = s0.clone()
    ys_e = [torch().empty((wl.B, 1, wl.H, wl.D), dtype=torch().bfloat16, device="cuda") for _ in steps]
    run(st_e, ys_e)
    torch().cuda.synchronize()
    expected = {f"y{t}": to_host(y) for t, y in enumerate(ys_e)}
    expected["state"] = to_host(st_e)

    st_g = s0.clone()
    ys_g = [torch().empty_like(y) for y in ys_e]
    g = torch().cuda.CUDAGraph()
    with torch().cuda.graph(g):
        run(st_g, ys_g)
    outputs = {f"y{t}": y for t, y in enumerate(ys_g)}
    outputs["state"] = st_g
    check_replays(g, lambda: st_g.copy_(s0), outputs, expected)


@pytest.mark.parametrize("D,algo,T", [(64, "chunked", 100), (128, "two_pass", 100), (128, "two_pass", 4096)])
def test_graph_forward(D, algo, T):
    """D = 128 at T = 4096: 128 chunks per (b, h) through the two-pass form."""
    wl = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", B=2, T=T, H=4, H_kv=2, D=D)
    x = G.make_inputs(wl)
    d = dev_inputs(x)
    ws = None
    if algo == "two_pass":
        ws = torch().empty(W().wkv7_workspace_bytes(wl.B, wl.T, wl.H, wl.D, H_kv=wl.H_kv, algo=algo),
                           dtype=torch().uint8, device="cuda")

    def run(y, s):
        W().wkv7_forward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"], w_mode=wl.w_mode,
                         algo=algo, y_scale=wl.y_scale, r_k=d["r_k"], ab_mode=wl.ab_mode, y=y, state_out=s,
                         workspace=ws)

    y_e = torch().empty((wl.B, wl.T, wl.H, wl.D), dtype=torch().bfloat16, device="cuda")
    s_e = torch().empty((wl.B, wl.H, wl.D, wl.D), dtype=torch().float32, device="cuda")
    run(y_e, s_e)
    torch().cuda.synchronize()
    expected = {"y": to_host(y_e), "state": to_host(s_e)}
    y_g, s_g = torch().empty_like(y_e), torch().empty_like(s_e)
    g = torch().cuda.CUDAGraph()
    with torch().cuda.graph(g):
        run(y_g, s_g)

    def reset():
        y_g.zero_()
        s_g.zero_()
    check_replays(g, reset, {"y": y_g, "state": s_g}, expected)


def test_graph_backward():
    """The backward (forward sweep, backward sweep, group and KV sums) in one graph;
    dr_k's LDS-atomic partial sums make it equal only to rounding."""
    wl = G.workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", B=2, T=70, H=4, H_kv=2, D=64, mask="holes")
    x = G.make_inputs(wl)
    gi = G.make_grad_inputs(wl, dstate=True)
    d = dev_inputs(x)
    dy, ds = to_dev(gi["dy"]), to_dev(gi["dstate"])
    ws = torch().empty(W().wkv7_backward_workspace_bytes(wl.B, wl.T, wl.H, wl.D, H_kv=wl.H_kv,
                                                         r_k_ptr=d["r_k"].data_ptr()),
                       dtype=torch().uint8, device="cuda")

    def run(grads):
        return W().wkv7_backward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], dy, d["state0"], ds,
                                 w_mode=wl.w_mode, y_scale=wl.y_scale, r_k=d["r_k"], mask=d["mask"],
                                 workspace=ws, grads=grads)

    ref = run(None)
    torch().cuda.synchronize()
    expected = {n: to_host(t) for n, t in ref.items() if t is not None}
    grads = {n: torch().empty_like(t) for n, t in ref.items() if t is not None}
    g = torch().cuda.CUDAGraph()
    with torch().cuda.graph(g):
        run(grads)

    def reset():
        for t in grads.values():
            t.zero_()
    check_replays(g, reset, grads, expected, inexact=("r_k",))


def test_graph_wkv4():
    """RWKV-4 (reset of the published states, then the single pass) in one graph.
    Its look-back takes whichever predecessor states are published first, so the
    summation order, and the last bits, can differ between runs."""
    wl = G.Wkv4Workload("t", B=2, T=300, C=300, in_dtype="bf16", y_dtype="f32", seed=9, state=True)
    x = G.make_wkv4_inputs(wl)
    w, u, k, v, s0 = (to_dev(x[n]) for n in ("w", "u", "k", "v", "state"))
    ws = torch().empty(W().wkv4_workspace_bytes(wl.B, wl.T, wl.C, in_dtype="bf16", y_dtype="f32"),
                       dtype=torch().uint8, device="cuda")
    y_e = torch().empty((wl.B, wl.T, wl.C), dtype=torch().float32, device="cuda")
    s_e = torch().empty_like(s0)
    W().wkv4_forward(w, u, k, v, s0, y_dtype="f32", y=y_e, state_out=s_e, workspace=ws)
    torch().cuda.synchronize()
    expected = {"y": to_host(y_e), "state": to_host(s_e)}
    y_g, s_g = torch().empty_like(y_e), torch().empty_like(s_e)
    g = torch().cuda.CUDAGraph()
    with torch().cuda.graph(g):
        W().wkv4_forward(w, u, k, v, s0, y_dtype="f32", y=y_g, state_out=s_g, workspace=ws)

    def reset():
        y_g.zero_()
        s_g.zero_()
    check_replays(g, reset, {"y": y_g, "state": s_g}, expected, inexact=("y", "state"))


def test_graph_forward_bench_workload_full_size():
    """The B8 T1024 H32 D64 bf16 workload's timed region at its full size: two
    forward steps captured as one graph; every replay equals the eager launch."""
    wl = G.WORKLOADS["fwd_bf16_b8_t1024_h32_d64"]
    d = dev_inputs(G.make_inputs(wl))

    def run(y, s):
        W().wkv7_forward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"], w_mode=wl.w_mode,
                         y_dtype=wl.y_dtype, chunk_len=wl.chunk_len, y=y, state_out=s)

    y_e = torch().empty((wl.B, wl.T, wl.H, wl.D), dtype=torch().bfloat16, device="cuda")
    s_e = torch().empty((wl.B, wl.H, wl.D, wl.D), dtype=torch().float32, device="cuda")
    run(y_e, s_e)
    torch().cuda.synchronize()
    expected = {"y": to_host(y_e), "state": to_host(s_e)}
    y_g, s_g = torch().empty_like(y_e), torch().empty_like(s_e)
    g = torch().cuda.CUDAGraph()
    with torch().cuda.graph(g):
        run(y_g, s_g)
        run(y_g, s_g)

    def reset():
        y_g.zero_()
        s_g.zero_()
    check_replays(g, reset, {"y": y_g, "state": s_g}, expected)


def test_graph_forward_headline_full_size():
    """The bench's default timed region at its full size (hxa07D B2 T16384 H32 H_kv8
    D128, two-pass, workspace allocated once): two forward steps captured as one
    graph; every replay equals the eager launch bit for bit."""
    wl = G.WORKLOADS["hxa07d_bf16_b2_t16384_h32_kv8_d128"]
    d = dev_inputs(G.make_inputs(wl))
    ws = torch().empty(W().wkv7_workspace_bytes(wl.B, wl.T, wl.H, wl.D, H_kv=wl.H_kv, algo="two_pass"),
                       dtype=torch().uint8, device="cuda")

    def run(y, s):
        W().wkv7_forward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"], w_mode=wl.w_mode,
                         y_dtype=wl.y_dtype, algo="two_pass", y_scale=wl.y_scale, r_k=d["r_k"],
                         ab_mode=wl.ab_mode, y=y, state_out=s, workspace=ws)

    y_e = torch().empty((wl.B, wl.T, wl.H, wl.D), dtype=torch().bfloat16, device="cuda")
    s_e = torch().empty((wl.B, wl.H, wl.D, wl.D), dtype=torch().float32, device="cuda")
    run(y_e, s_e)
    torch().cuda.synchronize()
    expected = {"y": to_host(y_e), "state": to_host(s_e)}
    y_g, s_g = torch().empty_like(y_e), torch().empty_like(s_e)
    g = torch().cuda.CUDAGraph()
    with torch().cuda.graph(g):
        run(y_g, s_g)
        run(y_g, s_g)

    def reset():
        y_g.zero_()
        s_g.zero_()
    check_replays(g, reset, {"y": y_g, "state": s_g}, expected)
