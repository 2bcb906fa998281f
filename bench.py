#!/usr/bin/env python3
"""Benchmark: one step = one wkv7_forward over the whole synthetic batch.

Default workload: the hxa07D-style long-context forward, B=2, T=16384, H=32,
8 KV heads (GQA x4), D=128, log-decay input, fused epilogue (y_scale =
128^-1/2, r_k bonus term), bf16 inputs and y, fp32 state, zero initial state;
at D = 128 the two-pass chunked form runs (two kernels per step, workspace
allocated before the timed region; the roofline covers the whole step).
Inputs are resident in HBM before the timed region; K steps are bracketed by a
device synchronisation on both sides and timed with HIP events on the stream
the kernels are launched on.  The K steps are captured once into a HIP graph
and the timed region replays it (--no-graph launches each step from the host
instead).

Prints one JSON line with the throughput (head-tokens/s), the roofline of the
dominant kernel and the fp64 CPU oracle timed on a bounded sample over a pool
of host processes (run before the GPU is touched).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--algo auto|scan|chunked|two_pass]
                    [--ab-mode given|from_k] [--mask pad|holes] [--backward]
                    [--cpu-pairs N] [--cpu-workers N]

--workload fwd_bf16_b8_t1024_h32_d64 (and the other names in inputs.WORKLOADS
and inputs.WKV4_WORKLOADS) selects another workload.  --ab-mode from_k passes
alpha in place of a and no b: the kernels form a = -kk, b = kk alpha and
k (1 - decay + alpha) themselves.  --mask adds an attention mask drawn by the
named recipe.  --backward times wkv7_backward (every input gradient, dS0 and
dr_k) for the workload, with seeded upstream gradients dy and dS_T resident
before the timed region.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "wkv7 head-tokens/sec + % of binding VALU/HBM roofline, 1×MI355X"
PEAK_FP32_VALU_TFLOPS = 157.3     # MI355X fp32 vector peak (AMD spec)
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E peak (AMD spec)
PEAK_BF16_MFMA_TFLOPS = 2500.0    # dense bf16 matrix peak

KERNEL_SOURCES = {
    "scan": "linear_rnn_sequence_wkv7_amd/csrc/wkv7_scan.hip",
    "chunked": "linear_rnn_sequence_wkv7_amd/csrc/wkv7_chunked.hip",
    "chunked128": "linear_rnn_sequence_wkv7_amd/csrc/wkv7_chunked128.hip",
    "twopass128": ("linear_rnn_sequence_wkv7_amd/csrc/wkv7_twopass128.hip",
                   "linear_rnn_sequence_wkv7_amd/csrc/wkv7_twopass128_scan.hip",
                   "linear_rnn_sequence_wkv7_amd/csrc/wkv7_twopass128.h"),
    "decode": "linear_rnn_sequence_wkv7_amd/csrc/wkv7_decode.hip",
    "backward": "linear_rnn_sequence_wkv7_amd/csrc/wkv7_backward.hip",
    "wkv4": "linear_rnn_sequence_wkv7_amd/csrc/wkv4.hip",
}


def source_sha(kind: str) -> str:
    h = hashlib.sha256()
    srcs = KERNEL_SOURCES[kind]
    for rel in (*((srcs,) if isinstance(srcs, str) else srcs), "linear_rnn_sequence_wkv7_amd/csrc/wkv7_device.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl) -> int:
    """Bytes the operation must move per launch: inputs read once (k, v once
    per KV head), y written once, the state read (if given) and written once."""
    sin = 2 if wl.in_dtype == "bf16" else 4
    sy = 2 if wl.y_dtype == "bf16" else 4
    ht = wl.B * wl.T * wl.H
    n_q = 3 if wl.ab_mode == "from_k" else 4         # r, w, a (, b)
    per_tok = wl.H * wl.D * (n_q * sin + sy) + wl.H_kv * wl.D * 2 * sin + (1 if wl.mask else 0)
    state = wl.B * wl.H * wl.D * wl.D * 4 * (2 if wl.s0_std > 0 else 1)
    rk = wl.H * wl.D * 4 if wl.rk_std > 0 else 0
    return wl.B * wl.T * per_tok + state + rk if ht else 0


def workload_label(wl) -> str:
    """The workload's name plus its input options (kernel vectors from k, mask recipe)."""
    return wl.name + ("+from_k" if wl.ab_mode == "from_k" else "") + (f"+mask_{wl.mask}" if wl.mask else "")


def algorithmic_flops(wl) -> int:
    """9 D^2 per head-token: S a (2 D^2), the update (5 D^2), S r (2 D^2)."""
    return 9 * wl.D * wl.D * wl.B * wl.T * wl.H


def backward_flops(wl) -> int:
    """28 D^2 per head-token: the token-level reverse step (U += dy r^T, S^T dy, U k,
    U^T v, S a, U^T sa, U b, S^T Ub, sum S * U: 2 D^2 each; U diag(w) + Ub a^T: 3 D^2)
    plus recomputing the state (7 D^2)."""
    return 28 * wl.D * wl.D * wl.B * wl.T * wl.H


def backward_bytes(wl) -> int:
    """Inputs and dy read once, the seven gradients written once (fp32), dS_T read
    and dS0 written."""
    sin = 2 if wl.in_dtype == "bf16" else 4
    sy = 2 if wl.y_dtype == "bf16" else 4
    per_tok = wl.H * wl.D * (4 * sin + sy + 4 * 4) + wl.H_kv * wl.D * 2 * (sin + 4)
    state = wl.B * wl.H * wl.D * wl.D * 4 * (3 if wl.s0_std > 0 else 2)
    return wl.B * wl.T * per_tok + state


def traffic_from_profile(kind: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs (FETCH_SIZE
    plus WRITE_SIZE, each scaled by what the counter reads for a plain copy of
    known size), or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(kind):
        return None
    return int(rec["hbm_bytes_per_launch"])


# ------------------------- CPU oracle baseline -------------------------
#
# The fp64 oracle, as it stands, on a bounded sample of the workload's
# (batch, head) sequences, spread over a pool of worker processes (one BLAS
# thread each).  The pool is forked before this process touches the GPU.

_CPU_JOB = {}


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:     # the pool still runs; BLAS may use more threads
        pass


def _cpu_noop(_):
    return os.getpid()


# The forward sample's oracle outputs come back at every REF_TOKEN_STRIDE-th token
# (and the final states), for the parity figures of the bench line.
REF_TOKEN_STRIDE = 16


def _cpu_work(pairs):
    """Oracle work on one share of the sampled pairs; returns its compute time and,
    for the forward, the oracle's y at every REF_TOKEN_STRIDE-th token and the
    final states of the share."""
    import numpy as np
    from oracle import wkv7_oracle as O
    from tests import parity as P
    kind, wl, x, gi = _CPU_JOB["kind"], _CPU_JOB["wl"], _CPU_JOB["x"], _CPU_JOB["gi"]
    t0 = time.perf_counter()
    if kind == "forward":
        y_ref, s_ref = P.oracle_pairs(x, wl, pairs)
        dt = time.perf_counter() - t0
        return dt, np.ascontiguousarray(y_ref[:, ::REF_TOKEN_STRIDE]), s_ref
    elif kind == "decode":
        # Successive decode tokens from the same state: one forward over the steps.
        bs = np.array([p[0] for p in pairs])
        hs = np.array([p[1] for p in pairs])
        hks = hs // (wl.H // wl.H_kv)
        seq = {}
        for n in ("r", "w", "a", "b", "k", "v"):
            if x.get(n) is None:
                seq[n] = None
                continue
            cols = hks if n in ("k", "v") else hs
            seq[n] = np.ascontiguousarray(x[n][:, bs, 0, cols][None])   # [1, steps, pairs, D]
        s0 = None if x.get("state0") is None else x["state0"][bs, hs][None]
        r_k = None if x.get("r_k") is None else x["r_k"][hs]
        O.wkv7_forward(seq["r"], seq["w"], seq["k"], seq["v"], seq["a"], seq["b"], s0, w_mode=wl.w_mode,
                       r_k=r_k, y_scale=wl.y_scale, kk_from_k=wl.ab_mode == "from_k")
    elif kind == "backward":
        # Each pair with its own KV head, so grouped heads are not summed: the
        # same work per head-token.
        sel = P.select_pairs(x, wl, pairs)
        bs = np.array([p[0] for p in pairs])
        hs = np.array([p[1] for p in pairs])
        dy = np.ascontiguousarray(np.moveaxis(gi["dy"][bs, :, hs], 0, 1)[None])
        ds = gi["dstate"][bs, hs][None]
        O.wkv7_backward(sel["r"], sel["w"], sel["k"], sel["v"], sel["a"], sel["b"], sel["state0"], dy, ds,
                        w_mode=wl.w_mode, r_k=sel["r_k"], y_scale=wl.y_scale)
    else:
        raise ValueError(kind)
    return time.perf_counter() - t0, None, None


def default_cpu_workers() -> int:
    """Host cores this process may use, capped at 16 (one GPU's share of a host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(kind: str, wl, x, gi, n_pairs: int, workers: int):
    """Time the oracle on n_pairs sampled sequences split over `workers` forked
    processes.  The value is head-tokens of the sample over the wall time of the
    parallel region (pool already started).  Returns the baseline record and, for
    the forward, the oracle outputs of the sample ({"pairs", "y", "s"}; y at every
    REF_TOKEN_STRIDE-th token), else None."""
    import multiprocessing as mp
    from tests import parity as P
    pairs = P.sample_pairs(wl, n_pairs, seed=wl.seed)[:n_pairs]
    n_w = max(1, min(workers, len(pairs)))
    shares = [pairs[i::n_w] for i in range(n_w)]
    _CPU_JOB.update(kind=kind, wl=wl, x=x, gi=gi)
    ctx = mp.get_context("fork")
    with ctx.Pool(n_w, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_noop, range(n_w), chunksize=1)
        t0 = time.perf_counter()
        res = pool.map(_cpu_work, shares, chunksize=1)
        dt = time.perf_counter() - t0
    _CPU_JOB.clear()
    busy = [r[0] for r in res]
    ref = None
    if kind == "forward":
        import numpy as np
        ref = {"pairs": [p for sh in shares for p in sh], "y": np.concatenate([r[1] for r in res]),
               "s": np.concatenate([r[2] for r in res])}
    steps = wl.steps if kind == "decode" else wl.T
    what = {"forward": "whole sequences", "decode": f"sequences x all {wl.steps} decode steps",
            "backward": "whole sequences, backward"}[kind]
    return {"value": len(pairs) * steps / dt, "unit": "head-tokens/s", "cores": n_w, "kind": "oracle",
            "sample": f"{len(pairs)} of {wl.B * wl.H} (batch, head) {what} ({steps} tokens each), fp64 numpy, "
                      f"{n_w} worker processes with one BLAS thread each, "
                      f"{dt:.1f} s wall, {sum(busy):.1f} s of worker compute"}, ref


# Parity bound of the forward kernels: max|x - x_ref| <= tau rms(x_ref), widened by
# the bf16 half-ulp 2^-8 |x_ref| elementwise for a bf16 y.
PARITY_TAU = {"scan": 5e-3, "chunked": 1e-2, "chunked128": 1e-2, "twopass128": 1e-2}


def forward_parity(kind, ref, y, s_out, y_bf16: bool):
    """The GPU forward's y (at the sample's tokens) and final states against the
    oracle outputs of the CPU baseline's sample."""
    import numpy as np
    import torch
    bs = torch.tensor([p[0] for p in ref["pairs"]], device=y.device)
    hs = torch.tensor([p[1] for p in ref["pairs"]], device=y.device)
    yg = y[bs, ::REF_TOKEN_STRIDE, hs].double().cpu().numpy()
    sg = s_out[bs, hs].double().cpu().numpy()
    tau = PARITY_TAU[kind]
    out = {"pairs": len(ref["pairs"]), "token_stride": REF_TOKEN_STRIDE, "tau": tau, "bf16_y_allowance": y_bf16}
    ok = True
    for name, got, want, allow in (("y", yg, ref["y"], y_bf16), ("state", sg, ref["s"], False)):
        scale = float(np.sqrt(np.mean(want * want)))
        diff = np.abs(got - want)
        bound = tau * scale + (2.0 ** -8 * np.abs(want) if allow else 0.0)
        out[f"{name}_max_err_over_rms"] = float(diff.max() / scale)
        ok = ok and bool(np.all(np.isfinite(got))) and bool(np.all(diff <= bound))
    out["within_bound"] = ok
    return out


def run_wkv4(a, wl, G, wkv7, torch, np):
    """RWKV-4 WKV workload: one step = one wkv4_forward over the batch."""
    x = G.make_wkv4_inputs(wl)

    def dev(arr):
        if arr is None:
            return None
        if arr.dtype == np.uint16:
            return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(arr).cuda()

    d = {k: dev(v) for k, v in x.items()}
    y = torch.empty((wl.B, wl.T, wl.C), dtype=torch.bfloat16 if wl.y_dtype == "bf16" else torch.float32, device="cuda")
    s_out = torch.empty((wl.B, 3, wl.C), dtype=torch.float32, device="cuda")
    ws = torch.empty(wkv7.wkv4_workspace_bytes(wl.B, wl.T, wl.C, in_dtype=wl.in_dtype, y_dtype=wl.y_dtype),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def one_step():
        wkv7.wkv4_forward(d["w"], d["u"], d["k"], d["v"], d["state"], y_dtype=wl.y_dtype, y=y, state_out=s_out,
                          workspace=ws)
    ms_total, t_wall = time_steps(torch, a, lambda i: one_step(), stream)
    ms = ms_total / a.steps
    sin = 2 if wl.in_dtype == "bf16" else 4
    sy = 2 if wl.y_dtype == "bf16" else 4
    # Algorithmic bytes: k, v read once, y written once, w and u, the final state written.
    nbytes = wl.B * wl.T * wl.C * (2 * sin + sy) + 2 * wl.C * 4 + wl.B * 3 * wl.C * 4 * (2 if wl.state else 1)
    ht = wl.B * wl.T * wl.C
    achieved = nbytes / (ms / 1e3) / 1e9
    out = {
        "metric": "rwkv4 wkv channel-tokens/sec + % of HBM roofline, 1xMI355X", "value": ht / (ms / 1e3),
        "unit": "channel-tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "C": wl.C, "io_dtype": wl.in_dtype,
                   "y_dtype": wl.y_dtype, "kernel": "wkv4"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_from_profile("wkv4", wl.name),
                     "kernel": "wkv4", "algorithmic_bytes": nbytes},
        "wall_s_timed_region": t_wall, "launch": "hip_graph" if a.graph else "host_per_step",
    }
    if a.cpu_pairs is None or a.cpu_pairs > 0:
        from oracle import wkv4_oracle as O4
        n = min(8 if a.cpu_pairs is None else a.cpu_pairs, 8)
        t0 = time.perf_counter()
        y_ref, _ = O4.wkv4_forward(x["w"][:n], x["u"][:n], x["k"][:1, :, :n], x["v"][:1, :, :n])
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n * wl.T / dt, "unit": "channel-tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} channels of batch 0 x all {wl.T} tokens (the oracle evaluates "
                                         f"the sum definition, O(T^2) per channel), fp64 numpy, {dt:.1f} s"}
        # The GPU's y of the same channels (from the zero state, as the oracle) against it.
        got = y[:1, :, :n].double().cpu().numpy()
        scale = float(np.sqrt(np.mean(y_ref * y_ref)))
        diff = np.abs(got - y_ref)
        bound = PARITY_TAU["scan"] * scale + (2.0 ** -8 * np.abs(y_ref) if wl.y_dtype == "bf16" else 0.0)
        out["parity"] = {"channels": n, "tau": PARITY_TAU["scan"], "bf16_y_allowance": wl.y_dtype == "bf16",
                         "y_max_err_over_rms": float(diff.max() / scale),
                         "within_bound": bool(np.all(np.isfinite(got)) and np.all(diff <= bound))}
    else:
        out["cpu_baseline"] = None
        out["parity"] = None
    print(json.dumps(out), flush=True)
    return 0


def time_steps(torch, a, one_step, stream):
    """Warm-up steps, then the timed region: a.steps steps between two HIP events
    on the stream the kernels run on, with a synchronisation on both sides.  By
    default the a.steps launches are captured once, before the timed region, into
    one HIP graph and the timed region is that graph's replay: the same kernels on
    the same inputs, with the host's per-launch dispatch taken out (--no-graph
    launches each step from the host instead)."""
    for i in range(a.warmup):
        one_step(i)
    torch.cuda.synchronize()
    graph = None
    if a.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(a.steps):
                one_step(i)
        graph.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(a.steps):
            one_step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1), time.perf_counter() - t_wall


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="hxa07d_bf16_b2_t16384_h32_kv8_d128")
    ap.add_argument("--algo", default="auto", choices=["auto", "scan", "chunked", "two_pass"])
    ap.add_argument("--ab-mode", default="given", choices=["given", "from_k"])
    ap.add_argument("--mask", default="", choices=["", "pad", "holes"])
    ap.add_argument("--backward", action="store_true", help="time wkv7_backward instead of the forward")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch each timed step from the host instead of replaying them as one captured HIP graph")
    ap.add_argument("--cpu-pairs", type=int, default=None,
                    help="sequences in the CPU-oracle sample (0: skip; default: a per-workload sample of "
                         "roughly 10-30 s of oracle work)")
    ap.add_argument("--cpu-workers", type=int, default=None,
                    help="worker processes of the CPU-oracle baseline (default: usable host cores, at most 16)")
    ap.add_argument("--decode-states", type=int, default=4,
                    help="decode workloads: independent state sets used round robin, each updated in place")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (a reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    a = ap.parse_args(argv)
    if a.decode_states < 1:
        ap.error("--decode-states must be at least 1")

    if a.copy_calibration_mib > 0:
        import torch
        n = a.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_mib": a.copy_calibration_mib, "copies": 3}), flush=True)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}); "
              "every (batch, head) pair is independent, so a multi-GPU run would shard the batch, "
              "which is not implemented.", file=sys.stderr)
        return 2

    import numpy as np  # noqa: F401

    from linear_rnn_sequence_wkv7_amd import inputs as G

    workers = a.cpu_workers or default_cpu_workers()
    if a.workload in G.WKV4_WORKLOADS:
        import torch
        from linear_rnn_sequence_wkv7_amd import wkv7
        torch.cuda.set_device(0)
        return run_wkv4(a, G.WKV4_WORKLOADS[a.workload], G, wkv7, torch, np)
    wl = dataclasses.replace(G.WORKLOADS[a.workload], ab_mode=a.ab_mode, mask=a.mask)
    if a.backward and wl.kind != "forward":
        print("--backward needs a forward workload", file=sys.stderr)
        return 2
    label = workload_label(wl)
    x = G.make_inputs(wl)
    gi = G.make_grad_inputs(wl) if a.backward else None

    # The CPU-oracle baseline runs first, in processes forked before any GPU call.
    base_kind = "backward" if a.backward else wl.kind
    n_cpu = a.cpu_pairs
    if n_cpu is None:
        # About 10-30 s of oracle work in total, spread over the workers.
        n_cpu = {"forward": 256 if wl.D == 64 else 16, "decode": 16384,
                 "backward": 4 * workers if wl.D == 64 else workers}[base_kind]
    cpu, ref = cpu_baseline(base_kind, wl, x, gi, n_cpu, workers) if n_cpu > 0 else (None, None)

    import torch

    from linear_rnn_sequence_wkv7_amd import wkv7

    torch.cuda.set_device(0)

    def dev(arr):
        if arr is None:
            return None
        if arr.dtype == np.uint16:
            return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(arr).cuda()

    d = {k: dev(v) for k, v in x.items()}
    stream = torch.cuda.current_stream()

    if a.backward:
        kind = "backward"
        dy, dst = dev(gi["dy"]), dev(gi["dstate"])
        ws_bytes = wkv7.wkv7_backward_workspace_bytes(
            wl.B, wl.T, wl.H, wl.D, H_kv=wl.H_kv, in_dtype=wl.in_dtype, y_dtype=wl.y_dtype, w_mode=wl.w_mode,
            r_k_ptr=None if d["r_k"] is None else d["r_k"].data_ptr())
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        f32 = dict(dtype=torch.float32, device="cuda")
        grads = {n: torch.empty((wl.B, wl.T, wl.H, wl.D), **f32) for n in ("r", "w", "a", "b")}
        grads.update({n: torch.empty((wl.B, wl.T, wl.H_kv, wl.D), **f32) for n in ("k", "v")})
        grads["state"] = torch.empty((wl.B, wl.H, wl.D, wl.D), **f32)
        if d["r_k"] is not None:
            grads["r_k"] = torch.empty((wl.H, wl.D), **f32)

        def one_step(i):
            wkv7.wkv7_backward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], dy, d["state0"], dst,
                               w_mode=wl.w_mode, y_scale=wl.y_scale, r_k=d["r_k"], mask=d["mask"],
                               workspace=ws, grads=grads)
        head_tokens_per_step = wl.B * wl.T * wl.H
        nbytes = backward_bytes(wl)
        flops = backward_flops(wl)
    elif wl.kind == "decode":
        kind = "decode"
        # a.decode_states independent state sets (the layers of a model), each
        # updated in place, used round robin: a step's state was last touched
        # decode_states - 1 steps earlier, with (decode_states - 1) x 2 x 256 MiB
        # of other state traffic in between, so with 4 sets it is not served from
        # the 256 MB memory-side cache.
        bufs = [d["state0"]] + [d["state0"].clone() for _ in range(a.decode_states - 1)]
        y = torch.empty((wl.B, 1, wl.H, wl.D), dtype=torch.bfloat16, device="cuda")
        n_steps_avail = wl.steps

        def one_step(i):
            st = bufs[i % len(bufs)]
            j = i % n_steps_avail
            wkv7.wkv7_decode_step(*(None if d[k] is None else d[k][j] for k in ("r", "w", "k", "v", "a", "b")),
                                  st, w_mode=wl.w_mode, y_scale=wl.y_scale, r_k=d["r_k"], y=y, state_out=st,
                                  ab_mode=wl.ab_mode, mask=None if d["mask"] is None else d["mask"][j])
        head_tokens_per_step = wl.B * wl.H
        n_q = 4 if wl.ab_mode == "from_k" else 5          # r, w, a (, b) and y
        nbytes = wl.B * wl.H * (2 * wl.D * wl.D * 4) + wl.B * wl.D * (wl.H * n_q + wl.H_kv * 2) * 2
        flops = 9 * wl.D * wl.D * wl.B * wl.H
    else:
        req = a.algo if a.algo != "auto" else wl.algo
        kw = dict(H_kv=wl.H_kv, in_dtype=wl.in_dtype, y_dtype=wl.y_dtype, w_mode=wl.w_mode, ab_mode=wl.ab_mode)
        ws_bytes = wkv7.wkv7_workspace_bytes(wl.B, wl.T, wl.H, wl.D, algo=req, **kw)
        algo = "two_pass" if ws_bytes > 0 else wkv7.wkv7_resolve_algo(wl.B, wl.T, wl.H, wl.D, algo=req, **kw)
        kind = {"two_pass": "twopass128", "chunked": "chunked128" if wl.D == 128 else "chunked"}.get(algo, algo)
        y = torch.empty((wl.B, wl.T, wl.H, wl.D), dtype=torch.bfloat16 if wl.y_dtype == "bf16" else torch.float32,
                        device="cuda")
        s_out = torch.empty((wl.B, wl.H, wl.D, wl.D), dtype=torch.float32, device="cuda")
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes > 0 else None

        def one_step(i):
            wkv7.wkv7_forward(d["r"], d["w"], d["k"], d["v"], d["a"], d["b"], d["state0"], w_mode=wl.w_mode,
                              y_dtype=wl.y_dtype, algo=algo, chunk_len=wl.chunk_len, y_scale=wl.y_scale,
                              r_k=d["r_k"], y=y, state_out=s_out, workspace=ws, ab_mode=wl.ab_mode,
                              mask=d["mask"])
        head_tokens_per_step = wl.B * wl.T * wl.H
        nbytes = algorithmic_bytes(wl)
        flops = algorithmic_flops(wl)

    ms_total, t_wall = time_steps(torch, a, one_step, stream)
    # One launch per step (two for the two-pass form, timed together): the step's average duration.
    ms = ms_total / a.steps

    value = head_tokens_per_step / (ms / 1e3)
    if kind == "backward":
        # fp32 throughout, on fp32 matrix cores: the fp32 peak (157.3 TFLOP/s, the same for VALU and MFMA).
        achieved = flops / (ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_FP32_VALU_TFLOPS}
        dtype = "f32"
    elif kind != "decode":
        # Forward: the algorithmic work (9 D^2 flop per head-token) binds on the fp32
        # vector ALU (intensity ~40 flop/B at D = 64, ~104 at D = 128).
        achieved = flops / (ms / 1e3) / 1e12
        roof = {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_FP32_VALU_TFLOPS}
        dtype = "f32" if kind == "scan" else "bf16"
    else:
        achieved = nbytes / (ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
        dtype = "f32"
    roof["traffic"] = traffic_from_profile(kind, label)
    roof["kernel"] = kind
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = flops
    roof["valu_frac"] = flops / (ms / 1e3) / 1e12 / PEAK_FP32_VALU_TFLOPS
    roof["hbm_frac"] = nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS

    out = {
        "metric": METRIC, "value": value, "unit": "head-tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": label, "B": wl.B, "T": wl.T, "H": wl.H, "H_kv": wl.H_kv, "D": wl.D,
                   "io_dtype": wl.in_dtype, "y_dtype": wl.y_dtype, "kernel": kind,
                   **({"state_sets": a.decode_states} if kind == "decode" else {})},
        "roofline": roof,
        "wall_s_timed_region": t_wall, "launch": "hip_graph" if a.graph else "host_per_step",
    }
    out["cpu_baseline"] = cpu
    # The forward's outputs after the timed steps (each step recomputes them from
    # the same inputs) against the oracle outputs of the CPU sample.
    out["parity"] = forward_parity(kind, ref, y, s_out, wl.y_dtype == "bf16") if ref is not None else None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
