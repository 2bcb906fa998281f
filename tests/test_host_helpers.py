"""Host-side helpers of the GPU tests and the benchmark (CPU only)."""
import pytest

from linear_rnn_sequence_wkv7_amd import inputs as G
from tests import parity as P


@pytest.mark.parametrize("name", list(G.WORKLOADS))
@pytest.mark.parametrize("n", [1, 2, 3, 8, 16, 128, 10 ** 6])
def test_sample_pairs_keeps_both_ends(name, n):
    wl = G.WORKLOADS[name]
    total = wl.B * wl.H
    pairs = P.sample_pairs(wl, n, seed=wl.seed)
    flat = [b * wl.H + h for b, h in pairs]
    assert len(flat) == len(set(flat)) == min(max(n, 2), total)
    assert all(0 <= i < total for i in flat)
    if total >= 2:
        assert flat[0] == 0 and flat[-1] == total - 1
    assert flat == sorted(flat)


def test_sample_pairs_spreads_over_batches_and_kv_groups():
    wl = G.WORKLOADS["hxa07d_bf16_b2_t16384_h32_kv8_d128"]
    pairs = P.sample_pairs(wl, 16, seed=wl.seed)
    rep = wl.H // wl.H_kv
    assert {b for b, _ in pairs} == set(range(wl.B))
    assert {h // rep for _, h in pairs} == set(range(wl.H_kv))
    for name in ("fwd_bf16_b8_t1024_h32_d64", "prefill_bf16_b4_t4096_h40_d64_l64"):
        wl = G.WORKLOADS[name]
        assert {b for b, _ in P.sample_pairs(wl, 16, seed=wl.seed)} == set(range(wl.B))


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 (or a multi-rank launch) exits with
    status 2 and a message, before touching any device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert r.returncode == 2, r.stderr
        assert "one GPU only" in r.stderr
        assert r.stdout.strip() == ""


def test_check_all_pairs_compares_every_pair():
    """The every-pair check (oracle in spawned workers, GPU outputs in shared memory),
    with the oracle's own outputs standing in for the GPU's: passes at fp32 rounding,
    and catches one wrong element, a non-finite value and a masked workload's pairs."""
    import numpy as np
    name = "fwd_f32_b1_t64_h2_d64"
    for ov in (dict(B=2, T=40, H=3, H_kv=3), dict(B=3, T=33, H=2, H_kv=1, mask="holes")):
        wl = G.workload(name, **ov)
        x = G.make_inputs(wl)
        pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
        y_ref, s_ref = P.oracle_pairs(x, wl, pairs)
        y = np.zeros((wl.B, wl.T, wl.H, wl.D), np.float32)
        s = np.zeros((wl.B, wl.H, wl.D, wl.D), np.float32)
        for i, (b, h) in enumerate(pairs):
            y[b, :, h] = y_ref[i]
            s[b, h] = s_ref[i]
        ey, es = P.check_all_pairs(name, ov, y, s, 1e-6, workers=2)
        assert ey < 1e-6 and es < 1e-6
    y[wl.B - 1, 5, wl.H - 1, 7] += 1.0
    with pytest.raises(AssertionError, match="y: max"):
        P.check_all_pairs(name, ov, y, s, 1e-2, workers=2)
    y[wl.B - 1, 5, wl.H - 1, 7] -= 1.0
    s[0, 0, 1, 1] = np.inf
    with pytest.raises(AssertionError, match="non-finite"):
        P.check_all_pairs(name, ov, y, s, 1e-2, workers=2)
