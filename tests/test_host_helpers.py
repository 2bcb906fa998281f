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
