"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before touching any device (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

from linear_rnn_sequence_wkv7_amd import wkv7 as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(W.lib_path()), reason="libwkv7.so not built")


def declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(wkv[47]_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) >= {"wkv7_forward", "wkv7_decode_step"}
    lib = W.load_library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(names) == set(W.EXPORTED_SYMBOLS)


def test_abi_version_and_strerror():
    lib = W.load_library()
    assert lib.wkv7_abi_version() == 6
    assert lib.wkv7_strerror(0) == b"ok"
    assert lib.wkv7_strerror(W.WKV7_EINVAL) == b"invalid argument"
    assert lib.wkv7_strerror(99) == b"unknown status"


FAKE = 0x10000   # aligned, never dereferenced: every case below fails validation first


def _call(desc, ptrs=None, fn="wkv7_forward"):
    lib = W.load_library()
    p = ptrs or {}
    args = [p.get(k, FAKE) for k in ("r", "w", "k", "v", "a", "b")] + \
           [p.get("s0"), p.get("y", FAKE + 4096), p.get("s1")]
    if fn == "wkv7_forward_ws":
        args += [p.get("ws"), p.get("ws_bytes", 0)]
    return getattr(lib, fn)(ctypes.byref(desc) if desc is not None else None, *args, None)


def good(**kw):
    d = dict(B=2, T=8, H=4, D=64)
    d.update(kw)
    return W.make_desc(d.pop("B"), d.pop("T"), d.pop("H"), d.pop("D"), **d)


@pytest.mark.parametrize("desc,code", [
    (None, W.WKV7_EINVAL),
    (good(D=96), W.WKV7_EUNSUPPORTED),
    (good(D=0), W.WKV7_EINVAL),
    (good(B=-1), W.WKV7_EINVAL),
    (good(T=-3), W.WKV7_EINVAL),
    (good(H=4, H_kv=3), W.WKV7_EINVAL),
    (good(H=4, H_kv=8), W.WKV7_EINVAL),
    (good(chunk_len=32), W.WKV7_EUNSUPPORTED),
    (good(D=128, chunk_len=64), W.WKV7_EUNSUPPORTED),
])
def test_bad_descriptor_rejected(desc, code):
    assert _call(desc) == code
    assert _call(desc, fn="wkv7_forward_ws") == code
    assert _call(desc, fn="wkv7_decode_step") == code


def test_bad_enums():
    d = good(); d.in_dtype = 7
    assert _call(d) == W.WKV7_EINVAL
    d = good(); d.w_mode = 2
    assert _call(d) == W.WKV7_EINVAL
    d = good(); d.algo = 9
    assert _call(d) == W.WKV7_EINVAL
    d = good(); d.ab_mode = 2
    assert _call(d) == W.WKV7_EINVAL
    assert b"ab_mode" in W.load_library().wkv7_last_error()
    d = good(); d.y_scale = float("nan")
    assert _call(d) == W.WKV7_EINVAL
    assert b"y_scale" in W.load_library().wkv7_last_error()


@pytest.mark.parametrize("key", ["r", "w", "k", "v", "a", "b", "y"])
def test_null_and_misaligned_pointers(key):
    assert _call(good(), {key: None}) == W.WKV7_EINVAL
    assert _call(good(), {key: FAKE + 8}) == W.WKV7_EINVAL
    assert _call(good(), {"s0": FAKE + 4}) == W.WKV7_EINVAL
    assert _call(good(), {"s1": FAKE + 4}) == W.WKV7_EINVAL


def test_y_aliasing_input_rejected():
    assert _call(good(), {"y": FAKE}) == W.WKV7_EINVAL


def test_decode_needs_one_token_and_state_out():
    assert _call(good(T=2), fn="wkv7_decode_step") == W.WKV7_EINVAL
    assert _call(good(T=1), fn="wkv7_decode_step") == W.WKV7_EINVAL  # state_out NULL


def test_empty_problem_is_a_no_op():
    # B*H == 0 returns before any device call.
    assert _call(good(B=0)) == W.WKV7_OK
    assert _call(good(H=0)) == W.WKV7_OK
    assert _call(good(B=0, T=1), {"s1": FAKE + 8192}, fn="wkv7_decode_step") == W.WKV7_OK


def test_resolve_algo():
    assert W.wkv7_resolve_algo(2, 8, 4, 64, algo="scan") == "scan"
    assert W.wkv7_resolve_algo(2, 8, 4, 64, algo="chunked") == "chunked"
    # AUTO: chunked once T covers one chunk (64 tokens at D = 64, 32 at D = 128).
    assert W.wkv7_resolve_algo(2, 63, 4, 64) == "scan"
    assert W.wkv7_resolve_algo(2, 64, 4, 64) == "chunked"
    assert W.wkv7_resolve_algo(2, 31, 4, 128) == "scan"
    assert W.wkv7_resolve_algo(2, 32, 4, 128) == "chunked"
    assert W.wkv7_resolve_algo(2, 32, 4, 128, chunk_len=32) == "chunked"
    with pytest.raises(W.Wkv7Error):
        W.wkv7_resolve_algo(2, 8, 4, 128, chunk_len=64)
    with pytest.raises(W.Wkv7Error):
        W.wkv7_resolve_algo(2, 8, 4, 96)


def test_workspace_bytes():
    rec = 35584   # one record per (b, h, chunk of 32 tokens)
    assert W.wkv7_workspace_bytes(2, 64, 4, 128) == 2 * 4 * 2 * rec
    assert W.wkv7_workspace_bytes(2, 70, 4, 128) == 2 * 4 * 3 * rec     # ragged last chunk
    assert W.wkv7_workspace_bytes(2, 31, 4, 128) == 0                  # AUTO: the scan below one chunk
    assert W.wkv7_workspace_bytes(2, 31, 4, 128, algo="two_pass") == 2 * 4 * 1 * rec
    assert W.wkv7_workspace_bytes(2, 0, 4, 128, algo="two_pass") == 0
    assert W.wkv7_workspace_bytes(2, 64, 4, 128, algo="chunked") == 0
    assert W.wkv7_workspace_bytes(2, 64, 4, 128, algo="scan") == 0
    assert W.wkv7_workspace_bytes(2, 128, 4, 64) == 0                  # D = 64 has no two-pass form
    assert W.wkv7_workspace_bytes(2, 16384, 32, 128, H_kv=8) == 2 * 32 * 512 * rec
    with pytest.raises(W.Wkv7Error) as e:
        W.wkv7_workspace_bytes(2, 64, 4, 64, algo="two_pass")
    assert e.value.code == W.WKV7_EUNSUPPORTED


def test_two_pass_argument_rules():
    d = good(D=128, T=64)
    need = W.wkv7_workspace_bytes(2, 64, 4, 128)
    # wkv7_forward never runs the two-pass form; asked for it explicitly, it refuses.
    assert _call(good(D=128, T=64, algo="two_pass")) == W.WKV7_EINVAL
    assert b"wkv7_forward_ws" in W.load_library().wkv7_last_error()
    # wkv7_forward_ws: the workspace must be present, aligned, large enough and not y.
    assert _call(d, {}, fn="wkv7_forward_ws") == W.WKV7_EINVAL
    assert _call(d, {"ws": FAKE + 65536 + 8, "ws_bytes": need}, fn="wkv7_forward_ws") == W.WKV7_EINVAL
    assert _call(d, {"ws": FAKE + 65536, "ws_bytes": need - 1}, fn="wkv7_forward_ws") == W.WKV7_EINVAL
    assert b"needed" in W.load_library().wkv7_last_error()
    assert _call(d, {"ws": FAKE + 4096, "ws_bytes": need}, fn="wkv7_forward_ws") == W.WKV7_EINVAL
    assert _call(good(D=128, T=64, algo="two_pass"), {}, fn="wkv7_forward_ws") == W.WKV7_EINVAL
    # Without a two-pass algorithm the workspace is not needed.
    assert _call(good(D=128, T=64, algo="scan", B=0), {}, fn="wkv7_forward_ws") == W.WKV7_OK
    assert _call(good(D=128, T=64, B=0), {}, fn="wkv7_forward_ws") == W.WKV7_OK
    assert W.wkv7_resolve_algo(2, 64, 4, 128, algo="two_pass") == "two_pass"


def test_desc_layout():
    # Field offsets of struct wkv7_desc on LP64 (the mask pointer follows r_k).
    assert W.Desc.ab_mode.offset == 44 and W.Desc.r_k.offset == 48 and W.Desc.mask.offset == 56
    assert ctypes.sizeof(W.Desc) == 64


def test_ab_mode_from_k_rules():
    # Every algorithm forms the kernel vectors from k (B = 0: accepted without any device call).
    for D in (64, 128):
        for algo in ("scan", "chunked"):
            assert _call(good(B=0, D=D, T=64, algo=algo, ab_mode="from_k")) == W.WKV7_OK
    # b is not read: NULL passes its check (the call then fails on the misaligned y).
    assert _call(good(ab_mode="from_k"), {"b": None, "y": FAKE + 4096 + 8}) == W.WKV7_EINVAL
    assert b"y is not" in W.load_library().wkv7_last_error()
    assert _call(good(), {"b": None}) == W.WKV7_EINVAL
    assert b"b is NULL" in W.load_library().wkv7_last_error()
    # AUTO: the chunked kernels once T covers a chunk (the two-pass form with a
    # workspace at D = 128), the scan below that.
    assert W.wkv7_resolve_algo(2, 64, 4, 64, ab_mode="from_k") == "chunked"
    assert W.wkv7_resolve_algo(2, 63, 4, 64, ab_mode="from_k") == "scan"
    assert W.wkv7_resolve_algo(2, 64, 4, 128, ab_mode="from_k") == "chunked"
    assert W.wkv7_resolve_algo(2, 31, 4, 128, ab_mode="from_k") == "scan"
    assert W.wkv7_workspace_bytes(2, 64, 4, 128, ab_mode="from_k") == 2 * 4 * 2 * 35584
    assert W.wkv7_workspace_bytes(2, 64, 4, 64, ab_mode="from_k") == 0


def _bwd(desc, **over):
    """wkv7_backward with fake aligned pointers (every case fails validation first)."""
    lib = W.load_library()
    names = ("r", "w", "k", "v", "a", "b", "s0", "dy", "ds1", "dr", "dw", "dk", "dv", "da", "db", "ds0",
             "drk", "ws")
    vals = {n: FAKE + 4096 * (i + 1) for i, n in enumerate(names)}
    vals.update(s0=None, ds1=None, ds0=None, drk=None)
    vals.update(over)
    ws_bytes = over.get("ws_bytes", 1 << 40)
    args = [vals[n] for n in names[:-1]] + [vals["ws"], ws_bytes, None]
    return lib.wkv7_backward(ctypes.byref(desc), *args)


def test_backward_workspace_bytes():
    # Checkpoints, dL/dS, triangular inverses per value-slice group, grouped-head
    # buffers, r_k partials and the key-axis gradients of groups 1 .. P - 1.
    al = lambda x: (x + 255) // 256 * 256

    def groups(B, H, D):
        P = 1
        while 2 * P <= D // 32 and B * H * 2 * P <= 256:
            P *= 2
        return P

    def expect(B, T, H, D, H_kv=None, r_k=False):
        H_kv = H if H_kv is None else H_kv
        nch, P, nq = (T + 31) // 32, groups(B, H, D), B * T * H * D
        n = al(B * H * (nch + 1) * D * D * 4) + al(B * H * D * D * 4) + al(P * B * H * nch * 32 * 32 * 4)
        if H_kv != H:
            n += 2 * al(nq * 4)
        if r_k:
            n += al(P * B * H * D * 4)
        return n + al((P - 1) * 5 * nq * 4)

    assert groups(2, 4, 64) == 2 and groups(2, 32, 128) == 4 and groups(8, 32, 64) == 1 and groups(1, 200, 128) == 1
    assert W.wkv7_backward_workspace_bytes(2, 64, 4, 64) == expect(2, 64, 4, 64)
    assert W.wkv7_backward_workspace_bytes(2, 65, 4, 64) == expect(2, 65, 4, 64)
    assert W.wkv7_backward_workspace_bytes(1, 32, 4, 128, H_kv=2) == expect(1, 32, 4, 128, H_kv=2)
    assert W.wkv7_backward_workspace_bytes(8, 1024, 32, 64) == expect(8, 1024, 32, 64)
    assert W.wkv7_backward_workspace_bytes(2, 0, 4, 64) == 0
    assert W.wkv7_backward_workspace_bytes(0, 8, 4, 64) == 0


def test_backward_argument_rules():
    lib = W.load_library()
    assert _bwd(good(ab_mode="from_k")) == W.WKV7_EUNSUPPORTED
    assert _bwd(good(), dy=None) == W.WKV7_EINVAL
    assert b"dy is NULL" in lib.wkv7_last_error()
    for name in ("dr", "dw", "dk", "dv", "da", "db"):
        assert _bwd(good(), **{name: None}) == W.WKV7_EINVAL
        assert f"{name} is NULL".encode() in lib.wkv7_last_error()
        assert _bwd(good(), **{name: FAKE + 4}) == W.WKV7_EINVAL
    assert _bwd(good(), dr=FAKE + 4096) == W.WKV7_EINVAL          # aliases r
    assert _bwd(good(r_k_ptr=FAKE)) == W.WKV7_EINVAL                # r_k without dr_k
    assert b"dr_k" in lib.wkv7_last_error()
    assert _bwd(good(), drk=FAKE + 8192 * 64) == W.WKV7_EINVAL      # dr_k without r_k
    assert _bwd(good(), ds1=FAKE + 8) == W.WKV7_EINVAL
    assert _bwd(good(), ws=None) == W.WKV7_EINVAL
    assert _bwd(good(), ws_bytes=100) == W.WKV7_EINVAL
    assert b"needed" in lib.wkv7_last_error()
    assert _bwd(good(B=0), ws=None, ws_bytes=0) == W.WKV7_OK         # empty: no device call


def _wkv4(desc, **over):
    lib = W.load_library()
    names = ("w", "u", "k", "v", "s0", "y", "s1", "ws")
    vals = {n: FAKE + 4096 * (i + 1) for i, n in enumerate(names)}
    vals.update(s0=None, s1=None)
    vals.update(over)
    d = ctypes.byref(desc) if desc is not None else None
    return lib.wkv4_forward(d, *(vals[n] for n in names), over.get("ws_bytes", 1 << 40), None)


def test_wkv4_argument_rules():
    lib = W.load_library()
    good4 = lambda **kw: W.Wkv4Desc(**{**dict(B=2, T=100, C=64, in_dtype=1, y_dtype=1, spin_limit=0), **kw})
    al = lambda x: (x + 255) // 256 * 256
    assert W.wkv4_workspace_bytes(2, 100, 64) == al(2 * 2 * 2 * 3 * 64 * 4) + 256
    assert W.wkv4_workspace_bytes(8, 4096, 4096) == al(2 * 8 * 64 * 3 * 4096 * 4) + 256
    assert W.wkv4_workspace_bytes(2, 0, 64) == 0
    assert _wkv4(None) == W.WKV7_EINVAL
    assert _wkv4(good4(spin_limit=-1)) == W.WKV7_EINVAL
    assert _wkv4(good4(T=-1)) == W.WKV7_EINVAL
    assert _wkv4(good4(in_dtype=5)) == W.WKV7_EINVAL
    assert _wkv4(good4(C=1 << 24)) == W.WKV7_EUNSUPPORTED
    for name in ("w", "u", "k", "v", "y"):
        assert _wkv4(good4(), **{name: None}) == W.WKV7_EINVAL
        assert _wkv4(good4(), **{name: FAKE + 2}) == W.WKV7_EINVAL
    assert _wkv4(good4(), y=FAKE + 4096 * 3) == W.WKV7_EINVAL      # y aliases k
    assert _wkv4(good4(), ws=None) == W.WKV7_EINVAL
    assert _wkv4(good4(), ws_bytes=10) == W.WKV7_EINVAL
    assert b"needed" in lib.wkv7_last_error()
    assert _wkv4(good4(B=0)) == W.WKV7_OK                          # empty: no device call


def test_wkv4_wait_status_argument_rules():
    """wkv4_wait_status validates before touching the device: a bad descriptor, a
    missing or too small workspace are EINVAL; nothing to compute is OK."""
    lib = W.load_library()
    good4 = lambda **kw: W.Wkv4Desc(**{**dict(B=2, T=100, C=64, in_dtype=1, y_dtype=1, spin_limit=0), **kw})
    need = W.wkv4_workspace_bytes(2, 100, 64)
    st = lambda d, ws, n: lib.wkv4_wait_status(ctypes.byref(d) if d is not None else None, ws, n, None)
    assert st(None, FAKE, need) == W.WKV7_EINVAL
    assert st(good4(spin_limit=-3), FAKE, need) == W.WKV7_EINVAL
    assert st(good4(), None, need) == W.WKV7_EINVAL
    assert st(good4(), FAKE, need - 1) == W.WKV7_EINVAL
    assert b"needed" in lib.wkv7_last_error()
    assert st(good4(T=0), None, 0) == W.WKV7_OK
    assert lib.wkv7_strerror(W.WKV7_ETIMEOUT) == b"a bounded device-side wait gave up"


def test_no_kernel_spills_to_scratch():
    """The build records each kernel's scratch bytes per lane: no kernel may spill
    registers.  (A spill store has been placed at a loop exit before the
    execution mask was restored, dropping the value.)"""
    import json
    path = os.path.join(ROOT, "_build", "scratch_bytes.json")
    if not os.path.exists(path):
        pytest.skip("no build record")
    usage = json.load(open(path))
    assert usage, "empty build record"
    bad = {k: v for k, v in usage.items() if v}
    assert not bad, f"kernels using scratch: {bad}"


SP = 1 << 26          # 64 MiB between fake arrays: disjoint unless a test makes them overlap
BASE = 1 << 36


def test_forward_workspace_must_not_overlap_any_array():
    lib = W.load_library()
    B, T, H, D = 2, 64, 4, 128
    need = W.wkv7_workspace_bytes(B, T, H, D)
    state = B * H * D * D * 4
    q = B * T * H * D * 2
    names = ("r", "w", "k", "v", "a", "b", "y", "s0", "s1")
    ptrs = {n: BASE + i * SP for i, n in enumerate(names)}
    sizes = dict(r=q, w=q, k=q, v=q, a=q, b=q, y=q, s0=state, s1=state)
    label = dict(s0="state_in", s1="state_out")
    for n in names:
        # The workspace's last 16 bytes on the array's first 16, then its first 16 on the array's last 16.
        for ws in (ptrs[n] - need + 16, ptrs[n] + sizes[n] - 16):
            assert _call(good(B=B, T=T, H=H, D=D), {**ptrs, "ws": ws, "ws_bytes": need},
                         fn="wkv7_forward_ws") == W.WKV7_EINVAL
            assert f"workspace overlaps {label.get(n, n)}".encode() in lib.wkv7_last_error(), n
    # Adjacent is not an overlap: with the workspace right before r (or right after
    # state_in) only the state_out placed across it is reported.
    for n, ws in (("r", ptrs["r"] - need), ("s0", ptrs["s0"] + state)):
        assert _call(good(B=B, T=T, H=H, D=D), {**ptrs, "s1": ws + need - 16, "ws": ws, "ws_bytes": need},
                     fn="wkv7_forward_ws") == W.WKV7_EINVAL
        assert lib.wkv7_last_error() == b"workspace overlaps state_out", n


def test_backward_workspace_must_not_overlap_any_array():
    lib = W.load_library()
    B, T, H, D = 2, 8, 4, 64
    need = W.wkv7_backward_workspace_bytes(B, T, H, D)
    names = ("r", "w", "k", "v", "a", "b", "s0", "dy", "ds1", "dr", "dw", "dk", "dv", "da", "db", "ds0", "drk")
    ptrs = {n: BASE + i * SP for i, n in enumerate(names)}
    ptrs["drk"] = None
    for n in ("k", "s0", "dy", "ds1", "dr", "dv", "ds0"):
        assert _bwd(good(B=B, T=T, H=H, D=D), **ptrs, ws=ptrs[n] + 16, ws_bytes=need) == W.WKV7_EINVAL
        assert b"workspace overlaps" in lib.wkv7_last_error(), n


def test_wkv4_workspace_must_not_overlap_any_array():
    lib = W.load_library()
    desc = W.Wkv4Desc(B=2, T=100, C=64, in_dtype=1, y_dtype=1, spin_limit=0)
    need = W.wkv4_workspace_bytes(2, 100, 64)
    names = ("w", "u", "k", "v", "s0", "y", "s1")
    ptrs = {n: BASE + i * SP for i, n in enumerate(names)}
    for n in names:
        assert _wkv4(desc, **ptrs, ws=ptrs[n] + 16, ws_bytes=need) == W.WKV7_EINVAL
        assert b"workspace overlaps" in lib.wkv7_last_error(), n


def test_scan_rejects_rows_too_wide_for_32_bit_offsets():
    """The scan addresses a few tokens of one row with 32-bit offsets: H * D * 68 must
    stay below 2^32.  H = 2^20 at D = 64 is past it (EUNSUPPORTED before any HIP call);
    the chunked form takes the same shape once T reaches a chunk."""
    lib = W.load_library()
    ptrs = [BASE + i * SP for i in range(8)]
    desc = W.make_desc(1, 1, 1 << 20, 64)
    assert lib.wkv7_forward(ctypes.byref(desc), *ptrs[:6], None, ptrs[6], ptrs[7], None) == W.WKV7_EUNSUPPORTED
    assert b"scan" in lib.wkv7_last_error()
    desc = W.make_desc(1, 1, 1 << 20, 64, algo="scan")
    assert lib.wkv7_forward(ctypes.byref(desc), *ptrs[:6], None, ptrs[6], ptrs[7], None) == W.WKV7_EUNSUPPORTED


def test_noalloc_rejects_more_heads_than_the_scratch_holds():
    """wkv7_forward_noalloc: one 32-token chunk record per (b, h) must fit the static
    scratch; B H = 2048 at D = 128 needs 77 MB > 64 MiB.  Rejected before any HIP call."""
    lib = W.load_library()
    ptrs = [BASE + i * SP for i in range(8)]
    desc = W.make_desc(1, 64, 2048, 128)
    assert lib.wkv7_forward_noalloc(ctypes.byref(desc), *ptrs[:6], None, ptrs[6], ptrs[7], None) == W.WKV7_EUNSUPPORTED
    assert b"static scratch" in lib.wkv7_last_error()
    # Without state_out the state carry takes room too: 1000 heads fit with it given, not without.
    need = 1000 * 35584
    assert need < W.NOALLOC_SCRATCH_BYTES < need + 1000 * 128 * 128 * 4
    desc = W.make_desc(1, 64, 1000, 128)
    assert lib.wkv7_forward_noalloc(ctypes.byref(desc), *ptrs[:6], None, ptrs[6], None, None) == W.WKV7_EUNSUPPORTED
    assert b"state carry" in lib.wkv7_last_error()
    # Other argument errors are those of wkv7_forward_ws.
    assert lib.wkv7_forward_noalloc(None, *ptrs[:6], None, ptrs[6], ptrs[7], None) == W.WKV7_EINVAL
    desc = W.make_desc(2, 64, 4, 128)
    assert lib.wkv7_forward_noalloc(ctypes.byref(desc), *ptrs[:6], None, ptrs[0], ptrs[7], None) == W.WKV7_EINVAL
