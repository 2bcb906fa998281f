"""Seeded synthetic inputs for the RWKV-7 WKV recurrence.

This module is shared by the GPU path's callers (tests, bench) and by the
tests that feed the fp64 oracle.  It holds only input synthesis: random draws,
the decay parameterisation that produces the kernel's w input, the
L2-normalised removal key, and bf16 encoding.  It contains none of the
recurrence's arithmetic.

Distributions (stated per workload below) follow the hxa07D time-mix
(zenn.dev "RWKV hxa07D architecture explained", forward listing and
sections 3, 6 and 8): the decay is w = exp(-exp(-softplus(-z) - 0.5)), the
kernel receives a = -kk and b = kk * alpha with kk the per-head L2-normalised
key, and grouped KV heads are repeated contiguously.

Layouts (all C-contiguous):
  r, w, a, b : [B, T, H, D]
  k, v       : [B, T, H_kv, D]
  state      : [B, H, D, D] fp32, state[b, h, i, j] = S_ij (i value row, j key column)
  r_k        : [H, D] fp32
  mask       : [B, T] uint8 (0 = masked token), or None
Decode workloads carry a leading step axis: r..b are [steps, B, 1, H, D].

bf16 tensors are returned as uint16 bit patterns (round-to-nearest-even from
fp32, which itself is round-to-nearest from the fp64 value).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "make_inputs", "make_grad_inputs", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "workload", "Wkv4Workload", "WKV4_WORKLOADS", "make_wkv4_inputs",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtypes, decay mode and the seed."""
    name: str
    kind: str                 # "forward" or "decode"
    B: int
    T: int
    H: int
    D: int
    H_kv: int
    in_dtype: str             # "f32" or "bf16" for r, w, k, v, a, b
    y_dtype: str              # "f32" or "bf16"
    w_mode: str               # "decay": w given; "logneglog": kernel input x, decay = exp(-exp(x))
    s0_std: float             # 0 -> zero initial state (passed as None)
    seed: int
    steps: int = 1            # decode steps (decode workloads only)
    chunk_len: int = 0          # 0: the chunked kernel's own length (64 at D=64, 32 at D=128)
    y_scale: float = 1.0
    rk_std: float = 0.0       # > 0 -> per-head/dim bonus weights r_k ~ N(0, rk_std^2)
    kk_from_k: bool = False   # removal key = normalise(repeated k) instead of an independent draw
    ab_mode: str = "given"    # "from_k": a carries alpha, b is None (the kernel forms both from k)
    mask: str = ""            # "": none; "pad": right padding; "holes": scattered masked tokens
    algo: str = "auto"
    note: str = ""

    @property
    def head_tokens(self) -> int:
        return self.B * self.T * self.H * self.steps


# The five workloads.  Seeds are 1000 + the workload's position in this list.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("fwd_f32_b1_t64_h2_d64", "forward", B=1, T=64, H=2, D=64, H_kv=2,
             in_dtype="f32", y_dtype="f32", w_mode="decay", s0_std=0.0, seed=1001,
             note="small fp32 forward, zero initial state"),
    Workload("fwd_bf16_b8_t1024_h32_d64", "forward", B=8, T=1024, H=32, D=64, H_kv=32,
             in_dtype="bf16", y_dtype="bf16", w_mode="decay", s0_std=0.0, seed=1002,
             note="bf16 forward, C=2048, zero initial state"),
    Workload("prefill_bf16_b4_t4096_h40_d64_l64", "forward", B=4, T=4096, H=40, D=64, H_kv=40,
             in_dtype="bf16", y_dtype="bf16", w_mode="decay", s0_std=0.1, seed=1003,
             chunk_len=64, algo="chunked",
             note="2.9B-shaped layer (C=2560), chunked prefill, random initial state"),
    Workload("decode_bf16_b256_h64_d64_x32", "decode", B=256, T=1, H=64, D=64, H_kv=64,
             in_dtype="bf16", y_dtype="bf16", w_mode="decay", s0_std=0.1, seed=1004, steps=32,
             note="256 sequences x 32 successive decode steps, 256 MiB fp32 state"),
    Workload("hxa07d_bf16_b2_t16384_h32_kv8_d128", "forward", B=2, T=16384, H=32, D=128, H_kv=8,
             in_dtype="bf16", y_dtype="bf16", w_mode="logneglog", s0_std=0.0, seed=1005,
             y_scale=128.0 ** -0.5, rk_std=0.1, kk_from_k=True,
             note="hxa07D-style long context: GQA 8 KV heads x4, log-decay input, fused epilogue"),
]}


def workload(name: str, **overrides) -> Workload:
    """Look up a workload by name, optionally overriding fields (e.g. smaller T)."""
    return replace(WORKLOADS[name], **overrides)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _l2_normalize(x: np.ndarray, eps: float = 1e-12) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def _encode(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def make_inputs(wl: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw the workload's inputs.

    Draw order from one PCG64 stream (float64 normals, C order): r, k, v, z,
    kappa_raw (skipped when kk_from_k or ab_mode == "from_k"), alpha_raw,
    state0 (when s0_std > 0), r_k (when rk_std > 0), then the mask draws.

    Returns a dict with keys r, w, k, v, a, b (encoded per in_dtype), state0
    (fp32 or None), r_k (fp32 or None), mask (uint8 or None).  With ab_mode
    "from_k", a holds alpha and b is None.  For decode workloads each per-token
    tensor has a leading [steps] axis (the mask too: [steps, B, 1]).

    Mask recipes: "pad" keeps a prefix of each sequence, its length uniform
    on [ceil(T / 2), T] (sequence 0 keeps all T tokens); "holes" masks each
    token independently with probability 1/8.
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    lead = (wl.steps,) if wl.kind == "decode" else ()
    shp_q = lead + (wl.B, wl.T, wl.H, wl.D)
    shp_kv = lead + (wl.B, wl.T, wl.H_kv, wl.D)
    rep = wl.H // wl.H_kv
    out: Dict[str, Optional[np.ndarray]] = {}

    out["r"] = _encode(rng.standard_normal(shp_q), wl.in_dtype)
    k64 = rng.standard_normal(shp_kv)
    out["k"] = _encode(k64, wl.in_dtype)
    out["v"] = _encode(rng.standard_normal(shp_kv), wl.in_dtype)

    z = rng.standard_normal(shp_q) * 2.0
    if wl.w_mode == "decay":
        w = np.exp(-np.exp(-_softplus(-z) - 0.5))
    elif wl.w_mode == "logneglog":
        w = -_softplus(z) - 0.5          # log(-log(decay)); decay = exp(-exp(w))
    else:
        raise ValueError(wl.w_mode)
    del z
    out["w"] = _encode(w, wl.in_dtype)
    del w

    if wl.ab_mode == "from_k":
        del k64
        alpha = 1.0 / (1.0 + np.exp(-rng.standard_normal(shp_q)))
        out["a"] = _encode(alpha, wl.in_dtype)
        out["b"] = None
        del alpha
    elif wl.ab_mode == "given":
        if wl.kk_from_k:
            kk = _l2_normalize(np.repeat(k64, rep, axis=-2))
        else:
            kk = _l2_normalize(rng.standard_normal(shp_q))
        del k64
        alpha = 1.0 / (1.0 + np.exp(-rng.standard_normal(shp_q)))
        out["a"] = _encode(-kk, wl.in_dtype)
        out["b"] = _encode(kk * alpha, wl.in_dtype)
        del kk, alpha
    else:
        raise ValueError(wl.ab_mode)

    if wl.s0_std > 0:
        out["state0"] = (rng.standard_normal((wl.B, wl.H, wl.D, wl.D)) * wl.s0_std).astype(np.float32)
    else:
        out["state0"] = None
    if wl.rk_std > 0:
        out["r_k"] = (rng.standard_normal((wl.H, wl.D)) * wl.rk_std).astype(np.float32)
    else:
        out["r_k"] = None
    out["mask"] = _mask(rng, wl, lead)
    return out


def _mask(rng, wl: Workload, lead) -> Optional[np.ndarray]:
    if not wl.mask:
        return None
    shp = lead + (wl.B, wl.T)
    if wl.mask == "holes":
        return (rng.random(shp) >= 0.125).astype(np.uint8)
    if wl.mask == "pad":
        lens = rng.integers((wl.T + 1) // 2, wl.T + 1, size=lead + (wl.B,))
        lens[..., 0] = wl.T
        return (np.arange(wl.T) < lens[..., None]).astype(np.uint8)
    raise ValueError(wl.mask)


def make_grad_inputs(wl: Workload, seed: Optional[int] = None, dstate: bool = True) -> Dict[str, np.ndarray]:
    """Upstream gradients for the backward: dy ~ N(0, 1) [B, T, H, D] encoded per
    y_dtype, and dstate ~ N(0, 1) [B, H, D, D] fp32 (or None).  Own PCG64 stream,
    seeded with the workload seed + 500 unless given."""
    rng = np.random.Generator(np.random.PCG64(wl.seed + 500 if seed is None else seed))
    out: Dict[str, Optional[np.ndarray]] = {}
    out["dy"] = _encode(rng.standard_normal((wl.B, wl.T, wl.H, wl.D)), wl.y_dtype)
    out["dstate"] = rng.standard_normal((wl.B, wl.H, wl.D, wl.D)).astype(np.float32) if dstate else None
    return out


# ------------------------------- RWKV-4 WKV -------------------------------

@dataclass(frozen=True)
class Wkv4Workload:
    """RWKV-4 WKV inputs: k, v [B, T, C], per-channel w, u."""
    name: str
    B: int
    T: int
    C: int
    in_dtype: str
    y_dtype: str
    seed: int
    state: bool = False       # random initial state (A, Bs, P) instead of zero
    k_offset: float = 0.0     # added to every k (exercises the exponent scaling)


WKV4_WORKLOADS: Dict[str, Wkv4Workload] = {w.name: w for w in [
    Wkv4Workload("rwkv4_bf16_b8_t4096_c4096", B=8, T=4096, C=4096, in_dtype="bf16", y_dtype="bf16", seed=1101),
]}


def make_wkv4_inputs(wl: Wkv4Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw order from one PCG64 stream: z (decay), u, k, v, then the state.

    w = exp(z), z ~ U(-5, 1) per channel (a spread of slow and fast decays);
    u ~ N(0, 1); k, v ~ N(0, 1) with k_offset added to k.  The optional state is
    (A, Bs, P) per (b, c): A ~ N(0, 1), Bs ~ U(0.5, 2), P ~ N(0, 1) (a = A e^P,
    b = Bs e^P).  k, v encoded per in_dtype; w, u, state fp32."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    out: Dict[str, Optional[np.ndarray]] = {}
    out["w"] = np.exp(rng.uniform(-5.0, 1.0, wl.C)).astype(np.float32)
    out["u"] = rng.standard_normal(wl.C).astype(np.float32)
    out["k"] = _encode(rng.standard_normal((wl.B, wl.T, wl.C)) + wl.k_offset, wl.in_dtype)
    out["v"] = _encode(rng.standard_normal((wl.B, wl.T, wl.C)), wl.in_dtype)
    if wl.state:
        st = np.empty((wl.B, 3, wl.C), dtype=np.float32)
        st[:, 0] = rng.standard_normal((wl.B, wl.C))
        st[:, 1] = rng.uniform(0.5, 2.0, (wl.B, wl.C))
        st[:, 2] = rng.standard_normal((wl.B, wl.C))
        out["state"] = st
    else:
        out["state"] = None
    return out
