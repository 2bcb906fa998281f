"""Rules on the HIP sources that the compiler does not enforce (CPU only)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_rnn_sequence_wkv7_amd", "csrc")


def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")))


def _code(name):
    """Source text without comments."""
    src = open(os.path.join(CSRC, name)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.sub(r"//[^\n]*", "", src)


@pytest.mark.parametrize("name", _sources())
def test_one_mfma_opcode_per_source(name):
    """Each kernel source issues one matrix-core opcode only, so no accumulator
    chain can mix shapes: a 16x16x32 bf16 result fed as the accumulator of a
    16x16x16 MFMA has given schedule-dependent wrong values on gfx950.  A
    16-deep term is zero-padded to 32 deep instead."""
    code = _code(name)
    builtins = set(re.findall(r"__builtin_amdgcn_mfma_\w+", code))
    asm = set(re.findall(r"\bv_mfma_\w+", code))
    smfmac = set(re.findall(r"__builtin_amdgcn_smfmac_\w+", code))
    assert not asm, f"{name}: MFMA written in inline asm: {sorted(asm)}"
    assert not smfmac, f"{name}: sparse MFMA: {sorted(smfmac)}"
    assert len(builtins) <= 1, f"{name}: more than one MFMA opcode: {sorted(builtins)}"


@pytest.mark.parametrize("name", _sources())
def test_no_hand_written_packed_fp32(name):
    """Packed fp32 VALU ops are disabled at compile time and never written by hand."""
    code = _code(name)
    assert not re.search(r"v_pk_(add|mul|fma)_f32", code), name


def test_build_disables_packed_fp32():
    from linear_rnn_sequence_wkv7_amd import build as B
    flags = " ".join(B.COMMON)
    assert "-target-feature -Xclang -packed-fp32-ops" in flags
    assert f"--offload-arch={B.ARCH}" in flags and B.ARCH == "gfx950"


def test_mfma_sources_are_known():
    """The kernels that use matrix cores, and which opcode each one uses."""
    found = {}
    for name in _sources():
        b = set(re.findall(r"__builtin_amdgcn_mfma_\w+", _code(name)))
        if b:
            found[name] = b.pop()
    assert found == {
        "wkv7_backward.hip": "__builtin_amdgcn_mfma_f32_16x16x4f32",
        "wkv7_chunked.hip": "__builtin_amdgcn_mfma_f32_16x16x32_bf16",
        "wkv7_chunked128.hip": "__builtin_amdgcn_mfma_f32_16x16x32_bf16",
        "wkv7_twopass128.hip": "__builtin_amdgcn_mfma_f32_16x16x32_bf16",
        "wkv7_twopass128_scan.hip": "__builtin_amdgcn_mfma_f32_16x16x32_f16",
    }, found
