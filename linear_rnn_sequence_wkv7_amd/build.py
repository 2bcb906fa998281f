"""Build libwkv7.so for gfx950 with hipcc (in-tree).

    python -m linear_rnn_sequence_wkv7_amd.build          # compile every source, link
    python -m linear_rnn_sequence_wkv7_amd.build --asm    # also write gfx950 assembly to _build/

Objects go to _build/ at the repository root; the library is written next to
this file.  Every call recompiles.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwkv7.so")
ARCH = "gfx950"

SOURCES = ["wkv7_api.cpp", "wkv7_scan.hip", "wkv7_decode.hip", "wkv7_chunked.hip", "wkv7_chunked128.hip",
           "wkv7_twopass128.hip", "wkv7_twopass128_scan.hip", "wkv7_backward.hip", "wkv4.hip"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 VALU ops are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source extras.  The two-pass kernels do VALU work on their MFMA
# accumulators (state tiles, partial products); kept in VGPRs they need no
# AGPR <-> VGPR copies (pass 2 without it: 1.093-1.097 against 1.063-1.069 ms
# per hxa07D step on one box).
EXTRA = {
    "wkv7_twopass128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "wkv7_twopass128_scan.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


# Host-side sanitizers for the CPU tests of the library's host code: each flag
# follows -Xarch_host, so it reaches the host compilation only and the device code
# is compiled as in the product build.  The library then leaves the sanitizer
# runtime's symbols undefined; the process that loads it preloads that runtime.
SANITIZE_HOST = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


# Per-kernel resource remarks of the device compile (scratch bytes per lane).
# Register spills to scratch are avoided: the compiler has placed a spill store at
# a loop exit before the execution mask was restored, losing the value.
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
SCRATCH_JSON = os.path.join(BUILD, "scratch_bytes.json")


def _scratch_of(output: str) -> dict:
    out, name = {}, None
    for line in output.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
            name = None
    return out


def build(asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        extra = EXTRA.get(src, [])
        remarks = RESOURCE_REMARKS if src.endswith(".hip") else []
        jobs.append([cc, *COMMON, *extra, *remarks, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        if asm and src.endswith(".hip"):
            jobs.append([cc, *COMMON, *extra, "-x", "hip", "--cuda-device-only", "-S",
                         os.path.join(CSRC, src), "-o",
                         os.path.join(BUILD, os.path.splitext(src)[0] + f"-{ARCH}.s")])
    scratch = {}
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            scratch.update(_scratch_of(out))
            if verbose and out.strip():
                print("\n".join(l for l in out.splitlines() if "remark:" not in l))
    with open(SCRATCH_JSON, "w") as f:
        json.dump(scratch, f, indent=0, sort_keys=True)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def sanitizer_runtime() -> str | None:
    """The clang AddressSanitizer runtime (it carries the UndefinedBehaviorSanitizer
    handlers too) of the ROCm toolchain, or None."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for base in (os.path.join(root, "lib", "llvm"), root):
        hits = sorted(glob.glob(os.path.join(base, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    return None


def build_host_sanitized(out_dir: str) -> str:
    """Compile every source with SANITIZE_HOST (and -O1 -g) into out_dir and link
    out_dir/libwkv7_hostsan.so; returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    common = [f for f in COMMON if f != "-O3"] + ["-O1", "-g"]
    jobs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append([cc, *common, *EXTRA.get(src, []), *SANITIZE_HOST, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(_run, jobs))
    lib = os.path.join(out_dir, "libwkv7_hostsan.so")
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", lib, *objs])
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(asm=a.asm, verbose=a.verbose))


if __name__ == "__main__":
    sys.exit(main())
