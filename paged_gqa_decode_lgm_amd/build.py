"""Build liblgm.so in-tree with hipcc for gfx950.

    python -m paged_gqa_decode_lgm_amd.build [--verbose] [--sanitize]

Each translation unit is compiled separately (the RoPE/append unit with
-ffp-contract=off so no multiply-add is fused) and linked into
paged_gqa_decode_lgm_amd/liblgm.so.  Packed-fp32 VALU ops are disabled for all
device code.

--sanitize builds liblgm_san.so instead, with the host code of every unit
(argument validation, plans, launches) under AddressSanitizer and
UndefinedBehaviorSanitizer; device code is built as usual.  Load it with
LGM_LIBRARY pointing at it and the ASan runtime preloaded, e.g.

    LGM_LIBRARY=$PWD/paged_gqa_decode_lgm_amd/liblgm_san.so \
    LD_PRELOAD=$(hipcc -print-file-name=libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    python -m pytest tests/test_abi.py
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblgm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
UNITS = {
    "lgm_api.cpp": ["-x", "hip"],
    "rope_kv_append.hip": ["-ffp-contract=off"],
    "paged_decode.hip": [],
    "paged_decode_mfma.hip": [],
    "paged_decode_fused.hip": [],
    # MFMA accumulators in VGPRs: the whole-row step loop then keeps them in
    # the registers its MFMAs use instead of copying them between register
    # files around every step.
    "paged_decode_rows.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "lse_merge.hip": [],
    "table_check.hip": [],
    "stream_probe.hip": [],
    "paged_mla.hip": [],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


# Host-only sanitizers: each -fsanitize= applies to the host pass alone.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN_LIB = os.path.join(PKG, "liblgm_san.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    bdir = BUILD + ("_san" if sanitize else "")
    lib = SAN_LIB if sanitize else LIB
    san = SANITIZE if sanitize else []
    os.makedirs(bdir, exist_ok=True)

    def compile_one(item):
        src, extra = item
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        _run([HIPCC, *COMMON, *san, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(min(len(UNITS), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, UNITS.items()))
    tmp = lib + ".tmp"
    link_san = ["-shared-libasan", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] if sanitize else []
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_san, *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, sanitize="--sanitize" in sys.argv))
