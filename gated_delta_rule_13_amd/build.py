"""Builds libkda.so, the HIP library behind the C ABI of include/kda.h, for gfx950.

Every kernel source under csrc/ is compiled with hipcc to an object in parallel and
linked into ``gated_delta_rule_13_amd/libkda.so`` (in-tree, so the built library
travels with the source tree). Packed-fp32 instructions are disabled for all device
code (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source flags. The backward's gradient kernel runs one wavefront per SIMD and may hold
# more than 256 registers; its matrix-core products keep their operands and results in the
# architectural vector registers (otherwise every product's result is moved out of the
# accumulation registers before the vector ALU can use it), and the accumulation registers
# serve only as spill space.
SOURCE_FLAGS = {
    "kda_chunk_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str, build_dir: str, extra) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src,
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


DEBUG_LIB = os.path.join(HERE, "libkda_debug.so")


def build(verbose: bool = False, host_sanitize: str = "", out: str = LIB,
          debug: bool = False) -> str:
    """Compiles every csrc/*.hip and links ``out`` (the in-tree libkda.so by default).

    ``debug`` builds the KDA_DEBUG library (``libkda_debug.so`` unless ``out`` is given): every
    operator entry point checks its value preconditions on the device first (kda.h).

    ``host_sanitize`` ("address" or "undefined") instruments the host code only
    (``-Xarch_host -fsanitize=...``; the GPU code is built as usual) for running the C-ABI
    checks, which launch nothing, under the sanitizer: load ``out`` with
    ``gated_delta_rule_13_amd.load_library(out)`` in a Python started with the sanitizer's
    runtime (``libclang_rt.asan-x86_64.so`` or ``libclang_rt.ubsan_standalone-x86_64.so``
    from ROCm's clang) in ``LD_PRELOAD``.
    """
    extra = []
    build_dir = BUILD
    if debug:
        # the precondition checks of every operator entry point (kda_debug.hip)
        extra = ["-DKDA_DEBUG=1"]
        build_dir = f"{BUILD}_debug"
        if out == LIB:
            out = DEBUG_LIB
    if host_sanitize:
        if host_sanitize not in ("address", "undefined"):
            raise ValueError(f"unknown sanitizer {host_sanitize!r}")
        extra += ["-Xarch_host", f"-fsanitize={host_sanitize}"]
        if host_sanitize == "undefined":
            extra += ["-Xarch_host", "-fno-sanitize-recover=undefined"]
        build_dir = f"{build_dir}_{host_sanitize}"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libkda.so for gfx950")
    ap.add_argument("-v", action="store_true", help="show the link step's output")
    ap.add_argument("--host-sanitize", choices=["address", "undefined"], default="")
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--debug", action="store_true",
                    help="build libkda_debug.so: device-side checks of the value preconditions")
    args = ap.parse_args()
    print(build(verbose=args.v, host_sanitize=args.host_sanitize, out=args.out,
                debug=args.debug))
