"""Builds the test probes (tests/probes/*.hip) into shared libraries beside them, for gfx950.

Test infrastructure only: the library under test is gated_delta_rule_13_amd/libkda.so."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
XCD_PROBE = os.path.join(HERE, "libxcd_probe.so")


def build_probes() -> None:
    src = os.path.join(HERE, "xcd_probe.hip")
    r = subprocess.run([HIPCC, *FLAGS, src, "-o", XCD_PROBE], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")


if __name__ == "__main__":
    build_probes()
