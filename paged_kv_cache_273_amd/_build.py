"""Builds libpagedkv.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SO = os.path.join(PKG, "libpagedkv.so")
SOURCES = ["abi.hip", "decode.hip", "prefill.hip", "append_reduce.hip", "blocks.hip",
           "block_manager.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-parameter",
]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose: bool = False, extra_flags=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
           "-o", SO + ".tmp", *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag: drop that notice
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
