"""Builds libpagedkv.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SO = os.path.join(PKG, "libpagedkv.so")
SOURCES = ["abi.hip", "decode.hip", "prefill.hip", "append_reduce.hip", "blocks.hip",
           "probe.hip", "block_manager.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-parameter",
    # leading scalar kernel arguments arrive preloaded in SGPRs
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]
# the host pass does not know the device-only feature flag: drop that notice
_NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if _NOISE not in l)
    return r.returncode, msgs


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compiles every source to an object in parallel, then links the shared
    library; the previous library is replaced only when everything succeeded."""
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
                   "-c", "-o", obj, os.path.join(CSRC, src)]
            return (src, obj) + _run(cmd)

        workers = min(len(SOURCES), os.cpu_count() or 1)
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(compile_one, SOURCES))
        failed = [(s, m) for s, _, rc, m in results if rc != 0]
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(f"{s}:\n{m}" for s, m in failed))
        if verbose:
            for s, _, _, m in results:
                if m.strip():
                    print(f"{s}:\n{m}")
        rc, msgs = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
                         "-o", SO + ".tmp", *[obj for _, obj, _, _ in results]])
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{msgs}")
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
