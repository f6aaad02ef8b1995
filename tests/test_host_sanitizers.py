"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.  CPU only.

The two pieces of plain host code -- the oracle (C, test infrastructure)
and the block manager (C++, product: pointer-linked eviction list, hash
map, per-sequence tables) -- are rebuilt with gcc / g++ and
-fsanitize=address,undefined (host compilers only; no GPU code is built
here), and the oracle pins and the block-manager parity tests run again
against those builds in child processes with the ASan runtime preloaded
into Python.  Any invalid access, leak-free use after free, misaligned or
overflowing arithmetic aborts the child, so the test fails.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ORACLE_PINS = ["tests/test_oracle_formula.py", "tests/test_oracle_fp8.py",
               "tests/test_oracle_attention.py", "tests/test_oracle_multiquery.py",
               "tests/test_oracle_blocks.py", "tests/test_oracle_quant.py",
               "tests/test_oracle_tables.py"]


def _runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's ASan runtime is not installed")
    return path


def _child(env_extra, tests):
    env = dict(os.environ, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **env_extra)
    # -s: a sanitizer report goes to the child's stderr as it aborts, which
    # pytest's capture would swallow
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p",
                        "no:cacheprovider", "-m", "not gpu", *tests], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail


def test_oracle_under_sanitizers(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", *SAN, "-o", so, os.path.join(ROOT, "oracle", "oracle.c"),
                    "-lm"], check=True)
    _child({"PKV_ORACLE_LIB": so}, ORACLE_PINS)


def test_block_manager_under_sanitizers(tmp_path):
    so = str(tmp_path / "libpkv_bm_san.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-I",
                    os.path.join(ROOT, "include"), "-o", so,
                    os.path.join(ROOT, "paged_kv_cache_273_amd", "csrc", "block_manager.cpp")],
                   check=True)
    _child({"PKV_TEST_BM_LIB": so}, ["tests/test_block_manager.py"])
