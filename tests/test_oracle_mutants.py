"""Plants plausible mistakes in a copy of the oracle source (on the CPU) and
checks that the oracle's pins catch every one of them.

Each mutant is one textual edit of oracle/oracle.c (a wrong index, a dropped
term, a flipped sign, a transposed layout), compiled with gcc into a
temporary library and run against the pin files in a child pytest process.
A mutant that survives means the pins would not notice that mistake.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_formula.py", "tests/test_oracle_fp8.py",
        "tests/test_oracle_attention.py", "tests/test_oracle_multiquery.py",
        "tests/test_oracle_blocks.py", "tests/test_oracle_quant.py",
        "tests/test_oracle_tables.py"]

# (name, original text, planted text, occurrence count expected)
MUTANTS = [
    ("size_drops_k_and_v", "return 2 * layers * kv_heads", "return layers * kv_heads"),
    ("gqa_interleaved_heads", "int32_t h = hq / G;", "int32_t h = hq % Hkv;"),
    ("slot_from_block_index", "int32_t slot = t % block_size;\n        double dot",
     "int32_t slot = (t / block_size) % block_size;\n        double dot"),
    ("table_column_off_by_one",
     "block_tables[(int64_t)b * max_blocks + t / block_size];\n        int32_t slot = t % block_size;\n        double dot",
     "block_tables[(int64_t)b * max_blocks + (t / block_size + 1) % ((t1 + block_size - 1) / block_size)];\n        int32_t slot = t % block_size;\n        double dot"),
    ("pool_layout_transposed", "return (((int64_t)phys * bs + slot) * Hkv + h) * D + d;",
     "return (((int64_t)phys * Hkv + h) * bs + slot) * D + d;"),
    ("scale_dropped", "s[i] = scale * dot;", "s[i] = dot;"),
    ("softmax_sign_flipped", "double w = exp(s[i] - m);", "double w = exp(m - s[i]);"),
    ("no_normalisation", "out[d] /= l;", "out[d] /= 1.0;"),
    ("lse_without_max", "lse = m + log(l);", "lse = log(l);"),
    ("max_not_taken", "if (s[i] > m)\n            m = s[i];", "if (s[i] < m)\n            m = s[i];"),
    ("e4m3_bias_8", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3_subnormal_scale", "mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    ("ties_away_from_even", "c = (lo & 1) == 0 ? lo : hi;", "c = hi;"),
    ("quantise_multiplies", "float y = x / scale;", "float y = x * scale;"),
    ("no_saturation", "if (a >= 448.0)\n        return (uint8_t)(sign | 0x7E);",
     "if (a >= 448.0)\n        return (uint8_t)(sign | 0x7F);"),
    ("fp8_scale_ignores_head", "case 1: return (int64_t)phys * Hkv + h;",
     "case 1: return (int64_t)phys * Hkv;"),
    ("merge_weight_sign", "w = exp(lse_parts[s] - M);", "w = exp(M - lse_parts[s]);"),
    ("merge_empty_as_lse_zero",
     "if (lse_parts[s] == -INFINITY)\n            continue;\n        w = exp(lse_parts[s] - M);",
     "w = lse_parts[s] == -INFINITY ? exp(-M) : exp(lse_parts[s] - M);"),
    ("append_wrong_slot", "slot = t % block_size;\n        for (h = 0; h < Hkv; ++h) {",
     "slot = (t + 1) % block_size;\n        for (h = 0; h < Hkv; ++h) {"),
    ("append_swaps_k_v", "store_value(k_cache, k_scale, kv_dtype, dst, k_new[src], phys, h, Hkv);",
     "store_value(k_cache, k_scale, kv_dtype, dst, v_new[src], phys, h, Hkv);"),
    ("block_scale_amax_over_all_slots",
     "double amax = 0.0;\n            for (slot = 0; slot < live[p]; ++slot)",
     "double amax = 0.0;\n            for (slot = 0; slot < (live[p] ? block_size : 0); ++slot)"),
    ("wide_scale_amax_over_all_slots",
     "for (p = 0; p < num_blocks; ++p)\n            for (slot = 0; slot < live[p]; ++slot)",
     "for (p = 0; p < num_blocks; ++p)\n            for (slot = 0; slot < (live[p] ? block_size : 0); ++slot)"),
    ("int8_params_over_all_slots",
     "for (slot = 0; slot < live[p]; ++slot)\n                for (d = 0; d < D; ++d) {\n                    double v = orc_bf16_value(",
     "for (slot = 0; slot < (live[p] ? block_size : 0); ++slot)\n                for (d = 0; d < D; ++d) {\n                    double v = orc_bf16_value("),
    ("check_skips_partial_last_block",
     "nblk = (T + block_size - 1) / block_size;\n        for (j = 0; j < nblk; ++j) {\n            int32_t p = block_tables",
     "nblk = T / block_size;\n        for (j = 0; j < nblk; ++j) {\n            int32_t p = block_tables"),
    ("check_pool_bound_inclusive", "if (p < 0 || p >= num_blocks)\n                return -(1 + b);",
     "if (p < 0 || p > num_blocks)\n                return -(1 + b);"),
    ("check_context_bound_strict", "(int64_t)T > (int64_t)max_blocks * block_size",
     "(int64_t)T >= (int64_t)max_blocks * block_size"),
    ("split_range_overlaps", "int32_t t0 = s * split_tokens;",
     "int32_t t0 = s > 0 ? s * split_tokens - 1 : 0;"),
    ("mq_position_off_by_one", "int32_t p = T - q + i;", "int32_t p = T - q + i - 1;"),
    ("mq_not_causal", "kv_dtype, scale, 0, hq, 0, p + 1,", "kv_dtype, scale, 0, hq, 0, T,"),
    ("mq_query_row_of_sequence", "const uint16_t* qrow = query + row * Hq * D;",
     "const uint16_t* qrow = query + (int64_t)b * Hq * D;"),
    ("write_rows_reversed", "int32_t t = T - q + i;", "int32_t t = T - 1 - i;"),
    ("int8_zero_point_added", "((double)((const uint8_t*)cache)[i] - (double)scales[si + 1])",
     "((double)((const uint8_t*)cache)[i] + (double)scales[si + 1])"),
    ("int8_truncates", "v = (double)rintf(y) + (double)zero_point;",
     "v = (double)truncf(y) + (double)zero_point;"),
    ("int8_clamp_254", "if (v > 255.0)\n        v = 255.0;", "if (v > 254.0)\n        v = 254.0;"),
    ("per_head_scale_by_block", "case 2: return h;", "case 2: return (int64_t)phys * Hkv + h;"),
    ("per_tensor_scale_by_head", "case 3: return 0;", "case 3: return h;"),
    ("int8_params_unpaired", "default: return 2 * ((int64_t)phys * Hkv + h);",
     "default: return (int64_t)phys * Hkv + h;"),
    ("gather_by_position", "(const char*)pool + (int64_t)ids[i] * block_bytes",
     "(const char*)pool + (int64_t)i * block_bytes"),
    ("scatter_by_position", "memcpy((char*)pool + (int64_t)ids[i] * block_bytes,",
     "memcpy((char*)pool + (int64_t)i * block_bytes,"),
    ("copy_reversed", "memcpy((char*)pool + (int64_t)dst[i] * block_bytes,\n               (const char*)pool + (int64_t)src[i] * block_bytes",
     "memcpy((char*)pool + (int64_t)src[i] * block_bytes,\n               (const char*)pool + (int64_t)dst[i] * block_bytes"),
    ("write_v_with_k_scale", "store_value(v_cache, v_scale, kv_dtype, dst, v_rows[src]",
     "store_value(v_cache, k_scale, kv_dtype, dst, v_rows[src]"),
]


def _run_mutant(tmpdir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"{name}: pattern not found"
    mut = src.replace(old, new)
    c_path = os.path.join(tmpdir, f"{name}.c")
    so_path = os.path.join(tmpdir, f"{name}.so")
    open(c_path, "w").write(mut)
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                    "-w", "-o", so_path, c_path, "-lm"], check=True)
    env = dict(os.environ, PKV_ORACLE_LIB=so_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return name, r.returncode


def test_every_planted_mistake_is_caught(tmp_path):
    with cf.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        futs = [ex.submit(_run_mutant, str(tmp_path), *m) for m in MUTANTS]
        results = [f.result() for f in futs]
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"


BM_SRC = os.path.join(ROOT, "oracle", "block_manager.py")
BM_MUTANTS = [
    ("key_not_cumulative", "return (self.ns, tuple(toks[:end]))",
     "return (self.ns, tuple(toks[end - self.bs:end]))"),
    ("last_token_reused", "for j in range((len(toks) - 1) // bs):",
     "for j in range(len(toks) // bs):"),
    ("evicts_newest", "victim = self.lru.pop(0)", "victim = self.lru.pop()"),
    ("releases_first_block_first", "for b in reversed(self.tables.pop(seq)):",
     "for b in self.tables.pop(seq):"),
    ("no_copy_on_write", "elif self.ref[table[-1]] > 1:", "elif False:"),
    ("highest_free_block", "return self.free.pop(0)", "return self.free.pop()"),
    ("evicted_key_kept", "del self.cache[self.key[victim]]", "pass"),
    ("evicts_before_free", "if self.free:\n            self.free.sort()",
     "if self.free and not self.lru:\n            self.free.sort()"),
]


def _run_bm_mutant(tmpdir, name, old, new):
    src = open(BM_SRC).read()
    assert src.count(old) >= 1, f"{name}: pattern not found"
    path = os.path.join(tmpdir, f"bm_{name}.py")
    open(path, "w").write(src.replace(old, new))
    env = dict(os.environ, PKV_ORACLE_BM=path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_block_manager.py"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_block_manager_mistake_is_caught(tmp_path):
    with cf.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        futs = [ex.submit(_run_bm_mutant, str(tmp_path), *m) for m in BM_MUTANTS]
        results = [f.result() for f in futs]
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, f"block-manager pins did not catch: {survivors}"


def test_unmutated_copy_passes(tmp_path):
    name, rc = _run_mutant(str(tmp_path), "identity", "#include <math.h>", "#include <math.h>")
    assert rc == 0
    name, rc = _run_bm_mutant(str(tmp_path), "identity", "class NoSpace", "class NoSpace")
    assert rc == 0
