"""The oracle's pins must catch plausible mistakes.  Each mutant below is a copy of the
oracle source with one planted error (built on the CPU into a temp dir); the pin suite
is run against it in a subprocess and must fail.  A mutant that crashes also counts as
caught."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")
PINS = ["tests/test_oracle_index.py", "tests/test_oracle_sizes_pack.py",
        "tests/test_oracle_attention.py"]

MUTANTS = {
    "causal_excludes_self": ("(seq_lens_kv[b] - n + i + 1)", "(seq_lens_kv[b] - n + i)"),
    "causal_top_left": ("(seq_lens_kv[b] - n + i + 1)", "(i + 1)"),
    "gqa_interleaved": ("const int32_t g = h / group;", "const int32_t g = h % num_kv_heads;"),
    "rope_dropped": ("for (int32_t d = 0; d < Dr; ++d)\n                    s +=",
                     "for (int32_t d = 0; d < 0; ++d)\n                    s +="),
    "offset_off_by_one": ("int64_t offset = pos % block_size;",
                          "int64_t offset = (pos + 1) % block_size;"),
    "block_off_by_one": ("int64_t logical_block = pos / block_size;",
                         "int64_t logical_block = (pos + 1) / block_size;"),
    "new_token_at_L_plus_1": ("int64_t pos = (int64_t)lens_before[b] + (t - cu_new[b]);",
                              "int64_t pos = (int64_t)lens_before[b] + (t - cu_new[b]) + 1;"),
    "scale_dropped": ("score[p] = scale * s;", "score[p] = s;"),
    "no_normalise": ("visible > 0 ? acc[d] / z : 0.0", "visible > 0 ? acc[d] : 0.0"),
    "lse_is_max": ("m + log(z) : -INFINITY", "m : -INFINITY"),
    "bf16_wrong_shift": ("<< 16;", "<< 15;"),
    "kv_head_stride": ("(slot * num_kv_heads + g) * head_dim_v + d",
                       "(slot * num_kv_heads) * head_dim_v + d"),
    "v_reads_k": ("acc[d] += w * load_elem(v_cache,", "acc[d] += w * load_elem(k_cache,"),
    "merge_ignores_weight": ("z += w * l[s * rows + r];", "z += l[s * rows + r];"),
    "write_wrong_row": ("memcpy(cache + slots[t] * row_bytes, rows + t * row_bytes,",
                        "memcpy(cache + slots[t] * row_bytes, rows + 0 * row_bytes,"),
    "dup_not_detected": ("if (seen[slots_out[t]]) { rc = ORC_ERR_DUP; break; }", ""),
    "window_ignored": ("if (window > 0 && visible - window > 0) lo = visible - window;", ""),
    "window_off_by_one": ("lo = visible - window;", "lo = visible - window + 1;"),
}


@pytest.fixture(scope="module")
def src():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src, tmp_path):
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-w",
                           "-o", str(so), str(c), "-lm"])
    env = dict(os.environ, PKV_ORACLE_LIB_OVERRIDE=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pin suite:\n{r.stdout[-2000:]}"
