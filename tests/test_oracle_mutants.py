"""Plant plausible mistakes in copies of the oracle source and check that the
pin suite catches every one of them (on the CPU; the real oracle is untouched).
"""
import json
import os
import subprocess
import sys

import pytest

import oracle

_RUNNER = """
import json, sys
sys.path[:0] = [{pkgroot!r}, {root!r}, {tests!r}]
import oracle
from oracle_pins import ALL_PINS
lib = oracle.load({so!r})
failed = []
for pin in ALL_PINS:
    try:
        pin(lib)
    except Exception:
        failed.append(pin.__name__)
print(json.dumps(failed))
"""

# (name, text in oracle/indexer_oracle.c, replacement)
MUTANTS = [
    ("no_relu", "double rect = dot > 0.0 ? dot : 0.0;", "double rect = dot;"),
    ("sum_then_relu", "total += (double)w[h] * rect;", "total += (double)w[h] * dot;"),
    ("wrong_weight_index", "total += (double)w[h] * rect;", "total += (double)w[0] * rect;"),
    ("key_index_shift", "dot += q_th[i] * k_s[i];", "dot += q_th[i] * k_s[(i + 1) % d];"),
    ("key_dot_reversed", "dot += q_th[i] * k_s[i];", "dot += q_th[i] * k_s[d - 1 - i];"),
    ("query_head_stride_wrong", "const double *q_th = q_t + (int64_t)h * d;", "const double *q_th = q_t + (int64_t)(h % 2) * d;"),
    ("mask_inside_relu", "            if (mask)\n                v += half_to_double(mask[(int64_t)t * mask_stride_t + s]);",
     "            if (mask)\n                v = fmax(v + half_to_double(mask[(int64_t)t * mask_stride_t + s]), 0.0);"),
    ("mask_dropped", "            if (mask)\n                v += half_to_double(mask[(int64_t)t * mask_stride_t + s]);", ""),
    ("f16_bias_off_by_one", "expo - 25", "expo - 24"),
    ("f16_subnormal_wrong", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("ties_to_higher_index", "return (x->index > y->index) - (x->index < y->index);",
     "return (x->index < y->index) - (x->index > y->index);"),
    ("neg_inf_selectable", "if (isnan(v) || (isinf(v) && v < 0))", "if (isnan(v))"),
    ("ascending_order", "if (x->score > y->score) return -1;\n    if (x->score < y->score) return 1;",
     "if (x->score < y->score) return -1;\n    if (x->score > y->score) return 1;"),
    ("no_padding", "idx_out[i] = -1;", "idx_out[i] = 0;"),
    ("decode_visibility_off_by_one", "(int64_t)seq_lens[r] - Q + 1 + j", "(int64_t)seq_lens[r] - Q + j"),
    ("decode_row_order_swapped", "int64_t t = (int64_t)r * Q + j;", "int64_t t = (int64_t)j * R + r;"),
    ("decode_ignores_block_table", "(phys * block_size + s % block_size)", "((int64_t)s)"),
    ("decode_first_block_only", "s / block_size];", "0];"),
    ("decode_mask_dropped", "                if (mask)\n                    v += half_to_double(mask[t * mask_stride_t + s]);", ""),
    ("decode_mask_row_by_request", "mask[t * mask_stride_t + s]", "mask[(int64_t)r * mask_stride_t + s]"),
    ("blocks_forced_last", "return x->forced ? -1 : 1;", "return x->forced ? 1 : -1;"),
    ("blocks_forced_by_score", "if (!x->forced) {                          /* others by score */",
     "if (1) {"),
    ("blocks_local_window_off_by_one", "s >= n - local_blocks);", "s > n - local_blocks);"),
    ("blocks_init_window_off_by_one", "scratch[m].forced = s < init_blocks ||", "scratch[m].forced = s <= init_blocks ||"),
    ("blocks_forced_masked_selected", "            continue;                          /* never selectable, forced or not */",
     "            if (!(s < init_blocks || (local_blocks > 0 && s >= n - local_blocks))) continue;"),
    ("decode_mask_inside_relu", "v += half_to_double(mask[t * mask_stride_t + s]);",
     "v = fmax(v + half_to_double(mask[t * mask_stride_t + s]), 0.0);"),
]


# (name, text in oracle/pooling.py, replacement): the Python part of the oracle
PY_MUTANTS = [
    ("pool_divides_by_window_size", "mean = total / window.shape[0]", "mean = total / pool"),
    ("pool_windows_overlap", "k[p * pool: min((p + 1) * pool, n)]", "k[p * pool: min((p + 1) * pool + 1, n)]"),
    ("pool_rounds_through_f32", "out[p] = mean.astype(np.float16)", "out[p] = mean.astype(np.float32).astype(np.float16)"),
    ("pool_last_window_dropped", "n_pool = -(-n // pool)", "n_pool = max(n // pool, 1)"),
]


def _run_pins(tmp_path, so, pkgroot):
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER.format(pkgroot=pkgroot, root=os.path.dirname(tests), tests=tests, so=so)
    # each mutant runs in its own process so that a planted mistake cannot
    # disturb the test process
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    return res


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_pins_catch_python_mutant(name, old, new, tmp_path):
    import shutil
    pkg = tmp_path / "oracle"
    shutil.copytree(os.path.dirname(oracle.SRC), pkg, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    src = (pkg / "pooling.py").read_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    (pkg / "pooling.py").write_text(src.replace(old, new))
    res = _run_pins(tmp_path, oracle.LIB, str(tmp_path))
    assert res.returncode == 0, f"mutant {name} crashed: {res.stderr[-400:]}"
    failed = json.loads(res.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} survived every pin"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    so = str(tmp_path / "libmutant.so")
    oracle.build(str(path), so, extra_flags=("-w",))
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _RUNNER.format(pkgroot=os.path.dirname(tests), root=os.path.dirname(tests), tests=tests, so=so)
    # each mutant runs in its own process so that a planted mistake cannot
    # disturb the test process
    res = subprocess.run([sys.executable, "-c", code], capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, f"mutant {name} crashed: {res.stderr[-400:]}"
    failed = json.loads(res.stdout.strip().splitlines()[-1])
    assert failed, f"mutant {name} survived every pin"
