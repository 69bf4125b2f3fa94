"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of the oracle (CPU only) and
runs the pin suite against that copy; the suite has to fail. The real oracle
is never modified.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "nibble_swap": ("q[:, 0::2] = wq & 0x0F\n    q[:, 1::2] = wq >> 4",
                    "q[:, 1::2] = wq & 0x0F\n    q[:, 0::2] = wq >> 4"),
    "drop_bias": ("return s[:, g] * q + b[:, g]", "return s[:, g] * q"),
    "bias_sign": ("return s[:, g] * q + b[:, g]", "return s[:, g] * q - b[:, g]"),
    "group_index": ("g = np.arange(K) // group", "g = np.arange(K) % (K // group)"),
    "group_fixed_64": ("g = np.arange(K) // group", "g = (np.arange(K) // 64) % (K // group)"),
    "reversed_columns": ("y[:, c0:c0 + sel.size] = xd @ w.T",
                         "y[:, c0:c0 + sel.size] = (w @ xd.T).T[:, ::-1]"),
    "argmax_last_tie": ("return int(np.flatnonzero(v == top)[0])",
                        "return int(np.flatnonzero(v == top)[-1])"),
    "nan_ignored": ("if nan.any():\n        return int(np.flatnonzero(nan)[0])",
                    "if False:\n        pass\n    v = np.where(nan, -np.inf, v)"),
    "walk_off_by_one": ("while L < limit and int(row_argmax[L]) == int(draft[L]):",
                        "while L < limit and int(row_argmax[L + 1]) == int(draft[L]):"),
    "walk_counts_all_matches": (
        "while L < limit and int(row_argmax[L]) == int(draft[L]):\n        L += 1",
        "for i in range(limit):\n        L += int(int(row_argmax[i]) == int(draft[i]))"),
    "walk_ignores_draft_len": ("limit = T - 1 if draft_len is None else min(max(int(draft_len), 0), T - 1)",
                               "limit = T - 1"),
    "walk_draft_len_off_by_one": (
        "limit = T - 1 if draft_len is None else min(max(int(draft_len), 0), T - 1)",
        "limit = T - 1 if draft_len is None else min(max(int(draft_len) + 1, 0), T - 1)"),
    "margin_distinct_second": ("second = np.delete(v, i).max()",
                               "second = v[v != top].max() if (v != top).any() else top"),
    "margin_ignores_nan": ("if np.isnan(v).any():\n        return np.float32(np.nan)",
                           "if False:\n        pass\n    v = np.where(np.isnan(v), -np.inf, v)"),
    "margin_sign": ("return np.float32(top) - np.float32(second)",
                    "return np.float32(second) - np.float32(top)"),
    "silu_no_gate_factor": ("return g / (1.0 + np.exp(-g))", "return 1.0 / (1.0 + np.exp(-g))"),
    "silu_exp_sign": ("return g / (1.0 + np.exp(-g))", "return g / (1.0 + np.exp(g))"),
    "swiglu_halves_swapped": ("return silu_ref(y[..., :nh]) * y[..., nh:]",
                              "return silu_ref(y[..., nh:]) * y[..., :nh]"),
    "swiglu_interleaved": ("return silu_ref(y[..., :nh]) * y[..., nh:]",
                           "return silu_ref(y[..., 0::2]) * y[..., 1::2]"),
    "swiglu_up_offset": ("up = qgemm_ref(x, act, wq, scales, biases, group, cols=nh + idx)",
                         "up = qgemm_ref(x, act, wq, scales, biases, group, cols=idx)"),
    "bf16_decode_shift": ("u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16",
                          "u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 15"),
    "fp16_scale_as_bf16": (
        "return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)",
        "return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16)"
        ".view(np.float32).astype(np.float64)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "vqv_ref.py")).read()
    old, new = MUTANTS[name]
    assert old in src, f"mutation site for {name} not found"
    for d in ("oracle", "gen"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    (tmp_path / "oracle" / "vqv_ref.py").write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle.py"], cwd=tmp_path, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
