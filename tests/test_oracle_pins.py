"""The oracle against its pins, and the pins against planted mistakes.

Every pin is a fact fixed independently of the oracle (the pages' parameter
count, hand-worked closed forms, library routines, a dense brute force).  The
second half compiles broken copies of the oracle's source, each with one
plausible mistake, and checks that at least one pin fails on each: a pin set
that passed a broken oracle would not be pinning anything.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import brute_mixture as brute
import oracle_pins as pins
from oracle import oracle as oracle_mod


@pytest.fixture(scope="module")
def orc():
    oracle_mod.build(force=False)
    return oracle_mod.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_brute_bf16_rounding_matches_torch():
    r = np.random.default_rng(2).standard_normal(50000).astype(np.float32) * np.float32(7.0)
    ref = torch.from_numpy(r).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(brute.bf16_round(r.astype(np.float64)), ref)


# (name, text in flint_oracle.c, replacement): one plausible mistake each.
MUTANTS = [
    ("softmax_weights", "scores[e] = (float)sigmoid((double)z);", "scores[e] = (float)exp((double)z);"),
    ("tie_to_higher_index", "if (best < 0 || scores[e] > scores[best]) best = e;",
     "if (best < 0 || scores[e] >= scores[best]) best = e;"),
    ("silu_sign", "double a = g * sigmoid(g) * u;", "double a = g * sigmoid(-g) * u;"),
    ("gate_up_swapped", "double a = g * sigmoid(g) * u;", "double a = u * sigmoid(u) * g;"),
    ("dropped_shared", "for (int n = 0; n < H; ++n) acc[n] += y[n];",
     "for (int n = 0; n < H; ++n) acc[n] += 0.0 * y[n];"),
    ("transposed_down", "acc += (double)wd[(size_t)n * width + i] * h_scratch[i];",
     "acc += (double)wd[(size_t)i * H + n] * h_scratch[i];"),
    ("no_normalisation", "if (sum > 0.0) return (float)(s / sum);", "if (sum > 0.0) return (float)s;"),
    ("zero_sum_gives_nan", "return (float)(1.0 / K);", "return (float)(s / sum);"),
    ("near_tie_threshold_1e-2", "tie = gap < 1e-5;", "tie = gap < 1e-2;"),
    ("near_tie_threshold_1e-6", "tie = gap < 1e-5;", "tie = gap < 1e-6;"),
    ("near_tie_gap_at_the_top", "double gap = (double)scores[picked[K - 1]] - (double)scores[next];",
     "double gap = (double)scores[picked[0]] - (double)scores[picked[K > 1 ? 1 : 0]];"),
    ("sigmoid_in_float32", "static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }",
     "static double sigmoid(double z) { return 1.0f / (1.0f + expf((float)-z)); }"),
    ("no_h_rounding", "h_scratch[i] = d->h_is_bf16 ? round_bf16(a) : round_f32(a);", "h_scratch[i] = a;"),
    ("bf16_truncation", "double q = rint(ldexp(a, -ulp_exp));", "double q = trunc(ldexp(a, -ulp_exp));"),
    ("bias_ignored_in_route", "        if (bias) acc += (double)bias[e];\n        float z = (float)acc;\n        scores[e]",
     "        float z = (float)acc;\n        scores[e]"),
    ("dispatch_tokens_descending", "        for (int t = 0; t < T; ++t)\n            for (int k = 0; k < K; ++k)\n                if (topk_idx",
     "        for (int t = T - 1; t >= 0; --t)\n            for (int k = 0; k < K; ++k)\n                if (topk_idx"),
    ("weight_not_applied", "acc[n] += (double)w[k] * y[n];", "acc[n] += y[n];"),
    ("unweighted_gate_input", "g += (double)wg[(size_t)i * H + k] * (double)x[k];",
     "g += (double)wg[(size_t)k * width + i] * (double)x[k];"),
    ("rms_without_mean", "double r = 1.0 / sqrt(ss / (double)H + eps);", "double r = 1.0 / sqrt(ss + eps);"),
    ("mx4_high_nibble_first", "(c & 1) ? (byte >> 4) : (byte & 15u)", "(c & 1) ? (byte & 15u) : (byte >> 4)"),
    ("mx4_scale_bias_128", "ldexp(1.0, (int)s - 127)", "ldexp(1.0, (int)s - 128)"),
    ("mx4_no_subnormal", "e == 0 ? 0.5 * m", "e == 0 ? 1.0 * m"),
    ("mx4_element_bias_0", "ldexp(1.0 + 0.5 * m, (int)e - 1)", "ldexp(1.0 + 0.5 * m, (int)e)"),
    ("mx4_untile_tiles_down_first", "const int64_t tile = rb * nkb + kb;",
     "const int64_t tile = kb * (rows / 16) + rb;"),
    ("mx4_untile_row_byte_swapped", "codes_t[(tile * 16 + r) * 16 + j]", "codes_t[(tile * 16 + j) * 16 + r]"),
    ("mx4_untile_scale_rows_reversed", "= scales_t[tile * 16 + r];", "= scales_t[tile * 16 + 15 - r];"),
    ("dense_h_always_f32", "d.h_is_bf16 = h_is_bf16;", "d.h_is_bf16 = 0;"),
    ("dense_token_stride", "expert_one(&d, I, x + (size_t)t * H, wg, wu, wd, hbuf, y);",
     "expert_one(&d, I, x, wg, wu, wd, hbuf, y);"),
]


_CHILD = """
import json, sys
sys.path[:0] = [{tests!r}, {root!r}]
import oracle_pins as pins
from oracle import oracle as oracle_mod
orc = oracle_mod.Oracle({lib!r})
failed = []
for pin in pins.ALL_PINS:
    try:
        pin(orc)
    except Exception as ex:
        failed.append(pin.__name__ + ": " + type(ex).__name__)
print("FAILED_PINS=" + json.dumps(failed))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(oracle_mod.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = tmp_path / f"oracle_{name}.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle_mod.compile_source(str(mutated), str(tmp_path / f"liboracle_{name}.so"))
    here = os.path.dirname(os.path.abspath(__file__))
    code = _CHILD.format(tests=here, root=os.path.dirname(here), lib=lib)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    try:
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           timeout=300, env=env)
    except subprocess.TimeoutExpired:
        pytest.fail(f"mutant {name}: pins hung")
    if r.returncode != 0:
        return  # the mutant crashed the pins: caught
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED_PINS=")][-1]
    failed = json.loads(line.split("=", 1)[1])
    assert failed, f"no pin caught the planted mistake '{name}'"
