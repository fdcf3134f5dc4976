"""Plant a mistake in a copy of the oracle and check that a pin catches it.

Each mutant changes one place of oracle.c (on the CPU, in a temporary
directory) to a plausible slip: a tie broken the wrong way, a missing
renormalisation, an unstable sort, swapped gate and up projections, a wrong
sign, a transposed operand, a dropped bias, an ignored weight, an off-by-one
in the partition, a wrong gather divisor, fp32 accumulation in the router, a
wrong FP8 exponent bias or subnormal scale, an FP8 weight scale from the
wrong row or dropped.
"""
import os
import shutil

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "tie_to_higher_id": ("if (best < 0 || l[e] > l[best]) best = e;",
                         "if (best < 0 || l[e] >= l[best]) best = e;"),
    "no_renormalisation": ("weights[(int64_t)t * k + j] = p[ids[(int64_t)t * k + j]] / s;",
                           "weights[(int64_t)t * k + j] = p[ids[(int64_t)t * k + j]];"),
    "unstable_within_expert": ("int32_t p = cursor[e - first]++;",
                               "int32_t p = offsets[e - first + 1] - 1 - (cursor[e - first]++ - offsets[e - first]);"),
    "gate_up_swapped": ("a[i] = g / (1.0 + exp(-g)) * u;", "a[i] = u / (1.0 + exp(-u)) * g;"),
    "silu_sign": ("a[i] = g / (1.0 + exp(-g)) * u;", "a[i] = g / (1.0 + exp(g)) * u;"),
    "w2_transposed": ("acc += bf16_val(w[i]) * a[i];",
                      "acc += bf16_val(w2e[(int64_t)i * H + c]) * a[i];"),
    "bias_dropped": ("if (bias) acc += (double)bias[e];", "(void)bias;"),
    "combine_ignores_weight": (
        "if (p >= 0) acc += weights[(int64_t)t * k + j] * expert_out[(int64_t)p * H + c];",
        "if (p >= 0) acc += expert_out[(int64_t)p * H + c];"),
    "partition_off_by_one": ("for (int32_t q = 0; q < s; ++q) f += base + (q < rem ? 1 : 0);",
                             "for (int32_t q = 0; q < s; ++q) f += base + (q <= rem ? 1 : 0);"),
    "gather_divisor": ("int32_t tok = permuted_rows[p] / k;", "int32_t tok = permuted_rows[p] % T;"),
    "router_fp32_accumulate": ("double acc = 0.0;\n        for (int32_t h = 0; h < H; ++h) acc += xr[h] * (double)w[h];",
                               "float acc = 0.0f;\n        for (int32_t h = 0; h < H; ++h) acc += (float)(xr[h] * (double)w[h]);"),
    "softmax_not_shifted_by_max": ("p[e] = exp((double)l[e] - m);", "p[e] = exp((double)l[e] - m) + 1e-3;"),
    "e4m3_exponent_bias": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);",
                           "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_subnormal_scale": ("v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    "fp8_up_scale_from_gate_row": ("const double sg = (double)w1s[i], su = (double)w1s[I + i];",
                                   "const double sg = (double)w1s[i], su = (double)w1s[i];"),
    "fp8_w2_scale_dropped": ("const double sc = (double)w2s[c];", "const double sc = 1.0;"),
    "counts_local_only": ("for (int64_t r = 0; r < n; ++r) counts[ids[r]] += 1;",
                          "for (int64_t r = 0; r < n; ++r) if (ids[r] >= first && ids[r] < first + L) counts[ids[r]] += 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "oracle_mutant.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / "liboracle_mutant.so")
    oracle.compile_oracle(str(path), so)
    orc = oracle.Oracle(so)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
