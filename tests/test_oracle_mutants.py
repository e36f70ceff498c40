"""Mutation check of the oracle's pins.

Each mutant is a copy of oracle.c with one plausible mistake planted in it (a
dropped term, a wrong sign, index or bias, a swapped nibble or pair order, a
wrong rounding rule). It is compiled on the CPU into a temporary library and
the whole pin suite is run against it in a child process; the test passes
when at least one pin fails (or the child crashes). A mutant that no pin
catches means the pins would not notice that mistake in the oracle.
"""
import json
import os
import subprocess
import sys
import tempfile

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("epilogue_drops_bias",
     "if (bias) v += (double)bias[n];",
     "(void)bias;"),
    ("epilogue_residual_sign",
     "if (res_f32) v += (double)res_f32[i];",
     "if (res_f32) v -= (double)res_f32[i];"),
    ("epilogue_residual_after_activation",
     "out[i] = act_apply(v, act);",
     "out[i] = act_apply(v - (res_f32 ? (double)res_f32[i] : 0.0), act) + (res_f32 ? (double)res_f32[i] : 0.0);"),
    ("silu_exponent_sign",
     "case 2: return x / (1.0 + exp(-x));",
     "case 2: return x / (1.0 + exp(x));"),
    ("gelu_sqrt2_inverted",
     "case 3: return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));",
     "case 3: return 0.5 * x * (1.0 + erf(x * sqrt(2.0)));"),
    ("relu_flipped",
     "case 1: return x > 0.0 ? x : 0.0;",
     "case 1: return x < 0.0 ? x : 0.0;"),
    ("round_half_quantum",
     "ldexp(1.0, exp2 - 10);",
     "ldexp(1.0, exp2 - 11);"),
    ("round_half_no_overflow",
     "const double y = r > 65504.0 ? INFINITY : r;",
     "const double y = r;"),
    ("round_half_truncates",
     "nearbyint(ax / quantum) * quantum;",
     "floor(ax / quantum) * quantum;"),
    ("dequant_drops_offset",
     "return offset + scale * (double)code_at(q, K, bits, n, k);",
     "return scale * (double)code_at(q, K, bits, n, k);"),
    ("dequant_drops_scale",
     "return offset + scale * (double)code_at(q, K, bits, n, k);",
     "return offset + (double)code_at(q, K, bits, n, k);"),
    ("dequant_sign_flip",
     "return offset + scale * (double)code_at(q, K, bits, n, k);",
     "return offset - scale * (double)code_at(q, K, bits, n, k);"),
    ("nibble_order_swapped",
     "return (k & 1) ? (byte >> 4) : (byte & 15);",
     "return (k & 1) ? (byte & 15) : (byte >> 4);"),
    ("pair_order_swapped",
     "double offset = pairs[((size_t)n * nblk + b) * 2 + 0];\n    double scale = pairs[((size_t)n * nblk + b) * 2 + 1];",
     "double offset = pairs[((size_t)n * nblk + b) * 2 + 1];\n    double scale = pairs[((size_t)n * nblk + b) * 2 + 0];"),
    ("block_index_wrong",
     "const int b = k / block;",
     "const int b = (k / block + 1) % nblk;"),
    ("f32_transposed_b",
     "(double)B[(size_t)k * N + n]",
     "(double)B[((size_t)n * K + k) % ((size_t)K * N)]"),
    ("f32_skips_last_k",
     "for (int k = 0; k < K; ++k)\n                acc += (double)A[(size_t)m * K + k] * (double)B",
     "for (int k = 0; k + 1 < K; ++k)\n                acc += (double)A[(size_t)m * K + k] * (double)B"),
    ("blockq_a_index_wrong",
     "acc += orc_half_to_double(A[(size_t)m * K + k]) *",
     "acc += orc_half_to_double(A[(size_t)m * K + (k ^ 1) % K]) *"),
    ("half_exponent_bias",
     "v = ldexp((double)(1024 + frac), expo - 25);",
     "v = ldexp((double)(1024 + frac), expo - 24);"),
    ("half_subnormal_scale",
     "v = ldexp((double)frac, -24);",
     "v = ldexp((double)frac, -25);"),
    ("half_drops_sign",
     "return sign ? -v : v;",
     "return v;"),
    ("quant_scale_denominator",
     "float scale = (float)((hi - lo) / (double)qmax);",
     "float scale = (float)((hi - lo) / (double)(qmax + 1));"),
    ("quant_floor_not_rint",
     "double r = rint(t);",
     "double r = floor(t);"),
    ("quant_offset_is_max",
     "float offset = (float)lo;",
     "float offset = (float)hi;"),
    ("quant_nibble_shift",
     "|= (uint8_t)(code << (4 * (k & 1)));",
     "|= (uint8_t)(code << (4 * ((k + 1) & 1)));"),
    ("actq_ties_away",
     "float r = rintf(t);              /* ties to even */",
     "float r = roundf(t);"),
    ("actq_range_128",
     "float s = amax / 127.0f;",
     "float s = amax / 128.0f;"),
    ("actq_rowsum_abs",
     "sum += (int32_t)r;",
     "sum += (int32_t)fabsf(r);"),
    ("actq_zero_row_scale",
     "sa[m] = 0.0f;",
     "sa[m] = 1.0f;"),
    ("actq_reciprocal_multiply",
     "float t = a / s;",
     "float t = a * (1.0f / s);"),
    ("w4a8_dot_k_swapped",
     "acc += (int64_t)qa[(size_t)m * K + k] * (int64_t)code_at(q, K, 4, n, k);",
     "acc += (int64_t)qa[(size_t)m * K + (k ^ 1)] * (int64_t)code_at(q, K, 4, n, k);"),
    ("w4a8_rescale_drops_offset",
     "(scale * (double)D[(size_t)m * N + n] + offset * (double)S[m]);",
     "(scale * (double)D[(size_t)m * N + n]);"),
    ("w4a8_rescale_drops_sa",
     "C[(size_t)m * N + n] = (double)sa[m] *",
     "C[(size_t)m * N + n] = 1.0 *"),
]

RUNNER = r"""
import json, sys
sys.path[:0] = [{root!r}, {tests!r}]
from oracle import oracle as O
import oracle_pins
lib = O.load({lib!r})
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except Exception as e:
        failed.append(pin.__name__)
print(json.dumps(failed))
"""


def _build_mutant(tmp, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutant {name}: pattern not found in oracle.c"
    mutated = src.replace(old, new)
    assert mutated != src
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(mutated)
    return O.build(path, os.path.join(tmp, f"lib{name}.so"))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_mutant(tmp, name, old, new)
        code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
        r = subprocess.run([sys.executable, "-c", code], capture_output=True,
                           text=True, timeout=300)
        if r.returncode != 0:
            return              # the mutant crashed the pins: caught
        failed = json.loads(r.stdout.strip().splitlines()[-1])
        assert failed, f"no pin catches mutant {name}"


def test_unmutated_oracle_passes_every_pin():
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=O.load()._name)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert json.loads(r.stdout.strip().splitlines()[-1]) == []
