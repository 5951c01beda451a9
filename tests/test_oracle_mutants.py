"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU
only), builds it into a temporary library, and runs the pin tests against it
in a child process: the run must fail.  A mutant that survives means a part
of the oracle is not really pinned.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "q4_oracle.c")

# (name, text to find, replacement)
MUTANTS = [
    ("q4_nibble_order_interleaved", "out[i] = (uint8_t)(code[i] | (code[i + 16] << 4));",
     "out[i] = (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));"),
    ("q4_scale_sign", "float dd = maxv / -8.0f;", "float dd = maxv / 8.0f;"),
    ("q4_scale_unsigned", "float dd = maxv / -8.0f;", "float dd = amax / -8.0f;"),
    ("q4_last_max_wins", "if (a > amax) { amax = a; maxv = blk[j]; }", "if (a >= amax) { amax = a; maxv = blk[j]; }"),
    ("q4_round_half_even", "int c = (int)u;              /* u >= 0.5: truncation == floor */",
     "int c = (int)rintf(t + 8.0f);"),
    ("q4_id_from_d16", "float dd = maxv / -8.0f;\n            float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;",
     "float dd = maxv / -8.0f;\n            float id = (dd != 0.0f) ? 1.0f / or_f16_to_f32(or_f32_to_f16(dd)) : 0.0f;"),
    ("q4_no_clamp", "code[j] = c < 15 ? c : 15;", "code[j] = c & 15;"),
    ("q4_dequant_offset", "out[n * K + b * 32 + j] = (double)(q4_code(blk, j) - 8) * dd;",
     "out[n * K + b * 32 + j] = (double)(q4_code(blk, j) - 7) * dd;"),
    ("q4_code_high_low_swapped", "return j < 16 ? (blk16[j] & 0x0F) : (blk16[j - 16] >> 4);",
     "return j < 16 ? (blk16[j] >> 4) : (blk16[j - 16] & 0x0F);"),
    ("q8_round_half_even", "int q = (int)roundf(t);", "int q = (int)rintf(t);"),
    ("q8_id_from_d16", "float dd = amax / 127.0f;\n            float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;",
     "float dd = amax / 127.0f;\n            float id = (dd != 0.0f) ? 1.0f / or_f16_to_f32(or_f32_to_f16(dd)) : 0.0f;"),
    ("q8_sum_unscaled", "float s = dd * (float)sum;", "float s = (float)sum;"),
    ("q8_scale_128", "float dd = amax / 127.0f;", "float dd = amax / 128.0f;"),
    ("dots_offset_dropped", "for (int j = 0; j < 32; j++) s += (q4_code(blk, j) - 8) * (int32_t)a[j];\n                isum",
     "for (int j = 0; j < 32; j++) s += (q4_code(blk, j)) * (int32_t)a[j];\n                isum"),
    ("gemv_uses_sum_not_scale", "double d8 = (double)or_f16_to_f32(xds[(m * nb + b) * 2]);",
     "double d8 = (double)or_f16_to_f32(xds[(m * nb + b) * 2 + 1]);"),
    ("matmul_transposed_output", "            y[m * N + n] = acc;\n        }\n}\n\n/* The same sum",
     "            y[n * M + m] = acc;\n        }\n}\n\n/* The same sum"),
    ("matmul_drops_last_k", "for (int64_t k = 0; k < K; k++) acc += xr[k] * wr[k];\n            y[m * N + n]",
     "for (int64_t k = 0; k + 1 < K; k++) acc += xr[k] * wr[k];\n            y[m * N + n]"),
    ("f16_ties_away", "if (rem > half || (rem == half && (q & 1))) q++;", "if (rem >= half) q++;"),
    ("f16_subnormal_flush", "bits = (uint32_t)q;                     /* subnormal units of 2^-24 */",
     "bits = 0;"),
    ("affine_scale_16_levels", "float s32 = (mx - mn) / 15.0f;", "float s32 = (mx - mn) / 16.0f;"),
    ("affine_round_down", "float f = floorf(r + 0.5f);", "float f = floorf(r);"),
    ("affine_round_half_even", "float f = floorf(r + 0.5f);", "float f = rintf(r);"),
    ("affine_nibble_swap", "wq[n * (K / 2) + (g * G + j) / 2] = (uint8_t)(c[0] | (c[1] << 4));",
     "wq[n * (K / 2) + (g * G + j) / 2] = (uint8_t)(c[1] | (c[0] << 4));"),
    ("affine_dequant_bias_dropped", "out[n * K + k] = (double)affine_code(wq, K, n, k) * s + b;",
     "out[n * K + k] = (double)affine_code(wq, K, n, k) * s;"),
    ("affine8_scale_256_levels", "float step32 = (hi - lo) / 255.0f;", "float step32 = (hi - lo) / 256.0f;"),
    ("affine8_round_down", "float f8 = floorf(t + 0.5f);", "float f8 = floorf(t);"),
    ("affine8_round_half_even", "float f8 = floorf(t + 0.5f);", "float f8 = rintf(t);"),
    ("affine8_clamp_254", "(f8 > 255.0f ? 255 : (int)f8)", "(f8 > 254.0f ? 254 : (int)f8)"),
    ("affine8_dequant_bias_dropped", "out[n * K + k] = (double)wq[n * K + k] * sv + bv;",
     "out[n * K + k] = (double)wq[n * K + k] * sv;"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(source, name, find, repl):
    assert source.count(find) == 1, f"mutation site for {name} not found exactly once"
    mutated = source.replace(find, repl)
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "mutant.c")
        so = os.path.join(td, "libmutant.so")
        with open(c, "w") as f:
            f.write(mutated)
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                               "-std=c11", c, "-o", so, "-lm"])
        env = dict(os.environ, Q4_ORACLE_LIB=so, OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
