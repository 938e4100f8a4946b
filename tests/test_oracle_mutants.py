"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
the pins catch every one of them.  The real oracle is never modified: each
mutant is a patched copy of oracle.c compiled into a temporary directory."""
import os
import shutil

import pytest

import oracle
from oracle import build as oracle_build
import oracle_pins

ORACLE_DIR = os.path.dirname(oracle_build.SRC)

MUTANTS = {
    "emb_drops_last_index": (
        "for (int64_t l = start; l < end; ++l) {\n"
        "          int64_t r = idx[l];\n"
        "          if (r < 0 || r >= rows[k]) return -2;\n"
        "          acc += (double)W",
        "for (int64_t l = start; l + 1 < end; ++l) {\n"
        "          int64_t r = idx[l];\n"
        "          if (r < 0 || r >= rows[k]) return -2;\n"
        "          acc += (double)W"),
    "emb_ext_drops_first_index": (
        "for (int64_t l = start; l < end; ++l) {\n"
        "          int64_t r = idx[l];\n"
        "          if (r < 0 || r >= rows[k]) return -2;\n"
        "          int64_t e",
        "for (int64_t l = start + 1; l < end; ++l) {\n"
        "          int64_t r = idx[l];\n"
        "          if (r < 0 || r >= rows[k]) return -2;\n"
        "          int64_t e"),
    "emb_wrong_column": (
        "acc += (double)W[r * (int64_t)D + d];",
        "acc += (double)W[r * (int64_t)D];"),
    "emb_transposed_output": (
        "out[((int64_t)b * K + k) * D + d] = (float)acc;",
        "out[((int64_t)k * B + b) * D + d] = (float)acc;", 0),
    "emb_ext_transposed_output": (
        "out[((int64_t)b * K + k) * D + d] = (float)acc;",
        "out[((int64_t)k * B + b) * D + d] = (float)acc;", 1),
    "emb_last_bag_empty": (
        "end = (b + 1 < B) ? (int64_t)offsets[k][b + 1] : n_idx[k];",
        "end = (b + 1 < B) ? (int64_t)offsets[k][b + 1] : start;", 0),
    "emb_ext_last_bag_empty": (
        "end = (b + 1 < B) ? (int64_t)offsets[k][b + 1] : n_idx[k];",
        "end = (b + 1 < B) ? (int64_t)offsets[k][b + 1] : start;", 1),
    "pair_order_column_major": (
        "for (int64_t i = 1; i < F; ++i)\n"
        "      for (int64_t j = 0; j < i; ++j) row[D + p++] = (float)Z[i * F + j];",
        "for (int64_t j = 0; j < F; ++j)\n"
        "      for (int64_t i = j + 1; i < F; ++i) row[D + p++] = (float)Z[i * F + j];"),
    "dot_drops_first_term": (
        "for (int32_t d = 0; d < D; ++d) acc += X[i * D + d] * X[j * D + d];",
        "for (int32_t d = 1; d < D; ++d) acc += X[i * D + d] * X[j * D + d];"),
    "dense_feature_sign": (
        "X[d] = (double)dense[(int64_t)b * D + d];",
        "X[d] = -(double)dense[(int64_t)b * D + d];"),
    "dense_copy_dropped": (
        "memcpy(row, dense + (int64_t)b * D, sizeof(float) * (size_t)D);",
        "memset(row, 0, sizeof(float) * (size_t)D);"),
    "linear_transposed_weight": (
        "(double)W[(int64_t)n * Kd + k];",
        "(double)W[(int64_t)k * N + n];"),
    "linear_drops_bias": (
        "double acc = bias ? (double)bias[n] : 0.0;",
        "double acc = 0.0;"),
    "relu_wrong_branch": (
        "acc = acc > 0.0 ? acc : 0.0;",
        "acc = acc > 0.0 ? acc : -acc;"),
    "sigmoid_wrong_sign": (
        "acc = 1.0 / (1.0 + exp(-acc));",
        "acc = 1.0 / (1.0 + exp(acc));"),
    "pair_column_formula": (
        "*j_out = p - i * (i - 1) / 2;",
        "*j_out = p - i * (i + 1) / 2;"),
    "mean_wrong_count": (
        "if (pool == ORACLE_POOL_MEAN && end > start) acc /= (double)(end - start);",
        "if (pool == ORACLE_POOL_MEAN && end > start) acc /= (double)(end - start + 1);"),
    "weights_first_only": (
        "double w = weights ? (double)weights[k][l] : 1.0;",
        "double w = weights ? (double)weights[k][start] : 1.0;"),
    "bf16_wrong_shift": (
        "uint32_t bits = (uint32_t)b << 16;",
        "uint32_t bits = (uint32_t)b << 15;"),
    "fp8_exponent_bias_8": (
        "v = ldexp((double)(8 + man), expo - 10);",
        "v = ldexp((double)(8 + man), expo - 11);"),
    "fp8_subnormal_scale": (
        "v = ldexp((double)man, -9);",
        "v = ldexp((double)man, -10);"),
    "fp8_no_nan_code": (
        "if (expo == 15 && man == 7) return NAN;",
        "if (expo == 16 && man == 7) return NAN;"),
    "scale_dropped": (
        "if (scales) acc *= (double)scales[k];",
        "if (scales) acc *= 1.0;"),
    "pair_float_sqrt_no_fixups": (
        "  int64_t i = (int64_t)floor((1.0 + sqrt(1.0 + 8.0 * (double)p)) / 2.0);\n"
        "  while (i * (i - 1) / 2 > p) --i;\n"
        "  while ((i + 1) * i / 2 <= p) ++i;\n",
        "  int64_t i = (int64_t)floorf((1.0f + sqrtf(1.0f + 8.0f * (float)p)) / 2.0f);\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new, *which = MUTANTS[name]
    src = open(oracle_build.SRC).read()
    if which:      # the site occurs once per emb-bag function: patch one of them
        sites = src.split(old)
        assert len(sites) == 3, f"mutation site for {name} not found exactly twice"
        patched = old.join(sites[:which[0] + 1]) + new + old.join(sites[which[0] + 1:])
    else:
        assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
        patched = src.replace(old, new)
    shutil.copy(os.path.join(ORACLE_DIR, "oracle.h"), tmp_path / "oracle.h")
    mutant_c = tmp_path / "oracle.c"
    mutant_c.write_text(patched)
    so = str(tmp_path / "liboracle_mutant.so")
    oracle_build.build(str(mutant_c), so, extra_flags=["-Wno-error"])
    lib = oracle.load(so)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError) as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
