"""Planted mistakes in the oracle: every one must be caught by at least one pin.

Each mutant is a copy of oracle/oracle.c with one plausible error (a dropped term, a
wrong sign, index, exponent or rounding rule), compiled into a temporary directory
on the CPU. None of them touches memory outside the arrays the pins pass in.
"""
import os

import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = [
    ("f16_subnormal_exponent", "ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    ("f16_normal_exponent", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    ("f16_dropped_hidden_bit", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)f, e - 25)"),
    ("bf16_exponent", "ldexp((double)(128 + f), e - 134)", "ldexp((double)(128 + f), e - 133)"),
    ("bf16_sign", "return sign ? -v : v;\n}\n\n/* Round", "return v;\n}\n\n/* Round"),
    ("f16_encode_truncates", "double q = nearbyint(ldexp(a, 10 - E));", "double q = floor(ldexp(a, 10 - E));"),
    ("f16_encode_ties_away_subnormal", "double q = nearbyint(ldexp(a, 24));", "double q = round(ldexp(a, 24));"),
    ("f16_encode_ties_away_normal", "double q = nearbyint(ldexp(a, 10 - E));", "double q = round(ldexp(a, 10 - E));"),
    ("quant_divisor_128", "float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    ("quant_ties_away", "float r = rintf(t);", "float r = roundf(t);"),
    ("quant_truncates", "float r = rintf(t);", "float r = truncf(t);"),
    ("quant_reciprocal", "float t = xb[i] / d;", "float t = xb[i] * (1.0f / d);"),
    ("quant_uses_f16_scale", "float t = xb[i] / d;", "float t = xb[i] / (float)orc_f16_value(orc_f32_to_f16(d));"),
    ("quant_zero_block_scale", "dx[b] = 0;\n            continue;", "dx[b] = 0x3c00;\n            continue;"),
    ("quant_amax_signed", "float a = fabsf(xb[i]);", "float a = xb[i];"),
    ("isum_wrong_x_index", "(int32_t)qx[b * ORC_QBLOCK + i];\n            isum", "(int32_t)qx[i];\n            isum"),
    ("gemv_wrong_dx_index", "orc_f16_value(dw[n * nb + b]) * orc_f16_value(dx[b]);",
     "orc_f16_value(dw[n * nb + b]) * orc_f16_value(dx[0]);"),
    ("gemv_reversed_dw", "orc_f16_value(dw[n * nb + b])", "orc_f16_value(dw[n * nb + (nb - 1 - b)])"),
    ("gemv_unsigned_weights", "int32_t p = (int32_t)qw[n * K + b * ORC_QBLOCK + i]",
     "int32_t p = (int32_t)(uint8_t)qw[n * K + b * ORC_QBLOCK + i]"),
    ("gemv_residual_sign", "acc += (double)residual[n];\n            mag += fabs((double)residual[n]);\n        }\n        y[n] = acc;\n        S[n] = mag;\n    }\n}\n\n/* ---- bf16",
     "acc -= (double)residual[n];\n            mag += fabs((double)residual[n]);\n        }\n        y[n] = acc;\n        S[n] = mag;\n    }\n}\n\n/* ---- bf16"),
    ("gemv_magnitude_signed", "* (int32_t)qx[b * ORC_QBLOCK + i];\n                s += p;\n                sa += p < 0 ? -p : p;",
     "* (int32_t)qx[b * ORC_QBLOCK + i];\n                s += p;\n                sa += p;"),
    ("ptq1_magnitude_signed", "* (int32_t)qx[b * ORC_PTQ1_BLOCK + i];\n                s += p;\n                sa += p < 0 ? -p : p;",
     "* (int32_t)qx[b * ORC_PTQ1_BLOCK + i];\n                s += p;\n                sa += p;"),
    ("gemv_dropped_last_block", "for (int64_t b = 0; b < nb; ++b) {\n            int32_t s = 0, sa = 0;",
     "for (int64_t b = 0; b < nb - 1; ++b) {\n            int32_t s = 0, sa = 0;"),
    ("bf16_wrong_x_index", "orc_bf16_value(x[k]);", "orc_bf16_value(x[0]);"),
    ("bf16_reversed_row", "orc_bf16_value(w[n * K + k])", "orc_bf16_value(w[n * K + (K - 1 - k)])"),
    ("bf16_dropped_residual", "acc += (double)residual[n];\n            mag += fabs((double)residual[n]);\n        }\n        y[n] = acc;\n        S[n] = mag;\n    }\n}\n\n/* ---- f16",
     "mag += fabs((double)residual[n]);\n        }\n        y[n] = acc;\n        S[n] = mag;\n    }\n}\n\n/* ---- f16"),
    ("f16_dropped_residual", "acc += (double)residual[n];\n            mag += fabs((double)residual[n]);\n        }\n        y[n] = acc;\n        S[n] = mag;\n    }\n}\n\n/* ---- small-batch",
     "mag += fabs((double)residual[n]);\n        }\n        y[n] = acc;\n        S[n] = mag;\n    }\n}\n\n/* ---- small-batch"),
    ("batch_shared_dx", "qx + b * K, dx + b * nb,", "qx + b * K, dx,"),
    ("batch_shared_residual", "residual ? residual + b * N : NULL", "residual"),
    ("batch_shared_codes", "orc_q8_gemv(qw, dw, qx + b * K,", "orc_q8_gemv(qw, dw, qx,"),
    ("rmsnorm_no_mean", "sqrt(ss / (double)K + (double)eps)", "sqrt(ss + (double)eps)"),
    ("rmsnorm_no_gamma", "h[i] = t * gamma[i];", "h[i] = t;"),
    ("rmsnorm_eps_outside", "sqrt(ss / (double)K + (double)eps)", "sqrt(ss / (double)K) + (double)eps"),
    ("silu_sign", "exp(-g)", "exp(g)"),
    ("silu_swapped_halves", "g = (double)gu[i], u = (double)gu[K + i]", "g = (double)gu[K + i], u = (double)gu[i]"),
    ("f16_reversed_row", "orc_f16_value(w[n * K + k])", "orc_f16_value(w[n * K + (K - 1 - k)])"),
    ("f16_decoded_as_bf16", "double p = orc_f16_value(w[n * K + k]) * orc_f16_value(x[k]);",
     "double p = orc_bf16_value(w[n * K + k]) * orc_f16_value(x[k]);"),
    ("threads_f16_as_bf16", "orc_job p = {2, w, NULL, x, NULL, residual, 0, 0, K, y, S};",
     "orc_job p = {1, w, NULL, x, NULL, residual, 0, 0, K, y, S};"),
    ("threads_drop_row", "jobs[t].n1 = N * (t + 1) / nthreads;", "jobs[t].n1 = N * (t + 1) / nthreads - (t == 0);"),
    # PTQ1_0: packing, scale, rotation
    ("ptq1_digit_msb_first", "for (int k = 0; k < i % 5; ++k)", "for (int k = 0; k < 4 - i % 5; ++k)"),
    ("ptq1_trit_offset", "return v % 3 - 1;", "return v % 3;"),
    ("ptq1_six_per_byte", "int v = blk[i / 5];", "int v = blk[i / 6];"),
    ("ptq1_block_stride_26", "const uint8_t *blk = w + (n * nb + b) * ORC_PTQ1_BYTES;",
     "const uint8_t *blk = w + (n * nb + b) * ORC_PTQ1_TRIT_BYTES;"),
    ("ptq1_scale_ignored", "double scale = orc_f16_value(orc_ptq1_scale(blk)) * orc_f16_value(dx[b]);",
     "double scale = orc_f16_value(dx[b]);"),
    ("ptq1_scale_big_endian", "return (uint16_t)(blk[ORC_PTQ1_TRIT_BYTES] | (blk[ORC_PTQ1_TRIT_BYTES + 1] << 8));",
     "return (uint16_t)(blk[ORC_PTQ1_TRIT_BYTES + 1] | (blk[ORC_PTQ1_TRIT_BYTES] << 8));"),
    ("hadamard_sign_or", "acc += orc_parity((unsigned)(i & j)) ? -v : v;", "acc += orc_parity((unsigned)(i | j)) ? -v : v;"),
    ("hadamard_unnormalized", "out[b * ORC_PTQ1_BLOCK + i] = (float)(acc / norm);", "out[b * ORC_PTQ1_BLOCK + i] = (float)acc;"),
    ("hadamard_norm_128", "const double norm = sqrt((double)ORC_PTQ1_BLOCK);", "const double norm = (double)ORC_PTQ1_BLOCK;"),
    ("hadamard_f32_sum", "double acc = 0.0;\n            for (int j = 0; j < ORC_PTQ1_BLOCK; ++j) {",
     "float acc = 0.0f;\n            for (int j = 0; j < ORC_PTQ1_BLOCK; ++j) {"),
    ("ptq1_no_rotation", "    orc_hadamard128(x, K, rot);\n    orc_quantize_blocks(rot, K, ORC_PTQ1_BLOCK, qx, dx);",
     "    for (int64_t i = 0; i < K; ++i)\n        rot[i] = x[i];\n    orc_quantize_blocks(rot, K, ORC_PTQ1_BLOCK, qx, dx);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = oracle.build(force=True, out=str(tmp_path / "mutant.so"), src=str(path))
    o = oracle.Oracle(oracle.load(so))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
