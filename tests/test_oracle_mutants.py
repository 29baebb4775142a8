"""The pins are strong enough: plant one plausible mistake at a time in a copy
of oracle.c (on the CPU), build it, and check that some pin rejects it."""
import os
import subprocess

import pytest

import oracle_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement): each a mistake someone could make
MUTANTS = [
    ("drop_last_k", "k < K; ++k)", "k + 1 < K; ++k)"),
    ("drop_first_k", "for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 1; k < K; ++k)"),
    ("sign_full_float", "acc[j] += aik * brow[j];", "acc[j] -= aik * brow[j];"),
    ("sign_full_int", "acc[j] += aik * brow[j];\n                    if", "acc[j] -= aik * brow[j];\n                    if"),
    ("transposed_b", "return b_col ? j * ldb + k : k * ldb + j;", "return b_col ? k * ldb + j : j * ldb + k;"),
    ("transposed_a", "return a_col ? k * lda + i : i * lda + k;", "return a_col ? i * lda + k : k * lda + i;"),
    ("b_ignores_col_flag", "return b_col ? j * ldb + k : k * ldb + j;", "return k * ldb + j;"),
    ("bias_by_row_int", "return bias ? v + bias[j] : v;", "return bias ? v + bias[i] : v;"),
    ("bias_by_row_float", "return bias ? v + (double)bias[j] : v;", "return bias ? v + (double)bias[i] : v;"),
    ("bias_dropped_float", "return bias ? v + (double)bias[j] : v;", "return v;"),
    ("bias_twice_int", "return bias ? v + bias[j] : v;", "return bias ? v + 2 * bias[j] : v;"),
    ("cin_ignored_float", "double v = cin ? elem_f(cin, cin_type, i * ldcin + j) : 0.0;", "double v = 0.0;"),
    ("cin_ignored_int", "int64_t v = cin ? (int64_t)cin[i * ldcin + j] : 0;", "int64_t v = 0;"),
    ("cin_transposed_float", "elem_f(cin, cin_type, i * ldcin + j)", "elem_f(cin, cin_type, j * ldcin + i)"),
    ("cin_transposed_int", "(int64_t)cin[i * ldcin + j]", "(int64_t)cin[j * ldcin + i]"),
    ("cin_ignores_ld", "acc[j] = init_f(cin, ldcin, cin_type, bf, i, j);", "acc[j] = init_f(cin, N, cin_type, bf, i, j);"),
    ("cin_wrong_type", "elem_f(cin, cin_type,", "elem_f(cin, OR_F16,"),
    ("cin_negated_int", "int64_t v = cin ? (int64_t)cin[i * ldcin + j] : 0;", "int64_t v = cin ? -(int64_t)cin[i * ldcin + j] : 0;"),
    ("conv_pad_sign", "const int64_t h = p * g->stride_h - g->pad_h + r * g->dil_h, w = q * g->stride_w - g->pad_w + s * g->dil_w;\n            if (h < 0",
     "const int64_t h = p * g->stride_h + g->pad_h + r * g->dil_h, w = q * g->stride_w - g->pad_w + s * g->dil_w;\n            if (h < 0"),
    ("conv_stride_ignored", "const int64_t h = p * g->stride_h - g->pad_h + r * g->dil_h, w = q * g->stride_w - g->pad_w + s * g->dil_w;\n            if (h < 0",
     "const int64_t h = p - g->pad_h + r * g->dil_h, w = q * g->stride_w - g->pad_w + s * g->dil_w;\n            if (h < 0"),
    ("conv_dilation_ignored", "const int64_t h = p * g->stride_h - g->pad_h + r * g->dil_h, w = q * g->stride_w - g->pad_w + s * g->dil_w;\n            if (h < 0",
     "const int64_t h = p * g->stride_h - g->pad_h + r * g->dil_h, w = q * g->stride_w - g->pad_w + s;\n            if (h < 0"),
    ("conv_filter_rs_swapped", "elem_f(f, dtype, ((k * R + r) * S + s) * C + c)", "elem_f(f, dtype, ((k * S + s) * R + r) * C + c)"),
    ("conv_edge_off_by_one", "if (h < 0 || h >= H || w < 0 || w >= W) continue;\n            for (int64_t c = 0; c < C; ++c)\n                acc += elem_f",
     "if (h < 0 || h > H || w < 0 || w >= W) continue;\n            for (int64_t c = 0; c < C; ++c)\n                acc += elem_f"),
    ("conv_bias_dropped_int", "int64_t acc = bias ? ((const int32_t*)bias)[k] : 0;", "int64_t acc = 0;"),
    ("conv_relu_missing_float", "*yf = relu ? relu_f(acc) : acc;", "*yf = acc;"),
    ("conv_int8_channel_offset", "(int64_t)x8[((n * H + h) * W + w) * C + c]", "(int64_t)x8[((n * H + h) * W + w) * C + c / 2]"),
    ("conv_entries_pixel_order", "p = mm[t] / g.Q % g.P, q = mm[t] % g.Q;", "p = mm[t] % g.P, q = mm[t] / g.P % g.Q;"),
    ("cin_overflow_unchecked", "            if (acc > INT32_MAX || acc < INT32_MIN) overflow = 1;\n            for (int64_t k = 0; k < K; ++k) {",
     "            for (int64_t k = 0; k < K; ++k) {"),
    ("relu_abs", "return x > 0.0 ? x : 0.0;", "return x > 0.0 ? x : -x;"),
    ("relu_int_missing", "if (relu && !(v > 0)) v = 0;", ""),
    ("f16_exponent_off_by_one", "expo - 25", "expo - 24"),
    ("f16_subnormal_scale", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("f16_no_implicit_bit", "(double)(1024 + frac)", "(double)(frac)"),
    ("bf16_frac_mask", "int frac = h & 0x7f;", "int frac = h & 0x3f;"),
    ("bf16_exponent_bias", "expo - 134", "expo - 133"),
    ("f16_sign_dropped", "return sign ? -v : v;\n}\n\ndouble oracle_decode_bf16", "return v;\n}\n\ndouble oracle_decode_bf16"),
    ("int8_as_uint8", "const int8_t* a8 = (const int8_t*)A;", "const uint8_t* a8 = (const uint8_t*)A;"),
    ("overflow_check_missing", "if (acc[j] > INT32_MAX || acc[j] < INT32_MIN) overflow = 1;", ""),
    ("entries_wrong_k_order_term", "elem_f(B, dtype, b_off(k, j, ldb, b_col));", "elem_f(B, dtype, b_off(k, j, ldb, !b_col));"),
]


def _build_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert old in text, f"mutant {name}: pattern not found in oracle.c"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
                    str(src), "-o", str(lib), "-lm"], check=True)
    return str(lib)


_RUNNER = """
import sys
sys.path.insert(0, {tests!r}); sys.path.insert(0, {root!r})
import oracle, oracle_pins as P
o = oracle.Oracle({lib!r})
failed = []
for pin in P.ALL_PINS:
    try:
        pin(o)
    except (AssertionError, OverflowError, oracle.OracleError):
        failed.append(pin.__name__)
print("FAILED_PINS", ",".join(failed))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    import sys
    lib = _build_mutant(tmp_path, name, old, new)
    code = _RUNNER.format(tests=os.path.join(ROOT, "tests"), root=ROOT, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return  # the planted mistake crashed the oracle (e.g. an out-of-bounds read): caught
    line = [l for l in r.stdout.splitlines() if l.startswith("FAILED_PINS")][-1]
    assert line.split(" ", 1)[1:] and line.split(" ", 1)[1].strip(), f"no pin rejects the planted mistake {name}"
