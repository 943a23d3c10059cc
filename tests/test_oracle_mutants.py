"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies ``oracle/ar_oracle.c`` with one plausible mistake written in
(a dropped rank, a reversed order, a wrong tie rule, an off-by-one shift, a lost
sign, ...), builds it into a temporary directory and runs the cheap pins
against it in a child process (a planted mistake may also crash, e.g. by
reading an inactive rank's NULL pointer; a crash counts as caught).  The real
oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle
import oracle_checks as oc

SRC = os.path.join(os.path.dirname(oracle.__file__), "ar_oracle.c")

# (name, [(exact text in ar_oracle.c, replacement), ...])
MUTANTS = [
    ("drop_last_rank", [("for (int r = 1; r < R; ++r)", "for (int r = 1; r < R - 1; ++r)")]),
    ("fold_from_plus_zero", [
        ("float acc = orc_wire_value(srcs[0], i, src_type, wire_type);", "float acc = 0.0f;"),
        ("for (int r = 1; r < R; ++r)", "for (int r = 0; r < R; ++r)")]),
    ("reverse_rank_order", [
        ("float acc = orc_wire_value(srcs[0], i, src_type, wire_type);",
         "float acc = orc_wire_value(srcs[R - 1], i, src_type, wire_type);"),
        ("const float w = orc_wire_value(srcs[r], i, src_type, wire_type);",
         "const float w = orc_wire_value(srcs[R - 1 - r], i, src_type, wire_type);")]),
    ("local_partial_not_rounded", [
        ("float acc = orc_wire_value(srcs[0], i, src_type, wire_type);",
         "float acc = src_type == ORC_F32 ? ((const float *)srcs[0])[i]"
         " : orc_wire_value(srcs[0], i, src_type, wire_type);")]),
    ("accumulate_in_double", [
        ("float acc = orc_wire_value", "double acc = orc_wire_value")]),
    ("bf16_truncates", [
        ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) {", "if (0) {")]),
    ("bf16_ties_away", [
        ("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)")]),
    ("bf16_nan_to_inf", [
        ("if (exp_field == 0x7F800000u && frac != 0) {", "if (0) {")]),
    ("f16_ties_away", [
        ("(dropped == 0x1000u && (kept & 1u))", "(dropped == 0x1000u)")]),
    ("f16_subnormal_shift_off_by_one", [("int s = -(E + 1);", "int s = -E;")]),
    ("f16_overflow_threshold", [("if (E > 15) {", "if (E > 16) {")]),
    ("f16_lost_sign", [("const uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);",
                        "const uint16_t sign = 0;")]),
    ("f16_subnormal_ties_away", [
        ("(dropped == half && (kept & 1ull))", "(dropped == half)")]),
    ("widen_f16_bias", [("((uint32_t)(e + 112) << 23)", "((uint32_t)(e + 111) << 23)")]),
    ("widen_f16_subnormal_as_zero", [("if (m == 0) {\n            return sign;", "if (1) {\n            return sign;")]),
    ("broadcast_only_first", [("for (int d = 0; d < n_dst; ++d)", "for (int d = 0; d < 1; ++d)")]),
    ("inactive_rank_skipped", [
        ("const float w = orc_wire_value(srcs[r], i, src_type, wire_type);\n            acc = acc + w;",
         "if (srcs[r] == NULL) continue;\n            const float w = orc_wire_value(srcs[r], i, src_type, wire_type);\n            acc = acc + w;")]),
    ("inactive_rank_as_minus_zero", [("        return 0.0f;                                      /* inactive rank */",
                                      "        return -0.0f;")]),
    ("add_keeps_ftz", [("_mm_setcsr(saved & ~((1u << 15) | (1u << 6)));",
                        "_mm_setcsr(saved | (1u << 15) | (1u << 6));")]),
    ("residual_skipped", [("if (residual != NULL) {", "if (0) {")]),
    ("residual_before_ranks", [
        ("float acc = orc_wire_value(srcs[0], i, src_type, wire_type);",
         "float acc = orc_wire_value(srcs[0], i, src_type, wire_type);\n"
         "        if (residual != NULL) acc = acc + orc_dst_value(residual, i % residual_len, dst_type);"),
        ("acc = acc + orc_dst_value(residual, i % residual_len, dst_type);\n            if",
         "(void)0;\n            if")]),
    ("residual_rounded_to_wire", [
        ("acc = acc + orc_dst_value(residual, i % residual_len, dst_type);\n            if",
         "acc = acc + orc_to_dst(orc_dst_value(residual, i % residual_len, dst_type), wire_type);\n            if")]),
    ("residual_row_index_swapped", [
        ("orc_dst_value(residual, i % residual_len, dst_type)",
         "orc_dst_value(residual, residual_len == n ? i : (i / residual_len) % residual_len, dst_type)")]),
    ("narrow_rounds_once_at_end", [
        ("            if (dst_type != ORC_F32) acc = orc_to_dst(acc, dst_type);\n        }\n        if (residual",
         "        }\n        if (dst_type != ORC_F32) acc = orc_to_dst(acc, dst_type);\n        if (residual")]),
    ("rows_src_index_uses_dst_stride", [("const size_t si = i * src_stride + j;",
                                        "const size_t si = i * dst_stride + j;")]),
    ("rows_broadcast_residual_advances", [("orc_dst_value(residual, i * res_stride + j, dst_type)",
                                          "orc_dst_value(residual, i * (res_stride ? res_stride : cols) + j, dst_type)")]),
    ("rows_writes_between_rows", [("orc_store_dst(dst[d], i * dst_stride + j, acc, dst_type);",
                                   "orc_store_dst(dst[d], i * dst_stride + j, acc, dst_type);\n"
                                   "                if (j + 1 == cols && cols < dst_stride && i + 1 < rows) "
                                   "orc_store_dst(dst[d], i * dst_stride + cols, acc, dst_type);")]),
    ("narrow_store_wrong_format", [
        ("dst_type == ORC_BF16 ? orc_round_bf16(bits) : orc_round_f16(bits)",
         "dst_type == ORC_BF16 ? orc_round_f16(bits) : orc_round_bf16(bits)")]),
]


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, edits):
    text = open(SRC).read()
    for old, new in edits:
        assert text.count(old) >= 1, f"anchor for {name} not found in the oracle source: {old!r}"
        text = text.replace(old, new)
    src = tmp_path / f"mutant_{name}.c"
    src.write_text(text)
    so = tmp_path / f"libmutant_{name}.so"
    oracle.build(str(src), str(so))
    here = os.path.dirname(os.path.abspath(__file__))
    code = (
        "import sys\n"
        f"sys.path[:0] = [{here!r}, {os.path.dirname(here)!r}]\n"
        "import oracle, oracle_checks as oc\n"
        f"lib = oracle.load({str(so)!r})\n"
        "caught = []\n"
        "for name, check in oc.cheap_checks():\n"
        "    try:\n"
        "        check(lib)\n"
        "    except AssertionError:\n"
        "        caught.append(name)\n"
        "print('caught:', caught)\n"
        "sys.exit(3 if caught else 0)\n"
    )
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    # 3: a pin's assertion failed; < 0: the planted mistake crashed the process.
    # Anything else (0, or a Python error outside the pins) is not a catch.
    assert res.returncode == 3 or res.returncode < 0, \
        f"planted mistake {name!r} not caught (rc={res.returncode}): {res.stdout}{res.stderr[-2000:]}"


def test_real_oracle_passes_cheap_checks(orc):
    for _, check in oc.cheap_checks():
        check(orc)
