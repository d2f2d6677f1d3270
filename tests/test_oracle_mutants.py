"""Mutation tests of the oracle's pins (CPU only).

Each mutant below is a plausible mistake in ``oracle/c128_oracle.c``: a wrong sign, index,
offset, rounding mode, constant or step order.  The test builds the mutated source with gcc into
a temporary library, points the oracle at it (``DSV4_ORACLE_LIB``) and runs the pin that guards
that step, in a fresh interpreter; the pin must fail, and it must pass on an unmutated build
loaded the same way.  So every pin here is shown to tie its step to something other than the
oracle's own code: a mistake there does not go unnoticed.

Mutants that would only change results outside the oracle's domain (clamps that the UE8M0
exponent already makes unreachable, say) are not listed: they are not mistakes.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "c128_oracle.c")
PINS = "tests/test_oracle_pins.py"
PINS_C4 = "tests/test_oracle_pins_c4.py"
PINS_IDX = "tests/test_oracle_pins_indexer.py"
PINS_FP4 = "tests/test_oracle_pins_mxfp4.py"


def M(name, edits, catch):
    """``edits``: (old, new) or (old, new, k) replacing the k-th occurrence of ``old`` (which
    must otherwise be unique); ``catch``: pin node ids, any of which must fail."""
    return {"name": name, "edits": edits, "catch": catch}


MUTANTS = [
    # gate
    M("gate on the first position of a window",
      [("(pos + 1) % CR != 0) return ST_INACTIVE;", "pos % CR != 0) return ST_INACTIVE;")],
      [f"{PINS}::test_gate_brute_force"]),
    M("gate ignores a negative state slot",
      [("if (slot < 0 || pos < 0 ||", "if (pos < 0 ||")],
      [f"{PINS}::test_gate_brute_force"]),
    # window addressing
    M("window starts one row early",
      [("int64_t start = pos - nrows + 1;", "int64_t start = pos - nrows;")],
      [f"{PINS}::test_one_hot_scores_select_each_window_row"]),
    M("block-table column from the window row instead of the position",
      [("a->block_table[req * a->bt_stride + q / a->state_bs]",
        "a->block_table[req * a->bt_stride + i / a->state_bs]")],
      [f"{PINS}::test_one_hot_scores_select_each_window_row"]),
    # pool
    M("softmax over the kv half",
      [("double s = row[i][SW + j];", "double s = row[i][j];"),
       ("exp((double)row[i][SW + j] - M)", "exp((double)row[i][j] - M)")],
      [f"{PINS}::test_pool_matches_library_softmax_on_tiny_window"]),
    M("pooled value taken from the scores",
      [("num += p * (double)row[i][j];", "num += p * (double)row[i][SW + j];")],
      [f"{PINS}::test_pool_matches_library_softmax_on_tiny_window"]),
    M("weights not normalised",
      [("double p = w[i] / L;", "double p = w[i];")],
      [f"{PINS}::test_pool_uniform_scores_give_the_mean"]),
    # RMSNorm
    M("mean square over the 448 nope dims",
      [("sqrt(ss / H + a->eps)", "sqrt(ss / NOPE + a->eps)")],
      [f"{PINS}::test_rmsnorm_closed_form"]),
    M("eps added outside the square root",
      [("1.0 / sqrt(ss / H + a->eps)", "1.0 / (sqrt(ss / H) + a->eps)")],
      [f"{PINS}::test_rmsnorm_weight_and_eps"]),
    M("RMSNorm divides by the mean square, not its root",
      [("double rrms = 1.0 / sqrt(ss / H + a->eps);", "double rrms = 1.0 / (ss / H + a->eps);")],
      [f"{PINS}::test_record_invariant_under_power_of_two_kv_scaling"]),
    M("RMSNorm weight not applied",
      [("n[j] = c[j] * rrms * (double)a->rms_w[j];", "n[j] = c[j] * rrms;")],
      [f"{PINS}::test_rmsnorm_weight_and_eps"]),
    # FP8 UE8M0 quantisation
    M("no bf16 round trip before the absmax",
      [("for (int j = 0; j < NOPE; ++j) u[j] = oracle_bf16_value(oracle_bf16_bits((double)(float)n[j]));",
        "for (int j = 0; j < NOPE; ++j) u[j] = (double)(float)n[j];")],
      [f"{PINS}::test_quant_rounds_through_bf16_first"]),
    M("absmax without the absolute value",
      [("    for (int j = g * QBLOCK; j < (g + 1) * QBLOCK; ++j)\n      if (fabs(u[j]) > amax) amax = fabs(u[j]);",
        "    for (int j = g * QBLOCK; j < (g + 1) * QBLOCK; ++j)\n      if (u[j] > amax) amax = u[j];")],
      [f"{PINS}::test_quant_invariants_on_random_windows"]),
    M("floor(log2) instead of ceil(log2)",
      [("return (f == 0.5) ? k - 1 : k;", "return k - 1;")],
      [f"{PINS}::test_ue8m0_exponent_exact_for_every_bf16_absmax"]),
    M("absmax floor 1e-6 instead of 1e-4",
      [("double floor_ = (double)(float)1e-4;", "double floor_ = (double)(float)1e-6;")],
      [f"{PINS}::test_zero_window_record"]),
    M("E4M3FNUZ largest value (240) instead of E4M3FN's 448",
      [("double inv = (double)(float)(1.0 / FP8_MAX);", "double inv = (double)(float)(1.0 / 240.0);")],
      [f"{PINS}::test_ue8m0_exponent_exact_for_every_bf16_absmax"]),
    M("E4M3 mantissa truncated",
      [("double m = rint((ldexp(a, -E) - 1.0) * 8.0);", "double m = floor((ldexp(a, -E) - 1.0) * 8.0);")],
      [f"{PINS}::test_e4m3_exhaustive_against_nearest_code_search"]),
    M("E4M3 subnormal step 2^-10",
      [("code = (unsigned)rint(ldexp(a, 9));", "code = (unsigned)rint(ldexp(a, 10));")],
      [f"{PINS}::test_e4m3_ocp_reference_points"]),
    M("scale byte biased by 128",
      [("int byte = e + 127;", "int byte = e + 128;")],
      [f"{PINS}::test_handworked_golden_record"]),
    M("pad scale byte left unwritten",
      [("scales[NQ] = 0;", ";")],
      [f"{PINS}::test_insert_byte_offsets"]),
    # RoPE
    M("rotation by minus the angle",
      [("oracle_bf16_bits(x * C - y * S);", "oracle_bf16_bits(x * C + y * S);"),
       ("oracle_bf16_bits(y * C + x * S);", "oracle_bf16_bits(y * C - x * S);")],
      [f"{PINS}::test_rope_rotation_against_complex_multiply"]),
    M("NeoX halves instead of GPT-J pairs",
      [("double x = n[NOPE + 2 * m], y = n[NOPE + 2 * m + 1];",
        "double x = n[NOPE + m], y = n[NOPE + m + HALF_ROPE];")],
      [f"{PINS}::test_rope_rotation_against_complex_multiply"]),
    M("angle row of the token's own position",
      [("int64_t P = (pos / CR) * CR;", "int64_t P = pos;")],
      [f"{PINS}::test_rope_identity_at_position_zero"]),
    M("cos/sin table read as interleaved pairs",
      [("double C = cs[m], S = cs[HALF_ROPE + m];", "double C = cs[2 * m], S = cs[2 * m + 1];", 2)],
      [f"{PINS}::test_rope_rotation_against_complex_multiply"]),
    # insert
    M("records and scales interleaved per token",
      [("uint8_t* data = blockp + koff * RECORD;", "uint8_t* data = blockp + koff * (RECORD + SCALE_DIM);"),
       ("uint8_t* scales = blockp + a->kv_bs * RECORD + koff * SCALE_DIM;",
        "uint8_t* scales = blockp + koff * (RECORD + SCALE_DIM) + RECORD;")],
      [f"{PINS}::test_insert_byte_offsets"]),
    # bf16
    M("bf16 by truncation",
      [("r = ldexp(rint(ldexp(a, -q)), q);", "r = ldexp(trunc(ldexp(a, -q)), q);")],
      [f"{PINS}::test_bf16_matches_torch_cast_on_structured_fp32"]),
    M("bf16 without the subnormal spacing",
      [("if (q < -133) q = -133;", ";")],
      [f"{PINS}::test_bf16_matches_torch_cast_on_structured_fp32"]),
    # C4
    M("C4 head offsets of the two halves swapped",
      [("int64_t head_offset = (i >= CR) ? a->head : 0;", "int64_t head_offset = (i < CR) ? a->head : 0;")],
      [f"{PINS_C4}::test_c4_one_hot_selects_each_row_and_half"]),
    M("C4 window without the previous window's rows",
      [("int64_t nrows = (1 + a->overlap) * CR;", "int64_t nrows = CR;")],
      [f"{PINS_C4}::test_c4_one_hot_selects_each_row_and_half"]),
    M("C4 first window drops position 0",
      [("valid[i] = q >= 0;", "valid[i] = q > 0;")],
      [f"{PINS_C4}::test_c4_one_hot_selects_each_row_and_half"]),
    # indexer FP8
    M("indexer quantises before rotating",
      [("    u[j] = oracle_bf16_value(oracle_bf16_bits((double)(float)r[j]));\n    if (fabs(u[j]) > amax)",
        "    u[j] = oracle_bf16_value(oracle_bf16_bits((double)(float)n[j]));\n    if (fabs(u[j]) > amax)")],
      [f"{PINS_IDX}::test_indexer_rotates_before_quantising"]),
    M("indexer scale stored as its inverse",
      [("float sv = (float)ldexp(1.0, e);", "float sv = (float)ldexp(1.0, -e);")],
      [f"{PINS_IDX}::test_indexer_quant_invariants"]),
    M("indexer angle row of the token's own position",
      [("int64_t P = (pos / a->cr) * a->cr;", "int64_t P = pos;", 0)],
      [f"{PINS_IDX}::test_indexer_rope_against_complex_multiply"]),
    M("indexer rotation by minus the angle",
      [("r[IDX_NOPE + 2 * m] = x * C - y * S;", "r[IDX_NOPE + 2 * m] = x * C + y * S;", 0),
       ("r[IDX_NOPE + 2 * m + 1] = y * C + x * S;", "r[IDX_NOPE + 2 * m + 1] = y * C - x * S;", 0)],
      [f"{PINS_IDX}::test_indexer_rope_against_complex_multiply"]),
    M("indexer records and scales interleaved per token",
      [("uint8_t* data = blockp + koff * IDX_RECORD;",
        "uint8_t* data = blockp + koff * (IDX_RECORD + IDX_SCALE);"),
       ("uint8_t* scale = blockp + a->kv_bs * IDX_RECORD + koff * IDX_SCALE;",
        "uint8_t* scale = blockp + koff * (IDX_RECORD + IDX_SCALE) + IDX_RECORD;")],
      [f"{PINS_IDX}::test_indexer_insert_byte_offsets"]),
    # indexer MXFP4
    M("MXFP4 one exponent for all 128 dims",
      [("    for (int j = g * FP4_BLOCK; j < (g + 1) * FP4_BLOCK; ++j)\n      if (fabs(u[j]) > amax)",
        "    for (int j = 0; j < IDX_HEAD; ++j)\n      if (fabs(u[j]) > amax)")],
      [f"{PINS_FP4}::test_mxfp4_one_hot_record"]),
    M("MXFP4 odd dim in the low nibble",
      [("data[j / 2] = (uint8_t)(lo | (hi << 4));", "data[j / 2] = (uint8_t)(hi | (lo << 4));")],
      [f"{PINS_FP4}::test_mxfp4_one_hot_record"]),
    M("E2M1 mantissa truncated",
      [("double m = rint((ldexp(a, -E) - 1.0) * 2.0);", "double m = floor((ldexp(a, -E) - 1.0) * 2.0);")],
      [f"{PINS_FP4}::test_e2m1_exhaustive_against_nearest_code_search"]),
    M("E2M1 without saturation at 6",
      [("code = E > 2 ? 7u : (((unsigned)(E + 1) << 1) | (unsigned)m);",
        "code = (((unsigned)(E + 1) << 1) | (unsigned)m) & 7u;")],
      [f"{PINS_FP4}::test_e2m1_exhaustive_against_nearest_code_search"]),
    M("MXFP4 exponent from absmax / 4",
      [("double inv = (double)(float)(1.0 / FP4_MAX);", "double inv = (double)(float)(1.0 / 4.0);")],
      [f"{PINS_FP4}::test_mxfp4_exponent_exact_for_every_bf16_absmax"]),
    M("MXFP4 scale byte biased by 128",
      [("scales[g] = (uint8_t)(e + 127);", "scales[g] = (uint8_t)(e + 128);")],
      [f"{PINS_FP4}::test_mxfp4_one_hot_record"]),
]


def apply(src: str, mutant) -> str:
    for edit in mutant["edits"]:
        old, new = edit[0], edit[1]
        n = src.count(old)
        if len(edit) == 2:
            assert n == 1, f"{mutant['name']}: {old!r} occurs {n} times"
            src = src.replace(old, new)
        else:
            k = edit[2]
            assert n > k, f"{mutant['name']}: {old!r} occurs {n} times"
            i = -1
            for _ in range(k + 1):
                i = src.index(old, i + 1)
            src = src[:i] + new + src[i + len(old):]
    return src


def build(src: str, d: str) -> str:
    c, so = os.path.join(d, "oracle.c"), os.path.join(d, "oracle.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
                           "-fPIC", "-shared", "-o", so, c, "-lm", "-lpthread"])
    return so


def run_pins(so: str, nodes) -> subprocess.CompletedProcess:
    env = dict(os.environ, DSV4_ORACLE_LIB=so)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                           "-m", "not gpu", *nodes], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=600)


def outcome(proc) -> str:
    tail = proc.stdout.strip().splitlines()[-1] if proc.stdout.strip() else ""
    if proc.returncode == 0:
        return "passed"
    if re.search(r"\d+ failed", tail) and "error" not in tail:
        return "failed"
    return f"broken (exit {proc.returncode}): {tail}"


def test_every_mutant_is_caught_by_its_pin():
    src = open(SRC).read()
    with tempfile.TemporaryDirectory() as tmp:
        base_dir = os.path.join(tmp, "base")
        os.mkdir(base_dir)
        base = build(src, base_dir)
        catchers = sorted({n for m in MUTANTS for n in m["catch"]})
        proc = run_pins(base, catchers)
        assert outcome(proc) == "passed", proc.stdout[-2000:]

        def one(i_m):
            i, m = i_m
            d = os.path.join(tmp, f"m{i}")
            os.mkdir(d)
            so = build(apply(src, m), d)
            return m["name"], outcome(run_pins(so, m["catch"]))

        with cf.ThreadPoolExecutor(4) as ex:
            results = list(ex.map(one, enumerate(MUTANTS)))
    missed = [(name, res) for name, res in results if res != "failed"]
    assert not missed, "mutants not caught by their pins: " + "; ".join(
        f"{name}: {res}" for name, res in missed)


@pytest.mark.parametrize("m", MUTANTS, ids=[m["name"] for m in MUTANTS])
def test_mutant_applies_to_the_source(m):
    """Each mutation still finds its text in the oracle (a refactor of the oracle must update
    the mutants rather than silently skip them)."""
    src = open(SRC).read()
    assert apply(src, m) != src
