"""Planted mistakes in the oracle.

Each mutant below is one plausible slip in ``oracle/kvfp4_oracle.c``: a
flipped tie rule, a dropped term or sign, a wrong index, operands multiplied
in another order. The mutated source is compiled into a scratch library and
the oracle's own pin tests run against it in a fresh process (the oracle
module loads the library named by ``KVFP4_ORACLE_LIB``); at least one pin
must fail. An unmutated copy built the same way must pass the same pins, so
a failure is the mutant's doing. This checks that the pins pin the oracle;
the pins themselves check the oracle against the pages.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvfp4_oracle.c")

# every pin file except the two slow exhaustive comparisons, which the
# mutants that need them name explicitly
PINS = ["tests/test_oracle_codecs.py", "tests/test_oracle_readings.py", "tests/test_oracle_ops.py",
        "tests/test_oracle_contiguous.py", "tests/test_oracle_attention.py",
        "-k", "not random_blocks_vs_exact and not fp16_error_and_choice_vs_exact"]
FAST_MATH_PINS = ["tests/test_oracle_fast_math.py"]

# (name, text in the oracle source, replacement, pin tests to run)
MUTANTS = [
    # E2M1 encode: ties go to the odd code
    ("e2m1_ties_to_odd", "if (d < best_d || (d == best_d && (k & 1) == 0)) {",
     "if (d < best_d || (d == best_d && (k & 1) == 1)) {", PINS),
    # E2M1 subnormal code 1 decoded as 1 instead of 0.5
    ("e2m1_subnormal_value", "return 0.5 * m;", "return 1.0 * m;", PINS),
    # E2M1 encode drops the sign bit
    ("e2m1_sign_dropped", "    return (signbit(v) ? 8 : 0) | best;", "    return best;", PINS),
    # E4M3 encode: ties go to the odd code
    ("e4m3_ties_to_odd", "if (d < best_d || (d == best_d && (c & 1) == 0)) {",
     "if (d < best_d || (d == best_d && (c & 1) == 1)) {", PINS),
    # E4M3 subnormal spacing 2^-10 instead of 2^-9
    ("e4m3_subnormal_spacing", "v = m * ldexp(1.0, -9);", "v = m * ldexp(1.0, -10);", PINS),
    # E4M3 exponent bias 8 instead of 7
    ("e4m3_bias", "v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);", "v = (1.0 + m / 8.0) * ldexp(1.0, e - 8);", PINS),
    # block scale not clamped at the recipe maximum
    ("scale_clamp_dropped", "float x = sf < e4m3_max ? sf : e4m3_max;", "float x = sf;", PINS),
    # block scale amax / C without the global scale
    ("scale_ignores_global", "float t = C * g;", "float t = C;", PINS),
    # elements divided by the decode factor instead of multiplied by its fp32 reciprocal
    ("encode_divides", "float v = x[i] * inv;", "float v = x[i] / dec;", PINS),
    # 4over6: a tie picks the amax/4 candidate
    ("four_over_six_tie_to_amax4", "int take4 = e4 < e6;", "int take4 = e4 <= e6;", PINS),
    # 4over6: the amax/4 candidate clamped at the recipe maximum too
    ("four_over_six_amax4_clamp", "quantize_candidate(x, amax, g, 4.0f, 448.0f, c4, &d4);",
     "quantize_candidate(x, amax, g, 4.0f, e4m3_max, c4, &d4);", PINS),
    # 4over6: MSE and MAE swapped
    ("mse_mae_swapped", "t[i] = (err_mode == 0) ? d * d : fabsf(d);",
     "t[i] = (err_mode == 1) ? d * d : fabsf(d);", PINS),
    # 4over6: the fp32 error summed left to right instead of as a balanced tree
    ("error_sum_sequential",
     "    for (int w = 16; w > 1; w /= 2)\n        for (int j = 0; j < w / 2; j++)\n"
     "            t[j] = t[2 * j] + t[2 * j + 1];\n    return t[0];",
     "    for (int i = 1; i < 16; i++)\n        t[0] += t[i];\n    return t[0];", PINS),
    # fp16 error: the difference taken in double, not rounded to fp16
    ("fast_math_unrounded_difference",
     "double d = f16_round(f16_round((double)x[i]) - f16_round((double)deq));",
     "double d = (double)x[i] - (double)deq;", FAST_MATH_PINS),
    # global scale amax / (4 e4m3_max)
    ("global_scale_divisor", "float denom = 6.0f * e4m3_max;", "float denom = 4.0f * e4m3_max;", PINS),
    # 16-bit rounding: ties away from zero
    ("half_rounding_ties_away", "if (r > 0.5 || (r == 0.5 && fmod(n, 2.0) != 0.0))", "if (r >= 0.5)", PINS),
    # append: odd element in the low nibble
    ("append_nibbles_swapped", "drow[blk * 8 + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));",
     "drow[blk * 8 + j] = (uint8_t)(codes[2 * j + 1] | (codes[2 * j] << 4));", PINS),
    # NHD and HND row orders swapped
    ("layouts_swapped", "return c->layout == 0 ? slot * c->num_heads + h : h * c->page_size + slot;",
     "return c->layout == 1 ? slot * c->num_heads + h : h * c->page_size + slot;", PINS),
    # append: page list of request b taken from the start of kv_indices
    ("append_ignores_indptr", "int64_t page = a->indices[a->indptr[b] + p / ps];",
     "int64_t page = a->indices[p / ps];", PINS),
    # dequant: code times global scale first, then the block scale
    ("dequant_multiply_order", "                        float y = dec * (float)orc_e2m1_value(code);",
     "                        float y = (float)orc_e4m3_value(s) * ((float)orc_e2m1_value(code) * g);\n"
     "                        (void)dec;", PINS),
    # dequant: odd element read from the low nibble
    ("dequant_nibbles_swapped",
     "int code = (e & 1) ? (byte >> 4) : (byte & 15);\n                        uint8_t s = sf[row * (D / 16) + e / 16];",
     "int code = (e & 1) ? (byte & 15) : (byte >> 4);\n                        uint8_t s = sf[row * (D / 16) + e / 16];",
     PINS),
    # dequant: positions past the sequence length zeroed instead of left untouched
    ("dequant_clears_tail",
     "        int64_t len = a->seq_lens[b] < T ? a->seq_lens[b] : T;\n",
     "        int64_t len = a->seq_lens[b] < T ? a->seq_lens[b] : T;\n"
     "        for (int64_t t = len; t < T; t++)\n"
     "            for (int64_t i = 0; i < H * D; i++) {\n"
     "                a->out_k[(b * T + t) * H * D + i] = 0;\n"
     "                a->out_v[(b * T + t) * H * D + i] = 0;\n"
     "            }\n", PINS),
    # materialize: output page p instead of p + 1 (page 0 not kept for zeros)
    ("materialize_dst_off_by_one", "int64_t dst = (int64_t)a->indptr[b] + j + 1;",
     "int64_t dst = (int64_t)a->indptr[b] + j;", PINS),
    # materialize: V scales read linearly although interleaved
    ("materialize_ignores_interleave",
     "                                sidx = h * ps * nb + ((t / 4) * nb + e / 16) * 4 + t % 4;",
     "                                sidx = (h * ps + t) * nb + e / 16;", PINS),
    # materialize: V pages taken from the K table
    ("materialize_shared_table",
     "int64_t vpage = a->shared ? kpage : a->bt[b * a->bt_row_stride + a->bt_kv_stride + j];",
     "int64_t vpage = kpage;", PINS),
    # FP8 conversion drops the sign
    ("satfinite_sign_dropped", "    return sign | e4m3_nearest_magnitude(fabs((double)p));",
     "    return e4m3_nearest_magnitude(fabs((double)p));", PINS),
    # pool quantizer: V scales written linearly although interleaved
    ("pool_ignores_interleave", "                            sidx = h * ps * nb + ((t / 4) * nb + blk) * 4 + t % 4;",
     "                            sidx = row * nb + blk;", PINS),
    # contiguous dequant: code times global scale first
    ("contiguous_dequant_order",
     "a->out[r * a->cols + e] = orc_round_half(dec * (float)orc_e2m1_value(code), a->bf16);",
     "a->out[r * a->cols + e] = orc_round_half((float)orc_e4m3_value(a->scales[r * (a->cols / 16) + e / 16])"
     " * ((float)orc_e2m1_value(code) * a->g), a->bf16);\n            (void)dec;", PINS),
    # attention: query head qh mapped to kv head qh % H instead of qh / G
    ("attention_head_mapping", "int64_t h = qh / group;", "int64_t h = qh % H;", PINS),
    # attention: V decoded with the K global scale
    ("attention_v_global_scale", "o[e] += p * cache_value(c, 1, page, t % ps, h, e, a->gv);",
     "o[e] += p * cache_value(c, 1, page, t % ps, h, e, a->gk);", PINS),
    # attention: softmax scale dropped
    ("attention_scale_dropped", "s[t] = a->sm * dot;", "s[t] = dot;", PINS),
]


def _build(tmp, name, text):
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    d = os.path.join(tmp, name)
    os.makedirs(d, exist_ok=True)
    src = os.path.join(d, "kvfp4_oracle.c")
    with open(src, "w") as f:
        f.write(text)
    shutil.copy(os.path.join(ROOT, "oracle", "kvfp4_oracle.h"), d)
    lib = os.path.join(d, "libkvfp4_oracle.so")
    ob.build(src=src, lib=lib)
    return lib


def _run_pins(lib, pins):
    env = dict(os.environ, KVFP4_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + pins
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-3000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("oracle_mutants"))
    with open(SRC) as f:
        original = f.read()
    jobs = {"unmutated": (original, PINS + FAST_MATH_PINS)}
    for name, old, new, pins in MUTANTS:
        assert original.count(old) == 1, f"{name}: the mutated text must occur exactly once"
        jobs[name] = (original.replace(old, new), pins)
    libs = {name: _build(tmp, name, text) for name, (text, _) in jobs.items()}
    workers = max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        futs = {name: ex.submit(_run_pins, libs[name], pins) for name, (_, pins) in jobs.items()}
        return {name: fut.result() for name, fut in futs.items()}


def test_unmutated_copy_passes_the_pins(outcomes):
    rc, out = outcomes["unmutated"]
    assert rc == 0, out


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_catch_mutant(outcomes, name):
    rc, out = outcomes[name]
    # 1: a pin failed. 0 would mean every pin passed with the mistake in place.
    assert rc == 1, f"mutant {name} not caught (pytest exit {rc}):\n{out}"
