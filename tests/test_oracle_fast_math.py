"""Pins for the oracle's fp16 error evaluation of the 4over6 search
("err_use_fast_math", flashinfer.quantization module page, "NVFP4 4over6
Recipes": the candidates' errors are scored in fp16 rather than in exact
fp32, so a close decision between the two candidates can come out reversed).

Reading pinned here: the input and the fp32 reconstruction are rounded to
fp16, then the difference, the square (MSE) and every pairwise sum are each
rounded to fp16 (nearest, ties to even, overflow to inf); amax/4 is kept only
when its error is strictly lower. The candidates' scales and codes come from
exact rational arithmetic (the same helper that pins the fp32 search), the
fp16 rounding from a bisection over the table of all finite fp16 values."""
import math
from fractions import Fraction

import numpy as np
import pytest

from test_oracle_ops import E2M1_SIGNED, E4M3_TORCH, exact_candidate

F16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)   # +finite, ascending


def nearest16(v: float) -> float:
    """v (exact in float64) -> nearest fp16 value, ties to the even code"""
    if math.isnan(v):
        return v
    a = abs(v)
    if a >= 65520.0:
        return math.copysign(math.inf, v)
    i = int(np.searchsorted(F16, a))
    if i < len(F16) and F16[i] == a:
        r = a
    else:
        lo, hi = F16[i - 1], F16[i]
        dl, dh = a - lo, hi - a
        r = lo if (dl < dh or (dl == dh and (i - 1) % 2 == 0)) else hi
    return math.copysign(r, v)


def fp16_error(x, s, codes, g, mode):
    # the fp32 reconstruction fp32(fp32(E4M3(s) * g) * e2m1), as float64
    dec = np.float32(E4M3_TORCH[s]) * np.float32(g)
    t = []
    for xi, c in zip(x, codes):
        deq = float(dec * np.float32(E2M1_SIGNED[c]))
        d = nearest16(nearest16(float(xi)) - nearest16(deq))
        t.append(nearest16(d * d) if mode == 0 else abs(d))
    while len(t) > 1:
        t = [nearest16(t[2 * j] + t[2 * j + 1]) for j in range(len(t) // 2)]
    return t[0]


def blocks(rng, n):
    out = []
    for k in range(n):
        kind = k % 5
        if kind == 0:
            x = rng.standard_normal(16) * np.exp(rng.uniform(-3, 3))
        elif kind == 1:
            x = rng.standard_t(3, 16)
        elif kind == 2:                                   # large: squares overflow fp16
            x = rng.standard_normal(16) * 3e3
        elif kind == 3:                                   # tiny: fp16 subnormals
            x = rng.standard_normal(16) * 1e-6
        else:                                             # grid-like, near ties
            x = E2M1_SIGNED[rng.integers(0, 16, 16)].astype(np.float64) * 0.75 + rng.normal(0, 0.02, 16)
        out.append(x.astype(np.float32))
    return out


@pytest.mark.parametrize("pow2_g", [True, False])
@pytest.mark.parametrize("mode", [0, 1])
def test_fp16_error_and_choice_vs_exact(orc, mode, pow2_g):
    """g a power of two: the reconstruction is exact in fp16 too; any other
    g: the fp32 reconstruction has more bits than fp16 keeps, so its rounding
    to fp16 shows."""
    rng = np.random.default_rng(90 + mode + 2 * pow2_g)
    rec = orc.four_over_six(mode, fast_math=True)
    checked = differs = deq_rounds = 0
    for x in blocks(rng, 1500):
        g = 2.0 ** int(rng.integers(-12, 1)) if pow2_g else float(np.float32(np.exp(rng.uniform(-8, 0))))
        s6, c6, _, m6 = exact_candidate(x, g, 6, 256, mode)
        s4, c4, _, m4 = exact_candidate(x, g, 4, 448, mode)
        if min(m6, m4) < Fraction(1, 10**5):
            continue                                      # too near an fp32 rounding boundary
        codes, s, e6, e4, chose4 = orc.quantize_block(x, g, rec)
        w6, w4 = fp16_error(x, s6, c6, g, mode), fp16_error(x, s4, c4, g, mode)
        assert (e6 == w6 or (math.isnan(e6) and math.isnan(w6))), (x, e6, w6)
        assert (e4 == w4 or (math.isnan(e4) and math.isnan(w4))), (x, e4, w4)
        want4 = bool(w4 < w6)
        assert bool(chose4) == want4
        assert s == (s4 if want4 else s6) and list(codes) == (c4 if want4 else c6)
        _, _, f6, f4, fchose = orc.quantize_block(x, g, orc.four_over_six(mode))
        differs += int(bool(fchose) != want4)
        dec = np.float32(E4M3_TORCH[s6]) * np.float32(g)
        deq = (dec * E2M1_SIGNED[np.array(c6)]).astype(np.float64)
        deq_rounds += int(np.any(deq.astype(np.float16).astype(np.float64) != deq))
        checked += 1
    assert checked > 1000
    assert differs > 0, "fp16 scoring never chose differently from fp32 scoring"
    if not pow2_g:
        assert deq_rounds > 100


def test_fp16_overflow_never_wins(orc):
    """Squares past 65504 are inf in fp16 and inf < inf is false: when both
    candidates' fp16 errors overflow, amax/6 is kept, even where fp32 scoring
    prefers amax/4."""
    rng = np.random.default_rng(95)
    both_inf = fp32_picks4 = 0
    for _ in range(400):
        x = (rng.standard_normal(16) * 4e3).astype(np.float32)
        _, _, e6, e4, chose4 = orc.quantize_block(x, 16.0, orc.four_over_six(0, fast_math=True))
        if math.isinf(e6) and math.isinf(e4):
            both_inf += 1
            assert not chose4
            fp32_picks4 += int(orc.quantize_block(x, 16.0, orc.four_over_six(0))[4])
    assert both_inf > 50 and fp32_picks4 > 0
