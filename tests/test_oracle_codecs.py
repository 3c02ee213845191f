"""Pins for the oracle's number formats, checked against things other than
the oracle: the grid and constants the pages state (tests/golden), exact
rational brute force, and torch's own float8_e4m3fn / bfloat16 / float16
casts (library routines written independently of this project)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32(x):
    return float(np.float32(x))


# --------------------------------------------------------------------------- E2M1
def test_e2m1_values_match_grid(orc):
    grid = _golden("e2m1_grid.json")["magnitudes"]
    for k in range(8):
        assert orc.e2m1_value(k) == grid[k]
        neg = orc.e2m1_value(8 | k)
        assert neg == -grid[k]
        assert math.copysign(1.0, neg) == -1.0          # 0x8 is -0
    assert max(abs(orc.e2m1_value(c)) for c in range(16)) == _golden("e2m1_grid.json")["largest"]


def test_e2m1_all_codes_round_trip(orc):
    vals = np.array([orc.e2m1_value(c) for c in range(16)], np.float32)
    assert list(orc.e2m1_encode(vals)) == list(range(16))


def _e2m1_exact_nearest(x: float, grid) -> int:
    """Brute force in exact rationals: nearest grid magnitude, ties to the
    even code, saturating; sign from the sign bit."""
    a = abs(Fraction(x))
    dists = [abs(a - Fraction(g)) for g in grid]
    best = min(dists)
    ks = [k for k, d in enumerate(dists) if d == best]
    k = ks[0] if len(ks) == 1 else [k for k in ks if k % 2 == 0][0]
    return (8 if math.copysign(1.0, x) < 0 else 0) | k


def test_e2m1_encode_vs_exact_brute_force(orc):
    grid = _golden("e2m1_grid.json")["magnitudes"]
    rng = np.random.default_rng(7)
    mids = [(grid[i] + grid[i + 1]) / 2 for i in range(7)]
    pts = []
    for m in mids + grid:
        f = np.float32(m)
        pts += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(100))]
    pts += list(rng.uniform(-8, 8, 4000).astype(np.float32))
    pts += list((rng.standard_normal(2000) * 100).astype(np.float32))
    pts += [np.float32(v) for v in (0.0, -0.0, 1e-40, -1e-40, 1e30, -1e30, 6.0, 7.0, 5.0, -5.0000005)]
    x = np.array(pts, np.float32)
    x = np.concatenate([x, -x])
    got = orc.e2m1_encode(x)
    want = np.array([_e2m1_exact_nearest(float(v), grid) for v in x], np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e2m1_ties_go_to_even_code(orc):
    # 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2.0, 2.5->2.0, 3.5->4.0, 5->4.0
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert list(orc.e2m1_encode(x)) == [0, 2, 2, 4, 4, 6, 6]


# --------------------------------------------------------------------------- E4M3
def test_e4m3_decode_matches_torch_for_all_bytes(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for b in range(256):
        v = orc.e4m3_value(b)
        if b in (0x7F, 0xFF):
            assert math.isnan(v) and math.isnan(ref[b])
        else:
            assert v == float(ref[b]), hex(b)
            assert math.copysign(1.0, v) == math.copysign(1.0, float(ref[b]))


def test_e4m3_golden_points(orc):
    pts = _golden("e4m3_points.json")["points"]
    x = np.array([p[0] for p in pts], np.float32)
    want = [p[1] for p in pts]
    assert list(orc.e4m3_encode_satfinite(x)) == want
    assert list(torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()) == want


def test_e4m3_encode_matches_torch_below_saturation(orc):
    rng = np.random.default_rng(11)
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    finite = np.sort(np.unique(np.abs(vals[np.isfinite(vals)])))
    mids = (finite[1:] + finite[:-1]) / 2
    pts = np.concatenate([finite, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                          np.exp(rng.uniform(np.log(1e-6), np.log(463.0), 20000)),
                          rng.uniform(0, 463.9, 5000), [448.0, 455.99, 463.99]]).astype(np.float32)
    pts = pts[pts < 464.0]
    pts = np.concatenate([pts, -pts])
    got = orc.e4m3_encode_satfinite(pts)
    want = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(pts[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e4m3_satfinite_saturates_and_keeps_sign(orc):
    x = np.array([464.0, 480.0, 672.0, 2688.0, 1e30, -500.0, -2688.0, 0.0, -0.0], np.float32)
    assert list(orc.e4m3_encode_satfinite(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80]


def test_e4m3_scale_clamp(orc):
    rng = np.random.default_rng(3)
    sf = np.exp(rng.uniform(np.log(1e-5), np.log(2000.0), 5000)).astype(np.float32)
    a = orc.e4m3_encode_scale(sf, 256.0)
    b = orc.e4m3_encode_scale(np.minimum(sf, np.float32(256.0)), 448.0)
    assert np.array_equal(a, b)
    assert orc.e4m3_encode_scale(np.array([300.0, 1e9], np.float32), 256.0).tolist() == [0x78, 0x78]
    assert orc.e4m3_encode_scale(np.array([300.0, 1e9], np.float32), 448.0).tolist() == [0x79, 0x7E]


# --------------------------------------------------------------------------- fp16 / bf16
@pytest.mark.parametrize("is_bf16", [True, False])
def test_round_half_matches_torch(orc, is_bf16):
    rng = np.random.default_rng(5 + is_bf16)
    bits = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    extra = []
    # every product E2M1 x E4M3 x g for a few g, subnormal and overflow regions
    e2 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for g in (1.0, 0.0013485863, 2.0 ** -20, 3.3e-5, 1.7e3, 37.0):
        extra.append((e4[:, None] * np.float32(g)).astype(np.float32)[:, :, None] * e2[None, None, :])
    extra.append(np.exp(rng.uniform(np.log(1e-9), np.log(7e4), 100000)).astype(np.float32))
    x = np.concatenate([x] + [e.reshape(-1).astype(np.float32) for e in extra])
    x = np.concatenate([x, -x, np.array([65504, 65519.99, 65520, 3.3895e38, 5.96e-8, 2.98e-8, 0.0, -0.0],
                                         np.float32)])
    got = orc.round_half(x, is_bf16)
    want = torch.from_numpy(x).to(torch.bfloat16 if is_bf16 else torch.float16).view(torch.int16)
    want = want.numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("is_bf16", [True, False])
def test_half_value_matches_torch(orc, is_bf16):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16 if is_bf16 else torch.float16)
    ref = ref.double().numpy()
    for b in range(0, 65536, 7):
        v = orc.half_value(b, is_bf16)
        r = ref[b]
        assert (math.isnan(v) and math.isnan(r)) or (v == r and math.copysign(1, v) == math.copysign(1, r)), hex(b)
