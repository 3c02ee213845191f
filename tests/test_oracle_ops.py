"""Pins for the oracle's block quantizer and its three paged operations.

Each test checks the oracle against something it does not compute itself:
exact rational brute force, the constants the pages state, torch's codecs
(float8_e4m3fn / bfloat16 / float16 casts), exact round trips, and the
page-table semantics (which bytes may change, which pages and entries are
written)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = json.load(open(os.path.join(GOLDEN, "e2m1_grid.json")))["magnitudes"]
CONST = json.load(open(os.path.join(GOLDEN, "recipe_constants.json")))
E4M3_TORCH = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
E2M1_SIGNED = np.array(GRID + [-v for v in GRID], np.float32)       # code -> value (library-free)
E2M1_SIGNED[8] = -0.0


# --------------------------------------------------------------------------- exact helpers
def _nearest_code(a: Fraction, values, even_tie=True):
    d = [abs(a - v) for v in values]
    m = min(d)
    ks = [k for k, x in enumerate(d) if x == m]
    return ks[0] if len(ks) == 1 else [k for k in ks if k % 2 == 0][0]


E4_FR = [Fraction(float(E4M3_TORCH[c])) for c in range(127)]
E2_FR = [Fraction(v) for v in GRID]


def exact_candidate(x, g, C, clamp, mode):
    """Exact-arithmetic candidate: nearest E4M3 to min(amax/(C g), clamp),
    nearest E2M1 per element to x / dec, exact summed error."""
    xs = [Fraction(float(v)) for v in x]
    amax = max(abs(v) for v in xs)
    sf = min(amax / (C * Fraction(g)), Fraction(clamp))
    s = _nearest_code(sf, E4_FR)
    dec = E4_FR[s] * Fraction(g)
    codes, err = [], Fraction(0)
    margin = Fraction(10**9)
    for v in xs:
        q = abs(v) / dec if dec else Fraction(0)
        k = _nearest_code(q, E2_FR) if q < 6 else 7
        # distance of q from the nearest decision boundary (midpoint)
        for i in range(7):
            mid = (E2_FR[i] + E2_FR[i + 1]) / 2
            if dec:
                margin = min(margin, abs(q - mid) / mid)
        c = (8 if float(v) < 0 or (v == 0 and math.copysign(1, float(v)) < 0) else 0) | k
        codes.append(c)
        deq = dec * E2_FR[k] * (-1 if c & 8 else 1)
        d = v - deq
        err += d * d if mode == 0 else abs(d)
    s_mid_margin = min(abs(sf - (E4_FR[i] + E4_FR[i + 1]) / 2) for i in range(126)) / max(sf, Fraction(1, 2**20))
    return s, codes, err, min(margin, s_mid_margin)


# --------------------------------------------------------------------------- block quantizer
def test_block_with_amax_6sg_is_reproduced(orc):
    """A block whose amax is 6 * s * g (g a power of two, grid-valued
    elements) gives back s and every code exactly, -0 included."""
    rng = np.random.default_rng(21)
    for g in (2.0 ** -4, 1.0, 8.0, 2.0 ** -9):
        for s in list(range(0x08, 0x7F)):
            codes = rng.integers(0, 16, 16)
            codes[rng.integers(0, 16)] = rng.choice([7, 15])           # one element at +-6
            x = (E2M1_SIGNED[codes].astype(np.float64) * float(E4M3_TORCH[s]) * g).astype(np.float32)
            got, sb, *_ = orc.quantize_block(x, g)
            assert sb == s, (g, hex(s))
            assert list(got) == list(codes), (g, hex(s), list(got), list(codes))


def test_block_nearest_and_error_bound(orc):
    """Every non-saturated element is within half a grid gap of its
    reconstruction (nearest rounding), relative to the decode factor."""
    rng = np.random.default_rng(22)
    for _ in range(3000):
        x = (rng.standard_normal(16) * np.exp(rng.uniform(-5, 5))).astype(np.float32)
        g = float(np.float32(np.exp(rng.uniform(-8, 0))))
        codes, s, *_ = orc.quantize_block(x, g)
        dec = np.float32(E4M3_TORCH[s]) * np.float32(g)
        q = np.abs(E2M1_SIGNED[codes])
        gap = np.array([0.5, 0.5, 0.5, 0.5, 1, 1, 2, 2], np.float32)[(codes & 7)]
        err = np.abs(np.abs(x.astype(np.float64)) - q * float(dec))
        ok = (np.abs(x) / dec <= 6.0) | ((codes & 7) != 7)
        assert np.all(err[ok] <= 0.5 * gap[ok] * float(dec) * (1 + 1e-5) + 1e-30)
        # the block scale is the nearest E4M3 value to amax / (6 g)
        sf = Fraction(float(np.max(np.abs(x)))) / (6 * Fraction(g))
        d = [abs(sf - v) for v in E4_FR]
        assert d[s] <= min(d) * (1 + 1e-5) + Fraction(1, 10**30)


def test_block_scale_zero_block(orc):
    codes, s, *_ = orc.quantize_block(np.zeros(16, np.float32), 0.01)
    assert s == 0 and list(codes) == [0] * 16
    codes, s, *_ = orc.quantize_block(np.full(16, -0.0, np.float32), 0.01)
    assert s == 0 and list(codes) == [8] * 16


HAND_BLOCKS = {
    "no_outlier": [4, 3, 2, 1.5, 1, 0.5, 0, 0] * 2,
    "dominant_outlier": [6] + [0.5] * 15,
    "zeros": [0.0] * 16,
    "mse_mae_disagree": [6, 0, 0.25, 0.5, 6, 4, 5.5, 0.5, 4.5, 2, 2.5, 0, 3.5, 5, 4, 0.5],
    "mae_tie": [6, 1, 6, 5.5, 0.5, 3, 6, 5, 4, 3.5, 0, 4.5, 2.5, 0.25, 1, 3],
}


@pytest.mark.parametrize("name", sorted(HAND_BLOCKS))
@pytest.mark.parametrize("mode", [0, 1])
def test_four_over_six_hand_blocks_vs_exact(orc, name, mode):
    """4over6 keeps the candidate whose exact reconstruction error is lower
    (amax/6 on ties), on hand-built blocks where fp32 arithmetic is exact."""
    x = np.array(HAND_BLOCKS[name], np.float32)
    recipe = orc.four_over_six(err_mode=mode, e4m3_max=256.0)
    codes, s, e6, e4, chose4 = orc.quantize_block(x, 1.0, recipe)
    s6, c6, x6, m6 = exact_candidate(x, 1.0, 6, 256, mode)
    s4, c4, x4, m4 = exact_candidate(x, 1.0, 4, 448, mode)
    assert Fraction(e6) == x6 and Fraction(e4) == x4           # fp32 errors are exact here
    want4 = x4 < x6
    assert chose4 == want4
    assert s == (s4 if want4 else s6)
    assert list(codes) == (c4 if want4 else c6)


def test_four_over_six_known_outcomes(orc):
    """The hand blocks' outcomes follow from the page's description: a block
    with no dominant outlier prefers the tighter amax/4 scale, a block with one
    dominant outlier keeps amax/6, and zero blocks tie (amax/6 kept)."""
    mse = orc.four_over_six(0)
    mae = orc.four_over_six(1)
    assert orc.quantize_block(np.array(HAND_BLOCKS["no_outlier"], np.float32), 1.0, mse)[4]
    assert orc.quantize_block(np.array(HAND_BLOCKS["no_outlier"], np.float32), 1.0, mae)[4]
    assert not orc.quantize_block(np.array(HAND_BLOCKS["dominant_outlier"], np.float32), 1.0, mse)[4]
    assert not orc.quantize_block(np.array(HAND_BLOCKS["dominant_outlier"], np.float32), 1.0, mae)[4]
    assert not orc.quantize_block(np.zeros(16, np.float32), 1.0, mse)[4]
    r_mse = orc.quantize_block(np.array(HAND_BLOCKS["mse_mae_disagree"], np.float32), 1.0, mse)[4]
    r_mae = orc.quantize_block(np.array(HAND_BLOCKS["mse_mae_disagree"], np.float32), 1.0, mae)[4]
    assert r_mse != r_mae
    _, _, e6, e4, c = orc.quantize_block(np.array(HAND_BLOCKS["mae_tie"], np.float32), 1.0, mae)
    assert e6 == e4 and not c


def test_four_over_six_random_blocks_vs_exact(orc):
    """Random blocks (t-distributed, some with an outlier): when the exact
    arithmetic is far from every rounding boundary and the two exact errors
    are not near a tie, the oracle's choice, scale and codes are the exact
    brute-force ones."""
    rng = np.random.default_rng(23)
    checked = 0
    for it in range(1500):
        x = rng.standard_t(3, 16).astype(np.float32)
        if it % 3 == 0:
            x[rng.integers(0, 16)] *= 20
        x = W.bits_to_f32(W.f32_to_bits(x, True), True)
        g = float(np.float32(np.max(np.abs(x)) / (6 * 256) * rng.uniform(1.0, 3.0)))
        mode = it % 2
        s6, c6, x6, m6 = exact_candidate(x, g, 6, 256, mode)
        s4, c4, x4, m4 = exact_candidate(x, g, 4, 448, mode)
        if min(m6, m4) < 1e-4 or abs(x4 - x6) <= Fraction(1, 10**4) * max(x4, x6):
            continue
        codes, s, e6, e4, chose4 = orc.quantize_block(x, g, orc.four_over_six(mode))
        want4 = x4 < x6
        assert chose4 == want4
        assert s == (s4 if want4 else s6)
        assert list(codes) == (c4 if want4 else c6)
        checked += 1
    assert checked > 1000


def test_recipe_constants_from_page(orc):
    """With a recipe-matched global scale the tensor-amax block gets block
    scale e4m3_max; its amax/4 candidate needs 1.5x that: 384 for the 256
    recipe (fits), 672 for a 448-based scale (saturates to 448)."""
    rng = np.random.default_rng(24)
    for e4m3_max, want_s4 in ((CONST["four_over_six_e4m3_max"], CONST["fits"]),
                              (CONST["e4m3_largest_finite"], CONST["saturates_at_448_recipe"])):
        x = W.f32_to_bits(rng.standard_normal((64, 16)).astype(np.float32), True)
        g = orc.global_scale(x, True, e4m3_max)
        xf = W.bits_to_f32(x, True)
        amax = float(np.max(np.abs(xf)))
        assert g == float(np.float32(amax) / np.float32(6.0 * e4m3_max))
        row = xf[np.argmax(np.max(np.abs(xf), axis=1))]
        _, s, *_ = orc.quantize_block(row, g, orc.Recipe(False, e4m3_max))
        assert E4M3_TORCH[s] == e4m3_max
        _, s4, *_ = orc.quantize_block(row, g, orc.Recipe(False, CONST["e4m3_largest_finite"]))
        s4c = orc.e4m3_encode_scale(np.array([amax / (4 * g)], np.float32), 448.0)[0]
        assert abs(amax / (4 * g) - want_s4) < 1e-2 * want_s4
        assert E4M3_TORCH[s4c] == min(want_s4, CONST["e4m3_largest_finite"])
    assert orc.global_scale(np.zeros(32, np.uint16), True, 448.0) == 1.0


# --------------------------------------------------------------------------- append
def _small_append_case(rng, layout, stacked=False, ps=16, H=4, D=64, B=5, pool=40, data_pad=0):
    lens = rng.integers(1, 60, B)
    start = np.array([rng.integers(0, l) for l in lens])          # existing length before append
    perm = rng.permutation(pool)
    indices, indptr, last = W.csr_for_lengths(lens, ps, perm)
    cache = W.make_cache(rng, pool, ps, H, D, layout, stacked=stacked, data_pad=data_pad)
    bi, pos = W.rows_for_positions(start, lens)
    nnz = len(bi)
    key = W.f32_to_bits(rng.standard_normal((nnz, H, D)).astype(np.float32), True)
    val = W.f32_to_bits((rng.standard_normal((nnz, H, D)) * 3).astype(np.float32), True)
    return cache, key, val, bi, pos, indices, indptr, last, lens


@pytest.mark.parametrize("layout", [W.NHD, W.HND])
def test_append_changes_only_addressed_bytes(orc, layout):
    rng = np.random.default_rng(31 + layout)
    cache, key, val, bi, pos, indices, indptr, last, _ = _small_append_case(rng, layout)
    before = cache.copy()
    gk, gv = orc.global_scale(key, True), orc.global_scale(val, True)
    orc.quantize_append(cache, key, val, True, bi, pos, indices, indptr, last, gk, gv)
    ps, H, D = cache.page_size, cache.num_heads, cache.head_dim
    touched = [np.zeros(a.shape, bool) for a in (cache.k_data, cache.v_data, cache.k_sf, cache.v_sf)]
    for r in range(len(bi)):
        b, p = bi[r], pos[r]
        page, slot = indices[indptr[b] + p // ps], p % ps
        for kv, (src, g) in enumerate(((key, gk), (val, gv))):
            d4 = cache.data_4d(kv)
            s4 = cache.sf_4d(kv)
            for h in range(H):
                row_d = d4[page, slot, h] if layout == W.NHD else d4[page, h, slot]
                row_s = s4[page, slot, h] if layout == W.NHD else s4[page, h, slot]
                xs = W.bits_to_f32(src[r, h], True)
                for blk in range(D // 16):
                    codes, s, *_ = orc.quantize_block(xs[blk * 16:(blk + 1) * 16], g)
                    assert row_s[blk] == s
                    packed = codes[0::2] | (codes[1::2] << 4)
                    assert np.array_equal(row_d[blk * 8:(blk + 1) * 8], packed)
                off_d = ((slot * H + h) if layout == W.NHD else (h * ps + slot)) * (D // 2)
                off_s = ((slot * H + h) if layout == W.NHD else (h * ps + slot)) * (D // 16)
                touched[kv][page, off_d:off_d + D // 2] = True
                touched[2 + kv][page, off_s:off_s + D // 16] = True
    for t, a, b0 in zip(touched, (cache.k_data, cache.v_data, cache.k_sf, cache.v_sf),
                        (before.k_data, before.v_data, before.k_sf, before.v_sf)):
        assert np.array_equal(a[~t], b0[~t])


def test_append_layouts_and_stacking_agree(orc):
    rng = np.random.default_rng(33)
    args = _small_append_case(rng, W.NHD)
    _, key, val, bi, pos, indices, indptr, last, _ = args
    ps, H, D, pool = 16, 4, 64, 40
    gk, gv = orc.global_scale(key, True), orc.global_scale(val, True)
    caches = {}
    for name, layout, stacked, pad in (("nhd", W.NHD, False, 0), ("hnd", W.HND, False, 0),
                                       ("nhd_stacked", W.NHD, True, 0), ("hnd_padded", W.HND, False, 48)):
        c = W.make_cache(np.random.default_rng(0), pool, ps, H, D, layout, stacked=stacked,
                         data_pad=pad, fill="zero")
        orc.quantize_append(c, key, val, True, bi, pos, indices, indptr, last, gk, gv)
        caches[name] = c
    for kv in (0, 1):
        a = caches["nhd"].data_4d(kv)
        assert np.array_equal(a, caches["hnd"].data_4d(kv).transpose(0, 2, 1, 3))
        assert np.array_equal(a, caches["nhd_stacked"].data_4d(kv))
        assert np.array_equal(caches["hnd"].data_4d(kv), caches["hnd_padded"].data_4d(kv))
        s = caches["nhd"].sf_4d(kv)
        assert np.array_equal(s, caches["hnd"].sf_4d(kv).transpose(0, 2, 1, 3))
        assert np.array_equal(s, caches["nhd_stacked"].sf_4d(kv))


def test_append_rejects_rows_outside_reserved_space(orc):
    rng = np.random.default_rng(34)
    cache, key, val, bi, pos, indices, indptr, last, lens = _small_append_case(rng, W.NHD)
    bad = pos.copy()
    bad[0] = lens[bi[0]]                        # one past the request's last reserved slot
    with pytest.raises(ValueError):
        orc.quantize_append(cache, key, val, True, bi, bad, indices, indptr, last, 0.01, 0.01)
    with pytest.raises(ValueError):
        orc.quantize_append(cache, key, val, True, bi, pos, indices, indptr, last, 0.0, 0.01)


# --------------------------------------------------------------------------- dequant
def _grid_cache(rng, layout, ps, H, D, pages, g, is_bf16):
    """A cache whose content is the exact encoding of grid-valued rows: each
    block holds one +-6 element, so quantizing x = e2m1 * E4M3(s) * g gives
    back (s, codes) and dequantizing must give back x exactly."""
    n_rows = pages * ps
    codes = rng.integers(0, 16, (n_rows, H, D)).astype(np.uint8)
    codes[..., ::16] = rng.choice([7, 15], (n_rows, H, D // 16))
    s = rng.integers(0x20, 0x70, (n_rows, H, D // 16)).astype(np.uint8)
    x = E2M1_SIGNED[codes].astype(np.float64) * E4M3_TORCH[np.repeat(s, 16, axis=2)] * g
    bits = W.f32_to_bits(x.astype(np.float32), is_bf16)
    assert np.array_equal(W.bits_to_f32(bits, is_bf16), x.astype(np.float32))   # exactly representable
    return bits


@pytest.mark.parametrize("layout", [W.NHD, W.HND])
@pytest.mark.parametrize("is_bf16", [True, False])
def test_dequant_exact_round_trip_and_tail(orc, layout, is_bf16):
    rng = np.random.default_rng(41 + 2 * layout + is_bf16)
    ps, H, D, B = 8, 2, 64, 3
    lens = np.array([3, 17, 24])
    pages = int(((lens + ps - 1) // ps).sum())
    g = 2.0 ** -3
    kb = _grid_cache(rng, layout, ps, H, D, pages, g, is_bf16)
    vb = _grid_cache(rng, layout, ps, H, D, pages, g, is_bf16)
    perm = rng.permutation(pages + 4)
    indices, indptr, last = W.csr_for_lengths(lens, ps, perm)
    bi, pos = W.rows_for_positions(np.zeros(B, int), lens)
    nnz = len(bi)
    cache = W.make_cache(rng, pages + 4, ps, H, D, layout)
    orc.quantize_append(cache, kb[:nnz], vb[:nnz], is_bf16, bi, pos, indices, indptr, last, g, g)
    T = 26
    for bt_dtype in (np.int32, np.int64):
        bt = W.block_table_from_csr(indices, indptr, 4, bt_dtype)
        ok = np.full((B, T, H, D), W.SENTINEL_16, np.uint16)
        ov = ok.copy()
        orc.dequantize_paged(cache, bt, lens.astype(np.int32), g, g, ok, ov, is_bf16)
        for b in range(B):
            rows = np.nonzero(bi == b)[0]
            assert np.array_equal(ok[b, :lens[b]], kb[rows])
            assert np.array_equal(ov[b, :lens[b]], vb[rows])
            assert np.all(ok[b, lens[b]:] == W.SENTINEL_16) and np.all(ov[b, lens[b]:] == W.SENTINEL_16)


@pytest.mark.parametrize("out_bf16", [True, False])
def test_dequant_matches_library_codecs(orc, out_bf16):
    """Random cache bytes: each output is torch's RNE cast of
    fp32(fp32(E4M3(s) * g) * e2m1), with torch decoding the E4M3 byte."""
    rng = np.random.default_rng(43 + out_bf16)
    ps, H, D, B, pool = 16, 3, 32, 4, 30
    lens = np.array([1, 16, 33, 70])
    cache = W.make_cache(rng, pool, ps, H, D, W.NHD)
    for a in (cache.k_sf, cache.v_sf):                 # include negative and subnormal scales
        a[...] = rng.integers(0, 256, a.shape, dtype=np.uint8)
        a[a == 0x7F] = 0x7E
        a[a == 0xFF] = 0xFE
    bt = rng.permutation(pool)[:B * 5].reshape(B, 5).astype(np.int32)
    T = 64                                              # request 3 is clamped at max_seq_len
    ok = np.full((B, T, H, D), W.SENTINEL_16, np.uint16)
    ov = ok.copy()
    gk, gv = 0.0123, 3.7e-5
    orc.dequantize_paged(cache, bt, lens.astype(np.int32), gk, gv, ok, ov, out_bf16)
    for kv, out, g in ((0, ok, gk), (1, ov, gv)):
        d4, s4 = cache.data_4d(kv), cache.sf_4d(kv)
        for b in range(B):
            L = min(lens[b], T)
            t = np.arange(L)
            pg, sl = bt[b, t // ps], t % ps
            bytes_ = d4[pg, sl]                          # [L, H, D/2]
            codes = np.stack([bytes_ & 15, bytes_ >> 4], -1).reshape(L, H, D)
            sc = np.repeat(s4[pg, sl], 16, axis=2)       # [L, H, D]
            dec = (E4M3_TORCH[sc].astype(np.float32) * np.float32(g)).astype(np.float32)
            y = (dec * E2M1_SIGNED[codes]).astype(np.float32)
            want = torch.from_numpy(y).to(torch.bfloat16 if out_bf16 else torch.float16)
            want = want.view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(out[b, :L], want)
            assert np.all(out[b, L:] == W.SENTINEL_16)


def test_dequant_is_recipe_agnostic(orc):
    """4over6 output is ordinary NVFP4: dequantizing it is the same formula,
    and the 4over6 reconstruction error never exceeds the standard one per
    block (its candidate set contains the standard choice)."""
    rng = np.random.default_rng(44)
    x = W.f32_to_bits(W.student_t_with_outliers(rng, (64, 1, 128)), True)
    xf = W.bits_to_f32(x, True).reshape(-1, 16)
    for mode in (0, 1):
        g = orc.global_scale(x, True, 256.0)
        for blk in xf:
            c46, s46, e6, e4, _ = orc.quantize_block(blk, g, orc.four_over_six(mode))
            cst, sst, *_ = orc.quantize_block(blk, g, orc.Recipe(False, 256.0))
            if not (e4 < e6):
                assert list(c46) == list(cst) and s46 == sst


# --------------------------------------------------------------------------- materialize
def _mat_case(rng, shared, compact=True, slack=0, ps=8, H=2, D=64):
    lens = np.array([1, 8, 21, 0, 9])
    B = len(lens)
    need = (lens + ps - 1) // ps
    P = int(need.sum()) + 3
    maxp = int(need.max()) + 1
    cache = W.make_cache(rng, P, ps, H, D, W.HND, data_pad=32)
    for a in (cache.k_sf, cache.v_sf):
        a[...] = rng.integers(0, 256, a.shape, dtype=np.uint8)
        a[a == 0x7F] = 0x7E
        a[a == 0xFF] = 0xFE
    res = need + (slack if not compact else 0)
    indptr = np.zeros(B + 1, np.int32)
    indptr[1:] = np.cumsum(res)
    pk = rng.permutation(P)
    pv = rng.permutation(P)
    if shared:
        bt = np.zeros((B, maxp), np.int32)
    else:
        bt = np.zeros((B, 2, maxp), np.int32)
    for b in range(B):
        if shared:
            bt[b, :need[b]] = pk[:need[b]]
        else:
            bt[b, 0, :need[b]] = pk[:need[b]]
            bt[b, 1, :need[b]] = pv[:need[b]]
        pk, pv = np.roll(pk, 3), np.roll(pv, 5)
    return cache, bt, lens.astype(np.int32), indptr, need, maxp


def _deinterleave(sf4, ps, nb):
    """[pages, H, ps, nb] interleaved scale bytes -> linear order."""
    flat = sf4.reshape(sf4.shape[0], sf4.shape[1], ps * nb)
    t = np.arange(ps)[:, None]
    c = np.arange(nb)[None, :]
    src = ((t // 4) * nb + c) * 4 + t % 4
    return flat[:, :, src]


@pytest.mark.parametrize("shared", [True, False])
def test_materialize_pages_table_and_values(orc, shared):
    rng = np.random.default_rng(51 + shared)
    cache, bt, lens, indptr, need, maxp = _mat_case(rng, shared, compact=False, slack=1)
    ps, H, D = cache.page_size, cache.num_heads, cache.head_dim
    n_out = int(indptr[-1]) + 3                         # workspace larger than the step needs
    out = np.full((n_out, 2, H, ps, D), W.SENTINEL_FP8, np.uint8)
    table = np.full((len(lens), maxp), -1, np.int32)
    orc.materialize_fp8(cache, bt, lens, indptr, out, table, shared=shared, v_sf_interleaved=True)
    assert np.all(out[0] == 0)
    written = {0}
    for b in range(len(lens)):
        for j in range(maxp):
            if j < need[b]:
                dst = indptr[b] + j + 1
                assert table[b, j] == dst
                written.add(dst)
                for kv in (0, 1):
                    page = bt[b, j] if shared else bt[b, kv, j]
                    codes_b = cache.data_4d(kv)[page]                    # [H, ps, D/2]
                    codes = np.stack([codes_b & 15, codes_b >> 4], -1).reshape(H, ps, D)
                    sfp = cache.sf_4d(kv)[page][None]
                    if kv == 1:
                        sfp = _deinterleave(sfp, ps, D // 16).reshape(1, H, ps, D // 16)
                    sc = np.repeat(sfp[0], 16, axis=2)
                    prod = (E2M1_SIGNED[codes] * E4M3_TORCH[sc]).astype(np.float32)
                    want = torch.from_numpy(np.clip(prod, -448, 448)).to(torch.float8_e4m3fn)
                    want = want.view(torch.uint8).numpy()
                    assert np.array_equal(out[dst, kv], want)
            else:
                assert table[b, j] == -1
    for p in range(n_out):
        if p not in written:
            assert np.all(out[p] == W.SENTINEL_FP8), p


def test_materialize_product_table_saturates(orc):
    """All 16 codes x all finite scale bytes: torch's cast where |product| <
    464, saturation to +-448 above (page: FP8 copy of E2M1 x E4M3 only)."""
    rng = np.random.default_rng(53)
    ps, H, D = 4, 1, 64
    cache = W.make_cache(rng, 2, ps, H, D, W.HND, fill="zero")
    pairs = [(c, s) for s in range(256) if s not in (0x7F, 0xFF) for c in range(16)]
    got = {}
    for start in range(0, len(pairs), ps * D):
        chunk = pairs[start:start + ps * D]
        codes = np.zeros(ps * D, np.uint8)
        scales = np.zeros(ps * D // 16, np.uint8)
        # one scale per 16-element block: lay pairs out so each block shares a scale
        for i, (c, s) in enumerate(chunk):
            codes[i] = c
        sblock = [chunk[min(i * 16, len(chunk) - 1)][1] for i in range(ps * D // 16)]
        scales[:] = sblock
        cache.k_data[0, :] = codes[0::2] | (codes[1::2] << 4)
        cache.k_sf[0, :] = scales
        cache.v_data[0, :] = cache.k_data[0]
        cache.v_sf[0, :] = scales
        out = np.zeros((2, 2, H, ps, D), np.uint8)
        table = np.zeros((1, 1), np.int32)
        orc.materialize_fp8(cache, np.zeros((1, 1), np.int32), np.array([ps], np.int32),
                            np.array([0, 1], np.int32), out, table, shared=True, v_sf_interleaved=False)
        flat = out[1, 0].reshape(-1)
        for i, (c, s) in enumerate(chunk):
            if sblock[i // 16] == s:
                got[(c, s)] = flat[i]
    for (c, s), byte in got.items():
        p = float(E2M1_SIGNED[c]) * float(E4M3_TORCH[s])
        if abs(p) < 464:
            want = torch.tensor([p]).to(torch.float8_e4m3fn).view(torch.uint8).item()
        else:
            want = 0x7E | (0x80 if p < 0 else 0)
        if p == 0:
            want = 0x80 if (math.copysign(1, float(E2M1_SIGNED[c])) * math.copysign(1, float(E4M3_TORCH[s]))) < 0 else 0
        assert byte == want, (c, hex(s), p, hex(byte), hex(want))
    assert len(got) >= 16 * 254 * 0.9


def test_materialize_interleave_and_tables_self_consistent(orc):
    rng = np.random.default_rng(54)
    cache, bt, lens, indptr, need, maxp = _mat_case(rng, shared=False)
    ps, H, D = cache.page_size, cache.num_heads, cache.head_dim
    n_out = int(indptr[-1]) + 1
    out_a = np.full((n_out, 2, H, ps, D), 1, np.uint8)
    tab_a = np.full((len(lens), maxp), -1, np.int32)
    orc.materialize_fp8(cache, bt, lens, indptr, out_a, tab_a, shared=False, v_sf_interleaved=True)
    lin = cache.copy()
    lin.v_sf[...] = _deinterleave(cache.sf_4d(1), ps, D // 16).reshape(lin.v_sf.shape)
    out_b = np.full_like(out_a, 1)
    tab_b = np.full_like(tab_a, -1)
    orc.materialize_fp8(lin, bt, lens, indptr, out_b, tab_b, shared=False, v_sf_interleaved=False)
    assert np.array_equal(out_a, out_b) and np.array_equal(tab_a, tab_b)
    # equal K and V tables: shared and separate forms agree
    same = bt.copy()
    same[:, 1] = same[:, 0]
    out_c = np.full_like(out_a, 1)
    tab_c = np.full_like(tab_a, -1)
    orc.materialize_fp8(cache, same, lens, indptr, out_c, tab_c, shared=False)
    out_d = np.full_like(out_a, 1)
    tab_d = np.full_like(tab_a, -1)
    orc.materialize_fp8(cache, np.ascontiguousarray(same[:, 0]), lens, indptr, out_d, tab_d, shared=True)
    assert np.array_equal(out_c, out_d) and np.array_equal(tab_c, tab_d)


def test_materialize_and_dequant_agree_where_fp8_is_exact(orc):
    """With g a power of two: wherever the FP8 copy holds the product
    exactly, fp8 * g equals dequant's fp32 value, so both give the same
    bf16 output."""
    rng = np.random.default_rng(55)
    cache, bt, lens, indptr, need, maxp = _mat_case(rng, shared=True)
    ps, H, D = cache.page_size, cache.num_heads, cache.head_dim
    for a in (cache.k_sf, cache.v_sf):
        a[...] = rng.integers(0x10, 0x60, a.shape, dtype=np.uint8)
    n_out = int(indptr[-1]) + 1
    out = np.zeros((n_out, 2, H, ps, D), np.uint8)
    tab = np.zeros((len(lens), maxp), np.int32)
    orc.materialize_fp8(cache, bt, lens, indptr, out, tab, shared=True, v_sf_interleaved=False)
    g = 2.0 ** -5
    T = int(lens.max())
    ok = np.zeros((len(lens), T, H, D), np.uint16)
    ov = ok.copy()
    orc.dequantize_paged(cache, bt, lens, g, g, ok, ov, True)
    n = 0
    for b in range(len(lens)):
        for t in range(lens[b]):
            j, slot = t // ps, t % ps
            for kv, o in ((0, ok), (1, ov)):
                fp8 = E4M3_TORCH[out[tab[b, j], kv, :, slot, :]]           # [H, D]
                page = bt[b, j]
                codes_b = cache.data_4d(kv)[page][:, slot]
                codes = np.stack([codes_b & 15, codes_b >> 4], -1).reshape(H, D)
                sc = np.repeat(cache.sf_4d(kv)[page][:, slot], 16, axis=1)
                exact = E2M1_SIGNED[codes].astype(np.float64) * E4M3_TORCH[sc]
                m = fp8 == exact
                want = W.f32_to_bits((fp8 * np.float32(g)).astype(np.float32), True)
                assert np.array_equal(o[b, t][m], want[m])
                n += int(m.sum())
    assert n > 1000
