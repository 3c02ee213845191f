"""Pins for the oracle's contiguous codec and whole-pool quantizer
(flashinfer.quantization module page, "FP4 KV Cache Quantization":
nvfp4_kv_quantize, nvfp4_kv_dequantize, nvfp4_quantize_paged_kv_cache).

The pins do not go through the oracle's own arithmetic: inputs are built in
closed form as e2m1 * E4M3(s) * g with one element of magnitude 6 in every
block and g a power of two, so the block scale is exactly s and every code is
the one the input was built from; dequantizing gives the input back bit for
bit. The E4M3 values come from torch's float8_e4m3fn decode, the E2M1 grid
from the fixture. The V-scale interleave is pinned by a hand-written table."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = json.load(open(os.path.join(GOLDEN, "e2m1_grid.json")))["magnitudes"]
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
E2M1 = np.array(GRID + [-v for v in GRID], np.float64)
E2M1[8] = -0.0


def exact_blocks(rng, n_blocks, max_scale_byte, g):
    """codes [n_blocks, 16] (one +-6 per block), scale bytes [n_blocks], and
    the values e2m1 * E4M3(s) * g as float64 (exact in fp16 and bf16)."""
    codes = rng.integers(0, 16, size=(n_blocks, 16)).astype(np.uint8)
    where = rng.integers(0, 16, size=n_blocks)
    sign = rng.integers(0, 2, size=n_blocks).astype(np.uint8) << 3
    codes[np.arange(n_blocks), where] = 7 | sign
    s = rng.integers(1, max_scale_byte + 1, size=n_blocks).astype(np.uint8)
    zero = rng.random(n_blocks) < 0.05                  # a few all-zero blocks: s = 0, codes 0
    s[zero] = 0
    codes[zero] = 0
    x = E2M1[codes] * E4M3[s][:, None] * g
    return codes, s, x


def to_bits(x64, bf16):
    t = torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16 if bf16 else torch.float16)
    assert np.array_equal(t.double().numpy(), x64), "built values must be exact in the 16-bit type"
    return t.view(torch.int16).numpy().view(np.uint16)


def pack(codes):
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


RECIPES = [("standard", 448), ("4over6 MSE", 256), ("4over6 MAE", 256)]


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("recipe_name,smax", RECIPES)
def test_contiguous_exact_blocks(orc, bf16, recipe_name, smax):
    rng = np.random.default_rng(11)
    rows, cols, g = 37, 96, 2.0 ** -4
    rec = {"standard": orc.STANDARD, "4over6 MSE": orc.four_over_six(orc.MSE),
           "4over6 MAE": orc.four_over_six(orc.MAE)}[recipe_name]
    max_byte = int(np.nonzero(E4M3[:127] <= smax)[0].max())
    codes, s, x = exact_blocks(rng, rows * cols // 16, max_byte, g)
    bits = to_bits(x.reshape(rows, cols), bf16)
    got_codes, got_s = orc.quantize_contiguous(bits, bf16, g, rec, threads=4)
    assert got_codes.shape == (rows, cols // 2) and got_s.shape == (rows, cols // 16)
    assert np.array_equal(got_s.ravel(), s)
    assert np.array_equal(got_codes.reshape(-1, 8), pack(codes))
    back = orc.dequantize_contiguous(got_codes, got_s, g, bf16, threads=4)
    assert np.array_equal(back, bits)


def test_contiguous_leading_dims_and_empty(orc):
    rng = np.random.default_rng(12)
    codes, s, x = exact_blocks(rng, 2 * 3 * 4, 0x77, 1.0)
    bits = to_bits(x.reshape(2, 3, 64), True)
    c, sc = orc.quantize_contiguous(bits, True, 1.0)
    assert c.shape == (2, 3, 32) and sc.shape == (2, 3, 4)
    assert np.array_equal(sc.ravel(), s)
    c0, s0 = orc.quantize_contiguous(np.zeros((0, 32), np.uint16), True, 1.0)
    assert c0.shape == (0, 16) and s0.shape == (0, 2)
    with pytest.raises(ValueError):
        orc.quantize_contiguous(np.zeros((2, 24), np.uint16), True, 1.0)       # not a multiple of 16


def test_contiguous_matches_append_rows(orc):
    """The same rows appended into one NHD page of a paged cache give the
    same codes and scales (the two calls only differ in addressing)."""
    rng = np.random.default_rng(13)
    H, D, n = 2, 64, 8
    x = W.f32_to_bits(W.normal_rows(rng, (n, H, D)), True)
    g = orc.global_scale(x, True)
    c, s = orc.quantize_contiguous(x, True, g)
    cache = W.make_cache(rng, 1, n, H, D, W.NHD, fill="zero")
    orc.quantize_append(cache, x, x, True, np.zeros(n, np.int32), np.arange(n, dtype=np.int32),
                        np.zeros(1, np.int32), np.array([0, 1], np.int32), np.array([n], np.int32), g, g)
    assert np.array_equal(cache.k_data.reshape(-1), c.reshape(-1))
    assert np.array_equal(cache.k_sf.reshape(-1), s.reshape(-1))


def _pool_case(orc, rng, layout, ps, H, D, P, g):
    """K built with decode scale g, V with 2 g"""
    nb = D // 16
    ck, sk, xk = exact_blocks(rng, P * ps * H * nb, 0x7E, g)
    cv, sv, xv = exact_blocks(rng, P * ps * H * nb, 0x7E, 2 * g)
    cache = W.make_cache(rng, P, ps, H, D, layout, data_pad=32, fill="random")
    kb, vb = to_bits(xk, True), to_bits(xv, True)
    return cache, (ck, sk, kb), (cv, sv, vb)


def test_pool_quantizer_interleaved_v_scales(orc):
    """HND pool, V scales interleaved: codes and K scales in page order, V
    scales at the positions of the hand-written table."""
    tab = json.load(open(os.path.join(GOLDEN, "v_scale_interleave_ps8_nb2.json")))
    ps, nb = tab["page_size"], tab["blocks_per_row"]
    H, D, P, g = 2, 16 * nb, 3, 2.0 ** -3
    rng = np.random.default_rng(14)
    cache, (ck, sk, kb), (cv, sv, vb) = _pool_case(orc, rng, W.HND, ps, H, D, P, g)
    orc.quantize_paged_cache(cache, kb, vb, True, g, 2 * g, v_sf_interleaved=True)
    assert np.array_equal(cache.k_data[:, :ps * H * D // 2].reshape(-1, 8), pack(ck))
    assert np.array_equal(cache.v_data[:, :ps * H * D // 2].reshape(-1, 8), pack(cv))
    assert np.array_equal(cache.k_sf.reshape(-1), sk)
    # sv is in page order (p, h, t, c); place it by the table inside each (p, h) tile
    want = np.zeros(P * H * ps * nb, np.uint8)
    for p in range(P):
        for h in range(H):
            base = (p * H + h) * ps * nb
            for t in range(ps):
                for c in range(nb):
                    want[base + tab["position"][f"t{t}"][c]] = sv[base + t * nb + c]
    assert np.array_equal(cache.v_sf.reshape(-1), want)


@pytest.mark.parametrize("layout", [W.NHD, W.HND])
def test_pool_quantizer_linear(orc, layout):
    ps, H, D, P, g = 5 if layout == W.NHD else 8, 3, 48, 4, 0.5
    rng = np.random.default_rng(15)
    cache, (ck, sk, kb), (cv, sv, vb) = _pool_case(orc, rng, layout, ps, H, D, P, g)
    pad_before = cache.k_data[:, ps * H * D // 2:].copy()
    orc.quantize_paged_cache(cache, kb, vb, True, g, 2 * g, v_sf_interleaved=False)
    assert np.array_equal(cache.k_data[:, :ps * H * D // 2].reshape(-1, 8), pack(ck))
    assert np.array_equal(cache.v_data[:, :ps * H * D // 2].reshape(-1, 8), pack(cv))
    assert np.array_equal(cache.k_sf.reshape(-1), sk) and np.array_equal(cache.v_sf.reshape(-1), sv)
    assert np.array_equal(cache.k_data[:, ps * H * D // 2:], pad_before)      # page padding untouched
    if layout == W.NHD:
        with pytest.raises(ValueError):
            orc.quantize_paged_cache(cache, kb, vb, True, g, 2 * g, v_sf_interleaved=True)


def test_pool_quantizer_feeds_materialize(orc):
    """Quantize a pool with interleaved V scales and materialize it reading
    them interleaved; quantize it with linear V scales and materialize it
    reading them linearly: the FP8 pages agree."""
    rng = np.random.default_rng(16)
    ps, H, D, P = 8, 2, 64, 5
    k = W.f32_to_bits(W.normal_rows(rng, (P, H, ps, D)), True)
    v = W.f32_to_bits(W.normal_rows(rng, (P, H, ps, D)), True)
    gk, gv = orc.global_scale(k, True), orc.global_scale(v, True)
    outs = []
    for inter in (True, False):
        cache = W.make_cache(np.random.default_rng(0), P, ps, H, D, W.HND, fill="zero")
        orc.quantize_paged_cache(cache, k, v, True, gk, gv, v_sf_interleaved=inter)
        out = np.full((P + 1, 2, H, ps, D), 0x5A, np.uint8)
        tab = np.zeros((1, P), np.int32)
        orc.materialize_fp8(cache, np.arange(P, dtype=np.int32)[None, :], np.array([P * ps], np.int32),
                            np.array([0, P], np.int32), out, tab, shared=True, v_sf_interleaved=inter)
        outs.append(out)
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("bf16", [True, False])
def test_contiguous_dequant_matches_paged_dequant(orc, bf16):
    """With a g that is not a power of two the fp32 multiply order shows in
    the 16-bit result; the contiguous dequant follows the same order as the
    paged one (whose order is pinned in test_oracle_readings)."""
    rng = np.random.default_rng(17)
    H, D, n = 4, 64, 24
    codes = np.frombuffer(rng.bytes(n * H * D // 2), np.uint8).reshape(n, H, D // 2)
    scales = W.scale_bytes(rng, (n, H, D // 16))
    for g in (0.3, 1.7e-3, 123.456):
        y = orc.dequantize_contiguous(codes, scales, g, bf16)
        cache = W.make_cache(rng, 1, n, H, D, W.NHD, fill="zero")
        cache.k_data[0, :] = codes.reshape(-1)
        cache.v_data[0, :] = codes.reshape(-1)
        cache.k_sf[0, :] = scales.reshape(-1)
        cache.v_sf[0, :] = scales.reshape(-1)
        ok = np.zeros((1, n, H, D), np.uint16)
        ov = np.zeros_like(ok)
        orc.dequantize_paged(cache, np.zeros((1, 1), np.int32), np.array([n], np.int32), g, g, ok, ov, bf16)
        assert np.array_equal(y.reshape(-1), ok.reshape(-1))


@pytest.mark.parametrize("bf16", [True, False])
def test_contiguous_dequant_multiply_order(orc, bf16):
    """R7 order, (E4M3(s) * g) first, then times the E2M1 value: g is built
    so that some products sit next to a 16-bit rounding midpoint, where the
    other order (E2M1 * g first) rounds to a different 16-bit value."""
    rng = np.random.default_rng(65)
    f32 = np.float32
    tdt = torch.bfloat16 if bf16 else torch.float16
    s_all = np.arange(0x08, 0x7F, dtype=np.uint8)
    S = E4M3[s_all].astype(f32)
    signed = E2M1.astype(f32)
    codes = np.arange(16, dtype=np.uint8)
    found = 0
    for _ in range(3000):
        s0, e0 = int(rng.choice(s_all)), f32(rng.choice([1.5, 3.0, 6.0]))
        b = torch.tensor([float(rng.uniform(0.01, 10))]).to(tdt).float().numpy()[0]
        ulp = np.spacing(f32(b)) * (2 ** 16 if bf16 else 2 ** 13)
        g0 = f32(f32(b + ulp / 2) / (f32(E4M3[s0]) * e0))
        g = (np.array([g0], f32).view(np.int32) + rng.integers(-4, 5)).view(f32)[0]
        y_r7 = (S * g).astype(f32)[:, None] * signed[None, :]
        y_other = (signed[None, :] * g).astype(f32) * S[:, None]
        want = torch.from_numpy(y_r7.astype(f32)).to(tdt).view(torch.int16).numpy().view(np.uint16)
        other = torch.from_numpy(y_other.astype(f32)).to(tdt).view(torch.int16).numpy().view(np.uint16)
        if np.array_equal(want, other):
            continue
        packed = np.tile(codes[0::2] | (codes[1::2] << 4), (len(s_all), 1)).astype(np.uint8)
        got = orc.dequantize_contiguous(packed, s_all[:, None].copy(), float(g), bf16)
        assert np.array_equal(got, want)
        found += int(np.sum(want != other))
        if found >= 10:
            break
    assert found >= 10
