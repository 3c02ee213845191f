"""The fp32 operation order of the oracle's readings, pinned on inputs where
that order changes the result.

The pages fix the formats, the amax/6 and amax/4 candidates, fp32 error
scoring and e2m1 * block_scale * global_scale, but not the order of the
fp32 steps. The oracle states one order per step (block scale amax / fp32(C*g);
encode through the reciprocal of the rounded decode factor; a pairwise error
tree; dequant (s * g) * e2m1 as the stated convention requires). These tests
restate each step with numpy fp32 operations and torch's E4M3 cast, then
search for inputs where a different order would give a different byte, so
that a change of order in the oracle cannot pass unnoticed."""
import numpy as np
import torch

import workloads as W

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
GRID = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
f32 = np.float32


def e4m3_rne(x):
    """torch's RNE cast to float8_e4m3fn (x in [0, 448])."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e2m1_rne(v):
    """Nearest grid index (ties to even), saturating; sign bit from v."""
    a = np.abs(v).astype(np.float64)
    d = np.abs(a[..., None] - GRID.astype(np.float64))
    m = d.min(-1, keepdims=True)
    cand = d == m
    k = np.where(cand[..., 0:1].any(-1), 0, 0)
    # lowest even index among the minima, else the single minimum
    idx = np.arange(8)
    even_hit = cand & (idx % 2 == 0)
    k = np.where(even_hit.any(-1), np.argmax(even_hit, -1), np.argmax(cand, -1))
    k = np.where(a >= 6, 7, k)
    return (np.signbit(v).astype(np.int64) * 8 + k).astype(np.uint8)


def signed_grid(codes):
    v = GRID[codes & 7]
    return np.where(codes & 8, -v, v).astype(np.float32)


def candidate_np(x, g, C, clamp):
    """x [N,16] fp32, g [N] fp32 -> scale bytes, codes, dec (R1, R2, R3)."""
    amax = np.max(np.abs(x), axis=1)
    t = (f32(C) * g).astype(np.float32)
    sf = (amax / t).astype(np.float32)
    s = e4m3_rne(np.minimum(sf, f32(clamp)))
    dec = (E4M3[s].astype(np.float32) * g).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(dec == 0, f32(0), (f32(1) / dec)).astype(np.float32)
    v = (x * inv[:, None]).astype(np.float32)
    return s, e2m1_rne(v), dec


def tree_error(x, codes, dec, mode):
    deq = (dec[:, None] * signed_grid(codes)).astype(np.float32)
    d = (x - deq).astype(np.float32)
    t = (d * d).astype(np.float32) if mode == 0 else np.abs(d)
    while t.shape[1] > 1:
        t = (t[:, 0::2] + t[:, 1::2]).astype(np.float32)
    return t[:, 0]


def seq_error(x, codes, dec, mode):
    deq = (dec[:, None] * signed_grid(codes)).astype(np.float32)
    d = (x - deq).astype(np.float32)
    t = (d * d).astype(np.float32) if mode == 0 else np.abs(d)
    acc = np.zeros(x.shape[0], np.float32)
    for i in range(16):
        acc = (acc + t[:, i]).astype(np.float32)
    return acc


def _oracle_blocks(orc, x, g, recipe):
    out = []
    for i in range(x.shape[0]):
        out.append(orc.quantize_block(x[i], float(g[i]), recipe))
    s = np.array([o[1] for o in out], np.uint8)
    c = np.stack([o[0] for o in out])
    return s, c, np.array([o[2] for o in out], np.float32), np.array([o[3] for o in out], np.float32), \
        np.array([o[4] for o in out])


def test_block_scale_order_amax_over_Cg(orc):
    """R1: sf = amax / fp32(C*g). Inputs where (amax/C)/g would round to a
    different E4M3 byte."""
    rng = np.random.default_rng(61)
    # amax values within a few ulps of C*g times an E4M3 midpoint
    c = rng.integers(0x08, 0x7D, 100000)
    mid = ((E4M3[c] + E4M3[c + 1]) / 2).astype(np.float32)
    g = rng.uniform(1e-4, 1e-1, c.size).astype(np.float32)
    amax = (mid * (f32(6) * g).astype(np.float32)).astype(np.float32)
    amax = (amax.view(np.int32) + rng.integers(-3, 4, c.size).astype(np.int32)).view(np.float32)
    r1 = e4m3_rne(np.minimum((amax / (f32(6) * g).astype(np.float32)).astype(np.float32), f32(448)))
    alt = e4m3_rne(np.minimum(((amax / f32(6)).astype(np.float32) / g).astype(np.float32), f32(448)))
    idx = np.nonzero(r1 != alt)[0][:200]
    assert idx.size >= 20
    x = np.zeros((idx.size, 16), np.float32)
    x[:, 5] = amax[idx]
    s, *_ = _oracle_blocks(orc, x, g[idx], orc.STANDARD)
    assert np.array_equal(s, r1[idx])


def test_element_encode_through_rounded_reciprocal(orc):
    """R2: v = x * fp32(1 / fp32(E4M3(s) * g)). Inputs whose exact x / dec
    sits on an E2M1 midpoint, where x / dec and x * inv round differently."""
    rng = np.random.default_rng(62)
    n = 200000
    s = rng.integers(0x20, 0x70, n).astype(np.uint8)
    g = rng.uniform(1e-3, 1e-2, n).astype(np.float32)
    dec = (E4M3[s].astype(np.float32) * g).astype(np.float32)
    inv = (f32(1) / dec).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    mid = mids[rng.integers(0, 7, n)]
    x = (mid * dec).astype(np.float32)                    # x / dec is (nearly) a midpoint
    by_recip = e2m1_rne((x * inv).astype(np.float32))
    by_div = e2m1_rne((x / dec).astype(np.float32))
    idx = np.nonzero(by_recip != by_div)[0][:300]
    assert idx.size >= 20
    # a block whose amax element sets the same scale byte s
    blk = np.zeros((idx.size, 16), np.float32)
    blk[:, 0] = (f32(6) * E4M3[s[idx]].astype(np.float32) * g[idx]).astype(np.float32)
    blk[:, 3] = x[idx]
    s_np, c_np, _ = candidate_np(blk, g[idx], 6, 448)
    keep = s_np == s[idx]
    assert keep.sum() >= 10
    s_or, c_or, *_ = _oracle_blocks(orc, blk[keep], g[idx][keep], orc.STANDARD)
    assert np.array_equal(s_or, s_np[keep])
    assert np.array_equal(c_or, c_np[keep])


def test_four_over_six_errors_and_choice_bit_exact(orc):
    """R4, R5: both candidates' fp32 errors (pairwise tree) and the choice
    equal the numpy restatement bit for bit, over random blocks and over any
    blocks where a sequential sum would have chosen differently."""
    rng = np.random.default_rng(63)
    n = 60000
    x = rng.standard_t(3, (n, 16)).astype(np.float32)
    x[rng.random(n) < 0.3, rng.integers(0, 16)] *= 20
    x = W.bits_to_f32(W.f32_to_bits(x, True), True)
    g = (np.max(np.abs(x), 1) / f32(1536) * rng.uniform(1, 4, n).astype(np.float32)).astype(np.float32)
    for mode in (0, 1):
        s6, c6, d6 = candidate_np(x, g, 6, 256)
        s4, c4, d4 = candidate_np(x, g, 4, 448)
        e6, e4 = tree_error(x, c6, d6, mode), tree_error(x, c4, d4, mode)
        q6, q4 = seq_error(x, c6, d6, mode), seq_error(x, c4, d4, mode)
        flip = np.nonzero((e4 < e6) != (q4 < q6))[0]
        pick = np.concatenate([np.arange(800), flip[:400]])
        # the errors themselves are compared bit for bit, so a change of
        # summation order shows even where it flips no choice
        assert np.any(e6[:800] != q6[:800]) or np.any(e4[:800] != q4[:800])
        s_or, c_or, e6_or, e4_or, ch_or = _oracle_blocks(orc, x[pick], g[pick], orc.four_over_six(mode))
        assert np.array_equal(e6_or, e6[pick]) and np.array_equal(e4_or, e4[pick])
        take4 = e4[pick] < e6[pick]
        assert np.array_equal(ch_or, take4)
        assert np.array_equal(s_or, np.where(take4, s4[pick], s6[pick]))
        assert np.array_equal(c_or, np.where(take4[:, None], c4[pick], c6[pick]))


def test_dequant_multiply_order_scale_times_global_first(orc):
    """R7: y = fp32(fp32(E4M3(s) * g) * e2m1), then one RNE to 16 bits.
    g is built so that some products land next to a 16-bit rounding midpoint,
    where fp32(fp32(e2m1 * g) * E4M3(s)) gives a different 16-bit output."""
    rng = np.random.default_rng(64)
    s_all = np.arange(0x08, 0x7F, dtype=np.uint8)
    e = np.array([1.5, 3.0, 6.0], np.float32)
    codes = np.arange(16, dtype=np.uint8)
    for is_bf16 in (True, False):
        tdt = torch.bfloat16 if is_bf16 else torch.float16
        found = 0
        for trial in range(2000):
            s0 = int(rng.choice(s_all))
            e0 = f32(rng.choice(e))
            # a 16-bit midpoint m in [0.01, 10): the 16-bit value's bits plus half an ulp
            b = torch.tensor([float(rng.uniform(0.01, 10))]).to(tdt).float().numpy()[0]
            ulp = np.spacing(b.astype(np.float32)) * (2 ** 16 if is_bf16 else 2 ** 13)
            m = f32(b + ulp / 2)
            g0 = f32(m / (f32(E4M3[s0]) * e0))
            g = (np.array([g0], np.float32).view(np.int32) + rng.integers(-4, 5)).view(np.float32)[0]
            y1 = ((E4M3[s_all].astype(np.float32) * g).astype(np.float32)[:, None] * e).astype(np.float32)
            y2 = ((e * g).astype(np.float32)[None, :] * E4M3[s_all].astype(np.float32)[:, None]).astype(np.float32)
            h1 = torch.from_numpy(y1).to(tdt).view(torch.int16).numpy()
            h2 = torch.from_numpy(y2).to(tdt).view(torch.int16).numpy()
            if not np.any(h1 != h2):
                continue
            # one token per scale byte: a 16-element block holding all 16 codes
            ps, H, D = len(s_all), 1, 16
            cache = W.make_cache(rng, 1, ps, H, D, W.NHD, fill="zero")
            cache.k_data[0] = np.tile(codes[0::2] | (codes[1::2] << 4), ps)
            cache.v_data[0] = cache.k_data[0]
            cache.k_sf[0] = s_all
            cache.v_sf[0] = s_all
            ok = np.zeros((1, ps, 1, 16), np.uint16)
            ov = ok.copy()
            orc.dequantize_paged(cache, np.zeros((1, 1), np.int32), np.array([ps], np.int32),
                                 float(g), float(g), ok, ov, is_bf16)
            yy = (E4M3[s_all].astype(np.float32) * g).astype(np.float32)[:, None] * signed_grid(codes)[None, :]
            want = torch.from_numpy(yy.astype(np.float32)).to(tdt).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(ok[0, :, 0, :], want)
            found += int(np.sum(h1 != h2))
            if found >= 10:
                break
        assert found >= 10
