"""Pins for the oracle's decode attention over the paged NVFP4 cache (the
dequantized values e2m1 * block_scale * global_scale, whose global scales the
flashinfer.quantization.nvfp4_kv_dequantize_paged page names as inputs of the
NVFP4 attention kernels).

The reference here is torch's scaled_dot_product_attention in float64 on K
and V decoded independently of the oracle (E4M3 values from torch's
float8_e4m3fn decode, E2M1 values from the grid fixture), plus closed forms:
equal keys give the mean of the values, an empty request gives zeros, a
dominant key gives its value, and scores far beyond exp's range still give
finite outputs."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = json.load(open(os.path.join(GOLDEN, "e2m1_grid.json")))["magnitudes"]
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E2M1 = np.array(GRID + [-v for v in GRID], np.float64)
E2M1[8] = -0.0


def decode_tensor(cache, kv, block_tables, seq_lens, g):
    """exact K or V [B, T, H, D] (float64) of every request, from the bytes"""
    B, ps, H, D = len(seq_lens), cache.page_size, cache.num_heads, cache.head_dim
    T = int(max(seq_lens)) if len(seq_lens) else 0
    data = cache.v_data if kv else cache.k_data
    sf = cache.v_sf if kv else cache.k_sf
    out = np.zeros((B, T, H, D))
    for b in range(B):
        for t in range(int(seq_lens[b])):
            page, slot = block_tables[b, t // ps], t % ps
            for h in range(H):
                row = slot * H + h if cache.layout == W.NHD else h * ps + slot
                codes = data[page, row * (D // 2):(row + 1) * (D // 2)]
                c = np.stack([codes & 15, codes >> 4], 1).reshape(-1)
                s = sf[page, row * (D // 16):(row + 1) * (D // 16)]
                out[b, t, h] = E2M1[c] * np.repeat(E4M3[s], 16) * g
    return out


def sdpa_reference(q, K, V, seq_lens, sm_scale):
    B, Hq, D = q.shape
    H = K.shape[2]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        k = torch.from_numpy(K[b, :n]).permute(1, 0, 2).repeat_interleave(Hq // H, 0)     # [Hq, n, D]
        v = torch.from_numpy(V[b, :n]).permute(1, 0, 2).repeat_interleave(Hq // H, 0)
        qq = torch.from_numpy(q[b]).unsqueeze(1)                                           # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=sm_scale)
        out[b] = o[:, 0].numpy()
    return out


def random_case(rng, layout, ps, H, Hq, D, lens):
    B = len(lens)
    maxp = int(max((l + ps - 1) // ps for l in lens)) or 1
    P = B * maxp + 2
    cache = W.make_cache(rng, P, ps, H, D, layout, data_pad=16)
    for a in (cache.k_sf, cache.v_sf):
        a[...] = W.scale_bytes(rng, a.shape, hi=0x70)
    bt = rng.permutation(P)[:B * maxp].reshape(B, maxp).astype(np.int32)
    qf = W.normal_rows(rng, (B, Hq, D))
    return cache, bt, np.array(lens, np.int32), qf


@pytest.mark.parametrize("layout", [W.NHD, W.HND])
@pytest.mark.parametrize("bf16", [True, False])
def test_attention_vs_torch_sdpa(orc, layout, bf16):
    rng = np.random.default_rng(500 + layout + 2 * bf16)
    ps, H, Hq, D = 8, 2, 8, 32
    cache, bt, lens, qf = random_case(rng, layout, ps, H, Hq, D, [1, 17, 40, 8, 0])
    qb = W.f32_to_bits(qf, bf16)
    q64 = W.bits_to_f32(qb, bf16).astype(np.float64)
    gk, gv, sm = (float(np.float32(v)) for v in (0.0123, 3.5, 0.17))   # the scales are fp32 arguments
    want = sdpa_reference(q64, decode_tensor(cache, 0, bt, lens, gk), decode_tensor(cache, 1, bt, lens, gv), lens, sm)
    got = orc.decode_attention(cache, qb, bf16, bt, lens, gk, gv, sm, threads=4)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def test_attention_closed_forms(orc):
    rng = np.random.default_rng(510)
    ps, H, Hq, D = 4, 1, 2, 16
    cache, bt, lens, qf = random_case(rng, W.HND, ps, H, Hq, D, [7, 0, 5])
    # request 0: every key identical -> the mean of its values
    for p in bt[0, :2]:
        cache.k_data[p, :ps * D // 2] = np.tile(cache.k_data[bt[0, 0], :D // 2], ps)
        cache.k_sf[p, :ps * D // 16] = np.tile(cache.k_sf[bt[0, 0], :D // 16], ps)
    qb = W.f32_to_bits(qf, True)
    gv = 2.0
    out = orc.decode_attention(cache, qb, True, bt, lens, 1.0, gv, 0.5)
    V = decode_tensor(cache, 1, bt, lens, gv)
    assert np.allclose(out[0], V[0, :7, 0].mean(0)[None, :], rtol=1e-12, atol=1e-14)
    # request 1: empty -> zeros
    assert np.all(out[1] == 0.0)
    # sm_scale 0: every request is the plain mean of its values
    out0 = orc.decode_attention(cache, qb, True, bt, lens, 1.0, gv, 0.0)
    assert np.allclose(out0[2], V[2, :5, 0].mean(0)[None, :], rtol=1e-12, atol=1e-14)


def test_attention_dominant_key_and_huge_scores(orc):
    """A query that matches one key by a margin far beyond exp's range picks
    that key's value (the max-subtracted softmax stays finite)."""
    rng = np.random.default_rng(520)
    ps, H, Hq, D = 16, 1, 1, 64
    cache, bt, lens, _ = random_case(rng, W.NHD, ps, H, Hq, D, [30])
    K = decode_tensor(cache, 0, bt, lens, 1.0)
    V = decode_tensor(cache, 1, bt, lens, 1.0)
    star = 13
    q = np.sign(K[0, star, 0]).astype(np.float32)                       # aligned with key 13 ...
    scores = K[0, :30, 0] @ q.astype(np.float64)
    assert np.argmax(scores) == star and np.sort(scores)[-1] > np.sort(scores)[-2]
    qb = W.f32_to_bits(q[None, None, :], True)
    out = orc.decode_attention(cache, qb, True, bt, lens, 1.0, 1.0, 1e4)   # ... with scores ~1e4 apart
    assert np.all(np.isfinite(out))
    assert np.allclose(out[0, 0], V[0, star, 0], rtol=0, atol=1e-12 * np.abs(V).max())
