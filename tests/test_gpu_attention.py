"""GPU parity of kv_decode_attention (NVFP4 paged decode attention) against
the oracle's fp64 attention over the exactly dequantized cache.

Tolerance, from the kernel's arithmetic: K and V are exact in fp16, a bf16
query row moves into fp16 exactly up to components 2^38 below its largest,
and scores, exponentials and sums are fp32, so the error is dominated by two
roundings: the softmax probabilities to fp16 for the value product
(relative 2^-11 for each p, below 2^-11 * max|V| in the output) and the
output to q's type (relative 2^-9 in bf16, 2^-11 in fp16). The bound used is
|gpu - exact| <= 2u (max|V| + |exact|) with u = 2^-9 (bf16) or 2^-12 (fp16),
max|V| over the request's values of that kv head."""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DeviceCache, bits_tensor, i32, oracle_threads, tensor_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_paged_amd as K
    return K


def say(*a):
    print(*a, flush=True)


def quantized_cache(orc, rng, P, ps, H, D, layout, spread=1.0, sf_pad=0):
    """a pool of P pages quantized by the oracle from N(0, spread^2) K and V"""
    shape = (P, ps, H, D) if layout == W.NHD else (P, H, ps, D)
    k = W.f32_to_bits(W.normal_rows(rng, shape) * np.float32(spread), True)
    v = W.f32_to_bits(W.normal_rows(rng, shape), True)
    gk, gv = orc.global_scale(k, True), orc.global_scale(v, True)
    pad = (-(ps * H * D // 2)) % 16 + 16
    cache = W.make_cache(rng, P, ps, H, D, layout, data_pad=pad, sf_pad=sf_pad, fill="zero")
    orc.quantize_paged_cache(cache, k, v, True, gk, gv, v_sf_interleaved=False, threads=oracle_threads())
    return cache, gk, gv


def max_abs_v(cache, bt, lens, gv, b, h):
    """max |V| of request b, kv head h (exact decode, for the tolerance)"""
    E4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ps, H, D = cache.page_size, cache.num_heads, cache.head_dim
    m = 0.0
    for t in range(int(lens[b])):
        page, slot = bt[b, t // ps], t % ps
        row = slot * H + h if cache.layout == W.NHD else h * ps + slot
        s = cache.v_sf[page, row * (D // 16):(row + 1) * (D // 16)]
        m = max(m, 6.0 * float(E4[s].max()) * gv)
    return m


def run_case(K, orc, seed, layout, ps, H, G, lens, bf16, spread=1.0, sm=None, check=None, q_exp=None, D=128,
             sf_pad=0):
    rng = np.random.default_rng(seed)
    B = len(lens)
    maxp = max(1, max((l + ps - 1) // ps for l in lens))
    P = B * maxp + 3
    cache, gk, gv = quantized_cache(orc, rng, P, ps, H, D, layout, spread, sf_pad)
    bt = rng.permutation(P)[:B * maxp].reshape(B, maxp).astype(np.int32)
    lens = np.array(lens, np.int32)
    Hq = H * G
    qf = W.normal_rows(rng, (B, Hq, D))
    if q_exp is not None:                         # power-of-two magnitudes per row (or element)
        qf = (qf * np.exp2(q_exp.astype(np.float64))).astype(np.float32)
    q = W.f32_to_bits(qf, bf16)
    sm = float(np.float32(1.0 / np.sqrt(D) if sm is None else sm))
    say(f"attention layout={layout} ps={ps} H={H} G={G} D={D} bf16={bf16} lens={list(lens)[:8]}")
    dev = DeviceCache(cache)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16 if bf16 else torch.float16, device="cuda")
    ws = torch.full((K.kv_decode_attention_workspace_size(B, H, Hq, maxp, ps, D),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    K.kv_decode_attention(dev.cache, bits_tensor(q, bf16), i32(bt), i32(lens), torch.tensor([gk], device="cuda"),
                          torch.tensor([gv], device="cuda"), sm, out, ws)
    got = out.float().cpu().numpy().astype(np.float64)
    sel = range(B) if check is None else check
    bsel = np.array(list(sel))
    want = orc.decode_attention(cache, q[bsel], bf16, bt[bsel], lens[bsel], gk, gv, sm, threads=oracle_threads())
    u = 2.0 ** -9 if bf16 else 2.0 ** -12
    for k_, b in enumerate(bsel):
        for hq in range(Hq):
            if lens[b] == 0:
                assert np.all(got[b, hq] == 0.0), (b, hq)
                continue
            vmax = max_abs_v(cache, bt, lens, gv, b, hq // G)
            err = np.abs(got[b, hq] - want[k_, hq])
            tol = 2 * u * (vmax + np.abs(want[k_, hq]))
            assert np.all(err <= tol), (b, hq, float(err.max()), float(tol.min()))
    return got


@pytest.mark.parametrize("layout", [W.NHD, W.HND])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_attention_parity(K, orc, layout, bf16, G):
    lens = [1, 0, 31, 32, 33, 100, 257, 16, 5, 64]
    run_case(K, orc, zlib.crc32(repr((layout, bf16, G)).encode()), layout, 16, 2, G, lens, bf16)


@pytest.mark.parametrize("D,sf_pad", [(128, 2), (128, 4), (64, 1), (64, 4), (256, 4), (256, 8)])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("layout", [W.HND, W.NHD])
def test_attention_scale_page_alignment(K, orc, D, sf_pad, bf16, layout):
    """pools read directly (HND at every head_dim, NHD at head_dim 64 and
    256; NHD at 128 is staged through LDS) take their scales as aligned
    dwords when every scale page starts 4-byte aligned, and byte by byte
    otherwise (a page stride 1 or 2 past a multiple of 4): all must give the
    same attention"""
    seed = 690 + sf_pad + bf16 + (0 if D == 128 else D) + 7 * layout
    run_case(K, orc, seed, layout, 16, 2, 4, [1, 31, 300, 77], bf16, sf_pad=sf_pad, D=D)


@pytest.mark.parametrize("ps", [1, 5, 8, 32, 64])
def test_attention_page_sizes(K, orc, ps):
    run_case(K, orc, 600 + ps, W.HND, ps, 3, 3, [7, 70, 300, 1], True)


# head_dim 64 and 256: the lane maps scale with D (D / 32 score MFMAs per
# 16 tokens, D / 16 output MFMAs); NHD pools read directly at these sizes
@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("layout", [W.NHD, W.HND])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_attention_head_dims(K, orc, D, layout, bf16, G):
    lens = [1, 0, 31, 32, 33, 100, 257, 16, 5, 64]
    run_case(K, orc, zlib.crc32(repr(("hd", D, layout, bf16, G)).encode()), layout, 16, 2, G, lens, bf16, D=D)


@pytest.mark.parametrize("D,G,H", [(128, 17, 2), (128, 32, 1), (64, 40, 2), (256, 24, 1)])
@pytest.mark.parametrize("layout", [W.NHD, W.HND])
def test_attention_many_query_heads_per_kv_head(K, orc, D, G, H, layout):
    """more query heads per kv head than the MFMA's 16 columns: passes of 16"""
    lens = [1, 0, 31, 300, 33, 257]
    run_case(K, orc, zlib.crc32(repr(("mq", D, G, H, layout)).encode()), layout, 16, H, G, lens, True, D=D)


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("ps", [5, 32])
def test_attention_head_dims_page_sizes(K, orc, D, ps):
    """page sizes that are not multiples of 16 take the per-token loader"""
    run_case(K, orc, 700 + ps + D, W.NHD if ps == 5 else W.HND, ps, 3, 2, [7, 70, 600, 1], True, D=D)


@pytest.mark.parametrize("D", [64, 256])
def test_attention_head_dims_long_requests(K, orc, D):
    """many 256-token splits per request, merged by the second kernel"""
    run_case(K, orc, 800 + D, W.HND, 16, 2, 4, [4099, 1000, 2047, 3], False, D=D)


@pytest.mark.parametrize("D", [128, 64, 256])
def test_attention_peaked_scores(K, orc, D):
    """large score spreads (keys 8x wider, sm_scale 1): near one-hot softmax,
    whose running maximum jumps by far more than the rescale slack from tile
    to tile, so every output channel's rescale is exercised"""
    run_case(K, orc, 610 if D == 128 else 610 + D, W.NHD, 16, 2, 4, [200, 45, 513], True, spread=8.0, sm=1.0, D=D)


def test_attention_long_requests_many_tiles(K, orc):
    """more tiles than waves (8 x 32 tokens), ragged tails"""
    run_case(K, orc, 620, W.HND, 16, 1, 8, [2049, 1500, 4099], True)


def test_attention_decode_workload_full_size(K, orc):
    """the decode workload's shape: 64 requests, lengths U{1..4096}+1, page
    16, 8 kv heads, 4 query heads each, NHD; the oracle checks 4 requests"""
    rng = np.random.default_rng(1002)
    old, new_len, *_ = W.decode_append_tables(rng, 64, 4096, 20000, 16)
    order = np.argsort(new_len)
    check = sorted({int(order[0]), int(order[31]), int(order[-1]), 7})
    run_case(K, orc, 630, W.NHD, 16, 8, 4, [int(x) for x in new_len], True, check=check)


@pytest.mark.parametrize("D", [128, 64, 256])
def test_attention_query_magnitudes(K, orc, D):
    """bf16 query rows from 2^-60 to 2^60 and rows spanning 2^-50..2^0 inside:
    the power-of-two move into fp16 must keep every score (the row's largest
    magnitude is found over all D / 4 channels of each lane group)"""
    lens = [40, 300, 17, 129]
    B, H, G = len(lens), 2, 4
    rng = np.random.default_rng(640 + D)
    row = rng.choice([-60, -30, -12, 0, 12, 30, 60], size=(B, H * G, 1))
    wide = rng.uniform(-50, 0, size=(B, H * G, D)) * (rng.random((B, H * G, 1)) < 0.5)
    run_case(K, orc, 641 + D, W.NHD, 16, H, G, lens, True, q_exp=np.floor(row + wide), D=D)


@pytest.mark.parametrize("case", range(96))
def test_attention_random_shapes(K, orc, case):
    """seeded draws over head_dim, layout, page size (any-page, direct and
    staged loaders), query dtype, kv heads, query heads per kv head (one or
    several passes), lengths and score spread"""
    rng = np.random.default_rng(7000 + case)
    D = int(rng.choice([64, 128, 256]))
    layout = W.NHD if rng.random() < 0.5 else W.HND
    ps = int(rng.choice([1, 4, 5, 8, 16, 32, 48]))
    bf16 = bool(rng.random() < 0.5)
    H = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 5, 8, 16, 17]))
    lens = [int(x) for x in rng.integers(0, 600, size=int(rng.integers(1, 6)))]
    spread = float(rng.choice([1.0, 4.0]))
    run_case(K, orc, 7100 + case, layout, ps, H, G, lens, bf16, spread=spread, D=D)


@pytest.mark.parametrize("D,G", [(128, 2), (256, 16)])
def test_attention_batch_beyond_one_launch(K, orc, D, G):
    """more requests than one launch's split table holds (2048): the requests
    go out in launches of 2048, each with its own slice of the workspace;
    head_dim 256 with 16 query heads is the largest LDS use per workgroup"""
    rng = np.random.default_rng(650)
    lens = [int(x) for x in rng.integers(0, 40, size=2100)]
    check = [0, 1, 2046, 2047, 2048, 2049, 2099]
    run_case(K, orc, 651 if D == 128 else 652, W.HND, 16, 1, G, lens, True, check=check, D=D)


@pytest.mark.parametrize("D", [128, 64, 256])
@pytest.mark.parametrize("sm", [0.0, -0.25, 3.0])
def test_attention_sm_scale_edge_values(K, orc, sm, D):
    """sm_scale 0 (every weight equal: the plain mean of V), a negative scale
    (the softmax of reversed scores) and a large one, on fp16 and bf16"""
    for bf16 in (True, False):
        seed = 660 + int(sm * 8) + bf16 + (0 if D == 128 else D)
        run_case(K, orc, seed, W.HND, 16, 2, 4, [1, 47, 260], bf16, sm=sm, D=D)


def test_attention_split_boundaries(K, orc):
    """lengths at and next to the 256-token split and 64-token wave edges"""
    run_case(K, orc, 670, W.NHD, 16, 2, 4, [256, 512, 768, 255, 511, 64, 65, 192, 193], True)


def test_attention_lengths_outside_the_table(K, orc):
    """seq_lens past what a table row addresses (bt_cols * page_size) or
    negative are values the host does not check: the kernels cut them to the
    row (and to 0), so every read stays in the caller's buffers and the other
    requests' outputs are exactly those of a call with in-range lengths"""
    rng = np.random.default_rng(680)
    ps, H, G, D, maxp = 16, 2, 4, 128, 5
    B = 6
    P = B * maxp + 3
    cache, gk, gv = quantized_cache(orc, rng, P, ps, H, D, W.NHD)
    bt = rng.permutation(P)[:B * maxp].reshape(B, maxp).astype(np.int32)
    good = np.array([70, 80, 33, 1, 80, 17], np.int32)
    bad = good.copy()
    bad[1] = 100_000                       # past the row's 80 tokens (and the workspace's splits)
    bad[3] = -7
    bad[4] = 81
    q = W.f32_to_bits(W.normal_rows(rng, (B, H * G, D)), True)
    dev = DeviceCache(cache)
    ws_bytes = K.kv_decode_attention_workspace_size(B, H, H * G, maxp, ps)
    outs = []
    for lens in (good, bad):
        say(f"attention lengths outside the table: {list(lens)}")
        out = torch.full((B, H * G, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
        K.kv_decode_attention(dev.cache, bits_tensor(q, True), i32(bt), i32(lens), torch.tensor([gk], device="cuda"),
                              torch.tensor([gv], device="cuda"), 1.0 / np.sqrt(D), out, ws)
        outs.append(tensor_bits(out))
    want_cut = good.copy()
    want_cut[3] = 0                         # the negative length counts as 0
    assert np.array_equal(outs[1][[0, 2, 5]], outs[0][[0, 2, 5]])
    assert np.array_equal(outs[1][1], outs[0][1]) and np.array_equal(outs[1][4], outs[0][4])
    assert np.all(outs[1][3] == 0)
    sel = np.array([0, 1, 2, 4, 5])
    want = orc.decode_attention(cache, q[sel], True, bt[sel], want_cut[sel], gk, gv,
                                float(np.float32(1.0 / np.sqrt(D))), threads=oracle_threads())
    got = outs[1].view(np.int16).view(np.uint16).astype(np.uint32) << 16
    got = got.view(np.float32).astype(np.float64)[sel]
    for k_, b in enumerate(sel):
        for hq in range(H * G):
            vmax = max_abs_v(cache, bt, want_cut, gv, b, hq // G)
            err = np.abs(got[k_, hq] - want[k_, hq])
            assert np.all(err <= 2 * 2.0 ** -9 * (vmax + np.abs(want[k_, hq]))), (b, hq)
