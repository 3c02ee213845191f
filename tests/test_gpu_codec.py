"""GPU parity of the contiguous NVFP4 codec (kv_quantize / kv_dequantize) and
the whole-pool quantizer (kv_quantize_paged_cache) against the CPU oracle,
through the C ABI. Codes, scales and 16-bit outputs must match bit for bit;
bytes the calls must not write (page padding) keep their prior values."""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DeviceCache, bits_tensor, first_mismatch, i32, oracle_threads, tensor_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_paged_amd as K
    return K


def say(*a):
    print(*a, flush=True)


def recipes(K, orc):
    return {"standard": (None, orc.STANDARD, 448.0),
            "mse": (K.Recipe(256.0, K.KVFP4_ERR_MSE), orc.four_over_six(orc.MSE), 256.0),
            "mae": (K.Recipe(256.0, K.KVFP4_ERR_MAE), orc.four_over_six(orc.MAE), 256.0),
            "mse16": (K.Recipe(256.0, K.KVFP4_ERR_MSE, True), orc.four_over_six(orc.MSE, fast_math=True), 256.0),
            "mae16": (K.Recipe(256.0, K.KVFP4_ERR_MAE, True), orc.four_over_six(orc.MAE, fast_math=True), 256.0)}


def values(rng, shape, kind):
    if kind == "normal":
        return W.normal_rows(rng, shape) * np.float32(rng.uniform(0.01, 100))
    x = W.student_t_with_outliers(rng, shape, frac=0.01)
    blocks = x.reshape(-1, 16)
    sel = rng.integers(0, 8, blocks.shape[0])
    blocks[sel == 0] = 0.0
    blocks[sel == 1] = -0.0
    blocks[sel == 2] *= np.float32(1e-5)
    return x


def g_dev(g):
    return torch.tensor([g], dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (257, 128), (5, 7, 256), (2049, 1024)])
@pytest.mark.parametrize("recipe", ["standard", "mse", "mae", "mse16", "mae16"])
@pytest.mark.parametrize("bf16", [True, False])
def test_contiguous_quantize_parity(K, orc, shape, recipe, bf16):
    rng = np.random.default_rng(zlib.crc32(repr((shape, recipe, bf16)).encode()))
    say(f"contiguous quantize {shape} {recipe} bf16={bf16}")
    k_rec, o_rec, e4max = recipes(K, orc)[recipe]
    x = W.f32_to_bits(values(rng, shape, "student_t" if recipe != "standard" else "normal"), bf16)
    g = orc.global_scale(x, bf16, e4max)
    xd = bits_tensor(x, bf16)
    data = torch.full(shape[:-1] + (shape[-1] // 2,), 0xA5, dtype=torch.uint8, device="cuda")
    sc = torch.full(shape[:-1] + (shape[-1] // 16,), 0xA5, dtype=torch.uint8, device="cuda")
    K.kv_quantize(xd, g_dev(g), data, sc, k_rec)
    wc, ws = orc.quantize_contiguous(x, bf16, g, o_rec, threads=oracle_threads())
    gc, gs = data.cpu().numpy(), sc.cpu().numpy()
    assert np.array_equal(gs, ws), first_mismatch(gs, ws)
    assert np.array_equal(gc, wc), first_mismatch(gc, wc)


@pytest.mark.parametrize("rows,cols", [(1, 16), (2, 64), (1, 4096 * 8 * 2), (333, 160), (4099, 128)])
@pytest.mark.parametrize("bf16", [True, False])
def test_contiguous_dequantize_parity(K, orc, rows, cols, bf16):
    """every chunk of the last workgroup's ragged range is checked; the bytes
    after the output keep their sentinel"""
    rng = np.random.default_rng(rows * 7919 + cols + bf16)
    say(f"contiguous dequantize {rows}x{cols} bf16={bf16}")
    codes = np.frombuffer(rng.bytes(rows * cols // 2), np.uint8).reshape(rows, cols // 2)
    scales = W.scale_bytes(rng, (rows, cols // 16))
    for g in (float(np.float32(rng.uniform(1e-4, 10))), 1.0):
        dt = torch.bfloat16 if bf16 else torch.float16
        buf = torch.full((rows * cols + 64,), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(dt)
        out = buf[:rows * cols].view(rows, cols)
        K.kv_dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), g_dev(g), out)
        want = orc.dequantize_contiguous(codes, scales, g, bf16, threads=oracle_threads())
        got = tensor_bits(out)
        assert np.array_equal(got, want), first_mismatch(got, want)
        assert np.all(tensor_bits(buf[rows * cols:]) == W.SENTINEL_16)


def test_contiguous_round_trip_and_empty(K, orc):
    rng = np.random.default_rng(5)
    x = W.f32_to_bits(W.normal_rows(rng, (64, 8, 128)), True)
    g = orc.global_scale(x, True)
    d, s = K.nvfp4_kv_quantize(bits_tensor(x, True), g_dev(g))
    y = K.nvfp4_kv_dequantize(d, s, g_dev(g), torch.bfloat16)
    wc, ws = orc.quantize_contiguous(x, True, g)
    want = orc.dequantize_contiguous(wc, ws, g, True)
    assert np.array_equal(tensor_bits(y), want)
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    de, se = K.nvfp4_kv_quantize(e, g_dev(1.0))
    assert de.shape == (0, 32) and se.shape == (0, 4)
    assert K.nvfp4_kv_dequantize(de, se, g_dev(1.0)).shape == (0, 64)


def pool_case(rng, layout, ps, H, D, P, bf16, kind, pad):
    k = W.f32_to_bits(values(rng, (P, ps, H, D) if layout == W.NHD else (P, H, ps, D), kind), bf16)
    v = W.f32_to_bits(values(rng, k.shape, kind), bf16)
    cache = W.make_cache(rng, P, ps, H, D, layout, data_pad=pad, sf_pad=pad, fill="random")
    return k, v, cache


@pytest.mark.parametrize("layout,ps,H,D,P,inter,pad", [
    (W.HND, 16, 8, 128, 37, True, 0),
    (W.HND, 4, 1, 64, 9, True, 48),
    (W.HND, 32, 3, 48, 6, True, 16),
    (W.HND, 8, 2, 256, 5, False, 0),
    (W.NHD, 16, 8, 128, 11, False, 32),
    (W.NHD, 5, 3, 16, 7, False, 8),
])
@pytest.mark.parametrize("recipe", ["standard", "mse", "mae16"])
def test_pool_quantizer_parity(K, orc, layout, ps, H, D, P, inter, pad, recipe):
    rng = np.random.default_rng(ps * 131 + H * 7 + D + P + pad + (recipe == "mse"))
    say(f"pool quantize layout={layout} ps={ps} H={H} D={D} P={P} interleaved={inter} pad={pad} {recipe}")
    k_rec, o_rec, e4max = recipes(K, orc)[recipe]
    k, v, cache = pool_case(rng, layout, ps, H, D, P, True, "student_t", pad)
    gk, gv = orc.global_scale(k, True, e4max), orc.global_scale(v, True, e4max)
    dev = DeviceCache(cache)
    K.kv_quantize_paged_cache(dev.cache, bits_tensor(k, True), bits_tensor(v, True), g_dev(gk), g_dev(gv),
                              k_rec, inter)
    orc.quantize_paged_cache(cache, k, v, True, gk, gv, o_rec, inter, threads=oracle_threads())
    got = dev.to_host()
    for name, a, b in zip(("k_data", "v_data", "k_sf", "v_sf"), got.bases, cache.bases):
        assert np.array_equal(a, b), (name, first_mismatch(a, b))


def test_pool_quantizer_then_materialize(K, orc):
    """The pool quantizer's interleaved V scales are what the materializer
    reads: GPU quantize -> GPU materialize equals the oracle chain."""
    rng = np.random.default_rng(77)
    ps, H, D, P = 16, 4, 128, 20
    k, v, cache = pool_case(rng, W.HND, ps, H, D, P, True, "normal", 0)
    gk, gv = orc.global_scale(k, True), orc.global_scale(v, True)
    kd, vd, ks, vs, gkt, gvt = K.nvfp4_quantize_paged_kv_cache(bits_tensor(k, True), bits_tensor(v, True), "HND")
    assert gkt.item() == gk and gvt.item() == gv
    orc.quantize_paged_cache(cache, k, v, True, gk, gv, v_sf_interleaved=True)
    lens = np.array([5 * ps - 3, 1, 3 * ps], np.int32)
    need = (lens + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(need)]).astype(np.int32)
    bt = np.zeros((3, 5), np.int32)
    perm = rng.permutation(P)
    for b in range(3):
        bt[b, :need[b]] = perm[indptr[b]:indptr[b + 1]]
    n_out = int(indptr[-1]) + 1
    out, tab = K.nvfp4_kv_materialize_fp8(kd, vd, ks, vs, i32(bt), i32(lens), max_kv_len=5 * ps,
                                          kv_page_indptr=i32(indptr), num_pages=n_out - 1)
    want = np.full((n_out, 2, H, ps, D), 0x5A, np.uint8)
    wtab = np.zeros((3, 5), np.int32)
    orc.materialize_fp8(cache, bt, lens, indptr, want, wtab, shared=True, v_sf_interleaved=True)
    assert np.array_equal(out.view(torch.uint8).cpu().numpy(), want)
    assert np.array_equal(tab.cpu().numpy(), wtab)


@pytest.mark.parametrize("bf16", [True, False])
def test_contiguous_dequant_rounds_the_fp32_product(K, orc, bf16):
    from test_gpu_parity import double_rounding_scales
    rng = np.random.default_rng(4343 + bf16)
    s_all = np.arange(0x00, 0x7F, dtype=np.uint8)
    codes = np.arange(16, dtype=np.uint8)
    packed = np.tile(codes[0::2] | (codes[1::2] << 4), (len(s_all), 1)).astype(np.uint8)
    sc = s_all[:, None].copy()
    dt = torch.bfloat16 if bf16 else torch.float16
    for g in double_rounding_scales(rng, bf16):
        out = torch.empty((len(s_all), 16), dtype=dt, device="cuda")
        K.kv_dequantize(torch.from_numpy(packed).cuda(), torch.from_numpy(sc).cuda(), g_dev(g), out)
        want = orc.dequantize_contiguous(packed, sc, g, bf16)
        assert np.array_equal(tensor_bits(out), want), g
