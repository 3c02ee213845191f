"""GPU parity: the HIP path through the C ABI against the CPU oracle, on
seeded inputs that span many tiles and end in ragged tails. Codes, scales,
page tables, FP8 pages and dequantized 16-bit values must match bit for bit
(the dequant bar of 0 ulp holds because both sides use the same fp32 order).
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DeviceCache, bits_tensor, first_mismatch, i32, oracle_threads, same_bytes, tensor_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_paged_amd as K
    return K


def say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------- inputs
def align_pad(ps, H, D):
    """bytes that make a data page stride a multiple of 16 (the ABI's rule)"""
    return (-(ps * H * D // 2)) % 16


def append_values(rng, nnz, H, D, kind):
    if kind == "normal":
        x = W.head_scaled_normal(rng, nnz, W.head_scales(rng, H), D)
    elif kind == "student_t":
        x = W.student_t_with_outliers(rng, (nnz, H, D), frac=0.01)
    else:   # "special": zero, -0, tiny, huge, grid-valued blocks mixed with normal ones
        x = rng.standard_normal((nnz, H, D)).astype(np.float32)
        blocks = x.reshape(-1, 16)
        n = blocks.shape[0]
        sel = rng.integers(0, 6, n)
        blocks[sel == 0] = 0.0
        blocks[sel == 1] = -0.0
        blocks[sel == 2] *= 1e-6
        blocks[sel == 3] *= 3e3
        grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6], np.float32)
        g4 = grid[rng.integers(0, 16, (int((sel == 4).sum()), 16))]
        g4[:, 0] = 6.0
        blocks[sel == 4] = g4 * np.float32(0.125)
    return x


def append_case(seed, layout, ps, H, D, in_bf16, kind="normal", stacked=False, data_pad=0, sf_pad=0,
                B=6, pool=None):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 5 * ps, B)
    lens[0] = 1
    start = np.array([rng.integers(0, l) for l in lens])
    start[-1] = 0
    n_pages = int(((lens + ps - 1) // ps).sum())
    pool = pool or n_pages + 5
    perm = rng.permutation(pool)
    indices, indptr, last = W.csr_for_lengths(lens, ps, perm)
    data_pad += align_pad(ps, H, D)
    cache = W.make_cache(rng, pool, ps, H, D, layout, stacked=stacked, data_pad=data_pad, sf_pad=sf_pad)
    bi, pos = W.rows_for_positions(start, lens)
    order = rng.permutation(len(bi))                 # rows in any order
    bi, pos = bi[order], pos[order]
    nnz = len(bi)
    key = W.f32_to_bits(append_values(rng, nnz, H, D, kind), in_bf16)
    val = W.f32_to_bits(append_values(rng, nnz, H, D, kind) * np.float32(0.5), in_bf16)
    return cache, key, val, bi, pos, indices, indptr, last, lens


def run_append_both(K, orc, seed, layout, ps, H, D, in_bf16, recipe_o, recipe_k, kind="normal", stacked=False,
                    data_pad=0, sf_pad=0, scale_mult=1.0):
    cache, key, val, bi, pos, indices, indptr, last, _ = append_case(seed, layout, ps, H, D, in_bf16, kind,
                                                                     stacked, data_pad, sf_pad)
    emax = recipe_o.e4m3_max if recipe_o.four_over_six else 448.0
    gk = orc.global_scale(key, in_bf16, emax) * scale_mult
    gv = orc.global_scale(val, in_bf16, emax) * scale_mult
    gk, gv = float(np.float32(gk)), float(np.float32(gv))
    dev = DeviceCache(cache)
    host = cache.copy()
    say(f"append seed={seed} layout={layout} ps={ps} H={H} D={D} bf16={in_bf16} nnz={len(bi)} "
        f"recipe={recipe_o} kind={kind} stacked={stacked} pad={data_pad}/{sf_pad}")
    K.kv_quantize_append(dev.cache, bits_tensor(key, in_bf16), bits_tensor(val, in_bf16), i32(bi), i32(pos),
                         i32(indices), i32(indptr), i32(last), gk, gv, recipe_k)
    torch.cuda.synchronize()
    orc.quantize_append(host, key, val, in_bf16, bi, pos, indices, indptr, last, gk, gv, recipe_o,
                        threads=oracle_threads())
    got = dev.to_host()
    for name, a, b in zip(("k_data", "v_data", "k_sf", "v_sf"), (got.k_data, got.v_data, got.k_sf, got.v_sf),
                          (host.k_data, host.v_data, host.k_sf, host.v_sf)):
        assert np.array_equal(a, b), (name, first_mismatch(a, b))
    assert same_bytes(got, host)          # padding and untouched bytes too


def recipes(K, orc, name):
    """standard, mse, mae, and mse16 / mae16 (the error evaluated in fp16)"""
    if name == "standard":
        return orc.STANDARD, None
    mode = orc.MSE if name.startswith("mse") else orc.MAE
    fast = name.endswith("16")
    return (orc.four_over_six(mode, fast_math=fast),
            K.Recipe(256.0, K.KVFP4_ERR_MSE if mode == orc.MSE else K.KVFP4_ERR_MAE, err_use_fast_math=fast))


# --------------------------------------------------------------------------- append
@pytest.mark.parametrize("layout", [W.NHD, W.HND])
@pytest.mark.parametrize("recipe", ["standard", "mse", "mae", "mse16", "mae16"])
@pytest.mark.parametrize("in_bf16", [True, False])
def test_append_parity(K, orc, layout, recipe, in_bf16):
    ro, rk = recipes(K, orc, recipe)
    run_append_both(K, orc, 100 + layout * 10 + in_bf16, layout, 16, 8, 128, in_bf16, ro, rk, kind="student_t")


@pytest.mark.parametrize("geom", [(1, 1, 16), (4, 2, 64), (64, 4, 256), (8, 3, 80), (32, 32, 256), (16, 5, 48)])
@pytest.mark.parametrize("recipe", ["standard", "mse"])
def test_append_geometries(K, orc, geom, recipe):
    ps, H, D = geom
    ro, rk = recipes(K, orc, recipe)
    run_append_both(K, orc, 200 + ps + H + D, W.HND if D % 32 else W.NHD, ps, H, D, True, ro, rk)


@pytest.mark.parametrize("kind", ["special", "normal"])
@pytest.mark.parametrize("recipe", ["standard", "mse", "mae", "mse16", "mae16"])
def test_append_special_values_and_clamp(K, orc, kind, recipe):
    ro, rk = recipes(K, orc, recipe)
    # scale_mult < 1 pushes block scales past the clamps (mismatched global scale)
    for mult in (1.0, 0.1):
        run_append_both(K, orc, 300, W.NHD, 16, 4, 128, False, ro, rk, kind=kind, scale_mult=mult)


@pytest.mark.parametrize("stacked,data_pad,sf_pad", [(True, 0, 0), (False, 48, 5), (True, 32, 0)])
def test_append_stacked_and_padded(K, orc, stacked, data_pad, sf_pad):
    ro, rk = recipes(K, orc, "mae")
    run_append_both(K, orc, 400, W.HND, 16, 8, 128, True, ro, rk, stacked=stacked, data_pad=data_pad, sf_pad=sf_pad)
    ro, rk = recipes(K, orc, "standard")
    run_append_both(K, orc, 401, W.NHD, 16, 8, 128, True, ro, rk, stacked=stacked, data_pad=data_pad, sf_pad=sf_pad)


def test_append_empty_is_noop(K, orc):
    cache, key, val, bi, pos, indices, indptr, last, _ = append_case(5, W.NHD, 16, 2, 64, True)
    dev = DeviceCache(cache)
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    K.kv_quantize_append(dev.cache, e, e, i32(bi[:0]), i32(pos[:0]), i32(indices), i32(indptr), i32(last), 1.0, 1.0)
    torch.cuda.synchronize()
    assert same_bytes(dev.to_host(), cache)


@pytest.mark.parametrize("case", range(100))
def test_append_random_shapes(K, orc, case):
    """seeded draws over layout, page size, heads and head_dim (rows that fill
    whole wavefronts take the row kernel for the 4over6 recipes, the others
    the flat kernel), input dtype, recipe and value distribution"""
    rng = np.random.default_rng(8000 + case)
    layout = W.NHD if rng.random() < 0.5 else W.HND
    ps = int(rng.choice([1, 4, 5, 8, 16, 32, 64]))
    H = int(rng.choice([1, 2, 3, 4, 8, 16]))
    D = int(rng.choice([16, 32, 48, 64, 80, 128, 256]))
    in_bf16 = bool(rng.random() < 0.5)
    recipe = str(rng.choice(["standard", "mse", "mae", "mse16", "mae16"]))
    kind = str(rng.choice(["normal", "student_t", "special"]))
    ro, rk = recipes(K, orc, recipe)
    run_append_both(K, orc, 8100 + case, layout, ps, H, D, in_bf16, ro, rk, kind=kind)


# --------------------------------------------------------------------------- dequant
def dequant_case(seed, layout, ps, H, D, B=7, pool=60, neg_scales=True, stacked=False, data_pad=0):
    rng = np.random.default_rng(seed)
    data_pad += align_pad(ps, H, D)
    cache = W.make_cache(rng, pool, ps, H, D, layout, stacked=stacked, data_pad=data_pad)
    for a in (cache.k_sf, cache.v_sf):
        a[...] = rng.integers(0, 256 if neg_scales else 0x7F, a.shape, dtype=np.uint8)
        a[(a & 0x7F) == 0x7F] = 0x7E
    T = 3 * ps + 5
    lens = rng.integers(0, T + 6, B).astype(np.int32)
    lens[0] = 0
    lens[1] = T + 9                 # longer than max_seq_len: clamped
    lens[2] = 1
    cols = (T + ps - 1) // ps + 1
    bt = rng.integers(0, pool, (B, cols)).astype(np.int32)
    return cache, bt, lens, T


@pytest.mark.parametrize("layout", [W.NHD, W.HND])
@pytest.mark.parametrize("out_bf16", [True, False])
@pytest.mark.parametrize("bt64", [False, True])
@pytest.mark.parametrize("geom", [(16, 8, 128), (32, 2, 64), (5, 3, 48), (1, 16, 256), (64, 4, 128), (32, 8, 64)])
def test_dequant_parity(K, orc, layout, out_bf16, bt64, geom):
    ps, H, D = geom
    run_dequant(K, orc, 500 + layout + 2 * out_bf16 + 4 * bt64 + ps, layout, ps, H, D, out_bf16, bt64)


@pytest.mark.parametrize("case", range(100))
def test_dequant_random_shapes(K, orc, case):
    """seeded draws over layout, page size, heads and head_dim (HND shapes on
    both sides of the LDS-staged path's conditions), output dtype, table
    dtype and batch"""
    rng = np.random.default_rng(8200 + case)
    layout = W.NHD if rng.random() < 0.5 else W.HND
    ps = int(rng.choice([1, 4, 5, 8, 16, 32, 64]))
    H = int(rng.choice([1, 2, 3, 4, 8, 16]))
    D = int(rng.choice([16, 32, 48, 64, 128, 256]))
    run_dequant(K, orc, 8300 + case, layout, ps, H, D, bool(rng.random() < 0.5), bool(rng.random() < 0.5),
                B=int(rng.integers(3, 12)))


def run_dequant(K, orc, seed, layout, ps, H, D, out_bf16, bt64, B=7):
    cache, bt, lens, T = dequant_case(seed, layout, ps, H, D, B=B)
    bt = bt.astype(np.int64 if bt64 else np.int32)
    B = len(lens)
    gk, gv = 0.0137, 2.7e-4
    ok = np.full((B, T, H, D), W.SENTINEL_16, np.uint16)
    ov = ok.copy()
    orc.dequantize_paged(cache, bt, lens, gk, gv, ok, ov, out_bf16, threads=oracle_threads())
    dev = DeviceCache(cache)
    tdt = torch.bfloat16 if out_bf16 else torch.float16
    dk = torch.full((B, T, H, D), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(tdt)
    dv = dk.clone()
    say(f"dequant seed={seed} layout={layout} geom={(ps, H, D)} bf16={out_bf16} bt64={bt64} B={B} T={T}")
    K.kv_dequantize_paged(dev.cache, torch.from_numpy(bt).cuda(), i32(lens),
                          torch.tensor([gk], dtype=torch.float32, device="cuda"),
                          torch.tensor([gv], dtype=torch.float32, device="cuda"), dk, dv)
    torch.cuda.synchronize()
    gk_bits, gv_bits = tensor_bits(dk), tensor_bits(dv)
    assert np.array_equal(gk_bits, ok), first_mismatch(gk_bits, ok)
    assert np.array_equal(gv_bits, ov), first_mismatch(gv_bits, ov)


# HND geometries on both sides of the LDS-staged path's conditions (H * D / 8
# a power of two up to 1024 whose item tokens divide the page, H <= 64,
# D >= 32): staged (16,16,64) (64,4,32) (16,32,32) (8,64,128) (32,1,256)
# (16,2,256); read in place (8,2,256) (16,64,256) (24,4,64) (16,8,16)
@pytest.mark.parametrize("geom", [(16, 16, 64), (64, 4, 32), (16, 32, 32), (8, 64, 128), (32, 1, 256),
                                  (16, 2, 256), (8, 2, 256), (16, 64, 256), (24, 4, 64), (16, 8, 16)])
def test_dequant_hnd_geometry_sweep(K, orc, geom):
    ps, H, D = geom
    seed = 900 + ps + 3 * H + D
    cache, bt, lens, T = dequant_case(seed, W.HND, ps, H, D, B=5, pool=24)
    B = len(lens)
    ok = np.full((B, T, H, D), W.SENTINEL_16, np.uint16)
    ov = ok.copy()
    orc.dequantize_paged(cache, bt, lens, 0.0625, 3.0, ok, ov, True, threads=oracle_threads())
    dev = DeviceCache(cache)
    dk = torch.full((B, T, H, D), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dv = dk.clone()
    one = lambda v: torch.tensor([v], dtype=torch.float32, device="cuda")  # noqa: E731
    say(f"dequant HND sweep geom={geom} seed={seed} T={T}")
    K.kv_dequantize_paged(dev.cache, i32(bt), i32(lens), one(0.0625), one(3.0), dk, dv)
    torch.cuda.synchronize()
    gk_bits, gv_bits = tensor_bits(dk), tensor_bits(dv)
    assert np.array_equal(gk_bits, ok), first_mismatch(gk_bits, ok)
    assert np.array_equal(gv_bits, ov), first_mismatch(gv_bits, ov)


@pytest.mark.parametrize("geom", [(16, 4, 128), (32, 8, 128)])
def test_dequant_stacked_padded_and_empty(K, orc, geom):
    """HND page 16 x 4 heads (read head row by head row) and page 32 x 8
    heads (whole head runs staged through LDS, two items per page)"""
    ps, H, D = geom
    cache, bt, lens, T = dequant_case(77 + ps, W.HND, ps, H, D, stacked=True, data_pad=64)
    B = len(lens)
    ok = np.full((B, T, H, D), W.SENTINEL_16, np.uint16)
    ov = ok.copy()
    orc.dequantize_paged(cache, bt, lens, 0.5, 0.25, ok, ov, True)
    dev = DeviceCache(cache)
    dk = torch.full((B, T, H, D), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dv = dk.clone()
    one = lambda v: torch.tensor([v], dtype=torch.float32, device="cuda")  # noqa: E731
    K.kv_dequantize_paged(dev.cache, i32(bt), i32(lens), one(0.5), one(0.25), dk, dv)
    # all-zero lengths: nothing may be written
    zk = torch.full_like(dk.view(torch.int16), 7).view(torch.bfloat16)
    zv = zk.clone()
    K.kv_dequantize_paged(dev.cache, i32(bt), i32(np.zeros(B)), one(0.5), one(0.25), zk, zv)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(dk), ok) and np.array_equal(tensor_bits(dv), ov)
    assert np.all(tensor_bits(zk) == 7) and np.all(tensor_bits(zv) == 7)


@pytest.mark.parametrize("layout,geom", [(W.NHD, (16, 2, 64)), (W.HND, (8, 2, 256)), (W.NHD, (5, 3, 48))])
def test_dequant_many_requests(K, orc, layout, geom):
    """more requests than a wavefront has lanes (the kernel finds each
    work item's request with a scan over per-lane request groups), with empty,
    clamped and single-token requests among them"""
    ps, H, D = geom
    seed = 1300 + ps + H
    cache, bt, lens, T = dequant_case(seed, layout, ps, H, D, B=150, pool=40)
    rng = np.random.default_rng(seed + 1)
    lens[rng.integers(3, 150, 30)] = 0
    lens[rng.integers(3, 150, 10)] = T + 3
    B = len(lens)
    ok = np.full((B, T, H, D), W.SENTINEL_16, np.uint16)
    ov = ok.copy()
    orc.dequantize_paged(cache, bt, lens, 0.5, 0.125, ok, ov, True, threads=oracle_threads())
    dev = DeviceCache(cache)
    dk = torch.full((B, T, H, D), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dv = dk.clone()
    one = lambda v: torch.tensor([v], dtype=torch.float32, device="cuda")  # noqa: E731
    say(f"dequant many requests layout={layout} geom={geom} seed={seed} B={B} T={T}")
    K.kv_dequantize_paged(dev.cache, i32(bt), i32(lens), one(0.5), one(0.125), dk, dv)
    torch.cuda.synchronize()
    gk_bits, gv_bits = tensor_bits(dk), tensor_bits(dv)
    assert np.array_equal(gk_bits, ok), first_mismatch(gk_bits, ok)
    assert np.array_equal(gv_bits, ov), first_mismatch(gv_bits, ov)


def test_append_then_dequant_round_trip(K, orc):
    """Tiny round trip workload: append every token, then dequantize into
    sentinel-filled outputs; both stages bit-exact against the oracle."""
    wl = W.tiny_round_trip()
    gk, gv = orc.global_scale(wl.key, True), orc.global_scale(wl.value, True)
    host = wl.cache.copy()
    dev = DeviceCache(wl.cache)
    K.kv_quantize_append(dev.cache, bits_tensor(wl.key, True), bits_tensor(wl.value, True), i32(wl.batch_indices),
                         i32(wl.positions), i32(wl.kv_indices), i32(wl.kv_indptr), i32(wl.kv_last_page_len), gk, gv)
    orc.quantize_append(host, wl.key, wl.value, True, wl.batch_indices, wl.positions, wl.kv_indices, wl.kv_indptr,
                        wl.kv_last_page_len, gk, gv)
    B, T, H, D = 2, wl.max_seq_len, 2, 64
    dk = torch.full((B, T, H, D), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dv = dk.clone()
    K.kv_dequantize_paged(dev.cache, i32(wl.block_tables), i32(wl.seq_lens),
                          torch.tensor([gk], dtype=torch.float32, device="cuda"),
                          torch.tensor([gv], dtype=torch.float32, device="cuda"), dk, dv)
    torch.cuda.synchronize()
    assert same_bytes(dev.to_host(), host)
    ok = np.full((B, T, H, D), W.SENTINEL_16, np.uint16)
    ov = ok.copy()
    orc.dequantize_paged(host, wl.block_tables, wl.seq_lens, gk, gv, ok, ov, True)
    assert np.array_equal(tensor_bits(dk), ok) and np.array_equal(tensor_bits(dv), ov)
    assert np.all(ok[0, 5:] == W.SENTINEL_16)


# --------------------------------------------------------------------------- materialize
def mat_case(seed, shared, compact, ps=16, H=4, D=128, B=6, data_pad=256, extra_out=3):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 8 * ps, B)
    lens[0] = 0
    lens[1] = 1
    lens[2] = 3 * ps
    need = (lens + ps - 1) // ps
    P = int(need.sum()) + 4
    maxp = int(need.max()) + 2
    cache = W.make_cache(rng, P, ps, H, D, W.HND, data_pad=data_pad)
    for a in (cache.k_sf, cache.v_sf):
        a[...] = rng.integers(0, 256, a.shape, dtype=np.uint8)
        a[(a & 0x7F) == 0x7F] = 0x7E
    res = need if compact else need + rng.integers(0, 3, B)
    indptr = np.zeros(B + 1, np.int32)
    indptr[1:] = np.cumsum(res)
    if shared:
        bt = rng.integers(0, P, (B, maxp + 1)).astype(np.int32)
    else:
        bt = rng.integers(0, P, (B, 2, maxp + 1)).astype(np.int32)
    n_out = int(indptr[-1]) + 1 + extra_out
    return cache, bt, lens.astype(np.int32), indptr, maxp, n_out


@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("compact", [True, False])
@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("geom", [(16, 4, 128), (4, 2, 64), (32, 8, 256), (8, 1, 192), (12, 3, 128), (4, 2, 512)])
def test_materialize_parity(K, orc, shared, compact, interleaved, geom):
    ps, H, D = geom
    seed = 600 + shared + 2 * compact + 4 * interleaved + ps
    cache, bt, lens, indptr, maxp, n_out = mat_case(seed, shared, compact, ps, H, D)
    B = len(lens)
    out = np.full((n_out, 2, H, ps, D), W.SENTINEL_FP8, np.uint8)
    tab = np.full((B, maxp), -1, np.int32)
    orc.materialize_fp8(cache, bt, lens, indptr, out, tab, shared=shared, v_sf_interleaved=interleaved,
                        threads=oracle_threads())
    dev = DeviceCache(cache)
    d_out = torch.full((n_out, 2, H, ps, D), W.SENTINEL_FP8, dtype=torch.uint8, device="cuda")
    d_tab = torch.full((B, maxp), -1, dtype=torch.int32, device="cuda")
    say(f"materialize seed={seed} geom={geom} shared={shared} compact={compact} interleaved={interleaved}")
    K.kv_materialize_fp8(dev.cache, torch.from_numpy(bt).cuda(), i32(lens), i32(indptr),
                         d_out.view(torch.float8_e4m3fn), d_tab, shared, interleaved)
    torch.cuda.synchronize()
    got = d_out.cpu().numpy()
    assert np.array_equal(got, out), first_mismatch(got, out)
    assert np.array_equal(d_tab.cpu().numpy(), tab)


@pytest.mark.parametrize("case", range(64))
def test_materialize_random_shapes(K, orc, case):
    """seeded draws over page size, heads, head_dim (V scales through the
    wavefront's dwords, or byte by byte when D / 16 does not divide 32),
    shared or separate tables, compact or padded reservations and the V
    scale layout"""
    rng = np.random.default_rng(8400 + case)
    ps = int(rng.choice([4, 8, 12, 16, 32, 64]))
    H = int(rng.choice([1, 2, 3, 4, 8]))
    D = int(rng.choice([64, 128, 192, 256, 320, 512]))
    shared, compact, interleaved = (bool(x) for x in rng.random(3) < 0.5)
    seed = 8500 + case
    cache, bt, lens, indptr, maxp, n_out = mat_case(seed, shared, compact, ps, H, D, B=int(rng.integers(3, 9)))
    B = len(lens)
    out = np.full((n_out, 2, H, ps, D), W.SENTINEL_FP8, np.uint8)
    tab = np.full((B, maxp), -1, np.int32)
    orc.materialize_fp8(cache, bt, lens, indptr, out, tab, shared=shared, v_sf_interleaved=interleaved,
                        threads=oracle_threads())
    dev = DeviceCache(cache)
    d_out = torch.full((n_out, 2, H, ps, D), W.SENTINEL_FP8, dtype=torch.uint8, device="cuda")
    d_tab = torch.full((B, maxp), -1, dtype=torch.int32, device="cuda")
    say(f"materialize sweep seed={seed} geom={(ps, H, D)} B={B} shared={shared} compact={compact} "
        f"interleaved={interleaved}")
    K.kv_materialize_fp8(dev.cache, torch.from_numpy(bt).cuda(), i32(lens), i32(indptr),
                         d_out.view(torch.float8_e4m3fn), d_tab, shared, interleaved)
    torch.cuda.synchronize()
    got = d_out.cpu().numpy()
    assert np.array_equal(got, out), first_mismatch(got, out)
    assert np.array_equal(d_tab.cpu().numpy(), tab)


def test_materialize_empty_batch_zeroes_page0(K, orc):
    cache, bt, lens, indptr, maxp, n_out = mat_case(9, True, True)
    dev = DeviceCache(cache)
    d_out = torch.full((3, 2, 4, 16, 128), 0x33, dtype=torch.uint8, device="cuda")
    d_tab = torch.full((1, 1), -1, dtype=torch.int32, device="cuda")
    K.kv_materialize_fp8(dev.cache, i32(bt[:0]), i32(lens[:0]), i32(np.zeros(1)), d_out.view(torch.float8_e4m3fn),
                         d_tab[:0], True, True)
    torch.cuda.synchronize()
    got = d_out.cpu().numpy()
    assert np.all(got[0] == 0) and np.all(got[1:] == 0x33)


def test_materializer_class_matches_functional(K, orc):
    cache, bt, lens, indptr, maxp, n_out = mat_case(11, True, True)
    dev = DeviceCache(cache)
    m = (int(lens.max()) + 15) // 16
    out_f, tab_f = K.nvfp4_kv_materialize_fp8(dev.k_data, dev.v_data, dev.k_sf, dev.v_sf, i32(bt), i32(lens),
                                              int(lens.max()), True, kv_page_indptr=i32(indptr),
                                              num_pages=int(indptr[-1]))
    mat = K.NVFP4KVMaterializer(4, 16, 128)
    out_r = torch.zeros_like(out_f)
    tab_r = torch.zeros((len(lens), m), dtype=torch.int32, device="cuda")
    mat.run(dev.k_data, dev.v_data, dev.k_sf, dev.v_sf, i32(bt), i32(lens), i32(indptr), out=out_r,
            fp8_block_tables=tab_r)
    torch.cuda.synchronize()
    assert torch.equal(out_f.view(torch.uint8), out_r.view(torch.uint8))
    assert torch.equal(tab_f, tab_r)


# --------------------------------------------------------------------------- global scale
@pytest.mark.parametrize("n", [0, 1, 7, 4096, 1_000_003])
@pytest.mark.parametrize("is_bf16", [True, False])
@pytest.mark.parametrize("emax", [448.0, 256.0])
def test_global_scale_parity(K, orc, n, is_bf16, emax):
    rng = np.random.default_rng(n + 7 * is_bf16)
    x = W.f32_to_bits((rng.standard_normal(n) * 3).astype(np.float32), is_bf16)
    want = orc.global_scale(x, is_bf16, emax)
    g = torch.full((1,), -5.0, dtype=torch.float32, device="cuda")
    K.kv_global_scale(bits_tensor(x, is_bf16) if n else torch.empty(0, dtype=torch.bfloat16 if is_bf16 else
                                                                    torch.float16, device="cuda"), emax, g)
    torch.cuda.synchronize()
    assert g.item() == want


@pytest.mark.parametrize("in_bf16", [True, False])
@pytest.mark.parametrize("recipe", ["standard", "mse", "mae", "mse16", "mae16"])
def test_append_encoder_sweeps_every_16bit_value(K, orc, in_bf16, recipe):
    """Every bf16 / fp16 value in [-6, 6] passes through the E2M1 encoder
    with a unit decode factor (g = 1 and a block amax of 6 give s = 1.0), so
    the device encoder meets every tie and every subnormal input; the 4over6
    recipes also run the amax/4 candidate (decode factor 1.5) on them."""
    ro, rk = recipes(K, orc, recipe)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = W.bits_to_f32(bits, in_bf16)
    keep = np.isfinite(vals) & (np.abs(vals) <= 6.0)
    sweep = bits[keep]
    n_rows = (sweep.size + 14) // 15
    pad = np.zeros(n_rows * 15, np.uint16)
    pad[:sweep.size] = sweep
    six = W.f32_to_bits(np.array([6.0], np.float32), in_bf16)[0]
    rows = np.concatenate([np.full((n_rows, 1), six, np.uint16), pad.reshape(n_rows, 15)], axis=1)
    key = rows.reshape(n_rows, 1, 16)
    val = key[::-1].copy()
    ps = 16
    lens = np.array([n_rows])
    pool = (n_rows + ps - 1) // ps + 2
    rng = np.random.default_rng(77)
    indices, indptr, last = W.csr_for_lengths(lens, ps, rng.permutation(pool))
    cache = W.make_cache(rng, pool, ps, 1, 16, W.NHD)
    bi, pos = W.rows_for_positions(np.zeros(1, np.int64), lens)
    host = cache.copy()
    dev = DeviceCache(cache)
    say(f"encoder sweep bf16={in_bf16} recipe={recipe} rows={n_rows}")
    K.kv_quantize_append(dev.cache, bits_tensor(key, in_bf16), bits_tensor(val, in_bf16), i32(bi), i32(pos),
                         i32(indices), i32(indptr), i32(last), 1.0, 1.0, rk)
    torch.cuda.synchronize()
    orc.quantize_append(host, key, val, in_bf16, bi, pos, indices, indptr, last, 1.0, 1.0, ro,
                        threads=oracle_threads())
    got = dev.to_host()
    for a, b in zip((got.k_data, got.v_data, got.k_sf, got.v_sf), (host.k_data, host.v_data, host.k_sf, host.v_sf)):
        assert np.array_equal(a, b), first_mismatch(a, b)


def double_rounding_scales(rng, is_bf16, want=12):
    """Global scales g for which some product fp32(E4M3(s) * g) * e2m1 has an
    exact value whose direct rounding to 16 bits differs from rounding its
    fp32 rounding: the definition rounds twice, a fused multiply-convert
    (one rounding of the exact product) would not."""
    from test_oracle_ops import E4M3_TORCH
    S = E4M3_TORCH[0x08:0x7F].astype(np.float32)
    E = np.array([0.5, 1.5, 3.0, 6.0], np.float32)
    bits = 8 if is_bf16 else 11                       # significant bits (normal range)

    def rne(p):
        """nearest value with `bits` significant bits, ties to even (the
        normal range of the 16-bit type is all these products reach)"""
        e = np.floor(np.log2(np.abs(p)))
        ulp = np.exp2(e - (bits - 1))
        return np.rint(p / ulp) * ulp                 # exact scaling; rint is ties-to-even

    found = []
    while len(found) < want:
        g = np.float32(np.exp(rng.uniform(-9, 2)))
        dec = (S * g).astype(np.float32)
        p = dec.astype(np.float64)[:, None] * E.astype(np.float64)[None, :]        # exact
        if np.any(rne(p.astype(np.float32).astype(np.float64)) != rne(p)):
            found.append(float(g))
    return found


@pytest.mark.parametrize("bf16", [True, False])
def test_dequant_rounds_the_fp32_product(K, orc, bf16):
    """Near-midpoint products: the device output must round the fp32 product
    (as the definition does), not the exact one."""
    rng = np.random.default_rng(4242 + bf16)
    gs = double_rounding_scales(rng, bf16)
    ps, H, D = 16, 1, 128
    s_all = np.arange(0x00, 0x7F, dtype=np.uint8)
    n_tok = len(s_all) * 2
    pages = (n_tok + ps - 1) // ps
    cache = W.make_cache(rng, pages, ps, H, D, W.NHD, fill="zero")
    codes = np.arange(16, dtype=np.uint8)
    row = np.tile(codes[0::2] | (codes[1::2] << 4), D // 16)
    for a in (cache.k_data, cache.v_data):
        a[...] = np.tile(row, (pages, ps))
    for a in (cache.k_sf, cache.v_sf):
        a[...] = np.resize(np.repeat(s_all, D // 16), a.size).reshape(a.shape)
    bt = np.arange(pages, dtype=np.int32)[None, :]
    lens = np.array([pages * ps], np.int32)
    dev = DeviceCache(cache)
    dt = torch.bfloat16 if bf16 else torch.float16
    for g in gs:
        ok = torch.empty((1, pages * ps, H, D), dtype=dt, device="cuda")
        ov = torch.empty_like(ok)
        K.kv_dequantize_paged(dev.cache, i32(bt), i32(lens), torch.tensor([g], device="cuda"),
                              torch.tensor([g], device="cuda"), ok, ov)
        wk = np.zeros((1, pages * ps, H, D), np.uint16)
        wv = wk.copy()
        orc.dequantize_paged(cache, bt, lens, g, g, wk, wv, bf16)
        got = tensor_bits(ok)
        assert np.array_equal(got, wk), (g, first_mismatch(got, wk))
