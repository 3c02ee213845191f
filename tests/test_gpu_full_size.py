"""GPU parity at the benchmark's full sizes and launch configurations.

The device processes the whole workload and the oracle recomputes all of it
(every request of the decode, prefill, materialize and 4over6 workloads), bit
for bit: codes, scales, untouched cache bytes, dequantized values, untouched
output tails, FP8 pages, page 0, pages past kv_page_indptr[-1] and the FP8
table.
"""
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


def test_decode_workload_full_size(K, orc):
    """64 requests (124,503 tokens): the whole history is quantized by the
    oracle; the GPU appends the 64 new tokens and dequantizes the whole
    context, and every request is compared."""
    rng = np.random.default_rng(1002)
    ps, H, D, pool = 16, 8, 128, 20000
    old, new_len, indices, indptr, last, bt = W.decode_append_tables(rng, 64, 4096, pool, ps)
    a_k, a_v = W.head_scales(rng, H), W.head_scales(rng, H)
    cache = W.make_cache(rng, pool, ps, H, D, W.NHD)
    for a in (cache.k_sf, cache.v_sf):              # unused pages: random bytes without NaN scales
        a[(a & 0x7F) == 0x7F] = 0x7E
    hist_rows = int(old.sum())
    hk = W.f32_to_bits(W.head_scaled_normal(rng, hist_rows, a_k, D), True)
    hv = W.f32_to_bits(W.head_scaled_normal(rng, hist_rows, a_v, D), True)
    nk = W.f32_to_bits(W.head_scaled_normal(rng, 64, a_k, D), True)
    nv = W.f32_to_bits(W.head_scaled_normal(rng, 64, a_v, D), True)
    gk = orc.global_scale(np.concatenate([hk.ravel(), nk.ravel()]), True)
    gv = orc.global_scale(np.concatenate([hv.ravel(), nv.ravel()]), True)
    hb, hp = W.rows_for_positions(np.zeros(64, np.int64), old)
    say(f"decode full size: oracle quantization of the whole history ({hist_rows} rows)")
    orc.quantize_append(cache, hk, hv, True, hb, hp, indices, indptr, last, gk, gv, threads=oracle_threads())
    del hk, hv

    dev = DeviceCache(cache)
    bi, pos = np.arange(64, dtype=np.int32), old.astype(np.int32)
    say("decode full size: GPU append of 64 rows")
    K.kv_quantize_append(dev.cache, bits_tensor(nk, True), bits_tensor(nv, True), i32(bi), i32(pos), i32(indices),
                         i32(indptr), i32(last), gk, gv)
    T = int(new_len.max())
    ok = torch.full((64, T, H, D), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ov = ok.clone()
    say("decode full size: GPU dequant of the full context")
    K.kv_dequantize_paged(dev.cache, i32(bt), i32(new_len), torch.tensor([gk], device="cuda"),
                          torch.tensor([gv], device="cuda"), ok, ov)
    torch.cuda.synchronize()

    host = cache.copy()
    orc.quantize_append(host, nk, nv, True, bi, pos, indices, indptr, last, gk, gv, threads=oracle_threads())
    got = dev.to_host()
    for a, b in zip(got.bases, host.bases):          # the 64 new rows and every other byte
        assert np.array_equal(a, b)
    del got, dev
    say("decode full size: oracle dequant of all 64 requests")
    wk = np.full((64, T, H, D), W.SENTINEL_16, np.uint16)
    wv = wk.copy()
    orc.dequantize_paged(host, bt, new_len.astype(np.int32), gk, gv, wk, wv, True, threads=oracle_threads())
    kb = tensor_bits(ok)
    del ok
    assert np.array_equal(kb, wk), first_mismatch(kb, wk)           # tails keep the sentinel on both sides
    del kb, wk
    vb = tensor_bits(ov)
    assert np.array_equal(vb, wv), first_mismatch(vb, wv)


def test_prefill_workload_full_size(K, orc):
    """16 x 8192 tokens, HND, int64 table, fp16 out: every page holds the
    oracle's quantization of bf16 N(0,1); one request is shorter (its tail
    stays untouched); all 16 requests are compared."""
    rng = np.random.default_rng(1003)
    B, T, ps, H, D = 16, 8192, 32, 8, 128
    n_pages = B * T // ps
    perm = rng.permutation(n_pages)
    bt = perm.reshape(B, T // ps).astype(np.int64)
    cache = W.make_cache(rng, n_pages, ps, H, D, W.HND, fill="zero")
    xk = W.f32_to_bits(W.normal_rows(rng, (B * T, H, D)), True)
    xv = W.f32_to_bits(W.normal_rows(rng, (B * T, H, D)), True)
    gk, gv = orc.global_scale(xk, True), orc.global_scale(xv, True)
    bi, pos = W.rows_for_positions(np.zeros(B, np.int64), np.full(B, T))
    say("prefill full size: oracle quantization of all 16 requests")
    orc.quantize_append(cache, xk, xv, True, bi, pos, perm.astype(np.int32), (np.arange(B + 1) * (T // ps)).astype(np.int32),
                        np.full(B, ps, np.int32), gk, gv, threads=oracle_threads())
    del xk, xv
    dev = DeviceCache(cache)
    ok = torch.full((B, T, H, D), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.float16)
    ov = ok.clone()
    lens = np.full(B, T, np.int32)
    lens[3] = 5000                                    # one shorter request: its tail stays untouched
    say("prefill full size: GPU dequant")
    K.kv_dequantize_paged(dev.cache, torch.from_numpy(bt).cuda(), i32(lens), torch.tensor([gk], device="cuda"),
                          torch.tensor([gv], device="cuda"), ok, ov)
    torch.cuda.synchronize()
    del dev
    say("prefill full size: oracle dequant of all 16 requests")
    wk = np.full((B, T, H, D), W.SENTINEL_16, np.uint16)
    wv = wk.copy()
    orc.dequantize_paged(cache, bt, lens, gk, gv, wk, wv, False, threads=oracle_threads())
    kb = tensor_bits(ok)
    del ok
    assert np.all(kb[3, 5000:] == W.SENTINEL_16)
    assert np.array_equal(kb, wk), first_mismatch(kb, wk)
    del kb, wk
    vb = tensor_bits(ov)
    assert np.array_equal(vb, wv), first_mismatch(vb, wv)


def test_materialize_workload_full_size(K, orc):
    """32 requests, 12,070 pages, padded HND pages, separate tables,
    interleaved V scales, a workspace larger than the step needs."""
    wl = W.materialize_fp8()
    c = wl.cache
    H, ps, D = c.num_heads, c.page_size, c.head_dim
    n_out = wl.num_pages_out + 1 + 8
    dev = DeviceCache(c)
    out = torch.full((n_out, 2, H, ps, D), W.SENTINEL_FP8, dtype=torch.uint8, device="cuda")
    tab = torch.full((32, wl.max_pages_per_seq), -1, dtype=torch.int32, device="cuda")
    say("materialize full size: GPU")
    mat = K.NVFP4KVMaterializer(H, ps, D, uses_shared_paged_kv_idx=False)
    mat.run(dev.k_data, dev.v_data, dev.k_sf, dev.v_sf, i32(wl.block_tables), i32(wl.seq_lens),
            i32(wl.kv_page_indptr), out=out.view(torch.float8_e4m3fn), fp8_block_tables=tab)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    gtab = tab.cpu().numpy()
    need = (wl.seq_lens + ps - 1) // ps
    assert np.all(got[0] == 0)
    assert np.all(got[wl.num_pages_out + 1:] == W.SENTINEL_FP8)          # past kv_page_indptr[-1]
    for b in range(32):
        n = need[b]
        assert np.array_equal(gtab[b, :n], wl.kv_page_indptr[b] + np.arange(n) + 1)
        assert np.all(gtab[b, n:] == -1)
    want = np.full_like(got, W.SENTINEL_FP8)
    wtab = np.full_like(gtab, -1)
    say(f"materialize full size: oracle for all 32 requests ({int(need.sum())} pages)")
    orc.materialize_fp8(c, wl.block_tables, wl.seq_lens, wl.kv_page_indptr, want, wtab, shared=False,
                        v_sf_interleaved=True, threads=oracle_threads())
    assert np.array_equal(got, want), first_mismatch(got, want)
    assert np.array_equal(gtab, wtab)


@pytest.mark.parametrize("mode", ["MSE", "MAE"])
def test_four_over_six_workload_full_size(K, orc, mode):
    """65,536 rows of Student-t(3) with 0.1% outliers x20, 4over6 e4m3_max
    256: every code and scale byte against the oracle, then the dequant of
    sampled requests."""
    wl = W.four_over_six_quantize()
    c = wl.cache
    emode = orc.MSE if mode == "MSE" else orc.MAE
    ro = orc.four_over_six(emode)
    rk = K.Recipe(256.0, K.KVFP4_ERR_MSE if mode == "MSE" else K.KVFP4_ERR_MAE)
    gk, gv = orc.global_scale(wl.key, True, 256.0), orc.global_scale(wl.value, True, 256.0)
    dev = DeviceCache(c)
    say(f"4over6 {mode} full size: GPU append of {len(wl.batch_indices)} rows")
    K.kv_quantize_append(dev.cache, bits_tensor(wl.key, True), bits_tensor(wl.value, True), i32(wl.batch_indices),
                         i32(wl.positions), i32(wl.kv_indices), i32(wl.kv_indptr), i32(wl.kv_last_page_len),
                         gk, gv, rk)
    B, T, H, D = 16, wl.max_seq_len, c.num_heads, c.head_dim
    ok = torch.full((B, T, H, D), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ov = ok.clone()
    K.kv_dequantize_paged(dev.cache, i32(wl.block_tables), i32(wl.seq_lens), torch.tensor([gk], device="cuda"),
                          torch.tensor([gv], device="cuda"), ok, ov)
    torch.cuda.synchronize()
    host = c.copy()
    say(f"4over6 {mode} full size: oracle append")
    orc.quantize_append(host, wl.key, wl.value, True, wl.batch_indices, wl.positions, wl.kv_indices, wl.kv_indptr,
                        wl.kv_last_page_len, gk, gv, ro, threads=oracle_threads())
    got = dev.to_host()
    for name, a, b in zip(("k_data", "v_data", "k_sf", "v_sf"), got.bases, host.bases):
        assert np.array_equal(a, b), (name, first_mismatch(a, b))
    say(f"4over6 {mode} full size: oracle dequant of all 16 requests")
    wk = np.full((B, T, H, D), W.SENTINEL_16, np.uint16)
    wv = wk.copy()
    orc.dequantize_paged(host, wl.block_tables, wl.seq_lens, gk, gv, wk, wv, True, threads=oracle_threads())
    kb, vb = tensor_bits(ok), tensor_bits(ov)
    assert np.array_equal(kb, wk), first_mismatch(kb, wk)
    assert np.array_equal(vb, wv), first_mismatch(vb, wv)
