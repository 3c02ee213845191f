"""Validate once, launch many: prepared calls (kv_*_prepare + kvfp4_launch)
and NVFP4KVMaterializer.run()'s per-tensor-set cache, against the oracle.
A prepared call reads the buffers' contents at launch time, so new rows,
lengths and tables written into the same tensors must give the oracle's
result for those new contents; a new tensor set is checked again."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DeviceCache, bits_tensor, first_mismatch, i32, oracle_threads, same_bytes, tensor_bits
from test_gpu_parity import append_case, dequant_case, mat_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_paged_amd as K
    return K


def say(*a):
    print(*a, flush=True)


def test_prepared_append_relaunch_with_new_rows(K, orc):
    cache, key, val, bi, pos, indices, indptr, last, lens = append_case(1500, W.NHD, 16, 4, 128, True)
    gk = float(np.float32(orc.global_scale(key, True)))
    gv = float(np.float32(orc.global_scale(val, True)))
    dev = DeviceCache(cache)
    host = cache.copy()
    tk, tv, tbi, tpos = bits_tensor(key, True), bits_tensor(val, True), i32(bi), i32(pos)
    call = K.prepare_quantize_append(dev.cache, tk, tv, tbi, tpos, i32(indices), i32(indptr), i32(last), gk, gv)
    rng = np.random.default_rng(1501)
    for step in range(3):
        say(f"prepared append: launch {step}")
        call.launch()
        orc.quantize_append(host, key, val, True, bi, pos, indices, indptr, last, gk, gv, threads=oracle_threads())
        torch.cuda.synchronize()
        got = dev.to_host()
        assert same_bytes(got, host), step
        # next launch: new row values and the rows in another order, same tensors
        key = W.f32_to_bits(rng.standard_normal(key.shape).astype(np.float32) * np.float32(0.7), True)
        val = W.f32_to_bits(rng.standard_normal(val.shape).astype(np.float32) * np.float32(0.3), True)
        order = rng.permutation(len(bi))
        bi, pos = bi[order], pos[order]
        tk.copy_(bits_tensor(key, True))
        tv.copy_(bits_tensor(val, True))
        tbi.copy_(i32(bi))
        tpos.copy_(i32(pos))


@pytest.mark.parametrize("layout", [W.NHD, W.HND])
def test_prepared_dequant_relaunch_with_new_lengths(K, orc, layout):
    cache, bt, lens, T = dequant_case(1510 + layout, layout, 16, 8, 128)
    B = len(lens)
    gk, gv = 0.0137, 2.7e-4
    dev = DeviceCache(cache)
    dk = torch.full((B, T, 8, 128), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dv = dk.clone()
    tbt, tlens = i32(bt), i32(lens)
    call = K.prepare_dequantize_paged(dev.cache, tbt, tlens, torch.tensor([gk], device="cuda"),
                                      torch.tensor([gv], device="cuda"), dk, dv)
    rng = np.random.default_rng(1512)
    for step in range(3):
        say(f"prepared dequant layout={layout}: launch {step}, lens={list(lens)}")
        dk.view(torch.int16).fill_(W.SENTINEL_16 - 65536)
        dv.view(torch.int16).fill_(W.SENTINEL_16 - 65536)
        call.launch()
        ok = np.full((B, T, 8, 128), W.SENTINEL_16, np.uint16)
        ov = ok.copy()
        orc.dequantize_paged(cache, bt, lens, gk, gv, ok, ov, True, threads=oracle_threads())
        torch.cuda.synchronize()
        assert np.array_equal(tensor_bits(dk), ok), (step, first_mismatch(tensor_bits(dk), ok))
        assert np.array_equal(tensor_bits(dv), ov), step
        lens = rng.integers(0, T + 1, B).astype(np.int32)
        bt = rng.integers(0, cache.num_pages, bt.shape).astype(np.int32)
        tlens.copy_(i32(lens))
        tbt.copy_(i32(bt))


def test_materializer_run_prepares_once_per_tensor_set(K, orc):
    cache, bt, lens, indptr, maxp, n_out = mat_case(1520, False, True)
    H, ps, D = 4, 16, 128
    B = len(lens)
    dev = DeviceCache(cache)
    mat = K.NVFP4KVMaterializer(H, ps, D, uses_shared_paged_kv_idx=False)
    tbt, tlens, tptr = i32(bt), i32(lens), i32(indptr)
    outs = [torch.full((n_out, 2, H, ps, D), W.SENTINEL_FP8, dtype=torch.uint8, device="cuda") for _ in range(2)]
    tab = torch.full((B, maxp), -1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(1521)

    def check(out_t, lens_now, tag):
        want = np.full((n_out, 2, H, ps, D), W.SENTINEL_FP8, np.uint8)
        wtab = np.full((B, maxp), -1, np.int32)
        orc.materialize_fp8(cache, bt, lens_now, indptr, want, wtab, shared=False, threads=oracle_threads())
        torch.cuda.synchronize()
        got = out_t.cpu().numpy()
        assert np.array_equal(got, want), (tag, first_mismatch(got, want))
        assert np.array_equal(tab.cpu().numpy(), wtab), tag

    fp8 = [o.view(torch.float8_e4m3fn) for o in outs]       # kept views: the same tensor objects every step
    for step in range(2):
        say(f"materializer run: step {step} (same tensors)")
        outs[0].fill_(W.SENTINEL_FP8)
        tab.fill_(-1)
        mat.run(dev.k_data, dev.v_data, dev.k_sf, dev.v_sf, tbt, tlens, tptr, out=fp8[0], fp8_block_tables=tab)
        check(outs[0], lens, f"step {step}")
        assert len(mat._prepared) == 1  # checked on first sight only
        # shorter requests next step: contents change, the prepared call stays
        lens = np.minimum(lens, rng.integers(0, 8 * ps, B)).astype(np.int32)
        tlens.copy_(i32(lens))
    say("materializer run: a second workspace")
    outs[1].fill_(W.SENTINEL_FP8)
    tab.fill_(-1)
    mat.run(dev.k_data, dev.v_data, dev.k_sf, dev.v_sf, tbt, tlens, tptr, out=fp8[1], fp8_block_tables=tab)
    check(outs[1], lens, "second workspace")
    assert len(mat._prepared) == 2
    # a freed workspace: a new tensor (possibly at the same id) is checked again
    del fp8[1], outs[1]
    out3 = torch.full((n_out, 2, H, ps, D), W.SENTINEL_FP8, dtype=torch.uint8, device="cuda")
    tab.fill_(-1)
    say("materializer run: a new workspace after the old one was freed")
    mat.run(dev.k_data, dev.v_data, dev.k_sf, dev.v_sf, tbt, tlens, tptr, out=out3.view(torch.float8_e4m3fn),
            fp8_block_tables=tab)
    check(out3, lens, "new workspace")


def test_prepared_launches_in_a_graph(K, orc):
    """prepared append + dequant captured in a HIP graph and replayed three
    times from the same start (eager work in between) match the eager calls"""
    cache, key, val, bi, pos, indices, indptr, last, lens = append_case(1530, W.HND, 16, 4, 128, True)
    gk = float(np.float32(orc.global_scale(key, True)))
    gv = float(np.float32(orc.global_scale(val, True)))
    dev = DeviceCache(cache)
    start = [b.clone() for b in dev.bases]
    tk, tv = bits_tensor(key, True), bits_tensor(val, True)
    app = K.prepare_quantize_append(dev.cache, tk, tv, i32(bi), i32(pos), i32(indices), i32(indptr), i32(last), gk, gv)
    cols = int(((lens + 15) // 16).max())
    bt = W.block_table_from_csr(indices, indptr, cols)
    T = int(lens.max())
    dk = torch.zeros((len(lens), T, 4, 128), dtype=torch.bfloat16, device="cuda")
    dv = torch.zeros_like(dk)
    deq = K.prepare_dequantize_paged(dev.cache, i32(bt), i32(lens), torch.tensor([gk], device="cuda"),
                                     torch.tensor([gv], device="cuda"), dk, dv)
    app.launch()
    deq.launch()
    torch.cuda.synchronize()
    want = [b.clone() for b in dev.bases] + [dk.clone(), dv.clone()]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    for b, s0 in zip(dev.bases, start):
        b.copy_(s0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        app.launch()
        deq.launch()
    for rep in range(3):
        say(f"prepared launches in a graph: replay {rep}")
        for b, s0 in zip(dev.bases, start):
            b.copy_(s0)
        dk.zero_()
        dv.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, w in zip(list(dev.bases) + [dk, dv], want):
            assert torch.equal(got.view(torch.uint8) if got.dtype != torch.uint8 else got,
                               w.view(torch.uint8) if w.dtype != torch.uint8 else w), rep
