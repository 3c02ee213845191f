"""Every entry point recorded into a HIP graph (torch.cuda.CUDAGraph) and
replayed: each replay must write exactly the bytes the eager call wrote.

All calls are asynchronous on the caller's stream, allocate nothing and clear
their own counters with kernels, so a graph holds only kernel nodes. Between
replays the outputs are overwritten with junk and unrelated eager work runs
with host synchronizations in between, so a replay that leaned on state left
from the capture or from a previous replay would show up as a mismatch."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import DeviceCache, i32

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_paged_amd as K
    return K


def say(*a):
    print(*a, flush=True)


def rand_bytes(n, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), generator=g, dtype=torch.uint8, device="cuda")


def rand_half(shape, seed, dtype=torch.bfloat16, scale=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(dtype)


def as_bytes(t):
    assert t.is_contiguous()
    return t.view(torch.uint8).reshape(-1)


def junk(shape, dtype, seed):
    """an output tensor whose every byte starts random"""
    t = torch.empty(shape, dtype=dtype, device="cuda")
    as_bytes(t).copy_(rand_bytes(as_bytes(t).numel(), seed))
    return t


def check_replays(fn, outputs, name):
    """Run ``fn`` eagerly from the outputs' current bytes, capture it, then
    replay REPLAYS times from those same starting bytes, with junk written
    and unrelated eager work run in between; every replay must leave the
    bytes the eager call left (regions the call does not write included)."""
    start = [as_bytes(o).clone() for o in outputs]

    def restore():
        for o, s in zip(outputs, start):
            as_bytes(o).copy_(s)
    torch.cuda.synchronize()
    fn()
    torch.cuda.synchronize()
    want = [as_bytes(o).clone() for o in outputs]
    assert any(bool((w != s).any()) for w, s in zip(want, start)), f"{name}: the eager call wrote nothing"
    side = torch.randn(512, 512, device="cuda")
    g = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for i, o in enumerate(outputs):
            as_bytes(o).copy_(rand_bytes(as_bytes(o).numel(), 7000 + 31 * r + i))
        side = torch.tanh(side @ side.t() * 1e-3)       # unrelated eager work on the same stream
        torch.cuda.synchronize()
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outputs, want)):
            bad = (as_bytes(o) != w).nonzero()
            assert bad.numel() == 0, (f"{name}: replay {r}, output {i}: {bad.numel()} bytes differ, "
                                      f"first at {int(bad[0])}")
    say(f"{name}: {REPLAYS} replays bit-exact")
    del g


def random_cache(K, P, ps, H, D, layout, seed, data_pad=0, sf_hi=0x7E):
    """device paged cache of random code bytes and finite scale bytes"""
    rng = np.random.default_rng(seed)
    host = W.make_cache(rng, P, ps, H, D, layout, data_pad=data_pad, fill="zero")
    for a in (host.k_data, host.v_data):
        a[...] = np.frombuffer(rng.bytes(a.size), dtype=np.uint8).reshape(a.shape)
    for a in (host.k_sf, host.v_sf):
        a[...] = W.scale_bytes(rng, a.shape, 0, sf_hi)
    return DeviceCache(host)


@pytest.mark.parametrize("recipe", ["standard", "4over6"])
def test_graph_append(K, recipe):
    ps, H, D, P = 16, 8, 128, 64
    dev = random_cache(K, P, ps, H, D, K.KVFP4_NHD, 11)
    lens = np.array([1, 17, 40, 16, 33], np.int64)
    old = np.array([0, 9, 3, 0, 20], np.int64)
    rng = np.random.default_rng(12)
    indices, indptr, last = W.csr_for_lengths(lens, ps, rng.permutation(P))
    bi, pos = W.rows_for_positions(old, lens)
    nnz = len(bi)
    key = rand_half((nnz, H, D), 13, scale=3.0)
    val = rand_half((nnz, H, D), 14, scale=0.5)
    rec = K.Recipe(256.0, K.KVFP4_ERR_MSE) if recipe == "4over6" else None
    args = (i32(bi), i32(pos), i32(indices), i32(indptr), i32(last))

    def fn():
        K.kv_quantize_append(dev.cache, key, val, *args, 0.75, 1.5, rec)
    check_replays(fn, dev.bases, f"kv_quantize_append[{recipe}]")


@pytest.mark.parametrize("layout,bt_i64,out_bf16", [("NHD", False, True), ("HND", True, False)])
def test_graph_dequantize_paged(K, layout, bt_i64, out_bf16):
    ps, H, D = 32, 4, 128
    lens = np.array([100, 1, 257, 0, 64], np.int32)
    maxp = int((lens.max() + ps - 1) // ps)
    P = len(lens) * maxp
    lay = K.KVFP4_NHD if layout == "NHD" else K.KVFP4_HND
    dev = random_cache(K, P, ps, H, D, lay, 21)
    bt = np.random.default_rng(22).permutation(P).reshape(len(lens), maxp)
    bt_t = torch.from_numpy(bt.astype(np.int64 if bt_i64 else np.int32)).cuda()
    T = int(lens.max()) + 5
    dt = torch.bfloat16 if out_bf16 else torch.float16
    ok, ov = junk((len(lens), T, H, D), dt, 23), junk((len(lens), T, H, D), dt, 24)
    gk, gv = torch.tensor([0.5], device="cuda"), torch.tensor([2.0], device="cuda")
    sl = i32(lens)

    def fn():
        K.kv_dequantize_paged(dev.cache, bt_t, sl, gk, gv, ok, ov)
    check_replays(fn, [ok, ov], f"kv_dequantize_paged[{layout}]")


@pytest.mark.parametrize("shared", [False, True])
def test_graph_materialize_fp8(K, shared):
    ps, H, D = 16, 4, 128
    rng = np.random.default_rng(31)
    lens, P, maxp, bt, indptr = W.materialize_tables(rng, 6, 5, 300, ps, shared, True)
    dev = random_cache(K, P, ps, H, D, K.KVFP4_HND, 32, data_pad=256)
    n_out = int(indptr[-1])
    out = junk((n_out + 1, 2, H, ps, D), torch.uint8, 33)
    tab = junk((len(lens), maxp), torch.int32, 34)
    bt_t, sl, ip = i32(bt), i32(lens), i32(indptr)

    def fn():
        K.kv_materialize_fp8(dev.cache, bt_t, sl, ip, out.view(torch.float8_e4m3fn), tab, shared, True)
    check_replays(fn, [out, tab], f"kv_materialize_fp8[shared={shared}]")


@pytest.mark.parametrize("n", [1, 4097, 3 * 2**20 + 11])
def test_graph_global_scale(K, n):
    x = rand_half((n,), 41 + n, scale=17.0)
    g_out = junk((1,), torch.float32, 42)

    def fn():
        K.kv_global_scale(x, 448.0, g_out)
    check_replays(fn, [g_out], f"kv_global_scale[n={n}]")


@pytest.mark.parametrize("recipe", ["standard", "4over6-mae-fast"])
def test_graph_contiguous_codec(K, recipe):
    rows, cols = 777, 256
    x = rand_half((rows, cols), 51, dtype=torch.float16, scale=4.0)
    gs = torch.tensor([1.0 / 3.0], device="cuda")
    rec = K.Recipe(256.0, K.KVFP4_ERR_MAE, True) if recipe != "standard" else None
    codes, scales = junk((rows, cols // 2), torch.uint8, 52), junk((rows, cols // 16), torch.uint8, 53)
    back = junk((rows, cols), x.dtype, 54)

    def fn():                     # quantize, then dequantize what it wrote, in one graph
        K.kv_quantize(x, gs, codes, scales, rec)
        K.kv_dequantize(codes, scales, gs, back)
    check_replays(fn, [codes, scales, back], f"kv_quantize+kv_dequantize[{recipe}]")


@pytest.mark.parametrize("layout,interleaved", [("NHD", False), ("HND", True)])
def test_graph_quantize_paged_cache(K, layout, interleaved):
    ps, H, D, P = 16, 2, 128, 9
    lay = K.KVFP4_NHD if layout == "NHD" else K.KVFP4_HND
    dev = random_cache(K, P, ps, H, D, lay, 61)
    kin = rand_half((P * ps * H * D,), 62, scale=2.0)
    vin = rand_half((P * ps * H * D,), 63)
    gk, gv = torch.tensor([0.25], device="cuda"), torch.tensor([0.125], device="cuda")

    def fn():
        K.kv_quantize_paged_cache(dev.cache, kin, vin, gk, gv, K.Recipe(), interleaved)
    check_replays(fn, dev.bases, f"kv_quantize_paged_cache[{layout}]")


@pytest.mark.parametrize("layout,bf16,G", [("NHD", True, 4), ("HND", False, 8)])
def test_graph_decode_attention(K, layout, bf16, G):
    ps, H, D = 16, 2, 128
    lens = np.array([1, 255, 256, 257, 700, 16], np.int32)
    maxp = int((lens.max() + ps - 1) // ps)
    B, P = len(lens), len(lens) * maxp + 2
    lay = K.KVFP4_NHD if layout == "NHD" else K.KVFP4_HND
    dev = random_cache(K, P, ps, H, D, lay, 71, data_pad=16, sf_hi=0x40)
    bt = i32(np.random.default_rng(72).permutation(P)[:B * maxp].reshape(B, maxp))
    dt = torch.bfloat16 if bf16 else torch.float16
    q = rand_half((B, H * G, D), 73, dtype=dt)
    out = junk(q.shape, dt, 74)
    ws = junk((K.kv_decode_attention_workspace_size(B, H, H * G, maxp, ps),), torch.uint8, 75)
    gk, gv = torch.tensor([0.05], device="cuda"), torch.tensor([0.5], device="cuda")
    sl = i32(lens)

    def fn():
        K.kv_decode_attention(dev.cache, q, bt, sl, gk, gv, D ** -0.5, out, ws)
    check_replays(fn, [out], f"kv_decode_attention[{layout}, G={G}]")


def test_graph_decode_step(K):
    """append one token per request, gather-dequantize the context and attend
    over it, all in one graph: later calls read what the append wrote"""
    ps, H, D, G = 16, 4, 128, 2
    old = np.array([0, 15, 16, 300, 77], np.int64)
    new = old + 1
    maxp = int((new.max() + ps - 1) // ps)
    B, P = len(old), len(old) * maxp + 4
    dev = random_cache(K, P, ps, H, D, K.KVFP4_NHD, 81, data_pad=16, sf_hi=0x40)
    indices, indptr, last = W.csr_for_lengths(new, ps, np.random.default_rng(82).permutation(P))
    bt = i32(W.block_table_from_csr(indices, indptr, maxp))
    key = rand_half((B, H, D), 83)
    val = rand_half((B, H, D), 84)
    sl = i32(new)
    bi, pos = i32(np.arange(B)), i32(old)
    ind, ptr, lst = i32(indices), i32(indptr), i32(last)
    gk, gv = torch.tensor([0.5], device="cuda"), torch.tensor([0.25], device="cuda")
    T = int(new.max())
    ok, ov = junk((B, T, H, D), torch.bfloat16, 86), junk((B, T, H, D), torch.bfloat16, 87)
    q = rand_half((B, H * G, D), 85)
    out = junk(q.shape, torch.bfloat16, 88)
    ws = junk((K.kv_decode_attention_workspace_size(B, H, H * G, maxp, ps),), torch.uint8, 89)

    def fn():
        K.kv_quantize_append(dev.cache, key, val, bi, pos, ind, ptr, lst, 0.5, 0.25)
        K.kv_dequantize_paged(dev.cache, bt, sl, gk, gv, ok, ov)
        K.kv_decode_attention(dev.cache, q, bt, sl, gk, gv, D ** -0.5, out, ws)
    check_replays(fn, list(dev.bases) + [ok, ov, out], "decode step")


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_graph_append_dequantize_paged(K, layout):
    """the one-launch decode step (append, then dequantize, one kernel) and
    the attention that reads its cache, in one graph"""
    ps, H, D, G = 16, 4, 128, 2
    old = np.array([0, 15, 16, 300, 77, 31], np.int64)
    new = old + 1
    maxp = int((new.max() + ps - 1) // ps)
    B, P = len(old), len(old) * maxp + 4
    lay = K.KVFP4_NHD if layout == "NHD" else K.KVFP4_HND
    dev = random_cache(K, P, ps, H, D, lay, 91, data_pad=16, sf_hi=0x40)
    indices, indptr, last = W.csr_for_lengths(new, ps, np.random.default_rng(92).permutation(P))
    bt = i32(W.block_table_from_csr(indices, indptr, maxp))
    key = rand_half((B, H, D), 93)
    val = rand_half((B, H, D), 94)
    sl = i32(new)
    order = np.random.default_rng(95).permutation(B)
    bi, pos = i32(order), i32(old[order])
    ind, ptr, lst = i32(indices), i32(indptr), i32(last)
    gk, gv = torch.tensor([0.5], device="cuda"), torch.tensor([0.25], device="cuda")
    T = int(new.max())
    ok, ov = junk((B, T, H, D), torch.bfloat16, 96), junk((B, T, H, D), torch.bfloat16, 97)
    q = rand_half((B, H * G, D), 98)
    out = junk(q.shape, torch.bfloat16, 99)
    ws = junk((K.kv_decode_attention_workspace_size(B, H, H * G, maxp, ps),), torch.uint8, 100)

    def fn():
        K.kv_append_dequantize_paged(dev.cache, key, val, bi, pos, ind, ptr, lst, 0.5, 0.25, bt, sl, gk, gv, ok, ov)
        K.kv_decode_attention(dev.cache, q, bt, sl, gk, gv, D ** -0.5, out, ws)
    check_replays(fn, list(dev.bases) + [ok, ov, out], f"one-launch decode step ({layout})")
