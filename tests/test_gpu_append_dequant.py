"""GPU parity of kv_append_dequantize_paged (one decode step in one call)
against the oracle's append followed by its dequantize: every byte of the
cache and both outputs, untouched tails included. Covers both layouts, page
sizes 1-64, head geometries whose rows take one workgroup or several,
input / output / table dtypes, request rows in any order, lengths cut by
max_seq_len, append and dequant global scales that differ, batches past one
append workgroup per row group, HND geometries of the LDS-staged gather, and
the 4over6 recipes (which run the two calls in sequence instead); then a
prepared step launched for two consecutive decode steps."""
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


def recipe_pair(K, orc, name):
    if name == "standard":
        return orc.STANDARD, None
    mode = orc.MSE if name.startswith("mse") else orc.MAE
    fast = name.endswith("16")
    return (orc.four_over_six(mode, fast_math=fast),
            K.Recipe(256.0, K.KVFP4_ERR_MSE if mode == orc.MSE else K.KVFP4_ERR_MAE, err_use_fast_math=fast))


class Step:
    """A decode step's inputs: a cache of random history bytes (no NaN
    scales), B requests of old length U{0..max_old} and one new token each
    (row order shuffled), their CSR append table and block table."""

    def __init__(self, seed, layout, ps, H, D, B, in_bf16, max_old=None, reserve=0):
        rng = np.random.default_rng(seed)
        self.ps, self.H, self.D, self.B, self.in_bf16 = ps, H, D, B, in_bf16
        max_old = 3 * ps + 7 if max_old is None else max_old
        self.old = rng.integers(0, max_old + 1, B)
        self.new_len = (self.old + 1).astype(np.int32)
        cap = self.new_len + reserve                      # tokens each request's pages are reserved for
        pool = int(((cap + ps - 1) // ps).sum()) + 5
        perm = rng.permutation(pool)
        self.indices, self.indptr, self.last = W.csr_for_lengths(cap, ps, perm)
        self.cols = int((cap.max() + ps - 1) // ps) + 1
        # data page strides padded to 16 bytes, as the calls require
        self.cache = W.make_cache(rng, pool, ps, H, D, layout, data_pad=(-(ps * H * D // 2)) % 16)
        for a in (self.cache.k_sf, self.cache.v_sf):
            a[(a & 0x7F) == 0x7F] = 0x7E
        self.bi = rng.permutation(B).astype(np.int32)
        self.pos = self.old[self.bi].astype(np.int32)
        self.rng = rng
        self.new_rows()

    def new_rows(self):
        a = W.head_scales(self.rng, self.H)
        self.nk = W.f32_to_bits(W.head_scaled_normal(self.rng, self.B, a, self.D), self.in_bf16)
        self.nv = W.f32_to_bits(W.head_scaled_normal(self.rng, self.B, a, self.D), self.in_bf16)

    def table(self, bt64):
        return W.block_table_from_csr(self.indices, self.indptr, self.cols, np.int64 if bt64 else np.int32)


def expected(orc, s, host, recipe, g_app, g_dq, T, out_bf16, bt):
    orc.quantize_append(host, s.nk, s.nv, s.in_bf16, s.bi, s.pos, s.indices, s.indptr, s.last, g_app[0], g_app[1],
                        recipe=recipe, threads=oracle_threads())
    wk = np.full((s.B, T, s.H, s.D), W.SENTINEL_16, np.uint16)
    wv = wk.copy()
    orc.dequantize_paged(host, bt, s.new_len, g_dq[0], g_dq[1], wk, wv, out_bf16, threads=oracle_threads())
    return wk, wv


def device_step(K, s, dev, bt, g_app, g_dq, ok, ov, rk):
    args = (dev.cache, bits_tensor(s.nk, s.in_bf16), bits_tensor(s.nv, s.in_bf16), i32(s.bi), i32(s.pos),
            i32(s.indices), i32(s.indptr), i32(s.last), g_app[0], g_app[1], torch.from_numpy(bt).cuda(),
            i32(s.new_len), torch.tensor([g_dq[0]], device="cuda"), torch.tensor([g_dq[1]], device="cuda"), ok, ov)
    K.kv_append_dequantize_paged(*args, recipe=rk)
    torch.cuda.synchronize()


def compare(dev, host, ok, ov, wk, wv):
    got = dev.to_host()
    for i, (a, b) in enumerate(zip(got.bases, host.bases)):
        assert np.array_equal(a, b), ("cache base", i, first_mismatch(a, b))
    kb, vb = tensor_bits(ok), tensor_bits(ov)
    assert np.array_equal(kb, wk), first_mismatch(kb, wk)
    assert np.array_equal(vb, wv), first_mismatch(vb, wv)


def run_step(K, orc, seed, layout, ps, H, D, B, in_bf16=True, out_bf16=True, bt64=False, T_delta=3,
             recipe="standard", g_dq_factor=1.0, max_old=None):
    s = Step(seed, layout, ps, H, D, B, in_bf16, max_old)
    ro, rk = recipe_pair(K, orc, recipe)
    g_app = (0.0173, 2.9e-4)
    g_dq = (g_app[0] * g_dq_factor, g_app[1] * g_dq_factor)
    T = max(1, int(s.new_len.max()) + T_delta)
    bt = s.table(bt64)
    say(f"append+dequant seed={seed} layout={layout} geom={(ps, H, D)} B={B} in_bf16={in_bf16} "
        f"out_bf16={out_bf16} bt64={bt64} T={T} recipe={recipe} g_dq_factor={g_dq_factor}")
    host = s.cache.copy()
    wk, wv = expected(orc, s, host, ro, g_app, g_dq, T, out_bf16, bt)
    dev = DeviceCache(s.cache)
    tdt = torch.bfloat16 if out_bf16 else torch.float16
    ok = torch.full((B, T, H, D), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(tdt)
    ov = ok.clone()
    device_step(K, s, dev, bt, g_app, g_dq, ok, ov, rk)
    compare(dev, host, ok, ov, wk, wv)


# one launch: standard recipe on the gather's layouts (NHD; HND outside the
# LDS-staged geometry), rows of one or several heads per workgroup, and rows
# wider than a workgroup (32 and 24 heads of 256)
@pytest.mark.parametrize("layout,ps,H,D", [(W.NHD, 16, 8, 128), (W.NHD, 1, 2, 64), (W.NHD, 5, 3, 48),
                                           (W.NHD, 64, 32, 256), (W.HND, 16, 2, 128), (W.HND, 8, 4, 64),
                                           (W.HND, 5, 1, 16), (W.HND, 4, 24, 256)])
@pytest.mark.parametrize("in_bf16,out_bf16,bt64", [(True, True, False), (False, True, True), (True, False, True),
                                                   (False, False, False)])
def test_append_dequant_parity(K, orc, layout, ps, H, D, in_bf16, out_bf16, bt64):
    run_step(K, orc, 9000 + 7 * ps + H + D, layout, ps, H, D, 11, in_bf16, out_bf16, bt64)


@pytest.mark.parametrize("layout", [W.NHD, W.HND])
def test_append_dequant_cut_lengths_and_separate_scales(K, orc, layout):
    """max_seq_len below some lengths (the newest token of a cut request is
    stored in the cache but not in the outputs) and dequant global scales
    that differ from the append's"""
    run_step(K, orc, 9101 + layout, layout, 16, 4, 128, 13, T_delta=-9, g_dq_factor=2.5)
    run_step(K, orc, 9103 + layout, layout, 8, 2, 64, 9, T_delta=-1, g_dq_factor=0.25)


@pytest.mark.parametrize("layout,geoms", [(W.NHD, ((4, 16, 256), (16, 8, 128))),
                                          (W.HND, ((5, 16, 256), (12, 8, 128)))])
def test_append_dequant_many_requests(K, orc, layout, geoms):
    """more rows than one launch gives append workgroups (1,024 of them, one
    row each at 16 heads of 256): the leading workgroups loop over rows (the
    HND page sizes keep these geometries off the LDS-staged gather)"""
    (ps1, H1, D1), (ps2, H2, D2) = geoms
    run_step(K, orc, 9200 + layout, layout, ps1, H1, D1, 1500, max_old=9)
    run_step(K, orc, 9202 + layout, layout, ps2, H2, D2, 700, max_old=40)


@pytest.mark.parametrize("recipe", ["mse", "mae16"])
def test_append_dequant_four_over_six_runs_the_two_calls(K, orc, recipe):
    run_step(K, orc, 9300, W.NHD, 16, 8, 128, 7, recipe=recipe)


@pytest.mark.parametrize("ps,H,D", [(32, 8, 128), (16, 8, 128), (64, 4, 64), (4, 32, 256)])
@pytest.mark.parametrize("in_bf16,out_bf16,bt64", [(True, True, False), (False, False, True)])
def test_append_dequant_lds_geometry(K, orc, ps, H, D, in_bf16, out_bf16, bt64):
    """HND geometries whose gather stages head runs through LDS: one launch
    of the LDS-staged variant"""
    run_step(K, orc, 9400 + ps + H + D, W.HND, ps, H, D, 9, in_bf16, out_bf16, bt64)


@pytest.mark.parametrize("layout", [W.NHD, W.HND])
def test_append_dequant_prepared_two_steps(K, orc, layout):
    """one prepared step launched twice: after the first, every request
    grows by one token (new rows written into the same input tensors, the
    positions and lengths updated in place), as a serving loop does"""
    s = Step(9500 + layout, layout, 16, 8, 64, 9, True, max_old=60, reserve=1)
    g_app = g_dq = (0.011, 3.1e-4)
    T = int(s.new_len.max()) + 3
    bt = s.table(False)
    host = s.cache.copy()
    dev = DeviceCache(s.cache)
    ok = torch.full((s.B, T, 8, 64), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ov = ok.clone()
    key, val = bits_tensor(s.nk, True), bits_tensor(s.nv, True)
    pos_t, lens_t = i32(s.pos), i32(s.new_len)
    call = K.prepare_append_dequantize_paged(dev.cache, key, val, i32(s.bi), pos_t, i32(s.indices), i32(s.indptr),
                                             i32(s.last), g_app[0], g_app[1], torch.from_numpy(bt).cuda(), lens_t,
                                             torch.tensor([g_dq[0]], device="cuda"),
                                             torch.tensor([g_dq[1]], device="cuda"), ok, ov)
    for step in range(2):
        say(f"prepared step {step} layout={layout}")
        wk = np.full((s.B, T, 8, 64), W.SENTINEL_16, np.uint16)
        wv = wk.copy()
        orc.quantize_append(host, s.nk, s.nv, True, s.bi, s.pos, s.indices, s.indptr, s.last, g_app[0], g_app[1],
                            threads=oracle_threads())
        orc.dequantize_paged(host, bt, s.new_len, g_dq[0], g_dq[1], wk, wv, True, threads=oracle_threads())
        call.launch()
        torch.cuda.synchronize()
        kb, vb = tensor_bits(ok), tensor_bits(ov)
        for b in range(s.B):                      # the step's tokens (later positions hold the first step's)
            n = int(s.new_len[b])
            assert np.array_equal(kb[b, :n], wk[b, :n]), (step, b, first_mismatch(kb[b, :n], wk[b, :n]))
            assert np.array_equal(vb[b, :n], wv[b, :n]), (step, b, first_mismatch(vb[b, :n], wv[b, :n]))
        got = dev.to_host()
        for a, b in zip(got.bases, host.bases):
            assert np.array_equal(a, b)
        # the next step: one more token per request, new rows in the same tensors
        s.pos = s.new_len[s.bi].astype(np.int32)
        s.new_len = (s.new_len + 1).astype(np.int32)
        s.new_rows()
        key.copy_(bits_tensor(s.nk, True))
        val.copy_(bits_tensor(s.nv, True))
        pos_t.copy_(i32(s.pos))
        lens_t.copy_(i32(s.new_len))


@pytest.mark.parametrize("case", range(40))
def test_append_dequant_random_shapes(K, orc, case):
    """seeded draws over layout, page size, heads and head_dim (HND shapes on
    both sides of the LDS-staged gather's conditions), dtypes, table dtype,
    batch, max_seq_len cuts and the recipe"""
    rng = np.random.default_rng(9600 + case)
    layout = W.NHD if rng.random() < 0.5 else W.HND
    ps = int(rng.choice([1, 4, 5, 8, 16, 32, 64]))
    H = int(rng.choice([1, 2, 3, 4, 8, 16]))
    D = int(rng.choice([16, 32, 48, 64, 128, 256]))
    in_bf16, out_bf16, bt64 = (bool(x) for x in rng.random(3) < 0.5)
    B = int(rng.integers(1, 40))
    T_delta = int(rng.choice([0, 3, -2]))
    recipe = "standard" if rng.random() < 0.85 else str(rng.choice(["mse", "mae", "mse16"]))
    run_step(K, orc, 9700 + case, layout, ps, H, D, B, in_bf16, out_bf16, bt64, T_delta=T_delta, recipe=recipe,
             g_dq_factor=float(rng.choice([1.0, 0.5])))


def test_append_dequant_page_api_stacked_cache(K, orc):
    """the page-style wrapper on a stacked 5-D cache ([pages, 2, ...] for the
    codes and the scales, "HND"), against the oracle"""
    s = Step(9900, W.HND, 16, 2, 64, 5, True)
    P = s.cache.k_data.shape[0]
    rng = np.random.default_rng(9901)
    codes = torch.from_numpy(rng.integers(0, 256, (P, 2, 2, 16, 32), dtype=np.uint8)).cuda()
    sf = torch.from_numpy(rng.integers(0, 0x7E, (P, 2, 2, 16, 4), dtype=np.uint8)).cuda()
    host = W.make_cache(np.random.default_rng(0), P, 16, 2, 64, W.HND, fill="zero")
    host.k_data[...] = codes[:, 0].reshape(P, -1).cpu().numpy()
    host.v_data[...] = codes[:, 1].reshape(P, -1).cpu().numpy()
    host.k_sf[...] = sf[:, 0].reshape(P, -1).cpu().numpy()
    host.v_sf[...] = sf[:, 1].reshape(P, -1).cpu().numpy()
    s.cache = host
    bt = s.table(False)
    T = int(s.new_len.max()) + 2
    wk, wv = expected(orc, s, host, orc.STANDARD, (0.02, 0.003), (0.02, 0.003), T, True, bt)
    ok = torch.full((5, T, 2, 64), W.SENTINEL_16 - 65536, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ov = ok.clone()
    K.nvfp4_append_dequantize_paged(bits_tensor(s.nk, True), bits_tensor(s.nv, True), i32(s.bi), i32(s.pos), codes, sf,
                                    i32(s.indices), i32(s.indptr), i32(s.last), 0.02, 0.003,
                                    torch.from_numpy(bt).cuda(), i32(s.new_len), torch.tensor([0.02], device="cuda"),
                                    torch.tensor([0.003], device="cuda"), ok, ov, kv_layout="HND")
    torch.cuda.synchronize()
    assert np.array_equal(codes[:, 0].reshape(P, -1).cpu().numpy(), host.k_data)
    assert np.array_equal(codes[:, 1].reshape(P, -1).cpu().numpy(), host.v_data)
    assert np.array_equal(sf[:, 0].reshape(P, -1).cpu().numpy(), host.k_sf)
    assert np.array_equal(sf[:, 1].reshape(P, -1).cpu().numpy(), host.v_sf)
    assert np.array_equal(tensor_bits(ok), wk) and np.array_equal(tensor_bits(ov), wv)
