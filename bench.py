"""Benchmark of the paged NVFP4 KV-cache path on one MI355X.

Headline step (the decode workload): quantize-append one new token for each
of 64 requests (bf16 K/V, 8 KV heads, head_dim 128, page_size 16, NHD pages
shuffled across a 20,000-page pool), then gather-dequantize every request's
full context (lengths U{1..4096} + 1) into bf16 [64, max_len, 8, 128], as one
kv_append_dequantize_paged call per step (the same step as the two calls
kv_quantize_append and kv_dequantize_paged is timed as a leg).
value = algorithmic bytes of the step / wall time of the step, with all
inputs resident in HBM; replicas of the workload in disjoint memory rotate so
that no step finds its inputs in the 256 MB Infinity Cache.

Legs (same JSON line; each kernel launched back to back over rotating
replicas of its workload in disjoint memory, mean of the per-launch HIP-event
times, the same steady state as the headline step): prefill dequantize (16 x 8192 tokens, HND, int64 table, fp16
out), materialize-FP8 (32 requests, log-uniform lengths, padded pages,
separate K/V tables), 4over6 quantize-append (65,536 rows, Student-t(3) with
0.1% outliers x20, MSE and MAE) and its dequantize, and a plain
device-to-device copy as the achievable-bandwidth context line.

Parity of the timed buffers: right after its first launch on the first
replica, each leg copies one or more sampled requests' inputs and outputs to
the host (the same buffers the timing then uses). The CPU leg - the only part
of this file that runs the oracle - checks every sample bit for bit (decode
attention within its derived bound) and exits with status 3 on any mismatch,
before anything is printed. It then times the oracle on the decode step at
the host's full core count and at one thread.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import json
import os
import statistics
import sys
import time
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
METRIC = "effective HBM GB/s and % of MI355X peak for paged NVFP4 KV append/dequant/FP8"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes (what the method must move)
# ---------------------------------------------------------------------------
def dequant_bytes(lens, ps, H, D, bt_elem_bytes):
    tokens = int(np.sum(lens))
    pages = int(np.sum((np.asarray(lens) + ps - 1) // ps))
    return 2 * tokens * H * (D // 2 + D // 16 + 2 * D) + pages * bt_elem_bytes + 4 * len(lens)


def append_bytes(nnz, H, D):
    return 2 * nnz * H * (2 * D + D // 2 + D // 16) + 8 * nnz


def materialize_bytes(lens, ps, H, D, B):
    pages = int(np.sum((np.asarray(lens) + ps - 1) // ps))
    per_page = 2 * H * ps * (D // 2 + D // 16) + 2 * H * ps * D
    return pages * per_page + 2 * H * ps * D + 12 * pages + 4 * (B + 1) + 4 * B


# ---------------------------------------------------------------------------
# device workloads
# ---------------------------------------------------------------------------
class Env:
    def __init__(self):
        import torch
        import kv_cache_quantization_paged_amd as K
        self.torch, self.K = torch, K
        self.dev = torch.device("cuda:0")

    def i32(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.dev)

    def gen(self, seed):
        g = self.torch.Generator(device=self.dev)
        g.manual_seed(seed)
        return g

    def cache(self, pages, ps, H, D, layout, seed, data_pad=0):
        """Pool of pages filled with random bytes; returns (PagedCache, tensors)."""
        torch = self.torch
        g = self.gen(seed)
        dbytes, sbytes = ps * H * D // 2, ps * H * D // 16
        bufs = [torch.randint(0, 256, (pages * (dbytes + data_pad),), generator=g, device=self.dev,
                              dtype=torch.uint8) for _ in range(2)]
        sfs = [torch.randint(0, 0x7F, (pages * sbytes,), generator=g, device=self.dev, dtype=torch.uint8)
               for _ in range(2)]
        inner_d = (ps, H, D // 2) if layout == self.K.KVFP4_NHD else (H, ps, D // 2)
        inner_s = (ps, H, D // 16) if layout == self.K.KVFP4_NHD else (H, ps, D // 16)
        dview = [b.as_strided((pages,) + inner_d, (dbytes + data_pad, inner_d[1] * inner_d[2], inner_d[2], 1))
                 for b in bufs]
        sview = [b.view((pages,) + inner_s) for b in sfs]
        return self.K.PagedCache(dview[0], dview[1], sview[0], sview[1], layout), (bufs, sfs, dview, sview)

    def steady(self, fns, iters, warmup, batches=3):
        """Launch fns[i % len(fns)] back to back (replicas in disjoint memory,
        so nothing is reused from the 256 MB Infinity Cache) in `batches`
        runs, each bracketed by one pair of HIP events on the current stream
        (the stream the library launches on), and return (mean, median) in ms
        per launch: the mean over all launches and the median of the batch
        averages. An event pair around every launch would add the events' own
        few microseconds to each launch; around a batch it is spread over
        the batch, and the per-launch time matches the profiler's kernel
        durations. In this steady state each launch also pays the write-back
        its predecessor left dirty in the cache, as a serving loop does; a
        kernel timed alone after a flush would leave up to 256 MB of its own
        output unwritten when its end event fires."""
        torch = self.torch
        batches = max(1, min(batches, iters))
        sizes = [iters // batches + (1 if b < iters % batches else 0) for b in range(batches)]
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sizes]
        with quiet_host():
            for i in range(warmup):
                fns[i % len(fns)]()
            torch.cuda.synchronize()
            i = 0
            for (ev0, ev1), n in zip(evs, sizes):
                ev0.record()
                for _ in range(n):
                    fns[i % len(fns)]()
                    i += 1
                ev1.record()
            torch.cuda.synchronize()
        per = [a.elapsed_time(b) / n for (a, b), n in zip(evs, sizes)]
        total = sum(a.elapsed_time(b) for a, b in evs)
        return total / iters, statistics.median(per)


@contextlib.contextmanager
def quiet_host():
    """Python's cyclic garbage collector off while launches are being timed:
    a collection inside a timed batch stalls the host that enqueues the
    launches, and the GPU idles for it (seen as one batch of a leg taking
    20-40 ms longer right after another leg's buffers were freed). No
    collection is forced here either: with one before each timed region
    (leaving the GPU idle meanwhile), the event-timed launches read 3-4%
    above the same run's kernel-trace durations, which otherwise agree
    within 1%."""
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def student_t3(env, shape, gen):
    """Student-t with 3 degrees of freedom from four normals, then exactly
    0.1% of the entries (without replacement) multiplied by 20."""
    torch = env.torch
    z = torch.randn(shape, generator=gen, device=env.dev)
    c = torch.zeros(shape, device=env.dev)
    for _ in range(3):
        w = torch.randn(shape, generator=gen, device=env.dev)
        c += w * w
    x = z / torch.sqrt(c / 3.0)
    n = x.numel()
    k = int(round(0.001 * n))
    idx = torch.randperm(n, generator=gen, device=env.dev)[:k]
    x.view(-1)[idx] *= 20.0
    return x


class Decode:
    """The decode workload on the device (one replica)."""

    def __init__(self, env, ps=16, H=8, D=128, pool=20000, seed=1002, keep_history_of=None):
        import workloads as W
        torch, K = env.torch, env.K
        self.env = env
        rng = np.random.default_rng(seed)
        old, new_len, indices, indptr, last, bt = W.decode_append_tables(rng, 64, 4096, pool, ps)
        a_k, a_v = W.head_scales(rng, H), W.head_scales(rng, H)
        self.old = old
        self.tables = (indices, indptr, last, bt)
        self.lens = new_len
        self.B, self.T, self.H, self.D, self.ps = 64, int(new_len.max()), H, D, ps
        self.cache, self._keep = env.cache(pool, ps, H, D, K.KVFP4_NHD, seed)
        g = env.gen(seed)
        n_hist = int(old.sum())
        ak = torch.from_numpy(a_k).to(env.dev)[None, :, None]
        av = torch.from_numpy(a_v).to(env.dev)[None, :, None]
        hk = (torch.randn((n_hist, H, D), generator=g, device=env.dev) * ak).to(torch.bfloat16)
        hv = (torch.randn((n_hist, H, D), generator=g, device=env.dev) * av).to(torch.bfloat16)
        self.key = (torch.randn((64, H, D), generator=g, device=env.dev) * ak).to(torch.bfloat16)
        self.value = (torch.randn((64, H, D), generator=g, device=env.dev) * av).to(torch.bfloat16)
        gk = torch.empty(1, dtype=torch.float32, device=env.dev)
        gv = torch.empty(1, dtype=torch.float32, device=env.dev)
        K.kv_global_scale(torch.cat([hk.view(-1), self.key.view(-1)]), 448.0, gk)
        K.kv_global_scale(torch.cat([hv.view(-1), self.value.view(-1)]), 448.0, gv)
        self.gk_t, self.gv_t = gk, gv
        self.gk, self.gv = float(gk.item()), float(gv.item())
        self.indices, self.indptr, self.last = env.i32(indices), env.i32(indptr), env.i32(last)
        hb = np.concatenate([np.full(o, b, np.int32) for b, o in enumerate(old)])
        hp = np.concatenate([np.arange(o, dtype=np.int32) for o in old])
        K.kv_quantize_append(self.cache, hk, hv, env.i32(hb), env.i32(hp), self.indices, self.indptr, self.last,
                             self.gk, self.gv)
        self.history = None
        if keep_history_of is not None:             # one request's history rows, for the parity check
            b = keep_history_of
            r0 = int(old[:b].sum())
            self.history = (b, host_bits(hk[r0:r0 + int(old[b])]), host_bits(hv[r0:r0 + int(old[b])]))
        del hk, hv
        self.bi = env.i32(np.arange(64))
        self.pos = env.i32(old)
        self.bt = env.i32(bt)
        self.seq_lens = env.i32(new_len)
        self.out_k = torch.empty((64, self.T, H, D), dtype=torch.bfloat16, device=env.dev)
        self.out_v = torch.empty_like(self.out_k)
        self.append_bytes = append_bytes(64, H, D)
        self.dequant_bytes = dequant_bytes(new_len, ps, H, D, 4)

        # the step's two calls, checked once (a serving loop's path)
        self.append_call = K.prepare_quantize_append(self.cache, self.key, self.value, self.bi, self.pos,
                                                     self.indices, self.indptr, self.last, self.gk, self.gv)
        self.dequant_call = K.prepare_dequantize_paged(self.cache, self.bt, self.seq_lens, self.gk_t, self.gv_t,
                                                       self.out_k, self.out_v)
        self.append = self.append_call.launch
        self.dequant = self.dequant_call.launch
        # the same step as one call: the append's rows and the dequant of
        # every request (with its newest token) in one launch
        self.step_call = K.prepare_append_dequantize_paged(self.cache, self.key, self.value, self.bi, self.pos,
                                                           self.indices, self.indptr, self.last, self.gk, self.gv,
                                                           self.bt, self.seq_lens, self.gk_t, self.gv_t, self.out_k,
                                                           self.out_v)
        self.step = self.step_call.launch

    def append_eager(self):
        """the functional call: every tensor checked again"""
        self.env.K.kv_quantize_append(self.cache, self.key, self.value, self.bi, self.pos, self.indices,
                                      self.indptr, self.last, self.gk, self.gv)

    def dequant_eager(self):
        self.env.K.kv_dequantize_paged(self.cache, self.bt, self.seq_lens, self.gk_t, self.gv_t, self.out_k,
                                       self.out_v)

    def sample_step(self, samples: Samples, picks):
        """one step on this replica with host copies around it: the cache
        before and after, the new rows, and the picked requests' outputs"""
        torch = self.env.torch
        pre = whole_cache(self.cache)
        self.step()
        torch.cuda.synchronize()
        post = whole_cache(self.cache)
        outs = {b: (host_bits(self.out_k[b, :int(self.lens[b])]), host_bits(self.out_v[b, :int(self.lens[b])]))
                for b in picks}
        indices, indptr, last, bt = self.tables
        samples.add("decode_step", "decode workload: history quantization, then the step (append and dequant in "
                                   "one kv_append_dequantize_paged call)", pre=pre, post=post,
                    key=host_bits(self.key), value=host_bits(self.value), bi=np.arange(64, dtype=np.int32),
                    pos=self.old.astype(np.int32), indices=indices, indptr=indptr, last=last, bt=bt,
                    lens=self.lens.astype(np.int32), old=self.old, gk=self.gk, gv=self.gv, outs=outs,
                    history=self.history, T=self.T)


# ---------------------------------------------------------------------------
# legs: each kernel in steady state, alternating two replicas of its workload
# ---------------------------------------------------------------------------
def prefill_replica(env, seed=1003, samples=None):
    torch, K = env.torch, env.K
    B, T, ps, H, D = 16, 8192, 32, 8, 128
    rng = np.random.default_rng(seed)
    n_pages = B * T // ps
    perm = rng.permutation(n_pages)
    cache, keep = env.cache(n_pages, ps, H, D, K.KVFP4_HND, seed)
    g = env.gen(seed)
    rows_b = env.i32(np.repeat(np.arange(B), T))
    rows_p = env.i32(np.tile(np.arange(T), B))
    kv, gks = [], []
    for _ in range(2):
        x = torch.randn((B * T, H, D), generator=g, device=env.dev).to(torch.bfloat16)
        gt = torch.empty(1, dtype=torch.float32, device=env.dev)
        K.kv_global_scale(x, 448.0, gt)
        kv.append(x)
        gks.append(gt)
    K.kv_quantize_append(cache, kv[0], kv[1], rows_b, rows_p, env.i32(perm), env.i32(np.arange(B + 1) * (T // ps)),
                         env.i32(np.full(B, ps)), gks[0].item(), gks[1].item())
    bt = torch.from_numpy(perm.reshape(B, T // ps).astype(np.int64)).to(env.dev)
    ok = torch.empty((B, T, H, D), dtype=torch.float16, device=env.dev)
    ov = torch.empty_like(ok)
    sl = env.i32(np.full(B, T))
    nbytes = dequant_bytes(np.full(B, T), ps, H, D, 8)
    fn = K.prepare_dequantize_paged(cache, bt, sl, gks[0], gks[1], ok, ov).launch
    if samples is not None:
        b = 5
        fn()
        torch.cuda.synchronize()
        pages = perm[b * (T // ps):(b + 1) * (T // ps)]
        samples.add("prefill", "prefill workload: quantization of request 5 and its dequant", b=b,
                    rows=(host_bits(kv[0][b * T:(b + 1) * T]), host_bits(kv[1][b * T:(b + 1) * T])),
                    cache=gather_pages(cache, pages), out=(host_bits(ok[b]), host_bits(ov[b])),
                    g=(gks[0].item(), gks[1].item()), T=T)
    del kv
    return fn, nbytes, (cache, keep, ok, ov)


def leg_prefill_dequant(env, iters, warmup, samples):
    fns, keep = [], []
    for i in range(replicas_for(151_000_000)):
        fn, nbytes, k = prefill_replica(env, samples=samples if i == 0 else None)
        fns.append(fn)
        keep.append(k)
    r = env.steady(fns, iters, warmup)
    return dict(kernel="kv_dequantize_paged", workload="prefill_dequantize: 16 x 8192 tokens, page_size 32, "
                "8 heads, head_dim 128, HND, int64 block table, fp16 out", bytes=nbytes, **rates(nbytes, r))


def materialize_replica(env, seed=1004, samples=None, placement="shuffled"):
    """The materialize workload. `placement` "shuffled" (the workload): K and
    V pages from independent permutations of the pool, separate tables;
    "shuffled_shared": one permutation and one shared table for K and V;
    "request_order": request b's pages are consecutive ids (shared table)."""
    torch, K = env.torch, env.K
    import workloads as W
    ps, H, D = 16, 8, 128
    rng = np.random.default_rng(seed)
    shared = placement != "shuffled"
    lens, P, maxp, bt, indptr = W.materialize_tables(rng, 32, 128, 32768, ps, shared=shared, compact=True)
    if placement == "request_order":
        bt = np.where(np.arange(maxp)[None, :] < np.diff(indptr)[:, None],
                      indptr[:-1, None] + np.arange(maxp)[None, :], 0).astype(np.int32)
    cache, keep = env.cache(P, ps, H, D, K.KVFP4_HND, seed, data_pad=256)
    out = torch.empty((P + 1, 2, H, ps, D), dtype=torch.float8_e4m3fn, device=env.dev)
    tab = torch.zeros((32, maxp), dtype=torch.int32, device=env.dev)
    bt_t, sl, ip = env.i32(bt), env.i32(lens), env.i32(indptr)
    mat = K.NVFP4KVMaterializer(H, ps, D, env.dev, uses_shared_paged_kv_idx=shared)
    kd, vd, ks, vs = cache.tensors
    nbytes = materialize_bytes(lens, ps, H, D, 32)
    fn = lambda: mat.run(kd, vd, ks, vs, bt_t, sl, ip, out=out, fp8_block_tables=tab)   # noqa: E731
    if samples is not None:
        out.view(torch.uint8).fill_(0x5A)
        tab.fill_(-1)
        fn()
        torch.cuda.synchronize()
        order = np.argsort(lens)
        picks = sorted({int(order[0]), int(order[len(lens) // 2]), int(order[-1])})
        reqs = []
        for b in picks:
            n = int((lens[b] + ps - 1) // ps)
            pages = np.concatenate([bt[b, :n], bt[b, :n]] if shared else [bt[b, 0, :n], bt[b, 1, :n]])
            dst = int(indptr[b]) + 1
            reqs.append(SimpleNamespace(b=b, n=n, cache=gather_pages(cache, pages), len=int(lens[b]),
                                        out=out.view(torch.uint8)[dst:dst + n].cpu().numpy(),
                                        table=tab[b].cpu().numpy(), dst=dst))
        what = "materialize workload" if placement == "shuffled" else f"materialize page-order context ({placement})"
        samples.add("materialize", f"{what}: shortest, median and longest requests", reqs=reqs,
                    page0=out.view(torch.uint8)[0].cpu().numpy(), H=H, ps=ps, D=D, maxp=maxp)
    return fn, nbytes, (cache, keep, out)


def leg_materialize(env, iters, warmup, samples):
    fns, keep = [], []
    for i in range(replicas_for(222_000_000)):
        fn, nbytes, k = materialize_replica(env, samples=samples if i == 0 else None)
        fns.append(fn)
        keep.append(k)
    r = env.steady(fns, iters, warmup)
    return dict(kernel="kv_materialize_fp8", workload="materialize_fp8: 32 requests, lengths log-uniform "
                "[128, 32768], page_size 16, 8 heads, head_dim 128, HND, data page stride 8448 B, separate K/V "
                "tables, compact kv_page_indptr, interleaved V scales", bytes=nbytes, **rates(nbytes, r))


def leg_materialize_page_order(env, iters, warmup, samples):
    """Context, not a workload of the method: the materialize workload's
    lengths and bytes with three page placements (separate shuffled K and V
    tables, as timed above; one shuffled table shared by K and V; pages in
    request order). The spread is what placement costs at the DRAM level."""
    torch = env.torch
    res = {"workload": "materialize_fp8 lengths and geometry; pages shuffled with separate K/V tables, shuffled "
                       "with a shared table, or in request order"}
    for placement in ("shuffled", "shuffled_shared", "request_order"):
        fns, keep = [], []
        for i in range(replicas_for(222_000_000)):
            fn, nbytes, k = materialize_replica(env, 1004, samples if i == 0 else None, placement)
            fns.append(fn)
            keep.append(k)
        res[placement] = dict(kernel="kv_materialize_fp8", bytes=nbytes,
                              **rates(nbytes, env.steady(fns, iters, warmup)))
        del fns, keep
        torch.cuda.empty_cache()
    return res


def four_over_six_replica(env, seed=1005):
    torch, K = env.torch, env.K
    B, T, ps, H, D = 16, 4096, 64, 8, 128
    rng = np.random.default_rng(seed)
    n_pages = B * T // ps
    perm = rng.permutation(n_pages)
    cache, keep = env.cache(n_pages, ps, H, D, K.KVFP4_NHD, seed)
    g = env.gen(seed)
    key = student_t3(env, (B * T, H, D), g).to(torch.bfloat16)
    val = student_t3(env, (B * T, H, D), g).to(torch.bfloat16)
    gk = torch.empty(1, dtype=torch.float32, device=env.dev)
    gv = torch.empty(1, dtype=torch.float32, device=env.dev)
    K.kv_global_scale(key, 256.0, gk)
    K.kv_global_scale(val, 256.0, gv)
    bi = env.i32(np.repeat(np.arange(B), T))
    pos = env.i32(np.tile(np.arange(T), B))
    ind = env.i32(perm)
    ptr = env.i32(np.arange(B + 1) * (T // ps))
    last = env.i32(np.full(B, ps))
    gkf, gvf = gk.item(), gv.item()
    bt = env.i32(perm.reshape(B, T // ps))
    ok = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=env.dev)
    ov = torch.empty_like(ok)
    sl = env.i32(np.full(B, T))
    fns = {}
    for name, recipe in (("mse", K.Recipe(256.0, K.KVFP4_ERR_MSE)), ("mae", K.Recipe(256.0, K.KVFP4_ERR_MAE)),
                         ("mse16", K.Recipe(256.0, K.KVFP4_ERR_MSE, True)),
                         ("mae16", K.Recipe(256.0, K.KVFP4_ERR_MAE, True)), ("standard", None)):
        fns["append_" + name] = (lambda r=recipe: K.kv_quantize_append(cache, key, val, bi, pos, ind, ptr, last,
                                                                       gkf, gvf, r))
    fns["dequant"] = lambda: K.kv_dequantize_paged(cache, bt, sl, gk, gv, ok, ov)
    return fns, (cache, keep, key, val, ok, ov, bi, pos, ind, ptr, last, bt, sl, gk, gv)


def leg_four_over_six(env, iters, warmup, samples):
    torch = env.torch
    # the append reads 268 MB of rows, the dequant 75 MB of cache per replica
    reps = [four_over_six_replica(env) for _ in range(replicas_for(75_000_000))]
    B, T, H, D, ps = 16, 4096, 8, 128, 64
    res = {}
    ab = append_bytes(B * T, H, D)
    # request 9 of the first replica: its rows, and its pages after each call
    cache0, key0, val0, ind0 = reps[0][1][0], reps[0][1][2], reps[0][1][3], reps[0][1][8]
    sb = 9
    pages = ind0[sb * (T // ps):(sb + 1) * (T // ps)].cpu().numpy()
    rows = (host_bits(key0[sb * T:(sb + 1) * T]), host_bits(val0[sb * T:(sb + 1) * T]))
    g = (reps[0][1][13].item(), reps[0][1][14].item())
    for name, recipe in (("mse", "4over6 e4m3_max=256 MSE"), ("mae", "4over6 e4m3_max=256 MAE"),
                         ("mse16", "4over6 e4m3_max=256 MSE, error in fp16"),
                         ("mae16", "4over6 e4m3_max=256 MAE, error in fp16"), ("standard", "standard amax/6")):
        reps[0][0]["append_" + name]()
        torch.cuda.synchronize()
        samples.add("four_over_six_append", f"4over6 workload, request {sb}: append {recipe}", recipe=name,
                    rows=rows, cache=gather_pages(cache0, pages), g=g, T=T)
        r = env.steady([rep[0]["append_" + name] for rep in reps], iters, warmup)
        res["append_" + name] = dict(kernel="kv_quantize_append", recipe=recipe, bytes=ab, **rates(ab, r))
    db = dequant_bytes(np.full(B, T), ps, H, D, 4)
    reps[0][0]["dequant"]()
    torch.cuda.synchronize()
    ok0, ov0 = reps[0][1][4], reps[0][1][5]
    samples.add("dequant", f"4over6 workload, request {sb}: dequant", cache=gather_pages(cache0, pages), g=g,
                out=(host_bits(ok0[sb]), host_bits(ov0[sb])), len=T, bf16=True)
    r = env.steady([rep[0]["dequant"] for rep in reps], iters, warmup)
    res["dequant"] = dict(kernel="kv_dequantize_paged", bytes=db, **rates(db, r))
    res["workload"] = ("four_over_six_quantize: 65,536 rows (16 x 4096), 8 heads, head_dim 128, bf16 Student-t(3) "
                       "with 0.1% entries x20, page_size 64 NHD, recipe-matched global scale")
    del reps
    torch.cuda.empty_cache()
    return res


def codec_bytes(n_elems):
    """16-bit values one way, packed codes and scales the other, plus g"""
    return 2 * n_elems + n_elems // 2 + n_elems // 16 + 4


def leg_contiguous(env, iters, warmup, samples):
    """kv_quantize / kv_dequantize of the 4over6 workload's K tensor seen as
    a contiguous [65536, 1024] bf16 matrix (Student-t(3), 0.1% outliers)."""
    torch, K = env.torch, env.K
    rows, cols = 65536, 8 * 128
    reps = []
    for i in range(replicas_for(rows * cols * 2)):
        g = env.gen(3000 + i)
        x = student_t3(env, (rows, cols), g).to(torch.bfloat16)
        gs = torch.empty(1, dtype=torch.float32, device=env.dev)
        K.kv_global_scale(x, 256.0, gs)
        d = torch.empty((rows, cols // 2), dtype=torch.uint8, device=env.dev)
        sc = torch.empty((rows, cols // 16), dtype=torch.uint8, device=env.dev)
        y = torch.empty_like(x)
        reps.append((x, gs, d, sc, y))
    nb = codec_bytes(rows * cols)
    res = {"workload": "contiguous [65536, 1024] bf16, Student-t(3) with 0.1% entries x20, global scale for "
                       "e4m3_max 256"}
    r0 = reps[0]
    lo, hi = 30000, 30256                              # the sampled rows of the first replica
    g0 = r0[1].item()
    for name, rec in (("quantize_standard", None), ("quantize_mse", K.Recipe(256.0, K.KVFP4_ERR_MSE)),
                      ("quantize_mae", K.Recipe(256.0, K.KVFP4_ERR_MAE))):
        fns = [(lambda r=r, rec=rec: K.kv_quantize(r[0], r[1], r[2], r[3], rec)) for r in reps]
        fns[0]()
        torch.cuda.synchronize()
        samples.add("contiguous_quantize", f"contiguous codec, rows {lo}..{hi - 1}: {name}", recipe=name,
                    x=host_bits(r0[0][lo:hi]), codes=r0[2][lo:hi].cpu().numpy(), scales=r0[3][lo:hi].cpu().numpy(),
                    g=g0)
        res[name] = dict(kernel="kv_quantize", bytes=nb, **rates(nb, env.steady(fns, iters, warmup)))
    fns = [(lambda r=r: K.kv_dequantize(r[2], r[3], r[1], r[4])) for r in reps]
    fns[0]()
    torch.cuda.synchronize()
    samples.add("contiguous_dequantize", f"contiguous codec, rows {lo}..{hi - 1}: dequantize",
                codes=r0[2][lo:hi].cpu().numpy(), scales=r0[3][lo:hi].cpu().numpy(), g=g0,
                out=host_bits(r0[4][lo:hi]))
    res["dequantize"] = dict(kernel="kv_dequantize", bytes=nb, **rates(nb, env.steady(fns, iters, warmup)))
    del reps
    torch.cuda.empty_cache()
    return res


def leg_pool_quantize(env, iters, warmup, samples):
    """kv_quantize_paged_cache of a bf16 N(0,1) pool in the materialize
    workload's geometry (12,070 HND pages of 16 tokens, 8 heads, head_dim
    128), V scales 4-token interleaved, standard recipe."""
    torch, K = env.torch, env.K
    P, ps, H, D = 12070, 16, 8, 128
    reps = []
    for i in range(replicas_for(2 * P * ps * H * D * 2)):
        g = env.gen(4000 + i)
        k = torch.randn((P, H, ps, D), generator=g, device=env.dev).to(torch.bfloat16)
        v = torch.randn((P, H, ps, D), generator=g, device=env.dev).to(torch.bfloat16)
        gk = torch.empty(1, dtype=torch.float32, device=env.dev)
        gv = torch.empty(1, dtype=torch.float32, device=env.dev)
        K.kv_global_scale(k, 448.0, gk)
        K.kv_global_scale(v, 448.0, gv)
        cache, keep = env.cache(P, ps, H, D, K.KVFP4_HND, 4100 + i)
        reps.append((k, v, gk, gv, cache, keep))
    nb = 2 * codec_bytes(P * ps * H * D)
    fns = [(lambda r=r: K.kv_quantize_paged_cache(r[4], r[0], r[1], r[2], r[3], None, True)) for r in reps]
    fns[0]()
    torch.cuda.synchronize()
    r0 = reps[0]
    pages = np.arange(5000, 5032)
    samples.add("pool_quantize", "whole-pool quantize, pages 5000..5031", k=host_bits(r0[0][5000:5032]),
                v=host_bits(r0[1][5000:5032]), g=(r0[2].item(), r0[3].item()), cache=gather_pages(r0[4], pages))
    res = dict(kernel="kv_quantize_paged_cache", bytes=nb, **rates(nb, env.steady(fns, iters, warmup)))
    res["workload"] = ("whole-pool quantize: 12,070 HND pages x (16 tokens, 8 heads, head_dim 128), bf16 N(0,1) "
                       "K and V, standard recipe, V scales 4-token interleaved")
    del reps
    torch.cuda.empty_cache()
    return res


def attention_bytes(lens, ps, H, D, Hq):
    """K and V codes and scales of every valid (token, kv head), q in and out
    (bf16), the block-table entries used and seq_lens"""
    tokens = int(np.sum(lens))
    pages = int(np.sum((np.asarray(lens) + ps - 1) // ps))
    B = len(lens)
    return 2 * tokens * H * (D // 2 + D // 16) + 2 * B * Hq * D * 2 + 4 * pages + 4 * B


def attention_sample(env, samples, label, cache, r, sm, picks):
    torch = env.torch
    torch.cuda.synchronize()
    reqs = []
    for b in picks:
        n = int((r.lens[b] + r.ps - 1) // r.ps)
        pages = r.bt[b, :n].cpu().numpy()
        reqs.append(SimpleNamespace(b=b, len=int(r.lens[b]), cache=gather_pages(cache, pages),
                                    q=host_bits(r.q[b]), out=host_bits(r.att_out[b])))
    samples.add("attention", label, reqs=reqs, g=(r.gk, r.gv), sm=sm, G=r.q.shape[1] // r.H)


def leg_attention(env, iters, warmup, samples, G=4):
    """kv_decode_attention on the decode workload's cache (64 requests,
    124,503 tokens, page 16, 8 kv heads x 4 query heads, NHD, bf16), and on
    an HND pool with the same lengths and pages."""
    torch, K = env.torch, env.K
    reps = [Decode(env) for _ in range(replicas_for(144_000_000))]
    r0 = reps[0]
    Hq = r0.H * G
    sm = 1.0 / float(np.sqrt(r0.D))
    nb = attention_bytes(r0.lens, r0.ps, r0.H, r0.D, Hq)
    res = {"workload": "decode attention: the decode workload's cache (64 requests, 124,503 tokens, page_size 16, "
                       "8 kv heads, head_dim 128), 4 query heads per kv head, bf16 q/out, sm_scale 1/sqrt(128)"}
    fns = []
    for i, r in enumerate(reps):
        g = env.gen(5000 + i)
        r.q = torch.randn((r.B, Hq, r.D), generator=g, device=env.dev).to(torch.bfloat16)
        r.att_out = torch.empty_like(r.q)
        r.ws = torch.empty(K.kv_decode_attention_workspace_size(r.B, r.H, Hq, r.bt.shape[1], r.ps), dtype=torch.uint8,
                           device=env.dev)
        fns.append(lambda r=r: K.kv_decode_attention(r.cache, r.q, r.bt, r.seq_lens, r.gk_t, r.gv_t, sm, r.att_out,
                                                     r.ws))
    order = np.argsort(r0.lens)
    picks = [int(order[0]), int(order[-1])]
    fns[0]()
    attention_sample(env, samples, "decode attention (NHD): shortest and longest requests", r0.cache, r0, sm, picks)
    res["nhd"] = dict(kernel="kv_decode_attention", bytes=nb, **rates(nb, env.steady(fns, iters, warmup)))
    fns = []
    for i, r in enumerate(reps):
        r.hnd_cache, r.hnd_keep = env.cache(20000, r.ps, r.H, r.D, K.KVFP4_HND, 6000 + i)
        fns.append(lambda r=r: K.kv_decode_attention(r.hnd_cache, r.q, r.bt, r.seq_lens, r.gk_t, r.gv_t, sm,
                                                     r.att_out, r.ws))
    fns[0]()
    attention_sample(env, samples, "decode attention (HND): shortest and longest requests", r0.hnd_cache, r0, sm,
                     picks)
    res["hnd"] = dict(kernel="kv_decode_attention", bytes=nb, **rates(nb, env.steady(fns, iters, warmup)))
    del reps, fns
    torch.cuda.empty_cache()
    return res


def page_order_replica(env, order, seed, samples=None):
    """64 full 4096-token requests in decode geometry (page_size 16, 8 heads,
    head_dim 128, NHD, bf16 out); `order` "random" shuffles the 16,384 pages
    over the requests, "sequential" gives request b pages 256 b .. 256 b + 255."""
    torch, K = env.torch, env.K
    B, T, ps, H, D = 64, 4096, 16, 8, 128
    P = B * T // ps
    cache, keep = env.cache(P, ps, H, D, K.KVFP4_NHD, seed)
    if order == "random":
        bt = torch.randperm(P, generator=env.gen(seed + 1), device=env.dev).to(torch.int32).view(B, T // ps)
    else:
        bt = torch.arange(P, dtype=torch.int32, device=env.dev).view(B, T // ps)
    sl = env.i32(np.full(B, T))
    ok = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=env.dev)
    ov = torch.empty_like(ok)
    g = torch.ones(1, dtype=torch.float32, device=env.dev)
    nbytes = dequant_bytes(np.full(B, T), ps, H, D, 4)
    fn = K.prepare_dequantize_paged(cache, bt, sl, g, g, ok, ov).launch
    if samples is not None:
        b = 33
        fn()
        torch.cuda.synchronize()
        samples.add("dequant", f"page-order context ({order} pages), request {b}",
                    cache=gather_pages(cache, bt[b].cpu().numpy()), g=(1.0, 1.0),
                    out=(host_bits(ok[b]), host_bits(ov[b])), len=T, bf16=True)
    return fn, nbytes, (cache, keep, bt, sl, ok, ov, g)


def leg_page_order(env, iters, warmup, samples):
    """Context, not a workload of the method: the same dequant over the same
    bytes, with the physical pages in request order or shuffled. The gap is
    what scattered page placement costs at the DRAM level."""
    torch = env.torch
    res = {"workload": "64 x 4096 tokens, page_size 16, 8 heads, head_dim 128, NHD, bf16 out; 16,384 pages in "
                       "request order vs shuffled"}
    for order in ("sequential", "random"):
        fns, keep = [], []
        for i in range(2):
            fn, nbytes, k = page_order_replica(env, order, 2000 + i, samples if i == 0 else None)
            fns.append(fn)
            keep.append(k)
        res[order] = dict(kernel="kv_dequantize_paged", bytes=nbytes, **rates(nbytes, env.steady(fns, iters, warmup)))
        del fns, keep
        torch.cuda.empty_cache()
    return res


def leg_copy(env, nbytes, iters, warmup):
    torch = env.torch
    pairs = []
    for _ in range(replicas_for(nbytes // 2)):
        src = torch.ones(nbytes // 2, dtype=torch.uint8, device=env.dev)
        pairs.append((src, torch.empty_like(src)))
    r = env.steady([(lambda s=s, d=d: d.copy_(s)) for s, d in pairs], iters, warmup)
    return dict(kernel="torch copy_ (device to device)", bytes=nbytes, **rates(nbytes, r))


DEQUANT_SOURCES = ("kv_cache_quantization_paged_amd/csrc/dequant.hip",
                   "kv_cache_quantization_paged_amd/csrc/quant_block.h",
                   "kv_cache_quantization_paged_amd/csrc/nvfp4_device.h",
                   "kv_cache_quantization_paged_amd/csrc/kvfp4_internal.h")
TRAFFIC_SUMMARY = "profiles/kv_append_dequantize_paged_decode_counters.md"


def dequant_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in DEQUANT_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the decode step's kernel from the committed
    rocprofv3 counter summary, or None when the kernel's sources have
    changed since those counters were taken."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if "=" in line and line.strip().startswith(("traffic_bytes_per_launch", "source_sha256")):
            k, v = line.strip().strip("`").split("=", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != dequant_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def graph_latency(env, fns, per_graph, replays):
    """Mean time per call of fns[i % len(fns)] captured `per_graph` times
    into one HIP graph and replayed `replays` times (ms)."""
    torch = env.torch
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fns[i % len(fns)]()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * per_graph)
    del g
    return ms


def replicas_for(read_bytes: int) -> int:
    """Replicas whose inputs together exceed ~2.5x the 256 MB Infinity Cache,
    so every launch reads its inputs from HBM, as a serving step does (a
    layer's cache is read again only after every other layer has run)."""
    return max(2, -(-640_000_000 // max(1, read_bytes)))


def rates(nbytes, r):
    avg, med = r
    return {"us_avg": avg * 1e3, "us_median": med * 1e3, "GBps": nbytes / (avg * 1e6),
            "frac": nbytes / (avg * 1e6) / PEAK_GBS}


# ---------------------------------------------------------------------------
# samples of the timed buffers (host copies; the CPU leg checks them)
# ---------------------------------------------------------------------------
class Samples:
    """Host copies of sampled inputs and outputs of the timed workloads,
    taken right after each leg's first launch on its first replica."""

    def __init__(self, enabled=True):
        self.enabled = enabled
        self.items = []

    def add(self, kind, label, **data):
        if self.enabled:
            self.items.append(SimpleNamespace(kind=kind, label=label, **data))


def host_bits(t):
    """a 16-bit float tensor's bit patterns on the host"""
    return t.contiguous().view(env_torch().int16).cpu().numpy().view(np.uint16)


def env_torch():
    import torch
    return torch


def gather_pages(cache, pages):
    """the listed pages of a device cache as a compact host cache (page i of
    the copy is pages[i]), in the layout the oracle reads"""
    torch = env_torch()
    idx = torch.as_tensor(np.asarray(pages, np.int64), device=cache.tensors[0].device)
    arrs = [t.index_select(0, idx).contiguous().view(len(pages), -1).cpu().numpy() for t in cache.tensors]
    return SimpleNamespace(k_data=arrs[0], v_data=arrs[1], k_sf=arrs[2], v_sf=arrs[3], page_size=cache.page_size,
                           num_heads=cache.num_kv_heads, head_dim=cache.head_dim, layout=cache.layout)


def whole_cache(cache):
    """every page of a device cache on the host (same layout, compact)"""
    return gather_pages(cache, np.arange(cache.num_pages))


# ---------------------------------------------------------------------------
# CPU leg: the oracle. It first checks every sample of the timed buffers (bit
# for bit; decode attention within the bound its arithmetic gives), then it
# is timed on the decode step. Nothing else in this file runs the oracle.
# ---------------------------------------------------------------------------
def _host_cache_like(c, zero):
    f = np.zeros_like if zero else np.copy
    return SimpleNamespace(k_data=f(c.k_data), v_data=f(c.v_data), k_sf=f(c.k_sf), v_sf=f(c.v_sf),
                           page_size=c.page_size, num_heads=c.num_heads, head_dim=c.head_dim, layout=c.layout)


def _same_cache(a, b):
    return all(np.array_equal(x, y) for x, y in ((a.k_data, b.k_data), (a.v_data, b.v_data), (a.k_sf, b.k_sf),
                                                  (a.v_sf, b.v_sf)))


def _oracle_recipe(oracle, name):
    if name.endswith("standard"):
        return oracle.STANDARD
    return oracle.four_over_six(oracle.MSE if "mse" in name else oracle.MAE, fast_math=name.endswith("16"))


def _oracle_dequant_one(oracle, cache, n_len, g, bf16, threads):
    """the oracle's dequant of a one-request cache whose pages are in table order"""
    n_pages = cache.k_data.shape[0]
    H, D = cache.num_heads, cache.head_dim
    ok = np.full((1, n_len, H, D), 0xA5A5, np.uint16)
    ov = ok.copy()
    oracle.dequantize_paged(cache, np.arange(n_pages, dtype=np.int32)[None], np.array([n_len], np.int32), g[0], g[1],
                            ok, ov, bf16, threads=threads)
    return ok[0], ov[0]


def cpu_check_decode_step(oracle, it, threads):
    host = _host_cache_like(it.pre, zero=False)
    if it.history is not None:
        # the pre-step cache holds the library's quantization of this
        # request's history: the oracle writing the same rows changes nothing
        b, hk, hv = it.history
        n = int(it.old[b])
        oracle.quantize_append(host, hk, hv, True, np.full(n, b, np.int32), np.arange(n, dtype=np.int32), it.indices,
                               it.indptr, it.last, it.gk, it.gv, threads=threads)
        if not _same_cache(host, it.pre):
            return f"history of request {b} differs from the oracle's quantization"
    oracle.quantize_append(host, it.key, it.value, True, it.bi, it.pos, it.indices, it.indptr, it.last, it.gk, it.gv,
                           threads=threads)
    if not _same_cache(host, it.post):
        return "the cache after the append differs from the oracle's"
    for b, (gk_out, gv_out) in it.outs.items():
        n = int(it.lens[b])
        ok = np.full((1, n) + gk_out.shape[1:], 0xA5A5, np.uint16)
        ov = ok.copy()
        oracle.dequantize_paged(it.post, np.ascontiguousarray(it.bt[b:b + 1]), it.lens[b:b + 1], it.gk, it.gv, ok, ov,
                                True, threads=threads)
        if not (np.array_equal(ok[0], gk_out) and np.array_equal(ov[0], gv_out)):
            return f"dequant of request {b} differs"
    return None


def cpu_check_prefill(oracle, it, threads):
    mini = _host_cache_like(it.cache, zero=True)
    n_pages = mini.k_data.shape[0]
    oracle.quantize_append(mini, it.rows[0], it.rows[1], True, np.zeros(it.T, np.int32), np.arange(it.T, dtype=np.int32),
                           np.arange(n_pages, dtype=np.int32), np.array([0, n_pages], np.int32),
                           np.array([it.cache.page_size], np.int32), it.g[0], it.g[1], threads=threads)
    if not _same_cache(mini, it.cache):
        return f"quantization of request {it.b} differs"
    ok, ov = _oracle_dequant_one(oracle, it.cache, it.T, it.g, False, threads)
    if not (np.array_equal(ok, it.out[0]) and np.array_equal(ov, it.out[1])):
        return f"dequant of request {it.b} differs"
    return None


def cpu_check_materialize(oracle, it, threads):
    if np.any(it.page0 != 0):
        return "page 0 is not zero"
    for r in it.reqs:
        n = r.n
        bt = np.stack([np.arange(n), n + np.arange(n)]).astype(np.int32)[None]
        out = np.full((n + 1, 2, it.H, it.ps, it.D), 0x5A, np.uint8)
        tab = np.full((1, n), -1, np.int32)
        oracle.materialize_fp8(r.cache, bt, np.array([r.len], np.int32), np.array([0, n], np.int32), out, tab,
                               shared=False, v_sf_interleaved=True, threads=threads)
        if not np.array_equal(out[1:], r.out):
            return f"FP8 pages of request {r.b} differ"
        if not (np.array_equal(tab[0] - 1 + r.dst, r.table[:n]) and np.all(r.table[n:] == -1)):
            return f"FP8 block-table row {r.b} differs"
    return None


def cpu_check_four_over_six_append(oracle, it, threads):
    mini = _host_cache_like(it.cache, zero=True)
    n_pages = mini.k_data.shape[0]
    oracle.quantize_append(mini, it.rows[0], it.rows[1], True, np.zeros(it.T, np.int32), np.arange(it.T, dtype=np.int32),
                           np.arange(n_pages, dtype=np.int32), np.array([0, n_pages], np.int32),
                           np.array([it.cache.page_size], np.int32), it.g[0], it.g[1],
                           _oracle_recipe(oracle, it.recipe), threads=threads)
    return None if _same_cache(mini, it.cache) else f"{it.recipe} codes or scales differ"


def cpu_check_dequant(oracle, it, threads):
    ok, ov = _oracle_dequant_one(oracle, it.cache, it.len, it.g, it.bf16, threads)
    return None if np.array_equal(ok, it.out[0]) and np.array_equal(ov, it.out[1]) else "dequant differs"


def cpu_check_contiguous_quantize(oracle, it, threads):
    codes, scales = oracle.quantize_contiguous(it.x, True, it.g, _oracle_recipe(oracle, it.recipe), threads=threads)
    return None if np.array_equal(codes, it.codes) and np.array_equal(scales, it.scales) else "codes or scales differ"


def cpu_check_contiguous_dequantize(oracle, it, threads):
    out = oracle.dequantize_contiguous(it.codes, it.scales, it.g, True, threads=threads)
    return None if np.array_equal(out, it.out) else "values differ"


def cpu_check_pool_quantize(oracle, it, threads):
    mini = _host_cache_like(it.cache, zero=True)
    oracle.quantize_paged_cache(mini, it.k, it.v, True, it.g[0], it.g[1], oracle.STANDARD, v_sf_interleaved=True,
                                threads=threads)
    return None if _same_cache(mini, it.cache) else "pages differ"


def cpu_check_attention(oracle, it, threads):
    """|gpu - exact| <= 2u (max|V| + |exact|), u = 2^-9 for bf16 out: one fp16
    rounding of each probability and one of the output (the kernel's
    arithmetic; K and V are exact in fp16)"""
    e4 = np.array([abs(oracle.e4m3_value(b)) if (b & 0x7F) != 0x7F else 0.0 for b in range(256)])
    u = 2.0 ** -9
    for r in it.reqs:
        c = r.cache
        n, ps, H, D = c.k_data.shape[0], c.page_size, c.num_heads, c.head_dim
        want = oracle.decode_attention(c, r.q[None], True, np.arange(n, dtype=np.int32)[None],
                                       np.array([r.len], np.int32), it.g[0], it.g[1], it.sm, threads=threads)[0]
        got = (r.out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        sf = c.v_sf.reshape((n, ps, H, D // 16) if c.layout == 0 else (n, H, ps, D // 16))
        if c.layout != 0:
            sf = sf.transpose(0, 2, 1, 3)
        vals = e4[sf.reshape(n * ps, H, D // 16)[:r.len]]              # [tokens, H, blocks]
        vmax = 6.0 * vals.max(axis=(0, 2)) * it.g[1]                     # per kv head
        for hq in range(got.shape[0]):
            tol = 2 * u * (vmax[hq // it.G] + np.abs(want[hq]))
            if not np.all(np.abs(got[hq] - want[hq]) <= tol):
                return f"request {r.b}, query head {hq} is outside the bound"
    return None


CPU_CHECKS = {"decode_step": cpu_check_decode_step, "prefill": cpu_check_prefill,
              "materialize": cpu_check_materialize, "four_over_six_append": cpu_check_four_over_six_append,
              "dequant": cpu_check_dequant, "contiguous_quantize": cpu_check_contiguous_quantize,
              "contiguous_dequantize": cpu_check_contiguous_dequantize, "pool_quantize": cpu_check_pool_quantize,
              "attention": cpu_check_attention}


def cpu_parity(samples: Samples, threads: int):
    """every sample against the oracle; returns (report, failures)"""
    import oracle
    report, failures = [], []
    for it in samples.items:
        t0 = time.perf_counter()
        err = CPU_CHECKS[it.kind](oracle, it, threads)
        report.append({"sample": it.label, "ok": err is None, "seconds": round(time.perf_counter() - t0, 2)})
        if err is not None:
            failures.append(f"{it.label}: {err}")
            report[-1]["error"] = err
        log(f"bench: parity {'ok ' if err is None else 'FAIL'} {it.label}" + ("" if err is None else f": {err}"))
    return report, failures


def cpu_baseline(min_seconds: float, ps=16, H=8, D=128, pool=20000, seed=1002):
    """The oracle on the host cores: the whole decode step (quantize-append of
    the 64 new tokens, then dequantize of the full 124,503-token context),
    repeated until at least `min_seconds` have passed (3 times at least) on
    every core the process may run on, then once on one thread; the median
    step time gives each rate. The history is quantized first, by the oracle,
    outside the timing."""
    import oracle
    import workloads as W
    rng = np.random.default_rng(seed)
    old, new_len, indices, indptr, last, bt = W.decode_append_tables(rng, 64, 4096, pool, ps)
    a_k, a_v = W.head_scales(rng, H), W.head_scales(rng, H)
    B = len(old)
    cores = len(os.sched_getaffinity(0))
    cache = W.make_cache(rng, pool, ps, H, D, W.NHD, fill="zero")
    hist = int(old.sum())
    hk = W.f32_to_bits(W.head_scaled_normal(rng, hist, a_k, D), True)
    hv = W.f32_to_bits(W.head_scaled_normal(rng, hist, a_v, D), True)
    nk = W.f32_to_bits(W.head_scaled_normal(rng, B, a_k, D), True)
    nv = W.f32_to_bits(W.head_scaled_normal(rng, B, a_v, D), True)
    gk = oracle.global_scale(np.concatenate([hk.ravel(), nk.ravel()]), True)
    gv = oracle.global_scale(np.concatenate([hv.ravel(), nv.ravel()]), True)
    hb, hp = W.rows_for_positions(np.zeros(B, np.int64), old)
    oracle.quantize_append(cache, hk, hv, True, hb, hp, indices, indptr, last, gk, gv, threads=cores)
    del hk, hv
    T = int(new_len.max())
    ok = np.zeros((B, T, H, D), np.uint16)
    ov = np.zeros_like(ok)
    bi, pos = np.arange(B, dtype=np.int32), old.astype(np.int32)
    lens = new_len.astype(np.int32)
    nbytes = append_bytes(B, H, D) + dequant_bytes(new_len, ps, H, D, 4)

    def step(threads):
        t0 = time.perf_counter()
        oracle.quantize_append(cache, nk, nv, True, bi, pos, indices, indptr, last, gk, gv, threads=threads)
        oracle.dequantize_paged(cache, bt, lens, gk, gv, ok, ov, True, threads=threads)
        return time.perf_counter() - t0

    times = []
    t_all = time.perf_counter()
    while len(times) < 3 or time.perf_counter() - t_all < min_seconds:
        times.append(step(cores))
    dt = statistics.median(times)
    wall = time.perf_counter() - t_all
    dt1 = step(1)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seconds_per_step": dt, "steps": len(times),
            "one_thread": {"value": nbytes / dt1 / 1e9, "unit": "GB/s", "cores": 1, "seconds_per_step": dt1,
                           "steps": 1},
            "sample": f"the whole decode step (quantize-append of 64 new tokens + dequantize of the full "
                      f"{int(new_len.sum())}-token context): {len(times)} repetitions in {wall:.1f} s on the "
                      f"{cores} cores of the process's CPU affinity (median step time), then one step on one "
                      f"thread ({dt1:.1f} s)"}


def host_cost_leg(env, reps_n=5, calls=40):
    """Host microseconds per eager call (the Python call through the C ABI
    up to the return of the launch), median of reps_n runs of `calls` calls
    issued back to back after a synchronization, so the GPU queue never
    fills: the functional calls (every tensor checked each time) against the
    prepared ones (checked once, kvfp4_launch after that)."""
    torch, K = env.torch, env.K
    r = Decode(env)
    fn, _, keep = materialize_replica(env)
    mat_cache, _, mat_out = keep
    torch.cuda.synchronize()

    def host_us(f):
        runs = []
        for _ in range(reps_n):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(calls):
                f()
            runs.append((time.perf_counter() - t0) / calls * 1e6)
        torch.cuda.synchronize()
        return statistics.median(runs)

    kd, vd, ks, vs = mat_cache.tensors
    import workloads as W
    lens, P, maxp, bt, indptr = W.materialize_tables(np.random.default_rng(1004), 32, 128, 32768, 16)
    bt_t, sl, ip = env.i32(bt), env.i32(lens), env.i32(indptr)
    tab = torch.zeros((32, maxp), dtype=torch.int32, device=env.dev)

    def functional_materialize():
        K.kv_materialize_fp8(mat_cache, bt_t, sl, ip, mat_out, tab, False, True)

    res = {"append_functional_us": host_us(r.append_eager), "append_prepared_us": host_us(r.append),
           "dequant_functional_us": host_us(r.dequant_eager), "dequant_prepared_us": host_us(r.dequant),
           "append_dequant_prepared_us": host_us(r.step),
           "materialize_functional_us": host_us(functional_materialize),
           "materializer_run_us": host_us(fn),
           "note": "host time per eager call, decode workload (append, dequant) and materialize workload"}
    del r, keep
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps before each timed run (the clocks and page tables settle within a few ms)")
    ap.add_argument("--leg-iters", type=int, default=50)
    ap.add_argument("--legs", default="prefill,materialize,four_over_six,contiguous,pool_quantize,attention,"
                                      "page_order,materialize_page_order,copy,host_cost",
                    help="comma list of legs to run after the headline step (empty: none)")
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle's timing (parity still runs)")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle's checks of the timed buffers")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="minimum host time spent timing the oracle on all cores (whole decode steps)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged NVFP4 path needs no collectives and this library has no "
              "multi-GPU step (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    env = Env()
    samples = Samples(enabled=not args.no_parity)
    n_rep = replicas_for(144_000_000)
    log(f"bench: building the decode workload ({n_rep} replicas)")
    picks = [0, 17, 40]                                   # requests whose outputs are checked
    reps = [Decode(env, keep_history_of=17 if i == 0 and samples.enabled else None) for i in range(n_rep)]
    torch.cuda.synchronize()
    if samples.enabled:
        order = np.argsort(reps[0].lens)
        picks = sorted(set(picks) | {int(order[0]), int(order[-1])})
        reps[0].sample_step(samples, picks)

    def step(i):
        reps[i % n_rep].step()

    def step_two_calls(i):
        r = reps[i % n_rep]
        r.append()
        r.dequant()

    def wall_ms(fn):
        # the timed region holds the steps alone: an event recorded between
        # two kernels adds a few microseconds of gap to every step (measured:
        # 127 vs 121 us per two-call step), which no serving loop has
        with quiet_host():
            for i in range(args.warmup):
                fn(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                fn(i)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / args.steps

    log(f"bench: timing {args.steps} steps")
    ms_step = wall_ms(step)
    log(f"bench: timing {args.steps} steps as two calls (append, then dequant)")
    ms_two = wall_ms(step_two_calls)
    # the step kernel's own launch time, for the roofline: as many launches
    # as timed steps, over the same replicas, back to back in three batches
    # bracketed by HIP events on the stream they are launched on
    log(f"bench: timing {args.steps} step launches and {args.steps} dequant launches")
    step_avg, step_med = env.steady([r.step for r in reps], args.steps, 5)
    deq_avg, deq_med = env.steady([r.dequant for r in reps], args.steps, 5)
    step_bytes = reps[0].append_bytes + reps[0].dequant_bytes
    value = step_bytes / (ms_step * 1e6)
    achieved = step_bytes / (step_avg * 1e6)
    deq_rate = reps[0].dequant_bytes / (deq_avg * 1e6)

    # append latency of the decode step: eager launches are bound by the
    # host-side launch path at this size, so the kernel time comes from
    # replays of a HIP graph holding 20 back-to-back appends
    app_eager_ms = env.steady([r.append for r in reps], 50, 5)[0]
    app_ms = graph_latency(env, [r.append for r in reps], 20, 10)
    legs = {"decode_step_kernel": {"kernel": "kv_append_dequantize_paged", "bytes": step_bytes,
                                   "us_avg": step_avg * 1e3, "us_median": step_med * 1e3,
                                   "GBps": achieved, "frac": achieved / PEAK_GBS},
            "decode_step_two_calls": {"calls": "kv_quantize_append, then kv_dequantize_paged", "bytes": step_bytes,
                                      "us_per_step": ms_two * 1e3, "GBps": step_bytes / (ms_two * 1e6),
                                      "frac": step_bytes / (ms_two * 1e6) / PEAK_GBS},
            "decode_append_us": app_ms * 1e3, "decode_append_us_eager": app_eager_ms * 1e3,
            "decode_dequant": {"kernel": "kv_dequantize_paged", "bytes": reps[0].dequant_bytes,
                               "us_avg": deq_avg * 1e3, "us_median": deq_med * 1e3,
                               "GBps": deq_rate, "frac": deq_rate / PEAK_GBS}}
    del reps
    torch.cuda.empty_cache()
    chosen = set() if args.no_legs else {x for x in args.legs.split(",") if x}
    if chosen:
        log(f"bench: legs {sorted(chosen)}")
    if "prefill" in chosen:
        legs["prefill_dequantize"] = leg_prefill_dequant(env, args.leg_iters, 5, samples)
        torch.cuda.empty_cache()
    if "materialize" in chosen:
        legs["materialize_fp8"] = leg_materialize(env, args.leg_iters, 5, samples)
        torch.cuda.empty_cache()
    if "four_over_six" in chosen:
        legs["four_over_six_quantize"] = leg_four_over_six(env, args.leg_iters, 5, samples)
        torch.cuda.empty_cache()
    if "contiguous" in chosen:
        legs["contiguous_codec"] = leg_contiguous(env, args.leg_iters, 5, samples)
    if "pool_quantize" in chosen:
        legs["pool_quantize"] = leg_pool_quantize(env, args.leg_iters, 5, samples)
        torch.cuda.empty_cache()
    if "attention" in chosen:
        legs["decode_attention"] = leg_attention(env, args.leg_iters, 5, samples)
    if "page_order" in chosen:
        legs["page_order_context"] = leg_page_order(env, args.leg_iters, 5, samples)
    if "materialize_page_order" in chosen:
        legs["materialize_page_order_context"] = leg_materialize_page_order(env, args.leg_iters, 5, samples)
    if "copy" in chosen:
        # also the known-size copy that calibrates the byte counters
        legs["copy_context"] = leg_copy(env, 1 << 29, args.leg_iters, 5)
    if "host_cost" in chosen:
        legs["host_cost"] = host_cost_leg(env)

    # ---- the CPU leg: the oracle checks the timed buffers, then is timed
    cores = len(os.sched_getaffinity(0))
    parity = None
    if samples.enabled:
        log(f"bench: CPU leg: parity of {len(samples.items)} samples of the timed buffers ({cores} threads)")
        report, failures = cpu_parity(samples, cores)
        parity = {"checked": len(report), "passed": sum(r["ok"] for r in report), "samples": report}
        if failures:
            print("bench: PARITY FAILURE on the timed buffers:\n  " + "\n  ".join(failures), file=sys.stderr,
                  flush=True)
            sys.exit(3)
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU leg: oracle baseline")
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "decode_append: 64 requests x 1 new bf16 token (append) + dequantize of the full "
                               "context (124,503 tokens, bf16 out); page_size 16, 8 KV heads, head_dim 128, NHD, "
                               "20,000-page shuffled pool, lengths U{1..4096}+1, seed 1002; one "
                               "kv_append_dequantize_paged call per step",
                   "batch": 64, "page_size": 16, "num_kv_heads": 8, "head_dim": 128, "layout": "NHD",
                   "step_bytes": step_bytes, "peak_GBps": PEAK_GBS},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBS, "traffic": recorded_traffic(),
                     "kernel": "kv_append_dequantize_paged (append_dequant_kernel<NHD, bf16 out, int32 table, "
                               "bf16 in>)"},
        "cpu_baseline": cpu,
        "parity": parity,
        "legs": legs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
