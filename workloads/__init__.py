"""Seeded synthetic inputs for the paged NVFP4 KV-cache path.

This module is shared by the tests, the smoke check and the benchmark. It
draws random numbers and lays out page tables and caches; it holds none of
the quantization arithmetic (no scale, no rounding rule of the method, no
codec). 16-bit floats are produced from fp32 draws by torch's CPU casts.

Shapes follow the serving workloads the FlashInfer KV-cache pages describe
(nvfp4_quantize_append_paged_kv_cache, nvfp4_kv_dequantize_paged,
nvfp4_kv_materialize_fp8): caches [pages, page_size, H, D/2] (NHD) or
[pages, H, page_size, D/2] (HND), scales with D/16 in place of D/2.

Seeds: workload i draws from ``numpy.random.default_rng(1000 + i)``;
sequence lengths first, then page permutations, then data.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

NHD, HND = 0, 1
SENTINEL_16 = 0xA5A5      # prefill of dequant outputs
SENTINEL_FP8 = 0x5A       # prefill of the FP8 page copy


# ---------------------------------------------------------------------------
# 16-bit float inputs
# ---------------------------------------------------------------------------
def f32_to_bits(x: np.ndarray, is_bf16: bool) -> np.ndarray:
    """fp32 -> bf16/fp16 bit patterns through torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16 if is_bf16 else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(bits: np.ndarray, is_bf16: bool) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16 if is_bf16 else torch.float16).float().numpy()


# ---------------------------------------------------------------------------
# paged caches on the host
# ---------------------------------------------------------------------------
@dataclass
class HostCache:
    """Four 2-D uint8 arrays [num_pages, bytes] (possibly strided views of a
    stacked or padded buffer) and the geometry. ``bases`` holds the owning
    buffers and ``offsets`` each view's byte offset into its base."""
    k_data: np.ndarray
    v_data: np.ndarray
    k_sf: np.ndarray
    v_sf: np.ndarray
    page_size: int
    num_heads: int
    head_dim: int
    layout: int
    bases: list = field(default_factory=list)
    views: list = field(default_factory=list)   # (base_index, byte_offset, page_stride, bytes)

    @property
    def num_pages(self) -> int:
        return self.k_data.shape[0]

    def copy(self) -> "HostCache":
        bases = [b.copy() for b in self.bases]
        arrs = [np.lib.stride_tricks.as_strided(bases[bi][off:], shape=(self.num_pages, nb), strides=(st, 1))
                for (bi, off, st, nb) in self.views]
        return HostCache(*arrs, self.page_size, self.num_heads, self.head_dim, self.layout, bases,
                         list(self.views))

    def data_4d(self, kv: int) -> np.ndarray:
        """Logical [pages, ps, H, D/2] (NHD) or [pages, H, ps, D/2] (HND) view."""
        a = self.v_data if kv else self.k_data
        n = self.page_size * self.num_heads * (self.head_dim // 2)
        inner = (self.page_size, self.num_heads) if self.layout == NHD else (self.num_heads, self.page_size)
        return a[:, :n].reshape((a.shape[0],) + inner + (self.head_dim // 2,))

    def sf_4d(self, kv: int) -> np.ndarray:
        a = self.v_sf if kv else self.k_sf
        n = self.page_size * self.num_heads * (self.head_dim // 16)
        inner = (self.page_size, self.num_heads) if self.layout == NHD else (self.num_heads, self.page_size)
        return a[:, :n].reshape((a.shape[0],) + inner + (self.head_dim // 16,))


def make_cache(rng: np.random.Generator, num_pages: int, page_size: int, num_heads: int,
               head_dim: int, layout: int, stacked: bool = False, data_pad: int = 0,
               sf_pad: int = 0, fill: str = "random") -> HostCache:
    """A paged NVFP4 cache. ``stacked`` puts K and V of a page side by side in
    one buffer (the 5-D format, K/V on dimension 1); ``data_pad``/``sf_pad``
    add bytes to every page stride. ``fill``: 'random' bytes or 'zero'."""
    dbytes = page_size * num_heads * head_dim // 2
    sbytes = page_size * num_heads * head_dim // 16
    dstride, sstride = dbytes + data_pad, sbytes + sf_pad

    def alloc(n):
        if fill == "random":
            return np.frombuffer(bytearray(rng.bytes(n)), dtype=np.uint8)
        return np.zeros(n, np.uint8)

    def view(base, off, stride, nb):
        return np.lib.stride_tricks.as_strided(base[off:], shape=(num_pages, nb), strides=(stride, 1))

    if stacked:
        db = alloc(num_pages * 2 * dstride)
        sb = alloc(num_pages * 2 * sstride)
        bases = [db, sb]
        views = [(0, 0, 2 * dstride, dbytes), (0, dstride, 2 * dstride, dbytes),
                 (1, 0, 2 * sstride, sbytes), (1, sstride, 2 * sstride, sbytes)]
    else:
        bases = [alloc(num_pages * dstride), alloc(num_pages * dstride),
                 alloc(num_pages * sstride), alloc(num_pages * sstride)]
        views = [(0, 0, dstride, dbytes), (1, 0, dstride, dbytes),
                 (2, 0, sstride, sbytes), (3, 0, sstride, sbytes)]
    arrs = [view(bases[bi], off, st, nb) for (bi, off, st, nb) in views]
    return HostCache(*arrs, page_size, num_heads, head_dim, layout, bases, views)


# ---------------------------------------------------------------------------
# page tables
# ---------------------------------------------------------------------------
def csr_for_lengths(lengths: np.ndarray, page_size: int, pool_perm: np.ndarray):
    """CSR append table for requests of the given total lengths: request b
    takes the next ceil(len/ps) pages of ``pool_perm`` in request order."""
    n_pages = (lengths + page_size - 1) // page_size
    indptr = np.zeros(len(lengths) + 1, np.int32)
    indptr[1:] = np.cumsum(n_pages)
    indices = pool_perm[: indptr[-1]].astype(np.int32)
    last = (lengths - (n_pages - 1) * page_size).astype(np.int32)
    return indices, indptr, last


def block_table_from_csr(indices, indptr, cols: int, dtype=np.int32, pad: int = 0):
    B = len(indptr) - 1
    bt = np.full((B, cols), pad, dtype=dtype)
    for b in range(B):
        n = indptr[b + 1] - indptr[b]
        bt[b, :n] = indices[indptr[b]:indptr[b + 1]]
    return bt


def rows_for_positions(starts: np.ndarray, ends: np.ndarray):
    """batch_indices/positions for rows [starts[b], ends[b]) of each request."""
    bi = np.concatenate([np.full(e - s, b, np.int32) for b, (s, e) in enumerate(zip(starts, ends))])
    pos = np.concatenate([np.arange(s, e, dtype=np.int32) for s, e in zip(starts, ends)])
    return bi, pos


# ---------------------------------------------------------------------------
# value distributions
# ---------------------------------------------------------------------------
def _bulk_normal(rng, shape) -> np.ndarray:
    """Standard normal fp32 draws in bulk: torch's (multithreaded) CPU
    generator, seeded by the next draw of ``rng``."""
    import torch
    g = torch.Generator().manual_seed(int(rng.integers(0, 2**62)))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).numpy()


def normal_rows(rng, shape) -> np.ndarray:
    return _bulk_normal(rng, shape)


def head_scales(rng, H: int, lo=0.1, hi=10.0) -> np.ndarray:
    """One scale per head, log-uniform in [lo, hi]."""
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=H)).astype(np.float32)


def head_scaled_normal(rng, nnz: int, a: np.ndarray, D: int) -> np.ndarray:
    """N(0,1) rows [nnz, H, D] times the per-head scales ``a``."""
    return _bulk_normal(rng, (nnz, len(a), D)) * a[None, :, None]


def sample_without_replacement(rng, n: int, k: int) -> np.ndarray:
    """k distinct indices in [0, n), uniformly (draw with replacement, keep
    the first occurrence of each value in draw order, top up until k)."""
    out = np.empty(0, np.int64)
    while out.size < k:
        draw = rng.integers(0, n, size=int((k - out.size) * 1.05) + 16)
        cat = np.concatenate([out, draw])
        _, first = np.unique(cat, return_index=True)
        out = cat[np.sort(first)]
    return out[:k]


def student_t_with_outliers(rng, shape, nu=3, frac=0.001, factor=20.0) -> np.ndarray:
    """Student-t with ``nu`` (integer) degrees of freedom, z / sqrt(chi2/nu)
    with chi2 a sum of nu squared normals; then exactly round(frac * n)
    entries, chosen without replacement, multiplied by ``factor``."""
    z = _bulk_normal(rng, shape)
    chi2 = np.zeros(shape, np.float32)
    for _ in range(int(nu)):
        w = _bulk_normal(rng, shape)
        chi2 += w * w
    x = (z / np.sqrt(chi2 / np.float32(nu))).astype(np.float32)
    n = x.size
    k = int(round(frac * n))
    idx = sample_without_replacement(rng, n, k)
    flat = x.reshape(-1)
    flat[idx] *= np.float32(factor)
    return x


def scale_bytes(rng, shape, lo=0x00, hi=0x7E) -> np.ndarray:
    """Random finite non-negative E4M3 byte values in [lo, hi]."""
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8)


# ---------------------------------------------------------------------------
# the five serving workloads (full size) and their small variants
# ---------------------------------------------------------------------------
@dataclass
class AppendDequant:
    """Append rows into a cache, then gather-dequantize the whole context."""
    cache: HostCache
    key: np.ndarray            # uint16 bits [nnz, H, D]
    value: np.ndarray
    in_bf16: bool
    batch_indices: np.ndarray
    positions: np.ndarray
    kv_indices: np.ndarray
    kv_indptr: np.ndarray
    kv_last_page_len: np.ndarray
    block_tables: np.ndarray   # [B, cols] int32/int64
    seq_lens: np.ndarray       # int32 [B]: context length after the append
    max_seq_len: int
    out_bf16: bool
    history_key: np.ndarray | None = None     # uint16 [n_hist, H, D], rows before the append
    history_value: np.ndarray | None = None
    history_batch_indices: np.ndarray | None = None
    history_positions: np.ndarray | None = None
    name: str = ""


def tiny_round_trip(seed: int = 1001) -> AppendDequant:
    """B=2, seq_lens {5, 19}, ps 16, H 2, D 64, NHD, bf16 N(0,1); 8 physical
    pages in random order; all tokens appended, then dequantized to bf16."""
    rng = np.random.default_rng(seed)
    ps, H, D = 16, 2, 64
    lens = np.array([5, 19], np.int64)
    perm = rng.permutation(8)
    cache = make_cache(rng, 8, ps, H, D, NHD)
    nnz = int(lens.sum())
    key = f32_to_bits(normal_rows(rng, (nnz, H, D)), True)
    value = f32_to_bits(normal_rows(rng, (nnz, H, D)), True)
    indices = np.array([perm[0], perm[1], perm[2]], np.int32)
    indptr = np.array([0, 1, 3], np.int32)
    last = np.array([5, 3], np.int32)
    bi, pos = rows_for_positions(np.zeros(2, np.int64), lens)
    bt = np.array([[perm[0], 0], [perm[1], perm[2]]], np.int32)
    return AppendDequant(cache, key, value, True, bi, pos, indices, indptr, last, bt,
                         lens.astype(np.int32), int(lens.max()), True, name="tiny_round_trip")


def decode_append_tables(rng, B: int = 64, max_old: int = 4096, pool: int = 20000, ps: int = 16):
    """Lengths and page tables of the decode workload (first draws of its
    seed): old lengths U{1..max_old}, one new token each, pages of a shuffled
    pool taken in request order."""
    old = rng.integers(1, max_old + 1, size=B).astype(np.int64)
    new_len = old + 1
    perm = rng.permutation(pool)
    indices, indptr, last = csr_for_lengths(new_len, ps, perm)
    cols = int(((new_len.max() + ps - 1) // ps))
    bt = block_table_from_csr(indices, indptr, cols, np.int32)
    return old, new_len, indices, indptr, last, bt


def materialize_tables(rng, B: int = 32, lo: int = 128, hi: int = 32768, ps: int = 16, shared: bool = False,
                       compact: bool = True):
    """Lengths, page tables and kv_page_indptr of the materialize workload
    (first draws of its seed): lengths log-uniform in [lo, hi], K and V pages
    from independent permutations of the pool."""
    lens = np.clip(np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi), size=B))), lo, hi).astype(np.int64)
    need = (lens + ps - 1) // ps
    P = int(need.sum())
    maxp = int(need.max())
    permk = rng.permutation(P)
    permv = rng.permutation(P)
    if compact:
        indptr = np.zeros(B + 1, np.int32)
        indptr[1:] = np.cumsum(need)
    else:
        indptr = (np.arange(B + 1) * maxp).astype(np.int32)
    off = np.concatenate([[0], np.cumsum(need)])
    bt = np.zeros((B, maxp), np.int32) if shared else np.zeros((B, 2, maxp), np.int32)
    for b in range(B):
        n = need[b]
        if shared:
            bt[b, :n] = permk[off[b]:off[b] + n]
        else:
            bt[b, 0, :n] = permk[off[b]:off[b] + n]
            bt[b, 1, :n] = permv[off[b]:off[b] + n]
    return lens, P, maxp, bt, indptr


def decode_append(seed: int = 1002, B: int = 64, max_old: int = 4096, pool: int = 20000,
                  ps: int = 16, H: int = 8, D: int = 128) -> AppendDequant:
    """B requests with old lengths U{1..max_old}, one new token each at
    position old_len, NHD pages shuffled across a pool; bf16 K/V are N(0,1)
    times a per-head log-uniform [0.1, 10] scale (independent for K and V).
    ``history_*`` hold the rows already in the cache (quantized untimed)."""
    rng = np.random.default_rng(seed)
    old, new_len, indices, indptr, last, bt = decode_append_tables(rng, B, max_old, pool, ps)
    cache = make_cache(rng, pool, ps, H, D, NHD)
    a_k, a_v = head_scales(rng, H), head_scales(rng, H)
    n_hist = int(old.sum())
    hk = f32_to_bits(head_scaled_normal(rng, n_hist, a_k, D), True)
    hv = f32_to_bits(head_scaled_normal(rng, n_hist, a_v, D), True)
    hbi, hpos = rows_for_positions(np.zeros(B, np.int64), old)
    key = f32_to_bits(head_scaled_normal(rng, B, a_k, D), True)
    value = f32_to_bits(head_scaled_normal(rng, B, a_v, D), True)
    bi = np.arange(B, dtype=np.int32)
    pos = old.astype(np.int32)
    return AppendDequant(cache, key, value, True, bi, pos, indices, indptr, last, bt,
                         new_len.astype(np.int32), int(new_len.max()), True,
                         hk, hv, hbi, hpos, name="decode_append")


def four_over_six_quantize(seed: int = 1005, B: int = 16, T: int = 4096, ps: int = 64,
                           H: int = 8, D: int = 128) -> AppendDequant:
    """nnz = B*T bf16 rows from Student-t (nu=3) with 0.1% of entries x20,
    appended into ps-token NHD pages of a permuted pool, then dequantized."""
    rng = np.random.default_rng(seed)
    lens = np.full(B, T, np.int64)
    n_pages = B * T // ps
    perm = rng.permutation(n_pages)
    indices, indptr, last = csr_for_lengths(lens, ps, perm)
    bt = block_table_from_csr(indices, indptr, T // ps, np.int32)
    cache = make_cache(rng, n_pages, ps, H, D, NHD)
    nnz = B * T
    key = f32_to_bits(student_t_with_outliers(rng, (nnz, H, D)), True)
    value = f32_to_bits(student_t_with_outliers(rng, (nnz, H, D)), True)
    bi, pos = rows_for_positions(np.zeros(B, np.int64), lens)
    return AppendDequant(cache, key, value, True, bi, pos, indices, indptr, last, bt,
                         lens.astype(np.int32), T, True, name="four_over_six_quantize")


@dataclass
class PrefillDequant:
    cache: HostCache           # zero-filled; filled by quantizing ``key``/``value`` rows
    key: np.ndarray            # uint16 bf16 bits [B*T, H, D] in (request, position) order
    value: np.ndarray
    batch_indices: np.ndarray
    positions: np.ndarray
    kv_indices: np.ndarray
    kv_indptr: np.ndarray
    kv_last_page_len: np.ndarray
    block_tables: np.ndarray   # int64 [B, T/ps]
    seq_lens: np.ndarray
    max_seq_len: int
    out_bf16: bool = False     # fp16 outputs
    name: str = "prefill_dequantize"


def prefill_dequantize(seed: int = 1003, B: int = 16, T: int = 8192, ps: int = 32,
                       H: int = 8, D: int = 128) -> PrefillDequant:
    """B requests of T tokens, HND pages of ps tokens; the cache holds the
    quantization of seeded bf16 N(0,1) K/V; block table = a random page
    permutation (int64); fp16 outputs."""
    rng = np.random.default_rng(seed)
    n_pages = B * T // ps
    perm = rng.permutation(n_pages)
    bt = perm.reshape(B, T // ps).astype(np.int64)
    lens = np.full(B, T, np.int64)
    indptr = (np.arange(B + 1) * (T // ps)).astype(np.int32)
    indices = perm.astype(np.int32)
    last = np.full(B, ps, np.int32)
    cache = make_cache(rng, n_pages, ps, H, D, HND)
    key = f32_to_bits(normal_rows(rng, (B * T, H, D)), True)
    value = f32_to_bits(normal_rows(rng, (B * T, H, D)), True)
    bi, pos = rows_for_positions(np.zeros(B, np.int64), lens)
    return PrefillDequant(cache, key, value, bi, pos, indices, indptr, last, bt,
                          lens.astype(np.int32), T)


@dataclass
class Materialize:
    cache: HostCache           # HND, padded data page stride, random codes/scales
    block_tables: np.ndarray   # int32 [B, max_pages] (shared) or [B, 2, max_pages]
    shared: bool
    seq_lens: np.ndarray
    kv_page_indptr: np.ndarray
    num_pages_out: int         # kv_page_indptr[-1]
    max_pages_per_seq: int
    max_kv_len: int
    name: str = "materialize_fp8"


def materialize_fp8(seed: int = 1004, B: int = 32, lo: int = 128, hi: int = 32768, ps: int = 16,
                    H: int = 8, D: int = 128, data_pad: int = 256, shared: bool = False,
                    compact: bool = True) -> Materialize:
    """seq_lens log-uniform in [lo, hi]; HND cache whose data page stride is
    padded by ``data_pad`` bytes; random code bytes and scale bytes in
    0x00..0x7E; K and V pages drawn from independent permutations of the
    pool (separate tables) unless ``shared``; compact kv_page_indptr."""
    rng = np.random.default_rng(seed)
    lens, P, maxp, bt, indptr = materialize_tables(rng, B, lo, hi, ps, shared, compact)
    cache = make_cache(rng, P, ps, H, D, HND, data_pad=data_pad, fill="zero")
    for a in (cache.k_data, cache.v_data):
        a[...] = np.frombuffer(rng.bytes(a.size), dtype=np.uint8).reshape(a.shape)
    for a in (cache.k_sf, cache.v_sf):
        a[...] = scale_bytes(rng, a.shape)
    return Materialize(cache, bt, shared, lens.astype(np.int32), indptr, int(indptr[-1]), maxp,
                       int(lens.max()))
