"""Python face of the CPU oracle (ctypes over ``libkvfp4_oracle.so``).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this module. The GPU package never
does, and the oracle never imports the GPU package.

Arrays are numpy. 16-bit floats travel as their uint16 bit patterns. A paged
cache is four 2-D uint8 arrays ``[num_pages, bytes_per_page]`` (views with a
larger page stride are fine: the stride is read from the array), plus the
geometry. Every function follows the passage cited in ``kvfp4_oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("KVFP4_ORACLE_LIB") or os.path.join(_HERE, "libkvfp4_oracle.so")
_lib = None

NHD, HND = 0, 1
MSE, MAE = 0, 1


class _Cache(C.Structure):
    _fields_ = [
        ("k_data", C.c_void_p), ("v_data", C.c_void_p),
        ("k_sf", C.c_void_p), ("v_sf", C.c_void_p),
        ("k_page_stride", C.c_int64), ("v_page_stride", C.c_int64),
        ("k_sf_page_stride", C.c_int64), ("v_sf_page_stride", C.c_int64),
        ("num_pages", C.c_int32), ("page_size", C.c_int32),
        ("num_heads", C.c_int32), ("head_dim", C.c_int32), ("layout", C.c_int32),
    ]


class _Recipe(C.Structure):
    _fields_ = [("four_over_six", C.c_int), ("e4m3_max", C.c_float), ("err_mode", C.c_int), ("err_fp16", C.c_int)]


@dataclass(frozen=True)
class Recipe:
    """Block-scale recipe: standard amax/6 (``four_over_six=False``) or the
    two-candidate 4over6 search with its own E4M3 clamp and error metric."""
    four_over_six: bool = False
    e4m3_max: float = 448.0
    err_mode: int = MSE
    err_fp16: bool = False

    def _c(self):
        return _Recipe(int(self.four_over_six), float(self.e4m3_max), int(self.err_mode), int(self.err_fp16))


STANDARD = Recipe()


def four_over_six(err_mode: int = MSE, e4m3_max: float = 256.0, fast_math: bool = False) -> Recipe:
    return Recipe(True, e4m3_max, err_mode, fast_math)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = C.CDLL(_LIB_PATH)
    P = C.c_void_p
    i64, i32, f32 = C.c_int64, C.c_int32, C.c_float
    lib.orc_e2m1_value.restype = C.c_double
    lib.orc_e2m1_value.argtypes = [C.c_int]
    lib.orc_e2m1_encode.restype = C.c_int
    lib.orc_e2m1_encode.argtypes = [f32]
    lib.orc_e4m3_value.restype = C.c_double
    lib.orc_e4m3_value.argtypes = [C.c_int]
    lib.orc_e4m3_encode_scale.restype = C.c_int
    lib.orc_e4m3_encode_scale.argtypes = [f32, f32]
    lib.orc_e4m3_encode_satfinite.restype = C.c_int
    lib.orc_e4m3_encode_satfinite.argtypes = [f32]
    lib.orc_half_value.restype = C.c_double
    lib.orc_half_value.argtypes = [C.c_uint16, C.c_int]
    lib.orc_round_half.restype = C.c_uint16
    lib.orc_round_half.argtypes = [f32, C.c_int]
    lib.orc_e2m1_encode_array.argtypes = [P, i64, P]
    lib.orc_e4m3_encode_scale_array.argtypes = [P, i64, f32, P]
    lib.orc_e4m3_encode_satfinite_array.argtypes = [P, i64, P]
    lib.orc_round_half_array.argtypes = [P, i64, C.c_int, P]
    lib.orc_quantize_block.restype = C.c_int
    lib.orc_quantize_block.argtypes = [P, f32, C.POINTER(_Recipe), P, P, P, P, P]
    lib.orc_global_scale.restype = f32
    lib.orc_global_scale.argtypes = [P, i64, C.c_int, f32]
    lib.orc_quantize_append.restype = C.c_int
    lib.orc_quantize_append.argtypes = [C.POINTER(_Cache), P, P, C.c_int, i64, P, P, P, P, P, i32,
                                        f32, f32, C.POINTER(_Recipe), C.c_int]
    lib.orc_dequantize_paged.restype = C.c_int
    lib.orc_dequantize_paged.argtypes = [C.POINTER(_Cache), P, C.c_int, i64, i32, P, i32, f32, f32,
                                         P, P, C.c_int, i32, C.c_int]
    lib.orc_materialize_fp8.restype = C.c_int
    lib.orc_materialize_fp8.argtypes = [C.POINTER(_Cache), C.c_int, P, C.c_int, i64, i64, i32, P, P,
                                        i32, P, i64, P, i32, C.c_int]
    lib.orc_quantize_contiguous.restype = C.c_int
    lib.orc_quantize_contiguous.argtypes = [P, C.c_int, i64, i64, f32, C.POINTER(_Recipe), P, P, C.c_int]
    lib.orc_dequantize_contiguous.restype = C.c_int
    lib.orc_dequantize_contiguous.argtypes = [P, P, i64, i64, f32, P, C.c_int, C.c_int]
    lib.orc_quantize_paged_cache.restype = C.c_int
    lib.orc_quantize_paged_cache.argtypes = [C.POINTER(_Cache), P, P, C.c_int, f32, f32, C.POINTER(_Recipe),
                                             C.c_int, C.c_int]
    lib.orc_decode_attention.restype = C.c_int
    lib.orc_decode_attention.argtypes = [C.POINTER(_Cache), P, C.c_int, i32, P, i64, i32, P, i32, f32, f32, f32, P,
                                         C.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return C.c_void_p(a.ctypes.data)


def _need(a: np.ndarray, dtype, name: str, contiguous: bool = True) -> np.ndarray:
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"{name}: expected {np.dtype(dtype)}, got {a.dtype}")
    if contiguous and not a.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous")
    return a


# ---------------------------------------------------------------------------
# scalar codecs, vectorised over numpy arrays
# ---------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().orc_e4m3_value(int(byte))


def half_value(bits: int, is_bf16: bool) -> float:
    return _load().orc_half_value(int(bits) & 0xFFFF, int(bool(is_bf16)))


def e2m1_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e2m1_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_encode_scale(sf, e4m3_max: float = 448.0) -> np.ndarray:
    sf = np.ascontiguousarray(sf, dtype=np.float32)
    out = np.empty(sf.shape, np.uint8)
    _load().orc_e4m3_encode_scale_array(_ptr(sf), sf.size, float(e4m3_max), _ptr(out))
    return out


def e4m3_encode_satfinite(p) -> np.ndarray:
    p = np.ascontiguousarray(p, dtype=np.float32)
    out = np.empty(p.shape, np.uint8)
    _load().orc_e4m3_encode_satfinite_array(_ptr(p), p.size, _ptr(out))
    return out


def round_half(x, is_bf16: bool) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().orc_round_half_array(_ptr(x), x.size, int(bool(is_bf16)), _ptr(out))
    return out


def quantize_block(x16, g: float, recipe: Recipe = STANDARD):
    """One 16-element block -> (codes[16] uint8, scale byte, err6, err4, chose4)."""
    x = np.ascontiguousarray(x16, dtype=np.float32)
    if x.size != 16:
        raise ValueError("a block has 16 elements")
    codes = np.zeros(16, np.uint8)
    s = np.zeros(1, np.uint8)
    e6 = C.c_float(0)
    e4 = C.c_float(0)
    ch = C.c_int(0)
    rc = _load().orc_quantize_block(_ptr(x), float(g), C.byref(recipe._c()), _ptr(codes), _ptr(s),
                                    C.byref(e6), C.byref(e4), C.byref(ch))
    if rc != 0:
        raise ValueError(f"orc_quantize_block rejected its arguments ({rc})")
    return codes, int(s[0]), e6.value, e4.value, bool(ch.value)


def global_scale(x_bits: np.ndarray, is_bf16: bool, e4m3_max: float = 448.0) -> float:
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    return float(_load().orc_global_scale(_ptr(x), x.size, int(bool(is_bf16)), float(e4m3_max)))


# ---------------------------------------------------------------------------
# the three paged operations
# ---------------------------------------------------------------------------
def _cache_struct(k_data, v_data, k_sf, v_sf, page_size, num_heads, head_dim, layout):
    arrs = (k_data, v_data, k_sf, v_sf)
    for a, n in zip(arrs, ("k_data", "v_data", "k_sf", "v_sf")):
        _need(a, np.uint8, n, contiguous=False)
        if a.ndim != 2 or a.strides[1] != 1:
            raise ValueError(f"{n} must be [num_pages, bytes_per_page] with unit inner stride")
    num_pages = k_data.shape[0]
    return _Cache(k_data.ctypes.data, v_data.ctypes.data, k_sf.ctypes.data, v_sf.ctypes.data,
                  k_data.strides[0], v_data.strides[0], k_sf.strides[0], v_sf.strides[0],
                  num_pages, page_size, num_heads, head_dim, layout)


def quantize_append(cache, key_bits, value_bits, in_is_bf16, batch_indices, positions,
                    kv_indices, kv_indptr, kv_last_page_len, k_scale, v_scale,
                    recipe: Recipe = STANDARD, threads: int = 1):
    """[AP] in place on ``cache`` (anything with k_data, v_data, k_sf, v_sf,
    page_size, num_heads, head_dim, layout attributes)."""
    cs = _cache_struct(cache.k_data, cache.v_data, cache.k_sf, cache.v_sf, cache.page_size,
                       cache.num_heads, cache.head_dim, cache.layout)
    key = _need(np.asarray(key_bits), np.uint16, "key")
    val = _need(np.asarray(value_bits), np.uint16, "value")
    bi = _need(np.asarray(batch_indices), np.int32, "batch_indices")
    pos = _need(np.asarray(positions), np.int32, "positions")
    ind = _need(np.asarray(kv_indices), np.int32, "kv_indices")
    ptr = _need(np.asarray(kv_indptr), np.int32, "kv_indptr")
    last = _need(np.asarray(kv_last_page_len), np.int32, "kv_last_page_len")
    nnz = bi.shape[0]
    if key.size != nnz * cache.num_heads * cache.head_dim or val.size != key.size:
        raise ValueError("key/value must be [nnz, H, D]")
    rc = _load().orc_quantize_append(C.byref(cs), _ptr(key), _ptr(val), int(bool(in_is_bf16)), nnz,
                                     _ptr(bi), _ptr(pos), _ptr(ind), _ptr(ptr), _ptr(last),
                                     ptr.shape[0] - 1, float(k_scale), float(v_scale),
                                     C.byref(recipe._c()), int(threads))
    if rc != 0:
        raise ValueError(f"oracle quantize_append rejected its arguments ({rc})")


def dequantize_paged(cache, block_tables, seq_lens, k_scale, v_scale, out_k, out_v,
                     out_is_bf16, threads: int = 1):
    """[DQ] into uint16 arrays ``out_k``/``out_v`` of shape [B, T, H, D], in place."""
    cs = _cache_struct(cache.k_data, cache.v_data, cache.k_sf, cache.v_sf, cache.page_size,
                       cache.num_heads, cache.head_dim, cache.layout)
    bt = np.asarray(block_tables)
    if bt.dtype not in (np.int32, np.int64) or bt.ndim != 2 or not bt.flags.c_contiguous:
        raise ValueError("block_tables: contiguous int32/int64 [B, max_pages]")
    sl = _need(np.asarray(seq_lens), np.int32, "seq_lens")
    _need(out_k, np.uint16, "out_k")
    _need(out_v, np.uint16, "out_v")
    B, T = out_k.shape[0], out_k.shape[1]
    if out_k.shape != out_v.shape or out_k.shape[2:] != (cache.num_heads, cache.head_dim):
        raise ValueError("outputs must be [B, max_seq_len, H, D]")
    if bt.shape[0] != B or sl.shape[0] != B:
        raise ValueError("batch mismatch")
    rc = _load().orc_dequantize_paged(C.byref(cs), _ptr(bt), int(bt.dtype == np.int64), bt.shape[1],
                                      bt.shape[1], _ptr(sl), B, float(k_scale), float(v_scale),
                                      _ptr(out_k), _ptr(out_v), int(bool(out_is_bf16)), T, int(threads))
    if rc != 0:
        raise ValueError(f"oracle dequantize_paged rejected its arguments ({rc})")


def materialize_fp8(cache, block_tables, seq_lens, kv_page_indptr, out, fp8_block_tables,
                    shared: bool = True, v_sf_interleaved: bool = True, threads: int = 1):
    """[MF] into ``out`` (uint8 [P, 2, H, ps, D]) and ``fp8_block_tables``
    (int32 [B, max_pages_per_seq]), in place; only live entries are written."""
    cs = _cache_struct(cache.k_data, cache.v_data, cache.k_sf, cache.v_sf, cache.page_size,
                       cache.num_heads, cache.head_dim, cache.layout)
    bt = _need(np.asarray(block_tables), np.int32, "block_tables")
    sl = _need(np.asarray(seq_lens), np.int32, "seq_lens")
    ip = _need(np.asarray(kv_page_indptr), np.int32, "kv_page_indptr")
    _need(out, np.uint8, "out")
    _need(fp8_block_tables, np.int32, "fp8_block_tables")
    B = sl.shape[0]
    if shared:
        if bt.ndim != 2:
            raise ValueError("shared block_tables are [B, max_pages]")
        cols, row, kvs = bt.shape[1], bt.shape[1], 0
    else:
        if bt.ndim != 3 or bt.shape[1] != 2:
            raise ValueError("separate block_tables are [B, 2, max_pages]")
        cols, row, kvs = bt.shape[2], 2 * bt.shape[2], bt.shape[2]
    rc = _load().orc_materialize_fp8(C.byref(cs), int(bool(v_sf_interleaved)), _ptr(bt), int(bool(shared)),
                                     row, kvs, cols, _ptr(sl), _ptr(ip), B, _ptr(out), out.shape[0],
                                     _ptr(fp8_block_tables), fp8_block_tables.shape[1], int(threads))
    if rc != 0:
        raise ValueError(f"oracle materialize_fp8 rejected its arguments ({rc})")


def quantize_contiguous(x_bits, in_is_bf16, g, recipe: Recipe = STANDARD, threads: int = 1):
    """[KV] R10: uint16 bit patterns [..., cols] (cols % 16 == 0) -> (codes
    uint8 [..., cols/2], scales uint8 [..., cols/16])."""
    x = _need(np.asarray(x_bits), np.uint16, "x")
    cols = x.shape[-1] if x.ndim else 0
    rows = x.size // cols if cols else 0
    codes = np.zeros(x.shape[:-1] + (cols // 2,), np.uint8)
    scales = np.zeros(x.shape[:-1] + (cols // 16,), np.uint8)
    rc = _load().orc_quantize_contiguous(_ptr(x), int(bool(in_is_bf16)), rows, cols, float(g),
                                         C.byref(recipe._c()), _ptr(codes), _ptr(scales), int(threads))
    if rc != 0:
        raise ValueError(f"oracle quantize_contiguous rejected its arguments ({rc})")
    return codes, scales


def dequantize_contiguous(codes, scales, g, out_is_bf16, threads: int = 1):
    """[KV] R10: codes [..., cols/2], scales [..., cols/16] -> uint16 [..., cols]."""
    cd = _need(np.asarray(codes), np.uint8, "codes")
    sc = _need(np.asarray(scales), np.uint8, "scales")
    cols = cd.shape[-1] * 2
    if sc.shape[:-1] != cd.shape[:-1] or sc.shape[-1] * 16 != cols:
        raise ValueError("codes / scales shapes disagree")
    rows = cd.size * 2 // cols if cols else 0
    out = np.zeros(cd.shape[:-1] + (cols,), np.uint16)
    rc = _load().orc_dequantize_contiguous(_ptr(cd), _ptr(sc), rows, cols, float(g), _ptr(out),
                                           int(bool(out_is_bf16)), int(threads))
    if rc != 0:
        raise ValueError(f"oracle dequantize_contiguous rejected its arguments ({rc})")
    return out


def quantize_paged_cache(cache, k_in_bits, v_in_bits, in_is_bf16, k_scale, v_scale,
                         recipe: Recipe = STANDARD, v_sf_interleaved: bool = True, threads: int = 1):
    """[KV] R11 in place on ``cache``: pools [num_pages, ps, H, D] (NHD) or
    [num_pages, H, ps, D] (HND) as uint16 bit patterns."""
    cs = _cache_struct(cache.k_data, cache.v_data, cache.k_sf, cache.v_sf, cache.page_size,
                       cache.num_heads, cache.head_dim, cache.layout)
    k = _need(np.asarray(k_in_bits), np.uint16, "k_in")
    v = _need(np.asarray(v_in_bits), np.uint16, "v_in")
    n = cs.num_pages * cache.page_size * cache.num_heads * cache.head_dim
    if k.size != n or v.size != n:
        raise ValueError("pools must hold num_pages pages of the cache's geometry")
    rc = _load().orc_quantize_paged_cache(C.byref(cs), _ptr(k), _ptr(v), int(bool(in_is_bf16)), float(k_scale),
                                          float(v_scale), C.byref(recipe._c()), int(bool(v_sf_interleaved)),
                                          int(threads))
    if rc != 0:
        raise ValueError(f"oracle quantize_paged_cache rejected its arguments ({rc})")


def decode_attention(cache, q_bits, q_is_bf16, block_tables, seq_lens, k_scale, v_scale, sm_scale,
                     threads: int = 1) -> np.ndarray:
    """R13: q [B, Hq, D] fp16/bf16 bits -> float64 [B, Hq, D]."""
    cs = _cache_struct(cache.k_data, cache.v_data, cache.k_sf, cache.v_sf, cache.page_size,
                       cache.num_heads, cache.head_dim, cache.layout)
    q = _need(np.asarray(q_bits), np.uint16, "q")
    bt = _need(np.asarray(block_tables), np.int32, "block_tables")
    sl = _need(np.asarray(seq_lens), np.int32, "seq_lens")
    B, Hq, D = q.shape
    if D != cache.head_dim or bt.shape[0] != B or sl.shape[0] != B:
        raise ValueError("shapes disagree")
    out = np.zeros((B, Hq, D), np.float64)
    rc = _load().orc_decode_attention(C.byref(cs), _ptr(q), int(bool(q_is_bf16)), Hq, _ptr(bt), bt.shape[1],
                                      bt.shape[1], _ptr(sl), B, float(k_scale), float(v_scale), float(sm_scale),
                                      _ptr(out), int(threads))
    if rc != 0:
        raise ValueError(f"oracle decode_attention rejected its arguments ({rc})")
    return out
