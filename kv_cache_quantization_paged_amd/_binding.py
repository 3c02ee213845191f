"""ctypes binding of ``libkvfp4.so`` (declared in ``include/kvfp4.h``).

Argument marshalling only: the functions here take torch tensors that live on
the GPU, check dtypes, shapes and devices, turn them into pointers and byte
strides, and call the C entry point of the same name on torch's current
stream. All computation happens in the HIP kernels. If the library has not
been built, importing this module raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # loads the HIP runtime that the library then shares

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libkvfp4.so")

KVFP4_OK, KVFP4_EINVAL, KVFP4_EALIGN, KVFP4_EUNSUPPORTED, KVFP4_ELAUNCH, KVFP4_ESCRATCH, KVFP4_EVALUE = range(7)
NOALLOC_SCRATCH_BYTES = 32 << 20      # KVFP4_NOALLOC_SCRATCH_BYTES
KVFP4_NHD, KVFP4_HND = 0, 1
KVFP4_F16, KVFP4_BF16 = 0, 1
KVFP4_I32, KVFP4_I64 = 0, 1
KVFP4_ERR_MSE, KVFP4_ERR_MAE = 0, 1

EXPORTED = ("kv_quantize_append", "kv_dequantize_paged", "kv_append_dequantize_paged", "kv_materialize_fp8",
            "kv_global_scale", "kv_quantize", "kv_dequantize", "kv_quantize_paged_cache", "kv_decode_attention",
            "kv_decode_attention_workspace_size", "kv_decode_attention_noalloc", "kv_quantize_append_prepare",
            "kv_dequantize_paged_prepare", "kv_append_dequantize_paged_prepare", "kv_materialize_fp8_prepare",
            "kvfp4_launch", "kvfp4_check_append_tables", "kvfp4_check_step_rows",
            "kvfp4_check_paged_tables", "kvfp4_check_materialize_tables", "kvfp4_table_problem_string",
            "kvfp4_status_string")


class PagedCacheDesc(C.Structure):
    """``kvfp4_paged_cache_t``"""
    _fields_ = [
        ("k_data", C.c_void_p), ("v_data", C.c_void_p),
        ("k_sf", C.c_void_p), ("v_sf", C.c_void_p),
        ("k_page_stride", C.c_int64), ("v_page_stride", C.c_int64),
        ("k_sf_page_stride", C.c_int64), ("v_sf_page_stride", C.c_int64),
        ("num_pages", C.c_int32), ("page_size", C.c_int32),
        ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("layout", C.c_int32),
    ]


class TableReport(C.Structure):
    """``kvfp4_table_report_t``"""
    _fields_ = [("problem", C.c_int32), ("index", C.c_int64), ("value", C.c_int64)]


class RecipeDesc(C.Structure):
    """``kvfp4_recipe_t``"""
    _fields_ = [("e4m3_max", C.c_float), ("err_mode", C.c_int32), ("err_use_fast_math", C.c_int32)]


class KVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def load_library():
    """Load ``libkvfp4.so``; raises if it is missing (build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run kv_cache_quantization_paged_amd.build.build() "
                          "(or __graft_entry__.build()) first")
    lib = C.CDLL(LIB_PATH)
    P, i32, i64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_float
    lib.kv_quantize_append.restype = i32
    lib.kv_quantize_append.argtypes = [C.POINTER(PagedCacheDesc), P, P, i32, i64, P, P, P, P, P, i32,
                                       f32, f32, C.POINTER(RecipeDesc), P]
    lib.kv_dequantize_paged.restype = i32
    lib.kv_dequantize_paged.argtypes = [C.POINTER(PagedCacheDesc), P, i32, i64, i32, P, i32, P, P,
                                        P, P, i32, i32, P]
    lib.kv_materialize_fp8.restype = i32
    lib.kv_materialize_fp8.argtypes = [C.POINTER(PagedCacheDesc), i32, P, i32, i64, i64, i32, P, P, i32,
                                       P, i64, P, i32, P]
    lib.kv_append_dequantize_paged.restype = i32
    lib.kv_append_dequantize_paged.argtypes = [C.POINTER(PagedCacheDesc), P, P, i32, i64, P, P, P, P, P, f32, f32,
                                               C.POINTER(RecipeDesc), P, i32, i64, i32, P, i32, P, P, P, P, i32,
                                               i32, P]
    lib.kv_global_scale.restype = i32
    lib.kv_global_scale.argtypes = [P, i32, i64, f32, P, P]
    lib.kv_quantize.restype = i32
    lib.kv_quantize.argtypes = [P, i32, i64, i64, P, C.POINTER(RecipeDesc), P, P, P]
    lib.kv_dequantize.restype = i32
    lib.kv_dequantize.argtypes = [P, P, i64, i64, P, P, i32, P]
    lib.kv_quantize_paged_cache.restype = i32
    lib.kv_quantize_paged_cache.argtypes = [C.POINTER(PagedCacheDesc), P, P, i32, P, P, C.POINTER(RecipeDesc),
                                            i32, P]
    lib.kv_decode_attention.restype = i32
    lib.kv_decode_attention.argtypes = [C.POINTER(PagedCacheDesc), P, i32, i32, P, i64, i32, P, i32, P, P, f32, P, P,
                                        i64, P]
    lib.kv_decode_attention_noalloc.restype = i32
    lib.kv_decode_attention_noalloc.argtypes = [C.POINTER(PagedCacheDesc), P, i32, i32, P, i64, i32, P, i32, P, P,
                                                f32, P, P]
    lib.kv_decode_attention_workspace_size.restype = i64
    lib.kv_decode_attention_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.kv_quantize_append_prepare.restype = i32
    lib.kv_quantize_append_prepare.argtypes = [P] + lib.kv_quantize_append.argtypes[:-1]
    lib.kv_dequantize_paged_prepare.restype = i32
    lib.kv_dequantize_paged_prepare.argtypes = [P] + lib.kv_dequantize_paged.argtypes[:-1]
    lib.kv_materialize_fp8_prepare.restype = i32
    lib.kv_materialize_fp8_prepare.argtypes = [P] + lib.kv_materialize_fp8.argtypes[:-1]
    lib.kv_append_dequantize_paged_prepare.restype = i32
    lib.kv_append_dequantize_paged_prepare.argtypes = [P] + lib.kv_append_dequantize_paged.argtypes[:-1]
    lib.kvfp4_launch.restype = i32
    lib.kvfp4_launch.argtypes = [P, P]
    lib.kvfp4_check_append_tables.restype = i32
    lib.kvfp4_check_append_tables.argtypes = [P, P, i64, P, P, P, i32, i32, i32, P, C.POINTER(TableReport)]
    lib.kvfp4_check_step_rows.restype = i32
    lib.kvfp4_check_step_rows.argtypes = [P, P, i64, P, i32, P, C.POINTER(TableReport)]
    lib.kvfp4_check_paged_tables.restype = i32
    lib.kvfp4_check_paged_tables.argtypes = [P, i32, i64, i32, P, i32, i32, i32, i32, C.POINTER(TableReport)]
    lib.kvfp4_check_materialize_tables.restype = i32
    lib.kvfp4_check_materialize_tables.argtypes = [P, i32, i64, i64, i32, P, P, i32, i32, i32, i32, i64,
                                                   C.POINTER(TableReport)]
    lib.kvfp4_table_problem_string.restype = C.c_char_p
    lib.kvfp4_table_problem_string.argtypes = [i32]
    lib.kvfp4_status_string.restype = C.c_char_p
    lib.kvfp4_status_string.argtypes = [i32]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().kvfp4_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != KVFP4_OK:
        raise KVFP4Error(status, where)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stride(t, dim):
    """Element stride of dimension `dim`; a dimension of size 1 may carry any
    stride (torch and numpy give 0 to an inserted axis), so it reports the
    stride it would have in a contiguous tensor instead."""
    if t.shape[dim] == 1:
        n = 1
        for d in range(dim + 1, t.dim()):
            n *= t.shape[d]
        return n
    return t.stride(dim)


# torch's current stream as a raw pointer: the private accessor costs ~0.1 us
# where torch.cuda.current_stream() builds a Stream object (~3 us per call)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_stream_ptr(device_index=None) -> int:
    if device_index is None:
        device_index = torch.cuda.current_device()
    if _raw_stream is not None:
        return _raw_stream(device_index)
    return torch.cuda.current_stream(device_index).cuda_stream


def _stream(stream=None):
    if stream is None:
        return C.c_void_p(_current_stream_ptr())
    return C.c_void_p(stream.cuda_stream)


def _half_enum(dtype) -> int:
    if dtype == torch.float16:
        return KVFP4_F16
    if dtype == torch.bfloat16:
        return KVFP4_BF16
    raise TypeError(f"expected float16 or bfloat16, got {dtype}")


def _need_i32(t, name):
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 CUDA tensor")


# ---------------------------------------------------------------------------
# cache descriptors
# ---------------------------------------------------------------------------
class PagedCache:
    """Describes a paged NVFP4 cache held in four uint8 CUDA tensors.

    ``k_data``/``v_data``: [num_pages, page_size, H, D/2] (NHD) or
    [num_pages, H, page_size, D/2] (HND); ``k_sf``/``v_sf`` the same with D/16.
    Any page stride is allowed (tuple, stacked 5-D views, padded pages) as long
    as each page is compact inside.
    """

    def __init__(self, k_data, v_data, k_sf, v_sf, layout: int):
        if layout not in (KVFP4_NHD, KVFP4_HND):
            raise ValueError("layout must be NHD (0) or HND (1)")
        for t, n in ((k_data, "k_data"), (v_data, "v_data"), (k_sf, "k_sf"), (v_sf, "v_sf")):
            if t.dtype != torch.uint8 or not t.is_cuda or t.dim() != 4:
                raise TypeError(f"{n} must be a 4-D uint8 CUDA tensor")
            if any(_stride(t, d) != want for d, want in ((1, t.shape[2] * t.shape[3]), (2, t.shape[3]), (3, 1))):
                raise ValueError(f"{n}: each page must be compact (strides {t.stride()})")
        if k_data.shape != v_data.shape or k_sf.shape != v_sf.shape or k_data.shape[:3] != k_sf.shape[:3]:
            raise ValueError("K/V data and scale shapes disagree")
        self.layout = layout
        if layout == KVFP4_NHD:
            _, self.page_size, self.num_kv_heads, half = k_data.shape
        else:
            _, self.num_kv_heads, self.page_size, half = k_data.shape
        self.head_dim = 2 * half
        if k_sf.shape[3] * 16 != self.head_dim:
            raise ValueError("scale tensors must have head_dim // 16 in the last dimension")
        self.tensors = (k_data, v_data, k_sf, v_sf)
        self.num_pages = min(k_data.shape[0], v_data.shape[0])
        self.desc = PagedCacheDesc(k_data.data_ptr(), v_data.data_ptr(), k_sf.data_ptr(), v_sf.data_ptr(),
                                   _stride(k_data, 0), _stride(v_data, 0), _stride(k_sf, 0), _stride(v_sf, 0),
                                   self.num_pages, self.page_size, self.num_kv_heads, self.head_dim, layout)


class Recipe:
    """4over6 recipe (``kvfp4_recipe_t``); ``None`` everywhere means standard NVFP4."""

    def __init__(self, e4m3_max: float = 256.0, err_mode: int = KVFP4_ERR_MSE, err_use_fast_math: bool = False):
        self.e4m3_max = float(e4m3_max)
        self.err_mode = int(err_mode)
        self.err_use_fast_math = bool(err_use_fast_math)

    def desc(self):
        return RecipeDesc(self.e4m3_max, self.err_mode, int(self.err_use_fast_math))


# ---------------------------------------------------------------------------
# the C entry points, one Python function each
# ---------------------------------------------------------------------------
class PreparedCall:
    """A call checked once (``kv_*_prepare``) and launched many times
    (``kvfp4_launch``): ``launch()`` queues the kernels on the current stream
    of the tensors' device (or on ``stream``) without checking anything
    again. Holds the tensors it was prepared with, so their memory stays
    valid; their contents may change between launches (that is the point:
    new lengths, new tables), their shapes and storage may not."""
    __slots__ = ("_rec", "_addr", "_dev", "_tensors", "_launch", "name")

    def __init__(self, name: str, device_index: int, tensors):
        self._rec = (C.c_uint64 * 40)()
        self._addr = C.addressof(self._rec)
        self._dev = device_index
        self._tensors = tensors
        self._launch = load_library().kvfp4_launch
        self.name = name

    def launch(self, stream=None):
        if stream is None:
            st = _raw_stream(self._dev) if _raw_stream is not None else _current_stream_ptr(self._dev)
        else:
            st = stream.cuda_stream
        status = self._launch(self._addr, st)
        if status:
            raise KVFP4Error(status, self.name)


def _prepared(name, prepare_fn, args, tensors, device_index):
    call = PreparedCall(name, device_index, tensors)
    _check(prepare_fn(call._addr, *args), name)
    return call


def _append_args(cache: PagedCache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                 kv_last_page_len, k_scale, v_scale, recipe):
    if append_key.shape != append_value.shape or append_key.dtype != append_value.dtype:
        raise ValueError("append_key and append_value must match")
    if append_key.dim() != 3 or tuple(append_key.shape[1:]) != (cache.num_kv_heads, cache.head_dim):
        raise ValueError("append rows must be [nnz, num_kv_heads, head_dim]")
    if not (append_key.is_cuda and append_key.is_contiguous() and append_value.is_contiguous()):
        raise ValueError("append rows must be contiguous CUDA tensors")
    for t, n in ((batch_indices, "batch_indices"), (positions, "positions"), (kv_indices, "kv_indices"),
                 (kv_indptr, "kv_indptr"), (kv_last_page_len, "kv_last_page_len")):
        _need_i32(t, n)
    nnz = append_key.shape[0]
    if batch_indices.numel() != nnz or positions.numel() != nnz:
        raise ValueError("batch_indices / positions must have nnz entries")
    batch = kv_indptr.numel() - 1
    if kv_last_page_len.numel() != batch:
        raise ValueError("kv_last_page_len must have batch_size entries")
    rd = recipe.desc() if recipe is not None else None
    return (C.byref(cache.desc), _ptr(append_key), _ptr(append_value), _half_enum(append_key.dtype), nnz,
            _ptr(batch_indices), _ptr(positions), _ptr(kv_indices), _ptr(kv_indptr), _ptr(kv_last_page_len), batch,
            float(k_scale), float(v_scale), C.byref(rd) if rd is not None else None)


def kv_quantize_append(cache: PagedCache, append_key, append_value, batch_indices, positions,
                       kv_indices, kv_indptr, kv_last_page_len, k_scale: float, v_scale: float,
                       recipe: Recipe | None = None, stream=None):
    lib = load_library()
    args = _append_args(cache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                        kv_last_page_len, k_scale, v_scale, recipe)
    _check(lib.kv_quantize_append(*args, _stream(stream)), "kv_quantize_append")


def prepare_quantize_append(cache: PagedCache, append_key, append_value, batch_indices, positions, kv_indices,
                            kv_indptr, kv_last_page_len, k_scale: float, v_scale: float,
                            recipe: Recipe | None = None) -> PreparedCall:
    """kv_quantize_append checked once; ``.launch()`` appends again (e.g. the
    next decode step's rows written into the same tensors)."""
    lib = load_library()
    args = _append_args(cache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                        kv_last_page_len, k_scale, v_scale, recipe)
    return _prepared("kv_quantize_append", lib.kv_quantize_append_prepare, args,
                     (cache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                      kv_last_page_len), append_key.device.index)


def _dequant_args(cache: PagedCache, block_tables, seq_lens, k_scale, v_scale, output_k, output_v):
    if block_tables.dtype not in (torch.int32, torch.int64) or block_tables.dim() != 2 or not block_tables.is_cuda:
        raise TypeError("block_tables must be a 2-D int32/int64 CUDA tensor")
    if _stride(block_tables, 1) != 1:
        raise ValueError("block_tables rows must be contiguous")
    _need_i32(seq_lens, "seq_lens")
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t.dtype != torch.float32 or not t.is_cuda or t.numel() < 1:
            raise TypeError(f"{n} must be a float32 CUDA tensor")
    if output_k.shape != output_v.shape or output_k.dtype != output_v.dtype:
        raise ValueError("output_k and output_v must match")
    if output_k.dim() != 4 or tuple(output_k.shape[2:]) != (cache.num_kv_heads, cache.head_dim):
        raise ValueError("outputs must be [batch, max_seq_len, num_heads, head_dim]")
    if not (output_k.is_cuda and output_k.is_contiguous() and output_v.is_contiguous()):
        raise ValueError("outputs must be contiguous CUDA tensors")
    B, T = output_k.shape[0], output_k.shape[1]
    if block_tables.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("block_tables / seq_lens batch size disagrees with the outputs")
    return (C.byref(cache.desc), _ptr(block_tables), KVFP4_I64 if block_tables.dtype == torch.int64 else KVFP4_I32,
            _stride(block_tables, 0), block_tables.shape[1], _ptr(seq_lens), B, _ptr(k_scale), _ptr(v_scale),
            _ptr(output_k), _ptr(output_v), _half_enum(output_k.dtype), T)


def kv_dequantize_paged(cache: PagedCache, block_tables, seq_lens, k_scale, v_scale, output_k, output_v,
                        stream=None):
    lib = load_library()
    args = _dequant_args(cache, block_tables, seq_lens, k_scale, v_scale, output_k, output_v)
    _check(lib.kv_dequantize_paged(*args, _stream(stream)), "kv_dequantize_paged")


def prepare_dequantize_paged(cache: PagedCache, block_tables, seq_lens, k_scale, v_scale, output_k,
                             output_v) -> PreparedCall:
    """kv_dequantize_paged checked once; ``.launch()`` dequantizes again with
    whatever the table, lengths and cache hold at that time."""
    lib = load_library()
    args = _dequant_args(cache, block_tables, seq_lens, k_scale, v_scale, output_k, output_v)
    return _prepared("kv_dequantize_paged", lib.kv_dequantize_paged_prepare, args,
                     (cache, block_tables, seq_lens, k_scale, v_scale, output_k, output_v), output_k.device.index)


def _append_dequant_args(cache: PagedCache, append_key, append_value, batch_indices, positions, kv_indices,
                         kv_indptr, kv_last_page_len, k_scale, v_scale, block_tables, seq_lens, dequant_k_scale,
                         dequant_v_scale, output_k, output_v, recipe):
    a = _append_args(cache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                     kv_last_page_len, k_scale, v_scale, recipe)
    d = _dequant_args(cache, block_tables, seq_lens, dequant_k_scale, dequant_v_scale, output_k, output_v)
    nnz, batch = a[4], a[10]
    if batch != d[6]:
        raise ValueError("the append tables and the dequant batch disagree")
    if nnz != batch:
        raise ValueError("a decode step appends one row per request (nnz == batch)")
    return a[:10] + a[11:] + d[1:]


def kv_append_dequantize_paged(cache: PagedCache, append_key, append_value, batch_indices, positions, kv_indices,
                               kv_indptr, kv_last_page_len, k_scale: float, v_scale: float, block_tables, seq_lens,
                               dequant_k_scale, dequant_v_scale, output_k, output_v, recipe: Recipe | None = None,
                               stream=None):
    """A decode step: kv_quantize_append of each request's newest token, then
    kv_dequantize_paged of every request (lengths including that token), in
    one launch where the recipe and layout allow it."""
    lib = load_library()
    args = _append_dequant_args(cache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                                kv_last_page_len, k_scale, v_scale, block_tables, seq_lens, dequant_k_scale,
                                dequant_v_scale, output_k, output_v, recipe)
    _check(lib.kv_append_dequantize_paged(*args, _stream(stream)), "kv_append_dequantize_paged")


def prepare_append_dequantize_paged(cache: PagedCache, append_key, append_value, batch_indices, positions,
                                    kv_indices, kv_indptr, kv_last_page_len, k_scale: float, v_scale: float,
                                    block_tables, seq_lens, dequant_k_scale, dequant_v_scale, output_k, output_v,
                                    recipe: Recipe | None = None) -> PreparedCall:
    """kv_append_dequantize_paged checked once; ``.launch()`` runs the step
    again with whatever the tensors hold at that time."""
    lib = load_library()
    args = _append_dequant_args(cache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                                kv_last_page_len, k_scale, v_scale, block_tables, seq_lens, dequant_k_scale,
                                dequant_v_scale, output_k, output_v, recipe)
    return _prepared("kv_append_dequantize_paged", lib.kv_append_dequantize_paged_prepare, args,
                     (cache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                      kv_last_page_len, block_tables, seq_lens, dequant_k_scale, dequant_v_scale, output_k,
                      output_v), output_k.device.index)


def _materialize_args(cache: PagedCache, block_tables, seq_lens, kv_page_indptr, out, fp8_block_tables,
                      uses_shared_paged_kv_idx, v_sf_interleaved):
    _need_i32(seq_lens, "seq_lens")
    _need_i32(kv_page_indptr, "kv_page_indptr")
    _need_i32(fp8_block_tables, "fp8_block_tables")
    if block_tables.dtype != torch.int32 or not block_tables.is_cuda or _stride(block_tables, block_tables.dim() - 1) != 1:
        raise TypeError("block_tables must be an int32 CUDA tensor with contiguous rows")
    B = seq_lens.numel()
    if uses_shared_paged_kv_idx:
        if block_tables.dim() != 2:
            raise ValueError("shared block_tables are [batch, max_num_pages]")
        cols, row, kvs = block_tables.shape[1], _stride(block_tables, 0), 0
    else:
        if block_tables.dim() != 3 or block_tables.shape[1] != 2:
            raise ValueError("separate block_tables are [batch, 2, max_num_pages]")
        cols, row, kvs = block_tables.shape[2], _stride(block_tables, 0), _stride(block_tables, 1)
    if block_tables.shape[0] != B or kv_page_indptr.numel() != B + 1 or fp8_block_tables.shape[0] != B:
        raise ValueError("batch sizes disagree")
    if out.dim() != 5 or out.shape[1:] != (2, cache.num_kv_heads, cache.page_size, cache.head_dim):
        raise ValueError("out must be [num_out_pages, 2, num_kv_heads, page_size, head_dim]")
    if out.element_size() != 1 or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous one-byte (float8_e4m3fn) CUDA tensor")
    return (C.byref(cache.desc), int(bool(v_sf_interleaved)), _ptr(block_tables), int(bool(uses_shared_paged_kv_idx)),
            row, kvs, cols, _ptr(seq_lens), _ptr(kv_page_indptr), B, _ptr(out), out.shape[0],
            _ptr(fp8_block_tables), fp8_block_tables.shape[1])


def kv_materialize_fp8(cache: PagedCache, block_tables, seq_lens, kv_page_indptr, out, fp8_block_tables,
                       uses_shared_paged_kv_idx: bool = True, v_sf_interleaved: bool = True, stream=None):
    lib = load_library()
    args = _materialize_args(cache, block_tables, seq_lens, kv_page_indptr, out, fp8_block_tables,
                             uses_shared_paged_kv_idx, v_sf_interleaved)
    _check(lib.kv_materialize_fp8(*args, _stream(stream)), "kv_materialize_fp8")


def prepare_materialize_fp8(cache: PagedCache, block_tables, seq_lens, kv_page_indptr, out, fp8_block_tables,
                            uses_shared_paged_kv_idx: bool = True, v_sf_interleaved: bool = True) -> PreparedCall:
    """kv_materialize_fp8 checked once; ``.launch()`` materializes again."""
    lib = load_library()
    args = _materialize_args(cache, block_tables, seq_lens, kv_page_indptr, out, fp8_block_tables,
                             uses_shared_paged_kv_idx, v_sf_interleaved)
    return _prepared("kv_materialize_fp8", lib.kv_materialize_fp8_prepare, args,
                     (cache, block_tables, seq_lens, kv_page_indptr, out, fp8_block_tables), out.device.index)


def kv_global_scale(x, e4m3_max: float, g_out, stream=None):
    lib = load_library()
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous CUDA tensor")
    if g_out.dtype != torch.float32 or not g_out.is_cuda:
        raise TypeError("g_out must be a float32 CUDA tensor")
    st = lib.kv_global_scale(_ptr(x), _half_enum(x.dtype), x.numel(), float(e4m3_max), _ptr(g_out),
                             _stream(stream))
    _check(st, "kv_global_scale")


def _need_scale(t, name):
    if t.dtype != torch.float32 or not t.is_cuda or t.numel() < 1:
        raise TypeError(f"{name} must be a float32 CUDA tensor")


def kv_quantize(x, global_scale, fp4_data, block_scales, recipe: Recipe | None = None, stream=None):
    """x [..., cols] fp16/bf16 -> fp4_data uint8 [..., cols/2], block_scales
    uint8 [..., cols/16] (all contiguous CUDA tensors)."""
    lib = load_library()
    _need_scale(global_scale, "global_scale")
    if not (x.is_cuda and x.is_contiguous() and fp4_data.is_contiguous() and block_scales.is_contiguous()):
        raise ValueError("x, fp4_data and block_scales must be contiguous CUDA tensors")
    if x.dim() < 1:
        raise ValueError("x needs a last dimension")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if fp4_data.dtype != torch.uint8 or block_scales.dtype != torch.uint8:
        raise TypeError("fp4_data and block_scales are uint8")
    if fp4_data.numel() != rows * (cols // 2) or block_scales.numel() != rows * (cols // 16):
        raise ValueError("fp4_data must hold [..., cols/2] and block_scales [..., cols/16] bytes")
    rd = recipe.desc() if recipe is not None else None
    st = lib.kv_quantize(_ptr(x), _half_enum(x.dtype), rows, cols, _ptr(global_scale),
                         C.byref(rd) if rd is not None else None, _ptr(fp4_data), _ptr(block_scales),
                         _stream(stream))
    _check(st, "kv_quantize")


def kv_dequantize(fp4_data, block_scales, global_scale, output, stream=None):
    """fp4_data uint8 [..., cols/2], block_scales uint8 [..., cols/16] ->
    output fp16/bf16 [..., cols]."""
    lib = load_library()
    _need_scale(global_scale, "global_scale")
    if not (output.is_cuda and output.is_contiguous() and fp4_data.is_contiguous() and block_scales.is_contiguous()):
        raise ValueError("fp4_data, block_scales and output must be contiguous CUDA tensors")
    cols = output.shape[-1]
    rows = output.numel() // cols if cols else 0
    if fp4_data.dtype != torch.uint8 or block_scales.dtype != torch.uint8:
        raise TypeError("fp4_data and block_scales are uint8")
    if fp4_data.numel() != rows * (cols // 2) or block_scales.numel() != rows * (cols // 16):
        raise ValueError("fp4_data must hold [..., cols/2] and block_scales [..., cols/16] bytes")
    st = lib.kv_dequantize(_ptr(fp4_data), _ptr(block_scales), rows, cols, _ptr(global_scale), _ptr(output),
                           _half_enum(output.dtype), _stream(stream))
    _check(st, "kv_dequantize")


def kv_quantize_paged_cache(cache: PagedCache, k_in, v_in, k_scale, v_scale, recipe: Recipe | None = None,
                            v_sf_interleaved: bool = True, stream=None):
    """Quantize whole 16-bit page pools (contiguous, the cache's layout and
    page count) into ``cache``."""
    lib = load_library()
    _need_scale(k_scale, "k_scale")
    _need_scale(v_scale, "v_scale")
    n = cache.num_pages * cache.page_size * cache.num_kv_heads * cache.head_dim
    for t, name in ((k_in, "k_in"), (v_in, "v_in")):
        if not (t.is_cuda and t.is_contiguous()) or t.numel() != n:
            raise ValueError(f"{name} must be a contiguous CUDA pool of num_pages pages of the cache's geometry")
    if k_in.dtype != v_in.dtype:
        raise ValueError("k_in and v_in must have the same dtype")
    rd = recipe.desc() if recipe is not None else None
    st = lib.kv_quantize_paged_cache(C.byref(cache.desc), _ptr(k_in), _ptr(v_in), _half_enum(k_in.dtype),
                                     _ptr(k_scale), _ptr(v_scale), C.byref(rd) if rd is not None else None,
                                     int(bool(v_sf_interleaved)), _stream(stream))
    _check(st, "kv_quantize_paged_cache")


def kv_decode_attention_workspace_size(batch: int, num_kv_heads: int, num_qo_heads: int, max_pages: int,
                                       page_size: int, head_dim: int = 128) -> int:
    return int(load_library().kv_decode_attention_workspace_size(batch, num_kv_heads, num_qo_heads, max_pages,
                                                                 page_size, head_dim))


def _attention_args(cache: PagedCache, q, block_tables, seq_lens, k_scale, v_scale, out):
    _need_i32(seq_lens, "seq_lens")
    _need_scale(k_scale, "k_scale")
    _need_scale(v_scale, "v_scale")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or not block_tables.is_cuda:
        raise TypeError("block_tables must be a 2-D int32 CUDA tensor")
    if _stride(block_tables, 1) != 1:
        raise ValueError("block_tables rows must be contiguous")
    if q.dim() != 3 or q.shape != out.shape or q.dtype != out.dtype or q.shape[2] != cache.head_dim:
        raise ValueError("q and out must be matching [batch, num_qo_heads, head_dim] tensors")
    if not (q.is_cuda and q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous CUDA tensors")
    B = q.shape[0]
    if block_tables.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("batch sizes disagree")
    return (C.byref(cache.desc), _ptr(q), _half_enum(q.dtype), q.shape[1], _ptr(block_tables), _stride(block_tables, 0),
            block_tables.shape[1], _ptr(seq_lens), B, _ptr(k_scale), _ptr(v_scale))


def kv_decode_attention(cache: PagedCache, q, block_tables, seq_lens, k_scale, v_scale, sm_scale: float, out,
                        workspace, stream=None):
    """q, out [batch, num_qo_heads, head_dim] bf16/fp16; block_tables int32
    [batch, max_pages]; k_scale / v_scale 1-element float32 CUDA tensors;
    workspace a CUDA byte tensor of kv_decode_attention_workspace_size()."""
    lib = load_library()
    args = _attention_args(cache, q, block_tables, seq_lens, k_scale, v_scale, out)
    st = lib.kv_decode_attention(*args, float(sm_scale), _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "kv_decode_attention")


def kv_decode_attention_noalloc(cache: PagedCache, q, block_tables, seq_lens, k_scale, v_scale, sm_scale: float, out,
                                stream=None):
    """kv_decode_attention without a workspace: the partials live in the
    library's fixed per-GPU scratch (NOALLOC_SCRATCH_BYTES). Calls that
    overlap on one GPU race; calls in order on one stream do not."""
    lib = load_library()
    args = _attention_args(cache, q, block_tables, seq_lens, k_scale, v_scale, out)
    st = lib.kv_decode_attention_noalloc(*args, float(sm_scale), _ptr(out), _stream(stream))
    _check(st, "kv_decode_attention_noalloc")


# ---------------------------------------------------------------------------
# host-side table checks (debugging aid: the device calls never check values)
# ---------------------------------------------------------------------------
class TableError(ValueError):
    """A table value a call would use out of range: ``problem`` (a
    KVFP4_TABLE_* code), ``index`` and ``value`` locate it."""

    def __init__(self, where: str, report: TableReport):
        self.problem, self.index, self.value = report.problem, report.index, report.value
        text = load_library().kvfp4_table_problem_string(report.problem).decode()
        super().__init__(f"{where}: {text} (element {report.index}, value {report.value})")


def _host_ints(a, dtype=None):
    """a host numpy copy of a tensor or array (int32 unless dtype says)"""
    import numpy as np
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    a = np.asarray(a)
    if dtype is not None:
        a = a.astype(dtype, copy=False)
    return np.ascontiguousarray(a)


def _np_ptr(a):
    return C.c_void_p(a.ctypes.data) if a.size else None


def _table_result(st, rep, where):
    if st == KVFP4_EVALUE:
        raise TableError(where, rep)
    _check(st, where)


def check_append_tables(batch_indices, positions, kv_indices, kv_indptr, kv_last_page_len, page_size: int,
                        num_pages: int, check_duplicates: bool = True):
    """Raise TableError unless every table value kv_quantize_append would use
    is in range (host copies; works on CPU or GPU tensors and arrays)."""
    import numpy as np
    bi, pos = _host_ints(batch_indices, np.int32), _host_ints(positions, np.int32)
    ind, ptr, last = _host_ints(kv_indices, np.int32), _host_ints(kv_indptr, np.int32), _host_ints(kv_last_page_len, np.int32)
    if bi.shape != pos.shape or ptr.size < 1 or last.size != ptr.size - 1 or ind.size < (ptr[-1] if ptr.size else 0):
        raise ValueError("table sizes disagree")
    scratch = np.empty(bi.size, np.int64) if check_duplicates else None
    rep = TableReport()
    st = load_library().kvfp4_check_append_tables(_np_ptr(bi), _np_ptr(pos), bi.size, _np_ptr(ind), _np_ptr(ptr),
                                                  _np_ptr(last), ptr.size - 1, page_size, num_pages,
                                                  None if scratch is None else _np_ptr(scratch), C.byref(rep))
    _table_result(st, rep, "append tables")


def check_step_rows(batch_indices, positions, seq_lens, check_duplicates: bool = True):
    """Raise TableError unless the rows follow kv_append_dequantize_paged's
    decode-step pattern: one row per request, at position seq_lens[b] - 1."""
    import numpy as np
    bi, pos, sl = _host_ints(batch_indices, np.int32), _host_ints(positions, np.int32), _host_ints(seq_lens, np.int32)
    if bi.shape != pos.shape or bi.size != sl.size:
        raise ValueError("a decode step has one row per request")
    scratch = np.empty(sl.size, np.int64) if check_duplicates else None
    rep = TableReport()
    st = load_library().kvfp4_check_step_rows(_np_ptr(bi), _np_ptr(pos), bi.size, _np_ptr(sl), sl.size,
                                              None if scratch is None else _np_ptr(scratch), C.byref(rep))
    _table_result(st, rep, "decode-step rows")


def check_paged_tables(block_tables, seq_lens, page_size: int, num_pages: int, max_seq_len: int = 2 ** 31 - 1):
    """Raise TableError unless every table value kv_dequantize_paged (with
    this max_seq_len) or kv_decode_attention (the default) would use is in
    range."""
    import numpy as np
    bt = _host_ints(block_tables)
    if bt.dtype not in (np.int32, np.int64) or bt.ndim != 2:
        raise ValueError("block_tables must be 2-D int32 or int64")
    sl = _host_ints(seq_lens, np.int32)
    if sl.size != bt.shape[0]:
        raise ValueError("table sizes disagree")
    rep = TableReport()
    st = load_library().kvfp4_check_paged_tables(_np_ptr(bt), KVFP4_I64 if bt.dtype == np.int64 else KVFP4_I32,
                                                 bt.shape[1], bt.shape[1], _np_ptr(sl), sl.size, page_size, num_pages,
                                                 max_seq_len, C.byref(rep))
    _table_result(st, rep, "paged tables")


def check_materialize_tables(block_tables, seq_lens, kv_page_indptr, page_size: int, num_pages: int,
                             max_pages_per_seq: int, num_out_pages: int, uses_shared_paged_kv_idx: bool = True):
    """Raise TableError unless every table value kv_materialize_fp8 would
    use is in range."""
    import numpy as np
    bt = _host_ints(block_tables, np.int32)
    sl, ip = _host_ints(seq_lens, np.int32), _host_ints(kv_page_indptr, np.int32)
    if uses_shared_paged_kv_idx:
        if bt.ndim != 2:
            raise ValueError("shared block_tables are [batch, max_num_pages]")
        cols, row, kvs = bt.shape[1], bt.shape[1], 0
    else:
        if bt.ndim != 3 or bt.shape[1] != 2:
            raise ValueError("separate block_tables are [batch, 2, max_num_pages]")
        cols, row, kvs = bt.shape[2], 2 * bt.shape[2], bt.shape[2]
    if bt.shape[0] != sl.size or ip.size != sl.size + 1:
        raise ValueError("table sizes disagree")
    rep = TableReport()
    st = load_library().kvfp4_check_materialize_tables(_np_ptr(bt), int(bool(uses_shared_paged_kv_idx)), row, kvs,
                                                       cols, _np_ptr(sl), _np_ptr(ip), sl.size, page_size, num_pages,
                                                       max_pages_per_seq, num_out_pages, C.byref(rep))
    _table_result(st, rep, "materialize tables")
