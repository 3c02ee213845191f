"""Torch-facing API with the signatures of the FlashInfer KV-cache pages.

* ``nvfp4_quantize_append_paged_kv_cache``  (flashinfer.page API page)
* ``nvfp4_kv_dequantize_paged``             (flashinfer.quantization API page)
* ``nvfp4_kv_materialize_fp8`` and ``NVFP4KVMaterializer`` (the
  nvfp4_kv_materialize API page and the materializer class on the
  flashinfer.quantization module page)
* ``NVFP44Over6Config``, ``make_nvfp4_global_scale``, ``nvfp4_e4m3_max``
  (module page, "NVFP4 4over6 Recipes")
* ``nvfp4_kv_quantize``, ``nvfp4_kv_dequantize``,
  ``nvfp4_quantize_paged_kv_cache`` (module page, "FP4 KV Cache Quantization")

Caches are given as on the pages: a (K, V) tuple of uint8 tensors or one
stacked 5-D tensor with K/V on dimension 1, in "NHD" or "HND" layout. This
module only reshapes arguments into the C ABI's descriptors; the work runs in
the library's kernels on torch's current stream.
"""
from __future__ import annotations

import weakref
from dataclasses import dataclass
from typing import Optional, Tuple, Union

import torch

from . import _binding as B

CacheArg = Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]]


# ---------------------------------------------------------------------------
# recipe
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class NVFP44Over6Config:
    """4over6 block-scale recipe: e4m3_max (256 by default), err_mode "MSE"
    or "MAE". ``err_use_fast_math=True`` evaluates the candidates' error in
    fp16 (a distinct recipe: fp16 scoring can reverse a close decision)."""
    e4m3_max: float = 256.0
    err_mode: str = "MSE"
    err_use_fast_math: bool = False

    def _recipe(self) -> B.Recipe:
        mode = {"MSE": B.KVFP4_ERR_MSE, "MAE": B.KVFP4_ERR_MAE}.get(str(self.err_mode).upper())
        if mode is None:
            raise ValueError(f"err_mode must be 'MSE' or 'MAE', got {self.err_mode!r}")
        return B.Recipe(self.e4m3_max, mode, self.err_use_fast_math)


def nvfp4_e4m3_max(nvfp4_4over6_config: Optional[NVFP44Over6Config] = None) -> float:
    """The clamp a recipe puts on its E4M3 block scales (448 for standard NVFP4)."""
    return 448.0 if nvfp4_4over6_config is None else float(nvfp4_4over6_config.e4m3_max)


def make_nvfp4_global_scale(x: torch.Tensor, per_token_activation: bool = False,
                            nvfp4_4over6_config: Optional[NVFP44Over6Config] = None,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-tensor global decode scale amax|x| / (6 * e4m3_max) as a 1-element
    float32 CUDA tensor. Use the same recipe as the quantize call."""
    if per_token_activation:
        raise NotImplementedError("per-token global scales are not part of the KV-cache path")
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    B.kv_global_scale(x.contiguous(), nvfp4_e4m3_max(nvfp4_4over6_config), out)
    return out


# ---------------------------------------------------------------------------
# cache arguments
# ---------------------------------------------------------------------------
def _layout(kv_layout: str) -> int:
    if kv_layout == "NHD":
        return B.KVFP4_NHD
    if kv_layout == "HND":
        return B.KVFP4_HND
    raise ValueError(f"kv_layout must be 'NHD' or 'HND', got {kv_layout!r}")


def _split(cache: CacheArg, name: str):
    if isinstance(cache, (tuple, list)):
        if len(cache) != 2:
            raise ValueError(f"{name}: a tuple cache has two tensors (K, V)")
        return cache[0], cache[1]
    if cache.dim() != 5 or cache.shape[1] != 2:
        raise ValueError(f"{name}: a stacked cache is 5-D with K/V on dimension 1")
    return cache[:, 0], cache[:, 1]


def paged_cache(paged_kv_cache: CacheArg, kv_cache_sf: CacheArg, kv_layout: str = "NHD") -> B.PagedCache:
    k, v = _split(paged_kv_cache, "paged_kv_cache")
    ks, vs = _split(kv_cache_sf, "kv_cache_sf")
    return B.PagedCache(k, v, ks, vs, _layout(kv_layout))


# ---------------------------------------------------------------------------
# the three calls
# ---------------------------------------------------------------------------
def nvfp4_quantize_append_paged_kv_cache(append_key, append_value, batch_indices, positions,
                                         paged_kv_cache: CacheArg, kv_cache_sf: CacheArg, kv_indices,
                                         kv_indptr, kv_last_page_len, k_scale: float, v_scale: float,
                                         kv_layout: str = "NHD",
                                         nvfp4_4over6: Optional[NVFP44Over6Config] = None) -> None:
    """Quantize and append K/V rows in place (standard NVFP4, or the given
    4over6 recipe)."""
    cache = paged_cache(paged_kv_cache, kv_cache_sf, kv_layout)
    recipe = nvfp4_4over6._recipe() if nvfp4_4over6 is not None else None
    B.kv_quantize_append(cache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                         kv_last_page_len, k_scale, v_scale, recipe)


def nvfp4_kv_dequantize_paged(paged_kv_cache: CacheArg, kv_cache_sf: CacheArg, block_tables, seq_lens,
                              k_scale: torch.Tensor, v_scale: torch.Tensor, output_k, output_v,
                              kv_layout: str = "NHD") -> None:
    """Dequantize into caller-owned [batch, max_seq_len, H, D] outputs;
    positions >= seq_lens[b] are left unchanged."""
    cache = paged_cache(paged_kv_cache, kv_cache_sf, kv_layout)
    B.kv_dequantize_paged(cache, block_tables, seq_lens, k_scale, v_scale, output_k, output_v)


def nvfp4_append_dequantize_paged(append_key, append_value, batch_indices, positions, paged_kv_cache: CacheArg,
                                  kv_cache_sf: CacheArg, kv_indices, kv_indptr, kv_last_page_len, k_scale: float,
                                  v_scale: float, block_tables, seq_lens, dequant_k_scale: torch.Tensor,
                                  dequant_v_scale: torch.Tensor, output_k, output_v, kv_layout: str = "NHD",
                                  nvfp4_4over6: Optional[NVFP44Over6Config] = None) -> None:
    """One decode step: nvfp4_quantize_append_paged_kv_cache of each
    request's newest token (one row per request, at position seq_lens[b] - 1),
    then nvfp4_kv_dequantize_paged of every request, as one call."""
    cache = paged_cache(paged_kv_cache, kv_cache_sf, kv_layout)
    recipe = nvfp4_4over6._recipe() if nvfp4_4over6 is not None else None
    B.kv_append_dequantize_paged(cache, append_key, append_value, batch_indices, positions, kv_indices, kv_indptr,
                                 kv_last_page_len, k_scale, v_scale, block_tables, seq_lens, dequant_k_scale,
                                 dequant_v_scale, output_k, output_v, recipe)


def _hnd_cache(k_cache, v_cache, k_block_scales, v_block_scales) -> B.PagedCache:
    return B.PagedCache(k_cache, v_cache, k_block_scales, v_block_scales, B.KVFP4_HND)


def nvfp4_kv_materialize_fp8(k_cache, v_cache, k_block_scales, v_block_scales, block_tables, seq_lens,
                             max_kv_len: int, uses_shared_paged_kv_idx: bool = True,
                             out: Optional[torch.Tensor] = None, kv_page_indptr: Optional[torch.Tensor] = None,
                             num_pages: Optional[int] = None, v_sf_interleaved: bool = True):
    """Functional form: validates, allocates what is not given, returns
    (kv_cache_fp8, fp8_block_tables) with padded table entries 0."""
    cache = _hnd_cache(k_cache, v_cache, k_block_scales, v_block_scales)
    batch = seq_lens.numel()
    ps = cache.page_size
    m = (int(max_kv_len) + ps - 1) // ps
    dev = k_cache.device
    if kv_page_indptr is None:
        kv_page_indptr = torch.arange(0, (batch + 1) * m, m, dtype=torch.int32, device=dev)
        num_pages = batch * m
    elif num_pages is None:
        raise ValueError("kv_page_indptr requires num_pages (its last element, known on the host)")
    if out is None:
        out = torch.empty((num_pages + 1, 2, cache.num_kv_heads, ps, cache.head_dim),
                          dtype=torch.float8_e4m3fn, device=dev)
    table = torch.zeros((batch, m), dtype=torch.int32, device=dev)
    B.kv_materialize_fp8(cache, block_tables, seq_lens, kv_page_indptr, out, table,
                         uses_shared_paged_kv_idx, v_sf_interleaved)
    return out, table


class NVFP4KVMaterializer:
    """Validate once, launch many times. The geometry is checked at
    construction; ``run()`` checks a set of tensors the first time it sees
    it (the C launcher's checks, through ``kv_materialize_fp8_prepare``) and
    afterwards only launches the prepared call (``kvfp4_launch``). ``run()``
    allocates nothing, does not synchronize, and launches on the current
    stream of the materializer's device.

    Prepared calls are kept per tensor set (by object identity, through weak
    references: a tensor freed by the caller drops its entries, and a new
    tensor is checked again). Changing a known tensor's storage in place
    (``set_``, ``resize_``) is not noticed; new contents (lengths, tables,
    cache bytes) are the normal case and need nothing."""

    _MAX_PREPARED = 128

    def __init__(self, num_kv_heads: int, page_size: int, head_dim: int, device="cuda",
                 uses_shared_paged_kv_idx: bool = True, v_sf_interleaved: bool = True):
        if page_size % 4 != 0:
            raise ValueError("page_size must be divisible by 4")
        if head_dim % 64 != 0:
            raise ValueError("head_dim must be divisible by 64")
        self.num_kv_heads, self.page_size, self.head_dim = num_kv_heads, page_size, head_dim
        self.device = torch.device(device)
        if self.device.type != "cuda":
            raise ValueError("the materializer runs on a CUDA (HIP) device")
        self.shared = bool(uses_shared_paged_kv_idx)
        self.v_sf_interleaved = bool(v_sf_interleaved)
        self._prepared = {}
        B.load_library()

    def prepare(self, k_cache, v_cache, k_block_scales, v_block_scales, block_tables, seq_lens, kv_page_indptr,
                *, out: torch.Tensor, fp8_block_tables: torch.Tensor) -> B.PreparedCall:
        """Check one tensor set and return its prepared call (run() does this
        on first sight)."""
        cache = _hnd_cache(k_cache, v_cache, k_block_scales, v_block_scales)
        if (cache.num_kv_heads, cache.page_size, cache.head_dim) != (self.num_kv_heads, self.page_size,
                                                                     self.head_dim):
            raise ValueError("cache geometry differs from the materializer's")
        for t in (k_cache, v_cache, k_block_scales, v_block_scales, block_tables, seq_lens, kv_page_indptr, out,
                  fp8_block_tables):
            if t.device != self.device and not (self.device.index is None and t.device.type == "cuda"):
                raise ValueError(f"tensors must be on the materializer's device {self.device}")
        return B.prepare_materialize_fp8(cache, block_tables, seq_lens, kv_page_indptr, out, fp8_block_tables,
                                         self.shared, self.v_sf_interleaved)

    def run(self, k_cache, v_cache, k_block_scales, v_block_scales, block_tables, seq_lens, kv_page_indptr,
            *, out: torch.Tensor, fp8_block_tables: torch.Tensor):
        ts = (k_cache, v_cache, k_block_scales, v_block_scales, block_tables, seq_lens, kv_page_indptr, out,
              fp8_block_tables)
        hit = self._prepared.get(tuple(map(id, ts)))
        if hit is not None:
            refs, call = hit
            for r, t in zip(refs, ts):
                if r() is not t:
                    break
            else:
                call.launch()
                return out, fp8_block_tables
        key = tuple(map(id, ts))
        call = self.prepare(*ts[:7], out=out, fp8_block_tables=fp8_block_tables)
        # the prepared call keeps the descriptor only; the weak references let
        # freed tensors go (their entries then never match again)
        call._tensors = None
        if len(self._prepared) >= self._MAX_PREPARED:
            self._prepared.clear()
        self._prepared[key] = (tuple(weakref.ref(t) for t in ts), call)
        call.launch()
        return out, fp8_block_tables


# ---------------------------------------------------------------------------
# contiguous codec and whole-pool quantizer ("FP4 KV Cache Quantization")
# ---------------------------------------------------------------------------
def nvfp4_kv_quantize(input: torch.Tensor, global_scale: torch.Tensor,
                      nvfp4_4over6: Optional[NVFP44Over6Config] = None):
    """NVFP4 with the linear block-scale layout: returns (fp4_data uint8
    [..., D/2], block_scales uint8 [..., D/16]). ``global_scale`` is the
    1-element float32 decode scale (``make_nvfp4_global_scale`` with the same
    recipe)."""
    x = input.contiguous()
    D = x.shape[-1]
    data = torch.empty(x.shape[:-1] + (D // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (D // 16,), dtype=torch.uint8, device=x.device)
    recipe = nvfp4_4over6._recipe() if nvfp4_4over6 is not None else None
    B.kv_quantize(x, global_scale, data, scales, recipe)
    return data, scales


def nvfp4_kv_dequantize(fp4_data: torch.Tensor, block_scales: torch.Tensor, global_scale: torch.Tensor,
                        output_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None):
    """Inverse of ``nvfp4_kv_quantize``: [..., D] in ``output_dtype``."""
    if out is None:
        out = torch.empty(fp4_data.shape[:-1] + (2 * fp4_data.shape[-1],), dtype=output_dtype,
                          device=fp4_data.device)
    B.kv_dequantize(fp4_data.contiguous(), block_scales.contiguous(), global_scale, out)
    return out


def nvfp4_quantize_paged_kv_cache(k_cache: torch.Tensor, v_cache: torch.Tensor, kv_layout: str = "HND",
                                  k_global_scale: Optional[torch.Tensor] = None,
                                  v_global_scale: Optional[torch.Tensor] = None,
                                  v_sf_interleaved: bool = True,
                                  nvfp4_4over6: Optional[NVFP44Over6Config] = None):
    """Quantize 16-bit page pools [num_pages, H, ps, D] (HND) or
    [num_pages, ps, H, D] (NHD) to NVFP4. Returns (k_data, v_data, k_sf,
    v_sf, k_global_scale, v_global_scale); V scales are 4-token interleaved
    (the layout the FP8 materializer reads) unless ``v_sf_interleaved`` is
    False. Missing global scales are built from the pools with the recipe."""
    layout = _layout(kv_layout)
    k, v = k_cache.contiguous(), v_cache.contiguous()
    if k.dim() != 4 or k.shape != v.shape:
        raise ValueError("k_cache and v_cache must be matching 4-D page pools")
    if k_global_scale is None:
        k_global_scale = make_nvfp4_global_scale(k, nvfp4_4over6_config=nvfp4_4over6)
    if v_global_scale is None:
        v_global_scale = make_nvfp4_global_scale(v, nvfp4_4over6_config=nvfp4_4over6)
    P, D = k.shape[0], k.shape[3]
    kd = torch.empty(k.shape[:3] + (D // 2,), dtype=torch.uint8, device=k.device)
    vd = torch.empty_like(kd)
    ks = torch.empty(k.shape[:3] + (D // 16,), dtype=torch.uint8, device=k.device)
    vs = torch.empty_like(ks)
    cache = B.PagedCache(kd, vd, ks, vs, layout)
    recipe = nvfp4_4over6._recipe() if nvfp4_4over6 is not None else None
    B.kv_quantize_paged_cache(cache, k, v, k_global_scale, v_global_scale, recipe, v_sf_interleaved)
    return kd, vd, ks, vs, k_global_scale, v_global_scale
