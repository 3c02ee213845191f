"""Paged NVFP4 KV-cache path for AMD MI355X (gfx950).

The compute lives in ``lib/libkvfp4.so`` (HIP kernels behind the C ABI of
``include/kvfp4.h``); this package is its Python binding:

* ``kv_quantize_append``, ``kv_dequantize_paged``, ``kv_append_dequantize_paged``, ``kv_materialize_fp8``,
  ``kv_global_scale``, ``kv_quantize``, ``kv_dequantize``,
  ``kv_quantize_paged_cache`` - one function per C entry point (marshalling
  only);
* the page-shaped API in :mod:`.api` (tuple/stacked caches, layouts given as
  strings, the functional materializer and ``NVFP4KVMaterializer``).
"""
from ._binding import (KVFP4Error, PagedCache, Recipe, kv_dequantize, kv_dequantize_paged,  # noqa: F401
                       kv_global_scale, kv_materialize_fp8, kv_quantize, kv_quantize_append,
                       kv_quantize_paged_cache, kv_decode_attention,
                       kv_decode_attention_workspace_size, kv_decode_attention_noalloc, load_library,
                       status_string, PreparedCall, prepare_quantize_append, prepare_dequantize_paged,
                       prepare_materialize_fp8, kv_append_dequantize_paged, prepare_append_dequantize_paged,
                       TableError, check_append_tables, check_step_rows, check_paged_tables,
                       check_materialize_tables)
from ._binding import (KVFP4_BF16, KVFP4_ERR_MAE, KVFP4_ERR_MSE, KVFP4_F16, KVFP4_HND,  # noqa: F401
                       KVFP4_I32, KVFP4_I64, KVFP4_NHD)
from .api import (NVFP44Over6Config, NVFP4KVMaterializer, make_nvfp4_global_scale,  # noqa: F401
                  nvfp4_append_dequantize_paged, nvfp4_e4m3_max, nvfp4_kv_dequantize, nvfp4_kv_dequantize_paged,
                  nvfp4_kv_materialize_fp8,
                  nvfp4_kv_quantize, nvfp4_quantize_append_paged_kv_cache, nvfp4_quantize_paged_kv_cache,
                  paged_cache)

load_library()
