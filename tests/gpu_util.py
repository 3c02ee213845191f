"""Helpers for the GPU parity tests: host caches <-> device tensors with the
same byte layout, and the oracle's thread count."""
import os

import numpy as np
import torch

import workloads as W


def oracle_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


class DeviceCache:
    """Device copy of a ``workloads.HostCache`` with identical strides."""

    def __init__(self, host: W.HostCache, device="cuda"):
        import kv_cache_quantization_paged_amd as K
        self.host = host
        self.bases = [torch.from_numpy(b.copy()).to(device) for b in host.bases]
        ps, H, D = host.page_size, host.num_heads, host.head_dim
        views = []
        for i, (bi, off, st, nb) in enumerate(host.views):
            last = D // 2 if i < 2 else D // 16
            if host.layout == W.NHD:
                shape, strides = (host.num_pages, ps, H, last), (st, H * last, last, 1)
            else:
                shape, strides = (host.num_pages, H, ps, last), (st, ps * last, last, 1)
            views.append(self.bases[bi].as_strided(shape, strides, off))
        self.k_data, self.v_data, self.k_sf, self.v_sf = views
        self.cache = K.PagedCache(self.k_data, self.v_data, self.k_sf, self.v_sf,
                                  K.KVFP4_NHD if host.layout == W.NHD else K.KVFP4_HND)

    def to_host(self) -> W.HostCache:
        """Copy the device bytes back into a new HostCache of the same layout."""
        out = self.host.copy()
        for b_host, b_dev in zip(out.bases, self.bases):
            b_host[...] = b_dev.cpu().numpy()
        return out


def bits_tensor(bits: np.ndarray, is_bf16: bool, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if is_bf16 else torch.float16).to(device)


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def same_bytes(a: W.HostCache, b: W.HostCache) -> bool:
    return all(np.array_equal(x, y) for x, y in zip(a.bases, b.bases))


def first_mismatch(a: np.ndarray, b: np.ndarray):
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return None
    i = tuple(idx[0])
    return i, a[i], b[i], int(idx.shape[0])
