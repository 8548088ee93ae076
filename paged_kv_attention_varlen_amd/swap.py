"""Swapping the cache pages of requests to pinned host memory and back.

The Transformers "continuous batching architecture" page (section "Offloading") moves the KV blocks of offloaded
requests into a pre-allocated pinned CPU buffer, batched into one transfer, and copies them back when GPU cache
space is free again, so that the requests resume without recomputing their prompts. Here a swap is two steps on
one stream: cb_kv_copy_pages gathers the pages into a contiguous device staging buffer (an HBM-bound copy kernel),
and one asynchronous copy moves the staging buffer to the pinned host buffer (PCIe-bound). Swapping in runs the
two steps the other way, scattering into whatever free pages the caller gives. The library allocates nothing: the
pinned host buffer and the staging buffer are allocated once here, through torch.
"""
from __future__ import annotations

from . import copy_pages


class HostSwap:
    """A pinned host swap pool of `capacity` pages for a (k_cache, v_cache) pair, with a device staging buffer."""

    def __init__(self, k_cache, v_cache, capacity: int):
        import torch
        if k_cache.shape[0] != v_cache.shape[0] or k_cache[0].numel() != v_cache[0].numel():
            raise ValueError("K and V caches must hold the same pages")
        self.capacity = int(capacity)
        dev = k_cache.device
        self.stage_k = torch.empty((capacity,) + tuple(k_cache.shape[1:]), dtype=k_cache.dtype, device=dev)
        self.stage_v = torch.empty((capacity,) + tuple(v_cache.shape[1:]), dtype=v_cache.dtype, device=dev)
        self.host_k = torch.empty(self.stage_k.shape, dtype=k_cache.dtype, pin_memory=True)
        self.host_v = torch.empty(self.stage_v.shape, dtype=v_cache.dtype, pin_memory=True)

    def swap_out(self, k_cache, v_cache, pages, stream=None) -> int:
        """Copy cache pages `pages` (int32 device tensor, n <= capacity) to host slots 0..n-1. Asynchronous on
        `stream` (default: current); the host copy is complete once that stream reaches this point."""
        import torch
        n = pages.numel()
        if n > self.capacity:
            raise ValueError("more pages than the swap pool holds")
        s = stream or torch.cuda.current_stream()
        copy_pages(self.stage_k[:n], k_cache, None, pages, stream=s)
        copy_pages(self.stage_v[:n], v_cache, None, pages, stream=s)
        with torch.cuda.stream(s):
            self.host_k[:n].copy_(self.stage_k[:n], non_blocking=True)
            self.host_v[:n].copy_(self.stage_v[:n], non_blocking=True)
        return n

    def swap_in(self, k_cache, v_cache, pages, stream=None) -> None:
        """Copy host slots 0..n-1 back into cache pages `pages` (int32 device tensor). Asynchronous on `stream`."""
        import torch
        n = pages.numel()
        if n > self.capacity:
            raise ValueError("more pages than the swap pool holds")
        s = stream or torch.cuda.current_stream()
        with torch.cuda.stream(s):
            self.stage_k[:n].copy_(self.host_k[:n], non_blocking=True)
            self.stage_v[:n].copy_(self.host_v[:n], non_blocking=True)
        copy_pages(k_cache, self.stage_k[:n], pages, None, stream=s)
        copy_pages(v_cache, self.stage_v[:n], pages, None, stream=s)
