"""Convenience wrapper: register a pool, keep assembled buffers, run a batch.

Allocation and call sequencing only (torch tensors for device memory, the
current torch stream for ordering).  All computation happens in libpic.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .binding import (DEFER_GATHER, DRY_RUN, PLAN_ONLY, VALUES_IN_POOL, VARIANT_MATERIALIZED,
                      Cache, Plan, Pool, Store, model_struct)


class Session:
    def __init__(self, layers, q_heads, kv_heads, head_dim, theta, dtype, pool_tensor,
                 page_tokens, chunk_len, chunk_page_ptr, page_ids, chunk_orig=None, keys="rotated",
                 hot_pages: int = 0, store_paths=None, store_threads: int = 8):
        import torch
        self.torch = torch
        self.layers, self.q_heads, self.kv_heads, self.head_dim = layers, q_heads, kv_heads, head_dim
        self.dtype = dtype
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.model = model_struct(layers, q_heads, kv_heads, head_dim, theta, dtype, keys)
        self.pool_tensor = pool_tensor
        # a pool in pinned host memory is the staging tier: the planes stay on the GPU
        self.host_pool = not pool_tensor.is_cuda
        self.device = torch.device("cuda") if self.host_pool else pool_tensor.device
        self.pool = Pool(self.model, pool_tensor, pool_tensor.numel() * pool_tensor.element_size(),
                         page_tokens, pool_tensor.shape[0], chunk_len, chunk_page_ptr, page_ids,
                         chunk_orig, host=self.host_pool)
        # an HBM hot set of `hot_pages` page slots in front of a host pool
        self.cache = Cache(self.pool, hot_pages) if self.host_pool and hot_pages > 0 else None
        # chunk files behind a host pool: pic_assemble reads the pages each
        # batch covers into the pool's memory
        self.store = None
        if store_paths is not None:
            if not self.host_pool:
                raise ValueError("chunk files fill a pool in pinned host memory")
            self.store = Store(self.pool, pool_tensor, pool_tensor.numel() * pool_tensor.element_size(),
                               store_paths, store_threads)
        self.plan = Plan(self.pool)
        self.asm_k = None
        self.asm_v = None
        self.capacity = 0

    def ensure_capacity(self, rows: int):
        """(Re)allocate the assembled planes [L][Hkv][rows][d] when too small."""
        if self.asm_k is not None and self.capacity >= rows:
            return
        t = self.torch
        shape = (self.layers, self.kv_heads, max(rows, 1), self.head_dim)
        self.asm_k = t.empty(shape, dtype=self.tdtype, device=self.device)
        self.asm_v = t.empty(shape, dtype=self.tdtype, device=self.device)
        self.capacity = max(rows, 1)

    def assemble(self, span_ptr, spans, new_ptr, new_pos=None, plan_only: bool = False, defer: bool = False,
                 values_in_pool: bool = False):
        d = self.plan_host(span_ptr, spans, new_ptr, new_pos)
        self.ensure_capacity(d["rows"])
        flags = (PLAN_ONLY if plan_only else 0) | (DEFER_GATHER if defer else 0) | (VALUES_IN_POOL if values_in_pool else 0)
        self.plan.assemble(span_ptr, spans, new_ptr, new_pos, self.asm_k, self.asm_v, self.capacity,
                           flags, self.torch.cuda.current_stream())
        return self.plan.summary()

    def plan_host(self, span_ptr, spans, new_ptr, new_pos=None) -> dict:
        """Validate and plan on the host only (no device work)."""
        self.plan.assemble(span_ptr, spans, new_ptr, new_pos, None, None, 2 ** 62, DRY_RUN, None)
        return self.plan.summary()

    def set_decode_rows(self, rows: int):
        """Reserve rows for decode tokens after each request (takes effect at the next assemble)."""
        self.plan.set_decode_rows(rows)

    def decode_layer(self, layer, step, q, k_new, v_new, out=None, variant: int = VARIANT_MATERIALIZED):
        if out is None:
            out = self.torch.empty_like(q)
        self.plan.decode_layer(layer, step, q, k_new, v_new, out, variant, self.torch.cuda.current_stream())
        return out

    def prefill_layer(self, layer, q, k_new, v_new, out=None, variant: int = VARIANT_MATERIALIZED):
        if out is None:
            out = self.torch.empty_like(q)
        self.plan.query_prefill(layer, q, k_new, v_new, out, variant, self.torch.cuda.current_stream())
        return out

    def close(self):
        self.plan.release()
        if self.store is not None:
            self.store.release()
        if self.cache is not None:
            self.cache.release()
        self.pool.release()
