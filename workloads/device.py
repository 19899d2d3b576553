"""Put a workload on the device and drive the library with it.

Glue only: allocate and fill the pool, register it, size the assembled
buffers, produce each layer's new-token inputs.  No arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import (Workload, alloc_pool, channel_scales, decode_tokens, fill_pool, new_tokens)


@dataclass
class DeviceWorkload:
    wl: Workload
    pool: object          # torch tensor [n_pages][L][2][Hkv][P][d]
    kscale: object
    vscale: object
    session: object       # position_independent_kv_pic_amd.session.Session

    def layer_inputs(self, layer: int):
        return new_tokens(self.wl, layer, self.kscale, self.vscale, self.kscale.device)

    def decode_inputs(self, layer: int, step: int):
        return decode_tokens(self.wl, layer, step, self.kscale, self.vscale, self.kscale.device)

    def assemble(self, plan_only: bool = False, defer: bool = False, values_in_pool: bool = False):
        wl = self.wl
        return self.session.assemble(wl.span_ptr(), wl.spans_flat(), wl.new_ptr(), wl.new_pos_flat(),
                                     plan_only=plan_only, defer=defer, values_in_pool=values_in_pool)

    def close(self):
        self.session.close()


def open_workload(wl: Workload, device="cuda", host_pool: bool = False, hot_pages: int = 0) -> DeviceWorkload:
    """Fill the pool on the device; with host_pool it is then moved to pinned
    host memory (the staging tier) and the device copy freed, and hot_pages > 0
    puts an HBM hot set of that many page slots in front of it."""
    import torch
    from position_independent_kv_pic_amd.session import Session
    ks, vs = channel_scales(wl, device)
    pool = fill_pool(wl, alloc_pool(wl, device), ks, vs)
    torch.cuda.synchronize()
    if host_pool:
        host = torch.empty(pool.shape, dtype=pool.dtype, pin_memory=True)
        host.copy_(pool)
        del pool
        torch.cuda.empty_cache()
        pool = host
    m, p = wl.model, wl.pool
    sess = Session(m.layers, m.q_heads, m.kv_heads, m.head_dim, m.theta, m.dtype, pool, p.page_tokens,
                   p.chunk_len, p.chunk_page_ptr, p.page_ids, p.chunk_orig, keys=wl.keys,
                   hot_pages=hot_pages if host_pool else 0)
    return DeviceWorkload(wl, pool, ks, vs, sess)
