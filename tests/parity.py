"""Helpers shared by the GPU parity tests: oracle inputs read back from the
device, comparison metrics with the tolerances the method fixes.

Tolerances:
  * gathered values and keys moved by a zero delta: bit-exact;
  * rotated bf16 keys (and rotated new keys): within 1 bf16 ulp of the fp64
    oracle rounded to bf16 (ordinal distance of the bit patterns, +0 == -0);
  * rotated fp32 keys: within 2^-21 * |(x_k, x_{k+d/2})| of the fp64 value;
  * attention: bf16 max-abs <= 1e-2 and relative L2 <= 5e-3 per checked
    layer; fp32 both <= 1e-5.  Attention is linear in V channel by channel,
    so an output channel whose value channel carries a scale s > 1 (the
    x20 outlier channels of the long-context workloads) is compared after
    dividing its error by s: one bf16 rounding of an exact output near 40 is
    already 0.125, which no bf16 result can beat in absolute terms.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W
from oracle import pic_oracle as orc

ATOL = {"bf16": 1e-2, "f32": 1e-5}
RL2 = {"bf16": 5e-3, "f32": 1e-5}


def bf16_ordinal(x: torch.Tensor) -> torch.Tensor:
    """Monotone integer code of bf16 values (+0 and -0 both map to 0)."""
    b = x.to(torch.bfloat16).contiguous().view(torch.int16).to(torch.int32)
    mag = b & 0x7FFF
    return torch.where(b < 0, -mag, mag)


def ulp_distance_bf16(a, b) -> torch.Tensor:
    a = torch.as_tensor(a)
    b = torch.as_tensor(b)
    return (bf16_ordinal(a) - bf16_ordinal(b)).abs()


def request_prefix(wl: W.Workload, pool, b: int, layers):
    """Oracle assembly of request b for the given layers (fp64 numpy)."""
    r = wl.requests[b]
    if len(r.spans) == 0:
        return orc.empty_prefix(len(layers), wl.model.kv_heads, wl.model.head_dim)
    chunks = sorted(set(int(c) for c in r.spans[:, 0]))
    ck, cv = {}, {}
    for c in chunks:
        k, v = W.chunk_kv(wl, pool, c, layers)
        ck[c] = k.numpy()
        cv[c] = v.numpy()
    return orc.assemble(ck, cv, [tuple(int(x) for x in s) for s in r.spans], wl.model.theta,
                        wl.model.dtype, chunk_orig=wl.pool.chunk_orig, keys=wl.keys)


def request_positions(wl: W.Workload, b: int):
    r = wl.requests[b]
    planned = orc.plan_spans([tuple(int(x) for x in s) for s in r.spans], wl.pool.chunk_orig)
    return orc.new_token_positions(planned, r.n_new, r.new_pos)


def channel_scale(vscale_layer: np.ndarray, group: int) -> np.ndarray:
    """[Hq][d] divisor for the max-abs check: max(1, scale of the value
    channel each output channel averages), query head h reading kv head h // G."""
    s = np.maximum(1.0, np.asarray(vscale_layer, np.float64))      # [Hkv][d]
    return np.repeat(s, group, axis=0)


def attn_metrics(got: np.ndarray, ref: np.ndarray, scale=None):
    """(max-abs error, with channels divided by `scale` [Hq][d] if given; relative L2)."""
    err = np.abs(got - ref)
    if scale is not None:
        err = err / scale[None]
    return float(err.max(initial=0.0)), float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def compare_keys(got: np.ndarray, ref: np.ndarray, dtype: str, exact_mask=None):
    """Return (max ulp or scaled error, count not bit-exact); raises on violation."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0, 0
    if dtype == "bf16":
        d = ulp_distance_bf16(torch.from_numpy(got), torch.from_numpy(ref))
        if exact_mask is not None:
            m = torch.from_numpy(np.broadcast_to(exact_mask, d.shape).copy())
            assert torch.equal(torch.from_numpy(got)[m], torch.from_numpy(ref)[m]), "zero-delta keys differ"
        assert int(d.max()) <= 1, f"rotated key off by {int(d.max())} bf16 ulp"
        return int(d.max()), int((d > 0).sum())
    half = got.shape[-1] // 2
    norm = np.sqrt(ref[..., :half] ** 2 + ref[..., half:] ** 2)
    bound = 2.0 ** -21 * np.concatenate([norm, norm], axis=-1)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"fp32 rotated key error {float((err / np.maximum(bound, 1e-300)).max())} x bound"
    return float(err.max()), int((err > 0).sum())
