"""Helpers shared by the GPU parity tests: oracle inputs read back from the
device, comparison metrics with the tolerances the method fixes.

Tolerances:
  * gathered values and keys moved by a zero delta: bit-exact;
  * rotated bf16 keys (and rotated new keys): within 1 bf16 ulp of the fp64
    oracle rounded to bf16 (ordinal distance of the bit patterns, +0 == -0);
  * rotated fp32 keys: within 2^-21 * |(x_k, x_{k+d/2})| of the fp64 value;
  * attention: relative L2 <= 5e-3 (bf16) or 1e-5 (fp32) per checked layer,
    and per element |got - ref| <= atol + e_out + e_p (atol 1e-2 bf16,
    1e-5 fp32), where the two other terms are the errors the bf16 path's
    own arithmetic forces, whatever the kernel:
      e_out = half a bf16 ulp of the output (the result is stored in bf16:
              an output near 40 already sits on a grid of 0.25);
      e_p   = 2^-9 * sum_r p_r |v_r - O| over the visible rows: each
              probability is rounded to bf16 (relative error <= 2^-9)
              before the P.V product, and the softmax denominator sums the
              same rounded weights, so the output moves by the weighted
              deviation of the values (first order; it matters where value
              channels are large, as the x20 outlier channels of the
              long-context workloads are).
    e_p is computed exactly, from the oracle's fp64 probabilities, for the
    elements whose error exceeds half of atol + e_out (fp32 outputs:
    e_out = e_p = 0).
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


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x|: 2^(e - 8) for |x| = m 2^e, 0.5 <= m < 1
    (8 significant bits); the smallest normal spacing below that range."""
    _, e = np.frexp(np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def prob_rounding_term(q_rot, k_rows, v_rows, pos_rows, pos_q, kv_heads, o_ref, elems):
    """2^-9 * sum_r p_r |v_r,c - O_c| for the output elements `elems`
    (indices (token, head, channel)), with p the fp64 softmax weights of the
    visible rows: the first-order effect of rounding every probability to
    bf16 when the denominator sums the same rounded weights.  The weights
    are formed once per (token, head)."""
    q_rot = np.asarray(q_rot, np.float64)
    d = q_rot.shape[-1]
    group = q_rot.shape[1] // kv_heads
    out = np.zeros(len(elems[0]))
    by_row = {}
    for i, (j, h) in enumerate(zip(elems[0], elems[1])):
        by_row.setdefault((int(j), int(h)), []).append(i)
    for (j, h), idx in by_row.items():
        g = h // group
        vis = np.asarray(pos_rows) <= pos_q[j]
        z = np.asarray(k_rows[g], np.float64)[vis] @ q_rot[j, h] / np.sqrt(d)
        p = np.exp(z - z.max())
        p /= p.sum()
        cs = np.asarray(elems[2])[idx]
        v = np.asarray(v_rows[g], np.float64)[vis][:, cs]
        out[idx] = 2.0 ** -9 * (p @ np.abs(v - o_ref[j, h, cs][None, :]))
    return out


def attn_check(got, o_ref, dtype, q_rot=None, k_rows=None, v_rows=None, pos_rows=None, pos_q=None,
               kv_heads=None):
    """Attention parity metrics (see the module header); returns a dict with
    max_abs, rel_l2, ratio = max |got - ref| / (atol + e_out + e_p), which
    must be <= 1, and ratio_without_p (the same without e_p).  e_p is formed
    for every element whose error exceeds half of atol + e_out, so `ratio` is
    the full bound's wherever it could come near 1.  For bf16 the oracle's
    q', rows and positions are needed."""
    got = np.asarray(got, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    err = np.abs(got - o_ref)
    rl2 = float(np.linalg.norm(got - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    bound = np.full(err.shape, ATOL[dtype])
    if dtype == "bf16":
        bound += 0.5 * ulp_bf16(np.maximum(np.abs(got), np.abs(o_ref)))
    ratio_without_p = float((err / bound).max(initial=0.0))
    near = np.nonzero(err > 0.5 * bound)
    if dtype == "bf16" and len(near[0]):
        bound[near] += prob_rounding_term(q_rot, k_rows, v_rows, pos_rows, np.asarray(pos_q), kv_heads,
                                          o_ref, near)
    return dict(max_abs=float(err.max(initial=0.0)), rel_l2=rl2, ratio=float((err / bound).max(initial=0.0)),
                ratio_without_p=ratio_without_p)


def attn_ok(st: dict, dtype: str) -> bool:
    return st["ratio"] <= 1.0 and st["rel_l2"] <= RL2[dtype]


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
