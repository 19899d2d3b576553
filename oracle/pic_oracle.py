"""Plain fp64 CPU oracle for position-independent KV-cache reuse.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the test-suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code, tables or helpers with the HIP library; it
reads nothing but the generated input values.

What it computes, step by step, in the order and notation of the pages:

* CoinRAG page, section 2.3 (RoPE position rotation and contiguous prefix
  concatenation): the assembled prefix is the prompt cache followed by each
  retrieved span C_b[s:e], each rotated to its new place; the i-th span's new
  start position is the prompt length plus the lengths (e - s + 1) of the spans
  before it; the query is then prefilled against that prefix.
* TurboRAG review page, section on the two inconsistencies (attention mask and
  position id), Figures 4 and 5: chunks never attend to each other, the query
  sees every chunk and itself; "reordered" positions are contiguous while
  "composite" positions restart at 0 in every chunk; keys are moved to their
  new positions by applying RoPE again.
* SemPIC page, paragraph on serving a cache hit: assign final logical
  positions, re-rotate the cached keys, run the inline tokens, interleave the
  compiled and inline caches under a causal mask.

Readings of points the pages leave open (each listed in the design notes):
  - span end e is inclusive (the length is e - s + 1);
  - RoPE is the standard half-split form, omega_k = theta^(-2k/d), no
    frequency scaling; the pages never write the formula out;
  - positions are 0-based; cached keys are stored already rotated at their
    original position o_c + t (o_c = 0 unless registered otherwise), or, for a
    cache built the TurboRAG review page's alternative way (Reordered
    Positions paragraph), stored un-rotated;
  - a span moved from original start o_c + s to target T is rotated by
    delta = T - (o_c + s), the same delta for every token of the span; an
    un-rotated key is rotated by its new position T + t;
  - a span may keep its original positions (target o_c + s, delta 0): the
    page's composite positions, where every chunk restarts at 0;
  - new tokens without explicit positions start right after the whole
    prefix: at the larger of the total span length and the furthest span
    end (Figure 5 puts the query after the concatenated chunks even when
    their positions restart);
  - a rotation by angle zero is the identity (values copied, not recomputed);
  - softmax scale 1/sqrt(d); query head h reads kv head floor(h / G);
  - a new token at position P sees every row (cached or new) whose position
    is <= P: this is the independent-attention mask for the TurboRAG and
    CoinRAG layouts and SemPIC's causal interleave for interleaved layouts;
  - rotated keys, rotated queries and rotated new keys are rounded to the
    storage type (round to nearest, ties to even); attention is evaluated in
    fp64 on those stored operands.

Every function below is pinned by the CPU tests (tests/test_oracle_pins.py)
against closed forms, a matrix-exponential construction of the rotation, a
dense causal prefill, the pages' worked example and bf16 rounding of a
library routine.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

# span target meaning "continue right after the previous span"
TARGET_AUTO = -1
# span target meaning "keep the span's original positions" (delta = 0)
TARGET_ORIGINAL = -2

# how the pool stores keys
KEYS_ROTATED = "rotated"       # RoPE applied at the original position o_c + t
KEYS_UNROTATED = "unrotated"   # raw keys; RoPE applied at the new position

STORAGE_TYPES = ("bf16", "f32", "f64")

# largest finite bfloat16: (2 - 2^-7) * 2^127
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# ---------------------------------------------------------------------------
# rounding to the storage type
# ---------------------------------------------------------------------------

def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (ties to even), directly.

    bfloat16 keeps 8 significant bits with fp32's exponent range.  Writing
    x = m * 2^e with 0.5 <= |m| < 1, the spacing of representable values near
    x is 2^(e-8), but never finer than the subnormal spacing 2^-133.  Rounding
    is done in one step from fp64 (no detour through fp32, which would round
    twice).  Returns fp64 values that are exactly representable in bf16.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)
    q = np.maximum(e - 8, -133)
    y = np.ldexp(np.round(np.ldexp(xf, -q)), q)  # np.round: half to even
    over = np.abs(y) > _BF16_MAX
    y[over] = np.copysign(np.inf, y[over])
    out[fin] = y
    return out


def round_f32(x) -> np.ndarray:
    """Round fp64 values to the nearest fp32 (numpy's cast rounds to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_storage(x, dtype: str) -> np.ndarray:
    """Round to the cache's storage type; "f64" keeps values unrounded (pins only)."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown storage type {dtype!r}")


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """omega_k = theta^(-2k/d), k = 0 .. d/2-1, in fp64 (standard RoPE)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * k / head_dim)


def rotate(x, pos, theta: float) -> np.ndarray:
    """R(pos) applied to the last axis of x (half-split pairs (k, k + d/2)).

    x'_k       = x_k cos(pos*w_k) - x_{k+d/2} sin(pos*w_k)
    x'_{k+d/2} = x_k sin(pos*w_k) + x_{k+d/2} cos(pos*w_k)

    `pos` broadcasts against x.shape[:-1].  Entries whose angle is exactly
    zero (pos == 0) are returned unchanged: R(0) is the identity.
    TurboRAG review page, Reordered Positions: keys are moved by applying RoPE
    at the new position; CoinRAG page section 2.3, Rot(.; Delta_i).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    w = rope_frequencies(d, theta)
    p = np.asarray(pos, dtype=np.float64)
    ang = p[..., None] * w
    c = np.cos(ang)
    s = np.sin(ang)
    a = x[..., :half]
    b = x[..., half:]
    out = np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
    ident = np.broadcast_to(p == 0, x.shape[:-1])
    if np.any(ident):
        out = np.where(ident[..., None], x, out)
    return out


# ---------------------------------------------------------------------------
# span planning: targets and deltas (CoinRAG page, section 2.3, Delta_i)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class PlannedSpan:
    chunk: int
    s: int
    e: int          # inclusive
    target: int     # new position of token s
    delta: int      # rotation applied to every key of the span

    @property
    def length(self) -> int:
        return self.e - self.s + 1


def plan_spans(spans: Sequence[Tuple[int, int, int, int]],
               chunk_orig: Optional[Sequence[int]] = None) -> List[PlannedSpan]:
    """Resolve targets and rotation deltas of one request's span table.

    A span is (chunk, s, e, target) with e inclusive.  target == TARGET_AUTO
    places the span right after the previous one (at 0 for the first):
    with the prompt cache as span 0 and every other span AUTO this is the
    CoinRAG Delta equation, Delta_i = |p| + sum_{j<i} (e_j - s_j + 1).
    target == TARGET_ORIGINAL keeps the span where it was encoded, o_c + s
    (TurboRAG review page, Figure 5: composite positions).
    delta = target - (o_c + s), where o_c is the chunk's original base.
    """
    out: List[PlannedSpan] = []
    nxt = 0
    for (c, s, e, t) in spans:
        if e < s:
            raise ValueError("span end before start")
        n = e - s + 1
        o = 0 if chunk_orig is None else int(chunk_orig[c])
        if t == TARGET_AUTO:
            target = nxt
        elif t == TARGET_ORIGINAL:
            target = o + int(s)
        else:
            target = int(t)
        out.append(PlannedSpan(int(c), int(s), int(e), target, target - (o + int(s))))
        nxt = target + n
    return out


def new_token_positions(planned: Sequence[PlannedSpan], n_new: int,
                        explicit: Optional[Sequence[int]] = None) -> np.ndarray:
    """Positions of the request's new tokens.

    Explicit positions are taken as given (SemPIC: final logical positions).
    Otherwise they start right after the whole prefix: at the larger of the
    total span length and the furthest span end.  For a contiguous prefix of
    length n both are n; with composite positions (every chunk restarting at
    0) the first is larger, and TurboRAG Figure 5 indeed places the query
    after the concatenated chunks (13..16 after three 4-token chunks).
    """
    if explicit is not None:
        p = np.asarray(explicit, dtype=np.int64)
        if p.shape != (n_new,):
            raise ValueError("explicit positions have the wrong length")
        return p
    total = sum(sp.length for sp in planned)
    furthest = max((sp.target + sp.length for sp in planned), default=0)
    return max(total, furthest) + np.arange(n_new, dtype=np.int64)


# ---------------------------------------------------------------------------
# assembly: gather + re-rotation (CoinRAG section 2.3, C_ctx equation)
# ---------------------------------------------------------------------------

def assemble(chunk_k: Sequence[np.ndarray], chunk_v: Sequence[np.ndarray],
             spans: Sequence[Tuple[int, int, int, int]], theta: float, dtype: str,
             chunk_orig: Optional[Sequence[int]] = None, keys: str = KEYS_ROTATED):
    """Gather every span's cached K/V rows into one contiguous prefix.

    chunk_k[c], chunk_v[c]: arrays [L][Hkv][len_c][d] of stored values.
    Returns (K [L][Hkv][rows][d], V [L][Hkv][rows][d], pos [rows]) with rows
    in span order: for span i and t = 0 .. e_i - s_i the row holds position
    target_i + t and value V_c[s_i + t] copied.  Its key, rounded to the
    storage type, is
      keys == KEYS_ROTATED:   R(delta_i) K_c[s_i + t]  (CoinRAG section 2.3,
                              Rot(.; Delta_i): one rotation per span);
      keys == KEYS_UNROTATED: R(target_i + t) K_c[s_i + t]  (TurboRAG review
                              page, Reordered Positions: RoPE applied once, at
                              the token's new position).
    """
    if keys not in (KEYS_ROTATED, KEYS_UNROTATED):
        raise ValueError(f"unknown key storage {keys!r}")
    planned = plan_spans(spans, chunk_orig)
    ks, vs, pos = [], [], []
    for sp in planned:
        k = np.asarray(chunk_k[sp.chunk], dtype=np.float64)[:, :, sp.s:sp.e + 1, :]
        v = np.asarray(chunk_v[sp.chunk], dtype=np.float64)[:, :, sp.s:sp.e + 1, :]
        p = sp.target + np.arange(sp.length, dtype=np.int64)
        if keys == KEYS_UNROTATED:
            angle = np.broadcast_to(p, k.shape[:-1])
            if np.any(p != 0):
                k = to_storage(rotate(k, angle, theta), dtype)
        elif sp.delta != 0:
            k = to_storage(rotate(k, sp.delta, theta), dtype)
        ks.append(k)
        vs.append(v)
        pos.append(p)
    if not ks:
        raise ValueError("assemble() needs at least one span; use empty_prefix()")
    return np.concatenate(ks, axis=2), np.concatenate(vs, axis=2), np.concatenate(pos)


def empty_prefix(layers: int, kv_heads: int, head_dim: int):
    """The prefix of a request with no spans."""
    z = np.zeros((layers, kv_heads, 0, head_dim))
    return z, z.copy(), np.zeros(0, dtype=np.int64)


# ---------------------------------------------------------------------------
# new tokens and attention (CoinRAG KV_M(q; C_ctx); TurboRAG Figure 4;
# SemPIC causal interleave)
# ---------------------------------------------------------------------------

def prologue(q, k_new, v_new, pos_new, theta: float, dtype: str):
    """Rotate new queries and keys to their positions and round them.

    q: [n][Hq][d], k_new/v_new: [n][Hkv][d], pos_new: [n].
    Returns (q', k', v) with q' = R(P_j) q_j and k' = R(P_j) k_j rounded to
    the storage type; v is used as given.
    """
    p = np.asarray(pos_new, dtype=np.float64)[:, None]
    qr = to_storage(rotate(q, p, theta), dtype)
    kr = to_storage(rotate(k_new, p, theta), dtype)
    return qr, kr, np.asarray(v_new, dtype=np.float64)


def attention(q_rot, k_rows, v_rows, pos_rows, pos_q, kv_heads: int) -> np.ndarray:
    """Brute-force masked softmax attention in fp64.

    q_rot: [n][Hq][d]; k_rows, v_rows: [Hkv][R][d]; pos_rows: [R]; pos_q: [n].
    For query token j and head h (kv head g = h // (Hq / Hkv)):
    z_r = <q'_j,h, k_r,g> / sqrt(d) over rows with pos_r <= pos_q[j],
    p = softmax(z), O_j,h = sum_r p_r v_r,g.
    """
    q_rot = np.asarray(q_rot, dtype=np.float64)
    n, hq, d = q_rot.shape
    group = hq // kv_heads
    pos_rows = np.asarray(pos_rows, dtype=np.int64)
    pos_q = np.asarray(pos_q, dtype=np.int64)
    visible = pos_rows[None, :] <= pos_q[:, None]          # [n][R]
    out = np.zeros((n, hq, d), dtype=np.float64)
    scale = 1.0 / math.sqrt(d)
    for h in range(hq):
        g = h // group
        z = (q_rot[:, h, :] @ np.asarray(k_rows[g], dtype=np.float64).T) * scale
        z = np.where(visible, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ np.asarray(v_rows[g], dtype=np.float64)
    return out


def query_prefill_layer(k_prefix, v_prefix, pos_prefix, q, k_new, v_new, pos_new,
                        theta: float, dtype: str, kv_heads: int,
                        query_subset: Optional[Sequence[int]] = None):
    """One layer of KV_M(q; C_ctx) for one request.

    k_prefix, v_prefix: [Hkv][R][d] (one layer of the assembled prefix),
    q: [n][Hq][d], k_new, v_new: [n][Hkv][d] (un-rotated), pos_new: [n].
    The new rows are appended after the prefix (C_ctx (+) KV_M(q; C_ctx)).
    Returns (O [n'][Hq][d] for the chosen query tokens, k' [n][Hkv][d],
    v [n][Hkv][d], q' [n][Hq][d]).
    """
    qr, kr, vr = prologue(q, k_new, v_new, pos_new, theta, dtype)
    k_all = np.concatenate([np.asarray(k_prefix, np.float64), kr.transpose(1, 0, 2)], axis=1)
    v_all = np.concatenate([np.asarray(v_prefix, np.float64), vr.transpose(1, 0, 2)], axis=1)
    pos_all = np.concatenate([np.asarray(pos_prefix, np.int64), np.asarray(pos_new, np.int64)])
    sel = np.arange(qr.shape[0]) if query_subset is None else np.asarray(query_subset)
    o = attention(qr[sel], k_all, v_all, pos_all, np.asarray(pos_new)[sel], kv_heads)
    return o, kr, vr, qr
