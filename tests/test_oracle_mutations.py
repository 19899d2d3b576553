"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch each one.

Each mutant replaces one oracle function with a version carrying a typical
slip (a wrong sign, a swapped pairing, a dropped term, an off-by-one mask,
a transposed head mapping, a twice-rounded conversion).  The pin tests are
run against the mutant; at least one must fail.
"""
import math

import numpy as np
import pytest

from oracle import pic_oracle as orc

import test_oracle_pins as pins

PINS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_") and callable(getattr(pins, n))]


def _run_pins():
    """Run every pin; return how many fail."""
    failed = 0
    for fn in PINS:
        params = getattr(fn, "pytestmark", [])
        cases = [()]
        for mark in params:
            if mark.name == "parametrize":
                cases = [tuple(c) if isinstance(c, (tuple, list)) else (c,) for c in mark.args[1]]
        for args in cases:
            try:
                fn(*args)
            except (AssertionError, ValueError, IndexError):
                failed += 1
    return failed


def _rotate_wrong_sign(x, pos, theta):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, np.float64)[..., None] * orc.rope_frequencies(d, theta)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * np.cos(ang) + b * np.sin(ang), -a * np.sin(ang) + b * np.cos(ang)], -1)


def _rotate_interleaved(x, pos, theta):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, np.float64)[..., None] * orc.rope_frequencies(d, theta)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(np.broadcast_to(x, np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,))))
    out[..., 0::2] = a * np.cos(ang) - b * np.sin(ang)
    out[..., 1::2] = a * np.sin(ang) + b * np.cos(ang)
    return out


def _freq_wrong_exponent(head_dim, theta):
    k = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -k / head_dim)


def _plan_delta_flipped(spans, chunk_orig=None):
    out = _ORIG["plan_spans"](spans, chunk_orig)
    return [orc.PlannedSpan(p.chunk, p.s, p.e, p.target, -p.delta) for p in out]


def _plan_exclusive_end(spans, chunk_orig=None):
    out, nxt = [], 0
    for (c, s, e, t) in spans:
        target = nxt if t == orc.TARGET_AUTO else t
        o = 0 if chunk_orig is None else chunk_orig[c]
        out.append(orc.PlannedSpan(c, s, e, target, target - (o + s)))
        nxt = target + (e - s)
    return out


def _attention_strict_mask(q_rot, k_rows, v_rows, pos_rows, pos_q, kv_heads):
    return _ORIG["attention"](q_rot, k_rows, v_rows, np.asarray(pos_rows) + 1, pos_q, kv_heads)


def _attention_head_modulo(q_rot, k_rows, v_rows, pos_rows, pos_q, kv_heads):
    q_rot = np.asarray(q_rot, np.float64)
    n, hq, d = q_rot.shape
    vis = np.asarray(pos_rows)[None, :] <= np.asarray(pos_q)[:, None]
    out = np.zeros((n, hq, d))
    for h in range(hq):
        g = h % kv_heads
        z = q_rot[:, h] @ np.asarray(k_rows[g]).T / math.sqrt(d)
        z = np.where(vis, z, -np.inf)
        p = np.exp(z - z.max(1, keepdims=True))
        out[:, h] = (p / p.sum(1, keepdims=True)) @ np.asarray(v_rows[g])
    return out


def _attention_no_scale(q_rot, k_rows, v_rows, pos_rows, pos_q, kv_heads):
    d = np.asarray(q_rot).shape[-1]
    return _ORIG["attention"](np.asarray(q_rot) * math.sqrt(d), k_rows, v_rows, pos_rows, pos_q, kv_heads)


def _bf16_via_fp32(x):
    return _ORIG["round_bf16"](np.asarray(x, np.float64).astype(np.float32).astype(np.float64))


def _bf16_truncate(x):
    x = np.asarray(x, np.float64).astype(np.float32)
    b = x.view(np.uint32) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


_ORIG = {n: getattr(orc, n) for n in ("rotate", "rope_frequencies", "plan_spans", "attention", "round_bf16",
                                     "prologue")}


def _prologue_unrounded(q, k_new, v_new, pos_new, theta, dtype):
    # q' and k' left in fp64: the new keys never take the cache's storage type
    _, _, v = _ORIG["prologue"](q, k_new, v_new, pos_new, theta, dtype)
    p = np.asarray(pos_new, dtype=np.float64)[:, None]
    return orc.rotate(q, p, theta), orc.rotate(k_new, p, theta), v


def _prologue_keys_unrounded(q, k_new, v_new, pos_new, theta, dtype):
    qr, _, v = _ORIG["prologue"](q, k_new, v_new, pos_new, theta, dtype)
    return qr, orc.rotate(k_new, np.asarray(pos_new, dtype=np.float64)[:, None], theta), v


def _prologue_rotates_values(q, k_new, v_new, pos_new, theta, dtype):
    qr, kr, _ = _ORIG["prologue"](q, k_new, v_new, pos_new, theta, dtype)
    p = np.asarray(pos_new, dtype=np.float64)[:, None]
    return qr, kr, orc.to_storage(orc.rotate(v_new, p, theta), dtype)


def _prologue_position_off_by_one(q, k_new, v_new, pos_new, theta, dtype):
    return _ORIG["prologue"](q, k_new, v_new, np.asarray(pos_new) + 1, theta, dtype)

_orig_assemble = orc.assemble
_orig_new_positions = orc.new_token_positions
_orig_plan_spans = orc.plan_spans


def _assemble_unrotated_by_span_delta(chunk_k, chunk_v, spans, theta, dtype, chunk_orig=None,
                                      keys=orc.KEYS_ROTATED):
    # un-rotated keys moved by the span's delta, as if they were stored rotated
    return _orig_assemble(chunk_k, chunk_v, spans, theta, dtype, chunk_orig=chunk_orig)


def _new_positions_after_last_span(planned, n_new, explicit=None):
    if explicit is not None:
        return _orig_new_positions(planned, n_new, explicit)
    start = planned[-1].target + planned[-1].length if planned else 0
    return start + np.arange(n_new, dtype=np.int64)


def _plan_original_ignores_base(spans, chunk_orig=None):
    # TARGET_ORIGINAL resolved to s, forgetting the chunk's original base
    fixed = [(c, s, e, s if t == orc.TARGET_ORIGINAL else t) for (c, s, e, t) in spans]
    return _orig_plan_spans(fixed, chunk_orig)


MUTANTS = [
    ("assemble", _assemble_unrotated_by_span_delta),
    ("new_token_positions", _new_positions_after_last_span),
    ("plan_spans", _plan_original_ignores_base),
    ("rotate", _rotate_wrong_sign),
    ("rotate", _rotate_interleaved),
    ("rope_frequencies", _freq_wrong_exponent),
    ("plan_spans", _plan_delta_flipped),
    ("plan_spans", _plan_exclusive_end),
    ("attention", _attention_strict_mask),
    ("attention", _attention_head_modulo),
    ("attention", _attention_no_scale),
    ("round_bf16", _bf16_via_fp32),
    ("round_bf16", _bf16_truncate),
    ("prologue", _prologue_unrounded),
    ("prologue", _prologue_keys_unrounded),
    ("prologue", _prologue_rotates_values),
    ("prologue", _prologue_position_off_by_one),
]


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == 0


@pytest.mark.parametrize("target,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, target, mutant):
    monkeypatch.setattr(orc, target, mutant)
    assert _run_pins() > 0
