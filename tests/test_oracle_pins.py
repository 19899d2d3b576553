"""Pins for the CPU oracle: closed forms, library routines, the pages' worked example.

Every check here is independent of the oracle's own formulas: rotations are
compared with a matrix exponential of the RoPE generator, attention with a
dense causal prefill over an explicit lower-triangular mask, bf16 rounding with
torch's fp32 -> bf16 conversion, positions with the worked example printed on
the TurboRAG review page (Figure 5).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

from oracle import pic_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent constructions used only by these pins
# ---------------------------------------------------------------------------

def rope_matrix(d, theta, pos):
    """R(pos) = expm(pos * A), A the skew generator coupling (k, k+d/2) at rate w_k.

    w_k is built as exp(-(2k/d) ln theta), not with the oracle's power().
    """
    h = d // 2
    a = np.zeros((d, d))
    for k in range(h):
        w = math.exp(-(2.0 * k / d) * math.log(theta))
        a[k + h, k] = w
        a[k, k + h] = -w
    return scipy.linalg.expm(pos * a)


def rope_ref(x, theta, pos):
    """Apply R(pos) row by row through the matrix exponential."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    flat = x.reshape(-1, d)
    p = np.broadcast_to(np.asarray(pos, np.float64), x.shape[:-1]).reshape(-1)
    out = np.empty_like(flat)
    cache = {}
    for i in range(flat.shape[0]):
        key = float(p[i])
        if key not in cache:
            cache[key] = rope_matrix(d, theta, key)
        out[i] = cache[key] @ flat[i]
    return out.reshape(x.shape)


def dense_causal_prefill(q, k, v, kv_heads):
    """Ordinary causal attention over a full sequence (rows already rotated).

    q: [N][Hq][d], k, v: [N][Hkv][d].  Explicit lower-triangular mask,
    scipy's softmax.  Returns [N][Hq][d].
    """
    n, hq, d = q.shape
    group = hq // kv_heads
    mask = np.tril(np.ones((n, n), dtype=bool))
    out = np.zeros_like(q)
    for h in range(hq):
        g = h // group
        s = q[:, h, :] @ k[:, g, :].T / math.sqrt(d)
        s[~mask] = -np.inf
        out[:, h, :] = scipy.special.softmax(s, axis=1) @ v[:, g, :]
    return out


# ---------------------------------------------------------------------------
# rounding
# ---------------------------------------------------------------------------

def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
        rng.standard_normal(2000) * 1e-39,                          # bf16 subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 3e38, -3e38, 1.0 + 2.0 ** -8]),
    ]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.round_bf16(vals.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_round_bf16_is_single_rounding_from_fp64():
    # 1 + 2^-8 + 2^-30 lies just above the tie between 1 and 1 + 2^-7; through
    # fp32 it would first become the exact tie and then round down to 1.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert orc.round_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    # exact ties go to the even neighbour
    assert orc.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert orc.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert np.isinf(orc.round_bf16(np.array([3.4e38]))[0])


def test_round_f32_matches_numpy_cast():
    x = np.random.default_rng(2).standard_normal(1000) * 1e3
    assert np.array_equal(orc.round_f32(x), x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,theta", [(8, 1e4), (64, 1e4), (128, 1e6), (128, 5e5)])
def test_rotation_matches_matrix_exponential(d, theta):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 511, 131071])
    got = orc.rotate(x, pos, theta)
    ref = rope_ref(x, theta, pos)
    # the matrix exponential's own error grows with the angle (scaling and
    # squaring), about 3e-14 per radian here; sign or pairing mistakes are O(1)
    tol = 1e-13 * (1.0 + pos[:, None]) * np.abs(x).max()
    assert np.all(np.abs(got - ref) <= tol)


def test_rotation_unit_vectors_give_cos_sin():
    d, theta, p = 16, 1e4, 3
    for k in range(d // 2):
        e = np.zeros(d)
        e[k] = 1.0
        r = orc.rotate(e, p, theta)
        w = theta ** (-2.0 * k / d)
        assert r[k] == pytest.approx(math.cos(p * w), abs=1e-15)
        assert r[k + d // 2] == pytest.approx(math.sin(p * w), abs=1e-15)


def test_rotation_composition_identity_and_norm():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 128))
    a, b = 1234, -987
    two = orc.rotate(orc.rotate(x, a, 1e6), b, 1e6)
    one = orc.rotate(x, a + b, 1e6)
    assert np.allclose(two, one, rtol=0, atol=1e-12 * 64)
    assert np.array_equal(orc.rotate(x, 0, 1e6), x)
    r = orc.rotate(x, 4096, 1e6)
    n0 = x[:, :64] ** 2 + x[:, 64:] ** 2
    n1 = r[:, :64] ** 2 + r[:, 64:] ** 2
    assert np.allclose(n0, n1, rtol=1e-13)


def test_scores_depend_only_on_position_difference():
    # TurboRAG review page, second key observation: RoPE scores depend only
    # on relative position.
    rng = np.random.default_rng(5)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    for m, n in [(10, 3), (700, 5), (131000, 129000)]:
        lhs = orc.rotate(q, m, 1e6) @ orc.rotate(k, n, 1e6)
        rhs = orc.rotate(q, m - n, 1e6) @ k
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)


# ---------------------------------------------------------------------------
# positions (TurboRAG Figure 5 worked example; CoinRAG Delta equation)
# ---------------------------------------------------------------------------

def test_worked_example_positions():
    with open(os.path.join(GOLDEN, "turborag_fig5_positions.json")) as f:
        g = json.load(f)
    l, k = g["chunk_length"], g["n_chunks"]
    reordered = orc.plan_spans([(c, 0, l - 1, orc.TARGET_AUTO) for c in range(k)])
    pos_r = np.concatenate([sp.target + np.arange(sp.length) for sp in reordered])
    assert pos_r.tolist() == g["reordered_positions"]
    composite = orc.plan_spans([(c, 0, l - 1, 0) for c in range(k)])
    pos_c = np.concatenate([sp.target + np.arange(sp.length) for sp in composite])
    assert pos_c.tolist() == g["composite_positions"]
    assert all(sp.delta == 0 for sp in composite)
    q = orc.new_token_positions(reordered, 4)
    assert q.tolist() == g["query_positions"]
    pr = g["probe"]
    qpos = q[pr["query_index"]]
    assert qpos - pos_c[pr["chunk"] * l + pr["token_in_chunk"]] == g["composite_distance"]
    assert qpos - pos_r[pr["chunk"] * l + pr["token_in_chunk"]] == g["true_distance"]


def test_worked_example_composite_query_follows_the_concatenated_chunks():
    # TurboRAG Figure 5: with composite positions every chunk restarts at 0
    # (kept where it was encoded: TARGET_ORIGINAL), yet the query sits after
    # the concatenated chunks (13..16 in the figure's 1-based labels)
    with open(os.path.join(GOLDEN, "turborag_fig5_positions.json")) as f:
        g = json.load(f)
    l, k = g["chunk_length"], g["n_chunks"]
    composite = orc.plan_spans([(c, 0, l - 1, orc.TARGET_ORIGINAL) for c in range(k)])
    pos_c = np.concatenate([sp.target + np.arange(sp.length) for sp in composite])
    assert pos_c.tolist() == g["composite_positions"]
    assert all(sp.delta == 0 for sp in composite)
    assert orc.new_token_positions(composite, 4).tolist() == g["query_positions"]


def test_target_original_keeps_encoded_positions():
    plan = orc.plan_spans([(0, 3, 7, orc.TARGET_ORIGINAL), (1, 0, 2, orc.TARGET_ORIGINAL),
                           (1, 5, 6, orc.TARGET_AUTO)], chunk_orig=[10, 0])
    assert [sp.target for sp in plan] == [13, 0, 3]
    assert [sp.delta for sp in plan] == [0, 0, 3 - 5]
    # new tokens follow the whole prefix: 5 + 3 + 2 rows, furthest end 18
    assert orc.new_token_positions(plan, 2).tolist() == [18, 19]


def test_delta_equation_with_prompt_and_nuggets():
    # CoinRAG section 2.3: Delta_i = |p| + sum_{j<i} (e_j - s_j + 1)
    prompt = (9, 0, 31, 0)
    nuggets = [(3, 100, 114), (0, 5, 5), (3, 20, 47), (7, 500, 511)]
    plan = orc.plan_spans([prompt] + [(c, s, e, orc.TARGET_AUTO) for c, s, e in nuggets])
    want, acc = [], 32
    for c, s, e in nuggets:
        want.append(acc)
        acc += e - s + 1
    assert [sp.target for sp in plan[1:]] == want
    assert [sp.delta for sp in plan[1:]] == [w - s for w, (_, s, _) in zip(want, nuggets)]
    assert orc.new_token_positions(plan, 3).tolist() == [acc, acc + 1, acc + 2]
    # original base positions shift the delta, not the target
    plan_o = orc.plan_spans([(0, 2, 5, 10)], chunk_orig=[100])
    assert plan_o[0].target == 10 and plan_o[0].delta == 10 - 102


# ---------------------------------------------------------------------------
# assembly
# ---------------------------------------------------------------------------

def _pool(rng, n_chunks, length, layers, kv_heads, d, theta, orig=None):
    """Raw (un-rotated) keys, stored keys pre-rotated at original positions
    through the matrix exponential, and values."""
    raw = [rng.standard_normal((layers, kv_heads, length, d)) for _ in range(n_chunks)]
    base = [0] * n_chunks if orig is None else orig
    stored = [rope_ref(r, theta, (base[c] + np.arange(length))[None, None, :])
              for c, r in enumerate(raw)]
    vals = [rng.standard_normal((layers, kv_heads, length, d)) for _ in range(n_chunks)]
    return raw, stored, vals


def test_assembled_keys_equal_keys_encoded_at_new_positions():
    rng = np.random.default_rng(6)
    theta, d = 1e4, 16
    orig = [0, 40, 7]
    raw, stored, vals = _pool(rng, 3, 24, 2, 2, d, theta, orig)
    spans = [(1, 0, 3, 0), (0, 5, 9, orc.TARGET_AUTO), (2, 23, 23, orc.TARGET_AUTO),
             (0, 5, 9, orc.TARGET_AUTO), (1, 10, 20, 100)]
    k, v, pos = orc.assemble(stored, vals, spans, theta, "f64", chunk_orig=orig)
    assert pos.tolist() == list(range(15)) + list(range(100, 111))
    row = 0
    for (c, s, e, _), p0 in zip(spans, [0, 4, 9, 10, 100]):
        for t in range(e - s + 1):
            want_k = rope_ref(raw[c][:, :, s + t, :], theta, p0 + t)
            assert np.allclose(k[:, :, row, :], want_k, atol=1e-9)
            assert np.array_equal(v[:, :, row, :], vals[c][:, :, s + t, :])
            row += 1
    assert row == k.shape[2]


def test_unrotated_keys_are_rotated_at_their_new_positions():
    # TurboRAG review page, Reordered Positions: store keys before RoPE and
    # apply it at the new position when the caches are concatenated
    rng = np.random.default_rng(16)
    theta, d = 1e4, 16
    orig = [0, 40, 7]
    raw, stored, vals = _pool(rng, 3, 24, 2, 2, d, theta, orig)
    spans = [(1, 0, 3, 0), (0, 5, 9, orc.TARGET_AUTO), (2, 23, 23, orc.TARGET_ORIGINAL),
             (0, 5, 9, orc.TARGET_AUTO), (1, 10, 20, 100)]
    k, v, pos = orc.assemble(raw, vals, spans, theta, "f64", chunk_orig=orig, keys=orc.KEYS_UNROTATED)
    assert pos.tolist() == list(range(9)) + [30] + list(range(31, 36)) + list(range(100, 111))
    row = 0
    for (c, s, e, _) in spans:
        for t in range(e - s + 1):
            want_k = rope_ref(raw[c][:, :, s + t, :], theta, pos[row])
            assert np.allclose(k[:, :, row, :], want_k, atol=1e-9)
            assert np.array_equal(v[:, :, row, :], vals[c][:, :, s + t, :])
            row += 1
    assert row == k.shape[2]
    # the same prefix as from keys stored rotated at their original positions
    k2, _, pos2 = orc.assemble(stored, vals, spans, theta, "f64", chunk_orig=orig)
    assert np.array_equal(pos, pos2)
    assert np.allclose(k, k2, atol=1e-9)


def test_unrotated_unit_keys_give_cos_sin_of_the_new_position():
    d, theta, T = 8, 1e4, 37
    h = d // 2
    chunk = np.zeros((1, 1, h, d))
    for t in range(h):
        chunk[0, 0, t, t] = 1.0          # token t holds the unit vector e_t
    k, _, pos = orc.assemble([chunk], [chunk], [(0, 0, h - 1, T)], theta, "f64",
                             keys=orc.KEYS_UNROTATED)
    for t in range(h):
        w = math.exp(-(2.0 * t / d) * math.log(theta))
        ang = (T + t) * w
        want = np.zeros(d)
        want[t], want[t + h] = math.cos(ang), math.sin(ang)
        assert np.allclose(k[0, 0, t], want, atol=1e-12)
    # a token that lands at position 0 is copied unchanged (R(0) = I)
    k0, _, _ = orc.assemble([chunk], [chunk], [(0, 0, 0, 0)], theta, "f64", keys=orc.KEYS_UNROTATED)
    assert np.array_equal(k0[0, 0, 0], chunk[0, 0, 0])


def test_zero_delta_is_an_exact_copy_and_rounding_applies_otherwise():
    rng = np.random.default_rng(7)
    chunk = [orc.round_bf16(rng.standard_normal((1, 1, 8, 8)))]
    chunk[0][0, 0, 2, 3] = -0.0
    k, _, _ = orc.assemble(chunk, chunk, [(0, 0, 7, 0)], 1e4, "bf16")
    assert np.array_equal(k, chunk[0]) and np.array_equal(np.signbit(k), np.signbit(chunk[0]))
    k2, _, _ = orc.assemble(chunk, chunk, [(0, 0, 7, 5)], 1e4, "bf16")
    assert np.array_equal(k2, orc.round_bf16(k2))
    assert not np.array_equal(k2, chunk[0])


def test_composite_and_reordered_differ_by_one_rotation_per_chunk():
    # TurboRAG Figure 5 vs Reordered Positions: chunk c moves by c*l
    rng = np.random.default_rng(8)
    l, theta = 6, 1e4
    _, stored, vals = _pool(rng, 3, l, 1, 1, 8, theta)
    comp, _, _ = orc.assemble(stored, vals, [(c, 0, l - 1, 0) for c in range(3)], theta, "f64")
    reord, _, _ = orc.assemble(stored, vals, [(c, 0, l - 1, orc.TARGET_AUTO) for c in range(3)],
                               theta, "f64")
    for c in range(3):
        sl = slice(c * l, (c + 1) * l)
        assert np.allclose(reord[:, :, sl], rope_ref(comp[:, :, sl], theta, c * l), atol=1e-12)


def test_edge_spans_one_token_chunk_end_duplicates_negative_delta():
    rng = np.random.default_rng(9)
    theta = 1e4
    raw, stored, vals = _pool(rng, 2, 10, 1, 1, 8, theta)
    spans = [(0, 9, 9, 0), (1, 0, 9, orc.TARGET_AUTO), (1, 0, 9, orc.TARGET_AUTO), (0, 4, 6, 2)]
    k, v, pos = orc.assemble(stored, vals, spans, theta, "f64")
    assert k.shape[2] == 1 + 10 + 10 + 3
    assert pos.tolist() == [0] + list(range(1, 11)) + list(range(11, 21)) + [2, 3, 4]
    assert np.allclose(k[:, :, 0], rope_ref(raw[0][:, :, 9], theta, 0), atol=1e-12)     # delta -9
    assert np.array_equal(v[:, :, 1:11], v[:, :, 11:21])                                # duplicate
    assert np.allclose(k[:, :, 21:24], rope_ref(raw[0][:, :, 4:7], theta, np.arange(2, 5)), atol=1e-12)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def test_single_chunk_at_original_positions_is_ordinary_causal_prefill():
    # TurboRAG: with one chunk nothing is lost; reuse of its cache followed by
    # the query's prefill must equal the last n rows of a full causal prefill.
    rng = np.random.default_rng(10)
    theta, d, hq, hkv, l, n = 1e4, 16, 4, 2, 20, 6
    raw, stored, vals = _pool(rng, 1, l, 1, hkv, d, theta)
    kp, vp, pp = orc.assemble(stored, vals, [(0, 0, l - 1, orc.TARGET_AUTO)], theta, "f64")
    qn = rng.standard_normal((n, hq, d))
    kn = rng.standard_normal((n, hkv, d))
    vn = rng.standard_normal((n, hkv, d))
    pos_new = orc.new_token_positions(orc.plan_spans([(0, 0, l - 1, orc.TARGET_AUTO)]), n)
    o, _, _, _ = orc.query_prefill_layer(kp[0], vp[0], pp, qn, kn, vn, pos_new, theta, "f64", hkv)

    seq_pos = np.arange(l + n)
    k_full = np.concatenate([raw[0][0].transpose(1, 0, 2), kn], axis=0)       # [N][Hkv][d]
    v_full = np.concatenate([vals[0][0].transpose(1, 0, 2), vn], axis=0)
    q_full = np.concatenate([rng.standard_normal((l, hq, d)), qn], axis=0)
    ref = dense_causal_prefill(rope_ref(q_full, theta, seq_pos[:, None]),
                               rope_ref(k_full, theta, seq_pos[:, None]), v_full, hkv)
    assert np.allclose(o, ref[l:], rtol=0, atol=1e-11)


def test_interleaved_layout_is_causal_prefill_in_position_order():
    # SemPIC hit path: documents at their final positions, inline tokens in
    # the gaps, everything interleaved under a causal mask.  Sorting every row
    # by position turns it into an ordinary causal prefill over that order.
    rng = np.random.default_rng(11)
    theta, d, hq, hkv = 5e5, 16, 4, 2
    raw, stored, vals = _pool(rng, 2, 12, 1, hkv, d, theta)
    spans = [(1, 0, 11, 0), (0, 0, 11, 17)]          # gap 12..16 holds inline tokens
    pos_new = np.array([12, 13, 14, 15, 16, 29, 30, 31])
    n = len(pos_new)
    kp, vp, pp = orc.assemble(stored, vals, spans, theta, "f64")
    qn = rng.standard_normal((n, hq, d))
    kn = rng.standard_normal((n, hkv, d))
    vn = rng.standard_normal((n, hkv, d))
    o, _, _, _ = orc.query_prefill_layer(kp[0], vp[0], pp, qn, kn, vn, pos_new, theta, "f64", hkv)

    # dense reference over the 32 positions in order; cached rows use raw keys
    total = 32
    k_seq = np.zeros((total, hkv, d))
    v_seq = np.zeros((total, hkv, d))
    q_seq = rng.standard_normal((total, hq, d))
    for c, s, e, t in [(1, 0, 11, 0), (0, 0, 11, 17)]:
        k_seq[t:t + 12] = raw[c][0].transpose(1, 0, 2)
        v_seq[t:t + 12] = vals[c][0].transpose(1, 0, 2)
    k_seq[pos_new] = kn
    v_seq[pos_new] = vn
    q_seq[pos_new] = qn
    p = np.arange(total)[:, None]
    ref = dense_causal_prefill(rope_ref(q_seq, theta, p), rope_ref(k_seq, theta, p), v_seq, hkv)
    assert np.allclose(o, ref[pos_new], rtol=0, atol=1e-11)


def test_decoding_one_token_at_a_time_equals_prefilling_them_together():
    # the step after the prefill is ordinary autoregressive decoding: a token
    # decoded after the earlier ones (their rotated keys appended as rows)
    # sees exactly what it would see had all been prefilled at once
    rng = np.random.default_rng(21)
    theta, d, hkv, hq = 1e4, 16, 2, 6
    rows = 13
    kp = orc.round_bf16(rng.standard_normal((hkv, rows, d)))
    vp = orc.round_bf16(rng.standard_normal((hkv, rows, d)))
    pp = np.array([0, 1, 2, 7, 8, 9, 10, 3, 4, 5, 6, 11, 12])
    n, steps = 4, 5
    tot = n + steps
    q = orc.round_bf16(rng.standard_normal((tot, hq, d)))
    k = orc.round_bf16(rng.standard_normal((tot, hkv, d)))
    v = orc.round_bf16(rng.standard_normal((tot, hkv, d)))
    pos = 13 + np.arange(tot)
    o_all, _, _, _ = orc.query_prefill_layer(kp, vp, pp, q, k, v, pos, theta, "bf16", hkv)
    o_pre, kr, vr, _ = orc.query_prefill_layer(kp, vp, pp, q[:n], k[:n], v[:n], pos[:n], theta, "bf16", hkv)
    assert np.allclose(o_pre, o_all[:n], atol=1e-13)
    ks = np.concatenate([kp, kr.transpose(1, 0, 2)], axis=1)
    vs = np.concatenate([vp, vr.transpose(1, 0, 2)], axis=1)
    ps = np.concatenate([pp, pos[:n]])
    for s_ in range(steps):
        j = n + s_
        o1, k1, v1, _ = orc.query_prefill_layer(ks, vs, ps, q[j:j + 1], k[j:j + 1], v[j:j + 1], pos[j:j + 1],
                                                theta, "bf16", hkv)
        assert np.allclose(o1[0], o_all[j], atol=1e-13)
        ks = np.concatenate([ks, k1.transpose(1, 0, 2)], axis=1)
        vs = np.concatenate([vs, v1.transpose(1, 0, 2)], axis=1)
        ps = np.concatenate([ps, pos[j:j + 1]])


def test_attention_weight_properties():
    rng = np.random.default_rng(12)
    d, hq, hkv, r, n = 8, 4, 2, 30, 5
    q = rng.standard_normal((n, hq, d))
    pos_rows = np.concatenate([rng.permutation(25), 25 + np.arange(5)])
    pos_q = 25 + np.arange(n)
    k = rng.standard_normal((hkv, r, d))
    # constant values -> constant output
    o = orc.attention(q, k, np.full((hkv, r, d), 2.5), pos_rows, pos_q, hkv)
    assert np.allclose(o, 2.5, atol=1e-14)
    # one-hot values expose the weights: they sum to one, vanish where masked
    eye = np.broadcast_to(np.eye(r)[None, :, :], (hkv, r, r))
    w = orc.attention(np.concatenate([q, np.zeros((n, hq, r - d))], axis=2),
                      np.concatenate([k, np.zeros((hkv, r, r - d))], axis=2), eye,
                      pos_rows, pos_q, hkv)
    assert np.allclose(w.sum(axis=2), 1.0, atol=1e-14)
    assert np.all(w[:, :, pos_rows > pos_q.min()][0] == 0.0)
    # identical keys -> plain mean of the visible values
    vals = rng.standard_normal((hkv, r, d))
    o = orc.attention(q, np.ones((hkv, r, d)), vals, pos_rows, pos_q, hkv)
    for j in range(n):
        vis = pos_rows <= pos_q[j]
        for h in range(hq):
            assert np.allclose(o[j, h], vals[h // 2][vis].mean(axis=0), atol=1e-13)


# ---------------------------------------------------------------------------
# new-token prologue: rotation to the token's position, one rounding
# ---------------------------------------------------------------------------

def bf16_nearest_ref(x):
    """Nearest bfloat16 of each fp64 value (ties to even), built from bit patterns.

    bf16 values are the fp32 values whose low 16 bits are zero.  The
    candidates are the three such patterns around fp32(x); the difference of
    x and a nearby candidate is exact in fp64 (Sterbenz), so the nearest one,
    and a tie, are decided exactly; a tie goes to the candidate whose last
    kept bit (bit 16) is 0.  Independent of the oracle's frexp/ldexp rounding.
    """
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    for i, xv in np.ndenumerate(x):
        u = int(np.array([xv], np.float32).view(np.uint32)[0])
        sign, mag = u & 0x80000000, u & 0x7FFF0000
        best, best_d = None, None
        for m in (mag - 0x10000, mag, mag + 0x10000):
            if m < 0:
                continue
            c = float(np.array([sign | m], np.uint32).view(np.float32)[0])
            dist = abs(xv - c)
            if best is None or dist < best_d or (dist == best_d and not (m & 0x10000)):
                best, best_d, best_m = c, dist, m
        out[i] = best
    return out


def _near_bf16_tie(x, tol):
    """True where x lies within tol of a midpoint between two bf16 values."""
    x = np.asarray(x, np.float64)
    u = x.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    lo = u.view(np.float32).astype(np.float64)
    step = np.ldexp(1.0, np.frexp(np.where(lo == 0, 1e-30, lo))[1] - 8)
    mids = np.stack([lo - step / 2, lo + step / 2, lo + 1.5 * step])
    return np.any(np.abs(np.abs(x)[None] - np.abs(mids)) <= tol, axis=0)


@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_prologue_rounds_rotated_queries_and_keys_once(theta):
    # KV_M(q; C_ctx) (CoinRAG page, section 2.3): new tokens are rotated to
    # their positions and their K' is appended to the cache in its storage
    # type; q' and k' are R(P) q and R(P) k rounded once, v is untouched
    gen = torch.Generator().manual_seed(31)
    n, hq, hkv, d = 5, 4, 2, 128
    bf = lambda *s: torch.randn(*s, generator=gen, dtype=torch.float64).to(torch.bfloat16).double().numpy()
    q, k, v = bf(n, hq, d), bf(n, hkv, d), bf(n, hkv, d)
    pos = np.array([0, 3, 77, 1000, 2999])
    qr, kr, vr = orc.prologue(q, k, v, pos, theta, "bf16")
    for got, x in ((qr, q), (kr, k)):
        exact = rope_ref(x, theta, pos[:, None])
        want = bf16_nearest_ref(exact)
        # the matrix exponential is accurate to about 1e-13 per radian; an
        # element that close to a rounding tie may go either way
        tol = 1e-13 * (1.0 + pos.max()) * np.abs(x).max()
        ok = (got == want) | (_near_bf16_tie(exact, tol) & (np.abs(got - exact) <= np.abs(want - exact) + tol))
        assert ok.all(), f"{int((~ok).sum())} elements are not the once-rounded rotation"
        assert np.array_equal(got[0], x[0])            # P = 0: R(0) = I, a copy
    assert np.array_equal(vr, v) and np.array_equal(np.signbit(vr), np.signbit(v))
    # the same with fp32 storage: fp32-representable and within half an fp32 ulp
    qf, kf, _ = orc.prologue(q, k, v, pos, theta, "f32")
    for got, x in ((qf, q), (kf, k)):
        exact = rope_ref(x, theta, pos[:, None])
        assert np.array_equal(got, got.astype(np.float32).astype(np.float64))
        half_ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64) / 2
        assert np.all(np.abs(got - exact) <= half_ulp + 1e-13 * (1.0 + pos.max()) * np.abs(x).max())
