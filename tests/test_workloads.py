"""CPU checks of the seeded input generators and the work accounting."""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layout_hash(wl):
    h = hashlib.sha256()
    for r in wl.requests:
        h.update(np.ascontiguousarray(r.spans).tobytes())
        h.update(np.int64(r.n_new).tobytes())
        if r.new_pos is not None:
            h.update(np.ascontiguousarray(r.new_pos).tobytes())
    h.update(wl.pool.page_ids.tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("name", W.FULL_SIZE + W.REDUCED)
def test_layouts_are_deterministic(name):
    assert _layout_hash(W.get(name)) == _layout_hash(W.get(name))


def test_kv_bytes_against_the_pages():
    with open(os.path.join(GOLDEN, "kv_bytes.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        b = W.kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["elem_bytes"]) * c["tokens"]
        assert abs(b - c["approx_bytes"]) <= c["rel_tol"] * c["approx_bytes"], c["note"]


def test_tiny_config_shape():
    wl = W.get("tiny_f32")
    m = wl.model
    assert (m.layers, m.q_heads, m.kv_heads, m.head_dim, m.theta, m.dtype) == (1, 2, 1, 64, 1e4, "f32")
    (r,) = wl.requests
    assert r.n_new == 8 and len(r.spans) == 7
    assert tuple(r.spans[0]) == (4, 0, 7, 0)                 # prompt cache first, at 0
    for c, s, e, t in r.spans[1:]:
        assert 0 <= c < 4 and 4 <= e - s + 1 <= 16 and 0 <= s and e < 64 and t == W.TARGET_AUTO


def test_nugget_spans_follow_the_recipe():
    wl = W.get("coinrag_b32")
    assert wl.batch == 32
    for r in wl.requests:
        body = r.spans[1:]
        assert len(body) == 64
        assert len(set(body[:, 0].tolist())) <= 20
        lens = body[:, 2] - body[:, 1] + 1
        assert lens.min() >= 3 and lens.max() <= 48
        for c in set(body[:, 0].tolist()):
            cov = np.zeros(512, int)
            for _, s, e, _ in body[body[:, 0] == c]:
                cov[s:e + 1] += 1
            assert cov.max() <= 1                               # no overlap inside a chunk
    lens = np.concatenate([r.spans[1:, 2] - r.spans[1:, 1] + 1 for r in wl.requests])
    assert 12 < lens.mean() < 17                                # geometric mean 15, clipped


def test_interleaved_layout_recipe():
    wl = W.get("sempic_b8")
    for r in wl.requests:
        assert len(r.spans) == 8 and len(set(r.spans[:, 0].tolist())) == 8
        pos = np.concatenate([np.arange(t, t + e - s + 1) for _, s, e, t in r.spans] + [r.new_pos])
        assert np.array_equal(np.sort(pos), np.arange(pos.size))   # one dense sequence
        assert r.n_new - 128 >= 7 * 64 and r.n_new - 128 <= 7 * 256
        assert r.new_pos[-1] == pos.size - 1                        # query last


def test_visible_pairs_brute_force():
    for name in ("sempic_small", "turborag_small", "tiny_f32"):
        wl = W.get(name)
        want = 0
        for r in wl.requests:
            if r.new_pos is None:
                n0 = r.prefix_rows
                rows = np.arange(n0 + r.n_new)
                q = n0 + np.arange(r.n_new)
            else:
                rows = np.concatenate([np.arange(t, t + e - s + 1) for _, s, e, t in r.spans] + [r.new_pos])
                q = r.new_pos
            want += sum(int((rows <= p).sum()) for p in q)
        assert W.visible_pairs(wl) == want


def test_pool_fill_and_readback_on_cpu():
    wl = W.get("tiny_f32")
    ks, vs = W.channel_scales(wl, "cpu")
    pool = W.fill_pool(wl, W.alloc_pool(wl, "cpu"), ks, vs)
    k, v = W.chunk_kv(wl, pool, 2)
    assert k.shape == (1, 1, 64, 64) and v.shape == (1, 1, 64, 64)
    # token t of chunk c lives in page page_ids[ptr[c] + t // P] at slot t % P
    p = wl.pool
    t = 37
    page = int(p.page_ids[p.chunk_page_ptr[2] + t // p.page_tokens])
    assert torch.equal(k[0, 0, t], pool[page, 0, 0, 0, t % p.page_tokens].double())
    assert torch.equal(v[0, 0, t], pool[page, 0, 1, 0, t % p.page_tokens].double())
    pool2 = W.fill_pool(wl, W.alloc_pool(wl, "cpu"), ks, vs)
    assert torch.equal(pool, pool2)
