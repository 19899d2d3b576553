"""CPU checks of the C ABI: exports, host validation, host planning.

No GPU is touched: pool registration copies host tables only, and
PIC_ASSEMBLE_DRY_RUN plans on the host.  Planning results (targets, deltas,
rows, new-token positions) are integers and must equal the oracle's exactly.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads as W
from oracle import pic_oracle as orc
from position_independent_kv_pic_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_POOL = 1 << 40          # aligned fake device address; registration never dereferences it


def _header_functions():
    text = open(os.path.join(ROOT, "include", "pic.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pic_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.lib()
    declared = _header_functions()
    assert declared, "no declarations parsed"
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(B.EXPORTED)
    assert lib.pic_version().decode().startswith("libpic")


def _model(wl):
    m = wl.model
    return B.model_struct(m.layers, m.q_heads, m.kv_heads, m.head_dim, m.theta, m.dtype, wl.keys)


def _pool(wl, base=FAKE_POOL):
    p = wl.pool
    return B.Pool(_model(wl), base, p.n_pages * W.page_bytes(wl.model, p.page_tokens), p.page_tokens,
                  p.n_pages, p.chunk_len, p.chunk_page_ptr, p.page_ids, p.chunk_orig)


def _dry(plan, wl, capacity=2 ** 40):
    plan.assemble(wl.span_ptr(), wl.spans_flat(), wl.new_ptr(), wl.new_pos_flat(), None, None,
                  capacity, B.DRY_RUN)


@pytest.mark.parametrize("name", W.FULL_SIZE + W.REDUCED + W.REDUCED_NEXT +
                         ("turborag_b16_unrot", "turborag_b16_composite"))
def test_host_plan_matches_oracle(name):
    wl = W.get(name)
    pool = _pool(wl)
    plan = B.Plan(pool)
    _dry(plan, wl)
    s = plan.summary()
    assert s["prefix_rows"] == wl.prefix_rows_total and s["new_rows"] == wl.n_new_total
    assert s["rows"] == wl.rows_total and s["batch"] == wl.batch
    tgt, dlt, first = plan.spans()
    rb, pr, fp = plan.requests()
    npos, nrow = plan.new_tokens()
    i = u = row = 0
    for b, r in enumerate(wl.requests):
        planned = orc.plan_spans([tuple(x) for x in r.spans], wl.pool.chunk_orig)
        assert rb[b] == row and pr[b] == sum(p.length for p in planned)
        acc = row
        for p in planned:
            assert (tgt[i], dlt[i], first[i]) == (p.target, p.delta, acc)
            acc += p.length
            i += 1
        pos = orc.new_token_positions(planned, r.n_new, r.new_pos)
        assert np.array_equal(npos[u:u + r.n_new], pos)
        assert np.array_equal(nrow[u:u + r.n_new], acc + np.arange(r.n_new))
        if r.n_new:
            assert fp[b] == pos[0]
        u += r.n_new
        row = acc + r.n_new
    plan.release()
    pool.release()


def test_original_targets_and_new_positions_after_the_whole_prefix():
    # composite positions with non-zero chunk bases: each span stays where it
    # was encoded (delta 0) and the new tokens follow the whole prefix
    wl = W.get("tiny_f32")
    p = wl.pool
    orig = np.zeros(p.n_chunks, np.int32)
    orig[:3] = [100, 0, 7]
    pool = B.Pool(_model(wl), FAKE_POOL, p.n_pages * W.page_bytes(wl.model, p.page_tokens), p.page_tokens,
                  p.n_pages, p.chunk_len, p.chunk_page_ptr, p.page_ids, orig)
    plan = B.Plan(pool)
    spans = np.array([[0, 2, 5, B.TARGET_ORIGINAL], [2, 0, 9, B.TARGET_ORIGINAL], [1, 3, 4, B.TARGET_AUTO]],
                     np.int32)
    plan.assemble(np.array([0, 3]), spans, np.array([0, 4]), None, None, None, 2 ** 40, B.DRY_RUN)
    tgt, dlt, _ = plan.spans()
    want = orc.plan_spans([tuple(int(x) for x in r) for r in spans], orig)
    assert tgt.tolist() == [sp.target for sp in want] == [102, 7, 17]
    assert dlt.tolist() == [sp.delta for sp in want] == [0, 0, 14]
    npos, _ = plan.new_tokens()
    assert npos.tolist() == orc.new_token_positions(want, 4).tolist() == [106, 107, 108, 109]
    plan.release()
    pool.release()


@pytest.mark.parametrize("name", ["turborag_small", "sempic_small"])
def test_decode_reserve_row_layout(name):
    # each request owns prefix + n_new + reserve rows; the plan keeps the
    # request's positions and rows otherwise unchanged
    wl = W.get(name)
    pool = _pool(wl)
    plan = B.Plan(pool)
    reserve = 5
    plan.set_decode_rows(reserve)
    _dry(plan, wl)
    s = plan.summary()
    assert s["rows"] == wl.rows_total + reserve * wl.batch
    rb, pr, _ = plan.requests()
    acc = 0
    for b, r in enumerate(wl.requests):
        assert rb[b] == acc and pr[b] == r.prefix_rows
        acc += r.prefix_rows + r.n_new + reserve
    # a capacity that does not cover the reserve is rejected
    with pytest.raises(B.PicError) as ei:
        plan.assemble(wl.span_ptr(), wl.spans_flat(), wl.new_ptr(), wl.new_pos_flat(), None, None,
                      wl.rows_total, B.DRY_RUN)
    assert ei.value.name == "PIC_ERANGE"
    assert _err(lambda: plan.set_decode_rows(-1)) == "PIC_EINVAL"
    # decoding needs an assembled batch (a dry run has none)
    assert _err(lambda: plan.decode_layer(0, 0, FAKE_POOL, FAKE_POOL, FAKE_POOL, FAKE_POOL)) == "PIC_ESTATE"
    plan.release()
    pool.release()


def test_deferred_gather_flags_and_states():
    wl = W.get("turborag_small")
    pool = _pool(wl)
    plan = B.Plan(pool)
    sp, spans, npt = wl.span_ptr(), wl.spans_flat(), wl.new_ptr()
    # PLAN_ONLY and DEFER_GATHER exclude each other
    assert _err(lambda: plan.assemble(sp, spans, npt, None, None, None, 2 ** 40,
                                      B.DRY_RUN | B.PLAN_ONLY | B.DEFER_GATHER)) == "PIC_EINVAL"
    # no planes yet: nothing to gather into
    assert _err(lambda: plan.gather_layers(0, 1)) == "PIC_ESTATE"
    _dry(plan, wl)
    assert _err(lambda: plan.gather_layers(0, 1)) == "PIC_ESTATE"
    plan.release()
    pool.release()


@pytest.mark.parametrize("name", ("turborag_small", "tiny_f32"))
def test_query_rotation_flag_is_refused(name):
    """Scoring against queries rotated back by a span's delta skips the
    storage rounding of the re-rotated keys (it cannot reproduce the
    assembled cache), so the option is refused, with or without PLAN_ONLY."""
    wl = W.get(name)
    pool = _pool(wl)
    plan = B.Plan(pool)
    sp, spans, npt, npos = wl.span_ptr(), wl.spans_flat(), wl.new_ptr(), wl.new_pos_flat()
    for flags in (B.DRY_RUN | B.QUERY_ROTATION, B.DRY_RUN | B.PLAN_ONLY | B.QUERY_ROTATION):
        assert _err(lambda: plan.assemble(sp, spans, npt, npos, None, None, 2 ** 40, flags)) == "PIC_EUNSUPPORTED"
    plan.assemble(sp, spans, npt, npos, None, None, 2 ** 40, B.DRY_RUN | B.PLAN_ONLY)
    assert plan.summary()["fused_query_rotation"] == 0
    plan.release()
    pool.release()


def test_values_in_pool_flag():
    wl = W.get("turborag_small")
    pool = _pool(wl)
    plan = B.Plan(pool)
    sp, spans, npt, npos = wl.span_ptr(), wl.spans_flat(), wl.new_ptr(), wl.new_pos_flat()
    # a gathered batch only: nothing to leave in the pool when nothing is gathered
    assert _err(lambda: plan.assemble(sp, spans, npt, npos, None, None, 2 ** 40,
                                      B.DRY_RUN | B.PLAN_ONLY | B.VALUES_IN_POOL)) == "PIC_EINVAL"
    plan.assemble(sp, spans, npt, npos, None, None, 2 ** 40, B.DRY_RUN | B.VALUES_IN_POOL)
    assert plan.summary()["values_in_pool"] == 1
    plan.assemble(sp, spans, npt, npos, None, None, 2 ** 40, B.DRY_RUN)
    assert plan.summary()["values_in_pool"] == 0
    plan.release()
    pool.release()
    # implemented where the bf16 attention reads the pool (head_dim 128)
    wl = W.get("tiny_f32")
    pool = _pool(wl)
    plan = B.Plan(pool)
    assert _err(lambda: plan.assemble(wl.span_ptr(), wl.spans_flat(), wl.new_ptr(), wl.new_pos_flat(), None,
                                      None, 2 ** 40, B.DRY_RUN | B.VALUES_IN_POOL)) == "PIC_EUNSUPPORTED"
    plan.release()
    pool.release()


def test_key_storage_is_validated():
    wl = W.get("tiny_f32")
    p = wl.pool
    m = _model(wl)
    m.key_storage = 7
    with pytest.raises(B.PicError) as ei:
        B.Pool(m, FAKE_POOL, p.n_pages * W.page_bytes(wl.model, p.page_tokens), p.page_tokens, p.n_pages,
               p.chunk_len, p.chunk_page_ptr, p.page_ids)
    assert ei.value.name == "PIC_EINVAL"


def _err(fn):
    with pytest.raises(B.PicError) as ei:
        fn()
    return ei.value.name


def test_pool_registration_errors():
    wl = W.get("tiny_f32")
    p = wl.pool
    m = _model(wl)
    pb = p.n_pages * W.page_bytes(wl.model, p.page_tokens)
    ok = dict(pool=FAKE_POOL, pool_bytes=pb, page_tokens=p.page_tokens, n_pages=p.n_pages,
              chunk_len=p.chunk_len, chunk_page_ptr=p.chunk_page_ptr, page_ids=p.page_ids)

    def reg(**kw):
        a = dict(ok)
        a.update(kw)
        return lambda: B.Pool(kw.get("model", m), a["pool"], a["pool_bytes"], a["page_tokens"],
                              a["n_pages"], a["chunk_len"], a["chunk_page_ptr"], a["page_ids"])

    assert _err(reg(pool=0)) == "PIC_EINVAL"
    assert _err(reg(pool=FAKE_POOL + 8)) == "PIC_EALIGN"
    assert _err(reg(page_tokens=12)) == "PIC_EINVAL"
    assert _err(reg(pool_bytes=pb - 1)) == "PIC_ERANGE"
    bad_ids = p.page_ids.copy()
    bad_ids[3] = p.n_pages
    assert _err(reg(page_ids=bad_ids)) == "PIC_ERANGE"
    short = p.chunk_page_ptr.copy()
    short[1:] -= 1
    short[0] = 0
    assert _err(reg(chunk_page_ptr=short)) == "PIC_EINVAL"
    bad_len = p.chunk_len.copy()
    bad_len[0] = -1
    assert _err(reg(chunk_len=bad_len)) == "PIC_EINVAL"
    for bad in (B.model_struct(1, 3, 2, 64, 1e4, "f32"), B.model_struct(1, 2, 1, 72, 1e4, "f32"),
                B.model_struct(1, 2, 1, 64, 0.5, "f32"), B.model_struct(0, 2, 1, 64, 1e4, "f32")):
        assert _err(lambda: B.Pool(bad, FAKE_POOL, pb, p.page_tokens, p.n_pages, p.chunk_len,
                                   p.chunk_page_ptr, p.page_ids)) == "PIC_EINVAL"


def test_assemble_validation_errors_enqueue_nothing():
    wl = W.get("tiny_f32")
    pool = _pool(wl)
    plan = B.Plan(pool)
    sp = wl.span_ptr()
    np_ = wl.new_ptr()
    good = wl.spans_flat()

    def dry(spans=good, span_ptr=sp, new_ptr=np_, new_pos=None, cap=2 ** 40):
        return lambda: plan.assemble(span_ptr, spans, new_ptr, new_pos, None, None, cap, B.DRY_RUN)

    def mod(i, col, val):
        t = good.copy()
        t[i, col] = val
        return t

    assert _err(dry(mod(1, 0, 99))) == "PIC_ERANGE"          # chunk id out of range
    assert _err(dry(mod(1, 0, -1))) == "PIC_ERANGE"
    assert _err(dry(mod(1, 1, good[1, 2] + 1))) == "PIC_ERANGE"   # s > e
    assert _err(dry(mod(1, 2, 64))) == "PIC_ERANGE"          # e >= len
    assert _err(dry(mod(1, 1, -3))) == "PIC_ERANGE"          # s < 0
    assert _err(dry(mod(2, 3, -7))) == "PIC_EINVAL"          # bad target
    assert _err(dry(mod(2, 3, 2 ** 31 - 2))) == "PIC_ERANGE"  # positions overflow
    with pytest.raises(ValueError):                           # table shorter than its CSR
        dry(span_ptr=np.array([0, 8]))()
    assert _err(dry(span_ptr=np.array([1, 7]))) == "PIC_EINVAL"
    assert _err(dry(new_ptr=np.array([0, -1]))) == "PIC_EINVAL"
    assert _err(dry(new_pos=np.array([70, 71, 72, 72, 73, 74, 75, 76]))) == "PIC_EINVAL"
    assert _err(dry(new_pos=np.array([-1, 71, 72, 73, 74, 75, 76, 77]))) == "PIC_EINVAL"
    assert _err(dry(cap=wl.rows_total - 1)) == "PIC_ERANGE"
    dry(cap=wl.rows_total)()                                  # exactly enough
    # non-dry calls need device buffers, checked before any device work
    assert _err(lambda: plan.assemble(sp, good, np_, None, None, None, 100, 0)) == "PIC_EINVAL"
    assert _err(lambda: plan.assemble(sp, good, np_, None, FAKE_POOL + 4, FAKE_POOL, 100, 0)) == "PIC_EALIGN"
    assert _err(lambda: plan.assemble(sp, good, np_, None, None, None, 100, 64)) == "PIC_EINVAL"
    plan.release()
    pool.release()


def test_query_prefill_state_errors():
    wl = W.get("tiny_f32")
    pool = _pool(wl)
    plan = B.Plan(pool)
    assert _err(lambda: plan.query_prefill(0, FAKE_POOL, FAKE_POOL, FAKE_POOL, FAKE_POOL)) == "PIC_ESTATE"
    _dry(plan, wl)
    assert _err(lambda: plan.query_prefill(0, FAKE_POOL, FAKE_POOL, FAKE_POOL, FAKE_POOL)) == "PIC_ESTATE"
    # releasing a pool that still has a plan is refused
    assert _err(pool.release) == "PIC_ESTATE"
    plan.release()
    pool.release()


def test_empty_and_degenerate_batches_plan():
    wl = W.get("tiny_f32")
    pool = _pool(wl)
    plan = B.Plan(pool)
    plan.assemble(np.array([0]), np.zeros((0, 4)), np.array([0]), None, None, None, 0, B.DRY_RUN)
    assert plan.summary()["rows"] == 0
    # requests with no spans (plain causal prefill) and with no new tokens
    plan.assemble(np.array([0, 0, 1]), np.array([[2, 0, 63, B.TARGET_AUTO]]), np.array([0, 5, 5]),
                  None, None, None, 100, B.DRY_RUN)
    npos, nrow = plan.new_tokens()
    assert npos.tolist() == [0, 1, 2, 3, 4] and nrow.tolist() == [0, 1, 2, 3, 4]
    rb, pr, _ = plan.requests()
    assert rb.tolist() == [0, 5] and pr.tolist() == [0, 64]
    plan.release()
    pool.release()


@pytest.mark.parametrize("name", tuple(n for n in W.FULL_SIZE + W.REDUCED + W.REDUCED_NEXT
                                       if n != "tiny_f32") + ("turborag_b16_composite",))
def test_attention_work_covers_every_visible_row_once(name):
    """The attention work list, checked against the visibility rule (a query
    at position P sees every row at a position <= P): for each column block,
    the tiles its items run (range minus skipped gap) hold every row that
    any of its queries can see, no tile twice; a range without a row split
    ends at the last such tile.  Both launch orders (over item pairs and
    over single items) cover every unit once and give each XCD a contiguous
    range of units, longest first."""
    wl = W.get(name)
    pool = _pool(wl)
    plan = B.Plan(pool)
    _dry(plan, wl)
    items, order = plan.attention_work()
    G = wl.model.q_heads // wl.model.kv_heads
    target, _, first_row = plan.spans()
    new_pos, new_row = plan.new_tokens()
    row_base, prefix_rows, _ = plan.requests()
    span_ptr, spans_flat = wl.span_ptr(), wl.spans_flat().reshape(-1, 4)
    new_ptr = wl.new_ptr()
    # positions of every request's rows, prefix then new tokens
    tile_min = []
    for b in range(wl.batch):
        n_new = int(new_ptr[b + 1] - new_ptr[b])
        pos = np.empty(int(prefix_rows[b]) + n_new, np.int64)
        for i in range(span_ptr[b], span_ptr[b + 1]):
            s, e = int(spans_flat[i, 1]), int(spans_flat[i, 2])
            r0 = int(first_row[i] - row_base[b])
            pos[r0:r0 + e - s + 1] = target[i] + np.arange(e - s + 1)
        pos[prefix_rows[b]:] = new_pos[new_ptr[b]:new_ptr[b + 1]]
        t = (len(pos) + 63) // 64
        padded = np.full(t * 64, np.iinfo(np.int64).max)
        padded[:len(pos)] = pos
        tile_min.append(padded.reshape(t, 64).min(axis=1))
    blocks = {}
    for i, it in enumerate(items):
        blocks.setdefault((int(it[0]), int(it[1]), int(it[2])), []).append(i)
    last_needed = {}   # item of an unsplit column block -> last tile it must run
    for (b, h, c0), idx in blocks.items():
        n_new = int(new_ptr[b + 1] - new_ptr[b])
        if c0 >= n_new * G:
            continue  # the empty partner of an odd count of column blocks
        last_tok = (min(c0 + 128, n_new * G) - 1) // G
        qmax = new_pos[new_ptr[b] + last_tok]
        needed = set(np.nonzero(tile_min[b] <= qmax)[0].tolist())
        run = []
        for i in idx:
            it = items[i]
            run += [t for t in range(it[3], it[4]) if not (it[5] <= t < it[6])]
        assert len(run) == len(set(run)), (name, b, h, c0)
        assert needed <= set(run), (name, b, h, c0, sorted(needed - set(run))[:5])
        if len(idx) == 1 and needed:
            last_needed[idx[0]] = max(needed)
    # two unsplit column blocks in one workgroup run one range: it ends at the
    # last tile that either of them needs
    for p in range(0, len(items) - 1, 2):
        if p in last_needed or p + 1 in last_needed:
            want = max(last_needed.get(p, -1), last_needed.get(p + 1, -1))
            if items[p][4] == items[p + 1][4] and items[p][3] == items[p + 1][3]:
                assert items[p][4] - 1 == want, (name, p)
    # launch orders: over item pairs (paired kernel), over single items
    _, item_order = plan.attention_work(single_items=True)
    for per_wg, seq in ((2, order), (1, item_order)):
        n_units = (len(items) + per_wg - 1) // per_wg
        assert len(seq) % 8 == 0 and len(seq) >= n_units
        assert sorted(seq[seq >= 0].tolist()) == list(range(n_units))
        steps = [max(int(it[4] - it[3] - (it[6] - it[5])) for it in items[per_wg * p:per_wg * (p + 1)])
                 for p in range(n_units)]
        for x in range(8):
            col = seq[x::8]
            live = col[col >= 0]
            assert (col[len(live):] == -1).all()
            if len(live):
                assert sorted(live.tolist()) == list(range(min(live), max(live) + 1))
                # longest first, in bands of a tenth of the longest (a unit
                # costs its steps plus 2 of set-up); the work list's order
                # inside a band
                c = np.array([steps[p] + 2 for p in live])
                band = (c.max() - c) * 10 // c.max()
                assert (np.diff(band) >= 0).all()
                assert all(live[i] < live[i + 1] for i in range(len(live) - 1) if band[i] == band[i + 1])
    plan.release()
    pool.release()


@pytest.mark.parametrize("prefix_rows", [2816, 2880 - 64 + 32, 1000, 64 * 16 - 64])
def test_row_splits_keep_the_minimum_tiles_per_part(prefix_rows):
    """A batch too small to fill the chip has its rows split, into parts of
    at least 3 tiles for the longest request, and into an even number of
    parts (two splits of a column block share a workgroup).  45 tiles must
    not round an odd 15 up to 16 parts of 2-3 tiles."""
    d, hq, hkv, L = 128, 28, 4, 2
    model = B.model_struct(L, hq, hkv, d, 1e6, "bf16")
    pt = 16
    pages = (prefix_rows + pt - 1) // pt
    pool = B.Pool(model, FAKE_POOL, pages * L * 2 * hkv * pt * d * 2, pt, pages, [prefix_rows], [0, pages],
                  list(range(pages)))
    plan = B.Plan(pool)
    plan.assemble([0, 1], [[0, 0, prefix_rows - 1, B.TARGET_AUTO]], [0, 64], None, None, None, 2 ** 40, B.DRY_RUN)
    items, _ = plan.attention_work()
    tiles = (prefix_rows + 64 + 63) // 64
    parts = {}
    for it in items:
        parts.setdefault((int(it[1]), int(it[2])), []).append(int(it[4] - it[3]))
    for key, lens in parts.items():
        if len(lens) > 1:
            assert len(lens) % 2 == 0, (key, lens)
            assert min(lens) >= 3, (prefix_rows, tiles, key, lens)
        assert sum(lens) == tiles
    plan.release()
    pool.release()


def test_hot_set_fronts_only_a_host_pool():
    """A hot set caches a pool in pinned host memory: on a device pool, with
    no pool, or with no slots the call is refused and nothing is created."""
    wl = W.get("turborag_small")
    pool = _pool(wl)
    assert _err(lambda: B.Cache(pool, 16)) == "PIC_EINVAL"
    h = ctypes.c_void_p()
    assert B.lib().pic_cache_create(None, 16, ctypes.byref(h)) == -1 and not h.value
    assert B.lib().pic_cache_create(pool.handle, 16, None) == -1
    assert B.lib().pic_cache_get_stats(None, None) == -1
    assert B.lib().pic_cache_release(None) == -1
    # the pool has no hot set, so it releases
    pool.release()
