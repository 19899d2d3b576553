"""GPU parity: libpic's HIP path against the fp64 CPU oracle, through the C ABI.

Reduced workloads (same structure, fewer layers/requests) are compared
element by element; the full-size workloads run exactly as the benchmark
launches them (assemble, then every layer's prefill) and are checked on
requests {0, last}, layers {0, L/2, L-1} and a spread of query tokens.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import pic_oracle as orc
from position_independent_kv_pic_amd import VARIANT_FUSED, VARIANT_MATERIALIZED
from workloads.device import open_workload

import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _say(*a):
    print(*a, flush=True)


def _np(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def run_prefill(dw, layers, variant):
    """Prefill the given layers; returns {layer: (q, k, v, out)}."""
    res = {}
    for l in layers:
        q, k, v = dw.layer_inputs(l)
        out = dw.session.prefill_layer(l, q, k, v, variant=variant)
        res[l] = (q, k, v, out)
    torch.cuda.synchronize()
    return res


def check_request(dw, b, layers, results, token_subset=None, check_tail=True, check_prefix=True):
    """Compare request b's assembled rows, new rows and outputs on `layers`
    (the assembled prefix rows only with check_prefix: a plan-only batch
    gathers nothing)."""
    wl = dw.wl
    m = wl.model
    sess = dw.session
    rb, pr, _ = sess.plan.requests()
    base, npre = int(rb[b]), int(pr[b])
    r = wl.requests[b]
    nb = int(wl.new_ptr()[b])
    kpre, vpre, ppre = P.request_prefix(wl, dw.pool, b, layers)
    pos_new = P.request_positions(wl, b)
    stats = {}
    for li, l in enumerate(layers):
        mx, nx = None, None
        if check_prefix:
            gk = _np(sess.asm_k[l, :, base:base + npre])
            gv = _np(sess.asm_v[l, :, base:base + npre])
            assert np.array_equal(gv, vpre[li]), f"values differ (request {b}, layer {l})"
            planned = orc.plan_spans([tuple(int(x) for x in s) for s in r.spans], wl.pool.chunk_orig)
            zero = (np.concatenate([np.full(p.length, p.delta == 0) for p in planned]) if planned
                    else np.zeros(0, bool))
            mx, nx = P.compare_keys(gk, kpre[li], m.dtype, exact_mask=zero[None, :, None])
        q, k, v, out = results[l]
        sl = slice(nb, nb + r.n_new)
        qn, kn, vn = _np(q[sl]), _np(k[sl]), _np(v[sl])
        o_ref, k_rot, v_ref, q_rot = orc.query_prefill_layer(kpre[li], vpre[li], ppre, qn, kn, vn, pos_new,
                                                             m.theta, m.dtype, m.kv_heads,
                                                             query_subset=token_subset)
        if check_tail and r.n_new:
            gkt = _np(sess.asm_k[l, :, base + npre:base + npre + r.n_new]).transpose(1, 0, 2)
            gvt = _np(sess.asm_v[l, :, base + npre:base + npre + r.n_new]).transpose(1, 0, 2)
            assert np.array_equal(gvt, v_ref), "new values not appended exactly"
            P.compare_keys(gkt, k_rot, m.dtype, exact_mask=(pos_new == 0)[:, None, None])
        got = _np(out[sl])
        if token_subset is not None:
            got = got[token_subset]
        sel = np.arange(r.n_new) if token_subset is None else np.asarray(token_subset)
        ast = P.attn_check(got, o_ref, m.dtype, q_rot[sel],
                           np.concatenate([kpre[li], k_rot.transpose(1, 0, 2)], axis=1),
                           np.concatenate([vpre[li], v_ref.transpose(1, 0, 2)], axis=1),
                           np.concatenate([ppre, pos_new]), pos_new[sel], m.kv_heads)
        stats[l] = dict(key_max=mx, key_not_exact=nx, attn_max_abs=ast["max_abs"], attn_rel_l2=ast["rel_l2"],
                        attn_ratio=ast["ratio"], attn_ratio_without_p=ast["ratio_without_p"])
        assert P.attn_ok(ast, m.dtype), f"attention off (request {b}, layer {l}): {ast}"
    return stats


def check_fused_plan_only(dw, layers, res_m):
    """Variant F after a plan-only assembly (nothing gathered; keys rotated
    on load): variant M's bits."""
    dw.assemble(plan_only=True)
    res_f = run_prefill(dw, layers, VARIANT_FUSED)
    for l in layers:
        assert torch.equal(res_m[l][3], res_f[l][3]), f"plan-only fused differs on layer {l}"


def check_query_rotation_refused(dw):
    """Scoring against queries rotated back by the span's delta is retired:
    the assemble refuses the flag and changes nothing."""
    from position_independent_kv_pic_amd import PLAN_ONLY, QUERY_ROTATION, PicError
    wl, sess = dw.wl, dw.session
    with pytest.raises(PicError, match="PIC_EUNSUPPORTED"):
        sess.plan.assemble(wl.span_ptr(), wl.spans_flat(), wl.new_ptr(), wl.new_pos_flat(), sess.asm_k,
                           sess.asm_v, sess.capacity, PLAN_ONLY | QUERY_ROTATION, torch.cuda.current_stream())


def check_values_in_pool(dw, layers, res_m):
    """Variant M after an assembly that gathers keys only (values read in
    the pool pages by attention): bit for bit what the full gather gives."""
    summ = dw.assemble(values_in_pool=True)
    assert summ["values_in_pool"] == 1
    res = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    for l in layers:
        assert torch.equal(res_m[l][3], res[l][3]), f"values in the pool differ on layer {l}"


def test_tiny_fp32_config_end_to_end():
    wl = W.get("tiny_f32")
    _say("case tiny_f32")
    dw = open_workload(wl)
    dw.assemble()
    res = run_prefill(dw, [0], VARIANT_MATERIALIZED)
    st = check_request(dw, 0, [0], res)
    _say("tiny_f32", st)
    dw.close()


@pytest.mark.parametrize("name", W.REDUCED + W.REDUCED_NEXT)
def test_reduced_workloads_every_element(name):
    wl = W.get(name)
    _say(f"case reduced {name}")
    dw = open_workload(wl)
    dw.assemble()
    layers = list(range(wl.model.layers))
    res_m = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    for b in range(wl.batch):
        st = check_request(dw, b, layers, res_m)
        _say(name, b, st)
    # repeated launches give identical bits (the split merge does not depend
    # on which split of a group finishes last)
    res_m2 = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    for l in layers:
        assert torch.equal(res_m[l][3], res_m2[l][3]), f"layer {l} not reproducible"
    # the fused variant reads the pool directly and must give identical bits
    res_f = run_prefill(dw, layers, VARIANT_FUSED)
    for l in layers:
        assert torch.equal(res_m[l][3], res_f[l][3]), f"fused != materialised on layer {l}"
    # keys gathered, values read in the pool: the same bits
    check_values_in_pool(dw, layers, res_m)
    dw.assemble()
    # and it also works from a plan-only assembly
    check_fused_plan_only(dw, layers, res_m)
    dw.close()
    del dw
    torch.cuda.empty_cache()


DECODE_STEPS = 3
def run_decode(dw, layers, steps, variant):
    """Decode `steps` tokens per request on the given layers, step by step;
    returns {layer: [(q, k, v, out) per step]}."""
    res = {l: [] for l in layers}
    for st in range(steps):
        for l in layers:
            q, k, v = dw.decode_inputs(l, st)
            out = dw.session.decode_layer(l, st, q, k, v, variant=variant)
            res[l].append((q, k, v, out))
    torch.cuda.synchronize()
    return res


def check_decode(dw, b, layers, prefill, decoded):
    """Request b after its prefill: every decoded token's output, and the rows
    it appended, against the oracle over the rows so far."""
    wl = dw.wl
    m = wl.model
    sess = dw.session
    rb, pr, _ = sess.plan.requests()
    base, npre = int(rb[b]), int(pr[b])
    r = wl.requests[b]
    nb = int(wl.new_ptr()[b])
    kpre, vpre, ppre = P.request_prefix(wl, dw.pool, b, layers)
    pos_new = P.request_positions(wl, b)
    last = int(max(ppre.max(initial=-1), pos_new.max(initial=-1)))
    worst = dict(attn_max_abs=0.0, attn_rel_l2=0.0, attn_ratio=0.0)
    for li, l in enumerate(layers):
        q, k, v, _ = prefill[l]
        sl = slice(nb, nb + r.n_new)
        _, kr, vr = orc.prologue(_np(q[sl]), _np(k[sl]), _np(v[sl]), pos_new, m.theta, m.dtype)
        ks = np.concatenate([kpre[li], kr.transpose(1, 0, 2)], axis=1)
        vs = np.concatenate([vpre[li], vr.transpose(1, 0, 2)], axis=1)
        ps = np.concatenate([ppre, pos_new])
        for st, (qd, kd, vd, od) in enumerate(decoded[l]):
            p_tok = np.array([last + 1 + st])
            o_ref, k1, v1, q1 = orc.query_prefill_layer(ks, vs, ps, _np(qd[b:b + 1]), _np(kd[b:b + 1]),
                                                       _np(vd[b:b + 1]), p_tok, m.theta, m.dtype, m.kv_heads)
            row = base + npre + r.n_new + st
            gk = _np(sess.asm_k[l, :, row:row + 1]).transpose(1, 0, 2)
            gv = _np(sess.asm_v[l, :, row:row + 1]).transpose(1, 0, 2)
            assert np.array_equal(gv, v1), f"decode value row differs (request {b}, layer {l}, step {st})"
            P.compare_keys(gk, k1, m.dtype, exact_mask=(p_tok == 0)[:, None, None])
            ast = P.attn_check(_np(od[b:b + 1]), o_ref, m.dtype, q1,
                               np.concatenate([ks, k1.transpose(1, 0, 2)], axis=1),
                               np.concatenate([vs, v1.transpose(1, 0, 2)], axis=1),
                               np.concatenate([ps, p_tok]), p_tok, m.kv_heads)
            worst["attn_max_abs"] = max(worst["attn_max_abs"], ast["max_abs"])
            worst["attn_rel_l2"] = max(worst["attn_rel_l2"], ast["rel_l2"])
            worst["attn_ratio"] = max(worst["attn_ratio"], ast["ratio"])
            assert P.attn_ok(ast, m.dtype), f"decode attention off (request {b}, layer {l}, step {st}): {ast}"
            ks = np.concatenate([ks, k1.transpose(1, 0, 2)], axis=1)
            vs = np.concatenate([vs, v1.transpose(1, 0, 2)], axis=1)
            ps = np.concatenate([ps, p_tok])
    return worst


@pytest.mark.parametrize("name", ["turborag_small", "coinrag_small", "sempic_small", "long_small",
                                  "turborag_small_unrot"])
def test_decode_after_prefill_reduced(name):
    wl = W.get(name)
    _say(f"case decode {name}")
    dw = open_workload(wl)
    dw.session.set_decode_rows(DECODE_STEPS + 2)
    dw.assemble()
    layers = list(range(wl.model.layers))
    pre = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    dec = run_decode(dw, layers, DECODE_STEPS, VARIANT_MATERIALIZED)
    for b in range(wl.batch):
        _say(name, b, check_decode(dw, b, layers, pre, dec))
    # the fused variant decodes to identical bits (same split, same rows)
    dec_f = run_decode(dw, layers, DECODE_STEPS, VARIANT_FUSED)
    for l in layers:
        for st in range(DECODE_STEPS):
            assert torch.equal(dec[l][st][3], dec_f[l][st][3]), f"fused decode differs (layer {l}, step {st})"
    # keys gathered, values read in the pool: prefill and decode, the same bits
    assert dw.assemble(values_in_pool=True)["values_in_pool"] == 1
    pre_p = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    dec_p = run_decode(dw, layers, DECODE_STEPS, VARIANT_MATERIALIZED)
    for l in layers:
        assert torch.equal(pre[l][3], pre_p[l][3]), f"values in the pool: prefill differs on layer {l}"
        for st in range(DECODE_STEPS):
            assert torch.equal(dec[l][st][3], dec_p[l][st][3]), f"values in the pool: decode differs ({l}, {st})"
    dw.close()
    del dw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["turborag_b16", "long_16k_b32"])
def test_decode_after_prefill_full_size(name):
    wl = W.get(name)
    _say(f"case decode full {name}")
    dw = open_workload(wl)
    dw.session.set_decode_rows(4)
    dw.assemble()
    L = wl.model.layers
    checked = sorted({0, L - 1})
    pre = run_prefill(dw, list(range(L)), VARIANT_MATERIALIZED)
    dec = run_decode(dw, checked, 2, VARIANT_MATERIALIZED)
    for b in sorted({0, wl.batch - 1}):
        _say(name, b, check_decode(dw, b, checked, pre, dec))
    dw.close()
    del dw, pre, dec
    torch.cuda.empty_cache()


def _token_subset(n, k=16):
    if n <= k:
        return None
    idx = np.unique(np.concatenate([[0, 1, n - 2, n - 1], np.linspace(0, n - 1, k - 4).round().astype(int)]))
    return idx


@pytest.mark.parametrize("name", [n for n in W.FULL_SIZE if n != "tiny_f32"] +
                         ["turborag_b16_unrot", "turborag_b16_composite"])
def test_full_size_workloads_sampled(name):
    wl = W.get(name)
    _say(f"case full {name}: batch {wl.batch}, rows {wl.rows_total}")
    dw = open_workload(wl)
    summ = dw.assemble()
    L = wl.model.layers
    checked = sorted({0, L // 2, L - 1})
    res = run_prefill(dw, list(range(L)), VARIANT_MATERIALIZED)   # whole path, as benchmarked
    for b in sorted({0, wl.batch - 1}):
        sub = _token_subset(wl.requests[b].n_new)
        st = check_request(dw, b, checked, res, token_subset=sub)
        _say(name, b, st)
    # a second launch gives the same bits (row splits merge in split order,
    # whichever finishes last; long_131k_b1 merges across workgroups)
    again = run_prefill(dw, checked[:1], VARIANT_MATERIALIZED)
    assert torch.equal(res[checked[0]][3], again[checked[0]][3]), f"{name}: not reproducible"
    res_f = run_prefill(dw, checked, VARIANT_FUSED)
    for l in checked:
        assert torch.equal(res[l][3], res_f[l][3]), f"fused != materialised on layer {l}"
    assert summ["rows"] == wl.rows_total
    del res_f, again
    check_values_in_pool(dw, checked, res)
    # plan-only, as the fused variant is benchmarked
    check_fused_plan_only(dw, checked, res)
    dw.close()
    del dw, res
    torch.cuda.empty_cache()


def test_layer_pipelined_gather_matches_one_gather():
    # plan first, then gather each layer on a second stream right before the
    # layer's prefill on the main stream: the same bits as one full gather
    wl = W.get("coinrag_small")
    _say("case pipelined gather")
    dw = open_workload(wl)
    dw.assemble()
    layers = list(range(wl.model.layers))
    ref = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    dw.assemble(defer=True)
    with pytest.raises(Exception):
        dw.session.prefill_layer(0, *dw.layer_inputs(0))          # layer 0 not gathered yet
    side = torch.cuda.Stream()
    res = {}
    dw.session.plan.gather_layers(0, 1, side)
    for l in layers:
        if l + 1 < wl.model.layers:
            dw.session.plan.gather_layers(l + 1, l + 2, side)
        q, k, v = dw.layer_inputs(l)
        res[l] = dw.session.prefill_layer(l, q, k, v)
    torch.cuda.synchronize()
    for l in layers:
        assert torch.equal(ref[l][3], res[l]), f"pipelined gather differs on layer {l}"
    dw.close()


@pytest.mark.parametrize("name", ["turborag_small", "coinrag_small_unrot"])
def test_pool_in_pinned_host_memory(name):
    # the staging tier: the pool in pinned host memory, only covered rows read
    wl = W.get(name)
    _say(f"case host pool {name}")
    dw = open_workload(wl, host_pool=True)
    assert not dw.pool.is_cuda
    dw.assemble()
    layers = list(range(wl.model.layers))
    res_m = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    for b in range(wl.batch):
        _say(name, b, check_request(dw, b, layers, res_m))
    check_fused_plan_only(dw, layers, res_m)
    check_values_in_pool(dw, layers, res_m)
    dw.close()


def _covered_pages(wl):
    """Pool pages (ids) the batch's spans cover."""
    pt = wl.pool.page_tokens
    pages = set()
    for r in wl.requests:
        for c, s0, e0, _t in r.spans:
            base = int(wl.pool.chunk_page_ptr[c])
            for q in range(base + int(s0) // pt, base + int(e0) // pt + 1):
                pages.add(int(wl.pool.page_ids[q]))
    return pages


@pytest.mark.parametrize("name", ["turborag_small", "coinrag_small_unrot"])
def test_hot_set_in_front_of_host_pool(name):
    """An HBM hot set with LRU eviction in front of the pinned-host pool.
    Batch layouts over one pool go through a hot set that holds any one
    batch but not all of them: every batch assembles and attends bit for bit
    as from the device pool (variant M, variant F after a plan-only
    assembly, values left in the pool); pages are admitted, reused and
    evicted; a batch whose pages are all resident copies nothing; decode
    after a prefill through the hot set gives the device pool's bits."""
    wls = [W.get(name, layout=k) for k in range(3)]
    need = [_covered_pages(w) for w in wls]
    cap = max(len(x) for x in need)
    assert len(set().union(*need)) > cap, "the layouts must not fit together"
    layers = list(range(wls[0].model.layers))
    ref = {}
    dref = open_workload(wls[0])
    for k, w in enumerate(wls):
        dref.wl = w
        dref.assemble()
        ref[k] = run_prefill(dref, layers, VARIANT_MATERIALIZED)
    dref.wl = wls[1]
    dref.session.set_decode_rows(2)
    dref.assemble()
    run_prefill(dref, layers, VARIANT_MATERIALIZED)
    dec_ref = run_decode(dref, layers, 2, VARIANT_MATERIALIZED)
    dref.close()
    _say(f"case hot set {name}: {cap} page slots, batches need {[len(x) for x in need]}")
    dw = open_workload(wls[0], host_pool=True, hot_pages=cap)
    assert not dw.pool.is_cuda
    cache = dw.session.cache
    for k in (0, 1, 2, 0):
        dw.wl = wls[k]
        dw.assemble()
        res = run_prefill(dw, layers, VARIANT_MATERIALIZED)
        for l in layers:
            assert torch.equal(ref[k][l][3], res[l][3]), f"layout {k}: hot set differs on layer {l}"
        check_fused_plan_only(dw, layers, res)
        check_values_in_pool(dw, layers, res)
        st = cache.stats()
        _say(f"  layout {k}: {st}")
        assert st["resident_pages"] <= cap
    st = cache.stats()
    assert st["misses"] > 0 and st["evictions"] > 0 and st["hits"] > 0, st
    # the same batch again: every page resident, nothing copied
    dw.assemble()
    run_prefill(dw, layers, VARIANT_MATERIALIZED)
    st2 = cache.stats()
    assert st2["bytes_copied"] == st["bytes_copied"] and st2["misses"] == st["misses"], (st, st2)
    # decode through the hot set: M, F after a plan-only assembly, values in the pool
    dw.wl = wls[1]
    dw.session.set_decode_rows(2)
    for how in ("gathered", "plan_only", "values_in_pool"):
        dw.assemble(plan_only=how == "plan_only", values_in_pool=how == "values_in_pool")
        variant = VARIANT_FUSED if how == "plan_only" else VARIANT_MATERIALIZED
        run_prefill(dw, layers, variant)
        dec = run_decode(dw, layers, 2, variant)
        for l in layers:
            for stp in range(2):
                assert torch.equal(dec_ref[l][stp][3], dec[l][stp][3]), f"hot set decode ({how}) differs ({l}, {stp})"
    _say(f"  decode through the hot set: {cache.stats()}")
    dw.close()


@pytest.mark.parametrize("name,hot", [("turborag_small", False), ("coinrag_small_unrot", True)])
def test_chunk_files_behind_the_host_pool(name, hot, tmp_path):
    """One file per chunk behind the pinned-host pool (and a hot set): the
    pool memory starts as NaN bytes and pic_assemble reads exactly the pages
    each batch covers from the files.  Every layout then attends bit for bit
    as from the device pool; pages outside every batch stay unread; a page
    already read is not read again; a request made ahead of the assembly
    (prefetch) leaves nothing for the assembly to read; decode after a
    prefill matches too."""
    wls = [W.get(name, layout=k) for k in range(3)]
    need = [_covered_pages(w) for w in wls]
    layers = list(range(wls[0].model.layers))
    ref = {}
    dref = open_workload(wls[0])
    for k, w in enumerate(wls):
        dref.wl = w
        dref.assemble()
        ref[k] = run_prefill(dref, layers, VARIANT_MATERIALIZED)
    dref.wl = wls[2]
    dref.session.set_decode_rows(2)
    dref.assemble()
    run_prefill(dref, layers, VARIANT_MATERIALIZED)
    dec_ref = run_decode(dref, layers, 2, VARIANT_MATERIALIZED)
    dref.close()
    cap = max(len(x) for x in need) if hot else 0
    _say(f"case chunk files {name}: hot set {cap} slots, batches cover {[len(x) for x in need]} pages")
    dw = open_workload(wls[0], host_pool=True, hot_pages=cap, store_dir=str(tmp_path), store_threads=4)
    store = dw.session.store
    page_bytes = W.page_bytes(wls[0].model, wls[0].pool.page_tokens)
    host = dw.pool.view(torch.uint8).reshape(dw.pool.shape[0], page_bytes)
    seen = set()
    for k in (0, 1):
        dw.wl = wls[k]
        dw.assemble()
        res = run_prefill(dw, layers, VARIANT_MATERIALIZED)
        for l in layers:
            assert torch.equal(ref[k][l][3], res[l][3]), f"layout {k}: chunk files differ on layer {l}"
        seen |= need[k]
        st = store.stats()
        _say(f"  layout {k}: {st}")
        assert st["pages_read"] == len(seen) == st["resident_pages"], (st, len(seen))
        # pages no batch has covered yet were never written
        untouched = [pg for pg in range(dw.pool.shape[0]) if pg not in seen]
        assert untouched or k > 0, "the first layout covers every page: nothing to check"
        assert bool((host[untouched] == 0xFF).all()), f"layout {k}: a page outside the batches was written"
    # layout 2 read ahead of its assembly: the assembly then reads nothing
    wl2 = wls[2]
    store.request(wl2.span_ptr(), wl2.spans_flat())
    store.wait()
    before = store.stats()["pages_read"]
    dw.wl = wl2
    dw.session.set_decode_rows(2)
    dw.assemble()
    assert store.stats()["pages_read"] == before
    run_prefill(dw, layers, VARIANT_MATERIALIZED)
    dec = run_decode(dw, layers, 2, VARIANT_MATERIALIZED)
    for l in layers:
        for stp in range(2):
            assert torch.equal(dec_ref[l][stp][3], dec[l][stp][3]), f"decode over chunk files differs ({l}, {stp})"
    # forgotten pages are read again, with the same bits
    torch.cuda.synchronize()
    store.forget(drop_os_cache=True)
    dw.wl = wls[0]
    dw.session.set_decode_rows(0)
    dw.assemble()
    res = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    for l in layers:
        assert torch.equal(ref[0][l][3], res[l][3]), f"re-read layout 0 differs on layer {l}"
    _say(f"  after forget: {store.stats()}")
    dw.close()


def _edge_workload(keys="rotated"):
    """Ragged shapes and degenerate spans on Qwen2-like heads, two layers."""
    rng = np.random.default_rng(77)
    model = W.ModelShape(2, 28, 4, 128, 1e6, "bf16")
    pool = W.make_pool(rng, [512, 300, 17, 1, 96], page_tokens=16)
    pool.chunk_orig = np.array([0, 1000, 5, 0, 70000], np.int32)
    A = W.TARGET_AUTO
    reqs = [
        # 1-token spans, a span at a chunk's end, a repeated span, negative deltas
        # (target before the original position), an explicit target that
        # overlaps positions already used, a large original base, a span kept
        # at its original positions (later than every query: fully masked)
        W.Request(np.array([[0, 511, 511, 0], [3, 0, 0, A], [1, 299, 299, A], [1, 0, 299, A],
                            [1, 0, 299, A], [2, 3, 9, 2], [4, 0, 95, A],
                            [4, 10, 20, W.TARGET_ORIGINAL]], np.int32), 37,
                  np.arange(105, 142, dtype=np.int32)),
        # no spans: plain causal prefill
        W.Request(np.zeros((0, 4), np.int32), 29, np.arange(29, dtype=np.int32)),
        # no new tokens
        W.Request(np.array([[0, 0, 63, A], [0, 64, 127, A]], np.int32), 0, np.zeros(0, np.int32)),
        # interleaved: new tokens before, between and after the cached spans, one at position 0
        W.Request(np.array([[0, 5, 70, 10], [2, 0, 16, 300]], np.int32), 9,
                  np.array([0, 1, 2, 200, 201, 250, 400, 401, 402], np.int32)),
    ]
    return W.Workload("edge", 0, model, pool, reqs, W.ValueRecipe("lognormal", "half"), 900, keys=keys)


@pytest.mark.parametrize("keys", ["rotated", "unrotated"])
def test_edge_cases_ragged_degenerate_and_canary(keys):
    wl = _edge_workload(keys)
    _say(f"case edge, keys {keys}")
    dw = open_workload(wl)
    sess = dw.session
    cap = wl.rows_total + 37
    sess.ensure_capacity(cap)
    nan_bits = torch.tensor(-1, dtype=torch.int16)           # 0xFFFF: a NaN bf16 canary
    sess.asm_k.view(torch.int16).fill_(nan_bits)
    sess.asm_v.view(torch.int16).fill_(nan_bits)
    dw.assemble()
    layers = [0, 1]
    res = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    for b in range(wl.batch):
        _say("edge", b, check_request(dw, b, layers, res))
    rows = wl.rows_total
    for t in (sess.asm_k, sess.asm_v):
        assert not torch.isnan(t[:, :, :rows].float()).any(), "a planned row was not written"
        assert bool((t[:, :, rows:].view(torch.int16) == -1).all()), "rows beyond the batch were written"
    res_f = run_prefill(dw, layers, VARIANT_FUSED)
    for l in layers:
        assert torch.equal(res[l][3], res_f[l][3])
    # keys only: the planes' prefix values keep the canary, the rest is written
    sess.asm_k.view(torch.int16).fill_(nan_bits)
    sess.asm_v.view(torch.int16).fill_(nan_bits)
    check_values_in_pool(dw, layers, res)
    rb, pr, _ = sess.plan.requests()
    for b in range(wl.batch):
        base, npre, nn = int(rb[b]), int(pr[b]), wl.requests[b].n_new
        for l in layers:
            assert not torch.isnan(sess.asm_k[l, :, base:base + npre + nn].float()).any()
            assert bool((sess.asm_v[l, :, base:base + npre].view(torch.int16) == -1).all()), \
                "prefix values were gathered"
            assert not torch.isnan(sess.asm_v[l, :, base + npre:base + npre + nn].float()).any()
    check_fused_plan_only(dw, layers, res)
    dw.close()


def _whole_block_edge_workload():
    """Spans of multiples of 32 rows with negative and large deltas, a span
    kept at its original positions, repeated spans, explicit targets, ragged
    new-token tails, interleaved new tokens, a request without spans and one
    without new tokens."""
    model = W.ModelShape(2, 28, 4, 128, 1e6, "bf16")
    rng = np.random.default_rng(78)
    pool = W.make_pool(rng, [512, 300, 96, 64], page_tokens=16)
    pool.chunk_orig = np.array([0, 1000, 70000, 5], np.int32)
    A = W.TARGET_AUTO
    reqs = [
        W.Request(np.array([[0, 0, 63, A], [1, 32, 95, A], [2, 0, 95, A], [0, 128, 159, A],
                            [3, 0, 31, W.TARGET_ORIGINAL]], np.int32), 37,
                  np.arange(288, 325, dtype=np.int32)),
        W.Request(np.zeros((0, 4), np.int32), 29, np.arange(29, dtype=np.int32)),
        W.Request(np.array([[0, 0, 63, A], [0, 64, 127, A]], np.int32), 0, np.zeros(0, np.int32)),
        W.Request(np.array([[0, 256, 287, 1000], [0, 256, 287, 1000], [1, 0, 31, 40]], np.int32), 5,
                  np.arange(1032, 1037, dtype=np.int32)),
        W.Request(np.array([[0, 0, 31, 10], [1, 0, 31, 300]], np.int32), 9,
                  np.array([0, 1, 2, 200, 201, 250, 400, 401, 402], np.int32)),
    ]
    return W.Workload("edge_blocks", 0, model, pool, reqs, W.ValueRecipe("lognormal", "half"), 901)


def test_whole_block_edge_cases_and_retired_query_rotation():
    wl = _whole_block_edge_workload()
    _say("case edge, whole 32-row blocks")
    dw = open_workload(wl)
    dw.assemble()
    layers = [0, 1]
    res = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    for b in range(wl.batch):
        _say("edge_blocks", b, check_request(dw, b, layers, res))
    check_query_rotation_refused(dw)
    check_fused_plan_only(dw, layers, res)
    # twice in a row: the same bits
    a1 = run_prefill(dw, layers, VARIANT_FUSED)
    a2 = run_prefill(dw, layers, VARIANT_FUSED)
    for l in layers:
        assert torch.equal(a1[l][3], a2[l][3]), f"fused variant not reproducible on layer {l}"
        assert torch.equal(a1[l][3], res[l][3]), f"fused != materialised on layer {l}"
    dw.close()


def test_decode_on_edge_layouts():
    """Decode over the whole-block edge layouts plus a request with neither
    spans nor new tokens, for 66 steps: its first token attends to itself
    only, and the earlier rows of every request cross a 64-row tile boundary
    (a column block's splits may hold no tiles).  Every step against the
    oracle; the fused variant gives the same bits."""
    base = _whole_block_edge_workload()
    reqs = list(base.requests) + [W.Request(np.zeros((0, 4), np.int32), 0, np.zeros(0, np.int32))]
    wl = W.Workload("edge_decode", 0, base.model, base.pool, reqs, base.values, 902)
    steps = 66
    _say("case decode, edge layouts")
    dw = open_workload(wl)
    dw.session.set_decode_rows(steps + 4)
    dw.assemble()
    layers = [0, 1]
    pre = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    dec = run_decode(dw, layers, steps, VARIANT_MATERIALIZED)
    for b in range(wl.batch):
        _say("edge_decode", b, check_decode(dw, b, layers, pre, dec))
    dec_f = run_decode(dw, layers, steps, VARIANT_FUSED)
    for l in layers:
        for st in range(steps):
            assert torch.equal(dec[l][st][3], dec_f[l][st][3]), f"fused decode differs (layer {l}, step {st})"
    dw.close()


def _random_workload(seed):
    """A seeded random layout on Qwen2-like heads, two layers: 3-8 chunks of
    1-299 tokens at random original positions; 1-5 requests of 0-6 spans
    (any sub-span, one token up to a whole chunk, repeats allowed) placed
    automatically, at their original positions or at explicit targets; 0-40
    new tokens that follow the prefix or (every request of the batch) sit at
    random increasing positions (the first request has at least one)."""
    rng = np.random.default_rng(4000 + seed)
    model = W.ModelShape(2, 28, 4, 128, 1e6, "bf16")
    n_chunks = int(rng.integers(3, 9))
    lens = rng.integers(1, 300, n_chunks)
    pool = W.make_pool(rng, lens, page_tokens=16)
    pool.chunk_orig = rng.integers(0, 5000, n_chunks).astype(np.int32)
    reqs = []
    explicit = rng.random() < 0.5
    for b in range(int(rng.integers(1, 6))):
        spans = []
        for _ in range(int(rng.integers(0, 7))):
            c = int(rng.integers(0, n_chunks))
            s0 = int(rng.integers(0, lens[c]))
            e0 = int(rng.integers(s0, lens[c]))
            kind = rng.random()
            t = W.TARGET_AUTO if kind < 0.6 else (W.TARGET_ORIGINAL if kind < 0.75 else int(rng.integers(0, 3000)))
            spans.append([c, s0, e0, t])
        n_new = int(rng.integers(1 if b == 0 else 0, 41))
        new_pos = np.sort(rng.choice(6000, n_new, replace=False)).astype(np.int32) if explicit else None
        reqs.append(W.Request(np.array(spans, np.int32).reshape(-1, 4), n_new, new_pos))
    return W.Workload(f"random_{seed}", 0, model, pool, reqs, W.ValueRecipe("lognormal", "half"), 950 + seed)


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts_every_element(seed):
    """Seeded random layouts: every output element and every assembled row
    against the oracle, the fused variant and values left in the pool bit
    for bit against M, and three decode steps."""
    wl = _random_workload(seed)
    _say(f"case random {seed}: (spans, new tokens) {[(len(r.spans), r.n_new) for r in wl.requests]}")
    dw = open_workload(wl)
    dw.session.set_decode_rows(3)
    dw.assemble()
    layers = [0, 1]
    res = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    for b in range(wl.batch):
        _say(f"random {seed}", b, check_request(dw, b, layers, res))
    res_f = run_prefill(dw, layers, VARIANT_FUSED)
    for l in layers:
        assert torch.equal(res[l][3], res_f[l][3]), f"fused != materialised on layer {l}"
    dec = run_decode(dw, layers, 3, VARIANT_MATERIALIZED)
    for b in range(wl.batch):
        check_decode(dw, b, layers, res, dec)
    check_values_in_pool(dw, layers, res)
    dw.close()


def test_plan_reuse_with_smaller_batch():
    wl = W.get("coinrag_small")
    _say("case reuse")
    dw = open_workload(wl)
    dw.assemble()
    run_prefill(dw, [0], VARIANT_MATERIALIZED)
    small = W.Workload("coinrag_small_1", wl.cfg, wl.model, wl.pool, wl.requests[1:2], wl.values, wl.seed)
    dw2 = type(dw)(small, dw.pool, dw.kscale, dw.vscale, dw.session)
    dw2.assemble()
    res = run_prefill(dw2, [0, 1], VARIANT_MATERIALIZED)
    _say("reuse", check_request(dw2, 0, [0, 1], res))
    dw.close()


def test_calls_of_one_plan_on_alternating_streams():
    """Calls on a plan share its scratch (rotated queries, split partials,
    merge counters): a call on another stream than the previous one waits for
    that stream's work, so alternating streams gives the one-stream bits.
    coinrag_small splits its rows (partials and merges on every layer)."""
    wl = W.get("coinrag_small")
    _say("case alternating streams")
    dw = open_workload(wl)
    dw.assemble()
    layers = list(range(wl.model.layers))
    ref = run_prefill(dw, layers, VARIANT_MATERIALIZED)
    inputs = {l: dw.layer_inputs(l) for l in layers}
    outs = {l: torch.empty_like(inputs[l][0]) for l in layers}
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(2):
        with torch.cuda.stream(streams[rep % 2]):
            dw.assemble()
        for i, l in enumerate(layers):
            for variant in (VARIANT_MATERIALIZED, VARIANT_FUSED):
                with torch.cuda.stream(streams[(i + rep + variant) % 2]):
                    q, k, v = inputs[l]
                    dw.session.prefill_layer(l, q, k, v, out=outs[l], variant=variant)
        torch.cuda.synchronize()
        for l in layers:
            assert torch.equal(ref[l][3], outs[l]), f"layer {l} differs with alternating streams (round {rep})"
    dw.close()
