"""The entry point that allocates nothing, against the one it varies.

pic_query_prefill_noalloc runs pic_query_prefill's kernels with their
scratch (rotated queries, row-split partials, merge counters) in the
library's fixed device array: its outputs, and the rows it appends to the
assembled planes, must be the same bits.  Two calls in a row, the second on
a smaller batch (the array keeps the first call's contents), and a batch too
large for the array (refused before anything is enqueued).
"""
import numpy as np
import pytest
import torch

import workloads as W
from position_independent_kv_pic_amd import VARIANT_FUSED, VARIANT_MATERIALIZED, PicError
from workloads.device import open_workload

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _both(dw, layers, variant):
    """Every layer through pic_query_prefill, then through the no-alloc entry
    point (re-assembled in between, so both start from the same planes)."""
    plan = dw.session.plan
    ins = {l: dw.layer_inputs(l) for l in layers}
    ref, got = {}, {}
    for tag, call, store in (("ref", plan.query_prefill, ref), ("noalloc", plan.query_prefill_noalloc, got)):
        dw.assemble(plan_only=variant == VARIANT_FUSED)
        for l in layers:
            q, k, v = ins[l]
            out = torch.empty_like(q)
            call(l, q, k, v, out, variant, torch.cuda.current_stream())
            store[l] = out
        torch.cuda.synchronize()
        if tag == "ref":
            planes = (dw.session.asm_k.clone(), dw.session.asm_v.clone())
    # the planes, bit for bit (a plan-only batch leaves its prefix rows
    # unwritten: whatever they held, NaN patterns included, must stay)
    rows = dw.wl.rows_total
    for before, after in zip(planes, (dw.session.asm_k, dw.session.asm_v)):
        assert torch.equal(before[:, :, :rows].view(torch.int16), after[:, :, :rows].view(torch.int16))
    return ref, got


def _across_workload():
    """One request of 16 whole 2048-token documents (512 tiles) and 256 new
    tokens on 4 kv heads of 8 query heads each, so few column blocks that the
    rows are split across workgroups (merge counters), then a smaller one."""
    model = W.ModelShape(1, 32, 4, 128, 1e6, "bf16")
    rng = np.random.default_rng(11)
    pool = W.make_pool(rng, [2048] * 16, page_tokens=16)
    A = W.TARGET_AUTO
    reqs = [W.Request(np.array([[c, 0, 2047, A] for c in range(16)], np.int32), 256, None),
            W.Request(np.array([[3, 0, 2047, A], [5, 0, 2047, A]], np.int32), 64, None)]
    return W.Workload("noalloc_across", 5, model, pool, reqs, W.ValueRecipe("outlier", "outlier"), 11)


def _splits_across_workgroups(plan) -> bool:
    """Every column block of request 0 runs 8 or more row ranges of at least
    64 tiles each, as only the cross-workgroup split does."""
    items, _ = plan.attention_work()
    ranges = {}
    for it in items:
        if it[0] == 0:
            ranges.setdefault((int(it[1]), int(it[2])), set()).add((int(it[3]), int(it[4])))
    return all(len(r) >= 2 and min(e - b for b, e in r) >= 64 for r in ranges.values())


@pytest.mark.parametrize("variant", [VARIANT_MATERIALIZED, VARIANT_FUSED])
def test_noalloc_prefill_equals_prefill_twice_second_smaller(variant):
    # coinrag_small splits its rows (partials merged in LDS and by the merge
    # kernel); the third workload splits them across workgroups (partials
    # merged by the last split to count itself in a merge counter)
    for name in ("coinrag_small", "long_small", "across"):
        wl = _across_workload() if name == "across" else W.get(name)
        _say(f"case noalloc {name} variant {variant}")
        dw = open_workload(wl)
        layers = list(range(wl.model.layers))
        ref, got = _both(dw, layers, variant)
        if name == "across":
            assert _splits_across_workgroups(dw.session.plan), "the layout does not split across workgroups"
        for l in layers:
            assert torch.equal(ref[l].view(torch.int16), got[l].view(torch.int16)), \
                f"{name} layer {l}: no-alloc output differs"
        # the second call on a smaller batch of the same pool (fewer requests)
        small = W.Workload(name + "_1", wl.cfg, wl.model, wl.pool, wl.requests[-1:], wl.values, wl.seed)
        dw2 = type(dw)(small, dw.pool, dw.kscale, dw.vscale, dw.session)
        ref2, got2 = _both(dw2, layers, variant)
        for l in layers:
            assert torch.equal(ref2[l].view(torch.int16), got2[l].view(torch.int16)), \
                f"{name} smaller batch layer {l}: no-alloc output differs"
        dw.close()
        del dw, dw2
        torch.cuda.empty_cache()


def test_noalloc_prefill_refuses_a_batch_beyond_its_scratch():
    # 16400 new tokens x 32 query heads x 128 bf16 = 134.3 MB of rotated
    # queries, more than the 128 MiB array: refused, nothing enqueued
    model = W.ModelShape(1, 32, 1, 128, 1e4, "bf16")
    rng = np.random.default_rng(5)
    pool = W.make_pool(rng, [64], page_tokens=16)
    req = W.Request(np.zeros((0, 4), np.int32), 16400, np.arange(16400, dtype=np.int32))
    wl = W.Workload("noalloc_big", 0, model, pool, [req], W.ValueRecipe("lognormal", "half"), 7)
    dw = open_workload(wl)
    dw.assemble()
    q, k, v = dw.layer_inputs(0)
    out = torch.full_like(q, 7.0)
    with pytest.raises(PicError, match="PIC_ERANGE"):
        dw.session.plan.query_prefill_noalloc(0, q, k, v, out, VARIANT_MATERIALIZED, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call wrote its output"
    dw.close()
