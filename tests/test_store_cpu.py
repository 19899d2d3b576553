"""CPU checks of the chunk-file store through the C ABI.

The store is host code only (files, threads, host memory), so it runs here
against a numpy destination: the pool is registered at a fake device address
that nothing dereferences.  Pool contents are seeded random bytes: the store
moves pages and never looks inside them.  The pages a batch covers are
derived here from the span table directly (chunk c's tokens s..e live in its
pages s // page_tokens .. e // page_tokens), independently of the library.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import workloads as W
from position_independent_kv_pic_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "position_independent_kv_pic_amd", "csrc")
FAKE_POOL = 1 << 40
CANARY = 0xA5


def _model(wl):
    m = wl.model
    return B.model_struct(m.layers, m.q_heads, m.kv_heads, m.head_dim, m.theta, m.dtype, wl.keys)


def _pool(wl, page_ids=None, base=FAKE_POOL):
    p = wl.pool
    ids = p.page_ids if page_ids is None else page_ids
    return B.Pool(_model(wl), base, p.n_pages * W.page_bytes(wl.model, p.page_tokens), p.page_tokens,
                  p.n_pages, p.chunk_len, p.chunk_page_ptr, ids, p.chunk_orig)


def _source(wl, seed=7):
    p = wl.pool
    pb = W.page_bytes(wl.model, p.page_tokens)
    return np.random.default_rng(seed).integers(0, 256, size=(p.n_pages, pb), dtype=np.uint8)


def _write_files(wl, src, folder):
    p = wl.pool
    paths = []
    for c in range(len(p.chunk_len)):
        path = os.path.join(folder, f"chunk{c:05d}.pic")
        lo = int(p.chunk_page_ptr[c])
        B.write_chunk_file(_model(wl), p.page_tokens, int(p.chunk_len[c]), int(p.chunk_orig[c]), src,
                           np.asarray(p.page_ids[lo:int(p.chunk_page_ptr[c + 1])], np.int32), path)
        paths.append(path)
    return paths


def _covered(wl, spans):
    """Logical pages (indices into page_ids) that the spans cover."""
    p = wl.pool
    out = set()
    for c, s, e, _t in np.asarray(spans).reshape(-1, 4):
        lo = int(p.chunk_page_ptr[c])
        out.update(range(lo + int(s) // p.page_tokens, lo + int(e) // p.page_tokens + 1))
    return sorted(out)


@pytest.fixture(scope="module")
def coinrag(tmp_path_factory):
    wl = W.get("coinrag_small")
    src = _source(wl)
    folder = str(tmp_path_factory.mktemp("chunks"))
    return wl, src, _write_files(wl, src, folder)


def test_chunk_file_layout(coinrag):
    """Header fields and page order as the header file states them."""
    wl, src, paths = coinrag
    p = wl.pool
    pb = W.page_bytes(wl.model, p.page_tokens)
    c = 3
    raw = np.fromfile(paths[c], dtype=np.uint8)
    need = -(-int(p.chunk_len[c]) // p.page_tokens)
    assert raw.size == 4096 + need * pb
    head = raw[:4096].tobytes()
    assert head[:8] == b"PICCHUNK"
    version, hbytes = struct.unpack_from("<II", head, 8)
    layers, q_heads, kv_heads, head_dim, dtype, keys, pt, length, orig = struct.unpack_from("<9i", head, 16)
    page_bytes, n_pages = struct.unpack_from("<qq", head, 56)
    (theta,) = struct.unpack_from("<d", head, 72)
    m = wl.model
    assert (version, hbytes) == (1, 4096)
    assert (layers, q_heads, kv_heads, head_dim) == (m.layers, m.q_heads, m.kv_heads, m.head_dim)
    assert (dtype, keys, pt, length, orig) == (B.PIC_BF16, 0, p.page_tokens, int(p.chunk_len[c]), int(p.chunk_orig[c]))
    assert (page_bytes, n_pages, theta) == (pb, need, m.theta)
    assert not head[80:].strip(b"\0")
    lo = int(p.chunk_page_ptr[c])
    for j in range(need):
        assert np.array_equal(raw[4096 + j * pb:4096 + (j + 1) * pb], src[p.page_ids[lo + j]])


def test_store_loads_exactly_the_covered_pages(coinrag):
    wl, src, paths = coinrag
    p = wl.pool
    pool = _pool(wl)
    dst = np.full_like(src, CANARY)
    store = B.Store(pool, dst, dst.nbytes, paths, threads=4)
    try:
        st = store.stats()
        assert st["resident_pages"] == 0 and st["pages_read"] == 0
        spans = np.asarray(wl.spans_flat())
        store.request(wl.span_ptr(), spans)
        store.wait()
        covered = _covered(wl, spans)
        cov = set(covered)
        for q in range(int(p.chunk_page_ptr[-1])):
            page = p.page_ids[q]
            if q in cov:
                assert np.array_equal(dst[page], src[page]), f"page {q} not loaded"
            else:
                assert (dst[page] == CANARY).all(), f"page {q} was written but not covered"
        st = store.stats()
        assert st["pages_read"] == len(covered) == st["resident_pages"]
        assert st["bytes_read"] == len(covered) * src.shape[1]
        assert st["requested"] == len(covered) and st["hits"] == 0
        assert 1 <= st["reads"] <= len(covered)
        # the same batch again: nothing is read
        store.request(wl.span_ptr(), spans)
        store.wait()
        st2 = store.stats()
        assert st2["pages_read"] == st["pages_read"] and st2["hits"] == len(covered)
        # forgotten pages are read again
        store.forget(drop_os_cache=True)
        assert store.stats()["resident_pages"] == 0
        dst[:] = CANARY
        store.request(wl.span_ptr(), spans)
        store.wait()
        assert store.stats()["pages_read"] == 2 * len(covered)
        for q in covered:
            assert np.array_equal(dst[p.page_ids[q]], src[p.page_ids[q]])
    finally:
        store.release()
        pool.release()


def test_store_one_request_per_batch_of_each_layout(coinrag):
    """Requests of one request's spans at a time add up to the whole batch."""
    wl, src, paths = coinrag
    pool = _pool(wl)
    dst = np.full_like(src, CANARY)
    store = B.Store(pool, dst, dst.nbytes, paths, threads=8)
    try:
        sp = wl.span_ptr()
        spans = np.asarray(wl.spans_flat())
        for b in range(wl.batch):
            part = spans[sp[b]:sp[b + 1]]
            store.request([0, len(part)], part)
        store.wait()
        covered = _covered(wl, spans)
        assert store.stats()["pages_read"] == len(covered)
        for q in covered:
            assert np.array_equal(dst[wl.pool.page_ids[q]], src[wl.pool.page_ids[q]])
    finally:
        store.release()
        pool.release()


def test_store_rejects_malformed_files_and_arguments(coinrag, tmp_path):
    wl, src, paths = coinrag
    p = wl.pool
    pool = _pool(wl)
    dst = np.full_like(src, CANARY)
    try:
        missing = list(paths)
        missing[5] = str(tmp_path / "absent.pic")
        with pytest.raises(B.PicError, match="absent.pic"):
            B.Store(pool, dst, dst.nbytes, missing)
        # a file of another chunk (other length) in chunk 0's place
        other = next(c for c in range(1, len(paths)) if p.chunk_len[c] != p.chunk_len[0])
        swapped = list(paths)
        swapped[0] = paths[other]
        with pytest.raises(B.PicError, match="tokens at origin"):
            B.Store(pool, dst, dst.nbytes, swapped)
        # a file cut short
        short = str(tmp_path / "short.pic")
        shutil.copy(paths[2], short)
        os.truncate(short, os.path.getsize(short) - 1)
        cut = list(paths)
        cut[2] = short
        with pytest.raises(B.PicError, match="shorter"):
            B.Store(pool, dst, dst.nbytes, cut)
        # not a chunk file
        junk = str(tmp_path / "junk.pic")
        with open(junk, "wb") as f:
            f.write(b"\0" * 8192)
        bad = list(paths)
        bad[1] = junk
        with pytest.raises(B.PicError, match="not a chunk file"):
            B.Store(pool, dst, dst.nbytes, bad)
        with pytest.raises(B.PicError, match="smaller"):
            B.Store(pool, dst, dst.nbytes - 1, paths)
        with pytest.raises(B.PicError, match="threads"):
            B.Store(pool, dst, dst.nbytes, paths, threads=0)
        with pytest.raises(B.PicError, match="device memory"):
            B.Store(pool, FAKE_POOL, dst.nbytes, paths)
        store = B.Store(pool, dst, dst.nbytes, paths, threads=2)
        try:
            with pytest.raises(B.PicError, match="chunk"):
                store.request([0, 1], [[len(paths), 0, 0, -1]])
            with pytest.raises(B.PicError, match="s <= e"):
                store.request([0, 1], [[0, 3, 2, -1]])
            with pytest.raises(B.PicError, match="s <= e"):
                store.request([0, 1], [[0, 0, int(p.chunk_len[0]), -1]])
            assert store.stats()["requested"] == 0
        finally:
            store.release()
    finally:
        pool.release()
    # two chunk pages on one pool page cannot both be file-backed
    ids = np.array(p.page_ids, np.int32)
    ids[1] = ids[0]
    dup = _pool(wl, page_ids=ids)
    try:
        with pytest.raises(B.PicError, match="distinct"):
            B.Store(dup, dst, dst.nbytes, paths)
    finally:
        dup.release()


def test_pool_release_waits_for_a_store_over_device_memory_only(coinrag):
    """A store over a device pool fills a separate buffer and is not attached:
    the pool can be released while it is open."""
    wl, src, paths = coinrag
    pool = _pool(wl)
    dst = np.full_like(src, CANARY)
    store = B.Store(pool, dst, dst.nbytes, paths, threads=1)
    pool.release()
    store.request([0, 1], [[0, 0, 0, -1]])
    store.wait()
    assert store.stats()["pages_read"] == 1
    store.release()


def test_write_rejects_bad_arguments(tmp_path):
    wl = W.get("coinrag_small")
    m = _model(wl)
    buf = np.zeros((4, W.page_bytes(wl.model, 16)), np.uint8)
    with pytest.raises(B.PicError, match="power of two"):
        B.write_chunk_file(m, 12, 10, 0, buf, [0], str(tmp_path / "a.pic"))
    with pytest.raises(B.PicError, match="negative"):
        B.write_chunk_file(m, 16, 10, 0, buf, [-1], str(tmp_path / "a.pic"))
    with pytest.raises(B.PicError):
        B.write_chunk_file(m, 16, 10, 0, buf, [0], str(tmp_path / "no_such_dir" / "a.pic"))
    assert not (tmp_path / "a.pic").exists()


@pytest.fixture(scope="module")
def drivers(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    out = tmp_path_factory.mktemp("store_native")
    srcs = [os.path.join(CSRC, "pic_plan.cpp"), os.path.join(CSRC, "pic_store.cpp"),
            os.path.join(ROOT, "tests", "native", "store_stress.cpp")]
    common = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'include')}",
              f"-I{CSRC}", *srcs, "-pthread"]
    built = {}
    for name, flags in (("asan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]),
                        ("tsan", ["-fsanitize=thread"])):
        exe = str(out / name)
        res = subprocess.run(common + flags + ["-o", exe], capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        built[name] = exe
    return built, out


@pytest.mark.parametrize("kind,seed", [("asan", 1), ("asan", 2), ("tsan", 3), ("tsan", 4)])
def test_store_is_clean_under_sanitizers(drivers, kind, seed):
    """Random pools and page sets through the loader: AddressSanitizer +
    UndefinedBehaviorSanitizer, and ThreadSanitizer for the worker threads."""
    built, out = drivers
    folder = out / f"{kind}{seed}"
    folder.mkdir()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    res = subprocess.run([built[kind], str(folder), str(seed), "15"], capture_output=True, text=True, env=env,
                         timeout=300)
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-4000:])
    assert res.stdout.startswith("ok "), res.stdout
    assert int(res.stdout.split()[1]) > 20, "too few verified loads"
