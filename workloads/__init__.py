"""Seeded synthetic inputs for position-independent KV-cache reuse.

This module is shared by the tests, the benchmark and the smoke check.  It
holds no arithmetic of the method (no rotation, no position planning, no
attention): it only draws random layouts and values with the shapes and
distributions of the pages' workloads, builds a paged pool from them, and
counts algorithmic bytes and FLOPs for the reports.

Pool layouts use numpy's default_rng(1000 * cfg), request layouts
default_rng([1000 * cfg, 1 + layout]) (the tiny configuration: seed 0); large
tensors use a torch.Generator on the target device seeded from 1000 * cfg.
The oracle reads back the exact values that were generated.

Stand-ins for the pages' workloads (the public QA suites they evaluate on are
not used):
  * chunks of 512 tokens and top-5 retrieval (TurboRAG review page, the
    author's own serving anecdote; CoinRAG section 2.1);
  * nugget spans about 15 tokens long, 64 per request drawn from 20 retrieved
    chunks (CoinRAG section 3.1, Table 4: 11-13 words per nugget, hundreds of
    candidates per question);
  * document caches with inline request segments between them (SemPIC hit
    path);
  * long documents of 2048 tokens, 64 of them for a 131,072-token prefix.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

TARGET_AUTO = -1
TARGET_ORIGINAL = -2   # keep the span where it was encoded (composite positions)


# ---------------------------------------------------------------------------
# shapes
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class ModelShape:
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    theta: float
    dtype: str          # "bf16" or "f32"

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


@dataclass
class PoolSpec:
    """Chunk caches stored in fixed-size pages.

    Page p holds `page_tokens` tokens of one chunk, laid out
    [layer][K=0 / V=1][kv_head][token][head_dim].  Chunk c owns pages
    page_ids[chunk_page_ptr[c] : chunk_page_ptr[c+1]] in token order.
    """
    chunk_len: np.ndarray        # int32 [n_chunks]
    chunk_orig: np.ndarray       # int32 [n_chunks]
    page_tokens: int
    n_pages: int
    chunk_page_ptr: np.ndarray   # int32 [n_chunks + 1]
    page_ids: np.ndarray         # int32 [chunk_page_ptr[-1]]

    @property
    def n_chunks(self) -> int:
        return int(self.chunk_len.shape[0])


@dataclass
class Request:
    spans: np.ndarray                    # int32 [n_spans][4]: chunk, s, e (inclusive), target
    n_new: int
    new_pos: Optional[np.ndarray] = None  # explicit int32 [n_new] or None (follow the prefix)

    @property
    def prefix_rows(self) -> int:
        if len(self.spans) == 0:
            return 0
        return int(np.sum(self.spans[:, 2] - self.spans[:, 1] + 1))


@dataclass
class ValueRecipe:
    k_scale: str = "unit"        # "unit" | "lognormal" | "outlier"
    v_scale: str = "unit"        # "unit" | "half" | "outlier"
    q_scale: str = "unit"


@dataclass
class Workload:
    name: str
    cfg: int
    model: ModelShape
    pool: PoolSpec
    requests: List[Request]
    values: ValueRecipe
    seed: int
    notes: str = ""
    extra: Dict = field(default_factory=dict)
    keys: str = "rotated"        # "rotated" (at the original position) or "unrotated"

    @property
    def batch(self) -> int:
        return len(self.requests)

    @property
    def n_new_total(self) -> int:
        return int(sum(r.n_new for r in self.requests))

    @property
    def prefix_rows_total(self) -> int:
        return int(sum(r.prefix_rows for r in self.requests))

    @property
    def rows_total(self) -> int:
        return self.prefix_rows_total + self.n_new_total

    def span_ptr(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([len(r.spans) for r in self.requests])]).astype(np.int32)

    def spans_flat(self) -> np.ndarray:
        if not self.requests:
            return np.zeros((0, 4), np.int32)
        return np.concatenate([r.spans.reshape(-1, 4) for r in self.requests]).astype(np.int32)

    def new_ptr(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([r.n_new for r in self.requests])]).astype(np.int32)

    def new_pos_flat(self) -> Optional[np.ndarray]:
        if all(r.new_pos is None for r in self.requests):
            return None
        if any(r.new_pos is None for r in self.requests):
            raise ValueError("mixing explicit and implicit new positions in one batch")
        return np.concatenate([np.asarray(r.new_pos, np.int32) for r in self.requests]).astype(np.int32)


# ---------------------------------------------------------------------------
# pool layout
# ---------------------------------------------------------------------------

def make_pool(rng: np.random.Generator, chunk_len, page_tokens: int = 16,
              shuffle_pages: bool = True, spare_pages: int = 0) -> PoolSpec:
    """Give every chunk ceil(len / page_tokens) pages, in a shuffled page order."""
    chunk_len = np.asarray(chunk_len, dtype=np.int32)
    npg = (chunk_len + page_tokens - 1) // page_tokens
    ptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    n_pages = int(ptr[-1]) + spare_pages
    perm = rng.permutation(n_pages).astype(np.int32) if shuffle_pages else np.arange(n_pages, dtype=np.int32)
    return PoolSpec(chunk_len=chunk_len, chunk_orig=np.zeros_like(chunk_len), page_tokens=page_tokens,
                    n_pages=n_pages, chunk_page_ptr=ptr, page_ids=perm[:int(ptr[-1])].copy())


def page_bytes(model: ModelShape, page_tokens: int) -> int:
    return model.layers * 2 * model.kv_heads * page_tokens * model.head_dim * model.elem_bytes


# ---------------------------------------------------------------------------
# request layouts for the five workloads
# ---------------------------------------------------------------------------

def _spans(rows) -> np.ndarray:
    return np.asarray(rows, dtype=np.int32).reshape(-1, 4)


def _tiny(seed_base: int) -> Workload:
    """1 layer, 2 q heads / 1 kv head, d = 64, theta 1e4, fp32; 4 chunks of 64
    tokens plus an 8-token system-prompt cache; 6 nugget spans of length
    U[4, 16] inside random chunks; 8 query tokens; batch 1, seed 0."""
    rng = np.random.default_rng(seed_base)
    model = ModelShape(1, 2, 1, 64, 1e4, "f32")
    prompt = 4
    pool = make_pool(rng, [64, 64, 64, 64, 8], page_tokens=16)
    rows = [(prompt, 0, 7, 0)]
    for _ in range(6):
        c = int(rng.integers(0, 4))
        n = int(rng.integers(4, 17))
        s = int(rng.integers(0, 64 - n + 1))
        rows.append((c, s, s + n - 1, TARGET_AUTO))
    return Workload("tiny_f32", 1, model, pool, [Request(_spans(rows), 8)], ValueRecipe(), seed_base)


QWEN2_7B = ModelShape(28, 28, 4, 128, 1e6, "bf16")
LLAMA31_8B = ModelShape(32, 32, 8, 128, 5e5, "bf16")
QWEN3_8B = ModelShape(36, 32, 8, 128, 1e6, "bf16")


def _layout_rng(seed: int, layout: int) -> np.random.Generator:
    """Requests draw from their own stream so that layout variants share the pool."""
    return np.random.default_rng([seed, 1 + layout])


def _turborag(batch: int, model: ModelShape = QWEN2_7B, n_chunks: int = 200,
              chunk: int = 512, top: int = 5, prompt_len: int = 32, n_new: int = 64,
              name: str = "", layout: int = 0, keys: str = "rotated",
              positions: str = "reordered") -> Workload:
    """Whole-chunk reuse: a 32-token prompt cache and top-5 whole 512-token
    chunks out of 200, in retrieval order; 64 query tokens.  Reordered
    positions make the chunks contiguous; composite positions keep every chunk
    where it was encoded (each restarting at 0).  Keys are stored rotated at
    their original positions or un-rotated."""
    seed = 2000
    pool = make_pool(np.random.default_rng(seed), [chunk] * n_chunks + [prompt_len])
    rng = _layout_rng(seed, layout)
    prompt = n_chunks
    tgt = TARGET_ORIGINAL if positions == "composite" else TARGET_AUTO
    reqs = []
    for _ in range(batch):
        sel = rng.choice(n_chunks, size=top, replace=False)
        rows = [(prompt, 0, prompt_len - 1, 0)] + [(int(c), 0, chunk - 1, tgt) for c in sel]
        reqs.append(Request(_spans(rows), n_new))
    return Workload(name or f"turborag_b{batch}", 2, model, pool, reqs,
                    ValueRecipe("lognormal", "half"), seed, keys=keys)


def _nugget_spans(rng, chunks, n_spans, chunk_len, p_geom=1.0 / 15, lo=3, hi=48):
    """n_spans spans over the retrieved chunks: chunk uniform over them, length
    clip(Geom(p), lo, hi), start uniform among positions that do not overlap
    spans already placed in that chunk; the global order is shuffled."""
    taken = {int(c): np.zeros(chunk_len, dtype=bool) for c in chunks}
    out = []
    while len(out) < n_spans:
        c = int(rng.choice(chunks))
        n = int(np.clip(rng.geometric(p_geom), lo, hi))
        for _ in range(64):
            s = int(rng.integers(0, chunk_len - n + 1))
            if not taken[c][s:s + n].any():
                taken[c][s:s + n] = True
                out.append((c, s, s + n - 1))
                break
    order = rng.permutation(len(out))
    return [out[i] for i in order]


def _coinrag(batch: int, model: ModelShape = QWEN2_7B, n_chunks: int = 2000,
             chunk: int = 512, retrieved: int = 20, n_spans: int = 64,
             prompt_len: int = 32, n_new: int = 64, name: str = "", layout: int = 0,
             keys: str = "rotated") -> Workload:
    """Nugget reuse: 20 retrieved chunks per request, 64 non-overlapping spans
    with geometric lengths (mean 15, clipped to [3, 48]) in shuffled order,
    contiguous after a 32-token prompt cache; 64 query tokens."""
    seed = 3000
    pool = make_pool(np.random.default_rng(seed), [chunk] * n_chunks + [prompt_len])
    rng = _layout_rng(seed, layout)
    prompt = n_chunks
    reqs = []
    for _ in range(batch):
        sel = rng.choice(n_chunks, size=retrieved, replace=False)
        spans = _nugget_spans(rng, sel, n_spans, chunk)
        rows = [(prompt, 0, prompt_len - 1, 0)] + [(c, s, e, TARGET_AUTO) for c, s, e in spans]
        reqs.append(Request(_spans(rows), n_new))
    return Workload(name or f"coinrag_b{batch}", 3, model, pool, reqs,
                    ValueRecipe("lognormal", "half"), seed, keys=keys)


def _sempic(batch: int, model: ModelShape = LLAMA31_8B, n_docs: int = 64,
            doc_lo: int = 1024, doc_hi: int = 4096, per_req: int = 8,
            inline_lo: int = 64, inline_hi: int = 256, n_query: int = 128,
            name: str = "", layout: int = 0) -> Workload:
    """Document reuse with interleaving: 8 distinct documents per request in
    random order, 7 inline segments of U[64, 256] fresh tokens between them,
    a 128-token query last.  Every item gets its final logical position in
    sequence order; the inline tokens and the query are the new tokens."""
    seed = 4000
    prng = np.random.default_rng(seed)
    lens = prng.integers(doc_lo, doc_hi + 1, size=n_docs)
    pool = make_pool(prng, lens)
    rng = _layout_rng(seed, layout)
    reqs = []
    for _ in range(batch):
        docs = rng.choice(n_docs, size=per_req, replace=False)
        rows, new_pos, cursor = [], [], 0
        for i, dc in enumerate(docs):
            n = int(lens[dc])
            rows.append((int(dc), 0, n - 1, cursor))
            cursor += n
            m = int(rng.integers(inline_lo, inline_hi + 1)) if i + 1 < per_req else n_query
            new_pos.extend(range(cursor, cursor + m))
            cursor += m
        reqs.append(Request(_spans(rows), len(new_pos), np.asarray(new_pos, np.int32)))
    return Workload(name or f"sempic_b{batch}", 4, model, pool, reqs,
                    ValueRecipe("lognormal", "half"), seed)


def _long(batch: int, docs_per_req: int, model: ModelShape = QWEN3_8B, n_docs: int = 64,
          doc_len: int = 2048, n_new: int = 256, name: str = "", layout: int = 0) -> Workload:
    """Long context: 64 documents of 2048 tokens; each request takes
    `docs_per_req` of them in random order, contiguous; a 256-token query.
    K/V ~ N(0, 1) with 1% outlier channels scaled x20."""
    seed = 5000
    pool = make_pool(np.random.default_rng(seed), [doc_len] * n_docs)
    rng = _layout_rng(seed, layout)
    reqs = []
    for _ in range(batch):
        docs = rng.choice(n_docs, size=docs_per_req, replace=False)
        rows = [(int(dc), 0, doc_len - 1, TARGET_AUTO) for dc in docs]
        reqs.append(Request(_spans(rows), n_new))
    return Workload(name or f"long_{docs_per_req * doc_len}_b{batch}", 5, model, pool, reqs,
                    ValueRecipe("outlier", "outlier"), seed)


def get(name: str, layout: int = 0) -> Workload:
    """Named workloads: the five full-size configurations and reduced variants
    that the oracle finishes in seconds (same structure, fewer layers or
    requests).  `layout` draws a different batch of requests over the same
    pool (the tiny configuration has one layout)."""
    small2 = ModelShape(2, 28, 4, 128, 1e6, "bf16")
    small4 = ModelShape(2, 32, 8, 128, 5e5, "bf16")
    small5 = ModelShape(2, 32, 8, 128, 1e6, "bf16")
    table = {
        "tiny_f32": lambda: _tiny(0),
        "turborag_b1": lambda: _turborag(1, layout=layout),
        "turborag_b16": lambda: _turborag(16, layout=layout),
        # the TurboRAG review page's other two layouts: keys stored un-rotated
        # (RoPE applied at the new position), and composite positions
        "turborag_b16_unrot": lambda: _turborag(16, name="turborag_b16_unrot", layout=layout, keys="unrotated"),
        "turborag_b16_composite": lambda: _turborag(16, name="turborag_b16_composite", layout=layout,
                                                    positions="composite"),
        "coinrag_b32": lambda: _coinrag(32, layout=layout),
        "sempic_b8": lambda: _sempic(8, layout=layout),
        "long_131k_b1": lambda: _long(1, 64, name="long_131k_b1", layout=layout),
        "long_16k_b32": lambda: _long(32, 8, name="long_16k_b32", layout=layout),
        # reduced variants
        "turborag_small": lambda: _turborag(3, small2, n_chunks=12, name="turborag_small", layout=layout),
        "coinrag_small": lambda: _coinrag(4, small2, n_chunks=40, name="coinrag_small", layout=layout),
        "turborag_small_unrot": lambda: _turborag(3, small2, n_chunks=12, name="turborag_small_unrot",
                                                  layout=layout, keys="unrotated"),
        "coinrag_small_unrot": lambda: _coinrag(4, small2, n_chunks=40, name="coinrag_small_unrot",
                                                layout=layout, keys="unrotated"),
        "turborag_small_composite": lambda: _turborag(3, small2, n_chunks=12, name="turborag_small_composite",
                                                      layout=layout, positions="composite"),
        "sempic_small": lambda: _sempic(2, small4, n_docs=6, doc_lo=100, doc_hi=700, per_req=3,
                                        inline_lo=20, inline_hi=90, n_query=40, name="sempic_small",
                                        layout=layout),
        "long_small": lambda: _long(2, 2, small5, n_docs=4, doc_len=1000, n_new=100, name="long_small",
                                    layout=layout),
    }
    for b in (1, 2, 4, 8, 16):
        table[f"long_16k_b{b}"] = (lambda b=b: _long(b, 8, name=f"long_16k_b{b}", layout=layout))
    if name not in table:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(table)}")
    return table[name]()


FULL_SIZE = ("tiny_f32", "turborag_b1", "turborag_b16", "coinrag_b32", "sempic_b8",
             "long_131k_b1", "long_16k_b32")
REDUCED = ("turborag_small", "coinrag_small", "sempic_small", "long_small")
REDUCED_NEXT = ("turborag_small_unrot", "coinrag_small_unrot", "turborag_small_composite")


# ---------------------------------------------------------------------------
# values (torch; on any device)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def torch_dtype(model: ModelShape):
    torch = _torch()
    return torch.bfloat16 if model.dtype == "bf16" else torch.float32


def _generator(device, seed: int):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def channel_scales(wl: Workload, device):
    """Per-(layer, kv head, channel) scales for keys and values (fp32).

    lognormal: exp(N(0, 0.5^2)); outlier: x20 with probability 0.01, else 1;
    half: 0.5; unit: 1.  Keys and values draw independently.
    """
    torch = _torch()
    m = wl.model
    g = _generator(device, wl.seed * 7 + 1)
    shape = (m.layers, m.kv_heads, m.head_dim)

    def draw(kind):
        if kind == "unit":
            return torch.ones(shape, device=device)
        if kind == "half":
            return torch.full(shape, 0.5, device=device)
        if kind == "lognormal":
            return torch.exp(0.5 * torch.randn(shape, generator=g, device=device))
        if kind == "outlier":
            u = torch.rand(shape, generator=g, device=device)
            return torch.where(u < 0.01, torch.full_like(u, 20.0), torch.ones_like(u))
        raise ValueError(kind)

    return draw(wl.values.k_scale), draw(wl.values.v_scale)


def alloc_pool(wl: Workload, device):
    """Uninitialised pool tensor [n_pages][L][2][Hkv][page_tokens][d]."""
    torch = _torch()
    m, p = wl.model, wl.pool
    return torch.empty((p.n_pages, m.layers, 2, m.kv_heads, p.page_tokens, m.head_dim),
                       dtype=torch_dtype(m), device=device)


def fill_pool(wl: Workload, pool, kscale, vscale, pages_per_block: int = 512):
    """Fill every page with N(0, 1) values times the channel scales.

    Stored keys are drawn directly in their stored (already rotated) form;
    the generator applies no rotation.
    """
    torch = _torch()
    m = wl.model
    g = _generator(pool.device, wl.seed * 7 + 2)
    scale = torch.stack([kscale, vscale], dim=1)[None, :, :, :, None, :]   # [1][L][2][Hkv][1][d]
    for p0 in range(0, pool.shape[0], pages_per_block):
        p1 = min(pool.shape[0], p0 + pages_per_block)
        x = torch.randn((p1 - p0,) + tuple(pool.shape[1:]), generator=g, device=pool.device,
                        dtype=torch.float32)
        pool[p0:p1] = (x * scale).to(pool.dtype)
    return pool


def new_tokens(wl: Workload, layer: int, kscale, vscale, device):
    """Un-rotated q [n][Hq][d], k_new [n][Hkv][d], v_new [n][Hkv][d] for one layer,
    all requests packed in request order."""
    torch = _torch()
    m = wl.model
    n = wl.n_new_total
    g = _generator(device, wl.seed * 7 + 1000 + layer)
    dt = torch_dtype(m)
    q = torch.randn((n, m.q_heads, m.head_dim), generator=g, device=device)
    k = torch.randn((n, m.kv_heads, m.head_dim), generator=g, device=device) * kscale[layer][None]
    v = torch.randn((n, m.kv_heads, m.head_dim), generator=g, device=device) * vscale[layer][None]
    return q.to(dt), k.to(dt), v.to(dt)


def decode_tokens(wl: Workload, layer: int, step: int, kscale, vscale, device):
    """Un-rotated q [batch][Hq][d], k [batch][Hkv][d], v [batch][Hkv][d] of decode
    step `step` (one token per request) for one layer."""
    torch = _torch()
    m = wl.model
    n = wl.batch
    g = _generator(device, wl.seed * 7 + 500000 + 1000 * step + layer)
    dt = torch_dtype(m)
    q = torch.randn((n, m.q_heads, m.head_dim), generator=g, device=device)
    k = torch.randn((n, m.kv_heads, m.head_dim), generator=g, device=device) * kscale[layer][None]
    v = torch.randn((n, m.kv_heads, m.head_dim), generator=g, device=device) * vscale[layer][None]
    return q.to(dt), k.to(dt), v.to(dt)


def chunk_kv(wl: Workload, pool, c: int, layers=None):
    """Read chunk c's stored K and V back out of the pages: two CPU float64
    tensors [L'][Hkv][len][d] (L' = the selected layers)."""
    torch = _torch()
    p = wl.pool
    ids = torch.as_tensor(p.page_ids[p.chunk_page_ptr[c]:p.chunk_page_ptr[c + 1]].astype(np.int64),
                          device=pool.device)
    pages = pool.index_select(0, ids)                      # [np][L][2][Hkv][P][d]
    if layers is not None:
        pages = pages[:, list(layers)]
    npg, nl, _, hkv, pt, d = pages.shape
    x = pages.permute(1, 2, 3, 0, 4, 5).reshape(nl, 2, hkv, npg * pt, d)[:, :, :, :int(p.chunk_len[c])]
    x = x.to("cpu").to(torch.float64)
    return x[:, 0].contiguous(), x[:, 1].contiguous()


# ---------------------------------------------------------------------------
# accounting (algorithmic work, for the reports)
# ---------------------------------------------------------------------------

def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of cached K and V for one token over all layers: 2 * L * Hkv * d * s."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def assembly_bytes(wl: Workload) -> int:
    """Gather + rotate moves every prefix row of every layer and head once in
    and once out, K and V: rows * 2 * L * Hkv * d * s * 2."""
    m = wl.model
    return wl.prefix_rows_total * kv_bytes_per_token(m.layers, m.kv_heads, m.head_dim, m.elem_bytes) * 2


def visible_pairs(wl: Workload) -> int:
    """Sum over new tokens of the number of rows (cached and new) each one may
    attend to.  Contiguous layouts: every prefix row plus the causal part of
    the new rows; explicit layouts: counted from the explicit positions."""
    total = 0
    for r in wl.requests:
        n = r.n_new
        if r.new_pos is None:
            total += n * r.prefix_rows + n * (n + 1) // 2
            continue
        if np.any(r.spans[:, 3] < 0):
            raise ValueError("explicit new positions need explicit span targets")
        rows = np.concatenate([np.arange(t, t + e - s + 1) for _, s, e, t in r.spans] +
                              [np.asarray(r.new_pos, np.int64)])
        rows.sort()
        total += int(np.searchsorted(rows, np.asarray(r.new_pos, np.int64), side="right").sum())
    return total


def attention_flops(wl: Workload, layers: Optional[int] = None) -> int:
    """4 * d * Hq * L * visible pairs (QK^T and PV multiply-adds, 2 FLOPs each)."""
    m = wl.model
    nl = m.layers if layers is None else layers
    return 4 * m.head_dim * m.q_heads * nl * visible_pairs(wl)
