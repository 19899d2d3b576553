/*
 * pic.h - position-independent KV-cache reuse on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpic.so.  Plain pointers and sizes only.  Every device buffer is
 * owned by the caller; the library owns only its opaque handles and their
 * device-side planning tables.  All GPU work is enqueued on the stream the
 * caller passes (a hipStream_t given as void*, NULL = the default stream);
 * the library never synchronises the device implicitly except where a call's
 * comment says so.
 *
 * Terms (the pages' notation):
 *   chunk c     a document or chunk whose per-layer K/V cache C_c was computed
 *               offline, tokens 0 .. len_c-1 (CoinRAG page, section 2.1: one
 *               forward pass of the whole chunk; TurboRAG review page,
 *               pipeline of Figure 3-b; SemPIC page: compiled document caches).
 *   span        (c, s, e, target): the tokens s..e (e INCLUSIVE) of chunk c,
 *               placed so that token s lands at position `target` (CoinRAG
 *               page, section 2.2: retrieval returns (b_i, s_i, e_i); section
 *               2.3: Rot(C_b[s:e]; Delta_i) concatenated into C_ctx).
 *   prefix      the spans of one request gathered in table order (C_ctx).
 *   new tokens  the request's fresh tokens (query, inline segments) that are
 *               prefilled against the prefix: KV_M(q; C_ctx).
 *
 * Conventions: positions are 0-based.  RoPE is the standard half-split form
 * (pairs (k, k + d/2), omega_k = theta^(-2k/d)).  Cached keys are stored
 * either rotated at their original position orig_c + t (PIC_KEYS_ROTATED: the
 * CoinRAG and SemPIC pages' caches) or before RoPE (PIC_KEYS_UNROTATED: the
 * TurboRAG review page's alternative, Reordered Positions paragraph).  A span
 * placed at `target` rotates each rotated key by delta = target - (orig_c + s)
 * (the same for the whole span), or each un-rotated key by its new position
 * target + t; values are copied.  A new token at
 * position P sees every row, cached or new, whose position is <= P: this is
 * the TurboRAG review page's independent attention (Figure 4: the query sees
 * all chunks and itself, chunks never see each other) and the SemPIC page's
 * causal interleave of compiled and inline caches.
 *
 * Errors: every call validates its arguments on the host before it enqueues
 * anything; on an error nothing is written and a message is available from
 * pic_last_error() (thread-local, valid until the next call on that thread).
 * A failure reported by the HIP runtime after a launch returns PIC_EDEVICE and
 * leaves the plan unusable (PIC_ESTATE afterwards).
 */
#ifndef PIC_H
#define PIC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PIC_OK = 0,
  PIC_EINVAL = -1,       /* malformed argument (null pointer, bad shape, bad table) */
  PIC_ERANGE = -2,       /* index or size out of range (chunk id, span bounds, capacity) */
  PIC_ENOMEM = -3,       /* host or device allocation for library-owned tables failed */
  PIC_EDEVICE = -4,      /* the HIP runtime reported an error */
  PIC_ESTATE = -5,       /* handle in the wrong state (released, not assembled, failed) */
  PIC_EALIGN = -6,       /* a device pointer is not 16-byte aligned */
  PIC_EUNSUPPORTED = -7, /* valid request this build does not implement */
  PIC_EIO = -8           /* reading or writing a chunk file failed */
} pic_status;

typedef enum { PIC_F32 = 0, PIC_BF16 = 1 } pic_dtype;

/* How the pool stores keys. */
typedef enum {
  PIC_KEYS_ROTATED = 0,   /* RoPE already applied at the original position orig_c + t */
  PIC_KEYS_UNROTATED = 1  /* raw keys; RoPE is applied at the new position on assembly */
} pic_key_storage;

/* Model shape.  head_dim even, a multiple of 16, at most 256; q_heads a
 * multiple of kv_heads (query head h reads kv head h / (q_heads / kv_heads)). */
typedef struct {
  int32_t layers;
  int32_t q_heads;
  int32_t kv_heads;
  int32_t head_dim;
  double rope_theta;
  int32_t dtype;          /* pic_dtype: storage and I/O type of every tensor */
  int32_t key_storage;    /* pic_key_storage of the pool's keys (0 = rotated) */
} pic_model;

/* One span of a request's span table.  e is inclusive.  target is the new
 * position of token s, or
 *   PIC_TARGET_AUTO:     right after the previous span of the same request
 *                        (0 for the first).  With the prompt cache as span 0
 *                        and every other span AUTO this is CoinRAG's
 *                        Delta_i = |p| + sum_{j<i}(e_j-s_j+1) (section 2.3,
 *                        Delta equation; TurboRAG's Reordered Positions);
 *   PIC_TARGET_ORIGINAL: where the span was encoded, orig_c + s (delta 0):
 *                        TurboRAG's Composite Positions (Figure 5), every
 *                        chunk restarting at its own base. */
typedef struct {
  int32_t chunk;
  int32_t s;
  int32_t e;
  int32_t target;
} pic_span;

#define PIC_TARGET_AUTO (-1)
#define PIC_TARGET_ORIGINAL (-2)

/* pic_assemble flags */
#define PIC_ASSEMBLE_PLAN_ONLY 1     /* plan on host and device, gather nothing (variant F) */
#define PIC_ASSEMBLE_DRY_RUN   2     /* validate and plan on the host only; touch no device */
#define PIC_ASSEMBLE_DEFER_GATHER 4  /* plan now; gather layers later with pic_gather_layers */
#define PIC_ASSEMBLE_QUERY_ROTATION 8  /* retired: refused with PIC_EUNSUPPORTED (see pic_query_prefill) */
#define PIC_ASSEMBLE_VALUES_IN_POOL 16 /* gather keys only; prefix values are read in the pool (below) */

/* pic_query_prefill variants */
#define PIC_VARIANT_MATERIALIZED 0  /* read keys/values from the assembled buffers */
#define PIC_VARIANT_FUSED        1  /* read cached rows from the pool, rotating on load (below) */

typedef struct pic_pool pic_pool;
typedef struct pic_plan pic_plan;

/*
 * Register a paged chunk-KV pool that already lives in device memory.
 *
 * Layout of `pool` (device, caller-owned, never copied or freed): n_pages
 * pages of page_bytes = layers * 2 * kv_heads * page_tokens * head_dim * s
 * bytes each (s = 2 for bf16, 4 for f32); inside a page
 * [layer][0 = K, 1 = V][kv_head][token slot][head_dim], row-major.
 * Token t of chunk c is in page page_ids[chunk_page_ptr[c] + t / page_tokens]
 * at slot t % page_tokens.
 *
 *   model          shape and dtype (copied)
 *   pool           device base pointer, 16-byte aligned
 *   pool_bytes     size of the allocation, >= n_pages * page_bytes
 *   page_tokens    tokens per page, a power of two in [1, 4096]
 *   n_pages        number of pages in the allocation
 *   n_chunks       number of chunk caches
 *   chunk_len      host int32[n_chunks], each >= 0
 *   chunk_orig     host int32[n_chunks] original base positions, or NULL (all 0)
 *   chunk_page_ptr host int32[n_chunks + 1], CSR offsets into page_ids, starting
 *                  at 0, non-decreasing, with room for ceil(len_c / page_tokens)
 *                  pages per chunk
 *   page_ids       host int32[chunk_page_ptr[n_chunks]], each in [0, n_pages)
 *   out            receives the handle
 * The host tables are copied; device copies are made on first use.
 */
pic_status pic_pool_register(const pic_model* model, void* pool, int64_t pool_bytes,
                             int32_t page_tokens, int32_t n_pages, int32_t n_chunks,
                             const int32_t* chunk_len, const int32_t* chunk_orig,
                             const int32_t* chunk_page_ptr, const int32_t* page_ids,
                             pic_pool** out);

/*
 * The same for a pool that lives in pinned host memory (hipHostMalloc): the
 * staging tier in front of HBM.  Assembly then reads only the rows the spans
 * cover, over the host link (CoinRAG page section 3.3 loads only the
 * selected slices; the TurboRAG review page's batch-scaling discussion names
 * this transfer as the cost that remains).  Combined with
 * PIC_ASSEMBLE_DEFER_GATHER and pic_gather_layers on a second stream, layer
 * l + 1 is transferred while layer l's attention runs.  PIC_EINVAL if `pool`
 * is not pinned host memory.  Needs a device (it asks the runtime for the
 * memory's device address).
 */
pic_status pic_pool_register_host(const pic_model* model, void* pool, int64_t pool_bytes,
                                  int32_t page_tokens, int32_t n_pages, int32_t n_chunks,
                                  const int32_t* chunk_len, const int32_t* chunk_orig,
                                  const int32_t* chunk_page_ptr, const int32_t* page_ids,
                                  pic_pool** out);

/* Release a pool handle (not the pool memory).  Plans made from it, and its
 * hot set, must be released first (PIC_ESTATE otherwise).  Synchronises the
 * device if device tables were made. */
pic_status pic_pool_release(pic_pool* pool);

/*
 * HBM-resident hot set in front of a pool in pinned host memory.  Pages the
 * batches cover are copied from the host into `capacity_pages` page slots of
 * device memory (capacity_pages x the pool's page size, allocated here) the
 * first time they are needed, and stay until evicted: least recently used
 * first, never while a plan's current batch covers them.  A batch whose
 * chunks are resident then assembles at HBM speed instead of streaming its
 * rows over the host link; only the pages that cover a batch's spans move
 * (the TurboRAG review page, its batch-scaling paragraph and its critique
 * section, caching high-frequency chunks near the GPU; the CoinRAG page
 * section 3.3, loading only the selected token ranges).
 *
 * After pic_cache_create, pic_assemble on any plan over the pool pins the
 * pages the batch's spans cover (evicting as needed) and points the batch at
 * the hot set: PIC_ERANGE, with nothing changed, if they do not fit beside
 * the pages other plans' batches pin.  A page's data moves one layer at a
 * time, just before the first call that reads that layer of it: the layer's
 * gather (pic_assemble, pic_gather_layers) or, when attention reads the pool
 * itself (variant F, PIC_ASSEMBLE_VALUES_IN_POOL), pic_query_prefill and
 * pic_decode_layer.  With deferred gathers on a second stream, layer l + 1's
 * pages therefore move while layer l's attention runs.  The copies are
 * enqueued on the calling stream, and are timed as the assembly gather
 * (pic_timing_read kernel 0).
 *
 * The pool must be registered with pic_pool_register_host (PIC_EINVAL
 * otherwise), have no plans yet and no hot set (PIC_ESTATE), and
 * capacity_pages must be >= 1 (PIC_EINVAL); PIC_ENOMEM if the device memory
 * cannot be allocated.  Plans sharing a pool with a hot set must not run
 * calls concurrently on different streams: one plan's pic_assemble may evict
 * and overwrite pages that another plan's earlier, still running, calls read
 * (calls on one stream, or synchronised between, are safe).
 */
typedef struct pic_cache pic_cache;

typedef struct {
  int64_t capacity_pages;   /* page slots */
  int64_t resident_pages;   /* slots holding a page */
  int64_t hits;             /* page look-ups by pic_assemble that found the page resident */
  int64_t misses;           /* ... that admitted it */
  int64_t evictions;        /* pages evicted to admit others */
  int64_t layer_copies;     /* page-layer slices copied from the host */
  int64_t bytes_copied;     /* bytes those copies moved */
} pic_cache_stats;

pic_status pic_cache_create(pic_pool* pool, int32_t capacity_pages, pic_cache** out);

/* Counters since the hot set was created. */
pic_status pic_cache_get_stats(const pic_cache* cache, pic_cache_stats* out);

/* Release the hot set and its device memory.  The plans over its pool must
 * be released first (PIC_ESTATE otherwise).  Synchronises the device. */
pic_status pic_cache_release(pic_cache* cache);

/*
 * Chunk files: the storage tier behind a pool in host memory.  Each chunk's
 * cache is one file, and only the pages that a batch's spans cover are read,
 * per chunk by a pool of host threads (the CoinRAG page, section 3.3: one
 * cache file per chunk on NVMe, loaded asynchronously per document, only the
 * selected token ranges).
 *
 * File layout (little-endian): a 4096-byte header (magic "PICCHUNK", version
 * 1, the model shape, page_tokens, len, orig, page_bytes, page count), then
 * the chunk's ceil(len / page_tokens) pages in the pool's page layout (see
 * pic_pool_register), page j at byte offset 4096 + j * page_bytes.
 *
 * pic_chunk_file_write writes one such file for a chunk of `len` tokens
 * encoded at original position `orig`: page j is copied from host memory at
 * pages + page_list[j] * page_bytes (page_list: host int32[ceil(len /
 * page_tokens)], each >= 0; the caller guarantees the memory is there).  The
 * file is created or truncated, and flushed to the device before the call
 * returns; on a failure it is removed.  PIC_EINVAL / PIC_ERANGE for bad
 * arguments, PIC_EIO if the file cannot be written.
 */
pic_status pic_chunk_file_write(const pic_model* model, int32_t page_tokens, int32_t len, int32_t orig,
                                const void* pages, const int32_t* page_list, const char* path);

/*
 * Open the files of a pool's chunks (paths: host array of n_chunks paths,
 * copied) to be loaded into `dst`, host memory of dst_bytes >= n_pages *
 * page_bytes laid out like the pool (page p at dst + p * page_bytes; the
 * memory stays the caller's).  Every header is checked against the pool
 * (model, page size, the chunk's length and origin) and every file's size
 * against its pages: PIC_EINVAL or PIC_EIO naming the file otherwise.  The
 * chunk pages the files back must be distinct pool pages (PIC_EINVAL).
 * `threads` (1..256) host threads do the reads.  No page counts as loaded
 * after opening.
 *
 * When `dst` is the pool's own memory and the pool was registered with
 * pic_pool_register_host, the store is attached to the pool: from then on
 * pic_assemble reads the pages its batch covers that are not loaded yet,
 * and returns only once they are in host memory (PIC_EIO, with nothing
 * enqueued, if a read fails), so every later reader (gathers over the host
 * link, the hot set's copies, attention reading the pool) finds them.  At
 * most one store is attached to a pool, before the pool's plans are created
 * (PIC_ESTATE otherwise); the pool cannot be released while it is attached.
 * A store over a pool in device memory fills a separate host buffer and is
 * not attached (dst equal to the device pool's own pointer is PIC_EINVAL).
 * None of the store calls touch the device.
 */
typedef struct pic_store pic_store;

typedef struct {
  int64_t resident_pages;   /* pages loaded and not forgotten */
  int64_t requested;        /* covered pages named by requests (pic_store_request, pic_assemble) */
  int64_t hits;             /* ... that were loaded or being loaded already */
  int64_t pages_read;       /* pages read from the files */
  int64_t bytes_read;       /* bytes those reads moved */
  int64_t reads;            /* vectored read calls (one per run of consecutive pages of a file) */
  double wait_seconds;      /* time callers were blocked waiting for loads */
} pic_store_stats;

pic_status pic_store_open(pic_pool* pool, void* dst, int64_t dst_bytes, const char* const* paths,
                          int32_t threads, pic_store** out);

/* Start loading the pages that a batch's spans cover (span_ptr: host
 * int32[batch + 1], spans: host pic_span[span_ptr[batch]], validated as
 * pic_assemble validates them; targets are not used) and return at once.
 * Pages loaded or being loaded are not read again.  Lets a caller read the
 * next batch's pages while the current batch runs. */
pic_status pic_store_request(pic_store* store, int32_t batch, const int32_t* span_ptr, const pic_span* spans);

/* Block until every requested load has finished.  PIC_EIO with the first
 * read error since the previous wait; the pages of a failed read stay
 * unloaded (a later request tries them again). */
pic_status pic_store_wait(pic_store* store);

/* Wait for the loads in flight, then count every page as not loaded, so the
 * next requests read them again; with drop_os_cache != 0, also ask the OS to
 * drop the files' cached pages (posix_fadvise DONTNEED), so those reads come
 * from the device.  The caller must make sure no device work still reads
 * the pool's pages (pages are rewritten with the same bytes). */
pic_status pic_store_forget(pic_store* store, int32_t drop_os_cache);

pic_status pic_store_get_stats(pic_store* store, pic_store_stats* out);

/* Wait for the loads in flight and release the store (not `dst`).  An
 * attached store needs the pool's plans released first (PIC_ESTATE). */
pic_status pic_store_release(pic_store* store);

/* Create a plan object for batches over `pool`.  Its host and device tables
 * grow on demand and are reused by later pic_assemble calls. */
pic_status pic_plan_create(pic_pool* pool, pic_plan** out);

/* Release a plan and its tables.  Synchronises the device. */
pic_status pic_plan_release(pic_plan* plan);

/*
 * Plan a batch and gather its prefixes (CoinRAG section 2.3, the C_ctx
 * equation; TurboRAG's Reordered Positions; SemPIC's hit path: assign final
 * logical positions and re-rotate the cached keys).
 *
 *   batch          number of requests (>= 0)
 *   span_ptr       host int32[batch + 1], CSR offsets into spans (from 0)
 *   spans          host pic_span[span_ptr[batch]]; 0 <= s <= e < len_chunk;
 *                  explicit targets >= 0; every position must fit int32
 *   new_ptr        host int32[batch + 1], CSR offsets of the new tokens
 *   new_pos        host int32[new_ptr[batch]] explicit positions, strictly
 *                  increasing within a request, or NULL: the new tokens of a
 *                  request then follow its whole prefix, P_j = max(sum of
 *                  span lengths, furthest span end target_i + len_i) + j
 *                  (for a contiguous prefix of n rows: n + j; TurboRAG Figure
 *                  5 also puts the query after the concatenated chunks when
 *                  their positions restart)
 *   asm_k, asm_v   device buffers [layers][kv_heads][asm_rows_capacity][head_dim]
 *                  of the model dtype, 16-byte aligned (may be NULL with DRY_RUN)
 *   asm_rows_capacity  rows per (layer, kv head) plane
 *   flags          0, PIC_ASSEMBLE_PLAN_ONLY,
 *                  PIC_ASSEMBLE_DRY_RUN or PIC_ASSEMBLE_DEFER_GATHER; 0 and
 *                  DEFER_GATHER may add PIC_ASSEMBLE_VALUES_IN_POOL (bf16,
 *                  head_dim 128): the gather then writes keys only, leaves
 *                  the prefix rows of asm_v untouched, and the materialised
 *                  variant (prefill and decode) copies the prefix values
 *                  from the pool pages as it streams them (a value is moved
 *                  unchanged, so the results are the same bits); new-token
 *                  values are still appended to asm_v
 *   stream         hipStream_t
 *
 * Row layout: request b owns rows [row_base_b, row_base_b + prefix_b + n_new_b)
 * of every plane, row_base_b = sum over earlier requests of (prefix + n_new).
 * Its prefix rows come first in span-table order (span i, token s_i + t at
 * row row_base_b + sum_{j<i} n_j + t), followed by the new tokens' rows, which
 * pic_query_prefill fills layer by layer.  Prefix keys are rotated (by their
 * span's delta, or for un-rotated pools by their new position) in fp64
 * arithmetic with fp64 cos/sin, and rounded once, to nearest even, to the
 * storage type; a rotation by 0 is a bit copy, as are all values.  Overlapping or repeated spans are legal and gathered as
 * often as they appear.  The call replaces the plan's previous batch.
 */
pic_status pic_assemble(pic_plan* plan, int32_t batch, const int32_t* span_ptr,
                        const pic_span* spans, const int32_t* new_ptr, const int32_t* new_pos,
                        void* asm_k, void* asm_v, int64_t asm_rows_capacity, int32_t flags,
                        void* stream);

/*
 * Gather layers [layer_begin, layer_end) of the current batch into the
 * assembled planes on `stream` (after an assemble with
 * PIC_ASSEMBLE_DEFER_GATHER; re-gathering is allowed).  The stream first
 * waits for the batch's plan kernels.  A later pic_query_prefill or
 * pic_decode_layer (variant M) of such a layer, on any stream, waits for this
 * gather to complete, so an engine can gather layer l + 1 on one stream while
 * layer l's attention runs on another (the per-layer dependency of a real
 * prefill: each layer's KV_M needs that layer's C_ctx only).
 */
pic_status pic_gather_layers(pic_plan* plan, int32_t layer_begin, int32_t layer_end, void* stream);

/*
 * One layer of the query prefill, KV_M(q; C_ctx) (CoinRAG section 2.3, last
 * equation; TurboRAG: only the query is prefilled online; SemPIC: inline
 * tokens run through the decoder and interleave with compiled caches under a
 * causal mask).
 *
 *   layer      in [0, layers)
 *   q          device [n_new_total][q_heads][head_dim], un-rotated
 *   k_new      device [n_new_total][kv_heads][head_dim], un-rotated
 *   v_new      device [n_new_total][kv_heads][head_dim]
 *   out        device [n_new_total][q_heads][head_dim]
 *   variant    PIC_VARIANT_MATERIALIZED or PIC_VARIANT_FUSED
 * New tokens are packed in request order (new_ptr of the assemble call).
 * Steps: rotate q and k_new to the tokens' positions (fp64 arithmetic, one
 * rounding to the storage type); write k' and v_new into the new-token rows of this layer's
 * assembled planes (so the planes hold C_ctx (+) KV_M(q; C_ctx) for decoding);
 * then for every new token j and query head h
 *   out[j][h] = sum_r softmax_r(<q'_j,h, k_r> / sqrt(d)) v_r
 * over the request's rows r with pos_r <= pos_j.  Variant FUSED reads the
 * prefix rows straight from the pool (its plan may come from PLAN_ONLY) and
 * is implemented for bf16 with head_dim 128.  It applies each span's
 * re-rotation R(delta) on load: each key is rotated in registers (fp64
 * arithmetic, one rounding), so the scores equal variant M's bit for bit.
 * (Scoring instead against queries rotated back by delta, since
 * <q', R(delta) k> = <R(-delta) q', k>, would skip the rounding of each
 * re-rotated key to the storage type and so not reproduce the assembled
 * cache; PIC_ASSEMBLE_QUERY_ROTATION, which asked for it, is refused.)
 * MATERIALIZED needs the layer gathered (a full assemble, or
 * pic_gather_layers after a deferred one).  bf16 attention uses bf16 MFMA products with fp32 accumulation
 * and an fp32 online softmax; f32 attention computes in fp32.
 */
pic_status pic_query_prefill(pic_plan* plan, int32_t layer, const void* q, const void* k_new,
                             const void* v_new, void* out, int32_t variant, void* stream);

/*
 * pic_query_prefill for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same steps, kernels and results (bit for bit) as
 * pic_query_prefill, with the same arguments and the same plan: the plan's
 * tables come from its pic_assemble, and the call's own scratch (the rotated
 * queries, the row-split partials and their merge counters) is taken from a
 * fixed device array of 128 MiB that the library holds on each device it
 * runs on, from its load until the process ends, instead of from the plan's
 * workspace.  The call allocates nothing (no hipMalloc, hipFree or event
 * creation; it records no kernel-timing events) and clears the merge
 * counters with a kernel, not a memset.
 *   PIC_ERANGE   the batch needs more than 128 MiB of scratch (about
 *                new_rows * q_heads * head_dim * 2 bytes in bf16, plus
 *                row-split partials); nothing is enqueued.
 * Every call on a device shares that device's array and leaves its
 * contents behind: calls that overlap on one device (two streams, two
 * threads, two plans) race and must be ordered by the caller.
 * With a hot set in front of a host pool (pic_cache_create), the FUSED
 * variant and plans assembled with PIC_ASSEMBLE_VALUES_IN_POOL copy the
 * layer's missing pages first, as pic_query_prefill does: that uploads a
 * copy list from the hot set's pinned staging and may wait on the host for
 * the previous list of the same layer, so such calls are not fit for graph
 * capture (they still allocate nothing).
 */
pic_status pic_query_prefill_noalloc(pic_plan* plan, int32_t layer, const void* q, const void* k_new,
                                     const void* v_new, void* out, int32_t variant, void* stream);

/*
 * Decode over the assembled cache (the step after the prefill: ordinary
 * autoregressive decoding; CoinRAG page section 2.3 after KV_M(q; C_ctx),
 * SemPIC page's hit path).
 *
 * pic_plan_set_decode_rows reserves `rows` assembled rows after each
 * request's new tokens at the NEXT pic_assemble (0 by default).  The row
 * layout becomes: request b owns rows [row_base_b, row_base_b + prefix_b +
 * n_new_b + rows), row_base_b = sum over earlier requests of (prefix + n_new
 * + rows); asm_rows_capacity must cover the reserve.
 */
pic_status pic_plan_set_decode_rows(pic_plan* plan, int32_t rows);

/*
 * One decode step of one layer: every request of the batch gets one token.
 *   layer     in [0, layers)
 *   step      0-based decode index, in [0, reserved rows).  The token of
 *             request b sits at position last_b + 1 + step (last_b: the
 *             largest position among the request's spans and new tokens; -1
 *             if it has none) and at assembled row prefix_b + n_new_b + step.
 *   q         device [batch][Hq][head_dim], un-rotated
 *   k_new     device [batch][Hkv][head_dim], un-rotated
 *   v_new     device [batch][Hkv][head_dim]
 *   out       device [batch][Hq][head_dim]
 *   variant   PIC_VARIANT_MATERIALIZED or PIC_VARIANT_FUSED (prefix rows
 *             straight from the pool; works after a PLAN_ONLY assemble)
 * Steps: rotate q and k_new to the token's position (fp64, one rounding),
 * write k' and v_new at the token's row of this layer's planes, then
 *   out[b][h] = sum_r softmax_r(<q'_b,h, k_r> / sqrt(d)) v_r
 * over all of request b's rows up to and including the token (every earlier
 * row has a smaller position).  The rows are split across workgroups
 * (split-KV) and merged by log-sum-exp.  When one request's query heads of
 * a kv head fit one wavefront (Hq / Hkv <= 32) the attention kernel does the
 * rotation, the writes and the token's own score itself; the bits of k', of
 * the rows written and of every output are the same either way for a given
 * variant pair (M and F agree bit for bit).  Requires that this layer was
 * prefilled (pic_query_prefill) and decoded for steps 0 .. step-1 of the
 * current batch, in order.  Implemented for bf16 with head_dim 128
 * (PIC_EUNSUPPORTED otherwise).
 */
pic_status pic_decode_layer(pic_plan* plan, int32_t layer, int32_t step, const void* q, const void* k_new,
                            const void* v_new, void* out, int32_t variant, void* stream);

/* Host-side description of the plan's current batch. */
typedef struct {
  int32_t batch;
  int32_t n_spans;
  int64_t prefix_rows;     /* sum of span lengths */
  int64_t new_rows;        /* new_ptr[batch] */
  int64_t rows;            /* prefix_rows + new_rows: rows used in each plane */
  int32_t max_position;    /* largest position of any row */
  int32_t materialized;    /* 1 if the prefix rows were gathered */
  int32_t fused_query_rotation;  /* always 0: query rotation is retired (kept for the layout) */
  int32_t values_in_pool;  /* 1 if the batch was assembled with PIC_ASSEMBLE_VALUES_IN_POOL */
  int32_t attention_items;       /* bf16 attention work items (0 for other models) */
  int32_t attention_workgroups;  /* entries of the paired kernel's launch order */
  int32_t attention_item_workgroups;  /* entries of the one-item kernel's launch order */
} pic_plan_summary;

pic_status pic_plan_get_summary(const pic_plan* plan, pic_plan_summary* out);

/* Per-request host arrays of the current batch (any pointer may be NULL):
 * row_base int64[batch], prefix_rows int32[batch], first new-token position
 * int32[batch]. */
pic_status pic_plan_get_requests(const pic_plan* plan, int64_t* row_base, int32_t* prefix_rows,
                                 int32_t* first_new_pos);

/* Per-span host arrays (any pointer may be NULL): resolved target int32[n_spans],
 * delta int32[n_spans], first assembled row int64[n_spans]. */
pic_status pic_plan_get_spans(const pic_plan* plan, int32_t* target, int32_t* delta,
                              int64_t* first_row);

/* Per-new-token host arrays: position int32[new_rows], assembled row int64[new_rows]. */
pic_status pic_plan_get_new_tokens(const pic_plan* plan, int32_t* position, int64_t* row);

/* The bf16 attention work list of the current batch, as the host planned it
 * (any pointer may be NULL; empty for other models):
 *   items     int32[attention_items][7]: request, kv head, first query column
 *             (column j*G + g is the request's new token j with query head g
 *             of the group), first tile, end tile, and the tiles
 *             [gap_begin, gap_end) skipped inside that range.  A tile is 64
 *             rows, counted from the request's first assembled row; the
 *             skipped and trimmed tiles hold no row that a query of the item
 *             can see.  Items 2p and 2p + 1 run in one workgroup.
 *   wg_order  int32[attention_workgroups]: the item pair p that workgroup b
 *             of the paired kernel runs (-1: none).  Workgroup b runs on XCD
 *             b mod 8; each XCD gets a contiguous range of pairs, longest
 *             first (pairs within a tenth of the range's longest keep the
 *             work list's order).
 *   item_order int32[attention_item_workgroups]: the same over single items
 *             (-1: none), for variant F without row splits, which runs one
 *             item per workgroup and two workgroups per CU.
 * Introspection only: the kernels read the device copy of these tables. */
pic_status pic_plan_get_attention_work(const pic_plan* plan, int32_t* items, int32_t* wg_order,
                                       int32_t* item_order);

/* Kernel timing: when enabled, the library brackets its main kernels with HIP
 * events on the caller's stream.  pic_timing_read synchronises on the last
 * recorded event and returns the number of launches and their summed
 * duration in milliseconds for one kernel class since the last reset.
 * kernel: 0 = assembly gather, 1 = new-token prologue, 2 = attention
 * (including its split merge), 3 = planning. */
pic_status pic_timing_enable(pic_plan* plan, int32_t on);
pic_status pic_timing_read(pic_plan* plan, int32_t kernel, int64_t* launches, double* total_ms);
pic_status pic_timing_reset(pic_plan* plan);

/* Message of the last failed call on this thread ("" if none). */
const char* pic_last_error(void);

/* Library version string. */
const char* pic_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PIC_H */
