// Host-side validation and planning for libpic (pure C++17, no HIP).
//
// Everything here is integer arithmetic on the caller's span tables: span
// lengths, row offsets, resolved targets (CoinRAG page, section 2.3, Delta
// equation: a span's new start is the prompt length plus the lengths of the
// spans before it; TurboRAG review page, Figure 5: composite positions keep
// each chunk where it was encoded), rotation deltas, new-token positions and
// the work list of the attention kernel.  The records below are uploaded to the device as
// they are, so their layouts are shared with the kernels.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "pic.h"

namespace pic {

struct ModelInfo {
  int32_t layers = 0, q_heads = 0, kv_heads = 0, head_dim = 0, dtype = 0;
  int32_t key_storage = PIC_KEYS_ROTATED;
  double theta = 0.0;
  int32_t elem_bytes = 0;   // 2 (bf16) or 4 (f32)
  int32_t group = 0;        // q_heads / kv_heads
  int64_t row_bytes = 0;    // head_dim * elem_bytes
};

struct PoolInfo {
  ModelInfo m;
  void* base = nullptr;         // as registered (device memory or pinned host memory)
  void* device_base = nullptr;  // the same memory as kernels address it
  bool host = false;            // the pool lives in pinned host memory
  int64_t bytes = 0;
  int32_t page_tokens = 0, page_shift = 0, n_pages = 0, n_chunks = 0;
  int64_t page_bytes = 0;
  std::vector<int32_t> chunk_len, chunk_orig, chunk_page_ptr, page_ids;
};

// Span record as the kernels read it (32 bytes).
struct SpanRec {
  int32_t crow;      // first compact prefix row of the span (over the whole batch)
  int32_t dst_row;   // first assembled row
  int32_t page_off;  // chunk_page_ptr[chunk]: index of the chunk's first page id
  int32_t s;         // first source token
  int32_t n;         // length e - s + 1
  int32_t target;    // new position of token s
  int32_t delta;     // rotation applied to every key of the span
  int32_t req;       // request index
};

// Request record (32 bytes).
struct ReqRec {
  int32_t row_base;     // first assembled row of the request
  int32_t prefix_rows;  // rows gathered from spans
  int32_t n_new;        // new tokens
  int32_t new_begin;    // index of the first new token in the packed arrays
  int32_t span_begin, span_end;
  int32_t first_new_pos;
  int32_t tile_base;    // index of the request's first 64-row attention tile
};

// Attention work item: query columns [col_begin, col_begin + cols) of
// request `req` and kv head `head`, over the request's row tiles
// [tile_begin, tile_end); split `split` of `n_split`.  Items 2p and 2p + 1
// share a workgroup.  `merge_pair` (set on item 2p) marks them as splits 2j
// and 2j + 1 of one column block, merged inside the workgroup.  Otherwise they
// are neighbouring column blocks, and when their rows are split over
// workgroups each split writes a partial and counts itself in counter `slot`;
// the last to arrive merges.
struct AttnWork {
  int32_t req;
  int32_t head;
  int32_t col_begin;
  int32_t tile_begin;
  int32_t tile_end;
  int32_t split;
  int32_t merge_pair;
  int32_t share_rows;   // items 2p and 2p + 1 cover the same rows of one (request, kv head)
  int32_t slot;         // merge counter of the column block (-1: rows not split over workgroups)
  int32_t gap_begin;    // tiles [gap_begin, gap_end) of the range are skipped: no query of the
  int32_t gap_end;      // item can see any of their rows (empty: gap_begin == gap_end)
};

struct HostPlan {
  int32_t batch = 0, n_spans = 0, max_position = 0;
  int64_t prefix_rows = 0, new_rows = 0, rows = 0;
  int32_t n_tiles = 0;              // 64-row attention tiles over all requests
  int32_t phase_rows = 0;           // rows of the prefix phase table (spans or positions)
  std::vector<SpanRec> spans;
  std::vector<int32_t> crow;        // n_spans + 1 compact-row offsets
  std::vector<ReqRec> reqs;
  std::vector<int32_t> new_pos;     // per new token
  std::vector<int32_t> new_row;     // assembled row of each new token
  std::vector<int32_t> new_req;     // request of each new token
  std::vector<int32_t> req_last_pos;  // per request: largest position of its rows (-1: none)
  int32_t decode_rows = 0;          // rows reserved after each request's new tokens
  // attention work list
  std::vector<AttnWork> work;
  int32_t n_split = 1;              // row splits per column block
  int32_t n_split_out = 1;          // partials left for merge_kernel
  int32_t n_split_wg = 1;           // splits in different workgroups, merged by the last (1: none)
  int32_t n_slots = 0;              // merge counters (column blocks) when n_split_wg > 1
  // Launch order of the paired attention kernel: workgroup b runs item pair
  // wg_map[b] (-1: none, it exits at once).  Workgroup b lands on XCD b mod
  // n_xcd as the (b / n_xcd)-th of that XCD, so the map gives each XCD a
  // contiguous range of pairs (the pairs of one request and kv head read the
  // same rows and share that XCD's L2), balanced by cost, and runs each
  // range's longest pairs first.
  std::vector<int32_t> wg_map;
  // The same for the unpaired kernel (one item per workgroup, two
  // workgroups per CU): item_map[b] is an item index.
  std::vector<int32_t> item_map;
};

// Validation helpers return PIC_OK or an error code and fill `err`.
pic_status check_model(const pic_model* m, ModelInfo* out, std::string* err);

pic_status build_pool(const pic_model* model, void* pool, int64_t pool_bytes, int32_t page_tokens,
                      int32_t n_pages, int32_t n_chunks, const int32_t* chunk_len,
                      const int32_t* chunk_orig, const int32_t* chunk_page_ptr,
                      const int32_t* page_ids, PoolInfo* out, std::string* err);

// Validate a batch and compute its plan.  `capacity` is the rows available in
// each assembled plane (ignored when < 0); `decode_rows` rows are left free
// after each request's new tokens for decode tokens.
pic_status build_plan(const PoolInfo& pool, int32_t batch, const int32_t* span_ptr,
                      const pic_span* spans, const int32_t* new_ptr, const int32_t* new_pos,
                      int64_t capacity, int32_t decode_rows, HostPlan* out, std::string* err);

// One decode step over a planned (and prefilled) batch: every request gets one
// token at position last_pos + 1 + step, stored at its row
// prefix + n_new + step.  The attention records describe, per request, the
// pool rows (prefix), the rows after them in the planes (new tokens, earlier
// decode tokens and this one) and the single query.
struct DecodePlan {
  int32_t step = -1;
  bool own_row = false;         // the kernel adds the token's own row (not among the tiles)
  std::vector<int32_t> pos;     // per request: the token's position
  std::vector<int32_t> row;     // per request: its assembled row
  std::vector<ReqRec> reqs;     // per request, for the attention kernel in decode mode
  std::vector<AttnWork> work;   // one column block per (request, kv head), split over rows
  int32_t n_split = 1, n_split_out = 1;
};

// `target_items`: about this many work items (row splits of at least
// `min_tiles_per_split` tiles, at most `max_split`, even).  With `own_row`
// the tiles cover only the rows before the token's own (the attention kernel
// scores that one from registers).
void build_decode(const HostPlan& plan, int32_t kv_heads, int32_t step, int32_t rows_per_tile,
                  int32_t target_items, int32_t max_split, int32_t min_tiles_per_split, bool own_row,
                  DecodePlan* out);

// Row split for the attention kernel, used when the batch alone gives fewer
// than `target_wgs` workgroups: at most `max_split` parts, and at most
// (longest request's tiles) / `min_tiles_per_split` parts, so that the
// longest request's parts hold at least `min_tiles_per_split` tiles (shorter
// requests' parts may hold fewer).  With at least `min_tiles_across`
// tiles per part (`across`), the neighbouring column blocks of a workgroup
// keep sharing their rows and the splits run in different workgroups, merged
// by the last to finish; otherwise the two splits of one column block share a
// workgroup and merge in LDS (an even count).
struct AttnSplit {
  int32_t split;
  bool across;
};
AttnSplit choose_attention_split(const HostPlan& plan, int32_t kv_heads, int32_t group, int32_t cols_per_wg,
                                 int32_t rows_per_tile, int32_t target_wgs, int32_t max_split,
                                 int32_t min_tiles_per_split, int32_t min_tiles_across);

// Attention work list: `cols_per_wg` query columns (token-major: column
// j*G + g is token j, head g of the group) per item, `rows_per_tile` rows per
// tile, each request's tiles cut into `split` contiguous ranges.  Without a
// split or with `across`, items are ordered (request, kv head, column-block
// pair, split, column block): the two column blocks of a pair share a
// workgroup over one row range (an odd count gets an empty partner), and
// with `across` every real column block gets a merge counter.  Otherwise they
// are ordered (request, kv head, column block, split), the two splits of a
// pair adjacent at an even index (merge_pair).  Fills work, n_split,
// n_split_out, n_split_wg and n_slots.
void build_attention_work(HostPlan* plan, int32_t kv_heads, int32_t group, int32_t cols_per_wg,
                          int32_t rows_per_tile, AttnSplit split);

// After build_attention_work: fill wg_map for `n_xcd` XCDs of
// `slots_per_xcd` concurrent paired workgroups each, and item_map.  A pair costs its tile steps
// plus a fixed setup; of two cuts of the pairs into contiguous ranges (equal
// counts, equal costs), the one with the shorter simulated longest-first
// schedule is kept.  Costs within a tenth of a range's longest keep the
// plan's order.
void build_wg_map(HostPlan* plan, int32_t n_xcd, int32_t slots_per_xcd);

// Logical pages (indices into the pool's page_ids) whose rows the batch's
// spans cover, ascending, each once.
std::vector<int32_t> covered_pages(const HostPlan& plan, int32_t page_tokens);

// Residency of pool pages in a device hot set of `capacity` page slots.
// Each owner (a plan) pins the pages of its current batch; a page that is not
// resident gets a free slot, or the slot of the least recently used page
// that no owner pins, whose copied layers are then forgotten.  A page's
// layers are copied on first use (take_layer), so the set records per slot
// which layers hold the page's data.  Host bookkeeping only.
class HotSet {
 public:
  HotSet(int32_t n_pages, int32_t capacity, int32_t layers);
  int32_t capacity() const { return int32_t(page_of_.size()); }
  // Replace owner's pinned pages with `pages` (pool page ids; repeats
  // allowed).  Fails, changing nothing, when they do not fit beside the
  // pages other owners pin.
  bool pin(int64_t owner, const std::vector<int32_t>& pages, std::string* err);
  void unpin(int64_t owner);
  bool pins_any() const { return !owners_.empty(); }
  int32_t slot_of(int32_t page) const { return slot_of_[size_t(page)]; }
  int32_t page_in(int32_t slot) const { return page_of_[size_t(slot)]; }
  // The owner's pinned pages whose `layer` is not copied yet, as (page,
  // slot) pairs, and mark them copied.
  void take_layer(int64_t owner, int32_t layer, std::vector<int32_t>* pairs);
  bool layer_valid(int32_t slot, int32_t layer) const;
  // counters since creation
  int64_t hits = 0, misses = 0, evictions = 0, layer_copies = 0;

 private:
  void touch(int32_t slot);   // move to the most recent end
  int32_t layers_, words_;
  std::vector<int32_t> slot_of_;   // per pool page: its slot or -1
  std::vector<int32_t> page_of_;   // per slot: its page or -1
  std::vector<int32_t> pins_;      // per slot: owners pinning it
  std::vector<uint64_t> valid_;    // per slot: words_ words of copied-layer bits
  std::vector<int32_t> prev_, next_;   // recency list over slots (head: least recent)
  int32_t head_ = -1, tail_ = -1;
  std::vector<std::pair<int64_t, std::vector<int32_t>>> owners_;   // pinned pages per owner
};

}  // namespace pic
