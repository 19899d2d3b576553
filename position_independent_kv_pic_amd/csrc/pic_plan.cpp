// Host-side validation and planning for libpic (pure C++17, no HIP).
#include "pic_plan.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <functional>

namespace pic {
namespace {

pic_status fail(std::string* err, pic_status code, const char* fmt, ...)
    __attribute__((format(printf, 3, 4)));

pic_status fail(std::string* err, pic_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (err) *err = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest position a row may take.  INT32_MAX itself is reserved: the
// attention kernel marks rows past the end of a request with it.
constexpr int64_t kMaxPosition = INT32_MAX - 1;

// rows per attention tile (the kernels' tile height)
constexpr int64_t kTileRows = 64;

// `want` clamped to [1, cap], then made even when above 1 (the two splits of
// a column block pair up in one workgroup): rounded up if that stays within
// the cap, else down.
int32_t even_split(int32_t want, int32_t cap) {
  int32_t split = std::max(1, std::min(want, std::max(cap, 1)));
  if (split > 1 && (split & 1)) split = split + 1 <= cap ? split + 1 : split - 1;
  return split;
}

}  // namespace

pic_status check_model(const pic_model* m, ModelInfo* out, std::string* err) {
  if (!m) return fail(err, PIC_EINVAL, "model is NULL");
  if (m->layers < 1 || m->q_heads < 1 || m->kv_heads < 1)
    return fail(err, PIC_EINVAL, "layers, q_heads and kv_heads must be >= 1");
  if (m->q_heads % m->kv_heads)
    return fail(err, PIC_EINVAL, "q_heads (%d) must be a multiple of kv_heads (%d)", m->q_heads,
                m->kv_heads);
  if (m->head_dim < 16 || m->head_dim > 256 || m->head_dim % 16)
    return fail(err, PIC_EINVAL, "head_dim must be a multiple of 16 in [16, 256], got %d",
                m->head_dim);
  if (!(m->rope_theta > 1.0) || !std::isfinite(m->rope_theta))
    return fail(err, PIC_EINVAL, "rope_theta must be finite and > 1");
  if (m->dtype != PIC_F32 && m->dtype != PIC_BF16)
    return fail(err, PIC_EINVAL, "dtype must be PIC_F32 or PIC_BF16");
  if (m->key_storage != PIC_KEYS_ROTATED && m->key_storage != PIC_KEYS_UNROTATED)
    return fail(err, PIC_EINVAL, "key_storage must be PIC_KEYS_ROTATED or PIC_KEYS_UNROTATED");
  ModelInfo mi;
  mi.layers = m->layers;
  mi.q_heads = m->q_heads;
  mi.kv_heads = m->kv_heads;
  mi.head_dim = m->head_dim;
  mi.dtype = m->dtype;
  mi.key_storage = m->key_storage;
  mi.theta = m->rope_theta;
  mi.elem_bytes = m->dtype == PIC_BF16 ? 2 : 4;
  mi.group = m->q_heads / m->kv_heads;
  mi.row_bytes = int64_t(m->head_dim) * mi.elem_bytes;
  *out = mi;
  return PIC_OK;
}

pic_status build_pool(const pic_model* model, void* pool, int64_t pool_bytes, int32_t page_tokens,
                      int32_t n_pages, int32_t n_chunks, const int32_t* chunk_len,
                      const int32_t* chunk_orig, const int32_t* chunk_page_ptr,
                      const int32_t* page_ids, PoolInfo* out, std::string* err) {
  PoolInfo p;
  pic_status st = check_model(model, &p.m, err);
  if (st != PIC_OK) return st;
  if (!pool) return fail(err, PIC_EINVAL, "pool pointer is NULL");
  if (!aligned16(pool)) return fail(err, PIC_EALIGN, "pool pointer is not 16-byte aligned");
  if (page_tokens < 1 || page_tokens > 4096 || (page_tokens & (page_tokens - 1)))
    return fail(err, PIC_EINVAL, "page_tokens must be a power of two in [1, 4096], got %d",
                page_tokens);
  if (n_pages < 0 || n_chunks < 0) return fail(err, PIC_EINVAL, "negative page or chunk count");
  if (n_chunks > 0 && (!chunk_len || !chunk_page_ptr))
    return fail(err, PIC_EINVAL, "chunk_len and chunk_page_ptr are required");
  p.base = pool;
  p.device_base = pool;
  p.bytes = pool_bytes;
  p.page_tokens = page_tokens;
  p.page_shift = 0;
  while ((1 << p.page_shift) < page_tokens) ++p.page_shift;
  p.n_pages = n_pages;
  p.n_chunks = n_chunks;
  p.page_bytes = int64_t(p.m.layers) * 2 * p.m.kv_heads * page_tokens * p.m.row_bytes;
  if (int64_t(n_pages) > 0 && pool_bytes / int64_t(n_pages) < p.page_bytes)
    return fail(err, PIC_ERANGE, "pool_bytes %lld too small for %d pages of %lld bytes",
                (long long)pool_bytes, n_pages, (long long)p.page_bytes);
  if (int64_t(n_pages) * page_tokens > INT32_MAX)
    return fail(err, PIC_ERANGE, "pool holds more than 2^31 token slots");
  if (n_chunks > 0 && chunk_page_ptr[0] != 0)
    return fail(err, PIC_EINVAL, "chunk_page_ptr[0] must be 0");
  p.chunk_len.assign(chunk_len, chunk_len + n_chunks);
  p.chunk_page_ptr.assign(chunk_page_ptr, chunk_page_ptr + n_chunks + 1);
  if (chunk_orig)
    p.chunk_orig.assign(chunk_orig, chunk_orig + n_chunks);
  else
    p.chunk_orig.assign(n_chunks, 0);
  for (int32_t c = 0; c < n_chunks; ++c) {
    int32_t len = p.chunk_len[c];
    if (len < 0) return fail(err, PIC_EINVAL, "chunk %d has negative length", c);
    if (p.chunk_orig[c] < 0) return fail(err, PIC_EINVAL, "chunk %d has a negative origin", c);
    if (int64_t(p.chunk_orig[c]) + len > INT32_MAX)
      return fail(err, PIC_ERANGE, "chunk %d positions overflow int32", c);
    int64_t have = int64_t(p.chunk_page_ptr[c + 1]) - p.chunk_page_ptr[c];
    int64_t need = (int64_t(len) + page_tokens - 1) / page_tokens;
    if (have < need)
      return fail(err, PIC_EINVAL, "chunk %d needs %lld pages, page table gives %lld", c,
                  (long long)need, (long long)have);
  }
  int32_t n_ids = n_chunks > 0 ? p.chunk_page_ptr[n_chunks] : 0;
  if (n_ids > 0 && !page_ids) return fail(err, PIC_EINVAL, "page_ids is NULL");
  p.page_ids.assign(page_ids ? page_ids : nullptr, page_ids ? page_ids + n_ids : nullptr);
  for (int32_t i = 0; i < n_ids; ++i)
    if (p.page_ids[i] < 0 || p.page_ids[i] >= n_pages)
      return fail(err, PIC_ERANGE, "page_ids[%d] = %d outside [0, %d)", i, p.page_ids[i], n_pages);
  *out = std::move(p);
  return PIC_OK;
}

pic_status build_plan(const PoolInfo& pool, int32_t batch, const int32_t* span_ptr,
                      const pic_span* spans, const int32_t* new_ptr, const int32_t* new_pos,
                      int64_t capacity, int32_t decode_rows, HostPlan* out, std::string* err) {
  if (decode_rows < 0) return fail(err, PIC_EINVAL, "decode_rows must be >= 0");
  if (batch < 0) return fail(err, PIC_EINVAL, "batch must be >= 0");
  if (batch > 0 && (!span_ptr || !new_ptr))
    return fail(err, PIC_EINVAL, "span_ptr and new_ptr are required");
  HostPlan p;
  p.batch = batch;
  if (batch > 0) {
    if (span_ptr[0] != 0 || new_ptr[0] != 0)
      return fail(err, PIC_EINVAL, "span_ptr[0] and new_ptr[0] must be 0");
    for (int32_t b = 0; b < batch; ++b) {
      if (span_ptr[b + 1] < span_ptr[b]) return fail(err, PIC_EINVAL, "span_ptr decreases at %d", b);
      if (new_ptr[b + 1] < new_ptr[b]) return fail(err, PIC_EINVAL, "new_ptr decreases at %d", b);
    }
    p.n_spans = span_ptr[batch];
    p.new_rows = new_ptr[batch];
    if (p.n_spans > 0 && !spans) return fail(err, PIC_EINVAL, "spans is NULL");
  }
  p.spans.resize(p.n_spans);
  p.crow.resize(size_t(p.n_spans) + 1);
  p.reqs.resize(batch);
  p.new_pos.resize(size_t(p.new_rows));
  p.new_row.resize(size_t(p.new_rows));
  p.new_req.resize(size_t(p.new_rows));
  p.req_last_pos.assign(size_t(batch), -1);
  p.decode_rows = decode_rows;

  int64_t row = 0, crow = 0, tiles = 0;
  int32_t max_pos = 0;
  int64_t max_prefix_pos = -1;
  for (int32_t b = 0; b < batch; ++b) {
    ReqRec& r = p.reqs[b];
    r.row_base = int32_t(row);  // range-checked below before it can overflow
    r.span_begin = span_ptr[b];
    r.span_end = span_ptr[b + 1];
    r.new_begin = new_ptr[b];
    r.n_new = new_ptr[b + 1] - new_ptr[b];
    int64_t next = 0;      // AUTO continuation position
    int64_t furthest = 0;  // largest span end (target + n)
    int64_t max_req_span_pos = -1;
    int64_t prefix = 0;
    for (int32_t i = span_ptr[b]; i < span_ptr[b + 1]; ++i) {
      const pic_span& sp = spans[i];
      if (sp.chunk < 0 || sp.chunk >= pool.n_chunks)
        return fail(err, PIC_ERANGE, "span %d: chunk %d outside [0, %d)", i, sp.chunk, pool.n_chunks);
      int32_t len = pool.chunk_len[sp.chunk];
      if (sp.s < 0 || sp.s > sp.e || sp.e >= len)
        return fail(err, PIC_ERANGE, "span %d: need 0 <= s <= e < len, got s=%d e=%d len=%d", i,
                    sp.s, sp.e, len);
      if (sp.target < 0 && sp.target != PIC_TARGET_AUTO && sp.target != PIC_TARGET_ORIGINAL)
        return fail(err, PIC_EINVAL,
                    "span %d: target %d is neither >= 0 nor PIC_TARGET_AUTO / PIC_TARGET_ORIGINAL", i,
                    sp.target);
      int64_t n = int64_t(sp.e) - sp.s + 1;
      const int64_t orig = int64_t(pool.chunk_orig[sp.chunk]) + sp.s;
      int64_t target = sp.target == PIC_TARGET_AUTO       ? next
                       : sp.target == PIC_TARGET_ORIGINAL ? orig
                                                          : int64_t(sp.target);
      if (target < 0) return fail(err, PIC_ERANGE, "span %d: original position is negative", i);
      if (target + n - 1 > kMaxPosition)
        return fail(err, PIC_ERANGE, "span %d: positions exceed %lld", i, (long long)kMaxPosition);
      int64_t delta = target - orig;
      SpanRec& s = p.spans[i];
      s.crow = int32_t(crow);
      s.dst_row = int32_t(row + prefix);
      s.page_off = pool.chunk_page_ptr[sp.chunk];
      s.s = sp.s;
      s.n = int32_t(n);
      s.target = int32_t(target);
      s.delta = int32_t(delta);
      s.req = b;
      p.crow[i] = int32_t(crow);
      max_pos = std::max<int64_t>(max_pos, target + n - 1);
      max_prefix_pos = std::max<int64_t>(max_prefix_pos, target + n - 1);
      max_req_span_pos = std::max<int64_t>(max_req_span_pos, target + n - 1);
      furthest = std::max<int64_t>(furthest, target + n);
      next = target + n;
      prefix += n;
      crow += n;
      if (crow > INT32_MAX || row + prefix > INT32_MAX)
        return fail(err, PIC_ERANGE, "batch has more than 2^31 rows");
    }
    r.prefix_rows = int32_t(prefix);
    for (int32_t j = 0; j < r.n_new; ++j) {
      int32_t u = r.new_begin + j;
      int64_t pos;
      if (new_pos) {
        pos = new_pos[u];
        if (pos < 0) return fail(err, PIC_EINVAL, "new token %d: negative position", u);
        if (pos > kMaxPosition) return fail(err, PIC_ERANGE, "new token %d: position too large", u);
        if (j > 0 && pos <= p.new_pos[u - 1])
          return fail(err, PIC_EINVAL,
                      "new token %d: positions must increase strictly within a request", u);
      } else {
        // after the whole prefix: the larger of its length and its furthest end
        pos = std::max(prefix, furthest) + j;
        if (pos > kMaxPosition) return fail(err, PIC_ERANGE, "new token %d: position too large", u);
      }
      p.new_pos[u] = int32_t(pos);
      p.new_row[u] = int32_t(row + prefix + j);
      p.new_req[u] = b;
      max_pos = std::max<int64_t>(max_pos, pos);
    }
    r.first_new_pos = r.n_new > 0 ? p.new_pos[r.new_begin] : 0;
    r.tile_base = int32_t(tiles);
    tiles += (prefix + r.n_new + kTileRows - 1) / kTileRows;
    row += prefix + r.n_new + decode_rows;
    int64_t last = prefix > 0 ? max_req_span_pos : -1;
    if (r.n_new > 0) last = std::max<int64_t>(last, p.new_pos[r.new_begin + r.n_new - 1]);
    if (last + int64_t(decode_rows) > kMaxPosition)
      return fail(err, PIC_ERANGE, "request %d: decode positions would exceed %lld", b,
                  (long long)kMaxPosition);
    p.req_last_pos[b] = int32_t(last);
    if (row > INT32_MAX) return fail(err, PIC_ERANGE, "batch has more than 2^31 rows");
  }
  p.crow[p.n_spans] = int32_t(crow);
  p.prefix_rows = crow;
  p.rows = row;
  p.n_tiles = int32_t(tiles);
  p.max_position = max_pos;
  // rows of the prefix phase table: one per span (rotated keys, one delta per
  // span) or one per position 0 .. largest prefix position (un-rotated keys)
  p.phase_rows = pool.m.key_storage == PIC_KEYS_UNROTATED ? int32_t(max_prefix_pos + 1) : p.n_spans;
  if (capacity >= 0 && p.rows > capacity)
    return fail(err, PIC_ERANGE, "batch needs %lld rows per plane, capacity is %lld",
                (long long)p.rows, (long long)capacity);
  *out = std::move(p);
  return PIC_OK;
}

AttnSplit choose_attention_split(const HostPlan& plan, int32_t kv_heads, int32_t group, int32_t cols_per_wg,
                                 int32_t rows_per_tile, int32_t target_wgs, int32_t max_split,
                                 int32_t min_tiles_per_split, int32_t min_tiles_across) {
  int64_t items = 0, units = 0;   // column blocks; pairs of them (workgroups without a split)
  int32_t max_tiles = 0;
  for (const ReqRec& r : plan.reqs) {
    const int64_t cols = int64_t(r.n_new) * group;
    if (cols == 0) continue;
    const int64_t ncb = (cols + cols_per_wg - 1) / cols_per_wg;
    items += kv_heads * ncb;
    units += kv_heads * ((ncb + 1) / 2);
    max_tiles = std::max(max_tiles, (r.prefix_rows + r.n_new + rows_per_tile - 1) / rows_per_tile);
  }
  AttnSplit out{1, false};
  if (units == 0 || units >= target_wgs) return out;
  const int32_t tile_cap = std::max(1, max_tiles / std::max(1, min_tiles_per_split));
  // long rows: column-block pairs keep sharing their rows, each split in its
  // own workgroup, merged by the last split to finish
  int32_t across = int32_t((target_wgs + units - 1) / units);
  across = std::max(1, std::min({across, max_split, tile_cap}));
  if (across > 1 && max_tiles / across >= min_tiles_across) return AttnSplit{across, true};
  // short rows: the two splits of a column block share a workgroup and merge
  // in LDS (an even split; merge_kernel combines what is left)
  int32_t split = int32_t((2 * int64_t(target_wgs) + items - 1) / items);
  split = even_split(split, std::min(max_split, tile_cap));
  return AttnSplit{split, false};
}

// Smallest row position of each prefix tile of request r (tiles before the
// one holding its first new row); INT32_MAX for rows past the prefix.
static void prefix_tile_min(const HostPlan& plan, const ReqRec& r, int32_t rows_per_tile,
                            std::vector<int32_t>* out) {
  const int32_t ft = r.prefix_rows / rows_per_tile;
  out->assign(size_t(ft), INT32_MAX);
  for (int32_t i = r.span_begin; i < r.span_end; ++i) {
    const SpanRec& s = plan.spans[size_t(i)];
    const int32_t r0 = s.dst_row - r.row_base;
    // within a span positions increase with the row: the first row of the
    // span inside a tile has the span's smallest position there
    for (int32_t rr = r0; rr < r0 + s.n;) {
      const int32_t t = rr / rows_per_tile;
      if (t >= ft) break;
      (*out)[size_t(t)] = std::min((*out)[size_t(t)], s.target + (rr - r0));
      rr = (t + 1) * rows_per_tile;
    }
  }
}

void build_attention_work(HostPlan* plan, int32_t kv_heads, int32_t group, int32_t cols_per_wg,
                          int32_t rows_per_tile, AttnSplit sp_cfg) {
  std::vector<AttnWork>& out = plan->work;
  out.clear();
  const int32_t split = sp_cfg.split;
  const bool across = sp_cfg.across && split > 1;
  const bool pairs = !across && split > 1 && (split % 2) == 0;
  int32_t slots = 0;
  std::vector<int32_t> tmin;
  for (int32_t b = 0; b < int32_t(plan->reqs.size()); ++b) {
    const ReqRec& r = plan->reqs[b];
    const int64_t cols = int64_t(r.n_new) * group;
    if (cols == 0) continue;
    const int32_t tiles = (r.prefix_rows + r.n_new + rows_per_tile - 1) / rows_per_tile;
    const int32_t ncb = int32_t((cols + cols_per_wg - 1) / cols_per_wg);
    auto item = [&](int32_t h, int32_t c, int32_t sp, int32_t slot) {
      AttnWork w;
      w.req = b;
      w.head = h;
      w.col_begin = c * cols_per_wg;
      w.tile_begin = int32_t(int64_t(tiles) * sp / split);
      w.tile_end = int32_t(int64_t(tiles) * (sp + 1) / split);
      w.split = sp;
      w.merge_pair = pairs && (sp % 2) == 0;
      w.share_rows = 0;
      w.slot = slot;
      w.gap_begin = w.gap_end = 0;
      out.push_back(w);
    };
    if (split == 1) prefix_tile_min(*plan, r, rows_per_tile, &tmin);
    const int32_t ft = r.prefix_rows / rows_per_tile;   // first tile holding a new row
    for (int32_t h = 0; h < kv_heads; ++h) {
      if (across || split == 1) {
        // column-block pairs over the same rows (c == ncb: the empty partner
        // of an odd count); with `across`, the splits of a pair are
        // neighbouring workgroups and every real column block has a counter
        for (int32_t c0 = 0; c0 < ncb; c0 += 2) {
          const size_t first = out.size();
          for (int32_t sp = 0; sp < split; ++sp)
            for (int32_t c = c0; c < c0 + 2; ++c) item(h, c, sp, across && c < ncb ? slots + (c - c0) : -1);
          if (across) slots += std::min(2, ncb - c0);
          if (split == 1) {
            // prefix tiles after the last one that the pair's latest query
            // (new positions increase) can see are skipped up to the tile of
            // the first new row; new rows after that query's own row are
            // later positions, so the range ends at the tile holding it
            const int64_t last_col = std::min<int64_t>(int64_t(c0 + 2) * cols_per_wg, cols) - 1;
            const int32_t qmax = plan->new_pos[size_t(r.new_begin + last_col / group)];
            int32_t a_end = ft;
            while (a_end > 0 && tmin[size_t(a_end - 1)] > qmax) --a_end;
            const int32_t t_end = int32_t((int64_t(r.prefix_rows) + last_col / group) / rows_per_tile) + 1;
            for (size_t k = first; k < out.size(); ++k) {
              out[k].tile_end = std::min(out[k].tile_end, t_end);
              if (a_end < ft) {
                out[k].gap_begin = a_end;
                out[k].gap_end = ft;
              }
            }
          }
        }
      } else {
        // splits of one column block next to each other (pairs: 2j, 2j + 1)
        for (int32_t c = 0; c < ncb; ++c)
          for (int32_t sp = 0; sp < split; ++sp) item(h, c, sp, -1);
      }
    }
  }
  for (size_t i = 0; i + 1 < out.size(); i += 2) {
    AttnWork& x = out[i];
    AttnWork& y = out[i + 1];
    if (!x.merge_pair && x.req == y.req && x.head == y.head && x.tile_begin == y.tile_begin &&
        x.tile_end == y.tile_end && x.tile_end > x.tile_begin)
      x.share_rows = y.share_rows = 1;
  }
  plan->n_split = split;
  plan->n_split_out = pairs ? split / 2 : (across ? 1 : split);
  plan->n_split_wg = across ? split : 1;
  plan->n_slots = slots;
}

namespace {

// Longest-first list schedule of `costs` (sorted, largest first) on `slots`
// workers: the time the last one finishes.
int64_t lpt_makespan(const std::vector<int64_t>& costs, int32_t slots) {
  std::vector<int64_t> busy(size_t(std::max(slots, 1)), 0);   // min-heap of finish times
  int64_t end = 0;
  for (int64_t c : costs) {
    std::pop_heap(busy.begin(), busy.end(), std::greater<int64_t>());
    busy.back() += c;
    end = std::max(end, busy.back());
    std::push_heap(busy.begin(), busy.end(), std::greater<int64_t>());
  }
  return end;
}

// Launch order over units of `per_wg` consecutive items (one workgroup each).
std::vector<int32_t> launch_order(const std::vector<AttnWork>& w, int32_t per_wg, int32_t n_xcd,
                                  int32_t slots_per_xcd) {
  const int32_t n_units = int32_t((w.size() + size_t(per_wg) - 1) / size_t(per_wg));
  std::vector<int32_t> map;
  if (n_units == 0) return map;
  // a workgroup's items run side by side: its time is the longest one's
  // steps (skipped gap tiles excluded), plus set-up and the epilogue
  constexpr int64_t kSetupSteps = 2;
  auto steps = [](const AttnWork& x) { return int64_t(x.tile_end - x.tile_begin - (x.gap_end - x.gap_begin)); };
  std::vector<int64_t> cost(static_cast<size_t>(n_units));
  int64_t total = 0;
  for (int32_t p = 0; p < n_units; ++p) {
    int64_t c = 0;
    for (int32_t k = 0; k < per_wg && size_t(per_wg * p + k) < w.size(); ++k)
      c = std::max(c, steps(w[size_t(per_wg * p + k)]));
    cost[size_t(p)] = c + kSetupSteps;
    total += cost[size_t(p)];
  }
  // candidate cuts: bounds[x] .. bounds[x + 1] is XCD x's range
  std::vector<int32_t> by_count(size_t(n_xcd) + 1), by_cost(size_t(n_xcd) + 1);
  const int32_t q = n_units / n_xcd, r = n_units % n_xcd;
  for (int32_t x = 0; x <= n_xcd; ++x) by_count[size_t(x)] = x * q + std::min(x, r);
  {
    int64_t acc = 0;
    int32_t p = 0;
    by_cost[0] = 0;
    for (int32_t x = 1; x < n_xcd; ++x) {
      const int64_t goal = total * x / n_xcd;
      // end the range where its running cost comes closest to the goal
      while (p < n_units && acc + cost[size_t(p)] <= goal) acc += cost[size_t(p++)];
      if (p < n_units && goal - acc > acc + cost[size_t(p)] - goal) acc += cost[size_t(p++)];
      by_cost[size_t(x)] = p;
    }
    by_cost[size_t(n_xcd)] = n_units;
  }
  // each range longest first.  Costs within a tenth of the range's longest
  // count as equal and keep the plan's order: the column blocks of one
  // request and head stay side by side, run together and share the L2
  auto order = [&](const std::vector<int32_t>& bounds, std::vector<std::vector<int32_t>>* ranges) {
    ranges->assign(size_t(n_xcd), {});
    int64_t span = 0;
    for (int32_t x = 0; x < n_xcd; ++x) {
      std::vector<int32_t>& g = (*ranges)[size_t(x)];
      int64_t top = 1;
      for (int32_t p = bounds[size_t(x)]; p < bounds[size_t(x) + 1]; ++p) {
        g.push_back(p);
        top = std::max(top, cost[size_t(p)]);
      }
      auto band = [&](int32_t p) { return (top - cost[size_t(p)]) * 10 / top; };
      std::stable_sort(g.begin(), g.end(), [&](int32_t a, int32_t b) { return band(a) < band(b); });
      std::vector<int64_t> c;
      for (int32_t p : g) c.push_back(cost[size_t(p)]);
      span = std::max(span, lpt_makespan(c, slots_per_xcd));
    }
    return span;
  };
  std::vector<std::vector<int32_t>> ra, rb;
  const int64_t span_count = order(by_count, &ra);
  const int64_t span_cost = order(by_cost, &rb);
  const std::vector<std::vector<int32_t>>& ranges = span_cost < span_count ? rb : ra;
  size_t longest = 0;
  for (const auto& g : ranges) longest = std::max(longest, g.size());
  map.assign(longest * size_t(n_xcd), -1);
  for (int32_t x = 0; x < n_xcd; ++x)
    for (size_t k = 0; k < ranges[size_t(x)].size(); ++k) map[k * size_t(n_xcd) + size_t(x)] = ranges[size_t(x)][k];
  return map;
}

}  // namespace

void build_wg_map(HostPlan* plan, int32_t n_xcd, int32_t slots_per_xcd) {
  plan->wg_map = launch_order(plan->work, 2, n_xcd, slots_per_xcd);
  // the unpaired kernel fits two workgroups on a CU
  plan->item_map = launch_order(plan->work, 1, n_xcd, 2 * slots_per_xcd);
}

std::vector<int32_t> covered_pages(const HostPlan& plan, int32_t page_tokens) {
  std::vector<int32_t> out;
  for (const SpanRec& sp : plan.spans) {
    if (sp.n <= 0) continue;
    const int32_t first = sp.page_off + sp.s / page_tokens;
    const int32_t last = sp.page_off + (sp.s + sp.n - 1) / page_tokens;
    for (int32_t q = first; q <= last; ++q) out.push_back(q);
  }
  std::sort(out.begin(), out.end());
  out.erase(std::unique(out.begin(), out.end()), out.end());
  return out;
}

HotSet::HotSet(int32_t n_pages, int32_t capacity, int32_t layers)
    : layers_(layers), words_((layers + 63) / 64), slot_of_(size_t(std::max(0, n_pages)), -1),
      page_of_(size_t(std::max(0, capacity)), -1), pins_(size_t(std::max(0, capacity)), 0),
      valid_(size_t(std::max(0, capacity)) * size_t(words_), 0), prev_(size_t(std::max(0, capacity)), -1),
      next_(size_t(std::max(0, capacity)), -1) {
  // the recency list starts as slots 0 .. capacity - 1, all free
  for (int32_t k = 0; k < capacity; ++k) {
    prev_[size_t(k)] = k - 1;
    next_[size_t(k)] = k + 1 < capacity ? k + 1 : -1;
  }
  head_ = capacity > 0 ? 0 : -1;
  tail_ = capacity > 0 ? capacity - 1 : -1;
}

void HotSet::touch(int32_t k) {
  if (tail_ == k) return;
  // unlink
  const int32_t p = prev_[size_t(k)], n = next_[size_t(k)];
  if (p >= 0) next_[size_t(p)] = n; else head_ = n;
  if (n >= 0) prev_[size_t(n)] = p; else tail_ = p;
  // append at the most recent end
  prev_[size_t(k)] = tail_;
  next_[size_t(k)] = -1;
  if (tail_ >= 0) next_[size_t(tail_)] = k; else head_ = k;
  tail_ = k;
}

void HotSet::unpin(int64_t owner) {
  for (size_t i = 0; i < owners_.size(); ++i) {
    if (owners_[i].first != owner) continue;
    for (int32_t page : owners_[i].second) --pins_[size_t(slot_of_[size_t(page)])];
    owners_.erase(owners_.begin() + std::ptrdiff_t(i));
    return;
  }
}

bool HotSet::pin(int64_t owner, const std::vector<int32_t>& pages, std::string* err) {
  std::vector<int32_t> want(pages);
  std::sort(want.begin(), want.end());
  want.erase(std::unique(want.begin(), want.end()), want.end());
  for (int32_t page : want)
    if (page < 0 || size_t(page) >= slot_of_.size()) {
      if (err) *err = "page id out of range";
      return false;
    }
  // capacity check before anything changes: slots pinned by other owners
  // stay, and every wanted page outside them needs a slot
  std::vector<char> by_me(page_of_.size(), 0);
  for (const auto& o : owners_)
    if (o.first == owner)
      for (int32_t page : o.second) by_me[size_t(slot_of_[size_t(page)])] = 1;
  int64_t others = 0;
  for (size_t k = 0; k < page_of_.size(); ++k)
    if (pins_[k] - by_me[k] > 0) ++others;
  int64_t fresh = 0;
  for (int32_t page : want) {
    const int32_t k = slot_of_[size_t(page)];
    if (k < 0 || pins_[size_t(k)] - by_me[size_t(k)] == 0) ++fresh;
  }
  if (others + fresh > int64_t(page_of_.size())) {
    if (err)
      *err = "the hot set holds " + std::to_string(page_of_.size()) + " pages; this batch needs " +
             std::to_string(want.size()) + " beside " + std::to_string(others) + " pinned by other plans";
    return false;
  }
  unpin(owner);
  // resident pages first, so that no page of the batch is evicted for another
  for (int32_t page : want) {
    const int32_t k = slot_of_[size_t(page)];
    if (k < 0) continue;
    ++hits;
    ++pins_[size_t(k)];
    touch(k);
  }
  for (int32_t page : want) {
    if (slot_of_[size_t(page)] >= 0) continue;
    // a free slot or the least recently used unpinned one (the capacity
    // check above guarantees one)
    int32_t k = head_;
    while (k >= 0 && pins_[size_t(k)] > 0) k = next_[size_t(k)];
    const int32_t old = page_of_[size_t(k)];
    if (old >= 0) {
      slot_of_[size_t(old)] = -1;
      ++evictions;
    }
    page_of_[size_t(k)] = page;
    slot_of_[size_t(page)] = k;
    std::fill(valid_.begin() + std::ptrdiff_t(size_t(k) * size_t(words_)),
              valid_.begin() + std::ptrdiff_t(size_t(k + 1) * size_t(words_)), uint64_t(0));
    ++misses;
    ++pins_[size_t(k)];
    touch(k);
  }
  owners_.emplace_back(owner, std::move(want));
  return true;
}

bool HotSet::layer_valid(int32_t slot, int32_t layer) const {
  return (valid_[size_t(slot) * size_t(words_) + size_t(layer / 64)] >> (layer % 64)) & 1u;
}

void HotSet::take_layer(int64_t owner, int32_t layer, std::vector<int32_t>* pairs) {
  pairs->clear();
  for (const auto& o : owners_) {
    if (o.first != owner) continue;
    for (int32_t page : o.second) {
      const int32_t k = slot_of_[size_t(page)];
      uint64_t& word = valid_[size_t(k) * size_t(words_) + size_t(layer / 64)];
      const uint64_t bit = uint64_t(1) << (layer % 64);
      if (word & bit) continue;
      word |= bit;
      pairs->push_back(page);
      pairs->push_back(k);
      ++layer_copies;
    }
  }
}

void build_decode(const HostPlan& plan, int32_t kv_heads, int32_t step, int32_t rows_per_tile,
                  int32_t target_items, int32_t max_split, int32_t min_tiles_per_split, bool own_row,
                  DecodePlan* out) {
  const int32_t batch = plan.batch;
  out->step = step;
  out->own_row = own_row;
  out->pos.assign(size_t(batch), 0);
  out->row.assign(size_t(batch), 0);
  out->reqs.assign(size_t(batch), ReqRec{});
  int32_t max_tiles = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const ReqRec& r = plan.reqs[b];
    ReqRec& d = out->reqs[b];
    d = r;
    // plane rows after the pool rows: the earlier tokens, then this one
    // (left out of the tiles when the kernel adds it itself)
    d.n_new = r.n_new + step + (own_row ? 0 : 1);
    d.new_begin = b;                // query b of the decode batch
    d.tile_base = 0;
    out->pos[b] = plan.req_last_pos[b] + 1 + step;
    out->row[b] = r.row_base + r.prefix_rows + r.n_new + step;
    d.first_new_pos = out->pos[b];
    max_tiles = std::max(max_tiles, (d.prefix_rows + d.n_new + rows_per_tile - 1) / rows_per_tile);
  }
  const int64_t base = int64_t(batch) * kv_heads;
  int32_t split = 1;
  if (base > 0 && base < target_items) {
    split = int32_t((target_items + base - 1) / base);
    split = even_split(split, std::min(max_split, std::max(1, max_tiles / std::max(1, min_tiles_per_split))));
  }
  const bool pairs = split > 1 && (split % 2) == 0;
  out->n_split = split;
  out->n_split_out = pairs ? split / 2 : split;
  out->work.clear();
  for (int32_t b = 0; b < batch; ++b) {
    const ReqRec& d = out->reqs[b];
    const int32_t tiles = (d.prefix_rows + d.n_new + rows_per_tile - 1) / rows_per_tile;
    for (int32_t h = 0; h < kv_heads; ++h) {
      for (int32_t sp = 0; sp < split; ++sp) {
        AttnWork w;
        w.req = b;
        w.head = h;
        w.col_begin = 0;
        w.tile_begin = int32_t(int64_t(tiles) * sp / split);
        w.tile_end = int32_t(int64_t(tiles) * (sp + 1) / split);
        w.split = sp;
        w.merge_pair = pairs && (sp % 2) == 0;
        w.share_rows = 0;
        w.slot = -1;
        w.gap_begin = w.gap_end = 0;
        out->work.push_back(w);
      }
    }
  }
}

}  // namespace pic
