// Randomised driver of the host planner (pic_plan.cpp), built by the CPU
// test suite with AddressSanitizer and UndefinedBehaviorSanitizer.  Every
// entry point of the planner runs on random pools and batches, valid and
// invalid; a valid plan is checked for internal consistency.  Prints
// "ok <plans>" and exits 0, or exits 1 at the first inconsistency (a
// sanitizer report aborts it).
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <random>
#include <string>
#include <vector>

#include "pic_plan.h"

namespace {

int fail(const char* what, int it) {
  std::fprintf(stderr, "inconsistent plan (%s) at iteration %d\n", what, it);
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  const unsigned seed = argc > 1 ? unsigned(std::strtoul(argv[1], nullptr, 10)) : 1u;
  const int iters = argc > 2 ? std::atoi(argv[2]) : 400;
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int plans = 0;
  for (int it = 0; it < iters; ++it) {
    pic_model m;
    m.kv_heads = uni(1, 8);
    m.q_heads = m.kv_heads * uni(1, 8);
    m.layers = uni(1, 4);
    m.head_dim = uni(0, 1) ? 128 : 64;
    m.rope_theta = 1e4;
    m.dtype = uni(0, 1) ? PIC_BF16 : PIC_F32;
    m.key_storage = uni(0, 1) ? PIC_KEYS_ROTATED : PIC_KEYS_UNROTATED;
    const int page_tokens = 1 << uni(0, 6);
    const int n_chunks = uni(0, 30);
    std::vector<int32_t> len(n_chunks), orig(n_chunks), ptr(n_chunks + 1, 0);
    for (int c = 0; c < n_chunks; ++c) {
      len[c] = uni(0, 4) ? uni(1, 300) : 0;
      orig[c] = uni(0, 3) ? 0 : uni(0, 5000);
      ptr[c + 1] = ptr[c] + (len[c] + page_tokens - 1) / page_tokens;
    }
    const int n_pages = ptr[n_chunks] + uni(0, 3);
    std::vector<int32_t> ids(ptr[n_chunks]);
    std::iota(ids.begin(), ids.end(), 0);
    std::shuffle(ids.begin(), ids.end(), rng);
    const int64_t page_bytes = int64_t(m.layers) * 2 * m.kv_heads * page_tokens * m.head_dim * (m.dtype ? 2 : 4);
    // sometimes a malformed pool: a page id out of range or a short page table
    const int bad_pool = uni(0, 9);
    if (bad_pool == 0 && !ids.empty()) ids[uni(0, int(ids.size()) - 1)] = n_pages + 3;
    if (bad_pool == 1 && n_chunks > 0 && len[0] > page_tokens) ptr[1] = 0, ptr[0] = 0;
    pic::PoolInfo pool;
    std::string err;
    pic_status st = pic::build_pool(&m, reinterpret_cast<void*>(uintptr_t(1) << 40),
                                    std::max<int64_t>(n_pages, 1) * page_bytes, page_tokens, n_pages, n_chunks,
                                    len.data(), uni(0, 1) ? orig.data() : nullptr, ptr.data(),
                                    ids.empty() ? nullptr : ids.data(), &pool, &err);
    if (st != PIC_OK) continue;
    for (int b_it = 0; b_it < 4; ++b_it) {
      const int batch = uni(0, 6);
      std::vector<int32_t> span_ptr(batch + 1, 0), new_ptr(batch + 1, 0);
      std::vector<pic_span> spans;
      std::vector<int32_t> new_pos;
      bool explicit_pos = uni(0, 1) == 1;
      for (int b = 0; b < batch; ++b) {
        const int ns = n_chunks ? uni(0, 10) : 0;
        for (int i = 0; i < ns; ++i) {
          pic_span s;
          s.chunk = uni(0, 20) ? uni(0, n_chunks - 1) : uni(-2, n_chunks + 2);
          const int L = s.chunk >= 0 && s.chunk < n_chunks ? len[s.chunk] : 10;
          s.s = L > 0 ? uni(0, L - 1) : 0;
          s.e = L > 0 ? uni(s.s, L - 1) : 0;
          if (uni(0, 25) == 0) s.e = s.s - 1;                       // malformed
          const int tk = uni(0, 5);
          s.target = tk == 0 ? PIC_TARGET_ORIGINAL : tk == 1 ? uni(0, 100000) : PIC_TARGET_AUTO;
          spans.push_back(s);
        }
        span_ptr[b + 1] = int32_t(spans.size());
        const int nn = uni(0, 4) ? uni(0, 300) : 0;
        int p = uni(0, 200000);
        for (int j = 0; j < nn; ++j) {
          p += uni(0, 30) ? uni(1, 3) : 0;                          // occasionally not increasing
          new_pos.push_back(p);
        }
        new_ptr[b + 1] = int32_t(new_pos.size());
      }
      const int64_t capacity = uni(0, 5) ? int64_t(1) << 40 : uni(0, 3000);
      const int decode_rows = uni(0, 3);
      pic::HostPlan hp;
      st = pic::build_plan(pool, batch, span_ptr.data(), spans.empty() ? nullptr : spans.data(), new_ptr.data(),
                           explicit_pos && !new_pos.empty() ? new_pos.data() : nullptr, capacity, decode_rows,
                           &hp, &err);
      if (st != PIC_OK) continue;
      ++plans;
      if (hp.crow.size() != size_t(hp.n_spans) + 1 || hp.reqs.size() != size_t(batch)) return fail("tables", it);
      int64_t rows = 0;
      for (const auto& r : hp.reqs) {
        if (r.row_base != rows) return fail("row_base", it);
        rows += int64_t(r.prefix_rows) + r.n_new + decode_rows;
      }
      if (rows != hp.rows) return fail("rows", it);
      const pic::AttnSplit sp = pic::choose_attention_split(hp, m.kv_heads, m.q_heads / m.kv_heads, 128, 64, 256, 16,
                                                            3, 64);
      pic::build_attention_work(&hp, m.kv_heads, m.q_heads / m.kv_heads, 128, 64, sp);
      pic::build_wg_map(&hp, 8, 32);
      const int units = int((hp.work.size() + 1) / 2);
      std::vector<int> seen(size_t(units), 0);
      for (int32_t u : hp.wg_map) {
        if (u < -1 || u >= units) return fail("wg_map entry", it);
        if (u >= 0 && seen[size_t(u)]++) return fail("wg_map repeat", it);
      }
      for (const auto& w : hp.work) {
        const auto& r = hp.reqs[size_t(w.req)];
        const int tiles = (r.prefix_rows + r.n_new + 63) / 64;
        if (w.tile_begin < 0 || w.tile_end > tiles || w.tile_begin > w.tile_end) return fail("tile range", it);
        if (w.gap_begin > w.gap_end || (w.gap_end > w.gap_begin && (w.gap_begin < w.tile_begin || w.gap_end > w.tile_end)))
          return fail("gap", it);
      }
      for (int step = 0; step < decode_rows; ++step) {
        for (int own = 0; own < 2; ++own) {
          pic::DecodePlan dp;
          pic::build_decode(hp, m.kv_heads, step, 64, 512, 16, 2, own != 0, &dp);
          if (dp.pos.size() != size_t(batch) || dp.work.size() != size_t(batch) * m.kv_heads * dp.n_split)
            return fail("decode", it);
          // each column block's splits cover its tiles in order, without gaps;
          // the token's own row is among them unless the kernel adds it
          for (size_t i = 0; i < dp.work.size(); ++i) {
            const auto& w = dp.work[i];
            const auto& r = hp.reqs[size_t(w.req)];
            const int rows = r.prefix_rows + r.n_new + step + (own ? 0 : 1);
            if (dp.reqs[size_t(w.req)].prefix_rows + dp.reqs[size_t(w.req)].n_new != rows)
              return fail("decode rows", it);
            const int tiles = (rows + 63) / 64;
            const int first = w.split == 0 ? 0 : dp.work[i - 1].tile_end;
            if (w.tile_begin != first || w.tile_end < w.tile_begin || w.tile_end > tiles ||
                (w.split == dp.n_split - 1 && w.tile_end != tiles))
              return fail("decode tiles", it);
          }
        }
      }
    }
  }
  // hot set: random owners pin random page sets, take layers and unpin; the
  // residency tables stay a bijection, every pinned page stays resident, no
  // page is evicted while pinned, and a layer is handed out once per
  // residency
  int hot_ops = 0;
  for (int round = 0; round < 20; ++round) {
    const int n_pages = uni(1, 300), cap = uni(1, 120), layers = uni(1, 70), n_owners = uni(1, 3);
    pic::HotSet hs(n_pages, cap, layers);
    std::vector<std::vector<int32_t>> pinned(static_cast<size_t>(n_owners));
    std::vector<std::vector<char>> taken(static_cast<size_t>(n_pages), std::vector<char>(static_cast<size_t>(layers), 0));
    for (int op = 0; op < 200; ++op, ++hot_ops) {
      const int owner = uni(0, n_owners - 1);
      const int kind = uni(0, 9);
      if (kind < 5) {
        std::vector<int32_t> want(static_cast<size_t>(uni(0, cap + 10)));
        for (auto& x : want) x = uni(0, n_pages - 1);
        std::vector<int32_t> before(static_cast<size_t>(n_pages));
        for (int q = 0; q < n_pages; ++q) before[size_t(q)] = hs.slot_of(q);
        std::string err;
        if (hs.pin(owner, want, &err)) {
          std::sort(want.begin(), want.end());
          want.erase(std::unique(want.begin(), want.end()), want.end());
          pinned[size_t(owner)] = want;
          // a page whose slot changed lost its copied layers
          for (int q = 0; q < n_pages; ++q)
            if (hs.slot_of(q) != before[size_t(q)]) std::fill(taken[size_t(q)].begin(), taken[size_t(q)].end(), 0);
        } else {
          for (int q = 0; q < n_pages; ++q)
            if (hs.slot_of(q) != before[size_t(q)]) return fail("failed pin changed residency", op);
        }
      } else if (kind < 8) {
        const int layer = uni(0, layers - 1);
        std::vector<int32_t> pairs;
        hs.take_layer(owner, layer, &pairs);
        for (size_t i = 0; i + 1 < pairs.size(); i += 2) {
          if (hs.slot_of(pairs[i]) != pairs[i + 1]) return fail("take_layer slot", op);
          if (taken[size_t(pairs[i])][size_t(layer)]++) return fail("layer handed out twice", op);
          if (!hs.layer_valid(pairs[i + 1], layer)) return fail("layer not marked", op);
        }
        for (int32_t q : pinned[size_t(owner)])
          if (!taken[size_t(q)][size_t(layer)]) return fail("pinned page layer missing", op);
      } else {
        hs.unpin(owner);
        pinned[size_t(owner)].clear();
      }
      // invariants
      int resident = 0;
      for (int q = 0; q < n_pages; ++q) {
        const int k = hs.slot_of(q);
        if (k < 0) continue;
        ++resident;
        if (k >= cap || hs.page_in(k) != q) return fail("residency tables", op);
      }
      if (resident > cap) return fail("over capacity", op);
      for (const auto& pv : pinned)
        for (int32_t q : pv)
          if (hs.slot_of(q) < 0) return fail("pinned page not resident", op);
    }
  }
  std::printf("ok %d %d\n", plans, hot_ops);
  return 0;
}
