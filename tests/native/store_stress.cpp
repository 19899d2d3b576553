// Randomised driver of the chunk-file store (pic_store.cpp), built by the CPU
// test suite with AddressSanitizer + UndefinedBehaviorSanitizer and, in a
// second build, ThreadSanitizer.  Random pools (shapes, chunk lengths,
// shuffled page tables) are written to chunk files under the directory given
// as the first argument; stores with random thread counts then load random
// page sets, and every wait is followed by a byte comparison of the loaded
// pages with the source and of the others with the canary.  Malformed files
// (wrong shape, short, missing) must be refused at open, and a file cut short
// after opening must fail the next wait and leave its pages unloaded.
// Prints "ok <loads>" and exits 0, or exits 1 at the first mismatch.
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <numeric>
#include <random>
#include <string>
#include <vector>

#include "pic_store.h"

namespace {

int fail(const char* what, int it) {
  std::fprintf(stderr, "store mismatch (%s) at iteration %d\n", what, it);
  return 1;
}

constexpr unsigned char kCanary = 0xA5;

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  const std::string dir = argv[1];
  const unsigned seed = argc > 2 ? unsigned(std::strtoul(argv[2], nullptr, 10)) : 1u;
  const int iters = argc > 3 ? std::atoi(argv[3]) : 20;
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int64_t loads = 0;
  for (int it = 0; it < iters; ++it) {
    pic_model m;
    m.kv_heads = uni(1, 2);
    m.q_heads = m.kv_heads * uni(1, 4);
    m.layers = uni(1, 3);
    m.head_dim = uni(0, 1) ? 32 : 16;
    m.rope_theta = 1e4;
    m.dtype = uni(0, 1) ? PIC_BF16 : PIC_F32;
    m.key_storage = PIC_KEYS_ROTATED;
    const int32_t pt = 1 << uni(0, 3);
    const int32_t n_chunks = uni(1, 12);
    std::vector<int32_t> len(static_cast<size_t>(n_chunks)), orig(static_cast<size_t>(n_chunks));
    std::vector<int32_t> ptr(static_cast<size_t>(n_chunks) + 1, 0);
    for (int32_t c = 0; c < n_chunks; ++c) {
      len[size_t(c)] = uni(0, 5) == 0 ? 0 : uni(1, 70);
      orig[size_t(c)] = uni(0, 3) == 0 ? uni(0, 100) : 0;
      // a chunk may own spare pages beyond the ones its tokens fill
      ptr[size_t(c) + 1] = ptr[size_t(c)] + (len[size_t(c)] + pt - 1) / pt + uni(0, 1);
    }
    const int32_t n_logical = ptr[size_t(n_chunks)];
    const int32_t n_pages = n_logical + uni(0, 4);
    std::vector<int32_t> perm(static_cast<size_t>(n_pages));
    std::iota(perm.begin(), perm.end(), 0);
    std::shuffle(perm.begin(), perm.end(), rng);
    std::vector<int32_t> ids(perm.begin(), perm.begin() + n_logical);
    pic::PoolInfo pi;
    std::string err;
    int64_t fake = int64_t(1) << 40;
    const int64_t page_bytes = int64_t(m.layers) * 2 * m.kv_heads * pt * m.head_dim * (m.dtype == PIC_BF16 ? 2 : 4);
    if (pic::build_pool(&m, reinterpret_cast<void*>(fake), int64_t(n_pages) * page_bytes, pt, n_pages, n_chunks,
                        len.data(), orig.data(), ptr.data(), ids.data(), &pi, &err) != PIC_OK) {
      std::fprintf(stderr, "pool: %s\n", err.c_str());
      return fail("pool registration", it);
    }
    // source pages: random bytes
    std::vector<unsigned char> src(size_t(n_pages) * size_t(page_bytes));
    for (auto& b : src) b = static_cast<unsigned char>(rng());
    std::vector<std::string> paths;
    for (int32_t c = 0; c < n_chunks; ++c) {
      paths.push_back(dir + "/s" + std::to_string(seed) + "_i" + std::to_string(it) + "_c" + std::to_string(c) + ".pic");
      if (pic::write_chunk_file(&m, pt, len[size_t(c)], orig[size_t(c)], src.data(), ids.data() + ptr[size_t(c)],
                                paths.back().c_str(), &err) != PIC_OK) {
        std::fprintf(stderr, "write: %s\n", err.c_str());
        return fail("write", it);
      }
    }
    std::vector<const char*> cpaths;
    for (auto& p : paths) cpaths.push_back(p.c_str());
    std::vector<unsigned char> dst(src.size(), kCanary);

    // malformed files are refused at open
    {
      std::unique_ptr<pic::ChunkStore> bad;
      std::vector<const char*> wrong = cpaths;
      const std::string missing = dir + "/missing.pic";
      wrong[size_t(uni(0, n_chunks - 1))] = missing.c_str();
      if (pic::ChunkStore::open(pi, reinterpret_cast<char*>(dst.data()), int64_t(dst.size()), wrong.data(), 2, &bad,
                                &err) == PIC_OK)
        return fail("a missing file was accepted", it);
      if (pic::ChunkStore::open(pi, reinterpret_cast<char*>(dst.data()), int64_t(dst.size()) - 1, cpaths.data(), 2,
                                &bad, &err) == PIC_OK && n_pages > 0)
        return fail("a short destination was accepted", it);
      // a file written for a deeper model (its own, larger source pages)
      pic_model other = m;
      other.layers = m.layers + 1;
      const int64_t other_bytes = page_bytes / m.layers * other.layers;
      std::vector<unsigned char> other_src(size_t(n_pages) * size_t(other_bytes), 0);
      const std::string op = dir + "/other.pic";
      if (pic::write_chunk_file(&other, pt, len[0], orig[0], other_src.data(), ids.data() + ptr[0], op.c_str(),
                                &err) != PIC_OK)
        return fail("write of the deeper model's file", it);
      wrong = cpaths;
      wrong[0] = op.c_str();
      if (pic::ChunkStore::open(pi, reinterpret_cast<char*>(dst.data()), int64_t(dst.size()), wrong.data(), 2, &bad,
                                &err) == PIC_OK)
        return fail("a file of another model was accepted", it);
      ::unlink(op.c_str());
    }

    const int rounds = uni(2, 5);
    for (int r = 0; r < rounds; ++r) {
      std::unique_ptr<pic::ChunkStore> st;
      if (pic::ChunkStore::open(pi, reinterpret_cast<char*>(dst.data()), int64_t(dst.size()), cpaths.data(),
                                uni(1, 8), &st, &err) != PIC_OK) {
        std::fprintf(stderr, "open: %s\n", err.c_str());
        return fail("open", it);
      }
      std::fill(dst.begin(), dst.end(), kCanary);
      std::vector<char> want(static_cast<size_t>(n_logical), 0);
      const int reqs = uni(1, 6);
      for (int k = 0; k < reqs; ++k) {
        std::vector<int32_t> pages;
        for (int32_t c = 0; c < n_chunks; ++c) {
          const int32_t need = (len[size_t(c)] + pt - 1) / pt;
          for (int32_t j = 0; j < need; ++j)
            if (uni(0, 2) == 0) pages.push_back(ptr[size_t(c)] + j);
        }
        std::shuffle(pages.begin(), pages.end(), rng);
        for (int32_t q : pages) want[size_t(q)] = 1;
        st->request_logical(pages);
        if (uni(0, 1)) {
          if (st->wait(&err) != PIC_OK) return fail("wait", it);
          // every requested page holds its source bytes, every other page the canary
          for (int32_t q = 0; q < n_logical; ++q) {
            const size_t off = size_t(ids[size_t(q)]) * size_t(page_bytes);
            const bool same = std::memcmp(dst.data() + off, src.data() + off, size_t(page_bytes)) == 0;
            bool canary = true;
            for (int64_t b = 0; b < page_bytes && canary; ++b) canary = dst[off + size_t(b)] == kCanary;
            if (want[size_t(q)] && !same) return fail("loaded page differs from its source", it);
            if (!want[size_t(q)] && !canary) return fail("a page nobody requested was written", it);
          }
          ++loads;
        }
      }
      if (st->wait(&err) != PIC_OK) return fail("final wait", it);
      const pic::StoreStats s = st->stats();
      int64_t wanted = 0;
      for (char w : want) wanted += w;
      if (s.pages_read != wanted || s.resident_pages != wanted) return fail("statistics", it);
      if (s.bytes_read != wanted * page_bytes) return fail("byte count", it);

      // a file cut short after opening fails the wait and stays unloaded
      if (r == rounds - 1) {
        int32_t c = -1;
        for (int32_t k = 0; k < n_chunks && c < 0; ++k)
          if (len[size_t(k)] > pt) c = k;
        if (c >= 0) {
          st->forget(false, &err);
          if (::truncate(paths[size_t(c)].c_str(), pic::kChunkHeaderBytes + page_bytes / 2) != 0)
            return fail("truncate", it);
          std::vector<int32_t> pages;
          const int32_t need = (len[size_t(c)] + pt - 1) / pt;
          for (int32_t j = 0; j < need; ++j) pages.push_back(ptr[size_t(c)] + j);
          st->request_logical(pages);
          if (st->wait(&err) != PIC_EIO) return fail("a short read was not reported", it);
          if (st->stats().resident_pages != 0) return fail("pages of a failed read count as loaded", it);
          // restored, the same pages load on the next request
          if (pic::write_chunk_file(&m, pt, len[size_t(c)], orig[size_t(c)], src.data(), ids.data() + ptr[size_t(c)],
                                    paths[size_t(c)].c_str(), &err) != PIC_OK)
            return fail("rewrite", it);
          st->request_logical(pages);
          if (st->wait(&err) != PIC_OK) return fail("retry", it);
          for (int32_t j = 0; j < need; ++j) {
            const size_t off = size_t(ids[size_t(ptr[size_t(c)] + j)]) * size_t(page_bytes);
            if (std::memcmp(dst.data() + off, src.data() + off, size_t(page_bytes)) != 0)
              return fail("retried page differs", it);
          }
        }
      }
      // destroyed with loads possibly still queued: it waits for them
      if (uni(0, 1)) {
        std::vector<int32_t> filled;
        for (int32_t c = 0; c < n_chunks; ++c)
          for (int32_t j = 0; j < (len[size_t(c)] + pt - 1) / pt; ++j) filled.push_back(ptr[size_t(c)] + j);
        st->forget(false, &err);
        st->request_logical(filled);
      }
    }
    for (auto& p : paths) ::unlink(p.c_str());
  }
  std::printf("ok %lld\n", (long long)loads);
  return 0;
}
