// File-backed chunk caches: writer, validation and the threaded loader.
#include "pic_store.h"

#include <fcntl.h>
#include <limits.h>
#include <sys/stat.h>
#include <sys/uio.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>

namespace pic {
namespace {

pic_status fail(std::string* err, pic_status code, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
pic_status fail(std::string* err, pic_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (err) *err = buf;
  return code;
}

constexpr char kMagic[8] = {'P', 'I', 'C', 'C', 'H', 'U', 'N', 'K'};

int64_t pages_of(int32_t len, int32_t page_tokens) { return (int64_t(len) + page_tokens - 1) / page_tokens; }

// Write all of [p, p + n) at `off`, retrying short writes.
bool pwrite_full(int fd, const char* p, int64_t n, int64_t off) {
  while (n > 0) {
    const ssize_t w = ::pwrite(fd, p, size_t(std::min<int64_t>(n, int64_t(1) << 30)), off);
    if (w < 0 && errno == EINTR) continue;
    if (w <= 0) return false;
    p += w;
    n -= w;
    off += w;
  }
  return true;
}

// Fill every buffer of `iov` from `off`, retrying short reads.  Returns 0,
// an errno value, or -1 at an unexpected end of the file.
int preadv_full(int fd, std::vector<iovec>& iov, int64_t off, int64_t* calls) {
  size_t i = 0;
  while (i < iov.size()) {
    const int cnt = int(std::min<size_t>(iov.size() - i, IOV_MAX));
    const ssize_t r = ::preadv(fd, iov.data() + i, cnt, off);
    ++*calls;
    if (r < 0 && errno == EINTR) continue;
    if (r < 0) return errno;
    if (r == 0) return -1;
    off += r;
    size_t got = size_t(r);
    while (got > 0 && i < iov.size()) {
      if (got >= iov[i].iov_len) {
        got -= iov[i].iov_len;
        ++i;
      } else {
        iov[i].iov_base = static_cast<char*>(iov[i].iov_base) + got;
        iov[i].iov_len -= got;
        got = 0;
      }
    }
  }
  return 0;
}

struct Fd {
  int fd = -1;
  explicit Fd(int f) : fd(f) {}
  ~Fd() {
    if (fd >= 0) ::close(fd);
  }
};

}  // namespace

pic_status write_chunk_file(const pic_model* model, int32_t page_tokens, int32_t len, int32_t orig,
                            const void* pages, const int32_t* page_list, const char* path, std::string* err) {
  ModelInfo mi;
  pic_status st = check_model(model, &mi, err);
  if (st != PIC_OK) return st;
  if (!path || !*path) return fail(err, PIC_EINVAL, "path is empty");
  if (page_tokens < 1 || page_tokens > 4096 || (page_tokens & (page_tokens - 1)))
    return fail(err, PIC_EINVAL, "page_tokens must be a power of two in [1, 4096], got %d", page_tokens);
  if (len < 0 || orig < 0) return fail(err, PIC_EINVAL, "len and orig must be >= 0");
  if (int64_t(orig) + len > INT32_MAX) return fail(err, PIC_ERANGE, "chunk positions overflow int32");
  const int64_t n = pages_of(len, page_tokens);
  if (n > 0 && (!pages || !page_list)) return fail(err, PIC_EINVAL, "pages and page_list are required");
  for (int64_t j = 0; j < n; ++j)
    if (page_list[j] < 0) return fail(err, PIC_ERANGE, "page_list[%lld] is negative", (long long)j);
  const int64_t page_bytes = int64_t(mi.layers) * 2 * mi.kv_heads * page_tokens * mi.row_bytes;

  std::vector<char> head(size_t(kChunkHeaderBytes), 0);
  ChunkHeader h;
  std::memset(&h, 0, sizeof(h));
  std::memcpy(h.magic, kMagic, sizeof(kMagic));
  h.version = kChunkVersion;
  h.header_bytes = uint32_t(kChunkHeaderBytes);
  h.layers = mi.layers;
  h.q_heads = mi.q_heads;
  h.kv_heads = mi.kv_heads;
  h.head_dim = mi.head_dim;
  h.dtype = mi.dtype;
  h.key_storage = mi.key_storage;
  h.page_tokens = page_tokens;
  h.len = len;
  h.orig = orig;
  h.page_bytes = page_bytes;
  h.n_pages = n;
  h.rope_theta = mi.theta;
  std::memcpy(head.data(), &h, sizeof(h));

  Fd f(::open(path, O_WRONLY | O_CREAT | O_TRUNC | O_CLOEXEC, 0644));
  if (f.fd < 0) return fail(err, PIC_EIO, "open %s for writing: %s", path, std::strerror(errno));
  bool good = pwrite_full(f.fd, head.data(), kChunkHeaderBytes, 0);
  const char* base = static_cast<const char*>(pages);
  for (int64_t j = 0; good && j < n; ++j)
    good = pwrite_full(f.fd, base + int64_t(page_list[j]) * page_bytes, page_bytes,
                       kChunkHeaderBytes + j * page_bytes);
  // flushed to the device: the file's cached pages are then clean, and a
  // later request to drop them from the OS cache is honoured
  if (good) good = ::fdatasync(f.fd) == 0;
  if (!good) {
    const int e = errno;
    ::unlink(path);
    return fail(err, PIC_EIO, "write %s: %s", path, std::strerror(e));
  }
  return PIC_OK;
}

pic_status ChunkStore::open(const PoolInfo& pool, char* dst, int64_t dst_bytes, const char* const* paths,
                            int32_t threads, std::unique_ptr<ChunkStore>* out, std::string* err) {
  if (!dst) return fail(err, PIC_EINVAL, "destination is NULL");
  if (dst_bytes < int64_t(pool.n_pages) * pool.page_bytes)
    return fail(err, PIC_ERANGE, "destination of %lld bytes is smaller than the pool's %d pages of %lld bytes",
                (long long)dst_bytes, pool.n_pages, (long long)pool.page_bytes);
  if (threads < 1 || threads > 256) return fail(err, PIC_EINVAL, "threads must be in [1, 256], got %d", threads);
  if (pool.n_chunks > 0 && !paths) return fail(err, PIC_EINVAL, "paths is NULL");
  std::unique_ptr<ChunkStore> s(new ChunkStore());
  s->pool_ = pool;
  s->dst_ = dst;
  const int32_t n_logical = pool.n_chunks > 0 ? pool.chunk_page_ptr[size_t(pool.n_chunks)] : 0;
  s->chunk_of_.assign(size_t(n_logical), -1);
  std::vector<char> used(size_t(pool.n_pages), 0);
  for (int32_t c = 0; c < pool.n_chunks; ++c) {
    const char* path = paths[c];
    if (!path || !*path) return fail(err, PIC_EINVAL, "path of chunk %d is empty", c);
    s->paths_.emplace_back(path);
    const int64_t need = pages_of(pool.chunk_len[size_t(c)], pool.page_tokens);
    // the pages a file backs are written by its reads alone
    for (int64_t j = 0; j < need; ++j) {
      const int32_t q = pool.chunk_page_ptr[size_t(c)] + int32_t(j);
      const int32_t pg = pool.page_ids[size_t(q)];
      if (used[size_t(pg)])
        return fail(err, PIC_EINVAL, "pool page %d backs two chunk pages; a file-backed pool needs distinct pages", pg);
      used[size_t(pg)] = 1;
      s->chunk_of_[size_t(q)] = c;
    }
    Fd f(::open(path, O_RDONLY | O_CLOEXEC));
    if (f.fd < 0) return fail(err, PIC_EIO, "open %s: %s", path, std::strerror(errno));
    ChunkHeader h;
    if (::pread(f.fd, &h, sizeof(h), 0) != ssize_t(sizeof(h)))
      return fail(err, PIC_EIO, "%s: cannot read a chunk header", path);
    if (std::memcmp(h.magic, kMagic, sizeof(kMagic)) != 0 || h.version != kChunkVersion ||
        h.header_bytes != uint32_t(kChunkHeaderBytes))
      return fail(err, PIC_EINVAL, "%s is not a chunk file of version %u", path, kChunkVersion);
    const ModelInfo& m = pool.m;
    if (h.layers != m.layers || h.q_heads != m.q_heads || h.kv_heads != m.kv_heads ||
        h.head_dim != m.head_dim || h.dtype != m.dtype || h.key_storage != m.key_storage ||
        h.rope_theta != m.theta || h.page_tokens != pool.page_tokens || h.page_bytes != pool.page_bytes)
      return fail(err, PIC_EINVAL, "%s was written for another model or page size", path);
    if (h.len != pool.chunk_len[size_t(c)] || h.orig != pool.chunk_orig[size_t(c)] || h.n_pages != need)
      return fail(err, PIC_EINVAL, "%s holds %d tokens at origin %d; the pool's chunk %d has %d at %d", path, h.len,
                  h.orig, c, pool.chunk_len[size_t(c)], pool.chunk_orig[size_t(c)]);
    struct stat sb;
    if (::fstat(f.fd, &sb) != 0 || int64_t(sb.st_size) < kChunkHeaderBytes + need * pool.page_bytes)
      return fail(err, PIC_EIO, "%s is shorter than its %lld pages", path, (long long)need);
  }
  s->state_.assign(size_t(n_logical), 0);
  for (int32_t t = 0; t < threads; ++t) s->threads_.emplace_back(&ChunkStore::worker, s.get());
  *out = std::move(s);
  return PIC_OK;
}

ChunkStore::~ChunkStore() {
  {
    std::unique_lock<std::mutex> lk(mu_);
    // the destination stays the caller's: no read may land after this
    done_cv_.wait(lk, [this] { return pending_ == 0; });
    stop_ = true;
  }
  work_cv_.notify_all();
  for (std::thread& t : threads_) t.join();
}

void ChunkStore::request_logical(const std::vector<int32_t>& logical) {
  std::map<int32_t, std::vector<int32_t>> by_chunk;
  {
    std::lock_guard<std::mutex> lk(mu_);
    for (int32_t q : logical) {
      ++st_.requested;
      uint8_t& s = state_[size_t(q)];
      if (s != 0) {
        ++st_.hits;
        continue;
      }
      s = 1;
      const int32_t c = chunk_of_[size_t(q)];
      by_chunk[c].push_back(q - pool_.chunk_page_ptr[size_t(c)]);
    }
    for (auto& kv : by_chunk) {
      std::sort(kv.second.begin(), kv.second.end());
      queue_.push_back(Task{kv.first, std::move(kv.second)});
      ++pending_;
    }
  }
  if (!by_chunk.empty()) work_cv_.notify_all();
}

void ChunkStore::worker() {
  for (;;) {
    Task t;
    {
      std::unique_lock<std::mutex> lk(mu_);
      work_cv_.wait(lk, [this] { return stop_ || !queue_.empty(); });
      if (queue_.empty()) return;  // stop_ with nothing left
      t = std::move(queue_.front());
      queue_.pop_front();
    }
    std::string e;
    const bool good = read_task(t, &e);
    {
      std::lock_guard<std::mutex> lk(mu_);
      const int32_t q0 = pool_.chunk_page_ptr[size_t(t.chunk)];
      for (int32_t j : t.pages) state_[size_t(q0 + j)] = good ? 2 : 0;
      if (good) {
        st_.resident_pages += int64_t(t.pages.size());
        st_.pages_read += int64_t(t.pages.size());
        st_.bytes_read += int64_t(t.pages.size()) * pool_.page_bytes;
      } else if (first_err_.empty()) {
        first_err_ = e;
      }
      if (--pending_ == 0) done_cv_.notify_all();
    }
  }
}

bool ChunkStore::read_task(const Task& t, std::string* err) {
  const std::string& path = paths_[size_t(t.chunk)];
  Fd f(::open(path.c_str(), O_RDONLY | O_CLOEXEC));
  if (f.fd < 0) {
    fail(err, PIC_EIO, "open %s: %s", path.c_str(), std::strerror(errno));
    return false;
  }
  const int32_t q0 = pool_.chunk_page_ptr[size_t(t.chunk)];
  int64_t calls = 0;
  std::vector<iovec> iov;
  // runs of consecutive file pages: one vectored read each, every page
  // straight into its pool slot
  for (size_t a = 0; a < t.pages.size();) {
    size_t b = a + 1;
    while (b < t.pages.size() && t.pages[b] == t.pages[b - 1] + 1) ++b;
    iov.clear();
    for (size_t k = a; k < b; ++k) {
      const int32_t pg = pool_.page_ids[size_t(q0 + t.pages[k])];
      iov.push_back(iovec{dst_ + int64_t(pg) * pool_.page_bytes, size_t(pool_.page_bytes)});
    }
    const int rc = preadv_full(f.fd, iov, kChunkHeaderBytes + int64_t(t.pages[a]) * pool_.page_bytes, &calls);
    if (rc != 0) {
      fail(err, PIC_EIO, "read %s: %s", path.c_str(), rc > 0 ? std::strerror(rc) : "unexpected end of file");
      std::lock_guard<std::mutex> lk(mu_);
      st_.reads += calls;
      return false;
    }
    a = b;
  }
  std::lock_guard<std::mutex> lk(mu_);
  st_.reads += calls;
  return true;
}

pic_status ChunkStore::wait(std::string* err) {
  std::unique_lock<std::mutex> lk(mu_);
  const auto t0 = std::chrono::steady_clock::now();
  done_cv_.wait(lk, [this] { return pending_ == 0; });
  st_.wait_seconds += std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  if (!first_err_.empty()) {
    if (err) *err = first_err_;
    first_err_.clear();
    return PIC_EIO;
  }
  return PIC_OK;
}

pic_status ChunkStore::forget(bool drop_os_cache, std::string* err) {
  pic_status st = wait(err);
  {
    std::lock_guard<std::mutex> lk(mu_);
    std::fill(state_.begin(), state_.end(), uint8_t(0));
    st_.resident_pages = 0;
  }
  if (drop_os_cache) {
    for (const std::string& p : paths_) {
      Fd f(::open(p.c_str(), O_RDONLY | O_CLOEXEC));
      if (f.fd >= 0) (void)::posix_fadvise(f.fd, 0, 0, POSIX_FADV_DONTNEED);
    }
  }
  return st;
}

StoreStats ChunkStore::stats() {
  std::lock_guard<std::mutex> lk(mu_);
  return st_;
}

}  // namespace pic
