// File-backed chunk caches: the storage tier behind a pool in host memory.
//
// Each chunk's per-layer K/V cache is one file (the CoinRAG page, section
// 3.3: one cache file per chunk on NVMe, loaded per document by a thread pool,
// only the token ranges the retrieved spans select).  A file holds a header
// and then the chunk's pages in the pool's page layout, so a page is one
// contiguous read straight into its slot of the pool.  Plain C++17 and POSIX
// I/O: no HIP, no device memory.
#pragma once

#include <condition_variable>
#include <cstdint>
#include <deque>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "pic.h"
#include "pic_plan.h"

namespace pic {

// Chunk file layout, little-endian.  The header is padded to kChunkHeaderBytes
// so that the pages start 4 KB-aligned; page j of the chunk (tokens
// j * page_tokens ...) follows at kChunkHeaderBytes + j * page_bytes.
constexpr int64_t kChunkHeaderBytes = 4096;
constexpr uint32_t kChunkVersion = 1;

struct ChunkHeader {
  char magic[8];          // "PICCHUNK"
  uint32_t version;       // kChunkVersion
  uint32_t header_bytes;  // kChunkHeaderBytes
  int32_t layers, q_heads, kv_heads, head_dim;
  int32_t dtype, key_storage, page_tokens, len;
  int32_t orig, reserved;
  int64_t page_bytes, n_pages;
  double rope_theta;
};

// Write one chunk file: header, then the chunk's ceil(len / page_tokens)
// pages, page j read from pages + page_list[j] * page_bytes.
pic_status write_chunk_file(const pic_model* model, int32_t page_tokens, int32_t len, int32_t orig,
                            const void* pages, const int32_t* page_list, const char* path, std::string* err);

struct StoreStats {
  int64_t resident_pages = 0;  // pages loaded into the destination
  int64_t requested = 0;       // covered pages named by requests
  int64_t hits = 0;            // ... found loaded or already being loaded
  int64_t pages_read = 0;      // pages read from the files
  int64_t bytes_read = 0;
  int64_t reads = 0;           // read system calls
  double wait_seconds = 0.0;   // time callers spent blocked in wait()
};

// Loader of a pool's chunk files into a host buffer laid out like the pool
// (page p at dst + p * page_bytes).  Requests queue one task per chunk on a
// fixed set of threads; each task reads its chunk's missing pages, runs of
// consecutive file pages with one vectored read each.  A page is read once
// and then stays loaded until forget().  request() and wait() are called from
// one thread at a time.
class ChunkStore {
 public:
  static pic_status open(const PoolInfo& pool, char* dst, int64_t dst_bytes, const char* const* paths,
                         int32_t threads, std::unique_ptr<ChunkStore>* out, std::string* err);
  ~ChunkStore();

  // Queue the loads of the pool pages (indices into page_ids, i.e. logical
  // pages) that are neither loaded nor being loaded.  Returns at once.
  void request_logical(const std::vector<int32_t>& logical);
  // Block until nothing is being loaded.  PIC_EINVAL with the first read
  // error since the previous wait (its pages stay unloaded).
  pic_status wait(std::string* err);
  // Wait, then mark every page unloaded; with drop_os_cache, also ask the
  // OS to drop the files' cached pages so that later reads reach the device.
  pic_status forget(bool drop_os_cache, std::string* err);
  StoreStats stats();

  const PoolInfo& pool() const { return pool_; }
  char* dst() const { return dst_; }

 private:
  struct Task {
    int32_t chunk;
    std::vector<int32_t> pages;  // chunk-local page indices, increasing
  };
  ChunkStore() = default;
  void worker();
  bool read_task(const Task& t, std::string* err);

  PoolInfo pool_;
  char* dst_ = nullptr;
  std::vector<std::string> paths_;
  std::vector<int32_t> chunk_of_;  // logical page -> chunk
  std::vector<std::thread> threads_;
  std::mutex mu_;  // guards everything below
  std::vector<uint8_t> state_;  // per logical page: 0 absent, 1 being loaded, 2 loaded
  std::condition_variable work_cv_, done_cv_;
  std::deque<Task> queue_;
  int64_t pending_ = 0;  // tasks queued or running
  bool stop_ = false;
  std::string first_err_;
  StoreStats st_;
};

}  // namespace pic
