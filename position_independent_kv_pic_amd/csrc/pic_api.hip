// C ABI of libpic: handles, validation, planning upload, kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "pic.h"
#include "pic_kernels.h"
#include "pic_plan.h"
#include "pic_store.h"

namespace {

thread_local std::string g_err;

pic_status set_err(pic_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pic_status set_err(pic_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

pic_status ok() {
  g_err.clear();
  return PIC_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kTimedKernels = 4;

}  // namespace

struct pic_pool {
  pic::PoolInfo info;
  int n_plans = 0;
  int device = -1;
  int32_t* d_page_ids = nullptr;
  pic_cache* cache = nullptr;   // hot set in front of a host pool
  pic_store* store = nullptr;   // chunk files that fill a host pool on demand
};

// Hot set: page slots in device memory, their residency (pic::HotSet), and
// per layer a device array of (page, slot) pairs to copy with its pinned
// staging, reused once the event of its last upload has passed.
struct pic_cache {
  pic_pool* pool = nullptr;
  pic::HotSet hs;
  char* buf = nullptr;            // capacity x page_bytes
  int32_t* d_pairs = nullptr;     // [layers][capacity][2]
  int32_t* h_pairs = nullptr;     // pinned staging of d_pairs
  std::vector<hipEvent_t> ev;     // per layer: its last pair upload
  std::vector<char> ev_live;
  int64_t bytes_copied = 0;
  int device = -1;
  pic_cache(int32_t n_pages, int32_t capacity, int32_t layers) : hs(n_pages, capacity, layers) {}
};

// Chunk files loaded into a host buffer laid out like the pool; attached to
// the pool when that buffer is the pool's own pinned memory.
struct pic_store {
  pic_pool* pool = nullptr;
  bool attached = false;
  std::unique_ptr<pic::ChunkStore> cs;
};

struct pic_plan {
  pic_pool* pool = nullptr;
  pic::HostPlan hp;
  bool has_batch = false;
  bool materialized = false;         // every layer's prefix rows are gathered
  bool values_in_pool = false;       // only keys are gathered; attention reads prefix values in the pool
  std::vector<char> gathered;        // per layer: prefix rows gathered into the planes
  std::vector<hipEvent_t> layer_ev;  // per layer: completion of a deferred gather
  std::vector<char> layer_ev_live;   // per layer: layer_ev was recorded for this batch
  hipEvent_t plan_ev = nullptr;      // the batch's plan kernels have been enqueued before it
  // Calls on a plan share its device tables and scratch (rotated queries,
  // split partials, merge counters, decode tables): the stream of the last
  // such call, and an event recorded on it when a call comes on another one
  hipStream_t last_stream = nullptr;
  bool has_last_stream = false;
  hipEvent_t switch_ev = nullptr;
  bool failed = false;
  char* asm_k = nullptr;
  char* asm_v = nullptr;
  int64_t cap = 0;
  int device = -1;

  // device workspace: uploaded tables followed by generated tables
  char* ws = nullptr;
  size_t ws_cap = 0;
  size_t off_spans = 0, off_crow = 0, off_reqs = 0, off_new_pos = 0, off_new_row = 0,
         off_new_req = 0, off_work = 0, off_omega = 0, off_wg_map = 0, off_item_map = 0, off_page_tab = 0,
         blob_bytes = 0;
  size_t off_pos = 0, off_rowsrc = 0, off_gsrc = 0, off_tile_pos = 0, off_phase_tab = 0, off_phase_new = 0,
         off_qrot = 0, off_opart = 0, off_ml = 0, off_spart = 0, off_sml = 0, off_count = 0,
         ws_bytes = 0;

  // pinned staging for the upload, reused once its copy has completed
  char* staging = nullptr;
  size_t staging_cap = 0;
  hipEvent_t staging_ev = nullptr;
  bool staging_pending = false;

  // decode: rows reserved per request at the next assemble, and the tables of
  // the current decode step (uploaded blob followed by generated tables)
  int32_t decode_rows_next = 0;
  pic::DecodePlan dec;
  char* dws = nullptr;
  size_t dws_cap = 0;
  size_t d_pos = 0, d_row = 0, d_reqs = 0, d_work = 0, d_blob = 0, d_phase = 0, d_qrot = 0, d_opart = 0,
         d_ml = 0, d_bytes = 0;

  // optional kernel timing
  bool timing = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events[kTimedKernels];
  size_t used[kTimedKernels] = {0, 0, 0, 0};
};

namespace {

// Scratch of pic_query_prefill_noalloc: the rotated queries, split partials
// and merge counters of one call live here instead of in memory the library
// allocates.  Each device holds its own copy (from the load of the library
// until the process ends), at its own address; every call on a device shares
// that copy, so calls that overlap on one device race.  Host code never uses
// the array's name as an address: the device address is looked up once per
// device (noalloc_scratch) and passed to the kernels.
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};

pic_status device_error(pic_plan* p, hipError_t e, const char* what) {
  if (p) p->failed = true;
  return set_err(PIC_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Bracket one launch with events when timing is on.
struct Timed {
  pic_plan* p;
  int k;
  hipStream_t s;
  hipEvent_t stop = nullptr;
  Timed(pic_plan* plan, int kernel, hipStream_t stream, bool on = true) : p(plan), k(kernel), s(stream) {
    if (!p->timing || !on) return;
    auto& v = p->events[k];
    if (p->used[k] == v.size()) {
      hipEvent_t a = nullptr, b = nullptr;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
        if (a) (void)hipEventDestroy(a);
        return;
      }
      v.emplace_back(a, b);
    }
    auto& pr = v[p->used[k]++];
    (void)hipEventRecord(pr.first, s);
    stop = pr.second;
  }
  ~Timed() {
    if (stop) (void)hipEventRecord(stop, s);
  }
};

pic_status ensure_pool_device(pic_pool* pool) {
  if (pool->d_page_ids || pool->info.page_ids.empty()) return PIC_OK;
  size_t bytes = pool->info.page_ids.size() * sizeof(int32_t);
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&pool->d_page_ids), bytes);
  if (e != hipSuccess) {
    pool->d_page_ids = nullptr;
    return set_err(PIC_ENOMEM, "hipMalloc of the page table failed: %s", hipGetErrorString(e));
  }
  e = hipMemcpy(pool->d_page_ids, pool->info.page_ids.data(), bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) return set_err(PIC_EDEVICE, "page table upload: %s", hipGetErrorString(e));
  return PIC_OK;
}

// Where kernels read the pool's pages: the hot set's slots, or the pool.
const char* pool_addr(const pic_pool* pool) {
  return pool->cache ? pool->cache->buf : static_cast<const char*>(pool->info.device_base);
}

// Copy into the hot set the slices of layers [l0, l1) of the pages that the
// plan's batch pins and that no earlier call has copied.
pic_status cache_fill(pic_plan* p, int32_t l0, int32_t l1, hipStream_t s);

// Device scratch of one prefill call: rotated queries, split partials and
// merge counters.
struct PrefillScratch {
  char* q_rot;
  float* opart;
  float2* ml;
  float* spart;
  float* sml;
  int32_t* count;
  bool clear_count;   // zero the merge counters before the kernels (shared scratch)
};

// Byte offsets of a prefill's scratch inside one buffer, each 256-aligned,
// and its total size (the same quantities layout_workspace reserves).
struct ScratchLayout {
  size_t q_rot = 0, opart = 0, ml = 0, spart = 0, sml = 0, count = 0, bytes = 0;
};

ScratchLayout prefill_scratch_layout(const pic::ModelInfo& m, const pic::HostPlan& hp) {
  ScratchLayout l;
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  l.q_rot = take(size_t(hp.new_rows) * m.q_heads * m.head_dim * m.elem_bytes);
  const size_t nsplit = hp.n_split_out > 1 ? size_t(hp.n_split_out) : 0;
  l.opart = take(nsplit * size_t(hp.new_rows) * m.q_heads * m.head_dim * sizeof(float));
  l.ml = take(nsplit * size_t(hp.new_rows) * m.q_heads * sizeof(float2));
  // row splits merged inside the attention kernel: per column block and
  // split, 4 waves of 64 lanes x (64 floats of O + (m, sum)), and a counter
  const size_t split_waves = size_t(hp.n_slots) * size_t(hp.n_split_wg > 1 ? hp.n_split_wg : 0) * 4;
  l.spart = take(split_waves * 64 * 64 * sizeof(float));
  l.sml = take(split_waves * 64 * 2 * sizeof(float));
  l.count = take(size_t(hp.n_slots) * sizeof(int32_t));
  l.bytes = o;
  return l;
}

void layout_workspace(pic_plan* p) {
  const pic::ModelInfo& m = p->pool->info.m;
  const pic::HostPlan& hp = p->hp;
  const size_t half = size_t(m.head_dim) / 2;
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  p->off_spans = take(hp.spans.size() * sizeof(pic::SpanRec));
  p->off_crow = take(hp.crow.size() * sizeof(int32_t));
  p->off_reqs = take(hp.reqs.size() * sizeof(pic::ReqRec));
  p->off_new_pos = take(hp.new_pos.size() * sizeof(int32_t));
  p->off_new_row = take(hp.new_row.size() * sizeof(int32_t));
  p->off_new_req = take(hp.new_req.size() * sizeof(int32_t));
  p->off_work = take(hp.work.size() * sizeof(pic::AttnWork));
  p->off_omega = take(half * sizeof(double));
  p->off_wg_map = take(hp.wg_map.size() * sizeof(int32_t));
  p->off_item_map = take(hp.item_map.size() * sizeof(int32_t));
  // with a hot set: the batch's page table, pool pages to hot-set slots
  p->off_page_tab = take(p->pool->cache ? p->pool->info.page_ids.size() * sizeof(int32_t) : 0);
  p->blob_bytes = o;
  p->off_pos = take(size_t(hp.rows) * sizeof(int32_t));
  p->off_rowsrc = take(size_t(hp.rows) * sizeof(int2));
  p->off_gsrc = take(size_t(hp.prefix_rows) * sizeof(int4));
  p->off_tile_pos = take(size_t(hp.n_tiles) * sizeof(int2));
  p->off_phase_tab = take(size_t(hp.phase_rows) * half * sizeof(pic::Phase));
  p->off_phase_new = take(size_t(hp.new_rows) * half * sizeof(pic::Phase));
  // the prefill's scratch (rotated queries, split partials, merge counters)
  const ScratchLayout sl = prefill_scratch_layout(m, hp);
  const size_t sb = take(sl.bytes);
  p->off_qrot = sb + sl.q_rot;
  p->off_opart = sb + sl.opart;
  p->off_ml = sb + sl.ml;
  p->off_spart = sb + sl.spart;
  p->off_sml = sb + sl.sml;
  p->off_count = sb + sl.count;
  p->ws_bytes = o;
}

pic_status ensure_staging(pic_plan* p, size_t bytes);

pic_status ensure_capacity(pic_plan* p) {
  if (p->ws_bytes > p->ws_cap) {
    if (p->ws) {
      hipError_t e = hipDeviceSynchronize();
      if (e != hipSuccess) return device_error(p, e, "synchronise before growing the workspace");
      (void)hipFree(p->ws);
      p->ws = nullptr;
      p->ws_cap = 0;
    }
    size_t want = align256(p->ws_bytes + p->ws_bytes / 4);
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&p->ws), want);
    if (e != hipSuccess) {
      p->ws = nullptr;
      return set_err(PIC_ENOMEM, "hipMalloc of %zu workspace bytes failed: %s", want,
                     hipGetErrorString(e));
    }
    p->ws_cap = want;
  }
  return ensure_staging(p, p->blob_bytes);
}

pic_status ensure_staging(pic_plan* p, size_t bytes) {
  if (bytes > p->staging_cap) {
    if (p->staging_pending) {
      hipError_t e = hipEventSynchronize(p->staging_ev);
      if (e != hipSuccess) return device_error(p, e, "wait for the previous plan upload");
      p->staging_pending = false;
    }
    if (p->staging) (void)hipHostFree(p->staging);
    p->staging = nullptr;
    p->staging_cap = 0;
    size_t want = align256(bytes + bytes / 4);
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&p->staging), want, hipHostMallocDefault);
    if (e != hipSuccess) {
      p->staging = nullptr;
      return set_err(PIC_ENOMEM, "hipHostMalloc of %zu staging bytes failed: %s", want,
                     hipGetErrorString(e));
    }
    p->staging_cap = want;
  }
  if (!p->staging_ev) {
    hipError_t e = hipEventCreateWithFlags(&p->staging_ev, hipEventDisableTiming);
    if (e != hipSuccess) return device_error(p, e, "create the staging event");
  }
  return PIC_OK;
}

template <typename T>
void put(char* base, size_t off, const std::vector<T>& v) {
  if (!v.empty()) std::memcpy(base + off, v.data(), v.size() * sizeof(T));
}

pic_status check_device(pic_plan* p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(nullptr, e, "hipGetDevice");
  if (p->device < 0) p->device = dev;
  if (p->device != dev)
    return set_err(PIC_ESTATE, "plan was created for device %d, current device is %d", p->device, dev);
  if (p->pool->device < 0) p->pool->device = dev;
  if (p->pool->device != dev)
    return set_err(PIC_ESTATE, "pool tables live on device %d, current device is %d", p->pool->device,
                   dev);
  return PIC_OK;
}

// Gather the prefix rows of layers [l0, l1) into the planes on stream s.  A
// deferred gather records each layer's completion so that the layer's
// prefill, on any stream, waits for it.
pic_status cache_fill(pic_plan* p, int32_t l0, int32_t l1, hipStream_t s) {
  pic_cache* c = p->pool->cache;
  if (!c) return PIC_OK;
  const pic::PoolInfo& pi = p->pool->info;
  // a page's layer: K and V planes of every kv head, page_tokens rows each
  const int64_t slice = int64_t(2) * pi.m.kv_heads * pi.page_tokens * pi.m.row_bytes;
  const int64_t cap = c->hs.capacity();
  std::vector<int32_t> pairs;
  for (int32_t l = l0; l < l1; ++l) {
    c->hs.take_layer(reinterpret_cast<int64_t>(p), l, &pairs);
    if (pairs.empty()) continue;
    const int32_t n = int32_t(pairs.size() / 2);
    // the layer's staging region is free once its last upload has passed
    if (c->ev_live[size_t(l)]) {
      hipError_t e = hipEventSynchronize(c->ev[size_t(l)]);
      if (e != hipSuccess) return device_error(p, e, "wait for the hot set's last copy list");
    }
    int32_t* hst = c->h_pairs + size_t(l) * size_t(cap) * 2;
    int32_t* dst = c->d_pairs + size_t(l) * size_t(cap) * 2;
    std::memcpy(hst, pairs.data(), pairs.size() * sizeof(int32_t));
    hipError_t e = hipMemcpyAsync(dst, hst, pairs.size() * sizeof(int32_t), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return device_error(p, e, "hot-set copy list upload");
    e = hipEventRecord(c->ev[size_t(l)], s);
    if (e != hipSuccess) return device_error(p, e, "record the copy list event");
    c->ev_live[size_t(l)] = 1;
    e = pic::launch_cache_fill(static_cast<const char*>(pi.device_base), c->buf, dst, n, pi.page_bytes,
                               int64_t(l) * slice, slice, s);
    if (e != hipSuccess) return device_error(p, e, "hot-set copy");
    c->bytes_copied += int64_t(n) * slice;
  }
  return PIC_OK;
}

pic_status gather_layers(pic_plan* p, int32_t l0, int32_t l1, hipStream_t s, bool deferred) {
  const pic::HostPlan& h = p->hp;
  const pic::PoolInfo& pi = p->pool->info;
  if (h.prefix_rows > 0 && l1 > l0) {
    Timed tm(p, 0, s);
    pic_status st = cache_fill(p, l0, l1, s);
    if (st != PIC_OK) return st;
    pic::GatherArgs ga;
    ga.gsrc = reinterpret_cast<const int4*>(p->ws + p->off_gsrc);
    ga.phase_tab = reinterpret_cast<const pic::Phase*>(p->ws + p->off_phase_tab);
    ga.pool = pool_addr(p->pool);
    ga.asm_k = p->asm_k;
    ga.asm_v = p->asm_v;
    ga.prefix_rows = h.prefix_rows;
    ga.cap = p->cap;
    ga.page_bytes = pi.page_bytes;
    ga.page_shift = pi.page_shift;
    ga.page_tokens = pi.page_tokens;
    ga.kv_heads = pi.m.kv_heads;
    ga.planes_per_block = 4;   // one iteration of four planes; 8 per block (two iterations) measured slower
    ga.plane_begin = l0 * pi.m.kv_heads;
    ga.plane_end = l1 * pi.m.kv_heads;
    ga.values = p->values_in_pool ? 0 : 1;
    hipError_t e = pic::launch_gather(pi.m.dtype, pi.m.head_dim, ga, s);
    if (e != hipSuccess) return device_error(p, e, "gather kernel");
  }
  if (p->layer_ev.size() != size_t(pi.m.layers)) p->layer_ev.resize(size_t(pi.m.layers), nullptr);
  for (int32_t l = l0; l < l1; ++l) {
    p->gathered[size_t(l)] = 1;
    if (!deferred) continue;
    if (!p->layer_ev[size_t(l)]) {
      hipError_t e = hipEventCreateWithFlags(&p->layer_ev[size_t(l)], hipEventDisableTiming);
      if (e != hipSuccess) return device_error(p, e, "create a layer event");
    }
    hipError_t e = hipEventRecord(p->layer_ev[size_t(l)], s);
    if (e != hipSuccess) return device_error(p, e, "record a layer event");
    p->layer_ev_live[size_t(l)] = 1;
  }
  return PIC_OK;
}

// Device address of `scratch` on the current device, looked up (with that
// device current) on the first call there and kept.
pic_status noalloc_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(nullptr, e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return set_err(PIC_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_error(nullptr, e, "hipGetSymbolAddress of the no-alloc scratch");
    if (!ptr) return set_err(PIC_EDEVICE, "hipGetSymbolAddress of the no-alloc scratch returned NULL");
    g_scratch_dev[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_dev[dev];
  return PIC_OK;
}

// Order a call that uses the plan's device tables or scratch on stream s
// after every earlier such call: when the previous one went to another
// stream, s waits for everything enqueued on that stream so far (an event
// recorded on it now).  Calls on one stream are ordered by the stream itself
// and cost nothing here.
pic_status order_after_last_call(pic_plan* p, hipStream_t s) {
  if (p->has_last_stream && p->last_stream != s) {
    if (!p->switch_ev) {
      hipError_t e = hipEventCreateWithFlags(&p->switch_ev, hipEventDisableTiming);
      if (e != hipSuccess) return device_error(p, e, "create the stream-switch event");
    }
    hipError_t e = hipEventRecord(p->switch_ev, p->last_stream);
    if (e != hipSuccess) return device_error(p, e, "record the stream-switch event");
    e = hipStreamWaitEvent(s, p->switch_ev, 0);
    if (e != hipSuccess) return device_error(p, e, "wait for the previous stream");
  }
  p->last_stream = s;
  p->has_last_stream = true;
  return PIC_OK;
}

// Before using layer `layer`'s planes on stream s: it must be gathered, and a
// deferred gather on another stream must have completed.
pic_status await_layer(pic_plan* p, int32_t layer, hipStream_t s) {
  if (!p->gathered[size_t(layer)]) return set_err(PIC_ESTATE, "layer %d was not gathered", layer);
  if (p->layer_ev_live[size_t(layer)]) {
    hipError_t e = hipStreamWaitEvent(s, p->layer_ev[size_t(layer)], 0);
    if (e != hipSuccess) return device_error(p, e, "wait for the layer's gather");
  }
  return PIC_OK;
}

}  // namespace

extern "C" {

const char* pic_last_error(void) { return g_err.c_str(); }

const char* pic_version(void) { return "libpic 0.1 (gfx950)"; }

pic_status pic_pool_register(const pic_model* model, void* pool, int64_t pool_bytes,
                             int32_t page_tokens, int32_t n_pages, int32_t n_chunks,
                             const int32_t* chunk_len, const int32_t* chunk_orig,
                             const int32_t* chunk_page_ptr, const int32_t* page_ids,
                             pic_pool** out) {
  if (!out) return set_err(PIC_EINVAL, "out is NULL");
  *out = nullptr;
  pic::PoolInfo info;
  std::string err;
  pic_status st = pic::build_pool(model, pool, pool_bytes, page_tokens, n_pages, n_chunks, chunk_len,
                                  chunk_orig, chunk_page_ptr, page_ids, &info, &err);
  if (st != PIC_OK) return set_err(st, "%s", err.c_str());
  pic_pool* p = new (std::nothrow) pic_pool;
  if (!p) return set_err(PIC_ENOMEM, "out of host memory");
  p->info = std::move(info);
  *out = p;
  return ok();
}

pic_status pic_pool_register_host(const pic_model* model, void* pool, int64_t pool_bytes,
                                  int32_t page_tokens, int32_t n_pages, int32_t n_chunks,
                                  const int32_t* chunk_len, const int32_t* chunk_orig,
                                  const int32_t* chunk_page_ptr, const int32_t* page_ids,
                                  pic_pool** out) {
  if (!out) return set_err(PIC_EINVAL, "out is NULL");
  *out = nullptr;
  if (!pool) return set_err(PIC_EINVAL, "pool pointer is NULL");
  // the memory must be pinned host memory the device can address
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, pool);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return set_err(PIC_EINVAL, "pool is not pinned host memory (allocate it with hipHostMalloc)");
  }
  void* dev = nullptr;
  e = hipHostGetDevicePointer(&dev, pool, 0);
  if (e != hipSuccess || !dev) return set_err(PIC_EDEVICE, "hipHostGetDevicePointer: %s", hipGetErrorString(e));
  pic_status st = pic_pool_register(model, pool, pool_bytes, page_tokens, n_pages, n_chunks, chunk_len,
                                    chunk_orig, chunk_page_ptr, page_ids, out);
  if (st != PIC_OK) return st;
  (*out)->info.device_base = dev;
  (*out)->info.host = true;
  return ok();
}

pic_status pic_pool_release(pic_pool* pool) {
  if (!pool) return set_err(PIC_EINVAL, "pool is NULL");
  if (pool->n_plans > 0) return set_err(PIC_ESTATE, "%d plans still use this pool", pool->n_plans);
  if (pool->cache) return set_err(PIC_ESTATE, "the pool's hot set must be released first");
  if (pool->store) return set_err(PIC_ESTATE, "the pool's chunk store must be released first");
  if (pool->d_page_ids) {
    (void)hipDeviceSynchronize();
    (void)hipFree(pool->d_page_ids);
  }
  delete pool;
  return ok();
}

pic_status pic_cache_create(pic_pool* pool, int32_t capacity_pages, pic_cache** out) {
  if (!out) return set_err(PIC_EINVAL, "out is NULL");
  *out = nullptr;
  if (!pool) return set_err(PIC_EINVAL, "pool is NULL");
  if (!pool->info.host) return set_err(PIC_EINVAL, "a hot set fronts a pool in pinned host memory");
  if (capacity_pages < 1) return set_err(PIC_EINVAL, "capacity_pages %d < 1", capacity_pages);
  if (pool->cache) return set_err(PIC_ESTATE, "the pool already has a hot set");
  if (pool->n_plans > 0) return set_err(PIC_ESTATE, "create the hot set before the pool's plans");
  const pic::PoolInfo& pi = pool->info;
  pic_cache* c = new (std::nothrow) pic_cache(pi.n_pages, capacity_pages, pi.m.layers);
  if (!c) return set_err(PIC_ENOMEM, "out of host memory");
  c->pool = pool;
  (void)hipGetDevice(&c->device);
  const size_t pairs = size_t(pi.m.layers) * size_t(capacity_pages) * 2 * sizeof(int32_t);
  hipError_t e = hipMalloc(reinterpret_cast<void**>(&c->buf), size_t(capacity_pages) * size_t(pi.page_bytes));
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&c->d_pairs), pairs);
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&c->h_pairs), pairs, hipHostMallocDefault);
  c->ev.assign(size_t(pi.m.layers), nullptr);
  c->ev_live.assign(size_t(pi.m.layers), 0);
  for (size_t l = 0; e == hipSuccess && l < c->ev.size(); ++l) e = hipEventCreateWithFlags(&c->ev[l], hipEventDisableTiming);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    if (c->buf) (void)hipFree(c->buf);
    if (c->d_pairs) (void)hipFree(c->d_pairs);
    if (c->h_pairs) (void)hipHostFree(c->h_pairs);
    for (hipEvent_t ev : c->ev)
      if (ev) (void)hipEventDestroy(ev);
    delete c;
    return set_err(PIC_ENOMEM, "hot set of %d pages: %s", capacity_pages, hipGetErrorString(e));
  }
  pool->cache = c;
  *out = c;
  return ok();
}

pic_status pic_cache_get_stats(const pic_cache* c, pic_cache_stats* out) {
  if (!c || !out) return set_err(PIC_EINVAL, "cache or out is NULL");
  out->capacity_pages = c->hs.capacity();
  int64_t resident = 0;
  for (int32_t k = 0; k < c->hs.capacity(); ++k) resident += c->hs.page_in(k) >= 0 ? 1 : 0;
  out->resident_pages = resident;
  out->hits = c->hs.hits;
  out->misses = c->hs.misses;
  out->evictions = c->hs.evictions;
  out->layer_copies = c->hs.layer_copies;
  out->bytes_copied = c->bytes_copied;
  return ok();
}

pic_status pic_cache_release(pic_cache* c) {
  if (!c) return set_err(PIC_EINVAL, "cache is NULL");
  if (c->pool->n_plans > 0) return set_err(PIC_ESTATE, "%d plans still use the pool", c->pool->n_plans);
  (void)hipDeviceSynchronize();
  (void)hipFree(c->buf);
  (void)hipFree(c->d_pairs);
  (void)hipHostFree(c->h_pairs);
  for (hipEvent_t ev : c->ev)
    if (ev) (void)hipEventDestroy(ev);
  c->pool->cache = nullptr;
  delete c;
  return ok();
}

pic_status pic_chunk_file_write(const pic_model* model, int32_t page_tokens, int32_t len, int32_t orig,
                                const void* pages, const int32_t* page_list, const char* path) {
  std::string err;
  const pic_status st = pic::write_chunk_file(model, page_tokens, len, orig, pages, page_list, path, &err);
  if (st != PIC_OK) return set_err(st, "%s", err.c_str());
  return ok();
}

pic_status pic_store_open(pic_pool* pool, void* dst, int64_t dst_bytes, const char* const* paths,
                          int32_t threads, pic_store** out) {
  if (!out) return set_err(PIC_EINVAL, "out is NULL");
  *out = nullptr;
  if (!pool) return set_err(PIC_EINVAL, "pool is NULL");
  const bool attach = pool->info.host && dst == pool->info.base;
  if (attach) {
    if (pool->store) return set_err(PIC_ESTATE, "the pool already has a chunk store");
    if (pool->n_plans > 0) return set_err(PIC_ESTATE, "open the pool's chunk store before its plans");
  } else if (dst == pool->info.base || dst == pool->info.device_base) {
    return set_err(PIC_EINVAL, "the pool's memory is device memory; the store fills host memory");
  }
  std::unique_ptr<pic::ChunkStore> cs;
  std::string err;
  const pic_status st = pic::ChunkStore::open(pool->info, static_cast<char*>(dst), dst_bytes, paths, threads, &cs, &err);
  if (st != PIC_OK) return set_err(st, "%s", err.c_str());
  pic_store* s = new (std::nothrow) pic_store;
  if (!s) return set_err(PIC_ENOMEM, "out of host memory");
  s->pool = pool;
  s->attached = attach;
  s->cs = std::move(cs);
  if (attach) pool->store = s;
  *out = s;
  return ok();
}

pic_status pic_store_request(pic_store* s, int32_t batch, const int32_t* span_ptr, const pic_span* spans) {
  if (!s) return set_err(PIC_EINVAL, "store is NULL");
  const pic::PoolInfo& pi = s->cs->pool();
  if (batch < 0) return set_err(PIC_EINVAL, "batch must be >= 0");
  if (batch == 0) return ok();
  if (!span_ptr) return set_err(PIC_EINVAL, "span_ptr is NULL");
  if (span_ptr[0] != 0) return set_err(PIC_EINVAL, "span_ptr[0] must be 0");
  for (int32_t b = 0; b < batch; ++b)
    if (span_ptr[b + 1] < span_ptr[b]) return set_err(PIC_EINVAL, "span_ptr decreases at %d", b);
  const int32_t n = span_ptr[batch];
  if (n > 0 && !spans) return set_err(PIC_EINVAL, "spans is NULL");
  std::vector<int32_t> pages;
  for (int32_t i = 0; i < n; ++i) {
    const pic_span& sp = spans[i];
    if (sp.chunk < 0 || sp.chunk >= pi.n_chunks)
      return set_err(PIC_ERANGE, "span %d: chunk %d outside [0, %d)", i, sp.chunk, pi.n_chunks);
    const int32_t len = pi.chunk_len[size_t(sp.chunk)];
    if (sp.s < 0 || sp.s > sp.e || sp.e >= len)
      return set_err(PIC_ERANGE, "span %d: need 0 <= s <= e < len, got s=%d e=%d len=%d", i, sp.s, sp.e, len);
    const int32_t q0 = pi.chunk_page_ptr[size_t(sp.chunk)];
    for (int32_t j = sp.s / pi.page_tokens; j <= sp.e / pi.page_tokens; ++j) pages.push_back(q0 + j);
  }
  std::sort(pages.begin(), pages.end());
  pages.erase(std::unique(pages.begin(), pages.end()), pages.end());
  s->cs->request_logical(pages);
  return ok();
}

pic_status pic_store_wait(pic_store* s) {
  if (!s) return set_err(PIC_EINVAL, "store is NULL");
  std::string err;
  const pic_status st = s->cs->wait(&err);
  if (st != PIC_OK) return set_err(st, "%s", err.c_str());
  return ok();
}

pic_status pic_store_forget(pic_store* s, int32_t drop_os_cache) {
  if (!s) return set_err(PIC_EINVAL, "store is NULL");
  std::string err;
  const pic_status st = s->cs->forget(drop_os_cache != 0, &err);
  if (st != PIC_OK) return set_err(st, "%s", err.c_str());
  return ok();
}

pic_status pic_store_get_stats(pic_store* s, pic_store_stats* out) {
  if (!s || !out) return set_err(PIC_EINVAL, "store or out is NULL");
  const pic::StoreStats st = s->cs->stats();
  out->resident_pages = st.resident_pages;
  out->requested = st.requested;
  out->hits = st.hits;
  out->pages_read = st.pages_read;
  out->bytes_read = st.bytes_read;
  out->reads = st.reads;
  out->wait_seconds = st.wait_seconds;
  return ok();
}

pic_status pic_store_release(pic_store* s) {
  if (!s) return set_err(PIC_EINVAL, "store is NULL");
  if (s->attached && s->pool->n_plans > 0)
    return set_err(PIC_ESTATE, "%d plans still use the pool", s->pool->n_plans);
  if (s->attached) s->pool->store = nullptr;
  delete s;   // waits for the loads in flight
  return ok();
}

pic_status pic_plan_create(pic_pool* pool, pic_plan** out) {
  if (!out) return set_err(PIC_EINVAL, "out is NULL");
  *out = nullptr;
  if (!pool) return set_err(PIC_EINVAL, "pool is NULL");
  pic_plan* p = new (std::nothrow) pic_plan;
  if (!p) return set_err(PIC_ENOMEM, "out of host memory");
  p->pool = pool;
  pool->n_plans++;
  *out = p;
  return ok();
}

pic_status pic_plan_release(pic_plan* p) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (p->ws || p->staging || p->staging_ev) (void)hipDeviceSynchronize();
  if (p->ws) (void)hipFree(p->ws);
  if (p->dws) (void)hipFree(p->dws);
  if (p->staging) (void)hipHostFree(p->staging);
  if (p->staging_ev) (void)hipEventDestroy(p->staging_ev);
  if (p->plan_ev) (void)hipEventDestroy(p->plan_ev);
  if (p->switch_ev) (void)hipEventDestroy(p->switch_ev);
  for (hipEvent_t e : p->layer_ev)
    if (e) (void)hipEventDestroy(e);
  for (auto& v : p->events)
    for (auto& pr : v) {
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
  if (p->pool->cache) p->pool->cache->hs.unpin(reinterpret_cast<int64_t>(p));
  p->pool->n_plans--;
  delete p;
  return ok();
}

pic_status pic_assemble(pic_plan* p, int32_t batch, const int32_t* span_ptr, const pic_span* spans,
                        const int32_t* new_ptr, const int32_t* new_pos, void* asm_k, void* asm_v,
                        int64_t asm_rows_capacity, int32_t flags, void* stream) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (p->failed) return set_err(PIC_ESTATE, "plan is unusable after a device error");
  if (flags & ~(PIC_ASSEMBLE_PLAN_ONLY | PIC_ASSEMBLE_DRY_RUN | PIC_ASSEMBLE_DEFER_GATHER |
                PIC_ASSEMBLE_QUERY_ROTATION | PIC_ASSEMBLE_VALUES_IN_POOL))
    return set_err(PIC_EINVAL, "unknown flags 0x%x", flags);
  if ((flags & PIC_ASSEMBLE_PLAN_ONLY) && (flags & PIC_ASSEMBLE_DEFER_GATHER))
    return set_err(PIC_EINVAL, "PIC_ASSEMBLE_PLAN_ONLY and PIC_ASSEMBLE_DEFER_GATHER exclude each other");
  if (flags & PIC_ASSEMBLE_QUERY_ROTATION)
    return set_err(PIC_EUNSUPPORTED,
                   "PIC_ASSEMBLE_QUERY_ROTATION is retired: scoring against queries rotated back by each "
                   "span's delta skips the storage rounding of the re-rotated keys, so it does not reproduce "
                   "the assembled cache's results; variant F rotates the keys on load instead");
  const bool values_in_pool = (flags & PIC_ASSEMBLE_VALUES_IN_POOL) != 0;
  if (values_in_pool && (flags & PIC_ASSEMBLE_PLAN_ONLY))
    return set_err(PIC_EINVAL, "PIC_ASSEMBLE_VALUES_IN_POOL applies to a gathered batch, not PLAN_ONLY");
  if (values_in_pool && !(p->pool->info.m.dtype == PIC_BF16 && p->pool->info.m.head_dim == 128))
    return set_err(PIC_EUNSUPPORTED, "PIC_ASSEMBLE_VALUES_IN_POOL is implemented for bf16 with head_dim 128");
  const bool defer = (flags & PIC_ASSEMBLE_DEFER_GATHER) != 0;
  const bool dry = (flags & PIC_ASSEMBLE_DRY_RUN) != 0;
  const bool plan_only = (flags & PIC_ASSEMBLE_PLAN_ONLY) != 0;
  if (asm_rows_capacity < 0) return set_err(PIC_EINVAL, "asm_rows_capacity must be >= 0");
  if (!dry) {
    if (!asm_k || !asm_v) return set_err(PIC_EINVAL, "asm_k and asm_v are required");
    if (!aligned16(asm_k) || !aligned16(asm_v))
      return set_err(PIC_EALIGN, "assembled buffers must be 16-byte aligned");
  }
  const pic::PoolInfo& pi = p->pool->info;
  pic::HostPlan hp;
  std::string err;
  pic_status st = pic::build_plan(pi, batch, span_ptr, spans, new_ptr, new_pos, asm_rows_capacity,
                                  p->decode_rows_next, &hp, &err);
  if (st != PIC_OK) return set_err(st, "%s", err.c_str());
  if (pi.m.dtype == PIC_BF16 && pi.m.head_dim == 128) {
    const pic::AttnSplit sp = pic::choose_attention_split(
        hp, pi.m.kv_heads, pi.m.group, pic::kAttnColsPerWG, pic::kAttnRowsPerTile, pic::kAttnTargetWGs,
        pic::kAttnMaxSplit, /*min_tiles_per_split=*/3, pic::kAttnMinTilesAcross);
    pic::build_attention_work(&hp, pi.m.kv_heads, pi.m.group, pic::kAttnColsPerWG, pic::kAttnRowsPerTile, sp);
    pic::build_wg_map(&hp, pic::kXcds, pic::kAttnTargetWGs / pic::kXcds);
  }
  p->dec.step = -1;  // decode tables describe the previous batch
  if (dry) {
    p->hp = std::move(hp);
    p->has_batch = true;
    p->materialized = false;
    p->values_in_pool = values_in_pool;
    p->asm_k = p->asm_v = nullptr;
    p->cap = asm_rows_capacity;
    return ok();
  }
  if (!pic::gather_supported(pi.m.dtype, pi.m.head_dim))
    return set_err(PIC_EUNSUPPORTED, "head_dim %d is not implemented (64 and 128 are)",
                   pi.m.head_dim);
  st = check_device(p);
  if (st != PIC_OK) return st;
  st = ensure_pool_device(p->pool);
  if (st != PIC_OK) return st;

  // pages the batch's spans cover (indices into the pool's page table)
  std::vector<int32_t> logical;
  if (p->pool->cache || p->pool->store) logical = pic::covered_pages(hp, pi.page_tokens);
  // with chunk files: the covered pages that are not in host memory yet are
  // read now (an earlier pic_store_request may have started them), before
  // anything can read them
  if (pic_store* ps = p->pool->store) {
    ps->cs->request_logical(logical);
    std::string lerr;
    st = ps->cs->wait(&lerr);
    if (st != PIC_OK) return set_err(st, "%s", lerr.c_str());
  }
  // with a hot set: pin the pages the batch covers (this changes nothing
  // when they do not fit) and map the pool's pages to their slots
  std::vector<int32_t> page_tab;
  if (pic_cache* c = p->pool->cache) {
    std::vector<int32_t> phys(logical.size());
    for (size_t i = 0; i < logical.size(); ++i) phys[i] = pi.page_ids[size_t(logical[i])];
    std::string perr;
    if (!c->hs.pin(reinterpret_cast<int64_t>(p), phys, &perr)) return set_err(PIC_ERANGE, "%s", perr.c_str());
    page_tab.assign(pi.page_ids.size(), 0);
    for (int32_t q : logical) page_tab[size_t(q)] = c->hs.slot_of(pi.page_ids[size_t(q)]);
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  st = order_after_last_call(p, s);
  if (st != PIC_OK) return st;
  // deferred gathers of the previous batch may still read its tables
  for (size_t l = 0; l < p->layer_ev_live.size(); ++l) {
    if (!p->layer_ev_live[l]) continue;
    hipError_t e = hipStreamWaitEvent(s, p->layer_ev[l], 0);
    if (e != hipSuccess) return device_error(p, e, "wait for the previous batch's gathers");
  }
  p->hp = std::move(hp);
  p->has_batch = false;
  p->values_in_pool = values_in_pool;
  p->gathered.assign(size_t(pi.m.layers), 0);
  p->layer_ev_live.assign(size_t(pi.m.layers), 0);
  p->asm_k = static_cast<char*>(asm_k);
  p->asm_v = static_cast<char*>(asm_v);
  p->cap = asm_rows_capacity;
  const pic::HostPlan& h = p->hp;
  if (batch == 0 || h.rows == 0) {
    p->has_batch = true;
    p->materialized = !plan_only && !defer;
    if (!plan_only) p->gathered.assign(size_t(pi.m.layers), 1);
    return ok();
  }

  layout_workspace(p);
  st = ensure_capacity(p);
  if (st != PIC_OK) return st;
  if (p->staging_pending) {
    hipError_t e = hipEventSynchronize(p->staging_ev);
    if (e != hipSuccess) return device_error(p, e, "wait for the previous plan upload");
    p->staging_pending = false;
  }
  std::vector<double> omega(size_t(pi.m.head_dim) / 2);
  for (size_t k = 0; k < omega.size(); ++k)
    omega[k] = std::pow(pi.m.theta, -2.0 * double(k) / double(pi.m.head_dim));
  put(p->staging, p->off_spans, h.spans);
  put(p->staging, p->off_crow, h.crow);
  put(p->staging, p->off_reqs, h.reqs);
  put(p->staging, p->off_new_pos, h.new_pos);
  put(p->staging, p->off_new_row, h.new_row);
  put(p->staging, p->off_new_req, h.new_req);
  put(p->staging, p->off_work, h.work);
  put(p->staging, p->off_omega, omega);
  put(p->staging, p->off_wg_map, h.wg_map);
  put(p->staging, p->off_item_map, h.item_map);
  put(p->staging, p->off_page_tab, page_tab);
  {
    Timed tm(p, 3, s);
    hipError_t e = hipMemcpyAsync(p->ws, p->staging, p->blob_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return device_error(p, e, "plan upload");
    e = hipEventRecord(p->staging_ev, s);
    if (e != hipSuccess) return device_error(p, e, "record the upload event");
    p->staging_pending = true;

    pic::PlanArgs pa;
    pa.spans = reinterpret_cast<const pic::SpanRec*>(p->ws + p->off_spans);
    pa.crow = reinterpret_cast<const int32_t*>(p->ws + p->off_crow);
    pa.new_pos = reinterpret_cast<const int32_t*>(p->ws + p->off_new_pos);
    pa.new_row = reinterpret_cast<const int32_t*>(p->ws + p->off_new_row);
    pa.page_ids = p->pool->cache ? reinterpret_cast<const int32_t*>(p->ws + p->off_page_tab) : p->pool->d_page_ids;
    pa.omega = reinterpret_cast<const double*>(p->ws + p->off_omega);
    pa.n_spans = h.n_spans;
    pa.n_new = int32_t(h.new_rows);
    pa.page_shift = pi.page_shift;
    pa.half_dim = pi.m.head_dim / 2;
    pa.prefix_rows = h.prefix_rows;
    pa.pos = reinterpret_cast<int32_t*>(p->ws + p->off_pos);
    pa.rowsrc = reinterpret_cast<int2*>(p->ws + p->off_rowsrc);
    pa.gsrc = reinterpret_cast<int4*>(p->ws + p->off_gsrc);
    pa.phase_tab = reinterpret_cast<pic::Phase*>(p->ws + p->off_phase_tab);
    pa.per_position = pi.m.key_storage == PIC_KEYS_UNROTATED;
    pa.phase_rows = h.phase_rows;
    pa.phase_new = reinterpret_cast<pic::Phase*>(p->ws + p->off_phase_new);
    pa.reqs = reinterpret_cast<const pic::ReqRec*>(p->ws + p->off_reqs);
    pa.batch = h.batch;
    pa.n_tiles = h.n_tiles;
    pa.tile_pos = reinterpret_cast<int2*>(p->ws + p->off_tile_pos);
    pa.split_count = reinterpret_cast<int32_t*>(p->ws + p->off_count);
    pa.n_slots = h.n_slots;
    e = pic::launch_plan(pa, s);
    if (e != hipSuccess) return device_error(p, e, "plan kernels");
  }
  if (!p->plan_ev) {
    hipError_t e = hipEventCreateWithFlags(&p->plan_ev, hipEventDisableTiming);
    if (e != hipSuccess) return device_error(p, e, "create the plan event");
  }
  if (!p->switch_ev) {
    hipError_t e = hipEventCreateWithFlags(&p->switch_ev, hipEventDisableTiming);
    if (e != hipSuccess) return device_error(p, e, "create the stream-switch event");
  }
  {
    hipError_t e = hipEventRecord(p->plan_ev, s);
    if (e != hipSuccess) return device_error(p, e, "record the plan event");
  }
  p->has_batch = true;
  if (!plan_only && !defer) {
    st = gather_layers(p, 0, pi.m.layers, s, /*deferred=*/false);
    if (st != PIC_OK) return st;
  }
  p->materialized = !plan_only && !defer;
  return ok();
}

pic_status pic_gather_layers(pic_plan* p, int32_t layer_begin, int32_t layer_end, void* stream) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (p->failed) return set_err(PIC_ESTATE, "plan is unusable after a device error");
  if (!p->has_batch || !p->asm_k) return set_err(PIC_ESTATE, "no assembled batch with planes");
  const int32_t L = p->pool->info.m.layers;
  if (layer_begin < 0 || layer_end > L || layer_begin > layer_end)
    return set_err(PIC_ERANGE, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end, L);
  pic_status st = check_device(p);
  if (st != PIC_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->plan_ev) {
    hipError_t e = hipStreamWaitEvent(s, p->plan_ev, 0);
    if (e != hipSuccess) return device_error(p, e, "wait for the plan kernels");
  }
  st = gather_layers(p, layer_begin, layer_end, s, /*deferred=*/true);
  if (st != PIC_OK) return st;
  bool all = true;
  for (char g : p->gathered) all = all && g;
  p->materialized = all;
  return ok();
}

}  // extern "C"

namespace {

pic_status prefill_impl(pic_plan* p, int32_t layer, const void* q, const void* k_new, const void* v_new,
                        void* out, int32_t variant, void* stream, const PrefillScratch* ext) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (p->failed) return set_err(PIC_ESTATE, "plan is unusable after a device error");
  if (!p->has_batch || !p->asm_k)
    return set_err(PIC_ESTATE, "no assembled batch (call pic_assemble without DRY_RUN first)");
  const pic::PoolInfo& pi = p->pool->info;
  const pic::ModelInfo& m = pi.m;
  if (layer < 0 || layer >= m.layers)
    return set_err(PIC_ERANGE, "layer %d outside [0, %d)", layer, m.layers);
  if (variant != PIC_VARIANT_MATERIALIZED && variant != PIC_VARIANT_FUSED)
    return set_err(PIC_EINVAL, "unknown variant %d", variant);
  const bool fused = variant == PIC_VARIANT_FUSED;
  if (!fused && (p->gathered.empty() || !p->gathered[size_t(layer)]))
    return set_err(PIC_ESTATE, "the materialised variant needs layer %d gathered (an assemble without "
                   "PLAN_ONLY or DEFER_GATHER, or pic_gather_layers)", layer);
  if (!pic::attention_supported(m.dtype, m.head_dim, fused))
    return set_err(PIC_EUNSUPPORTED, "attention variant %d is not implemented for dtype %d, head_dim %d",
                   variant, m.dtype, m.head_dim);
  const pic::HostPlan& h = p->hp;
  if (h.new_rows == 0) return ok();
  // the plan's own scratch, or the caller-provided one
  PrefillScratch sc;
  if (ext) {
    sc = *ext;
  } else {
    sc.q_rot = p->ws + p->off_qrot;
    sc.opart = reinterpret_cast<float*>(p->ws + p->off_opart);
    sc.ml = reinterpret_cast<float2*>(p->ws + p->off_ml);
    sc.spart = reinterpret_cast<float*>(p->ws + p->off_spart);
    sc.sml = reinterpret_cast<float*>(p->ws + p->off_sml);
    sc.count = reinterpret_cast<int32_t*>(p->ws + p->off_count);
    sc.clear_count = false;   // cleared by the plan kernels, left at 0 by every launch
  }
  // timing brackets create events on first use: only on the plan's own path
  const bool timed = p->timing && !ext;
  if (!q || !k_new || !v_new || !out) return set_err(PIC_EINVAL, "q, k_new, v_new and out are required");
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return set_err(PIC_EALIGN, "q, k_new, v_new and out must be 16-byte aligned");
  pic_status st = check_device(p);
  if (st != PIC_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = order_after_last_call(p, s);
  if (st != PIC_OK) return st;
  if (!fused) {
    st = await_layer(p, layer, s);
    if (st != PIC_OK) return st;
  }
  if (sc.clear_count && h.n_slots > 0 && h.n_split_wg > 1) {
    hipError_t e = pic::launch_fill_zero(sc.count, h.n_slots, s);
    if (e != hipSuccess) return device_error(p, e, "clear the merge counters");
  }
  const int64_t plane_bytes = p->cap * m.row_bytes;
  char* kpl = p->asm_k + int64_t(layer) * m.kv_heads * plane_bytes;
  char* vpl = p->asm_v + int64_t(layer) * m.kv_heads * plane_bytes;
  {
    Timed tm(p, 1, s, timed);
    pic::PrologueArgs pa;
    pa.q = static_cast<const char*>(q);
    pa.k_new = static_cast<const char*>(k_new);
    pa.v_new = static_cast<const char*>(v_new);
    pa.new_pos = reinterpret_cast<const int32_t*>(p->ws + p->off_new_pos);
    pa.new_row = reinterpret_cast<const int32_t*>(p->ws + p->off_new_row);
    pa.phase_new = reinterpret_cast<const pic::Phase*>(p->ws + p->off_phase_new);
    pa.q_rot = sc.q_rot;
    pa.asm_k = kpl;
    pa.asm_v = vpl;
    pa.cap = p->cap;
    pa.n_new = int32_t(h.new_rows);
    pa.q_heads = m.q_heads;
    pa.kv_heads = m.kv_heads;
    hipError_t e = pic::launch_prologue(m.dtype, m.head_dim, pa, s);
    if (e != hipSuccess) return device_error(p, e, "prologue kernel");
  }
  // attention that reads prefix rows in the pool reads them in the hot set
  if (fused || p->values_in_pool) {
    Timed tm(p, 0, s, timed);
    pic_status fst = cache_fill(p, layer, layer + 1, s);
    if (fst != PIC_OK) return fst;
  }
  {
    Timed tm(p, 2, s, timed);
    hipError_t e;
    if (m.dtype == PIC_BF16) {
      pic::AttnArgs aa{};
      aa.q_rot = reinterpret_cast<const uint16_t*>(sc.q_rot);
      aa.k_plane = reinterpret_cast<const uint16_t*>(kpl);
      aa.v_plane = reinterpret_cast<const uint16_t*>(vpl);
      aa.cap = p->cap;
      aa.pos = reinterpret_cast<const int32_t*>(p->ws + p->off_pos);
      aa.tile_pos = reinterpret_cast<const int2*>(p->ws + p->off_tile_pos);
      aa.reqs = reinterpret_cast<const pic::ReqRec*>(p->ws + p->off_reqs);
      aa.new_pos = reinterpret_cast<const int32_t*>(p->ws + p->off_new_pos);
      aa.work = reinterpret_cast<const pic::AttnWork*>(p->ws + p->off_work);
      aa.n_work = int32_t(h.work.size());
      aa.q_heads = m.q_heads;
      aa.group = m.group;
      aa.n_new = int32_t(h.new_rows);
      aa.n_split_out = h.n_split_out;
      aa.paired = h.n_split > 1;
      aa.n_split_wg = h.n_split_wg;
      aa.split_count = sc.count;
      aa.spart = sc.spart;
      aa.sml = sc.sml;
      aa.decode = 0;
      aa.scale_log2 = float(1.4426950408889634 / std::sqrt(double(m.head_dim)));
      aa.out = static_cast<uint16_t*>(out);
      aa.opart = sc.opart;
      aa.ml = sc.ml;
      aa.pool = pool_addr(p->pool);
      aa.rowsrc = reinterpret_cast<const int2*>(p->ws + p->off_rowsrc);
      aa.phase_tab = reinterpret_cast<const pic::Phase*>(p->ws + p->off_phase_tab);
      aa.page_bytes = pi.page_bytes;
      aa.kv_plane_off = int64_t(layer) * 2 * m.kv_heads * pi.page_tokens * m.row_bytes;
      aa.v_off = int64_t(m.kv_heads) * pi.page_tokens * m.row_bytes;
      aa.page_shift = pi.page_shift;
      aa.page_tokens = pi.page_tokens;
      aa.kv_heads = m.kv_heads;
      aa.v_pool = !fused && p->values_in_pool ? 1 : 0;
      // launch order: the fused variant without row splits runs one item per
      // workgroup, every other kernel a pair
      const bool unpaired = fused && !aa.paired;
      const std::vector<int32_t>& order = unpaired ? h.item_map : h.wg_map;
      aa.wg_map = order.empty() ? nullptr
                                : reinterpret_cast<const int32_t*>(p->ws + (unpaired ? p->off_item_map : p->off_wg_map));
      aa.n_wg = int32_t(order.size());
      e = pic::launch_attention_bf16(aa, fused, s);
    } else {
      pic::AttnF32Args aa;
      aa.q_rot = sc.q_rot;
      aa.k_plane = kpl;
      aa.v_plane = vpl;
      aa.cap = p->cap;
      aa.pos = reinterpret_cast<const int32_t*>(p->ws + p->off_pos);
      aa.reqs = reinterpret_cast<const pic::ReqRec*>(p->ws + p->off_reqs);
      aa.new_pos = reinterpret_cast<const int32_t*>(p->ws + p->off_new_pos);
      aa.new_req = reinterpret_cast<const int32_t*>(p->ws + p->off_new_req);
      aa.n_new = int32_t(h.new_rows);
      aa.q_heads = m.q_heads;
      aa.group = m.group;
      aa.out = static_cast<char*>(out);
      e = pic::launch_attention_f32(m.head_dim, aa, s);
    }
    if (e != hipSuccess) return device_error(p, e, "attention kernel");
  }
  return ok();
}

}  // namespace

extern "C" {

pic_status pic_query_prefill(pic_plan* p, int32_t layer, const void* q, const void* k_new,
                             const void* v_new, void* out, int32_t variant, void* stream) {
  return prefill_impl(p, layer, q, k_new, v_new, out, variant, stream, nullptr);
}

pic_status pic_query_prefill_noalloc(pic_plan* p, int32_t layer, const void* q, const void* k_new,
                                     const void* v_new, void* out, int32_t variant, void* stream) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (p->failed) return set_err(PIC_ESTATE, "plan is unusable after a device error");
  if (!p->has_batch || !p->asm_k)
    return set_err(PIC_ESTATE, "no assembled batch (call pic_assemble without DRY_RUN first)");
  const ScratchLayout sl = prefill_scratch_layout(p->pool->info.m, p->hp);
  if (sl.bytes > kNoAllocScratchBytes)
    return set_err(PIC_ERANGE,
                   "the batch needs %zu bytes of prefill scratch; pic_query_prefill_noalloc has %zu "
                   "(use pic_query_prefill)",
                   sl.bytes, kNoAllocScratchBytes);
  char* base = nullptr;
  pic_status st = noalloc_scratch(&base);
  if (st != PIC_OK) return st;
  PrefillScratch sc;
  sc.q_rot = base + sl.q_rot;
  sc.opart = reinterpret_cast<float*>(base + sl.opart);
  sc.ml = reinterpret_cast<float2*>(base + sl.ml);
  sc.spart = reinterpret_cast<float*>(base + sl.spart);
  sc.sml = reinterpret_cast<float*>(base + sl.sml);
  sc.count = reinterpret_cast<int32_t*>(base + sl.count);
  sc.clear_count = true;
  return prefill_impl(p, layer, q, k_new, v_new, out, variant, stream, &sc);
}

pic_status pic_plan_set_decode_rows(pic_plan* p, int32_t rows) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (rows < 0) return set_err(PIC_EINVAL, "decode rows must be >= 0");
  p->decode_rows_next = rows;
  return ok();
}

pic_status pic_decode_layer(pic_plan* p, int32_t layer, int32_t step, const void* q, const void* k_new,
                            const void* v_new, void* out, int32_t variant, void* stream) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (p->failed) return set_err(PIC_ESTATE, "plan is unusable after a device error");
  if (!p->has_batch || !p->asm_k) return set_err(PIC_ESTATE, "no assembled batch");
  const pic::HostPlan& h = p->hp;
  const pic::PoolInfo& pi = p->pool->info;
  const pic::ModelInfo& m = pi.m;
  if (layer < 0 || layer >= m.layers) return set_err(PIC_ERANGE, "layer %d outside [0, %d)", layer, m.layers);
  if (step < 0 || step >= h.decode_rows)
    return set_err(PIC_ERANGE, "decode step %d outside the %d reserved rows", step, h.decode_rows);
  if (variant != PIC_VARIANT_MATERIALIZED && variant != PIC_VARIANT_FUSED)
    return set_err(PIC_EINVAL, "unknown variant %d", variant);
  const bool fused = variant == PIC_VARIANT_FUSED;
  if (!fused && (p->gathered.empty() || !p->gathered[size_t(layer)]))
    return set_err(PIC_ESTATE, "variant M needs layer %d gathered", layer);
  if (m.dtype != PIC_BF16 || m.head_dim != 128)
    return set_err(PIC_EUNSUPPORTED, "decode is implemented for bf16 with head_dim 128");
  if (h.batch == 0) return ok();
  if (!q || !k_new || !v_new || !out) return set_err(PIC_EINVAL, "q, k_new, v_new and out are required");
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return set_err(PIC_EALIGN, "q, k_new, v_new and out must be 16-byte aligned");
  pic_status st = check_device(p);
  if (st != PIC_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = order_after_last_call(p, s);
  if (st != PIC_OK) return st;
  if (!fused) {
    st = await_layer(p, layer, s);
    if (st != PIC_OK) return st;
  }

  // the attention kernel rotates the queries and adds the token's own row
  // itself when one wave holds a column block's query heads (no prologue and
  // no merge kernel); wider groups take the prologue and merge_kernel
  const bool own = m.group <= 32;
  if (p->dec.step != step || p->dec.own_row != own) {
    pic::build_decode(h, m.kv_heads, step, pic::kAttnRowsPerTile, pic::kDecodeTargetItems, pic::kAttnMaxSplit,
                      /*min_tiles_per_split=*/2, own, &p->dec);
    const pic::DecodePlan& d = p->dec;
    size_t o = 0;
    auto take = [&o](size_t bytes) {
      size_t at = o;
      o = align256(o + bytes);
      return at;
    };
    const size_t nb = size_t(h.batch);
    p->d_pos = take(nb * sizeof(int32_t));
    p->d_row = take(nb * sizeof(int32_t));
    p->d_reqs = take(nb * sizeof(pic::ReqRec));
    p->d_work = take(d.work.size() * sizeof(pic::AttnWork));
    p->d_blob = o;
    p->d_phase = take(nb * (m.head_dim / 2) * sizeof(pic::Phase));
    // rotated queries (prologue path only) and merge_kernel's partials
    p->d_qrot = take(own ? 0 : nb * m.q_heads * m.row_bytes);
    const size_t np = d.n_split_out > 1 ? size_t(d.n_split_out) : 0;
    p->d_opart = take(np * nb * m.q_heads * m.head_dim * sizeof(float));
    p->d_ml = take(np * nb * m.q_heads * sizeof(float2));
    p->d_bytes = o;
    if (p->d_bytes > p->dws_cap) {
      if (p->dws) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return device_error(p, e, "synchronise before growing the decode tables");
        (void)hipFree(p->dws);
        p->dws = nullptr;
        p->dws_cap = 0;
      }
      hipError_t e = hipMalloc(reinterpret_cast<void**>(&p->dws), p->d_bytes);
      if (e != hipSuccess) {
        p->dws = nullptr;
        p->dec.step = -1;
        return set_err(PIC_ENOMEM, "hipMalloc of %zu decode bytes failed: %s", p->d_bytes, hipGetErrorString(e));
      }
      p->dws_cap = p->d_bytes;
    }
    if (p->staging_pending) {
      hipError_t e = hipEventSynchronize(p->staging_ev);
      if (e != hipSuccess) return device_error(p, e, "wait for the previous upload");
      p->staging_pending = false;
    }
    st = ensure_staging(p, p->d_blob);
    if (st != PIC_OK) {
      p->dec.step = -1;
      return st;
    }
    put(p->staging, p->d_pos, d.pos);
    put(p->staging, p->d_row, d.row);
    put(p->staging, p->d_reqs, d.reqs);
    put(p->staging, p->d_work, d.work);
    hipError_t e = hipMemcpyAsync(p->dws, p->staging, p->d_blob, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return device_error(p, e, "decode table upload");
    e = hipEventRecord(p->staging_ev, s);
    if (e != hipSuccess) return device_error(p, e, "record the upload event");
    p->staging_pending = true;
    pic::DecodePlanArgs da{};
    da.dec_pos = reinterpret_cast<const int32_t*>(p->dws + p->d_pos);
    da.dec_row = reinterpret_cast<const int32_t*>(p->dws + p->d_row);
    da.omega = reinterpret_cast<const double*>(p->ws + p->off_omega);
    da.batch = h.batch;
    da.half_dim = m.head_dim / 2;
    da.phase = reinterpret_cast<pic::Phase*>(p->dws + p->d_phase);
    da.pos = reinterpret_cast<int32_t*>(p->ws + p->off_pos);
    e = pic::launch_decode_plan(da, s);
    if (e != hipSuccess) return device_error(p, e, "decode plan kernel");
  }
  const pic::DecodePlan& d = p->dec;
  const int64_t plane_bytes = p->cap * m.row_bytes;
  char* kpl = p->asm_k + int64_t(layer) * m.kv_heads * plane_bytes;
  char* vpl = p->asm_v + int64_t(layer) * m.kv_heads * plane_bytes;
  if (!own) {
    Timed tm(p, 1, s);
    pic::PrologueArgs pa;
    pa.q = static_cast<const char*>(q);
    pa.k_new = static_cast<const char*>(k_new);
    pa.v_new = static_cast<const char*>(v_new);
    pa.new_pos = reinterpret_cast<const int32_t*>(p->dws + p->d_pos);
    pa.new_row = reinterpret_cast<const int32_t*>(p->dws + p->d_row);
    pa.phase_new = reinterpret_cast<const pic::Phase*>(p->dws + p->d_phase);
    pa.q_rot = p->dws + p->d_qrot;
    pa.asm_k = kpl;
    pa.asm_v = vpl;
    pa.cap = p->cap;
    pa.n_new = h.batch;
    pa.q_heads = m.q_heads;
    pa.kv_heads = m.kv_heads;
    hipError_t e = pic::launch_prologue(m.dtype, m.head_dim, pa, s);
    if (e != hipSuccess) return device_error(p, e, "decode prologue kernel");
  }
  if (fused || p->values_in_pool) {
    Timed tm(p, 0, s);
    pic_status fst = cache_fill(p, layer, layer + 1, s);
    if (fst != PIC_OK) return fst;
  }
  {
    Timed tm(p, 2, s);
    pic::AttnArgs aa{};
    aa.q_rot = own ? static_cast<const uint16_t*>(q) : reinterpret_cast<const uint16_t*>(p->dws + p->d_qrot);
    aa.k_plane = reinterpret_cast<const uint16_t*>(kpl);
    aa.v_plane = reinterpret_cast<const uint16_t*>(vpl);
    aa.cap = p->cap;
    aa.pos = reinterpret_cast<const int32_t*>(p->ws + p->off_pos);
    aa.tile_pos = nullptr;
    aa.reqs = reinterpret_cast<const pic::ReqRec*>(p->dws + p->d_reqs);
    aa.new_pos = reinterpret_cast<const int32_t*>(p->dws + p->d_pos);
    aa.work = reinterpret_cast<const pic::AttnWork*>(p->dws + p->d_work);
    aa.n_work = int32_t(d.work.size());
    aa.wg_map = nullptr;
    aa.n_wg = 0;
    aa.q_heads = m.q_heads;
    aa.group = m.group;
    aa.n_new = h.batch;
    aa.n_split_out = d.n_split_out;
    aa.paired = d.n_split_out < d.n_split;
    aa.n_split_wg = 1;
    aa.split_count = nullptr;
    aa.spart = nullptr;
    aa.sml = nullptr;
    aa.decode = 1;
    aa.dec_own = own ? 1 : 0;
    aa.dec_split = d.n_split;
    aa.k_new = static_cast<const uint16_t*>(k_new);
    aa.v_new = static_cast<const uint16_t*>(v_new);
    aa.dec_phase = reinterpret_cast<const pic::Phase*>(p->dws + p->d_phase);
    aa.dec_row = reinterpret_cast<const int32_t*>(p->dws + p->d_row);
    aa.k_own = reinterpret_cast<uint16_t*>(kpl);
    aa.v_own = reinterpret_cast<uint16_t*>(vpl);
    aa.v_pool = !fused && p->values_in_pool ? 1 : 0;
    aa.scale_log2 = float(1.4426950408889634 / std::sqrt(double(m.head_dim)));
    aa.out = static_cast<uint16_t*>(out);
    aa.opart = reinterpret_cast<float*>(p->dws + p->d_opart);
    aa.ml = reinterpret_cast<float2*>(p->dws + p->d_ml);
    aa.pool = pool_addr(p->pool);
    aa.rowsrc = reinterpret_cast<const int2*>(p->ws + p->off_rowsrc);
    aa.phase_tab = reinterpret_cast<const pic::Phase*>(p->ws + p->off_phase_tab);
    aa.page_bytes = pi.page_bytes;
    aa.kv_plane_off = int64_t(layer) * 2 * m.kv_heads * pi.page_tokens * m.row_bytes;
    aa.v_off = int64_t(m.kv_heads) * pi.page_tokens * m.row_bytes;
    aa.page_shift = pi.page_shift;
    aa.page_tokens = pi.page_tokens;
    aa.kv_heads = m.kv_heads;
    hipError_t e = pic::launch_attention_bf16(aa, fused, s);
    if (e != hipSuccess) return device_error(p, e, "decode attention kernel");
  }
  return ok();
}

pic_status pic_plan_get_summary(const pic_plan* p, pic_plan_summary* out) {
  if (!p || !out) return set_err(PIC_EINVAL, "plan and out are required");
  if (!p->has_batch) return set_err(PIC_ESTATE, "no batch planned");
  out->batch = p->hp.batch;
  out->n_spans = p->hp.n_spans;
  out->prefix_rows = p->hp.prefix_rows;
  out->new_rows = p->hp.new_rows;
  out->rows = p->hp.rows;
  out->max_position = p->hp.max_position;
  out->materialized = p->materialized ? 1 : 0;
  out->fused_query_rotation = 0;
  out->values_in_pool = p->values_in_pool ? 1 : 0;
  out->attention_items = int32_t(p->hp.work.size());
  out->attention_workgroups = int32_t(p->hp.wg_map.size());
  out->attention_item_workgroups = int32_t(p->hp.item_map.size());
  return ok();
}

pic_status pic_plan_get_attention_work(const pic_plan* p, int32_t* items, int32_t* wg_order, int32_t* item_order) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (!p->has_batch) return set_err(PIC_ESTATE, "no batch planned");
  for (size_t i = 0; items && i < p->hp.work.size(); ++i) {
    const pic::AttnWork& w = p->hp.work[i];
    int32_t* o = items + 7 * i;
    o[0] = w.req;
    o[1] = w.head;
    o[2] = w.col_begin;
    o[3] = w.tile_begin;
    o[4] = w.tile_end;
    o[5] = w.gap_begin;
    o[6] = w.gap_end;
  }
  for (size_t b = 0; wg_order && b < p->hp.wg_map.size(); ++b) wg_order[b] = p->hp.wg_map[b];
  for (size_t b = 0; item_order && b < p->hp.item_map.size(); ++b) item_order[b] = p->hp.item_map[b];
  return ok();
}

pic_status pic_plan_get_requests(const pic_plan* p, int64_t* row_base, int32_t* prefix_rows,
                                 int32_t* first_new_pos) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (!p->has_batch) return set_err(PIC_ESTATE, "no batch planned");
  for (size_t b = 0; b < p->hp.reqs.size(); ++b) {
    const pic::ReqRec& r = p->hp.reqs[b];
    if (row_base) row_base[b] = r.row_base;
    if (prefix_rows) prefix_rows[b] = r.prefix_rows;
    if (first_new_pos) first_new_pos[b] = r.first_new_pos;
  }
  return ok();
}

pic_status pic_plan_get_spans(const pic_plan* p, int32_t* target, int32_t* delta, int64_t* first_row) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (!p->has_batch) return set_err(PIC_ESTATE, "no batch planned");
  for (size_t i = 0; i < p->hp.spans.size(); ++i) {
    const pic::SpanRec& s = p->hp.spans[i];
    if (target) target[i] = s.target;
    if (delta) delta[i] = s.delta;
    if (first_row) first_row[i] = s.dst_row;
  }
  return ok();
}

pic_status pic_plan_get_new_tokens(const pic_plan* p, int32_t* position, int64_t* row) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (!p->has_batch) return set_err(PIC_ESTATE, "no batch planned");
  for (size_t u = 0; u < p->hp.new_pos.size(); ++u) {
    if (position) position[u] = p->hp.new_pos[u];
    if (row) row[u] = p->hp.new_row[u];
  }
  return ok();
}

pic_status pic_timing_enable(pic_plan* p, int32_t on) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  p->timing = on != 0;
  return ok();
}

pic_status pic_timing_read(pic_plan* p, int32_t kernel, int64_t* launches, double* total_ms) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  if (kernel < 0 || kernel >= kTimedKernels) return set_err(PIC_ERANGE, "kernel %d outside [0, 4)", kernel);
  double sum = 0.0;
  for (size_t i = 0; i < p->used[kernel]; ++i) {
    auto& pr = p->events[kernel][i];
    hipError_t e = hipEventSynchronize(pr.second);
    if (e != hipSuccess) return device_error(p, e, "timing event");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) return device_error(p, e, "timing event");
    sum += ms;
  }
  if (launches) *launches = int64_t(p->used[kernel]);
  if (total_ms) *total_ms = sum;
  return ok();
}

pic_status pic_timing_reset(pic_plan* p) {
  if (!p) return set_err(PIC_EINVAL, "plan is NULL");
  for (auto& u : p->used) u = 0;
  return ok();
}

}  // extern "C"
