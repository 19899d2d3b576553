// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pic_plan.h"

namespace pic {

// Phase of one rotation: (cos, sin) of the angle, in fp64.
using Phase = double2;

struct PlanArgs {
  const SpanRec* spans;
  const int32_t* crow;
  const int32_t* new_pos;
  const int32_t* new_row;
  const int32_t* page_ids;
  const double* omega;      // [head_dim / 2]
  int32_t n_spans, n_new, page_shift, half_dim;
  int32_t per_position;     // keys stored un-rotated: the prefix phases are per position
  int32_t phase_rows;       // rows of phase_tab: n_spans, or largest prefix position + 1
  int64_t prefix_rows;
  int32_t* pos;             // [rows]
  int2* rowsrc;             // [rows]: (pool token slot, phase_tab row or -1 for no rotation)
  int4* gsrc;               // [prefix_rows]: per gathered row (assembled row, pool slot, phase row or -1, 0)
  Phase* phase_tab;         // [phase_rows][half_dim]: per span delta, or per position
  Phase* phase_new;         // [n_new][half_dim]
  const ReqRec* reqs;       // for the tile bounds
  int32_t batch, n_tiles;
  int2* tile_pos;           // [n_tiles]: (min, max) row position; max = INT_MAX for a partial tile
  int32_t* split_count;     // [n_slots]: the attention kernel's merge counters, cleared here
  int32_t n_slots;
};

struct GatherArgs {
  const int4* gsrc;         // [prefix_rows]: (assembled row, pool slot, phase_tab row or -1, 0)
  const Phase* phase_tab;   // per span (rotated keys) or per position (un-rotated keys)
  const char* pool;
  char* asm_k;
  char* asm_v;
  int64_t prefix_rows, cap, page_bytes;
  int32_t page_shift, page_tokens, kv_heads, planes_per_block;
  int32_t plane_begin, plane_end;  // (layer, kv head) planes l * Hkv + h to gather
  int32_t values;           // 0: keys only (values stay in the pool, attention reads them there)
  int64_t row_blocks8;      // (set by the launcher) row blocks rounded up to a multiple of 8
};

struct PrologueArgs {
  const char* q;
  const char* k_new;
  const char* v_new;
  const int32_t* new_pos;
  const int32_t* new_row;
  const Phase* phase_new;
  char* q_rot;
  char* asm_k;              // plane base of this layer
  char* asm_v;
  int64_t cap;
  int32_t n_new, q_heads, kv_heads;
};

struct AttnArgs {
  const uint16_t* q_rot;    // [n_new][Hq][128]
  const uint16_t* k_plane;  // this layer: [Hkv][cap][128]
  const uint16_t* v_plane;
  int64_t cap;
  const int32_t* pos;
  const int2* tile_pos;
  const ReqRec* reqs;
  const int32_t* new_pos;
  const AttnWork* work;
  int32_t n_work, q_heads, group, n_new;
  const int32_t* wg_map;    // item pair (paired kernel) or item of each workgroup (-1: none);
  int32_t n_wg;             // null: in order, spread over XCDs by xcd_remap.  n_wg: map entries
  int32_t n_split_out;      // partials written for merge_kernel (1: outputs written directly)
  int32_t paired;           // two work items per workgroup
  int32_t n_split_wg;       // row splits of a column block in different workgroups (1: none)
  int32_t* split_count;     // per column block: splits stored so far (left at 0 after the merge)
  float* spart;             // [column blocks][n_split_wg][4 waves][32][64 lanes] float2: split partial O
  float* sml;               // [column blocks][n_split_wg][4 waves][64 lanes] float2: (m, sum)
  int32_t decode;           // one query per request (new_begin = its index), every row visible:
                            // tile bounds are not read, rows past the end are masked
  // decode with the token's own row handled in the kernel (no prologue):
  // q_rot holds the raw queries, rotated on load by dec_phase; the column
  // block's last split scores the token's own key (k_new rotated) and value
  // from registers and writes both to its plane row dec_row
  int32_t dec_own;
  int32_t dec_split;        // row splits per column block
  const uint16_t* k_new;    // [batch][Hkv][128] raw
  const uint16_t* v_new;
  const Phase* dec_phase;   // [batch][64]: phases of each request's position
  const int32_t* dec_row;   // [batch]: assembled row of the token
  uint16_t* k_own;          // this layer's planes, where the token's rows go
  uint16_t* v_own;
  float scale_log2;         // log2(e) / sqrt(head_dim)
  uint16_t* out;            // n_split == 1
  float* opart;             // [n_split_out][n_new][Hq][128]
  float2* ml;               // [n_split_out][n_new][Hq]: (max in log2 units, sum)
  // fused variant: prefix rows come from the pool
  const char* pool;
  const int2* rowsrc;       // (pool slot, phase_tab row or -1)
  const Phase* phase_tab;
  int64_t page_bytes;
  int64_t kv_plane_off;     // byte offset of (layer, K, head 0) inside a page
  int64_t v_off;            // byte offset from a K row to its V row inside a page
  int32_t page_shift, page_tokens, kv_heads;
  // assembled-plane variant with values left in the pool: prefix rows' values
  // are copied from the pool pages (through rowsrc), the rest from v_plane
  int32_t v_pool;
};

struct AttnF32Args {
  const char* q_rot;
  const char* k_plane;
  const char* v_plane;
  int64_t cap;
  const int32_t* pos;
  const ReqRec* reqs;
  const int32_t* new_pos;
  const int32_t* new_req;
  int32_t n_new, q_heads, group;
  char* out;
};

constexpr int kAttnRowsPerTile = 64;
constexpr int kAttnColsPerWG = 128;   // work item: 4 waves x 32 query columns
constexpr int kAttnTargetWGs = 256;   // prefill workgroups (two work items each): one per CU
constexpr int kXcds = 8;              // XCDs; workgroup b is dispatched to XCD b mod kXcds
constexpr int kAttnMinTilesAcross = 64;  // tiles per split that pay for a merge across workgroups
constexpr int kDecodeTargetItems = 512;  // decode work items: two per CU (one workgroup of two)
constexpr int kAttnMaxSplit = 16;     // merge_kernel handles at most this many row splits

// Decode step tables: per request, the phases of its decode position and the
// position of its decode row.
struct DecodePlanArgs {
  const int32_t* dec_pos;   // [batch]
  const int32_t* dec_row;   // [batch]
  const double* omega;      // [half_dim]
  int32_t batch, half_dim;
  Phase* phase;             // [batch][half_dim]
  int32_t* pos;             // assembled row positions
};

hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_decode_plan(const DecodePlanArgs& a, hipStream_t s);
hipError_t launch_gather(int dtype, int head_dim, const GatherArgs& a, hipStream_t s);
hipError_t launch_prologue(int dtype, int head_dim, const PrologueArgs& a, hipStream_t s);
hipError_t launch_attention_bf16(const AttnArgs& a, bool fused, hipStream_t s);
hipError_t launch_attention_f32(int head_dim, const AttnF32Args& a, hipStream_t s);
// Zero n int32 values with a kernel (no memset node, for callers that
// capture the stream into a graph).
hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t s);
// Copy `bytes` at byte offset `off` of n_pairs (pool page, cache slot) pairs
// (device array) from the host pool to the cache (16-byte multiples).
hipError_t launch_cache_fill(const char* src_pool, char* cache, const int32_t* pairs, int32_t n_pairs,
                             int64_t page_bytes, int64_t off, int64_t bytes, hipStream_t s);
// head_dim, dtype combinations the kernels implement
bool gather_supported(int dtype, int head_dim);
bool attention_supported(int dtype, int head_dim, bool fused);

}  // namespace pic
