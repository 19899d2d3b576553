// HIP kernels for position-independent KV-cache reuse on gfx950 (CDNA4).
//
//   plan      per-row positions and pool sources, per-span and per-token
//             RoPE phases, per-tile position bounds
//   gather    assembly: copy every span's cached rows out of the paged pool
//             into the contiguous prefix, rotating keys by the span's delta
//             (CoinRAG page, section 2.3, the C_ctx equation and Rot(.; Delta_i);
//             TurboRAG review page, Reordered Positions: apply RoPE again at
//             the new position)
//   prologue  rotate the new tokens' queries and keys to their positions and
//             append the new keys/values after the prefix (decode does this
//             inside its attention instance)
//   attention query-prefill attention over prefix + new rows with the mask
//             pos_row <= pos_query (TurboRAG Figure 4: the query sees every
//             chunk and itself; SemPIC: causal interleave), GQA, bf16 MFMA
//             32x32x16 with fp32 accumulation and online softmax; optional
//             split of the rows with a log-sum-exp merge
//
// Rotation arithmetic.  Each key pair (x, y) = (k, k + d/2) is rotated in fp64
// (fp64 FMA runs at the fp32 rate on CDNA) by an angle whose cos/sin were
// computed in fp64 once per span or per position.  The fp64 result is rounded
// once to bf16 (nearest even; see pack_bf16) or to fp32.  A rotation by zero
// is a bit copy.
#include "pic_kernels.h"

#include <climits>
#include <cmath>
#include <type_traits>

namespace pic {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// fp64 -> fp32 with round-to-odd: truncate toward zero, then set the last bit
// if anything was lost.
__device__ __forceinline__ float to_f32_odd(double x) {
  float r = float(x);  // round to nearest even
  double back = double(r);
  unsigned u = __float_as_uint(r);
  if (back != x) {
    if (fabs(back) > fabs(x)) u -= 1u;
    u |= 1u;
  }
  return __uint_as_float(u);
}

// Two fp64 values to a packed pair of bf16 (first in the low half), rounded
// once to nearest even.  Rounding through fp32 first can only differ when the
// fp32 value lands exactly on a bf16 midpoint (low 16 bits 0x8000): every
// midpoint is an fp32 number, so otherwise the fp32 value and the fp64 value
// lie on the same side of all of them.  Those rare cases (any lane of the
// wave) redo the step with round-to-odd.
__device__ __forceinline__ unsigned pack_bf16(double a, double b) {
  float fa = float(a), fb = float(b);
  const bool tie = ((__float_as_uint(fa) & 0xffffu) == 0x8000u) | ((__float_as_uint(fb) & 0xffffu) == 0x8000u);
  if (__builtin_amdgcn_ballot_w64(tie)) {
    fa = to_f32_odd(a);
    fb = to_f32_odd(b);
  }
  const __bf16 ha = (__bf16)fa;
  const __bf16 hb = (__bf16)fb;
  return unsigned(__builtin_bit_cast(uint16_t, ha)) | (unsigned(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// Rotate the 16-byte vectors a (elements k) and b (elements k + d/2).
template <bool BF16>
__device__ __forceinline__ void rotate_vec(u32x4& a, u32x4& b, const Phase* ph);

template <>
__device__ __forceinline__ void rotate_vec<true>(u32x4& a, u32x4& b, const Phase* ph) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const double x0 = bf16_lo(a[w]), x1 = bf16_hi(a[w]);
    const double y0 = bf16_lo(b[w]), y1 = bf16_hi(b[w]);
    const Phase p0 = ph[2 * w], p1 = ph[2 * w + 1];
    const double rx0 = fma(x0, p0.x, -y0 * p0.y), ry0 = fma(x0, p0.y, y0 * p0.x);
    const double rx1 = fma(x1, p1.x, -y1 * p1.y), ry1 = fma(x1, p1.y, y1 * p1.x);
    a[w] = pack_bf16(rx0, rx1);
    b[w] = pack_bf16(ry0, ry1);
  }
}

template <>
__device__ __forceinline__ void rotate_vec<false>(u32x4& a, u32x4& b, const Phase* ph) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const double x = __uint_as_float(a[w]), y = __uint_as_float(b[w]);
    const Phase p = ph[w];
    a[w] = __float_as_uint(float(fma(x, p.x, -y * p.y)));
    b[w] = __float_as_uint(float(fma(x, p.y, y * p.x)));
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Last entry of a non-decreasing table whose value is <= u.
__device__ __forceinline__ int find_le(const int32_t* tbl, int n, int64_t u) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (tbl[mid] <= u)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Give each
// XCD a contiguous range of logical work items so that neighbours, which read
// the same keys and values, share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  int x = bid & 7, k = bid >> 3;
  int q = n >> 3, r = n & 7;
  return x * q + min(x, r) + k;
}

// max(a, b, c) as one instruction.  fmaxf in IEEE mode first quiets each
// MFMA result (one extra instruction per input); scores are never NaN here.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Max of a value and its copy in the lane 32 away.
__device__ __forceinline__ float max_halves(float v) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max3(__uint_as_float(s[0]), __uint_as_float(s[1]), __uint_as_float(s[1]));
}

// ---------------------------------------------------------------------------
// plan: positions, pool sources, phases, tile bounds
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void plan_rows_kernel(PlanArgs a) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < a.prefix_rows) {
    int sp = find_le(a.crow, a.n_spans, i);
    SpanRec s = a.spans[sp];
    int t = int(i - s.crow);
    int tok = s.s + t;
    int page = a.page_ids[s.page_off + (tok >> a.page_shift)];
    int slot = (page << a.page_shift) | (tok & ((1 << a.page_shift) - 1));
    int row = s.dst_row + t;
    const int p = s.target + t;
    a.pos[row] = p;
    // phase row: the span's delta, or for un-rotated keys the row's position;
    // -1 where the rotation is by 0 (a bit copy)
    const int ph = a.per_position ? (p != 0 ? p : -1) : (s.delta != 0 ? sp : -1);
    a.rowsrc[row] = make_int2(slot, ph);
    a.gsrc[i] = make_int4(row, slot, ph, 0);
  } else if (i < a.prefix_rows + a.n_new) {
    int u = int(i - a.prefix_rows);
    int row = a.new_row[u];
    a.pos[row] = a.new_pos[u];
    a.rowsrc[row] = make_int2(-1, -1);
  }
}

__global__ __launch_bounds__(256) void plan_phase_kernel(PlanArgs a) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t total = (int64_t(a.phase_rows) + a.n_new) * a.half_dim;
  if (i >= total) return;
  int64_t which = i / a.half_dim;
  int k = int(i % a.half_dim);
  double p;
  Phase* dst;
  if (which < a.phase_rows) {
    p = a.per_position ? double(which) : double(a.spans[which].delta);
    dst = a.phase_tab + which * a.half_dim + k;
  } else {
    int u = int(which - a.phase_rows);
    p = double(a.new_pos[u]);
    dst = a.phase_new + int64_t(u) * a.half_dim + k;
  }
  double ang = p * a.omega[k];
  const double c = cos(ang), sn = sin(ang);
  *dst = make_double2(c, sn);
}

__global__ __launch_bounds__(256) void decode_plan_kernel(DecodePlanArgs a) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(a.batch) * a.half_dim) return;
  const int b = int(i / a.half_dim), k = int(i % a.half_dim);
  const double ang = double(a.dec_pos[b]) * a.omega[k];
  a.phase[i] = make_double2(cos(ang), sin(ang));
  if (k == 0) a.pos[a.dec_row[b]] = a.dec_pos[b];
}

// One thread per 64-row tile: the smallest and largest row position, with the
// largest replaced by INT_MAX when the tile runs past the request's rows.
// The first n_slots threads also clear the attention merge counters.
__global__ __launch_bounds__(256) void plan_tiles_kernel(PlanArgs a) {
  int tix = int(blockIdx.x) * blockDim.x + threadIdx.x;
  if (tix < a.n_slots) a.split_count[tix] = 0;
  if (tix >= a.n_tiles) return;
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a.reqs[mid].tile_base <= tix)
      lo = mid;
    else
      hi = mid;
  }
  // requests without rows own no tiles: step to the last one starting here
  while (lo + 1 < a.batch && a.reqs[lo + 1].tile_base <= tix) ++lo;
  const ReqRec r = a.reqs[lo];
  const int rows = r.prefix_rows + r.n_new;
  const int r0 = (tix - r.tile_base) * kAttnRowsPerTile;
  const int r1 = min(r0 + kAttnRowsPerTile, rows);
  int mn = INT_MAX, mx = INT_MIN;
  for (int rr = r0; rr < r1; ++rr) {
    int p = a.pos[r.row_base + rr];
    mn = min(mn, p);
    mx = max(mx, p);
  }
  if (r1 - r0 < kAttnRowsPerTile) mx = INT_MAX;
  a.tile_pos[tix] = make_int2(mn, mx);
}

// ---------------------------------------------------------------------------
// gather + re-rotate
// ---------------------------------------------------------------------------

// Each row (one token of one layer / kv head plane) is handled by LPR lanes;
// lane j owns the 16-byte vector j of the first half of the row and vector j
// of the second half, so the half-split rotation pairs stay in one lane.  A
// block covers 256 / LPR rows of the span table and `planes_per_block`
// (layer, kv head) planes, reusing each row's source record and phases.  The
// record (assembled row, pool slot, phase row) was resolved once per row by
// the plan, so a row costs one load before its data loads are issued.  A
// phase row is fetched once per run of rows sharing it within a wave (the
// rows of one span) and handed to the run's other rows through LDS.
template <bool BF16, int D, bool VALUES>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int LPR = D / (2 * EPV);
  constexpr int RPB = 256 / LPR;
  constexpr int64_t RB = int64_t(D) * ES;
  const int rl = threadIdx.x / LPR;
  const int j = threadIdx.x % LPR;
  // Workgroup b runs on XCD b mod 8.  The row blocks (padded to a multiple
  // of 8) are cut into 8 slices; XCD x takes slice x under every plane
  // group, rows fastest, so the source records and phase rows it reads stay
  // in its own L2.  (A bijection: per XCD, k < per * groups.)
  const int per = int(a.row_blocks8 >> 3);
  const int bid = int(blockIdx.x);
  const int xcd = bid & 7, k = bid >> 3;
  const int pgrp = k / per;
  const int64_t rb = int64_t(xcd) * per + (k - pgrp * per);
  const int64_t u = rb * RPB + rl;
  if (u >= a.prefix_rows) return;
  const int4 g = a.gsrc[u];
  const char* __restrict__ src_row =
      a.pool + int64_t(g.y >> a.page_shift) * a.page_bytes + int64_t(g.y & (a.page_tokens - 1)) * RB;
  const int64_t dst_row = g.x;
  // rotation: the span's delta, or for un-rotated keys the row's new position
  // (phase row g.z; none where the rotation is by 0)
  const bool rot = g.z >= 0;
  // Phase rows: consecutive rows of a span share one.  Within a wave only
  // the first row of each run of equal phase rows (a leader) loads it; the
  // leader stages it in LDS and the other rows of the run read it there.
  constexpr int RPW = 64 / LPR;
  __shared__ Phase ph_lds[4][RPW][D / 2];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int riw = lane / LPR;
  const int zprev = __shfl_up(g.z, LPR);
  const bool lead = rot && (riw == 0 || zprev != g.z);
  Phase ph[EPV];
  if (lead) {
    const Phase* pp = a.phase_tab + int64_t(g.z) * (D / 2) + j * EPV;
#pragma unroll
    for (int e = 0; e < EPV; ++e) ph[e] = pp[e];
  }
  const uint64_t leaders = __builtin_amdgcn_ballot_w64(lead && j == 0);
  const int p0 = a.plane_begin + pgrp * a.planes_per_block;
  const int p1 = min(p0 + a.planes_per_block, a.plane_end);
  const int64_t plane_stride = int64_t(a.page_tokens) * RB;  // one (layer, K/V, head) run
  char* __restrict__ ak = a.asm_k;
  char* __restrict__ av = a.asm_v;
  // four planes per iteration, all loads in flight before any store (a
  // store issued between two planes' loads would hold the later loads' wait
  // behind its own completion); past the group's end the last plane is
  // loaded again and not stored
  constexpr int NPI = 4;
  for (int pl = p0; pl < p1; pl += NPI) {
    u32x4 k0[NPI], k1[NPI], v0[NPI], v1[NPI];
#pragma unroll
    for (int q = 0; q < NPI; ++q) {
      const int pq = min(pl + q, p1 - 1);
      const int l = pq / a.kv_heads;
      const int h = pq - l * a.kv_heads;
      const char* ks = src_row + (int64_t(l) * 2 * a.kv_heads + h) * plane_stride;
      const char* vs = ks + int64_t(a.kv_heads) * plane_stride;
      k0[q] = ld16(ks + j * 16);
      k1[q] = ld16(ks + RB / 2 + j * 16);
      if (VALUES) {
        v0[q] = ld16(vs + j * 16);
        v1[q] = ld16(vs + RB / 2 + j * 16);
      }
    }
    if (pl == p0 && leaders != 0) {
      // leaders publish their phase rows; every rotating row takes its run's
      // (one wave: LDS operations complete in order)
      if (lead) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) ph_lds[wv][riw][j * EPV + e] = ph[e];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (rot && !lead) {
        const uint64_t below = leaders & ((uint64_t(2) << (riw * LPR)) - 1);
        const int lr = (63 - __builtin_clzll(below)) / LPR;
#pragma unroll
        for (int e = 0; e < EPV; ++e) ph[e] = ph_lds[wv][lr][j * EPV + e];
      }
    }
#pragma unroll
    for (int q = 0; q < NPI; ++q) {
      if (pl + q >= p1) break;
      const int64_t off = (int64_t(pl + q) * a.cap + dst_row) * RB;
      if (rot) rotate_vec<BF16>(k0[q], k1[q], ph);
      st16(ak + off + j * 16, k0[q]);
      st16(ak + off + RB / 2 + j * 16, k1[q]);
      if (VALUES) {
        st16(av + off + j * 16, v0[q]);
        st16(av + off + RB / 2 + j * 16, v1[q]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// new-token prologue
// ---------------------------------------------------------------------------

// Each token owns Hq query rows, Hkv key rows and Hkv value rows.  A group of
// LPR lanes takes one token and kPrologueRows consecutive rows of it, so the
// token's phases are loaded once per group and reused for every row (and
// once per wave: the wave's other groups on the token read them from LDS).
// The phases, the rows and the token's position are requested together
// (nothing waits on another load before its own loads are issued).
constexpr int kPrologueRows = 2;

template <bool BF16, int D>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int LPR = D / (2 * EPV);
  constexpr int GPB = 256 / LPR;   // lane groups per block
  constexpr int64_t RB = int64_t(D) * ES;
  const int per_tok = a.q_heads + 2 * a.kv_heads;
  const int chunks = (per_tok + kPrologueRows - 1) / kPrologueRows;
  const int64_t grp = int64_t(blockIdx.x) * GPB + threadIdx.x / LPR;
  const int j = threadIdx.x % LPR;
  if (grp >= int64_t(a.n_new) * chunks) return;
  const int u = int(grp / chunks);
  const int w0 = int(grp - int64_t(u) * chunks) * kPrologueRows;
  const int w1 = min(w0 + kPrologueRows, per_tok);
  const int pos = a.new_pos[u];
  const int row = a.new_row[u];
  // A token's phase row is loaded once per wave: the first of the wave's
  // lane groups on that token (a leader) loads it and hands it to the
  // token's other groups through LDS.
  constexpr int GPW = 64 / LPR;   // lane groups per wave
  __shared__ Phase ph_lds[4][GPW][D / 2];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int giw = lane / LPR;
  const int uprev = __shfl_up(u, LPR);
  const bool needs = w0 < a.q_heads + a.kv_heads;
  const bool lead = needs && (giw == 0 || uprev != u);
  Phase ph[EPV];
  if (lead) {
    const Phase* pp = a.phase_new + int64_t(u) * (D / 2) + j * EPV;
#pragma unroll
    for (int e = 0; e < EPV; ++e) ph[e] = pp[e];
  }
  const uint64_t leaders = __builtin_amdgcn_ballot_w64(lead && j == 0);
  const bool rot_tok = pos != 0;
  // issue every row's loads before any rotation or store
  u32x4 x0[kPrologueRows], x1[kPrologueRows];
  char* dst[kPrologueRows];
  bool rot[kPrologueRows];
#pragma unroll
  for (int i = 0; i < kPrologueRows; ++i) {
    const int w = w0 + i;
    dst[i] = nullptr;
    rot[i] = false;
    if (w >= w1) continue;
    const char* src;
    if (w < a.q_heads) {
      src = a.q + (int64_t(u) * a.q_heads + w) * RB;
      dst[i] = a.q_rot + (int64_t(u) * a.q_heads + w) * RB;
      rot[i] = rot_tok;
    } else if (w < a.q_heads + a.kv_heads) {
      const int h = w - a.q_heads;
      src = a.k_new + (int64_t(u) * a.kv_heads + h) * RB;
      dst[i] = a.asm_k + (int64_t(h) * a.cap + row) * RB;
      rot[i] = rot_tok;
    } else {
      const int h = w - a.q_heads - a.kv_heads;
      src = a.v_new + (int64_t(u) * a.kv_heads + h) * RB;
      dst[i] = a.asm_v + (int64_t(h) * a.cap + row) * RB;
    }
    x0[i] = ld16(src + j * 16);
    x1[i] = ld16(src + RB / 2 + j * 16);
  }
  if (leaders != 0) {
    if (lead) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) ph_lds[wv][giw][j * EPV + e] = ph[e];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (needs && !lead) {
      const uint64_t below = leaders & ((uint64_t(2) << (giw * LPR)) - 1);
      const int lg = (63 - __builtin_clzll(below)) / LPR;
#pragma unroll
      for (int e = 0; e < EPV; ++e) ph[e] = ph_lds[wv][lg][j * EPV + e];
    }
  }
#pragma unroll
  for (int i = 0; i < kPrologueRows; ++i) {
    if (!dst[i]) continue;
    if (rot[i]) rotate_vec<BF16>(x0[i], x1[i], ph);
    st16(dst[i] + j * 16, x0[i]);
    st16(dst[i] + RB / 2 + j * 16, x1[i]);
  }
}

// ---------------------------------------------------------------------------
// bf16 query-prefill attention, head_dim 128
// ---------------------------------------------------------------------------
//
// Query columns.  Column c of a request is token c / G, query head c % G of
// the group, so the G heads that share a kv head share every K/V tile.  A
// wave owns 32 consecutive columns; with them as the MFMA N dimension
//   S^T = K Q^T   (A = 32-row K fragments from LDS, B = the wave's rotated
//                  queries, held in registers), 2 x 8 MFMA 32x32x16 per tile;
//   O^T += V^T P^T (A = V^T fragments read with the LDS transpose load,
//                  B = the wave's own probabilities: the S^T accumulator puts
//                  each column's 16 row values of a 32-row block in one lane,
//                  which is the B layout needed here once the row order inside
//                  a k-step is permuted identically for A), 4 x 2 x 2 MFMA.
// Each lane therefore owns one query column: the softmax statistics are
// lane-local plus one exchange with the lane 32 away.
//
// Tiles: K and V, 64 rows x 256 bytes each, row-major with 16-byte granules
// XOR-swizzled by row, are copied global -> LDS directly (no registers) by
// 16-byte lane loads whose source addresses apply the swizzle, together with
// the rows' positions.  Rows past the request's end repeat its last row and
// are masked by index.
//
// Softmax: scores are kept relative to a reference maximum that is raised
// only when a block's maximum exceeds it by more than 8 (log2 units), so the
// accumulator rescale is rare; probabilities stay below 2^8.  The denominator
// sums (v_dot2) the same bf16 probabilities the PV product uses, so the
// output is an exact weighted mean of the values.
//
// A tile runs as two 32-row blocks pipelined against each other
// (tile_pipelined).

constexpr int kTileBytes = 16384;
constexpr int kPosOffset = 2 * kTileBytes;          // 64 row positions after K and V
constexpr float kRescaleSlack = 8.0f;

// LDS swizzles of the 16-byte granules of a tile row (64 banks of 4 bytes:
// one 256-byte row spans every bank once).  Keys are read as one 16-byte
// granule per lane from 32 consecutive rows, so granules are XORed with the
// row index (mod 16).  Values are read with the transpose load: each group of
// 32 lanes touches 4 consecutive rows x 2 granule pairs, so rows r mod 4 take
// disjoint quarters of the granules (XOR with 4 * (row mod 4)) and the group
// hits every bank once.
__device__ __forceinline__ int k_swz(int r) { return r & 15; }
__device__ __forceinline__ int v_swz(int r) { return 4 * (r & 3); }

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS-local byte address (not the flat address) of a shared-memory pointer.
__device__ __forceinline__ unsigned lds_addr(const char* p) {
  return unsigned(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// LDS reads as inline asm.  The intrinsic forms make the compiler wait for
// every outstanding global->LDS copy before them (it cannot tell that those
// target another stage); the callers wait with an explicit lgkmcnt(0) whose
// operands are the results, so no use can move above it.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(unsigned addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

template <int OFF>
__device__ __forceinline__ s16x4 tr_read(unsigned addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

struct KFrags {
  u32x4 x[8];   // the k steps of one 32-row block
};

__device__ __forceinline__ void kfrag_wait(KFrags& f) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(f.x[0]), "+v"(f.x[1]), "+v"(f.x[2]), "+v"(f.x[3]), "+v"(f.x[4]), "+v"(f.x[5]),
                 "+v"(f.x[6]), "+v"(f.x[7]));
}

struct TrBlock {
  s16x4 x[8];   // [kb][s2][half] of one 32-wide d block
};

template <int OFF>
__device__ __forceinline__ void tr_block_read(unsigned a0, unsigned a1, TrBlock& b) {
  b.x[0] = tr_read<OFF>(a0);
  b.x[1] = tr_read<OFF>(a1);
  b.x[2] = tr_read<OFF + 16 * 256>(a0);
  b.x[3] = tr_read<OFF + 16 * 256>(a1);
  b.x[4] = tr_read<OFF + 32 * 256>(a0);
  b.x[5] = tr_read<OFF + 32 * 256>(a1);
  b.x[6] = tr_read<OFF + 48 * 256>(a0);
  b.x[7] = tr_read<OFF + 48 * 256>(a1);
}

__device__ __forceinline__ void lds_wait(TrBlock& b) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(b.x[0]), "+v"(b.x[1]), "+v"(b.x[2]), "+v"(b.x[3]), "+v"(b.x[4]), "+v"(b.x[5]),
                 "+v"(b.x[6]), "+v"(b.x[7]));
}

// Row positions of a tile, read as inline asm like the fragments (so that
// the compiler does not wait for copies into other stages first): a lane's 8
// groups of 4 rows.
template <int OFF>
__device__ __forceinline__ i32x4 lds_read_i4(unsigned addr) {
  i32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

struct PosFrags {
  i32x4 x[8];
};

__device__ __forceinline__ void pos_wait(PosFrags& p) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(p.x[0]), "+v"(p.x[1]), "+v"(p.x[2]), "+v"(p.x[3]), "+v"(p.x[4]), "+v"(p.x[5]),
                 "+v"(p.x[6]), "+v"(p.x[7]));
}

// Max of the 32 scores a lane holds, as a depth-4 tree of 3-input maxima.
__device__ __forceinline__ float max32(const f32x16& a, const f32x16& b) {
  const float t0 = max3(a[0], a[1], a[2]), t1 = max3(a[3], a[4], a[5]), t2 = max3(a[6], a[7], a[8]);
  const float t3 = max3(a[9], a[10], a[11]), t4 = max3(a[12], a[13], a[14]), t5 = max3(a[15], b[0], b[1]);
  const float t6 = max3(b[2], b[3], b[4]), t7 = max3(b[5], b[6], b[7]), t8 = max3(b[8], b[9], b[10]);
  const float t9 = max3(b[11], b[12], b[13]);
  const float u0 = max3(t0, t1, t2), u1 = max3(t3, t4, t5), u2 = max3(t6, t7, t8);
  const float u3 = max3(t9, b[14], b[15]);
  return max3(max3(u0, u1, u2), u3, u3);
}

// Per-lane state of one query column and its wave.
struct Col {
  bool ok;          // the column exists
  int u;            // packed index of its new token
  int hq;           // its query head
  int qpos;         // its position
  int wq_min, wq_max;  // range of the wave's query positions (empty: INT_MAX, INT_MIN)
  unsigned kaddr[8];     // LDS addresses of the lane's K fragments in stage 0
  unsigned vaddr[4][2];  // LDS addresses of the lane's V^T transpose reads in stage 0
};

// The lane's query column: its indices, its position and its query
// fragments, all requested before anything waits on them.  New positions
// increase strictly within a request, so the range of the wave's query
// positions is that of its first and last valid column (wave-uniform loads,
// no cross-lane reduction: a lane exchange would be an LDS instruction, which
// waits for every outstanding copy into LDS).  `lds` is the LDS address of
// stage 0; later stages are reached through the instructions' immediate
// offsets.
__device__ __forceinline__ void col_setup(const AttnArgs& a, const AttnWork& w, const ReqRec& rq, int wave,
                                          unsigned lds, Col& c, bf16x8 qb[8]) {
  const int lane = threadIdx.x & 63;
  const int g2 = lane >> 5, lq = lane & 31;
  const int ncols = (a.decode ? 1 : rq.n_new) * a.group;
  const int c0 = w.col_begin + wave * 32;
  const int col = c0 + lq;
  c.ok = col < ncols;
  const int colc = c.ok ? col : ncols - 1;
  const int tokj = colc / a.group;
  c.hq = w.head * a.group + (colc - tokj * a.group);
  c.u = rq.new_begin + tokj;
  c.qpos = a.new_pos[c.u];
  c.wq_min = INT_MAX;
  c.wq_max = INT_MIN;
  if (c0 < ncols) {
    const int c1 = min(c0 + 31, ncols - 1);
    c.wq_min = a.new_pos[rq.new_begin + c0 / a.group];
    c.wq_max = a.new_pos[rq.new_begin + c1 / a.group];
  }
  const u32x4* qp = reinterpret_cast<const u32x4*>(a.q_rot + (int64_t(c.u) * a.q_heads + c.hq) * 128);
#pragma unroll
  for (int s = 0; s < 8; ++s) qb[s] = __builtin_bit_cast(bf16x8, qp[2 * s + g2]);
#pragma unroll
  for (int s = 0; s < 8; ++s) c.kaddr[s] = lds + lq * 256 + 16 * ((2 * s + g2) ^ k_swz(lq));
  const int l16 = lane & 15, gm = (lane >> 4) & 1;
  const int cc = 2 * gm + ((l16 & 3) >> 1);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rowi = 8 * h + 4 * g2 + (l16 >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db)
      c.vaddr[db][h] = lds + kTileBytes + rowi * 256 + 16 * ((4 * db + cc) ^ v_swz(rowi)) + 8 * (l16 & 1);
  }
}

// ---- one tile, pipelined by 32-row block ----
// S of block 1 runs on the matrix core while block 0's probabilities are
// formed, and block 0's PV while block 1's are (independent work in one basic
// block, which the scheduler interleaves).  A raise of the reference maximum
// by block 0 rescales O and the sum before block 0's PV; one by block 1
// rescales them after it, since block 0's probabilities are relative to the
// old maximum.  Each O element accumulates its products in the same order as
// the unpipelined tile.

__device__ __forceinline__ float max16(const f32x16& a) {
  const float t0 = max3(a[0], a[1], a[2]), t1 = max3(a[3], a[4], a[5]), t2 = max3(a[6], a[7], a[8]);
  const float t3 = max3(a[9], a[10], a[11]), t4 = max3(a[12], a[13], a[14]);
  return fmaxf(max3(t0, t1, t2), max3(t3, t4, a[15]));
}

// Mask the scores of 32-row block KB of a tile (rows later than the lane's
// query, or past the request's end).  The tile's row positions sit in LDS at
// byte offset POFF from `paddr` (the lane's address in stage 0): group
// 4 KB + qq of the lane holds rows 32 KB + 8 qq + 4 g2 .. + 3; `r0` is the
// tile's first row, `rows` the request's rows.  (Offsets past the 16-bit
// immediate go into the address.)
template <int POFF, int KB>
__device__ __forceinline__ void mask_block(f32x16& sc, unsigned paddr, int r0, int rows, const Col& c) {
  const int g2 = (threadIdx.x & 63) >> 5;
  constexpr int B = POFF + 128 * KB;
  constexpr unsigned EXTRA = B + 96 > 65535 ? unsigned(B) : 0u;
  constexpr int PO = int(B - EXTRA);
  const unsigned pa = paddr + EXTRA;
  i32x4 p[4];
  p[0] = lds_read_i4<PO>(pa);
  p[1] = lds_read_i4<PO + 32>(pa);
  p[2] = lds_read_i4<PO + 64>(pa);
  p[3] = lds_read_i4<PO + 96>(pa);
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]));
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int r4 = 32 * KB + 8 * qq + 4 * g2;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (p[qq][e] > c.qpos || r0 + r4 + e >= rows) sc[4 * qq + e] = -INFINITY;
  }
}

// The block's probabilities relative to the reference maximum mb.
__device__ __forceinline__ void block_probs(const f32x16& sc, float scale_log2, float mb, bf16x8 pb[2]) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    pb[i >> 3][i & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], scale_log2, -mb));
}

// O^T += V^T P^T and the denominator for 32-row block KB of the tile in the
// stage at byte offset STAGE: per 32-wide d block, 4 transpose reads (double
// buffered across d blocks) and 2 MFMAs.  The denominator adds the same bf16
// probabilities that feed the products (v_dot2 against ones, while the first
// reads are in flight); a lane holds 16 of the block's 32 rows of its column,
// lane ^ 32 the other 16, and the two halves are added at the end.
template <int STAGE, int KB>
__device__ __forceinline__ void pv_block(const Col& c, const bf16x8 pb[2], f32x16 o[4], float& lsum) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  constexpr int OFF = STAGE + 8192 * KB;
  s16x4 vb[2][4];
  auto rd = [&](int db, s16x4* x) {
    x[0] = tr_read<OFF>(c.vaddr[db][0]);
    x[1] = tr_read<OFF>(c.vaddr[db][1]);
    x[2] = tr_read<OFF + 4096>(c.vaddr[db][0]);
    x[3] = tr_read<OFF + 4096>(c.vaddr[db][1]);
  };
  auto wt = [](s16x4* x) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
  };
  rd(0, vb[0]);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // (pairs built element by element: bit-casting the vector's 32-bit
      // words to bf16x2 made the compiler feed one register to all four)
      const bf16x2 pr = {pb[s2][2 * e], pb[s2][2 * e + 1]};
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, lsum, false);
    }
  wt(vb[0]);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    s16x4* cur = vb[db & 1];
    if (db + 1 < 4) rd(db + 1, vb[(db + 1) & 1]);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const s16x8 xv = __builtin_shufflevector(cur[2 * s2], cur[2 * s2 + 1], 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xv), pb[s2], o[db], 0, 0, 0);
    }
    if (db + 1 < 4) wt(vb[(db + 1) & 1]);
  }
}

// The reference-maximum update of a block whose scaled maximum is mt: lanes
// whose maximum exceeds the reference by more than the slack raise it; the
// returned factor rescales what was accumulated against the old reference
// (1 where nothing is raised; a lane whose maximum is still -inf does not
// raise, so it never forms exp2(-inf - -inf)).
__device__ __forceinline__ float raise_ref(float mt, float& m, bool& raise) {
  raise = mt > m + kRescaleSlack;
  const float alpha = raise ? __builtin_amdgcn_exp2f(m - mt) : 1.0f;
  m = raise ? mt : m;
  return alpha;
}

// The whole tile in the stage at byte offset STAGE (see above).
template <int STAGE>
__device__ __forceinline__ void tile_pipelined(const Col& c, const bf16x8 qb[8], int2 bnd, unsigned paddr, int r0,
                                               int rows, float scale_log2, float& m, f32x16 o[4], float& lsum) {
  constexpr int POFF = STAGE + kPosOffset;
  const bool masked = bnd.y > c.wq_min;
  // block 0's key fragments, then block 1's into the same registers (an
  // MFMA takes its A operand when it issues).  An asm read and the wait that
  // publishes its result enclose straight-line code only: the compiler
  // treats the result as available at the read and may copy it anywhere
  // before the wait (a branch in between would allow that).
  KFrags kf;
#pragma unroll
  for (int s = 0; s < 8; ++s) kf.x[s] = lds_read16<STAGE>(c.kaddr[s]);
  kfrag_wait(kf);
  f32x16 s0 = f32x16{};
#pragma unroll
  for (int s = 0; s < 8; ++s)
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf.x[s]), qb[s], s0, 0, 0, 0);
  if (masked) mask_block<POFF, 0>(s0, paddr, r0, rows, c);
#pragma unroll
  for (int s = 0; s < 8; ++s) kf.x[s] = lds_read16<STAGE + 8192>(c.kaddr[s]);
  bool raise0;
  const float alpha0 = raise_ref(max_halves(max16(s0)) * scale_log2, m, raise0);
  kfrag_wait(kf);
  // block 1's S on the matrix core while block 0's probabilities form
  f32x16 s1 = f32x16{};
#pragma unroll
  for (int s = 0; s < 8; ++s)
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf.x[s]), qb[s], s1, 0, 0, 0);
  bf16x8 p0[2];
  block_probs(s0, scale_log2, m == -INFINITY ? 0.0f : m, p0);
  // (kept in this block rather than sunk to their use in block 0's PV)
  asm volatile("" ::"v"(p0[0]), "v"(p0[1]));
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // then five VALU
  }
  if (__builtin_amdgcn_ballot_w64(raise0)) {
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha0;
    lsum *= alpha0;
  }
  if (masked) mask_block<POFF, 1>(s1, paddr, r0, rows, c);
  bool raise1;
  const float alpha1 = raise_ref(max_halves(max16(s1)) * scale_log2, m, raise1);
  // block 0's PV while block 1's probabilities form
  pv_block<STAGE, 0>(c, p0, o, lsum);
  bf16x8 p1[2];
  block_probs(s1, scale_log2, m == -INFINITY ? 0.0f : m, p1);
  asm volatile("" ::"v"(p1[0]), "v"(p1[1]));
  if (__builtin_amdgcn_ballot_w64(raise1)) {
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha1;
    lsum *= alpha1;
  }
  pv_block<STAGE, 1>(c, p1, o, lsum);
}

// Write a column's result: a partial (unnormalised O, reference maximum m,
// sum lt) at partial index `part` for merge_kernel, or the normalised bf16
// output.
__device__ __forceinline__ void store_column(const AttnArgs& a, const Col& c, const f32x16 o[4], float lt,
                                             float m, bool partial, int part) {
  if (!c.ok) return;
  const int g2 = (threadIdx.x & 63) >> 5;
  if (partial) {
    const int64_t idx = (int64_t(part) * a.n_new + c.u) * a.q_heads + c.hq;
    float* pp = a.opart + idx * 128;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d0 = 32 * db + 8 * qq + 4 * g2;
        const f32x4 v = {o[db][4 * qq], o[db][4 * qq + 1], o[db][4 * qq + 2], o[db][4 * qq + 3]};
        *reinterpret_cast<f32x4*>(pp + d0) = v;
      }
    }
    if (g2 == 0) a.ml[idx] = make_float2(m, lt);
    return;
  }
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  uint16_t* op = a.out + (int64_t(c.u) * a.q_heads + c.hq) * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int d0 = 32 * db + 8 * qq + 4 * g2;
      u32x2 pk;
      const __bf16 b0 = (__bf16)(o[db][4 * qq + 0] * inv), b1 = (__bf16)(o[db][4 * qq + 1] * inv);
      const __bf16 b2 = (__bf16)(o[db][4 * qq + 2] * inv), b3 = (__bf16)(o[db][4 * qq + 3] * inv);
      pk[0] = unsigned(__builtin_bit_cast(uint16_t, b0)) | (unsigned(__builtin_bit_cast(uint16_t, b1)) << 16);
      pk[1] = unsigned(__builtin_bit_cast(uint16_t, b2)) | (unsigned(__builtin_bit_cast(uint16_t, b3)) << 16);
      *reinterpret_cast<u32x2*>(op + d0) = pk;
    }
  }
}

// Row-split partials of a column block.  Each wave stores its unnormalised
// O and its (m, sum) exactly as its lanes hold them: per (column block,
// split, wave), 32 float2 of O per lane (fragment-major, lane-minor, so every
// store and load moves 512 contiguous bytes) and one float2 (m, sum) per lane.
// The stores are agent-scope atomic stores and the merging split reads them
// with agent-scope atomic loads; the arrival count that orders them is an
// agent-scope acquire-release read-modify-write (store_split_partial's
// caller), taken after the stores have completed.
constexpr int kSplitWaveFloats = 32 * 64 * 2;

__device__ __forceinline__ void st_dev2(float* p, float x, float y) {
  const unsigned long long u = (unsigned long long)__float_as_uint(x) | ((unsigned long long)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 ld_dev2(const float* p) {
  const unsigned long long u =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(unsigned(u)), __uint_as_float(unsigned(u >> 32)));
}

__device__ __forceinline__ int64_t split_wave_block(const AttnArgs& a, int slot, int sp, int wave) {
  return (int64_t(slot) * a.n_split_wg + sp) * 4 + wave;
}

__device__ __forceinline__ void store_split_partial(const AttnArgs& a, int slot, int sp, int wave,
                                                    const f32x16 o[4], float m, float lt) {
  const int lane = threadIdx.x & 63;
  const int64_t wb = split_wave_block(a, slot, sp, wave);
  float* base = a.spart + wb * kSplitWaveFloats + lane * 2;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int db = j >> 3, e = 2 * (j & 7);
    st_dev2(base + j * 128, o[db][e], o[db][e + 1]);
  }
  st_dev2(a.sml + (wb * 64 + lane) * 2, m, lt);
}

// The last split of a column block to arrive merges every split's partial
// (its own included, read back like the others) by log-sum-exp with a running
// maximum, in split order, so the result does not depend on which split came
// last.  Two splits' (m, sum) and O are requested together.  Returns (m,
// sum); o receives the merged unnormalised output.
__device__ __forceinline__ float2 merge_split_partials(const AttnArgs& a, int slot, int wave, f32x16 o[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float mrun = -INFINITY, den = 0.0f;
  auto add = [&](float2 x, const float2 v[32]) {
    if (!(x.y > 0.0f)) return;
    const float mnew = den > 0.0f ? fmaxf(mrun, x.x) : x.x;
    const float sold = den > 0.0f ? __builtin_amdgcn_exp2f(mrun - mnew) : 0.0f;
    const float wgt = __builtin_amdgcn_exp2f(x.x - mnew);
    den = __builtin_fmaf(wgt, x.y, den * sold);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int db = j >> 3, e = 2 * (j & 7);
      o[db][e] = __builtin_fmaf(wgt, v[j].x, o[db][e] * sold);
      o[db][e + 1] = __builtin_fmaf(wgt, v[j].y, o[db][e + 1] * sold);
    }
    mrun = mnew;
  };
  for (int sp = 0; sp < a.n_split_wg; sp += 2) {
    const bool two = sp + 1 < a.n_split_wg;
    const int64_t wb0 = split_wave_block(a, slot, sp, wave);
    const int64_t wb1 = two ? wb0 + 4 : wb0;
    const float* b0 = a.spart + wb0 * kSplitWaveFloats + lane * 2;
    const float* b1 = a.spart + wb1 * kSplitWaveFloats + lane * 2;
    const float2 x0 = ld_dev2(a.sml + (wb0 * 64 + lane) * 2);
    const float2 x1 = ld_dev2(a.sml + (wb1 * 64 + lane) * 2);
    float2 v0[32], v1[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v0[j] = ld_dev2(b0 + j * 128);
#pragma unroll
    for (int j = 0; j < 32; ++j) v1[j] = ld_dev2(b1 + j * 128);
    add(x0, v0);
    if (two) add(x1, v1);
  }
  return make_float2(mrun, den);
}

// ---- decode with the token's own row in the kernel ----
// A lane's query fragments are the 16-byte granules 2 s + g2 (s = 0..7) of
// its column's row, so granule s < 4 (elements k) pairs with granule s + 4
// (elements k + 64) in the same lane: the rotation by the token's position
// needs no lane exchange, and it rounds exactly as the prologue does.  x[s]
// holds granule 2 s + g2 of a row of request u's token.  (Holding the
// lane's 32 phases from before the first tile's copies, so that this waits
// for them only, made the decode instances spill and ran slower.)
__device__ __forceinline__ void dec_rotate(const AttnArgs& a, int u, u32x4 x[8]) {
  if (a.new_pos[u] == 0) return;
  const int g2 = (threadIdx.x & 63) >> 5;
  const Phase* pp = a.dec_phase + int64_t(u) * 64;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    Phase ph[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ph[e] = pp[8 * (2 * s + g2) + e];
    rotate_vec<true>(x[s], x[s + 4], ph);
  }
}

// The column block's last split starts from the token's own row, which the
// tiles leave out: the key rotated like the queries and scored from registers
// (a lane holds half of its column's dot product, lane ^ 32 the other half)
// sets the reference maximum, so its probability is exp2(0) = 1 (exact in
// bf16): the sum starts at 1 and O at the value (d = 32 db + 8 qq + 4 g2 + e,
// as the accumulators hold them).  The tiles then continue the online
// softmax.  The rotated key and the value also go to the token's rows of the
// planes, for the steps that follow (lanes 0 and 32 hold the whole key
// between them).
__device__ __forceinline__ void dec_own_row(const AttnArgs& a, const Col& c, const bf16x8 qb[8], int head,
                                            float& m, float& lsum, f32x16 o[4]) {
  const int lane = threadIdx.x & 63, g2 = lane >> 5;
  const int64_t src = (int64_t(c.u) * a.kv_heads + head) * 128;
  const uint16_t* vr = a.v_new + src;
  u32x4 kx[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kx[s] = ld16(a.k_new + src + 8 * (2 * s + g2));
  u32x2 vv[4][4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) vv[db][qq] = *reinterpret_cast<const u32x2*>(vr + 32 * db + 8 * qq + 4 * g2);
  dec_rotate(a, c.u, kx);
  const int64_t dst = (int64_t(head) * a.cap + a.dec_row[c.u]) * 128;
  if ((lane & 31) == 0) {
#pragma unroll
    for (int s = 0; s < 8; ++s) st16(a.k_own + dst + 8 * (2 * s + g2), kx[s]);
  }
  if (lane < 16) st16(a.v_own + dst + 8 * lane, ld16(vr + 8 * lane));
  float sc = 0.0f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x4 q = __builtin_bit_cast(u32x4, qb[s]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sc = __builtin_fmaf(bf16_lo(q[w]), bf16_lo(kx[s][w]), sc);
      sc = __builtin_fmaf(bf16_hi(q[w]), bf16_hi(kx[s][w]), sc);
    }
  }
  sc += __shfl_xor(sc, 32);
  m = sc * a.scale_log2;
  lsum = g2 == 0 ? 1.0f : 0.0f;   // the column's two lanes add up to 1
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      o[db][4 * qq + 0] = bf16_lo(vv[db][qq][0]);
      o[db][4 * qq + 1] = bf16_hi(vv[db][qq][0]);
      o[db][4 * qq + 2] = bf16_lo(vv[db][qq][1]);
      o[db][4 * qq + 3] = bf16_hi(vv[db][qq][1]);
    }
}

// ---------------------------------------------------------------------------
// attention kernel
// ---------------------------------------------------------------------------
// A work item is 128 query columns of one (request, kv head) over a range of
// tiles, run by a group of 4 waves that streams its tiles through its own two
// LDS stages (the next tile streams in while the current one is consumed),
// one barrier per tile.  Unpaired: one item per workgroup, two workgroups per
// CU, independent of each other.  Paired (row splits): one workgroup of 8
// waves per CU runs the two splits of one column block; they share the
// per-tile barrier, and after the last tile the second group hands its
// (O, m, sum) to the first through LDS, which writes the merged result, so
// no partials leave the CU.  The fused variant
// reads prefix rows straight from the pool: values with direct copies, keys
// through registers, rotated on the way.

constexpr int kStageBytes = 2 * kTileBytes + 256;
constexpr int kGroupLdsBytes = 2 * kStageBytes;
constexpr int kAttnLdsBytes = 2 * kGroupLdsBytes;

// Per-lane byte offsets, inside a 64-row tile of one plane, of the 16-byte
// granules a lane copies: 4 blocks of 1 KB (4 rows) per wave, the granule
// order swizzled as the readers expect.
struct TileLanes {
  unsigned k[4], v[4];
};

// Blocks b0 .. b0 + 3 (a group's wave w copies b0 = 4 w; with rows shared
// by both groups of a workgroup, wave w8 of the 8 copies b0 = 2 w8, 2 blocks).
__device__ __forceinline__ void tile_lanes(int b0, TileLanes& tl) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (b0 + i) * 4 + (lane >> 4);
    tl.k[i] = r * 256 + ((lane & 15) ^ k_swz(r)) * 16;
    tl.v[i] = r * 256 + ((lane & 15) ^ v_swz(r)) * 16;
  }
}

// Copy NB blocks (b0 .. b0 + NB - 1, 4 rows of 256 bytes each) of one
// 64-row tile of one plane into LDS.  `base` is the request's row 0, `t0` the
// tile's first row.  A full tile is addressed as one uniform base plus the
// fixed lane offsets; the request's last tile repeats its last row past the
// end.
template <bool VALUE, int NB>
__device__ __forceinline__ void tile_to_lds(const char* base, int t0, int rows, const TileLanes& tl, char* lds,
                                            int b0) {
  const unsigned* off = VALUE ? tl.v : tl.k;
  if (t0 + kAttnRowsPerTile <= rows) {
    const char* tbase = base + int64_t(t0) * 256;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      __builtin_amdgcn_global_load_lds(tbase + off[i], (lds_void_ptr)(lds + (b0 + i) * 1024), 16, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int rr = min(t0 + int(off[i] >> 8), rows - 1);
      __builtin_amdgcn_global_load_lds(base + int64_t(rr) * 256 + (off[i] & 255u),
                                       (lds_void_ptr)(lds + (b0 + i) * 1024), 16, 0, 0);
    }
  }
}

// Row positions of one tile into LDS (wave 0 of the group, one 4-byte lane
// load each).
__device__ __forceinline__ void pos_to_lds(const int32_t* pos_row0, int t0, int rows, char* lds, int wave) {
  if (wave == 0) {
    const int rr = min(t0 + int(threadIdx.x & 63), rows - 1);
    __builtin_amdgcn_global_load_lds(pos_row0 + rr, (lds_void_ptr)lds, 4, 0, 0);
  }
}

// Fused variant: value rows straight from the pool pages (prefix rows) or the
// assembled tail (new rows).
__device__ __forceinline__ const char* fused_row(const AttnArgs& a, const ReqRec& rq, int head,
                                                 int rr, bool value, int2* src_out) {
  if (rr < rq.prefix_rows) {
    const int2 src = a.rowsrc[rq.row_base + rr];
    if (src_out) *src_out = src;
    return a.pool + int64_t(src.x >> a.page_shift) * a.page_bytes + a.kv_plane_off +
           (value ? a.v_off : 0) + (int64_t(head) * a.page_tokens + (src.x & (a.page_tokens - 1))) * 256;
  }
  if (src_out) *src_out = make_int2(-1, -1);
  const uint16_t* plane = value ? a.v_plane : a.k_plane;
  return reinterpret_cast<const char*>(plane + (int64_t(head) * a.cap + rq.row_base + rr) * 128);
}

__device__ __forceinline__ void fused_v_to_lds(const AttnArgs& a, const ReqRec& rq, int head, int t0,
                                               int rows, char* lds, int wave) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = wave * 4 + i;
    const int r = blk * 4 + (lane >> 4);
    const int rr = min(t0 + r, rows - 1);
    const int gran = (lane & 15) ^ v_swz(r);
    const char* row = fused_row(a, rq, head, rr, true, nullptr);
    __builtin_amdgcn_global_load_lds(row + gran * 16, (lds_void_ptr)(lds + blk * 1024), 16, 0, 0);
  }
}

// Fused variant: keys through registers (rotated on the way) into the same
// swizzled layout.  Thread units (tid: the thread within its 4-wave group):
// rows (tid >> 3) + 32 i, pair vector j = tid & 7.
struct FusedK {
  u32x4 k[2][2];
  int phase[2];   // phase_tab row of each key, -1 for none
};

__device__ __forceinline__ void fused_k_load(const AttnArgs& a, const ReqRec& rq, int head, int t0,
                                             int rows, FusedK& f) {
  const int tid = threadIdx.x & 255;
  const int j = tid & 7;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int rr = min(t0 + r, rows - 1);
    int2 src;
    const char* row = fused_row(a, rq, head, rr, false, &src);
    f.k[i][0] = ld16(row + j * 16);
    f.k[i][1] = ld16(row + 128 + j * 16);
    f.phase[i] = src.y;
  }
}

__device__ __forceinline__ void fused_k_store(const AttnArgs& a, FusedK& f, char* lds) {
  const int tid = threadIdx.x & 255;
  const int j = tid & 7;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 3) + 32 * i;
    if (f.phase[i] >= 0) {
      Phase ph[8];
      const Phase* pp = a.phase_tab + int64_t(f.phase[i]) * 64 + j * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) ph[e] = pp[e];
      rotate_vec<true>(f.k[i][0], f.k[i][1], ph);
    }
    st16(lds + r * 256 + 16 * (j ^ k_swz(r)), f.k[i][0]);
    st16(lds + r * 256 + 16 * ((j + 8) ^ k_swz(r)), f.k[i][1]);
  }
}

// Source of row rr of a request's rows in plane K or V of the layer: the pool
// page slot of a prefix row, or the assembled planes for a new-token row
// (slot < 0).
__device__ __forceinline__ const char* pool_or_plane_row(const AttnArgs& a, const ReqRec& rq, int head, int rr,
                                                         int slot, bool value) {
  if (slot >= 0)
    return a.pool + int64_t(slot >> a.page_shift) * a.page_bytes + a.kv_plane_off + (value ? a.v_off : 0) +
           (int64_t(head) * a.page_tokens + (slot & (a.page_tokens - 1))) * 256;
  const uint16_t* plane = value ? a.v_plane : a.k_plane;
  return reinterpret_cast<const char*>(plane + (int64_t(head) * a.cap + rq.row_base + rr) * 128);
}

// Values left in the pool (assembled keys, pooled values): copy NB row
// blocks (b0 .. b0 + NB - 1, 4 rows each) of tile t0's values into LDS, the
// lane's row i from pool slot slots[i] (prefix rows) or the planes (the rest),
// granules swizzled as the transpose reads expect.
template <int NB>
__device__ __forceinline__ void vpool_to_lds(const AttnArgs& a, const ReqRec& rq, int head, int t0, int rows,
                                             const int* slots, char* lds, int b0) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = (b0 + i) * 4 + (lane >> 4);
    const int rr = min(t0 + r, rows - 1);
    const char* row = pool_or_plane_row(a, rq, head, rr, slots[i], true);
    __builtin_amdgcn_global_load_lds(row + ((lane & 15) ^ v_swz(r)) * 16, (lds_void_ptr)(lds + (b0 + i) * 1024),
                                     16, 0, 0);
  }
}

// DEC: decode with the token's own row handled here (a.dec_own), a separate
// instance so that the prefill's register allocation is untouched.
template <bool FUSED, bool PAIRED, bool VPOOL = false, bool DEC = false>
__global__ __launch_bounds__(PAIRED ? 512 : 256, PAIRED ? 1 : 2) void attention_bf16_kernel(AttnArgs a) {
  static_assert(!VPOOL || (!FUSED && PAIRED), "pooled values are read by the assembled-plane variant");
  extern __shared__ __attribute__((aligned(1024))) char lds_all[];
  constexpr int G = PAIRED ? 2 : 1;           // work items per workgroup
  const int blk = a.wg_map ? ((const __attribute__((address_space(4))) int*)(a.wg_map))[blockIdx.x]
                          : xcd_remap(blockIdx.x, gridDim.x);
  if (blk < 0) return;   // a slot of the launch order left empty
  const int wave8 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = PAIRED ? wave8 >> 2 : 0;
  // wave within the group.  A decode item has one query token, so only its
  // first wave has columns; the second group's waves are rotated by one so
  // that the two groups' live waves sit on different SIMDs (wave8 mod 4).
  const int wave = (PAIRED && grp == 1 && a.decode) ? ((wave8 + 3) & 3) : (wave8 & 3);
  const int item = G * blk + grp;
  const bool has = item < a.n_work;
  const AttnWork w = a.work[has ? item : G * blk];
  // tiles in [gap_begin, gap_end) are skipped
  const int gap = w.gap_end - w.gap_begin;
  const int T = has ? w.tile_end - w.tile_begin - gap : 0;
  // both groups of a pair pass the same number of barriers
  const AttnWork w0 = a.work[G * blk];
  // the pair covers the same rows: one stream of copies shared by all 8 waves
  const bool shared = PAIRED && !FUSED && w0.share_rows != 0;
  int steps = T;
  if (PAIRED) {
    auto len = [](const AttnWork& x) { return x.tile_end - x.tile_begin - (x.gap_end - x.gap_begin); };
    const int T_other = grp == 0 ? (item + 1 < a.n_work ? len(a.work[item + 1]) : 0) : len(w0);
    steps = max(T, T_other);
  }
  char* smem = lds_all + (shared ? 0 : grp * kGroupLdsBytes);
  const ReqRec rq = a.reqs[w.req];
  const int rows = rq.prefix_rows + rq.n_new;

  Col c;
  bf16x8 qb[8];
  col_setup(a, w, rq, wave, lds_addr(smem), c, qb);
  // this lane's row-position reads in stage 0 (minus kPosOffset)
  const unsigned paddr = lds_addr(smem) + 16 * ((threadIdx.x & 63) >> 5);
  TileLanes tl;
  tile_lanes(shared ? 2 * wave8 : 4 * wave, tl);

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float lsum = 0.0f;   // this lane's half of its column's denominator
  float m = -INFINITY;

  const char* kbase = reinterpret_cast<const char*>(a.k_plane + (int64_t(w.head) * a.cap + rq.row_base) * 128);
  const char* vbase = reinterpret_cast<const char*>(a.v_plane + (int64_t(w.head) * a.cap + rq.row_base) * 128);
  const int32_t* pbase = a.pos + rq.row_base;
  const int tb = w.tile_begin;
  // the group's i-th tile: tiles from step `gap_at` on come `gap` later
  const int gap_at = __builtin_amdgcn_readfirstlane(gap > 0 ? w.gap_begin - tb : INT_MAX);
  auto tile_of = [&](int i) { return i >= gap_at ? tb + i + gap : tb + i; };
  FusedK fk;
  // pooled values: pool slots of the lane's value rows in the next tile to
  // copy (-1: not a prefix row), fetched a step ahead
  int vslot[4] = {-1, -1, -1, -1};
  auto vpool_src = [&](int t) {
    const int b0 = shared ? 2 * wave8 : 4 * wave;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= 2 && shared) break;
      const int rr = min(t * kAttnRowsPerTile + (b0 + i) * 4 + int((threadIdx.x & 63) >> 4), rows - 1);
      vslot[i] = rr < rq.prefix_rows ? a.rowsrc[rq.row_base + rr].x : -1;
    }
  };

  // copies of tile t into stage S (0 or 1)
  auto issue = [&](auto stage_c, int t) {
    constexpr int S = decltype(stage_c)::value;
    char* st = smem + S * kStageBytes;
    const int t0 = t * kAttnRowsPerTile;
    if (FUSED) {
      fused_k_load(a, rq, w.head, t0, rows, fk);
      fused_v_to_lds(a, rq, w.head, t0, rows, st + kTileBytes, wave);
    } else {
      if (shared) {
        tile_to_lds<false, 2>(kbase, t0, rows, tl, st, 2 * wave8);
        if (VPOOL)
          vpool_to_lds<2>(a, rq, w.head, t0, rows, vslot, st + kTileBytes, 2 * wave8);
        else
          tile_to_lds<true, 2>(vbase, t0, rows, tl, st + kTileBytes, 2 * wave8);
      } else {
        tile_to_lds<false, 4>(kbase, t0, rows, tl, st, 4 * wave);
        if (VPOOL)
          vpool_to_lds<4>(a, rq, w.head, t0, rows, vslot, st + kTileBytes, 4 * wave);
        else
          tile_to_lds<true, 4>(vbase, t0, rows, tl, st + kTileBytes, 4 * wave);
      }
    }
    pos_to_lds(pbase, t0, rows, st + kPosOffset, shared ? wave8 : wave);
  };

  // position bounds of tile t; in decode mode every row is visible and only
  // the last tile (rows past the end) needs the mask
  // (scalar loads through the constant address space, so they never wait on
  // copies in flight)
  const int tile_base = __builtin_amdgcn_readfirstlane(rq.tile_base);
  const __attribute__((address_space(4))) int* tile_pos_c =
      (const __attribute__((address_space(4))) int*)(a.tile_pos);
  auto bounds = [&](int t) {
    if (a.decode) return make_int2(INT_MIN, (t + 1) * kAttnRowsPerTile > rows ? INT_MAX : INT_MIN);
    const int k = 2 * (tile_base + t);
    return make_int2(tile_pos_c[k], tile_pos_c[k + 1]);
  };
  int2 tp_next = make_int2(INT_MAX, INT_MAX);
  if (T > 0) {
    tp_next = bounds(tile_of(0));
    if (VPOOL) vpool_src(tile_of(0));
    issue(std::integral_constant<int, 0>{}, tile_of(0));
    if (VPOOL && T > 1) vpool_src(tile_of(1));
  }
  if (FUSED && T > 0) fused_k_store(a, fk, smem);
  // decode with the token's own row: the raw queries, loaded by col_setup,
  // are rotated once the first tile's copies are on their way
  if (DEC && c.wq_max != INT_MIN) {
    u32x4 qx[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) qx[s] = __builtin_bit_cast(u32x4, qb[s]);
    dec_rotate(a, c.u, qx);
#pragma unroll
    for (int s = 0; s < 8; ++s) qb[s] = __builtin_bit_cast(bf16x8, qx[s]);
    if (has && w.split == a.dec_split - 1) dec_own_row(a, c, qb, w.head, m, lsum, o);
  }
  // step i: the group's tile tb + i sits in stage S (i even: 0); wait for its
  // copies, start the next tile's copies into the other stage, consume it
  auto step = [&](auto stage_c, int i) {
    constexpr int S = decltype(stage_c)::value;
    wait_vm();
    __syncthreads();
    if (i >= T) return;
    const int t = tile_of(i);
    const bool more = i + 1 < T;
    const int2 tp = tp_next;
    if (more) {
      const int tn = tile_of(i + 1);
      tp_next = bounds(tn);
      issue(std::integral_constant<int, 1 - S>{}, tn);
      if (VPOOL && i + 2 < T) vpool_src(tile_of(i + 2));
    }
    // (a wave without columns has wq_max INT_MIN and computes nothing)
    if (tp.x <= c.wq_max && c.wq_max != INT_MIN)
      tile_pipelined<S * kStageBytes>(c, qb, tp, paddr, t * kAttnRowsPerTile, rows, a.scale_log2, m, o, lsum);
    if (FUSED && more) fused_k_store(a, fk, smem + (1 - S) * kStageBytes);
  };
  for (int i = 0; i < steps; i += 2) {
    step(std::integral_constant<int, 0>{}, i);
    if (i + 1 < steps) step(std::integral_constant<int, 1>{}, i + 1);
  }

  // the column's denominator: this lane's rows and lane ^ 32's
  float lt = lsum + __shfl_xor(lsum, 32);
  if (PAIRED && w0.merge_pair) {
    // the second split of the pair hands (O, m, sum) to the first through LDS,
    // laid out [wave][16-byte chunk][lane] so that both sides are
    // conflict-free; split order is kept: first + second
    __syncthreads();
    const int lane = threadIdx.x & 63;
    f32x4* xo = reinterpret_cast<f32x4*>(lds_all) + wave * 16 * 64 + lane;
    float2* xml = reinterpret_cast<float2*>(lds_all + 4 * 16 * 64 * 16) + wave * 64 + lane;
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          xo[(db * 4 + qq) * 64] = f32x4{o[db][4 * qq], o[db][4 * qq + 1], o[db][4 * qq + 2], o[db][4 * qq + 3]};
      *xml = make_float2(m, lt);
    }
    __syncthreads();
    if (grp == 1) return;
    const float2 ml1 = *xml;
    const bool l0 = lt > 0.0f, l1 = ml1.y > 0.0f;
    const float mm = l0 ? (l1 ? fmaxf(m, ml1.x) : m) : ml1.x;
    const float w0f = l0 ? __builtin_amdgcn_exp2f(m - mm) : 0.0f;
    const float w1f = l1 ? __builtin_amdgcn_exp2f(ml1.x - mm) : 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x4 x = xo[(db * 4 + qq) * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[db][4 * qq + e] = w0f * o[db][4 * qq + e] + w1f * x[e];
      }
    lt = w0f * lt + w1f * ml1.y;
    m = (l0 || l1) ? mm : -INFINITY;
  } else if (!DEC && a.n_split_wg > 1) {
    // rows split over workgroups: each split stores its partial and then
    // counts itself in the column block's counter; the last to arrive merges
    // and writes the output, and leaves the counter at 0 for the next launch
    __shared__ int arrived[G];
    const bool counted = has && w.slot >= 0;
    if (counted) store_split_partial(a, w.slot, w.split, wave, o, m, lt);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the stores have reached device scope
    __syncthreads();
    // release: this split's partials (stored above by every wave of the
    // group, ordered before this by the barrier) happen before the count;
    // acquire: the last split to count sees every other split's partials
    if (counted && (threadIdx.x & 255) == 0)
      arrived[grp] = __hip_atomic_fetch_add(a.split_count + w.slot, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (!counted || arrived[grp] != a.n_split_wg - 1) return;
    if ((threadIdx.x & 255) == 0) a.split_count[w.slot] = 0;
    const float2 ml = merge_split_partials(a, w.slot, wave, o);
    m = ml.x;
    lt = ml.y;
  } else if (!has) {
    return;
  }
  if (DEC) {
    // decode: one wave of the group has columns (the group's query heads of
    // one token); the others are done.  Row splits go to merge_kernel: a
    // merge by the last split here needs an agent-scope acquire-release
    // count per workgroup, whose L2 write-back and invalidate cost more than
    // the extra launch.
    if (c.wq_max == INT_MIN) return;
    const bool merged = PAIRED && w0.merge_pair;
    const int part = merged ? w.split / 2 : w.split;
    store_column(a, c, o, lt, m, a.n_split_out > 1, part);
    return;
  }
  // merged pairs write partial split/2 (or the output when that was the only
  // pair); unpaired items write partial `split` (or the output)
  const int part = PAIRED && w0.merge_pair ? w.split / 2 : w.split;
  store_column(a, c, o, lt, m, a.n_split_out > 1, part);
}

// Log-sum-exp merge of the row splits, in split order.  32 threads per
// (new token, query head), 4 output values each; every split's partial is
// requested before any is combined.
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const int64_t item = int64_t(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int d0 = (threadIdx.x & 31) * 4;
  const int64_t n_items = int64_t(a.n_new) * a.q_heads;
  if (item >= n_items) return;
  float2 ml[kAttnMaxSplit];
  f32x4 part[kAttnMaxSplit];
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplit; ++sp) {
    if (sp < a.n_split_out) {
      const int64_t idx = int64_t(sp) * n_items + item;
      ml[sp] = a.ml[idx];
      part[sp] = *reinterpret_cast<const f32x4*>(a.opart + idx * 128 + d0);
    }
  }
  float mmax = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplit; ++sp)
    if (sp < a.n_split_out && ml[sp].y > 0.0f) mmax = fmaxf(mmax, ml[sp].x);
  float den = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplit; ++sp) {
    if (sp < a.n_split_out && ml[sp].y > 0.0f) {
      const float wgt = __builtin_amdgcn_exp2f(ml[sp].x - mmax);
      den += wgt * ml[sp].y;
      acc += wgt * part[sp];
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const __bf16 b0 = (__bf16)(acc[0] * inv), b1 = (__bf16)(acc[1] * inv);
  const __bf16 b2 = (__bf16)(acc[2] * inv), b3 = (__bf16)(acc[3] * inv);
  u32x2 pk;
  pk[0] = unsigned(__builtin_bit_cast(uint16_t, b0)) | (unsigned(__builtin_bit_cast(uint16_t, b1)) << 16);
  pk[1] = unsigned(__builtin_bit_cast(uint16_t, b2)) | (unsigned(__builtin_bit_cast(uint16_t, b3)) << 16);
  *reinterpret_cast<u32x2*>(a.out + item * 128 + d0) = pk;
}

// ---------------------------------------------------------------------------
// fp32 attention (plain VALU; one wave per new token and query head)
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void attention_f32_kernel(AttnF32Args a) {
  constexpr int EPL = D / 64;
  const int64_t item = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= int64_t(a.n_new) * a.q_heads) return;
  const int u = int(item / a.q_heads);
  const int hq = int(item - int64_t(u) * a.q_heads);
  const int h = hq / a.group;
  const ReqRec rq = a.reqs[a.new_req[u]];
  const int rows = rq.prefix_rows + rq.n_new;
  const int qpos = a.new_pos[u];
  const float* qv = reinterpret_cast<const float*>(a.q_rot) + item * D;
  const float* kp = reinterpret_cast<const float*>(a.k_plane) + (int64_t(h) * a.cap + rq.row_base) * D;
  const float* vp = reinterpret_cast<const float*>(a.v_plane) + (int64_t(h) * a.cap + rq.row_base) * D;
  float q[EPL], acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    q[e] = qv[lane + 64 * e];
    acc[e] = 0.0f;
  }
  const float scale = 1.0f / sqrtf(float(D));
  float m = -INFINITY, l = 0.0f;
  for (int r = 0; r < rows; ++r) {
    if (a.pos[rq.row_base + r] > qpos) continue;
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) dot = fmaf(q[e], kp[int64_t(r) * D + lane + 64 * e], dot);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
    const float s = dot * scale;
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn);
    const float p = expf(s - mn);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, vp[int64_t(r) * D + lane + 64 * e], acc[e] * alpha);
    m = mn;
  }
  float* op = reinterpret_cast<float*>(a.out) + item * D;
#pragma unroll
  for (int e = 0; e < EPL; ++e) op[lane + 64 * e] = acc[e] / l;
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {
// Hot-set fill: bytes [off, off + 16 n16) of pool page pairs[2i] (the
// pinned host pool as the device addresses it) to the same bytes of cache
// slot pairs[2i + 1]; 16 KB per workgroup, `chunks` workgroups per pair.
__global__ __launch_bounds__(256) void cache_fill_kernel(const char* src_pool, char* cache, const int32_t* pairs,
                                                         int64_t page_bytes, int64_t off, int64_t n16, int chunks) {
  const int i = blockIdx.x / chunks, ch = blockIdx.x - i * chunks;
  const int64_t page = pairs[2 * i], slot = pairs[2 * i + 1];
  const u32x4* src = reinterpret_cast<const u32x4*>(src_pool + page * page_bytes + off);
  u32x4* dst = reinterpret_cast<u32x4*>(cache + slot * page_bytes + off);
  const int64_t k0 = int64_t(ch) * 256 + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k = k0 + int64_t(j) * chunks * 256;
    if (k < n16) v[j] = src[k];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k = k0 + int64_t(j) * chunks * 256;
    if (k < n16) dst[k] = v[j];
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t* p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
}  // namespace

hipError_t launch_cache_fill(const char* src_pool, char* cache, const int32_t* pairs, int32_t n_pairs,
                             int64_t page_bytes, int64_t off, int64_t bytes, hipStream_t s) {
  if (n_pairs <= 0 || bytes <= 0) return hipSuccess;
  const int64_t n16 = bytes / 16;
  const int chunks = int((n16 + 1023) / 1024);
  hipLaunchKernelGGL(cache_fill_kernel, dim3(unsigned(int64_t(n_pairs) * chunks)), dim3(256), 0, s, src_pool, cache,
                     pairs, page_bytes, off, n16, chunks);
  return hipGetLastError();
}

hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_decode_plan(const DecodePlanArgs& a, hipStream_t s) {
  const int64_t n = int64_t(a.batch) * a.half_dim;
  if (n > 0) hipLaunchKernelGGL(decode_plan_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const int64_t n1 = a.prefix_rows + a.n_new;
  if (n1 > 0) {
    hipLaunchKernelGGL(plan_rows_kernel, dim3(unsigned((n1 + 255) / 256)), dim3(256), 0, s, a);
  }
  const int64_t n2 = (int64_t(a.phase_rows) + a.n_new) * a.half_dim;
  if (n2 > 0) {
    hipLaunchKernelGGL(plan_phase_kernel, dim3(unsigned((n2 + 255) / 256)), dim3(256), 0, s, a);
  }
  const int n3 = max(a.n_tiles, a.n_slots);
  if (n3 > 0) {
    hipLaunchKernelGGL(plan_tiles_kernel, dim3(unsigned((n3 + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool gather_supported(int dtype, int head_dim) {
  (void)dtype;
  return head_dim == 64 || head_dim == 128;
}

template <bool BF16, int D>
static void gather_launch(const GatherArgs& a, hipStream_t s) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int LPR = D / (2 * (16 / ES));
  constexpr int RPB = 256 / LPR;
  const int n_planes = a.plane_end - a.plane_begin;
  const int64_t groups = (n_planes + a.planes_per_block - 1) / a.planes_per_block;
  GatherArgs b = a;
  b.row_blocks8 = ((a.prefix_rows + RPB - 1) / RPB + 7) / 8 * 8;
  dim3 grid(unsigned(b.row_blocks8 * groups));
  if constexpr (BF16 && D == 128) {
    if (!a.values) {
      hipLaunchKernelGGL((gather_kernel<BF16, D, false>), grid, dim3(256), 0, s, b);
      return;
    }
  }
  hipLaunchKernelGGL((gather_kernel<BF16, D, true>), grid, dim3(256), 0, s, b);
}

hipError_t launch_gather(int dtype, int head_dim, const GatherArgs& a, hipStream_t s) {
  if (a.prefix_rows <= 0 || a.plane_end <= a.plane_begin) return hipSuccess;
  // keys only is implemented where attention can read values from the pool
  if (!a.values && !(dtype == PIC_BF16 && head_dim == 128)) return hipErrorInvalidValue;
  if (dtype == PIC_BF16) {
    if (head_dim == 128) gather_launch<true, 128>(a, s);
    else gather_launch<true, 64>(a, s);
  } else {
    if (head_dim == 128) gather_launch<false, 128>(a, s);
    else gather_launch<false, 64>(a, s);
  }
  return hipGetLastError();
}

template <bool BF16, int D>
static void prologue_launch(const PrologueArgs& a, hipStream_t s) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int LPR = D / (2 * (16 / ES));
  constexpr int GPB = 256 / LPR;
  const int per_tok = a.q_heads + 2 * a.kv_heads;
  const int64_t groups = int64_t(a.n_new) * ((per_tok + kPrologueRows - 1) / kPrologueRows);
  hipLaunchKernelGGL((prologue_kernel<BF16, D>), dim3(unsigned((groups + GPB - 1) / GPB)), dim3(256), 0,
                     s, a);
}

hipError_t launch_prologue(int dtype, int head_dim, const PrologueArgs& a, hipStream_t s) {
  if (a.n_new <= 0) return hipSuccess;
  if (dtype == PIC_BF16) {
    if (head_dim == 128) prologue_launch<true, 128>(a, s);
    else prologue_launch<true, 64>(a, s);
  } else {
    if (head_dim == 128) prologue_launch<false, 128>(a, s);
    else prologue_launch<false, 64>(a, s);
  }
  return hipGetLastError();
}

bool attention_supported(int dtype, int head_dim, bool fused) {
  if (dtype == PIC_BF16) return head_dim == 128;
  return !fused && (head_dim == 64 || head_dim == 128);
}

hipError_t launch_attention_bf16(const AttnArgs& a, bool fused, hipStream_t s) {
  if (a.n_work <= 0) return hipSuccess;
  // dynamic LDS above 64 KB has to be allowed per kernel, once
  static const hipError_t attr = [] {
    const void* fns[8] = {reinterpret_cast<const void*>(attention_bf16_kernel<true, true>),
                          reinterpret_cast<const void*>(attention_bf16_kernel<false, true>),
                          reinterpret_cast<const void*>(attention_bf16_kernel<true, false>),
                          reinterpret_cast<const void*>(attention_bf16_kernel<false, true, true>),
                          reinterpret_cast<const void*>(attention_bf16_kernel<true, true, false, true>),
                          reinterpret_cast<const void*>(attention_bf16_kernel<false, true, false, true>),
                          reinterpret_cast<const void*>(attention_bf16_kernel<true, false, false, true>),
                          reinterpret_cast<const void*>(attention_bf16_kernel<false, true, true, true>)};
    const int bytes[8] = {kAttnLdsBytes, kAttnLdsBytes, kGroupLdsBytes, kAttnLdsBytes,
                          kAttnLdsBytes, kAttnLdsBytes, kGroupLdsBytes, kAttnLdsBytes};
    for (int i = 0; i < 8; ++i) {
      hipError_t e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, bytes[i]);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
  // the assembled-plane variant always runs two items per workgroup: row
  // splits merged in LDS, or neighbouring column blocks sharing their rows'
  // copies; the fused variant pairs only the row splits it merges
  const unsigned pairs = a.wg_map ? unsigned(a.n_wg) : unsigned((a.n_work + 1) / 2);
  const unsigned singles = a.wg_map ? unsigned(a.n_wg) : unsigned(a.n_work);
  if (a.dec_own) {
    if (!fused && a.v_pool)
      hipLaunchKernelGGL((attention_bf16_kernel<false, true, true, true>), dim3(pairs), dim3(512), kAttnLdsBytes,
                         s, a);
    else if (!fused)
      hipLaunchKernelGGL((attention_bf16_kernel<false, true, false, true>), dim3(pairs), dim3(512), kAttnLdsBytes,
                         s, a);
    else if (a.paired)
      hipLaunchKernelGGL((attention_bf16_kernel<true, true, false, true>), dim3(pairs), dim3(512), kAttnLdsBytes,
                         s, a);
    else
      hipLaunchKernelGGL((attention_bf16_kernel<true, false, false, true>), dim3(singles), dim3(256),
                         kGroupLdsBytes, s, a);
  } else if (!fused && a.v_pool)
    hipLaunchKernelGGL((attention_bf16_kernel<false, true, true>), dim3(pairs), dim3(512), kAttnLdsBytes, s, a);
  else if (!fused)
    hipLaunchKernelGGL((attention_bf16_kernel<false, true>), dim3(pairs), dim3(512), kAttnLdsBytes, s, a);
  else if (a.paired)
    hipLaunchKernelGGL((attention_bf16_kernel<true, true>), dim3(pairs), dim3(512), kAttnLdsBytes, s, a);
  else
    hipLaunchKernelGGL((attention_bf16_kernel<true, false>), dim3(singles), dim3(256), kGroupLdsBytes, s, a);
  if (a.n_split_out > 1) {
    const int64_t items = int64_t(a.n_new) * a.q_heads;
    hipLaunchKernelGGL(merge_kernel, dim3(unsigned((items + 7) / 8)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attention_f32(int head_dim, const AttnF32Args& a, hipStream_t s) {
  const int64_t items = int64_t(a.n_new) * a.q_heads;
  if (items <= 0) return hipSuccess;
  if (head_dim == 128)
    hipLaunchKernelGGL(attention_f32_kernel<128>, dim3(unsigned((items + 3) / 4)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attention_f32_kernel<64>, dim3(unsigned((items + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pic
