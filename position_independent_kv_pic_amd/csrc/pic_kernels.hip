// HIP kernels for position-independent KV-cache reuse on gfx950 (CDNA4).
//
//   plan      per-row positions and pool sources, per-span and per-token
//             RoPE phases (fp64 cos/sin split into fp32 head + remainder)
//   gather    assembly: copy every span's cached rows out of the paged pool
//             into the contiguous prefix, rotating keys by the span's delta
//             (CoinRAG page, section 2.3, the C_ctx equation and Rot(.; Delta_i);
//             TurboRAG review page, Reordered Positions: apply RoPE again at
//             the new position)
//   prologue  rotate the new tokens' queries and keys to their positions and
//             append the new keys/values after the prefix
//   attention query-prefill attention over prefix + new rows with the mask
//             pos_row <= pos_query (TurboRAG Figure 4: the query sees every
//             chunk and itself; SemPIC: causal interleave), GQA, bf16 MFMA
//             32x32x16 with fp32 accumulation and online softmax; optional
//             split of the rows with a log-sum-exp merge
//
// Rotation arithmetic.  Each key pair (x, y) = (k, k + d/2) is rotated by an
// angle whose cos/sin were computed in fp64 and stored as fp32 head + fp32
// remainder.  The products are formed exactly with FMA (error-free
// transformations) and summed with two-sum, so the result carries about 48
// good bits in two fp32 words; it is then rounded once to bf16 (ties to even,
// with the remainder breaking exact ties) or to fp32.  A rotation by zero is a
// bit copy.
#include "pic_kernels.h"

#include <climits>
#include <cmath>

namespace pic {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct DF {
  float hi, lo;
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Error-free double-float rotation of one pair.
__device__ __forceinline__ void rotate_pair(float x, float y, Phase ph, DF& xo, DF& yo) {
#pragma clang fp contract(off)
  // x' = x cos - y sin
  float p1 = x * ph.x;
  float e1 = __builtin_fmaf(x, ph.x, -p1);
  float p2 = y * ph.z;
  float e2 = __builtin_fmaf(y, ph.z, -p2);
  float a = p1 - p2;
  float av = a - p1;
  float ea = (p1 - (a - av)) + (-p2 - av);
  float t = ((e1 - e2) + ea) + (x * ph.y - y * ph.w);
  float h = a + t;
  float hv = h - a;
  xo.hi = h;
  xo.lo = (a - (h - hv)) + (t - hv);
  // y' = x sin + y cos
  float q1 = x * ph.z;
  float f1 = __builtin_fmaf(x, ph.z, -q1);
  float q2 = y * ph.x;
  float f2 = __builtin_fmaf(y, ph.x, -q2);
  float b = q1 + q2;
  float bv = b - q1;
  float eb = (q1 - (b - bv)) + (q2 - bv);
  float u = ((f1 + f2) + eb) + (x * ph.w + y * ph.y);
  float g = b + u;
  float gv = g - b;
  yo.hi = g;
  yo.lo = (b - (g - gv)) + (u - gv);
}

// Round a double-float value to bf16 bits, ties to even; an exact tie in the
// head is broken by the sign of the remainder.
__device__ __forceinline__ unsigned round_bf16(DF v) {
  unsigned u = __float_as_uint(v.hi);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  if ((u & 0xffffu) == 0x8000u && v.lo != 0.0f) {
    bool away = (v.lo > 0.0f) == ((u >> 31) == 0u);
    return (u >> 16) + (away ? 1u : 0u);
  }
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Rotate the 16-byte vectors a (elements k) and b (elements k + d/2).
template <bool BF16>
__device__ __forceinline__ void rotate_vec(u32x4& a, u32x4& b, const Phase* ph);

template <>
__device__ __forceinline__ void rotate_vec<true>(u32x4& a, u32x4& b, const Phase* ph) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    DF x0, y0, x1, y1;
    rotate_pair(bf16_lo(a[w]), bf16_lo(b[w]), ph[2 * w], x0, y0);
    rotate_pair(bf16_hi(a[w]), bf16_hi(b[w]), ph[2 * w + 1], x1, y1);
    a[w] = round_bf16(x0) | (round_bf16(x1) << 16);
    b[w] = round_bf16(y0) | (round_bf16(y1) << 16);
  }
}

template <>
__device__ __forceinline__ void rotate_vec<false>(u32x4& a, u32x4& b, const Phase* ph) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    DF x, y;
    rotate_pair(__uint_as_float(a[w]), __uint_as_float(b[w]), ph[w], x, y);
    a[w] = __float_as_uint(x.hi);
    b[w] = __float_as_uint(y.hi);
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Last span whose first compact row is <= u (spans are never empty).
__device__ __forceinline__ int find_span(const int32_t* crow, int n_spans, int64_t u) {
  int lo = 0, hi = n_spans;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (crow[mid] <= u)
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

// ---------------------------------------------------------------------------
// plan: positions, pool sources, phases
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void plan_rows_kernel(PlanArgs a) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < a.prefix_rows) {
    int sp = find_span(a.crow, a.n_spans, i);
    SpanRec s = a.spans[sp];
    int t = int(i - s.crow);
    int tok = s.s + t;
    int page = a.page_ids[s.page_off + (tok >> a.page_shift)];
    int slot = (page << a.page_shift) | (tok & ((1 << a.page_shift) - 1));
    int row = s.dst_row + t;
    a.pos[row] = s.target + t;
    a.rowsrc[row] = make_int2(slot, s.delta != 0 ? sp : -1);
  } else if (i < a.prefix_rows + a.n_new) {
    int u = int(i - a.prefix_rows);
    int row = a.new_row[u];
    a.pos[row] = a.new_pos[u];
    a.rowsrc[row] = make_int2(-1, -1);
  }
}

__global__ __launch_bounds__(256) void plan_phase_kernel(PlanArgs a) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t total = int64_t(a.n_spans + a.n_new) * a.half_dim;
  if (i >= total) return;
  int which = int(i / a.half_dim);
  int k = int(i % a.half_dim);
  double p;
  Phase* dst;
  if (which < a.n_spans) {
    p = double(a.spans[which].delta);
    dst = a.phase_span + int64_t(which) * a.half_dim + k;
  } else {
    int u = which - a.n_spans;
    p = double(a.new_pos[u]);
    dst = a.phase_new + int64_t(u) * a.half_dim + k;
  }
  double ang = p * a.omega[k];
  double c = cos(ang), s = sin(ang);
  float ch = float(c), sh = float(s);
  *dst = make_float4(ch, float(c - double(ch)), sh, float(s - double(sh)));
}

// ---------------------------------------------------------------------------
// gather + re-rotate
// ---------------------------------------------------------------------------

// Each row (one token of one layer / kv head plane) is handled by LPR lanes;
// lane j owns the 16-byte vector j of the first half of the row and vector j
// of the second half, so the half-split rotation pairs stay in one lane.  A
// block covers 256 / LPR rows of the span table and `planes_per_block`
// (layer, kv head) planes, reusing each row's source lookup and phases.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int LPR = D / (2 * EPV);
  constexpr int RPB = 256 / LPR;
  constexpr int64_t RB = int64_t(D) * ES;
  const int rl = threadIdx.x / LPR;
  const int j = threadIdx.x % LPR;
  const int64_t u = int64_t(blockIdx.x) * RPB + rl;
  if (u >= a.prefix_rows) return;
  const int sp = find_span(a.crow, a.n_spans, u);
  const SpanRec s = a.spans[sp];
  const int t = int(u - s.crow);
  const int tok = s.s + t;
  const int page = a.page_ids[s.page_off + (tok >> a.page_shift)];
  const int slot = tok & (a.page_tokens - 1);
  const char* src_row = a.pool + int64_t(page) * a.page_bytes + int64_t(slot) * RB;
  const int64_t dst_row = int64_t(s.dst_row) + t;
  const bool rot = s.delta != 0;
  Phase ph[EPV];
  if (rot) {
    const Phase* pp = a.phase_span + int64_t(sp) * (D / 2) + j * EPV;
#pragma unroll
    for (int e = 0; e < EPV; ++e) ph[e] = pp[e];
  }
  const int n_planes = a.layers * a.kv_heads;
  const int p0 = blockIdx.y * a.planes_per_block;
  const int p1 = min(p0 + a.planes_per_block, n_planes);
  const int64_t plane_stride = int64_t(a.page_tokens) * RB;  // one (layer, K/V, head) run
  for (int pl = p0; pl < p1; ++pl) {
    const int l = pl / a.kv_heads;
    const int h = pl - l * a.kv_heads;
    const char* ks = src_row + (int64_t(l) * 2 * a.kv_heads + h) * plane_stride;
    const char* vs = ks + int64_t(a.kv_heads) * plane_stride;
    u32x4 k0 = ld16(ks + j * 16);
    u32x4 k1 = ld16(ks + RB / 2 + j * 16);
    u32x4 v0 = ld16(vs + j * 16);
    u32x4 v1 = ld16(vs + RB / 2 + j * 16);
    const int64_t off = (int64_t(pl) * a.cap + dst_row) * RB;
    if (rot) rotate_vec<BF16>(k0, k1, ph);
    st16(a.asm_k + off + j * 16, k0);
    st16(a.asm_k + off + RB / 2 + j * 16, k1);
    st16(a.asm_v + off + j * 16, v0);
    st16(a.asm_v + off + RB / 2 + j * 16, v1);
  }
}

// ---------------------------------------------------------------------------
// new-token prologue
// ---------------------------------------------------------------------------

// Row units: for each new token u, Hq query rows, Hkv key rows, Hkv value rows.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int LPR = D / (2 * EPV);
  constexpr int RPB = 256 / LPR;
  constexpr int64_t RB = int64_t(D) * ES;
  const int per_tok = a.q_heads + 2 * a.kv_heads;
  const int64_t unit = int64_t(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int j = threadIdx.x % LPR;
  if (unit >= int64_t(a.n_new) * per_tok) return;
  const int u = int(unit / per_tok);
  const int w = int(unit - int64_t(u) * per_tok);
  const char* src;
  char* dst;
  bool rot;
  if (w < a.q_heads) {
    src = a.q + (int64_t(u) * a.q_heads + w) * RB;
    dst = a.q_rot + (int64_t(u) * a.q_heads + w) * RB;
    rot = true;
  } else if (w < a.q_heads + a.kv_heads) {
    int h = w - a.q_heads;
    src = a.k_new + (int64_t(u) * a.kv_heads + h) * RB;
    dst = a.asm_k + (int64_t(h) * a.cap + a.new_row[u]) * RB;
    rot = true;
  } else {
    int h = w - a.q_heads - a.kv_heads;
    src = a.v_new + (int64_t(u) * a.kv_heads + h) * RB;
    dst = a.asm_v + (int64_t(h) * a.cap + a.new_row[u]) * RB;
    rot = false;
  }
  rot = rot && a.new_pos[u] != 0;
  u32x4 x0 = ld16(src + j * 16);
  u32x4 x1 = ld16(src + RB / 2 + j * 16);
  if (rot) {
    Phase ph[EPV];
    const Phase* pp = a.phase_new + int64_t(u) * (D / 2) + j * EPV;
#pragma unroll
    for (int e = 0; e < EPV; ++e) ph[e] = pp[e];
    rotate_vec<BF16>(x0, x1, ph);
  }
  st16(dst + j * 16, x0);
  st16(dst + RB / 2 + j * 16, x1);
}

// ---------------------------------------------------------------------------
// bf16 query-prefill attention, head_dim 128
// ---------------------------------------------------------------------------
//
// One workgroup = 4 waves = 128 query columns of one (request, kv head) and a
// range of 64-row tiles.  Column c of a request is token c / G, query head
// c % G of the group, so the G heads that share a kv head share every K/V
// tile.  Per wave, with its 32 columns as the MFMA N dimension:
//   S^T = K Q^T   (A = K rows from LDS, B = the wave's rotated queries held in
//                  registers), 2 x 8 MFMA 32x32x16 per tile;
//   O^T += V^T P^T (A = V^T from LDS, B = the wave's own probabilities: the
//                  S^T accumulator layout puts each column's 16 row values of
//                  a 32-row block in one lane, which is the B layout needed
//                  here once the row order inside a k-step is permuted the
//                  same way for A), 4 x 2 x 2 MFMA per tile.
// Each lane therefore owns one query column: the softmax statistics are
// lane-local plus one exchange with the lane 32 away.
//
// LDS per stage: K tile [64 rows][128] with 16-byte granules XOR-swizzled by
// row (conflict-free row-strided reads), V^T tile [128][64 rows] in 8-byte
// granules of 4 rows rotated by (d + d/16) mod 16 (conflict-free transposed
// writes and reads), 64 row positions and the tile's min/max position.
// Two stages: the next tile is fetched into registers while the current one
// is consumed.

constexpr int kStageBytes = 33280;  // 16384 K + 16384 V^T + 272 pos, padded
constexpr int kPosOff = 32768;

__device__ __forceinline__ int vt_offset(int d, int gran) {
  return d * 128 + 8 * ((gran + ((d + (d >> 4)) & 15)) & 15);
}

template <bool FUSED>
struct TileRegs {
  u32x4 k[2][2];   // [unit][half]
  u32x4 v[4];      // rows 4*kv4 + 0..3, granule c
  int pos;
};

template <bool FUSED>
__device__ __forceinline__ void load_tile(const AttnArgs& a, int row_base, int prefix_rows,
                                          int rows, int head, int tile, TileRegs<FUSED>& r) {
  const int tid = threadIdx.x;
  const int t0 = tile * kAttnRowsPerTile;
  // keys: units (row, j) with j = tid & 7 and rows (tid >> 3) + 32 i
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = t0 + (tid >> 3) + 32 * i;
    const int j = tid & 7;
    if (rr < rows) {
      if (FUSED && rr < prefix_rows) {
        const int2 src = a.rowsrc[row_base + rr];
        const char* p = a.pool + int64_t(src.x >> a.page_shift) * a.page_bytes + a.kv_plane_off +
                        (int64_t(head) * a.page_tokens + (src.x & (a.page_tokens - 1))) * 256;
        r.k[i][0] = ld16(p + j * 16);
        r.k[i][1] = ld16(p + 128 + j * 16);
        if (src.y >= 0) {
          Phase ph[8];
          const Phase* pp = a.phase_span + int64_t(src.y) * 64 + j * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) ph[e] = pp[e];
          rotate_vec<true>(r.k[i][0], r.k[i][1], ph);
        }
      } else {
        const uint16_t* p = a.k_plane + (int64_t(head) * a.cap + row_base + rr) * 128;
        r.k[i][0] = ld16(p + j * 8);
        r.k[i][1] = ld16(p + 64 + j * 8);
      }
    } else {
      r.k[i][0] = u32x4{0, 0, 0, 0};
      r.k[i][1] = u32x4{0, 0, 0, 0};
    }
  }
  // values: rows 4 * (tid >> 4) + 0..3, granule tid & 15
  const int c = tid & 15;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int rr = t0 + 4 * (tid >> 4) + q;
    if (rr < rows) {
      if (FUSED && rr < prefix_rows) {
        const int2 src = a.rowsrc[row_base + rr];
        const char* p = a.pool + int64_t(src.x >> a.page_shift) * a.page_bytes + a.kv_plane_off +
                        a.v_off + (int64_t(head) * a.page_tokens + (src.x & (a.page_tokens - 1))) * 256;
        r.v[q] = ld16(p + c * 16);
      } else {
        r.v[q] = ld16(a.v_plane + (int64_t(head) * a.cap + row_base + rr) * 128 + c * 8);
      }
    } else {
      r.v[q] = u32x4{0, 0, 0, 0};
    }
  }
  if (tid < 64) {
    const int rr = t0 + tid;
    r.pos = rr < rows ? a.pos[row_base + rr] : INT_MAX;
  }
}

template <bool FUSED>
__device__ __forceinline__ void store_tile(char* st, const TileRegs<FUSED>& r) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (tid >> 3) + 32 * i;
    const int j = tid & 7;
    st16(st + row * 256 + 16 * (j ^ (row & 15)), r.k[i][0]);
    st16(st + row * 256 + 16 * ((j + 8) ^ (row & 15)), r.k[i][1]);
  }
  // transpose 4 rows x 8 d into 8 granules of 4 rows (one per d)
  const int kv4 = tid >> 4;
  const int c = tid & 15;
  char* vt = st + 16384;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const unsigned a0 = r.v[0][w], a1 = r.v[1][w], a2 = r.v[2][w], a3 = r.v[3][w];
    const int d0 = 8 * c + 2 * w;
    u32x2 lo, hi;
    lo[0] = (a0 & 0xffffu) | (a1 << 16);
    lo[1] = (a2 & 0xffffu) | (a3 << 16);
    hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
    hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
    *reinterpret_cast<u32x2*>(vt + vt_offset(d0, kv4)) = lo;
    *reinterpret_cast<u32x2*>(vt + vt_offset(d0 + 1, kv4)) = hi;
  }
  if (tid < 64) {
    int* ps = reinterpret_cast<int*>(st + kPosOff);
    ps[tid] = r.pos;
    int mn = r.pos, mx = r.pos;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      mn = min(mn, __shfl_xor(mn, o));
      mx = max(mx, __shfl_xor(mx, o));
    }
    if (tid == 0) {
      ps[64] = mn;
      ps[65] = mx;
    }
  }
}

template <bool FUSED>
__global__ __launch_bounds__(256, 2) void attention_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const AttnWork w = a.work[bid];
  const ReqRec rq = a.reqs[w.req];
  const int rows = rq.prefix_rows + rq.n_new;
  const int ncols = rq.n_new * a.group;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g2 = lane >> 5;
  const int lq = lane & 31;
  const int col = w.col_begin + wave * 32 + lq;
  const bool col_ok = col < ncols;
  const int colc = col_ok ? col : ncols - 1;
  const int tokj = colc / a.group;
  const int hq = w.head * a.group + (colc - tokj * a.group);
  const int u = rq.new_begin + tokj;
  const int qpos = a.new_pos[u];

  // the wave's query range decides per tile whether to skip or mask
  int wq_min = col_ok ? qpos : INT_MAX;
  int wq_max = col_ok ? qpos : INT_MIN;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    wq_min = min(wq_min, __shfl_xor(wq_min, o));
    wq_max = max(wq_max, __shfl_xor(wq_max, o));
  }

  bf16x8 qb[8];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q_rot + (int64_t(u) * a.q_heads + hq) * 128);
#pragma unroll
    for (int s = 0; s < 8; ++s) qb[s] = __builtin_bit_cast(bf16x8, qp[2 * s + g2]);
  }

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.0f;

  const int tb = w.tile_begin, te = w.tile_end;
  if (tb < te) {
    TileRegs<FUSED> regs;
    load_tile<FUSED>(a, rq.row_base, rq.prefix_rows, rows, w.head, tb, regs);
    store_tile<FUSED>(smem, regs);
    __syncthreads();
    for (int t = tb; t < te; ++t) {
      const int stage = (t - tb) & 1;
      if (t + 1 < te) load_tile<FUSED>(a, rq.row_base, rq.prefix_rows, rows, w.head, t + 1, regs);
      const char* st = smem + stage * kStageBytes;
      const int* ps = reinterpret_cast<const int*>(st + kPosOff);
      const int tmin = ps[64], tmax = ps[65];
      if (tmin <= wq_max) {
        // S^T = K Q^T
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sacc[kb] = f32x16{};
          const int row = 32 * kb + lq;
          const char* kr = st + row * 256;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const bf16x8 kf = __builtin_bit_cast(bf16x8, ld16(kr + 16 * ((2 * s + g2) ^ (row & 15))));
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qb[s], sacc[kb], 0, 0, 0);
          }
        }
        if (tmax > wq_min) {
          // rows of this tile may be later than some query: mask pos_row > pos_q
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const i32x4 p4 = *reinterpret_cast<const i32x4*>(ps + 32 * kb + 8 * qq + 4 * g2);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (p4[e] > qpos) sacc[kb][4 * qq + e] = -INFINITY;
            }
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m, mx * a.scale_log2);
        const float mb = mnew == -INFINITY ? 0.0f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m - mb);
        float rs = 0.0f;
        bf16x8 pb[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], a.scale_log2, -mb));
            rs += p;
            pb[kb][i >> 3][i & 7] = (__bf16)p;
          }
        }
        l = l * alpha + rs;
        m = mnew;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
        // O^T += V^T P^T
        const char* vt = st + 16384;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = 32 * db + lq;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const int ga = 8 * kb + 4 * s2 + g2;
              const u32x2 x0 = *reinterpret_cast<const u32x2*>(vt + vt_offset(d, ga));
              const u32x2 x1 = *reinterpret_cast<const u32x2*>(vt + vt_offset(d, ga + 2));
              const u32x4 xv = {x0[0], x0[1], x1[0], x1[1]};
              o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xv),
                                                              pb[kb][s2], o[db], 0, 0, 0);
            }
          }
        }
      }
      if (t + 1 < te) store_tile<FUSED>(smem + (stage ^ 1) * kStageBytes, regs);
      __syncthreads();
    }
  }

  const float lt = l + __shfl_xor(l, 32);
  if (!col_ok) return;
  if (a.n_split == 1) {
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    uint16_t* op = a.out + (int64_t(u) * a.q_heads + hq) * 128;
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
  } else {
    const int64_t idx = (int64_t(w.split) * a.n_new + u) * a.q_heads + hq;
    float* op = a.opart + idx * 128;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d0 = 32 * db + 8 * qq + 4 * g2;
        const f32x4 v = {o[db][4 * qq], o[db][4 * qq + 1], o[db][4 * qq + 2], o[db][4 * qq + 3]};
        *reinterpret_cast<f32x4*>(op + d0) = v;
      }
    }
    if (g2 == 0) a.ml[idx] = make_float2(m, lt);
  }
}

// Log-sum-exp merge of the row splits: one wave per (new token, query head).
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  const int64_t item = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= int64_t(a.n_new) * a.q_heads) return;
  float mmax = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) {
    const float2 v = a.ml[int64_t(s) * a.n_new * a.q_heads + item];
    if (v.y > 0.0f) mmax = fmaxf(mmax, v.x);
  }
  float den = 0.0f, n0 = 0.0f, n1 = 0.0f;
  for (int s = 0; s < a.n_split; ++s) {
    const int64_t idx = int64_t(s) * a.n_new * a.q_heads + item;
    const float2 v = a.ml[idx];
    if (!(v.y > 0.0f)) continue;
    const float wgt = __builtin_amdgcn_exp2f(v.x - mmax);
    den += wgt * v.y;
    const float* op = a.opart + idx * 128;
    n0 += wgt * op[2 * lane];
    n1 += wgt * op[2 * lane + 1];
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const __bf16 b0 = (__bf16)(n0 * inv), b1 = (__bf16)(n1 * inv);
  reinterpret_cast<unsigned*>(a.out + item * 128)[lane] =
      unsigned(__builtin_bit_cast(uint16_t, b0)) | (unsigned(__builtin_bit_cast(uint16_t, b1)) << 16);
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

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const int64_t n1 = a.prefix_rows + a.n_new;
  if (n1 > 0) {
    hipLaunchKernelGGL(plan_rows_kernel, dim3(unsigned((n1 + 255) / 256)), dim3(256), 0, s, a);
  }
  const int64_t n2 = int64_t(a.n_spans + a.n_new) * a.half_dim;
  if (n2 > 0) {
    hipLaunchKernelGGL(plan_phase_kernel, dim3(unsigned((n2 + 255) / 256)), dim3(256), 0, s, a);
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
  const int n_planes = a.layers * a.kv_heads;
  dim3 grid(unsigned((a.prefix_rows + RPB - 1) / RPB),
            unsigned((n_planes + a.planes_per_block - 1) / a.planes_per_block));
  hipLaunchKernelGGL((gather_kernel<BF16, D>), grid, dim3(256), 0, s, a);
}

hipError_t launch_gather(int dtype, int head_dim, const GatherArgs& a, hipStream_t s) {
  if (a.prefix_rows <= 0) return hipSuccess;
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
  constexpr int RPB = 256 / LPR;
  const int64_t units = int64_t(a.n_new) * (a.q_heads + 2 * a.kv_heads);
  hipLaunchKernelGGL((prologue_kernel<BF16, D>), dim3(unsigned((units + RPB - 1) / RPB)), dim3(256), 0,
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
  if (fused)
    hipLaunchKernelGGL(attention_bf16_kernel<true>, dim3(unsigned(a.n_work)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attention_bf16_kernel<false>, dim3(unsigned(a.n_work)), dim3(256), 0, s, a);
  if (a.n_split > 1) {
    const int64_t items = int64_t(a.n_new) * a.q_heads;
    hipLaunchKernelGGL(merge_kernel, dim3(unsigned((items + 3) / 4)), dim3(256), 0, s, a);
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
