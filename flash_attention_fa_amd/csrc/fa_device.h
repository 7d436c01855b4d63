// fa_device.h - gfx950 building blocks shared by the attention kernels.
//
// MFMA lane maps (checked on hardware by tests/test_lane_maps.py):
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l%32][8*(l/32) + e], e = 0..7
//     B: lane l holds B[8*(l/32) + e][l%32]
//     C: lane l, register i holds C[8*(i/4) + 4*(l/32) + i%4][l%32]
//   ds_read_b64_tr_b16: in each group of 16 lanes, lane r supplies the address
//     of 4 consecutive 16-bit values (row r of a 16x4 block M); lane i then
//     receives M[4e + i/4][i%4] for e = 0..3.  With lane r pointing at
//     X[k0 + r/4][n0 + 4*(r%4)] of a row-major [k][n] tile, lane i receives the
//     column X[k0 .. k0+3][n0 + i]: a transposed operand read straight from a
//     row-major tile.
//   v_permlane32_swap(x, x): max/sum of the two results reduces x across the
//     two 32-lane halves of the wave.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define FA_LDS(T, p) ((T __attribute__((address_space(3)))*)(p))

enum { MASK_FULL = 0, MASK_CAUSAL = 1, MASK_TTT = 2 };
enum { TILE_SKIP = 0, TILE_FULL = 1, TILE_PART = 2 };

constexpr float kLn2 = 0.6931471805599453f;
// Running max starts here instead of -inf so exp2(x - m) never sees
// (-inf) - (-inf); any finite score exceeds it and triggers a rescale.
constexpr float kMaxInit = -1.0e30f;
// Rescale the accumulators only when a row max grows by more than this many
// powers of two; the stale max keeps every exp2 argument <= kRescaleSlack, so
// P stays <= 2^8 and the final O / l, LSE are unchanged.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 lds_read8(const bf16* p) {
  return *FA_LDS(const bf16x8, p);
}
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(i16x4, p));
  return __builtin_bit_cast(bf16x4, t);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void lds_write16(bf16* p, i32x4 v) { *FA_LDS(i32x4, p) = v; }

// Four fp32 accumulator values -> 4 bf16 (round to nearest even).
__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (bf16)a; r[1] = (bf16)b; r[2] = (bf16)c; r[3] = (bf16)d;
  return r;
}

// --------------------------------------------------------------------------
// Mask: the resolved descriptor for one batch entry.

struct MaskB {
  int kind, shift, Sq, Skv, L, kvv;  // L = Sq (TTT step length); kvv clamped
};

__device__ __forceinline__ MaskB resolve_mask(const Params& p, int b) {
  MaskB m;
  m.kind = p.mask.kind;
  m.shift = p.mask.shift;
  m.Sq = p.Sq;
  m.Skv = p.Skv;
  m.L = p.Sq;
  const int cap = p.mask.kind == MASK_TTT ? p.Sq : p.Skv;
  int v = p.mask.kv_valid ? p.mask.kv_valid[b] : cap;
  m.kvv = v < 0 ? 0 : (v > cap ? cap : v);
  return m;
}

// May query i attend key j?  (The three mask kinds of fa.h.)
__device__ __forceinline__ bool allowed(const MaskB& m, int i, int j) {
  if (m.kind == MASK_FULL) return j < m.kvv;
  const bool causal = (j <= i - m.shift) && (j < m.kvv);
  if (m.kind == MASK_CAUSAL || causal) return causal;
  // TTT suffix: key of a later step at the query's own position.
  if (j < m.L) return false;
  const int jm = j % m.L;
  return jm == i && jm < m.kvv;
}

// Is key j a real key (its K/V row may be used at all)?
__device__ __forceinline__ bool key_valid(const MaskB& m, int j) {
  if (j >= m.Skv) return false;
  if (m.kind == MASK_TTT) return (j % m.L) < m.kvv;
  return j < m.kvv;
}

__device__ __forceinline__ int num_segments(const MaskB& m) {
  return m.kind == MASK_TTT ? (m.L > 0 ? m.Skv / m.L : 0) : 1;
}

// Key tiles [t0, t1) of segment s that queries [qa, qb) may touch.  Segment 0
// is the causal (or full) range; TTT segment s >= 1 is the diagonal band of
// step s.  Ranges are increasing in s; callers clip each start to the previous
// end so no tile is visited twice.
__device__ __forceinline__ void segment_tiles(const MaskB& m, int s, int qa, int qb, int TK,
                                              int& t0, int& t1) {
  int lo, hi;
  if (s == 0) {
    lo = 0;
    hi = m.kind == MASK_FULL ? m.kvv : min(m.kvv, qb - m.shift);
  } else {
    lo = s * m.L + qa;
    hi = s * m.L + min(qb, m.kvv);
  }
  if (hi <= lo) { t0 = t1 = 0; return; }
  t0 = lo / TK;
  t1 = (hi + TK - 1) / TK;
}

// Keys [k0, k1) against queries [qa, qb): skip, no predicate needed, or
// predicate needed per element.
__device__ __forceinline__ int rect_state(const MaskB& m, int k0, int k1, int qa, int qb) {
  if (qb <= qa || k1 <= k0) return TILE_SKIP;
  if (m.kind == MASK_FULL) return k1 <= m.kvv ? TILE_FULL : (k0 < m.kvv ? TILE_PART : TILE_SKIP);
  const bool c_any = (k0 <= qb - 1 - m.shift) && (k0 < m.kvv);
  const bool c_all = (k1 - 1 <= qa - m.shift) && (k1 <= m.kvv);
  if (m.kind == MASK_CAUSAL) return c_all ? TILE_FULL : (c_any ? TILE_PART : TILE_SKIP);
  if (c_all && k1 <= m.L) return TILE_FULL;
  if (c_any) return TILE_PART;
  const int qbv = min(qb, m.kvv);
  if (qbv <= qa || m.L <= 0) return TILE_SKIP;
  const int nseg = m.Skv / m.L;
  int s = max(1, k0 / m.L);
  for (; s < nseg && s * m.L < k1 + m.L; ++s) {
    const int lo = s * m.L + qa, hi = s * m.L + qbv;
    if (lo < k1 && k0 < hi) return TILE_PART;
  }
  return TILE_SKIP;
}

__device__ __forceinline__ int tile_state(const MaskB& m, int k0, int TK, int qa, int qb) {
  return rect_state(m, k0, k0 + TK, qa, qb);
}

// Queries [lo, hi) that may attend some key in [k0, k1) (a hull; the caller
// still classifies each query tile).
__device__ __forceinline__ void query_hull(const MaskB& m, int k0, int k1, int& lo, int& hi) {
  lo = m.Sq; hi = 0;
  if (m.kind == MASK_FULL) {
    if (k0 < m.kvv) { lo = 0; hi = m.Sq; }
    return;
  }
  if (k0 < m.kvv) { lo = min(m.Sq, max(0, k0 + m.shift)); hi = m.Sq; }
  if (m.kind != MASK_TTT || m.L <= 0) return;
  const int nseg = m.Skv / m.L;
  for (int s = max(1, k0 / m.L); s < nseg && s * m.L < k1; ++s) {
    const int a = max(k0, s * m.L) - s * m.L, b = min(min(k1, (s + 1) * m.L) - s * m.L, m.kvv);
    if (a < b) { lo = min(lo, a); hi = max(hi, b); }
  }
}

// Walks the tiles of all segments in increasing order, each tile once.
struct TileWalk {
  int seg, nseg, t, t1, prev_end;
  __device__ __forceinline__ void start(const MaskB& m, int qa, int qb, int TK) {
    nseg = num_segments(m);
    seg = -1; t = 0; t1 = 0; prev_end = 0;
    advance(m, qa, qb, TK);
  }
  // Move to the next segment with tiles left.
  __device__ __forceinline__ void advance(const MaskB& m, int qa, int qb, int TK) {
    while (t >= t1 && ++seg < nseg) {
      int a, b;
      segment_tiles(m, seg, qa, qb, TK, a, b);
      a = max(a, prev_end);
      if (a < b) { t = a; t1 = b; prev_end = b; }
    }
  }
  __device__ __forceinline__ bool valid() const { return t < t1; }
  __device__ __forceinline__ void next(const MaskB& m, int qa, int qb, int TK) {
    ++t;
    if (t >= t1) advance(m, qa, qb, TK);
  }
};

// --------------------------------------------------------------------------
// Block -> (column, rank).  Workgroup i runs on XCD i % 8; when the number of
// (batch, head) columns is a multiple of 8, each XCD gets a contiguous run of
// columns (neighbouring heads share a K/V head, so its L2 serves them all) and
// walks its ranks in order, rank 0 first.
__device__ __forceinline__ void map_block(int bid, int ncol, int nrank, int& col, int& rank) {
  if ((ncol & 7) == 0) {
    const int x = bid & 7, slot = bid >> 3, c8 = ncol >> 3;
    rank = slot / c8;
    col = x * c8 + slot % c8;
  } else {
    rank = bid / ncol;
    col = bid % ncol;
  }
}

}  // namespace fa
