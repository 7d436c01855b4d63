// fa_device.h - gfx950 building blocks shared by the attention kernels.
//
// MFMA lane maps (measured on gfx950; every parity test depends on them):
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

enum { MASK_FULL = 0, MASK_CAUSAL = 1, MASK_TTT = 2, MASK_WINDOW = 3 };
enum { TILE_SKIP = 0, TILE_FULL = 1, TILE_PART = 2 };

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;
// Running max starts here instead of -inf so exp2(x - m) never sees
// (-inf) - (-inf); any finite score exceeds it and triggers a rescale.
constexpr float kMaxInit = -1.0e30f;

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

// c + the dot product of two bf16x8 (four two-way dot products, fp32).
__device__ __forceinline__ float dot_bf16x8(bf16x8 x, bf16x8 y, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), __builtin_shufflevector(y, y, 0, 1), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), __builtin_shufflevector(y, y, 2, 3), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), __builtin_shufflevector(y, y, 4, 5), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), __builtin_shufflevector(y, y, 6, 7), c, false);
  return c;
}

// c + the sum of the eight bf16 values of x (four two-way dot products with
// ones, accumulated in fp32).
__device__ __forceinline__ float sum_bf16x8(bf16x8 x, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, c, false);
  return c;
}

__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(i16x4, p));
  return __builtin_bit_cast(bf16x4, t);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Four fp32 accumulator values -> 4 bf16 (round to nearest even).
__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (bf16)a; r[1] = (bf16)b; r[2] = (bf16)c; r[3] = (bf16)d;
  return r;
}

// --------------------------------------------------------------------------
// Asynchronous tile staging (HBM -> LDS without registers).  A 64-row tile of
// a row-major [rows][D] bf16 matrix is stored unpadded; inside each row the
// 16-byte chunk c lives at slot c ^ swz(row), which keeps both the row reads
// (16 rows x one chunk) and the transposing reads (4 rows x 64 bytes) free of
// bank conflicts.  One load instruction moves 64 chunks (1 KB, contiguous in
// LDS): each lane fetches the global chunk that belongs in its slot.

template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else if constexpr (D == 32) return (r >> 2) & 3;
  else return (r >> 3) & 1;
}

// Byte offset of element e (multiple of 4) of row r inside a swizzled tile.
template <int D>
__device__ __forceinline__ int swz_off(int r, int e) {
  return r * (2 * D) + 16 * ((e >> 3) ^ swz<D>(r)) + 2 * (e & 7);
}

// One asynchronous 1 KB copy: lane l's 16 bytes at g land at lds_base + 16 l.
// Issued through inline assembly so the compiler does not treat every later
// LDS read as possibly aliasing the copy (it would drain all outstanding
// copies before each read); completion is awaited explicitly with
// wait_vmcnt() and ordered across waves by barrier_lds().  M0 carries the LDS
// address; one wait state separates its write from the copy.
__device__ __forceinline__ void lds_dma16(const void* g, unsigned char* lds_base) {
  const unsigned lds_addr = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}

// The LDS byte address of a shared-memory pointer (uniform when p is).
__device__ __forceinline__ unsigned lds_addr_of(const unsigned char* p) {
  return __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p);
}

// lds_dma16 with the LDS byte address given directly (a uniform value).
__device__ __forceinline__ void lds_dma16_at(const void* g, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}

// lds_dma16_at with a wave-uniform 64-bit base address (held in scalar
// registers) and a per-lane 32-bit byte offset: lane l's 16 bytes at
// sbase + voff land at lds_addr + 16 l.  The address arithmetic of a tile's
// copies then costs no vector instructions: the offsets are computed once and
// only the scalar base moves from tile to tile.
// A wave-uniform pointer moved to scalar registers (both 32-bit halves read
// from the first active lane).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(lo | (hi << 32));
}

__device__ __forceinline__ void lds_dma16_s(const void* sbase, unsigned voff, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(uniform_ptr(sbase)), "s"(lds_addr)
               : "memory", "m0");
}

// s_waitcnt with only the vector-memory counter constrained (<= n).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0), others free
}
// Workgroup barrier that does not wait for outstanding HBM loads (the caller
// has waited for the ones it needs); a compiler fence keeps LDS accesses on
// their side of it.
__device__ __forceinline__ void barrier_lds() {
  wait_lgkm0();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// --------------------------------------------------------------------------
// Mask: the resolved descriptor for one batch entry.

struct MaskB {
  int kind, shift, Sq, Skv, L, kvv;  // L = Sq (TTT step length); kvv clamped
  int wl, wr;                        // WINDOW band: keys before / after the diagonal
};

// Shift and window are clamped to +-2 (Sq + Skv): past that the predicate no
// longer changes (a larger shift already leaves every row empty, a more
// negative one already shows every row every key, a wider window already
// covers every key), and the band arithmetic stays far from int overflow.
// `kv` is the batch entry's valid key count (any int; clamped here).
__host__ __device__ __forceinline__ MaskB make_mask(int kind, int shift, int Sq, int Skv, int kv, int wl, int wr) {
  MaskB m;
  const int lim = 2 * (Sq + Skv);
  m.kind = kind;
  m.shift = shift < lim ? (shift > -lim ? shift : -lim) : lim;
  m.Sq = Sq;
  m.Skv = Skv;
  m.L = Sq;
  m.wl = wl < lim ? wl : lim;
  m.wr = wr < lim ? wr : lim;
  const int cap = kind == MASK_TTT ? Sq : Skv;
  m.kvv = kv < 0 ? 0 : (kv > cap ? cap : kv);
  return m;
}

__device__ __forceinline__ MaskB resolve_mask(const Params& p, int b) {
  return make_mask(p.mask.kind, p.mask.shift, p.Sq, p.Skv, p.mask.kv_valid ? p.mask.kv_valid[b] : p.Skv,
                   p.mask.wl, p.mask.wr);
}

// May query i attend key j?  (The three mask kinds of fa.h.)  Written
// without per-lane branches (the mask kind is uniform), so callers can use it
// as a select on score registers.
__host__ __device__ __forceinline__ bool allowed(const MaskB& m, int i, int j) {
  const bool valid = j < m.kvv;
  if (m.kind == MASK_FULL) return valid;
  if (m.kind == MASK_WINDOW) {
    const int d = j - (i - m.shift);   // offset from the shifted diagonal
    return (d >= -m.wl) & (d <= m.wr) & valid;
  }
  const bool causal = (j <= i - m.shift) & valid;
  if (m.kind == MASK_CAUSAL) return causal;
  // TTT suffix: key of a later step at the query's own position (keys past
  // Skv in a ragged last tile are not keys of any step).
  const int jm = j - (j / m.L) * m.L;
  return causal | ((j >= m.L) & (j < m.Skv) & (jm == i) & (jm < m.kvv));
}

// Instruction-class masks of the scheduler's group barriers, and a group
// barrier: the next `n` instructions of class `mask` in the current
// straight-line block are placed here, in order.
enum : int { SCHED_VALU = 0x002, SCHED_SALU = 0x004, SCHED_MFMA = 0x008, SCHED_VMEM_READ = 0x020,
             SCHED_DS_READ = 0x100, SCHED_DS_WRITE = 0x200, SCHED_TRANS = 0x400 };
#define sched_group(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// The wave index as a provably uniform (scalar) value, so everything derived
// from it (tile ranges, tile states, loop bounds) stays in scalar registers.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Is key j a real key (its K/V row may be used at all)?
__host__ __device__ __forceinline__ bool key_valid(const MaskB& m, int j) {
  if (j >= m.Skv) return false;
  if (m.kind == MASK_TTT) return (j % m.L) < m.kvv;
  return j < m.kvv;
}

// key_valid without branches on the lane's key (the mask kind is uniform).
__host__ __device__ __forceinline__ bool key_valid_nb(const MaskB& m, int j) {
  const int jm = m.kind == MASK_TTT ? j - (j / m.L) * m.L : j;
  return (j < m.Skv) & (jm < m.kvv);
}

__host__ __device__ __forceinline__ int num_segments(const MaskB& m) {
  return m.kind == MASK_TTT ? (m.L > 0 ? m.Skv / m.L : 0) : 1;
}

// Key tiles [t0, t1) of segment s that queries [qa, qb) may touch.  Segment 0
// is the causal (or full) range; TTT segment s >= 1 is the diagonal band of
// step s.  Ranges are increasing in s; callers clip each start to the previous
// end so no tile is visited twice.
__host__ __device__ __forceinline__ void segment_tiles(const MaskB& m, int s, int qa, int qb, int TK,
                                              int& t0, int& t1) {
  int lo, hi;
  if (s == 0) {
    lo = m.kind == MASK_WINDOW ? max(0, qa - m.shift - m.wl) : 0;
    hi = m.kind == MASK_FULL ? m.kvv : min(m.kvv, qb - m.shift + (m.kind == MASK_WINDOW ? m.wr : 0));
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
__host__ __device__ __forceinline__ int rect_state(const MaskB& m, int k0, int k1, int qa, int qb) {
  if (qb <= qa || k1 <= k0) return TILE_SKIP;
  if (m.kind == MASK_FULL) return k1 <= m.kvv ? TILE_FULL : (k0 < m.kvv ? TILE_PART : TILE_SKIP);
  if (m.kind == MASK_WINDOW) {
    // the rows' bands [i - shift - wl, i - shift + wr] move by one key per
    // row, so together they cover [qa - shift - wl, qb - 1 - shift + wr]
    const bool w_any = (k0 <= qb - 1 - m.shift + m.wr) && (k1 - 1 >= qa - m.shift - m.wl) && (k0 < m.kvv);
    const bool w_all = (k0 >= qb - 1 - m.shift - m.wl) && (k1 - 1 <= qa - m.shift + m.wr) && (k1 <= m.kvv);
    return w_all ? TILE_FULL : (w_any ? TILE_PART : TILE_SKIP);
  }
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

// Number of leading TK-key tiles that every query row >= qa may attend in
// full (keys below kv_valid and, unless FULL, at most qa - shift): tiles
// [0, result) need neither classification nor a mask for rows >= qa.
__host__ __device__ __forceinline__ int full_tiles_below(const MaskB& m, int qa, int TK) {
  if (m.kind == MASK_WINDOW) return 0;   // a band has no fully visible prefix in general
  int lim = m.kvv;
  if (m.kind != MASK_FULL) lim = min(lim, qa - m.shift + 1);
  return lim > 0 ? lim / TK : 0;
}

__host__ __device__ __forceinline__ int tile_state(const MaskB& m, int k0, int TK, int qa, int qb) {
  return rect_state(m, k0, k0 + TK, qa, qb);
}

// Queries [lo, hi) that may attend some key in [k0, k1) (a hull; the caller
// still classifies each query tile).
__host__ __device__ __forceinline__ void query_hull(const MaskB& m, int k0, int k1, int& lo, int& hi) {
  lo = m.Sq; hi = 0;
  if (m.kind == MASK_FULL) {
    if (k0 < m.kvv) { lo = 0; hi = m.Sq; }
    return;
  }
  if (m.kind == MASK_WINDOW) {
    // rows i whose band meets [k0, k1): k0 + shift - wr <= i <= k1 - 1 + shift + wl
    if (k0 < m.kvv && k0 < k1) {
      lo = max(0, k0 + m.shift - m.wr);
      hi = min(m.Sq, k1 + m.shift + m.wl);
      if (hi < lo) { lo = m.Sq; hi = 0; }
    }
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
  __host__ __device__ __forceinline__ void start(const MaskB& m, int qa, int qb, int TK) {
    nseg = num_segments(m);
    seg = -1; t = 0; t1 = 0; prev_end = 0;
    advance(m, qa, qb, TK);
  }
  // Move to the next segment with tiles left.
  __host__ __device__ __forceinline__ void advance(const MaskB& m, int qa, int qb, int TK) {
    while (t >= t1 && ++seg < nseg) {
      int a, b;
      segment_tiles(m, seg, qa, qb, TK, a, b);
      a = max(a, prev_end);
      if (a < b) { t = a; t1 = b; prev_end = b; }
    }
  }
  __host__ __device__ __forceinline__ bool valid() const { return t < t1; }
  __host__ __device__ __forceinline__ void next(const MaskB& m, int qa, int qb, int TK) {
    ++t;
    if (t >= t1) advance(m, qa, qb, TK);
  }
};

// --------------------------------------------------------------------------
// Transposed key tiles.  The forward's PV product reads V^T as MFMA A
// operands whose k index runs over keys; a small pre-pass writes such a
// transposed copy, X^T[b, hk, d, keys] of a [b, hk, keys, d] tensor X, into
// the caller's workspace, in tiles of kVtTile keys.
//
// Row d of a tile is 64 keys (128 bytes, eight 16-byte chunks); in LDS chunk
// c of row d sits at slot c ^ vt_swz(d), so the 16 rows one 16-lane group of
// a 16-byte read touches cover all 64 banks.
__device__ __forceinline__ int vt_swz(int d) { return (d >> 1) & 7; }

// Stored position of key tile offset j in a transposed row: within each
// group of 16 keys, bits 2 and 3 of the offset swap places.  The B operand
// that meets these rows comes straight from transposed score registers,
// where lane half hh holds keys 4hh..4hh+3 and 8+4hh..8+4hh+3 of each 16-key
// step in its eight k slots; with this order those eight keys are one
// 16-byte run of the row.
__host__ __device__ constexpr int vt_pos(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// The pre-pass: dst[b, hk, d, tile*64 + vt_pos(j)] = src[b, hk, tile*64 + j, d]
// for real keys and 0 for every other position of the padded key range
// (past Skv, or not valid under the mask), so copies of these tiles need no
// per-row selection and masked keys meet zeros.  Under TTT only the step-0
// keys are real here (the tile loops walk those; the later steps' keys are
// taken one per row).  A block converts one (b, hk, tile) at a time,
// striding over all of them, `ntile` tiles per (b, hk); rows of dst hold
// dst_ss keys.
template <int D>
__global__ void __launch_bounds__(256) transpose_keys_kernel(Params p, Tensor src, bf16* dst, int64_t dst_ss,
                                                             int ntile, int64_t nblk) {
  constexpr int TK = kVtTile;
  constexpr int CPR = D / 8;
  __shared__ bf16 tile[TK][D + 8];
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int t = (int)(blk % ntile), bh = (int)(blk / ntile);
    const int b = bh / p.Hkv, hk = bh % p.Hkv;
    MaskB m = resolve_mask(p, b);
    if (m.kind == MASK_TTT) {
      m.kind = MASK_CAUSAL;
      m.Skv = min(m.Skv, m.L);
    }
    const bf16* Xg = static_cast<const bf16*>(src.ptr) + b * src.sb + hk * src.sh;
    __syncthreads();   // the previous tile's reads of `tile` are done
    for (int i = threadIdx.x; i < TK * CPR; i += 256) {
      const int r = i / CPR, c = i % CPR, j = t * TK + r;
      bf16x8 x = {};
      if (key_valid(m, j)) x = *reinterpret_cast<const bf16x8*>(Xg + (int64_t)j * src.ss + 8 * c);
      *reinterpret_cast<bf16x8*>(&tile[r][8 * c]) = x;
    }
    __syncthreads();
    bf16* Xt = dst + (int64_t)bh * D * dst_ss + (int64_t)t * TK;
    for (int i = threadIdx.x; i < D * (TK / 8); i += 256) {
      const int d = i / (TK / 8), c = i % (TK / 8);
      bf16x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = tile[vt_pos(8 * c + e)][d];
      *reinterpret_cast<bf16x8*>(Xt + (int64_t)d * dst_ss + 8 * c) = y;
    }
  }
}

// Mask-kind instances of the tile kernels.  Each instance fixes, visibly to
// the compiler, which arms of the mask helpers its tile loop can reach:
// MK_FC FULL or CAUSAL, MK_TTT the causal view of TTT's step-0 keys (the
// later steps' keys are taken one per row outside the loop), MK_WIN WINDOW.
enum { MK_FC = 0, MK_TTT = 1, MK_WIN = 2 };

__host__ __device__ __forceinline__ int mask_instance(int kind) {
  return kind == MASK_TTT ? MK_TTT : (kind == MASK_WINDOW ? MK_WIN : MK_FC);
}

template <int MK>
__host__ __device__ __forceinline__ void set_instance_kind(MaskB& m) {
  if constexpr (MK == MK_WIN) {
    m.kind = MASK_WINDOW;
  } else {
    m.kind = MK == MK_FC && m.kind == MASK_FULL ? MASK_FULL : MASK_CAUSAL;
    if constexpr (MK == MK_TTT) m.Skv = min(m.Skv, m.L);
  }
}

// Keys the tile loops walk: all of them, or under TTT the Sq step-0 keys.
__device__ __host__ __forceinline__ int walk_keys(const Params& p) {
  return p.mask.kind == MASK_TTT && p.Sq < p.Skv ? p.Sq : p.Skv;
}

// Launches the pre-pass for the tiles the tile loops read.
template <int D>
hipError_t launch_transpose_keys(const Params& p, const Tensor& src, void* dst, int64_t dst_ss, hipStream_t s) {
  const int ntile = (walk_keys(p) + kVtTile - 1) / kVtTile;
  const int64_t nblk = (int64_t)p.B * p.Hkv * ntile;
  if (nblk == 0) return hipSuccess;
  const unsigned grid = (unsigned)(nblk < (1 << 20) ? nblk : (1 << 20));
  hipLaunchKernelGGL(transpose_keys_kernel<D>, dim3(grid), dim3(256), 0, s, p, src, static_cast<bf16*>(dst),
                     dst_ss, ntile, nblk);
  return hipGetLastError();
}

// The key bias divided by the scale, float32 [B, vt_ss] with zeros past Skv:
// the value a score's matrix-core accumulation starts from, so the scaled
// score comes out as scale * (q.k + bias / scale) = scale q.k + bias.
template <int Unused = 0>
__global__ void __launch_bounds__(256) bias_scale_kernel(Params p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t b = i / p.vt_ss, j = i % p.vt_ss;
    p.bias_s[i] = j < p.Skv ? p.mask.bias[b * p.mask.bias_sb + j] / p.scale : 0.f;
  }
}

inline hipError_t launch_bias_scale(const Params& p, hipStream_t s) {
  if (p.mask.bias == nullptr || p.bias_s == nullptr) return hipSuccess;
  const int64_t n = (int64_t)p.B * p.vt_ss;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(bias_scale_kernel<0>, dim3((unsigned)(blocks < (1 << 16) ? blocks : (1 << 16))), dim3(256), 0,
                     s, p, n);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Block -> (column, rank).  Workgroup i runs on XCD i % 8; when the number of
// (batch, head) columns is a multiple of 8, each XCD gets a contiguous run of
// columns (neighbouring heads share a K/V head, so its L2 serves them all) and
// walks its ranks in order, rank 0 first.
__host__ __device__ __forceinline__ void map_block(int bid, int ncol, int nrank, int& col, int& rank) {
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
