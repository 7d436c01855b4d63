// fa_fwd.hip - bf16 forward attention for gfx950 (MFMA 32x32x16).
//
// What it computes: for every (batch, query head, query row i)
//   O_i = sum_j P_ij V_j,  P_ij = exp(s q_i.k_j - LSE_i) over allowed keys j,
//   LSE_i = ln sum_j exp(s q_i.k_j),
// the attention formula of "Flex Attention and Triton, Supporting Long
// Context Training in SpecForge" (section EAGLE3 Training) under that page's
// EAGLE3 mask (section Flex Attention), computed tile by tile with a running
// max and normaliser (CS336 "Flash Attention (Triton)", How it works) so only
// O and LSE ever reach HBM (ggml flash-attn-training playbook, section 1).
//
// Work split.  A workgroup owns NW*32 query rows of one (batch, head); each
// wave owns one block of 32 rows, two or more waves per SIMD.  Keys stream through
// LDS in tiles of 64.  Scores are computed transposed, S^T = K Q^T, so each
// lane owns one query column and 32 keys of it: the softmax scale, running
// max and normaliser are one scalar per lane.  O^T = V^T P^T takes P straight
// from the score registers and V^T from a transposed copy of V that a small
// pre-pass (transpose_keys_kernel) writes into the caller's workspace:
// 16-byte LDS reads serve it, where the row-major V tile would need
// transposing reads that move half as many bytes per instruction at about
// half the rate.
//
// Vector-ALU budget.  At D = 128 a wave's 32 MFMAs per tile take about as long
// as a few hundred vector instructions, so the exponentials and their
// bookkeeping are kept to two instructions plus one exp2 per score: one FMA
// (scale and running max), the exp2, half a bf16 pack and half a two-way dot
// product that sums the packed P for the normaliser (so l sums exactly the P
// the PV product uses).  No per-tile row max is taken: P is computed against
// a reference kSlack above a stale row max and saturated at 1 (the exp2's
// clamp bit, no extra instruction), so it is bounded before anything is
// checked and the PV products follow the exponentials in one stretch of code.
// Only when some row's tile sum reaches 1 (which any saturated P forces) is
// the true max taken, after the PV products, and the tile corrected (fixup).
// LDS addresses are lane constants plus immediates: the loop is unrolled over
// the four ring buffers.
//
// Pipeline.  Iteration i issues the QK^T products of tile i+1, then the
// exponentials of tile i (independent of those products, so the matrix cores
// and the vector ALUs work at once), then the PV products of tile i; the mask
// of tile i+1 (partial tiles only) closes the iteration.  K and V^T rows are
// copied HBM -> LDS asynchronously (no registers, no vector instructions)
// into a ring of four K and four V^T buffers.  Iterations go in pairs with
// one barrier per pair: the first of a pair copies what the next pair reads
// (K rows of tiles i+3, i+4, V^T rows of i+2, i+3: K runs a tile ahead of
// V^T because QK^T does), into buffers the previous pair finished with.
#include <algorithm>
#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace {

constexpr int TK = 64;    // keys per LDS tile
static_assert(TK == kVtTile, "the V^T workspace is laid out in forward key tiles");
constexpr int NBUF = 4;   // tiles in flight in LDS
// The running max is lazy: P = exp2(x - mref), x the scaled score in log2
// units, against a reference mref that moves only when a tile's P grows too
// large.  At D >= 64 (LATE) mref sits kSlack above a row max and P saturates
// at 1: every P is bounded before anything is checked, the PV products run
// first, and a row whose P could have saturated (lane's tile sum >= 1) is
// corrected afterwards (fixup); the common 2^-kSlack factor of P cancels in
// O = acc / l and returns in the LSE through mref.  At D <= 32 mref is a row
// max and a lane's tile sum above kSumLimit = 2^kSlack (which bounds every P
// in it) rescales O and l and recomputes P before the PV products (refresh):
// the late correction keeps the scores live through the PV products, which
// at these D costs a wave per SIMD.
constexpr float kSlack = 12.0f;
constexpr float kSumLimit = 4096.0f;

__device__ __forceinline__ float exp2_sat(float x) {
  return __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x), 0.0f, 1.0f);
}

// LDS: the NBUF K tiles (64 swizzled rows of D), then the NBUF V^T tiles (D
// swizzled rows of 64 keys), so every operand address of a ring buffer is a
// lane constant plus an immediate below 64 KB.
// With a key bias, NBUF 1 KB slots follow: the tile's 64 scaled bias values
// (256 bytes; the copy instruction that brings them writes 1 KB).
template <int D>
struct FwdLds {
  static constexpr int TILE_BYTES = TK * D * 2;          // one K or V^T tile
  static constexpr int VT_BASE = NBUF * TILE_BYTES;
  static constexpr int BYTES = 2 * NBUF * TILE_BYTES;
  static constexpr int BIAS_BASE = BYTES;
  static constexpr int BIAS_BYTES = NBUF * 1024;
};

template <int K>
struct Buf {
  static constexpr int value = K;
};

// MK: the mask-kind instance (MK_FC, MK_TTT, MK_WIN).  TTT's step-0 part
// (keys below L = Sq) is the causal mask with the same shift and kv_valid,
// so the MK_TTT tile loop is the causal one.  The keys of steps 1 .. n-1
// that row i sees are the single keys s*L + i (when i < kv_valid): instead
// of a 64-key tile per step that holds one key per row, each lane folds its
// row's keys into the running max, normaliser and O before the tile loop
// (ttt_fold).
// At D = 16 (4-wave workgroups, no key bias) the kernel is bounded to 128
// registers, so four waves share a SIMD; at D = 32 the same bound would
// spill many registers.
template <int D, int NW, int MK, bool BIAS>
__global__ void __launch_bounds__(NW * 64, D == 16 && NW == 4 && !BIAS ? 4 : 2)
fwd_kernel(Params p) {
  constexpr bool TTT = MK == MK_TTT;
  constexpr bool LATE = D >= 64;
  constexpr float SLACK = LATE ? kSlack : 0.0f;
  constexpr int TQ = NW * 32;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;              // rows per 1 KB copy instruction
  constexpr int NINS = TK / RPI;             // copy instructions per tile per tensor
  constexpr int LPW = (2 * NINS + NW - 1) / NW;  // copy instructions per wave per tile
  constexpr bool ALL_COPY = LPW * NW == 2 * NINS;
  constexpr int NDB = D >= 32 ? D / 32 : 1;  // 32-wide d blocks of O^T
  constexpr int NJ = D / 16;                 // 16-wide d steps of S^T
  constexpr int ROW16 = 16 * 2 * D;          // bytes of 16 tile rows
  static_assert(NINS == D / 8, "a V^T tile takes as many copy instructions as a K tile");
  using L = FwdLds<D>;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hh = lane >> 5;

  const int nq = (p.Sq + TQ - 1) / TQ;
  int col, rank;
  map_block(blockIdx.x, p.B * p.Hq, nq, col, rank);
  const int b = col / p.Hq, h = col % p.Hq, hk = h / p.G;
  const int qtile = p.mask.kind == MASK_FULL ? rank : nq - 1 - rank;
  MaskB m = resolve_mask(p, b);
  set_instance_kind<MK>(m);

  const int qa = qtile * TQ, qb = min(p.Sq, qa + TQ);
  const int wa = qa + wave * 32, wb = min(p.Sq, wa + 32);
  const int qi = wa + l32;                  // this lane's query row

  const bf16* Qg = static_cast<const bf16*>(p.q.ptr) + b * p.q.sb + h * p.q.sh;
  const bf16* Kg = static_cast<const bf16*>(p.k.ptr) + b * p.k.sb + hk * p.k.sh;
  const bf16* VTg = static_cast<const bf16*>(p.vt) + (int64_t)(b * p.Hkv + hk) * D * p.vt_ss;
  // BIAS: the scaled key bias of this batch entry, [vt_ss]
  constexpr bool has_bias = BIAS;
  const float* Bsg = BIAS ? p.bias_s + (int64_t)b * p.vt_ss : nullptr;

  // Q^T as the B operand: lane (q = l32, half hh) holds Q[q][16j + 8hh .. +8].
  bf16x8 qreg[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    qreg[j] = qi < p.Sq ? *reinterpret_cast<const bf16x8*>(Qg + (int64_t)qi * p.q.ss + 16 * j + 8 * hh)
                        : bf16x8{};
  wait_vmcnt<0>();  // Q is in registers before any copy is queued behind it

  f32x16 acc[NDB];
#pragma unroll
  for (int c = 0; c < NDB; ++c) acc[c] = f32x16{};
  float mrun = kMaxInit, lsum = 0.f;

  if constexpr (TTT) {
    // ttt_fold: key s*L + i of each later step s, one per row, with the exact
    // running max (plus the tile loop's slack) and no lazy bound,
    // before the tile loop (the order of the keys does not change the
    // result).  The score's two lane halves each
    // hold half of q_i.k (the d of qreg), summed across the halves; O^T
    // takes p * V row in the lane's own d positions.  Rows that are not real
    // or not below kv_valid take score -inf, which leaves O, l and the max
    // unchanged.
    const bf16* Vg = static_cast<const bf16*>(p.v.ptr) + b * p.v.sb + hk * p.v.sh;
    const int nseg = p.Skv / p.Sq;
    const bool rok = qi < p.Sq && qi < m.kvv;
#pragma unroll 1
    for (int s = 1; s < nseg; ++s) {
      const int64_t j = (int64_t)s * p.Sq + (rok ? qi : 0);
      const bf16* kr = Kg + j * p.k.ss + 8 * hh;
      const bf16* vr = Vg + j * p.v.ss + 4 * hh;
      float dot = 0.f;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) dot = dot_bf16x8(qreg[jj], *reinterpret_cast<const bf16x8*>(kr + 16 * jj), dot);
      dot = half_swap_sum(dot);
      const float x = rok ? (dot + (has_bias ? Bsg[j] : 0.f)) * p.scale_log2 : -INFINITY;
      const float mn = fmaxf(mrun, x + SLACK);
      const float alpha = exp2_fast(mrun - mn);
      const float pr = exp2_fast(x - mn);
      mrun = mn;
      lsum = lsum * alpha + (hh == 0 ? pr : 0.f);   // l's two halves are summed at the end
#pragma unroll
      for (int c = 0; c < NDB; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (32 * c + 8 * g >= D) continue;   // d = 32c + 8g + 4hh does not exist (D = 16)
          const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(vr + 32 * c + 8 * g);
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[c][4 * g + u] = acc[c][4 * g + u] * alpha + pr * (float)v4[u];
        }
    }
  }

  // Copy instructions: instruction idx (of 2 * NINS per ring step) moves 1 KB,
  // K rows RPI*idx .. +RPI when idx < NINS, else V^T d rows 8*(idx - NINS)
  // .. +8.  Wave w issues idx = w*LPW .. +LPW, all of one kind (wk).  A lane's
  // global offset is a per-wave row step (uniform), the lane's row (rbase)
  // and its swizzled chunk (cofs); the copies are selects, not branches.
  static_assert(NINS % LPW == 0, "a wave's copies are all K rows or all V^T rows");
  const int crow = lane / CPR, cslot = lane % CPR;
  const unsigned lds0 = lds_addr_of(smem);
  const bool wk = wave * LPW < NINS;
  const int rbase = wk ? (int)(crow * p.k.ss) : (int)((lane / (TK / 8)) * p.vt_ss);
  int cofs[LPW], rstep[LPW], ldso[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) {
    const int idx = wave * LPW + x;
    if (wk) {
      cofs[x] = 8 * (cslot ^ swz<D>(idx * RPI + crow));
      rstep[x] = (int)(idx * RPI * p.k.ss);
      ldso[x] = idx * 1024;
    } else {
      const int row = (idx - NINS) * (64 / (TK / 8)) + lane / (TK / 8);   // d row of V^T
      cofs[x] = 8 * ((lane % (TK / 8)) ^ vt_swz(row));
      rstep[x] = (int)((idx - NINS) * (64 / (TK / 8)) * p.vt_ss);
      ldso[x] = L::VT_BASE + (idx - NINS) * 1024;
    }
  }
  // Asynchronous copy of key tile t into ring buffer k (K rows and V^T rows):
  // this wave's share of the 2 * NINS instructions.  K rows that are not real
  // keys (and every row when t < 0) are fetched from key 0 instead: a real
  // row, so the scores stay finite, and the mask drops them.  (Only reached
  // when the walk has a tile, so key 0 is real.)  V^T rows need no
  // selection: the pre-pass zeroed every position that is not a real key,
  // and t < 0 reads tile 0.  Keys below kv_valid are real (kv_valid <= the
  // walked key count).
  // A tile whose K rows are all real keys (every tile but a ragged last one)
  // takes the scalar-base form: per-lane byte offsets computed once (voff),
  // the tile's base in scalar registers, no vector instructions.  The offsets
  // are unsigned there, so a K view with a negative sequence stride always
  // takes the general form.
  unsigned voff[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) voff[x] = 2u * (unsigned)(rstep[x] + rbase + cofs[x]);
  const bool soff_ok = p.k.ss >= 0;
  auto copy_tiles = [&](int t, int k) __attribute__((always_inline)) {
    const int tb = t * TK;
    const unsigned lbuf = lds0 + k * L::TILE_BYTES;
    if (soff_ok && t >= 0 && tb + TK <= m.kvv) {
      const bf16* sbase = wk ? Kg + (int64_t)tb * p.k.ss : VTg + tb;
#pragma unroll
      for (int x = 0; x < LPW; ++x) {
        const int idx = wave * LPW + x;
        if (ALL_COPY || idx < 2 * NINS) lds_dma16_s(sbase, voff[x], lbuf + ldso[x]);
      }
      return;
    }
    const int lim = t >= 0 ? m.kvv - tb : 0;   // K rows below lim are real keys
    const bf16* base = wk ? Kg + (int64_t)tb * p.k.ss : VTg + (t >= 0 ? tb : 0);
#pragma unroll
    for (int x = 0; x < LPW; ++x) {
      const int idx = wave * LPW + x;
      if (ALL_COPY || idx < 2 * NINS) {
        const bool ok = !wk || crow < lim - idx * RPI;
        const bf16* g = ok ? base + (rstep[x] + rbase + cofs[x]) : Kg + cofs[x];
        lds_dma16_at(g, lbuf + ldso[x]);
      }
    }
  };
  // With a key bias the last wave also copies each tile's 64 scaled bias
  // values into slot k (lanes 16..63 repeat lanes 0..15; the slot is 1 KB).
  const bool bias_wave = has_bias && wave == NW - 1;
  auto copy_bias = [&](int t, int k) __attribute__((always_inline)) {
    if (bias_wave) lds_dma16_at(Bsg + (t >= 0 ? t * TK : 0) + 4 * (lane & 15), lds0 + L::BIAS_BASE + k * 1024);
  };
  // Where the scores of the tile in buffer k start: the scaled bias of their
  // keys (register i of key block kb holds key 32 kb + 8 (i / 4) + 4 hh +
  // i % 4 of the tile), or zero.
  auto score_init = [&](int k, f32x16 (&s)[2]) __attribute__((always_inline)) {
    if (has_bias) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 b4 = *FA_LDS(const f32x4, smem + L::BIAS_BASE + k * 1024 + 4 * (32 * kb + 8 * g + 4 * hh));
#pragma unroll
          for (int u = 0; u < 4; ++u) s[kb][4 * g + u] = b4[u];
        }
    } else {
      s[0] = f32x16{};
      s[1] = f32x16{};
    }
  };

  // Lane-constant byte offsets into a tile: the swizzle of a row depends only
  // on its index mod 16, so key blocks and 16-key steps are immediates.
  int koff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) koff[j] = swz_off<D>(l32, 16 * j + 8 * hh);
  // V^T operand of 16-key step st: lane (l32, hh) reads row 32c + l32 of
  // the V^T tile, stored keys 16st + 8hh .. +8 (one 16-byte chunk).  Lanes
  // whose d row does not exist (D = 16) read a real row and use zeros.
  const bool d_lane_ok = D >= 32 || l32 < 16;
  const int vrow = D >= 32 ? l32 : (l32 & 15);
  int vto[TK / 16];
#pragma unroll
  for (int st = 0; st < TK / 16; ++st)
    vto[st] = L::VT_BASE + vrow * (2 * TK) + 16 * ((2 * st + hh) ^ vt_swz(vrow));

  // S^T of the tile in buffer k: 2 key blocks of 32.
  auto qk = [&](auto kc, f32x16 (&s)[2]) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    score_init(k, s);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *FA_LDS(const bf16x8, smem + k * L::TILE_BYTES + 2 * kb * ROW16 + koff[j]);
        s[kb] = mfma32(a, qreg[j], s[kb]);
      }
  };
  // O^T += V^T P^T for the tile in buffer k; V operands are read PF
  // products ahead of their use.
  auto pv = [&](auto kc, const bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    constexpr int NOP = 4 * NDB;   // (kb, st, c) products
    constexpr int PF = 3;
    auto vread = [&](int n) __attribute__((always_inline)) {
      const int c = n % NDB, st = n / NDB;
      const bf16x8 a = *FA_LDS(const bf16x8, smem + k * L::TILE_BYTES + c * 32 * (2 * TK) + vto[st]);
      return d_lane_ok ? a : bf16x8{};
    };
    bf16x8 va[PF + 1];
#pragma unroll
    for (int n = 0; n < PF && n < NOP; ++n) va[n] = vread(n);
#pragma unroll
    for (int n = 0; n < NOP; ++n) {
      if (n + PF < NOP) va[(n + PF) % (PF + 1)] = vread(n + PF);
      const int c = n % NDB, ks = n / NDB;
      acc[c] = mfma32(va[n % (PF + 1)], pb[ks >> 1][ks & 1], acc[c]);
    }
    // Keep the reads ahead of their products: left alone, the scheduler
    // moves each read next to its product and the wave waits out every
    // read's latency.
    sched_group(SCHED_DS_READ, PF);
#pragma unroll
    for (int n = 0; n < NOP; ++n) {
      sched_group(SCHED_MFMA, 1);
      if (n + PF < NOP) sched_group(SCHED_DS_READ, 1);
    }
  };
  // qk() and softmax() interleaved in program order: after product n come
  // the exponentials of score registers 2n and 2n+1 of the other tile.
  auto qk_softmax = [&](auto kc, f32x16 (&s)[2], const f32x16 (&sp)[2], bf16x8 (&pb)[2][2])
      __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    score_init(k, s);
    float e[2][2][8];
    float ls = 0.f;
    // K operands are read PF products ahead of their use.
    constexpr int PF = 3;
    auto kread = [&](int n) __attribute__((always_inline)) {
      return *FA_LDS(const bf16x8, smem + k * L::TILE_BYTES + 2 * (n & 1) * ROW16 + koff[n >> 1]);
    };
    bf16x8 ka[PF + 1];
#pragma unroll
    for (int n = 0; n < PF; ++n) ka[n] = kread(n);
#pragma unroll
    for (int n = 0; n < 2 * NJ; ++n) {
      const int j = n >> 1, kb = n & 1;
      if (n + PF < 2 * NJ) ka[(n + PF) % (PF + 1)] = kread(n + PF);
      s[kb] = mfma32(ka[n % (PF + 1)], qreg[j], s[kb]);
#pragma unroll
      for (int x = 0; x < 32 / (2 * NJ); ++x) {
        const int idx = n * (32 / (2 * NJ)) + x;   // 0..31: (kb', st', u)
        const int kb2 = idx >> 4, st2 = (idx >> 3) & 1, u = idx & 7;
        const float arg = sp[kb2][8 * st2 + u] * p.scale_log2 - mrun;
        e[kb2][st2][u] = LATE ? exp2_sat(arg) : exp2_fast(arg);
        if (u == 7) {
          pb[kb2][st2] = cat8(to_bf16x4(e[kb2][st2][0], e[kb2][st2][1], e[kb2][st2][2], e[kb2][st2][3]),
                              to_bf16x4(e[kb2][st2][4], e[kb2][st2][5], e[kb2][st2][6], e[kb2][st2][7]));
          ls = sum_bf16x8(pb[kb2][st2], ls);
        }
      }
    }
    return ls;
  };
  // !LATE: P of a tile against the running max, rounded to bf16, and its row
  // sum over the rounded values (two-way dot products with ones).
  auto softmax = [&](const f32x16 (&s)[2], bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) e[u] = exp2_fast(s[kb][8 * st + u] * p.scale_log2 - mrun);
        pb[kb][st] = cat8(to_bf16x4(e[0], e[1], e[2], e[3]), to_bf16x4(e[4], e[5], e[6], e[7]));
        ls = sum_bf16x8(pb[kb][st], ls);
      }
    return ls;
  };
  // Row max of a tile's scores, in log2 units (both lane halves).
  auto tile_max = [&](const f32x16 (&s)[2]) __attribute__((always_inline)) {
    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
    return half_swap_max(mx) * p.scale_log2;
  };
  // !LATE: running-max refresh from a tile's scores (rare): O^T and l move
  // to the new max.
  auto refresh = [&](const f32x16 (&s)[2]) __attribute__((always_inline)) {
    const float mn = fmaxf(mrun, tile_max(s));
    const float alpha = exp2_fast(mrun - mn);
    mrun = mn;
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < NDB; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] *= alpha;
  };
  // LATE: correction of a tile whose P may have saturated (rare: a row max
  // that grew by more than kSlack, or a row with no allowed key before),
  // after its PV products ran with Ps = min(1, exp2(x - mref)).  With mn = max(mref, row
  // max + kSlack) and alpha = exp2(mref - mn): O^T and l are scaled by alpha,
  // then the difference D = exp2(x - mn) - alpha * Ps goes through the PV
  // product and into l, so the tile's weights become exp2(x - mn) (up to
  // rounding) and l sums the same weights O^T holds.
  auto fixup = [&](auto kc, const f32x16 (&s)[2], const bf16x8 (&pb)[2][2]) __attribute__((always_inline)) {
    const float mn = fmaxf(mrun, tile_max(s) + kSlack);
    const float alpha = exp2_fast(mrun - mn);
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < NDB; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][i] *= alpha;
    bf16x8 db[2][2];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float d[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          d[u] = exp2_fast(s[kb][8 * st + u] * p.scale_log2 - mn) - alpha * (float)pb[kb][st][u];
        db[kb][st] = cat8(to_bf16x4(d[0], d[1], d[2], d[3]), to_bf16x4(d[4], d[5], d[6], d[7]));
        ls = sum_bf16x8(db[kb][st], ls);
      }
    lsum += ls;
    mrun = mn;
    pv(kc, db);
  };
  // Mask of tile t (partial and skipped tiles only).
  // Tiles below full_end hold only keys every row of this wave may attend
  // (the causal part's interior): no classification, no mask.
  const int full_end = full_tiles_below(m, wa, TK);
  auto mask = [&](int t, f32x16 (&s)[2]) __attribute__((always_inline)) {
    if (t < full_end) return;
    const int k0 = t * TK;
    const int state = tile_state(m, k0, TK, wa, wb);
    if (state != TILE_FULL) {
      const bool skip = state == TILE_SKIP;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
          s[kb][i] = (!skip && allowed(m, qi, key)) ? s[kb][i] : -INFINITY;
        }
    }
  };

  // The walk: key tiles [t, tend).  Every instance's mask is one segment
  // here (FULL, CAUSAL or WINDOW; TTT's later steps were folded above), so
  // the walk is a contiguous range.
  int t, tend;
  segment_tiles(m, 0, qa, qb, TK, t, tend);
  auto tile_or_none = [&](int u) __attribute__((always_inline)) { return u < tend ? u : -1; };

  // Ring buffers: tile t of the walk sits in buffer (t - t0) mod 4.  K rows
  // (and the bias) are read one iteration before V^T rows (QK^T of tile i+1
  // runs with PV of tile i), so they are copied one tile further ahead.
  f32x16 scur[2], snxt[2];
  if (t < tend) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {   // K rows of tiles t .. t+2, V^T rows of t, t+1
      if (wk || u < 2) copy_tiles(tile_or_none(t + u), u);
      copy_bias(tile_or_none(t + u), u);
    }
    wait_vmcnt<0>();
  }
  barrier_lds();
  if (t < tend) {
    qk(Buf<0>{}, scur);
    mask(t, scur);
    // The reference starts at (slack above) the first tile's row max, so only
    // a later jump of the max needs a correction.  (After the TTT fold O^T and
    // l already hold weights against the old reference.)
    const float mn = fmaxf(mrun, tile_max(scur) + SLACK);
    if constexpr (TTT) {
      const float alpha = exp2_fast(mrun - mn);
      lsum *= alpha;
#pragma unroll
      for (int c = 0; c < NDB; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] *= alpha;
    }
    mrun = mn;
  }
  barrier_lds();   // the first pair's copies refill K buffer 0

  // One iteration with tile i in buffer k; false when the walk has ended.
  // Iterations go in pairs with one barrier per pair: the first of a pair
  // issues the copies the next pair reads (K rows and bias of tiles i+3,
  // i+4, V^T rows of i+2, i+3, into the buffers the previous pair finished
  // with), the second waits for them and closes the pair with the barrier.
  auto step = [&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    if constexpr ((k & 1) == 0) {
      const int a = wk ? 3 : 2;
      copy_tiles(tile_or_none(t + a), (k + a) & (NBUF - 1));
      copy_tiles(tile_or_none(t + a + 1), (k + a + 1) & (NBUF - 1));
      copy_bias(tile_or_none(t + 3), (k + 3) & (NBUF - 1));
      copy_bias(tile_or_none(t + 4), k);
    }
    // QK^T of tile i+1 (its buffer may hold a stale tile at the end: unused)
    // with the exponentials of tile i spread between its products (they are
    // independent: matrix cores and vector ALUs overlap).
    // At D = 128 the wave raises its issue priority for this phase: its
    // exponentials then issue ahead of the other wave's vector work while
    // that wave's PV products keep the matrix cores busy.  (At D <= 64,
    // where the vector work per tile is as large as the matrix work, it was
    // slower.)
    bf16x8 pb[2][2];
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
    float ls = qk_softmax(Buf<(k + 1) & (NBUF - 1)>{}, snxt, scur, pb);
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(0);
    if constexpr (LATE) {
      lsum += ls;
      pv(kc, pb);
      // A P of 1 (saturated) makes its lane's sum at least 1.
      if (__any(!(ls < 1.0f))) fixup(kc, scur, pb);
    } else {
      if (__any(!(ls <= kSumLimit))) {
        refresh(scur);
        ls = softmax(scur, pb);
      }
      lsum += ls;
      pv(kc, pb);
    }
    if (t + 1 < tend) mask(t + 1, snxt);
    if constexpr ((k & 1) == 1) {
      wait_vmcnt<0>();
      barrier_lds();
    }
    scur[0] = snxt[0];
    scur[1] = snxt[1];
    return ++t < tend;
  };
  if (t < tend) {
    while (step(Buf<0>{}) && step(Buf<1>{}) && step(Buf<2>{}) && step(Buf<3>{})) {
    }
  }
  wait_vmcnt<0>();   // copies of tiles past the end land before the workgroup ends

  // Epilogue: O = acc / l, LSE = ln(sum exp(scaled scores)); empty rows -> 0.
  bf16* Og = static_cast<bf16*>(const_cast<void*>(p.o.ptr)) + b * p.o.sb + h * p.o.sh;
  float* Lg = p.lse + ((int64_t)b * p.Hq + h) * p.Sq;
  const float lt = half_swap_sum(lsum);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qi < p.Sq) {
    if (hh == 0) Lg[qi] = lt > 0.f ? (mrun + log2_fast(lt)) * kLn2 : 0.f;
#pragma unroll
    for (int c = 0; c < NDB; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * c + 8 * g + 4 * hh;
        if (d < D) {
          const bf16x4 o = to_bf16x4(acc[c][4 * g] * inv, acc[c][4 * g + 1] * inv,
                                     acc[c][4 * g + 2] * inv, acc[c][4 * g + 3] * inv);
          *reinterpret_cast<bf16x4*>(Og + (int64_t)qi * p.o.ss + d) = o;
        }
      }
  }
}

template <int D, int NW>
hipError_t launch(const Params& p, hipStream_t stream) {
  constexpr int TQ = NW * 32;
  const int nq = (p.Sq + TQ - 1) / TQ;
  const int64_t nblk = (int64_t)p.B * p.Hq * nq;
  if (nblk == 0) return hipSuccess;
  // V^T of the keys the tile walk reads, and the scaled key bias
  hipError_t e = launch_transpose_keys<D>(p, p.v, p.vt, p.vt_ss, stream);
  if (e != hipSuccess) return e;
  if ((e = launch_bias_scale(p, stream)) != hipSuccess) return e;
  const int lds = FwdLds<D>::BYTES + (p.bias_s ? FwdLds<D>::BIAS_BYTES : 0);
  const int mk = mask_instance(p.mask.kind);
  auto pick = [&](auto bc) {
    constexpr bool BI = decltype(bc)::value;
    return mk == MK_TTT ? fwd_kernel<D, NW, MK_TTT, BI>
                        : (mk == MK_WIN ? fwd_kernel<D, NW, MK_WIN, BI> : fwd_kernel<D, NW, MK_FC, BI>);
  };
  auto k = p.bias_s ? pick(std::true_type{}) : pick(std::false_type{});
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(NW * 64), lds, stream, p);
  return hipGetLastError();
}

// D = 128: 8-wave workgroups (256 query rows) when there are enough of them
// to fill the chip twice over, 4-wave ones (128 rows) for small problems.
// D <= 64: always 4-wave workgroups.  Their LDS ring (64 KB or less) lets two
// share a compute unit, so while one waits at its per-tile barrier the
// other's waves keep the SIMDs busy (an 8-wave workgroup's barrier stalls all
// of a compute unit's waves at once); at D = 128 one 4-wave workgroup's ring
// (128 KB) fills the LDS and leaves each SIMD a single wave.
template <int D>
hipError_t launch_d(const Params& p, hipStream_t s) {
  const int64_t wg8 = (int64_t)p.B * p.Hq * ((p.Sq + 255) / 256);
  if (D >= 128 && wg8 >= 512) return launch<D, 8>(p, s);
  return launch<D, 4>(p, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const Params& p, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_d<16>(p, s);
    case 32: return launch_d<32>(p, s);
    case 64: return launch_d<64>(p, s);
    case 128: return launch_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
