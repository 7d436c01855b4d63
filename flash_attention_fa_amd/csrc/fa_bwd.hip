// fa_bwd.hip - bf16 backward attention for gfx950 (MFMA 32x32x16).
//
// Gradient of L = sum(O * dO) through O = softmax(s Q K^T + mask) V, with P
// rebuilt from the saved LSE instead of being stored (CS336 "Flash Attention
// (Triton)": the backward recomputes the weights from the logsumexp; the
// ggml flash-attn-training playbook, section 1: a fused backward that is
// bitwise deterministic, no floating-point atomics, fixed schedules):
//   Delta_i = sum_d dO_id O_id                      (delta_kernel)
//   P_ij    = exp(s q_i.k_j - LSE_i)  on allowed pairs, else 0
//   dP_ij   = dO_i . v_j,   dS_ij = P_ij (dP_ij - Delta_i)
//   dV_j    = sum_i P_ij dO_i                        (dkdv_split_kernel)
//   dK_j    = s sum_i dS_ij q_i                      (dkdv_split_kernel)
//   dQ_i    = s sum_j dS_ij k_j                      (dq_dma_kernel)
// dK/dV are owned by key tiles and dQ by query tiles, so every output element
// is summed by exactly one workgroup in a fixed order: reruns are bitwise
// identical.  Keys no query may attend get exact zeros.
#include <climits>

#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace {

template <int K>
struct Buf {
  static constexpr int value = K;
};

// ---------------------------------------------------------------------------
// Delta = rowsum(dO * O), fp32, and the row's LSE in log2 units (the
// backward kernels rebuild P as exp2(scale*log2(e) * s - LSE*log2(e))).
// D/8 lanes per row, 16-byte loads.
template <int D>
__global__ void __launch_bounds__(256) delta_kernel(Params p) {
  constexpr int LPR = D / 8;        // lanes per row
  constexpr int RPB = 256 / LPR;    // rows per block
  const int64_t rows = (int64_t)p.B * p.Hq * p.Sq;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (r < rows) {
    const int i = (int)(r % p.Sq);
    const int64_t bh = r / p.Sq;
    const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    const bf16x8 o = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.o.ptr) + b * p.o.sb +
                                                      h * p.o.sh + (int64_t)i * p.o.ss + 8 * c);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.dout.ptr) + b * p.dout.sb +
                                                      h * p.dout.sh + (int64_t)i * p.dout.ss + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)o[e] * (float)g[e];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (r < rows && c == 0) {
    p.delta[r] = acc;
    p.lse2[r] = p.lse_in[r] * 1.4426950408889634f;
  }
}

// ---------------------------------------------------------------------------
// dQ with asynchronous staging: the forward's pipeline with a third
// product.  Key tiles of K and V rows are copied HBM -> LDS into a ring of
// four XOR-swizzled buffers three tiles ahead (three buffers, two ahead, at
// D = 64); per tile, S^T = K Q^T and
// dP^T = V dO^T (Q and dO in registers, K and V rows from LDS), dS^T =
// P^T (dP^T - Delta) with P^T = exp2(scale log2(e) S^T - LSE log2(e)), and
// dQ^T += K^T dS^T with K^T read transposed from the row-major K tile.
constexpr int DQ_TK = 64;     // keys per LDS tile

// The ring holds NBUF tiles, copied NBUF - 1 tiles ahead: four, except at
// D = 64, where three (48 KB) let three 4-wave workgroups share a compute
// unit (the kernel's 166 registers allow three waves per SIMD; a 64 KB ring
// allowed two workgroups).  With a key bias, NBUF 1 KB slots follow: each
// tile's 64 scaled bias values (256 bytes; the copy instruction that brings
// them writes 1 KB).
template <int D>
struct DqDma {
  static constexpr int NBUF = D == 64 ? 3 : 4;   // tiles in the ring
  static constexpr int TILE = DQ_TK * D * 2;   // K or V rows of one tile
  static constexpr int BUF = 2 * TILE;
  static constexpr int BYTES = NBUF * BUF;
  static constexpr int BIAS_BASE = BYTES;
  static constexpr int BIAS_BYTES = NBUF * 1024;
};

// MK: the mask-kind instance.  As in the forward, the MK_TTT tile loop walks
// the step-0 keys, which the causal mask describes, and adds the single key
// s*L + i of each later step s to row i's dQ with vector arithmetic
// (ttt_fold).
template <int D, int NW, int MK, bool BIAS>
__device__ __forceinline__ void dq_dma_body(const Params& p, int bid) {
  constexpr bool TTT = MK == MK_TTT;
  using L = DqDma<D>;
  constexpr int TQ = NW * 32;
  constexpr int TK = DQ_TK;
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int NINS = TK / RPI;
  constexpr int LPW = (2 * NINS + NW - 1) / NW;
  constexpr bool ALL_COPY = LPW * NW == 2 * NINS;
  // 32-wide d blocks of dQ^T; at D = 16 one block whose rows d >= 16 hold
  // nothing real (their operands read real columns again and are never written)
  constexpr int NDB = D >= 32 ? D / 32 : 1;
  constexpr int NJ = D / 16;
  constexpr int ROW16 = 16 * 2 * D;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hh = lane >> 5;
  (void)tid;

  const int nq = (p.Sq + TQ - 1) / TQ;
  int col, rank;
  map_block(bid, p.B * p.Hq, nq, col, rank);
  const int b = col / p.Hq, h = col % p.Hq, hk = h / p.G;
  const int qtile = p.mask.kind == MASK_FULL ? rank : nq - 1 - rank;
  MaskB m = resolve_mask(p, b);
  set_instance_kind<MK>(m);
  const int qa = qtile * TQ, qb = min(p.Sq, qa + TQ);
  const int wa = qa + wave * 32, wb = min(p.Sq, wa + 32);
  const int qi = wa + l32;

  const bf16* Qg = static_cast<const bf16*>(p.q.ptr) + b * p.q.sb + h * p.q.sh;
  const bf16* Gg = static_cast<const bf16*>(p.dout.ptr) + b * p.dout.sb + h * p.dout.sh;
  const bf16* Kg = static_cast<const bf16*>(p.k.ptr) + b * p.k.sb + hk * p.k.sh;
  const bf16* Vg = static_cast<const bf16*>(p.v.ptr) + b * p.v.sb + hk * p.v.sh;
  const int64_t rowbase = ((int64_t)b * p.Hq + h) * p.Sq;
  // BIAS: the scaled key bias of this batch entry, [vt_ss]
  constexpr bool has_bias = BIAS;
  const float* Bsg = BIAS ? p.bias_s + (int64_t)b * p.vt_ss : nullptr;

  // Q^T and dO^T as B operands; LSE (log2 units) and Delta one per lane.
  bf16x8 qreg[NJ], greg[NJ];
  const bool qok = qi < p.Sq;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    qreg[j] = qok ? *reinterpret_cast<const bf16x8*>(Qg + (int64_t)qi * p.q.ss + 16 * j + 8 * hh) : bf16x8{};
    greg[j] = qok ? *reinterpret_cast<const bf16x8*>(Gg + (int64_t)qi * p.dout.ss + 16 * j + 8 * hh) : bf16x8{};
  }
  const float l2 = qok ? p.lse2[rowbase + qi] : 0.f;
  const float dlt = qok ? p.delta[rowbase + qi] : 0.f;
  wait_vmcnt<0>();

  f32x16 acc[NDB];
#pragma unroll
  for (int c = 0; c < NDB; ++c) acc[c] = f32x16{};

  if constexpr (TTT) {
    // ttt_fold: for key j = s*L + i of each later step s (row i below
    // kv_valid), P = exp2(scale log2(e) q_i.k_j - LSE_i log2(e)), dP =
    // dO_i.v_j, dS = P (dP - Delta_i) and dQ_i^T += k_j dS, in fp32, before
    // the tile loop.  Each lane half holds half of every dot product (the d
    // of qreg / greg), summed across the halves.
    const int nseg = p.Skv / p.Sq;
    const bool rok = qok && qi < m.kvv;
#pragma unroll 1
    for (int s = 1; s < nseg; ++s) {
      const int64_t j = (int64_t)s * p.Sq + (rok ? qi : 0);
      const bf16* kr = Kg + j * p.k.ss;
      const bf16* vr = Vg + j * p.v.ss + 8 * hh;
      float sd = 0.f, pd = 0.f;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        sd = dot_bf16x8(qreg[jj], *reinterpret_cast<const bf16x8*>(kr + 8 * hh + 16 * jj), sd);
        pd = dot_bf16x8(greg[jj], *reinterpret_cast<const bf16x8*>(vr + 16 * jj), pd);
      }
      sd = half_swap_sum(sd);
      pd = half_swap_sum(pd);
      const float pr = rok ? exp2_fast((sd + (has_bias ? Bsg[j] : 0.f)) * p.scale_log2 - l2) : 0.f;
      const float ds = pr * (pd - dlt);
      const bf16* kd = kr + 4 * hh;
#pragma unroll
      for (int c = 0; c < NDB; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (32 * c + 8 * g >= D) continue;   // d = 32c + 8g + 4hh does not exist (D = 16)
          const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(kd + 32 * c + 8 * g);
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[c][4 * g + u] += ds * (float)k4[u];
        }
    }
  }

  // Copy instructions: instruction idx (of 2 * NINS per tile) moves 1 KB,
  // rows RPI*(idx % NINS) .. +RPI of K (idx < NINS) or V.  Wave w issues idx =
  // w*LPW .. +LPW, all of one tensor; a lane's global offset is a per-
  // instruction row step (uniform), the lane's row (rbase) and its swizzled
  // chunk (cofs), so the copies are selects, not branches.
  static_assert(NINS % LPW == 0, "a wave's copies all come from one tensor");
  const int crow = lane / CPR, cslot = lane % CPR;
  const unsigned lds0 = lds_addr_of(smem);
  const bool wk = wave * LPW < NINS;
  const bf16* Xg = wk ? Kg : Vg;
  const int64_t xss = wk ? p.k.ss : p.v.ss;
  const int rbase = (int)(crow * xss);
  int cofs[LPW], rstep[LPW], ldso[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) {
    const int idx = wave * LPW + x, ii = idx % NINS;
    cofs[x] = 8 * (cslot ^ swz<D>(ii * RPI + crow));
    rstep[x] = (int)(ii * RPI * xss);
    ldso[x] = (idx / NINS) * L::TILE + ii * 1024;
  }
  // Key tile t (K rows then V rows) into buffer k; keys that are not real
  // (and every key when t < 0) come from key 0: finite, and masked.  Keys
  // below kv_valid are real (kv_valid <= the walked key count).
  // A tile whose rows are all real keys takes the scalar-base form (per-lane
  // byte offsets computed once, no vector instructions per copy); a negative
  // sequence stride, a ragged last tile and tiles past the end take the
  // general form.
  unsigned voff[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) voff[x] = 2u * (unsigned)(rstep[x] + rbase + cofs[x]);
  const bool soff_ok = xss >= 0;
  // With a key bias the last wave also copies the tile's 64 scaled bias
  // values (lanes 16..63 repeat lanes 0..15; the slot is 1 KB).
  const bool bias_wave = has_bias && wave == NW - 1;
  auto copy_tile = [&](int t, int k) __attribute__((always_inline)) {
    const int tb = t * TK;
    const unsigned lbuf = lds0 + k * L::BUF;
    if (bias_wave)
      lds_dma16_at(Bsg + (t >= 0 ? tb : 0) + 4 * (lane & 15), lds0 + L::BIAS_BASE + k * 1024);
    if (soff_ok && t >= 0 && tb + TK <= m.kvv) {
      const bf16* sbase = Xg + (int64_t)tb * xss;
#pragma unroll
      for (int x = 0; x < LPW; ++x) {
        const int idx = wave * LPW + x;
        if (ALL_COPY || idx < 2 * NINS) lds_dma16_s(sbase, voff[x], lbuf + ldso[x]);
      }
      return;
    }
    const int lim = t >= 0 ? m.kvv - tb : 0;   // rows below lim are real keys
    const bf16* base = Xg + (int64_t)tb * xss;
#pragma unroll
    for (int x = 0; x < LPW; ++x) {
      const int idx = wave * LPW + x;
      if (ALL_COPY || idx < 2 * NINS) {
        const bool ok = crow < lim - (idx % NINS) * RPI;
        const bf16* g = ok ? base + (rstep[x] + rbase + cofs[x]) : Xg + cofs[x];
        lds_dma16_at(g, lbuf + ldso[x]);
      }
    }
  };
  const int my_ins = (ALL_COPY ? LPW : (wave * LPW < 2 * NINS ? LPW : 0)) + (bias_wave ? 1 : 0);
  auto wait_copies = [&]() __attribute__((always_inline)) {
    if (my_ins == LPW) wait_vmcnt<LPW>();
    else if (my_ins == LPW + 1) wait_vmcnt<LPW + 1>();
    else if (my_ins == 1) wait_vmcnt<1>();
    else wait_vmcnt<0>();
  };

  int koff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) koff[j] = swz_off<D>(l32, 16 * j + 8 * hh);
  const int tr_row = (lane & 15) >> 2;
  // (at D = 16 the lanes that would address columns 16..31 address real
  // columns instead; what they deliver lands in rows d >= 16 only)
  const int tr_col = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) & (D >= 32 ? 31 : D - 1);
  int toff[2][NDB];
#pragma unroll
  for (int c = 0; c < NDB; ++c) {
    toff[0][c] = swz_off<D>(4 * hh + tr_row, 32 * c + tr_col);
    toff[1][c] = swz_off<D>(4 * hh + tr_row + 8, 32 * c + tr_col);
  }

  // tiles below full_end: every key allowed for every row of this wave
  const int full_end = full_tiles_below(m, wa, TK);
  // The walk: key tiles [t, tend).  Every instance's mask is one segment
  // here (FULL, CAUSAL or WINDOW; TTT's later steps were folded above), so
  // the walk is a contiguous range.
  int t, tend;
  segment_tiles(m, 0, qa, qb, TK, t, tend);
  auto tile_or_none = [&](int u) __attribute__((always_inline)) { return u < tend ? u : -1; };
  constexpr int NB = L::NBUF;
  if (t < tend) {
    copy_tile(t, 0);
    copy_tile(tile_or_none(t + 1), 1);
    if constexpr (NB == 4) copy_tile(tile_or_none(t + 2), 2);
    wait_copies();
  }
  barrier_lds();

  auto step = [&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    copy_tile(tile_or_none(t + NB - 1), (k + NB - 1) % NB);
    const int k0 = t * TK;
    const int state = t < full_end ? TILE_FULL : tile_state(m, k0, TK, wa, wb);
    if (state != TILE_SKIP) {
      const unsigned char* Kt = smem + k * L::BUF;
      const unsigned char* Vt = Kt + L::TILE;
      // The tile's two 32-key blocks one after the other (a wave cannot
      // overlap a block's exponentials with its own products anyway, and one
      // block's S^T and dP^T hold half the registers of two): S^T and dP^T of
      // the block, whose A operands (K and V rows) are read PF products ahead
      // of their use; dS^T; then the block's dQ^T products, whose transposed
      // K operands are read before the exponentials so their latency hides
      // behind them.
      constexpr int NSD = 2 * NJ;   // S^T and dP^T products of one key block
      constexpr int NDQ = 2 * NDB;  // dQ^T products of one key block
      constexpr int PF = 3;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // At D >= 64, raised issue priority while this wave forms S, dP and
        // dS: its exponentials issue ahead of the other wave's vector work
        // while that wave's dQ products keep the matrix cores busy (at
        // D <= 32 it was slower).
        if constexpr (D >= 64) __builtin_amdgcn_s_setprio(1);
        // dP^T accumulates onto -Delta (the lane's row), so it comes out as
        // dP^T - Delta; S^T onto the scaled bias of each register's key
        // (32 kb + 8 (i / 4) + 4 hh + i % 4 of the tile), or zero.
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) dp[i] = -dlt;
        if (has_bias) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 b4 = *FA_LDS(const f32x4, smem + L::BIAS_BASE + k * 1024 + 4 * (32 * kb + 8 * g + 4 * hh));
#pragma unroll
            for (int u = 0; u < 4; ++u) s[4 * g + u] = b4[u];
          }
        } else {
          s = f32x16{};
        }
        auto opread = [&](int n) __attribute__((always_inline)) {
          return *FA_LDS(const bf16x8, ((n & 1) ? Vt : Kt) + 2 * kb * ROW16 + koff[n >> 1]);
        };
        bf16x8 op[PF + 1];
#pragma unroll
        for (int n = 0; n < PF; ++n) op[n] = opread(n);
#pragma unroll
        for (int n = 0; n < NSD; ++n) {
          if (n + PF < NSD) op[(n + PF) % (PF + 1)] = opread(n + PF);
          if (n & 1) dp = mfma32(op[n % (PF + 1)], greg[n >> 1], dp);
          else s = mfma32(op[n % (PF + 1)], qreg[n >> 1], s);
        }
        // keep the operand reads ahead of their products
        sched_group(SCHED_DS_READ, PF);
#pragma unroll
        for (int n = 0; n < NSD; ++n) {
          sched_group(SCHED_MFMA, 1);
          if (n + PF < NSD) sched_group(SCHED_DS_READ, 1);
        }
        // K^T operands of this block's dQ^T products (two transposing reads each)
        auto tread = [&](int n) __attribute__((always_inline)) {
          const int rows = (2 * kb + n / NDB) * ROW16, c = n % NDB;
          return cat8(lds_read_tr4(reinterpret_cast<const bf16*>(Kt + rows + toff[0][c])),
                      lds_read_tr4(reinterpret_cast<const bf16*>(Kt + rows + toff[1][c])));
        };
        constexpr int TPF = 2;
        bf16x8 ta[TPF + 1];
#pragma unroll
        for (int n = 0; n < TPF; ++n) ta[n] = tread(n);
        if (state == TILE_PART) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
            s[i] = allowed(m, qi, key) ? s[i] : -INFINITY;
          }
        }
        // dS^T = P^T (dP^T - Delta), rounded to bf16 for the K^T dS^T product.
        bf16x8 dsb[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          float e[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = 8 * st + u;
            e[u] = exp2_fast(s[i] * p.scale_log2 - l2) * dp[i];
          }
          dsb[st] = cat8(to_bf16x4(e[0], e[1], e[2], e[3]), to_bf16x4(e[4], e[5], e[6], e[7]));
        }
        if constexpr (D >= 64) __builtin_amdgcn_s_setprio(0);
        // dQ^T += K^T dS^T, K^T read transposed from the K rows.
#pragma unroll
        for (int n = 0; n < NDQ; ++n) {
          if (n + TPF < NDQ) ta[(n + TPF) % (TPF + 1)] = tread(n + TPF);
          acc[n % NDB] = mfma32(ta[n % (TPF + 1)], dsb[n / NDB], acc[n % NDB]);
        }
      }
    }
    wait_copies();
    barrier_lds();
    return ++t < tend;
  };
  if (t < tend) {
    if constexpr (NB == 4) {
      while (step(Buf<0>{}) && step(Buf<1>{}) && step(Buf<2>{}) && step(Buf<3>{})) {
      }
    } else {
      while (step(Buf<0>{}) && step(Buf<1>{}) && step(Buf<2>{})) {
      }
    }
  }
  wait_vmcnt<0>();   // copies of tiles past the end

  bf16* Dg = static_cast<bf16*>(const_cast<void*>(p.dq.ptr)) + b * p.dq.sb + h * p.dq.sh;
  if (qok) {
#pragma unroll
    for (int c = 0; c < NDB; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * c + 8 * g + 4 * hh;
        if (32 * c + 8 * g >= D) continue;   // rows d >= D of the block (D = 16)
        const float sc = p.scale;
        *reinterpret_cast<bf16x4*>(Dg + (int64_t)qi * p.dq.ss + d) =
            to_bf16x4(acc[c][4 * g] * sc, acc[c][4 * g + 1] * sc, acc[c][4 * g + 2] * sc, acc[c][4 * g + 3] * sc);
      }
  }
}

template <int D, int NW, int MK, bool BIAS>
__global__ void __launch_bounds__(NW * 64, 2)
dq_dma_kernel(Params p) {
  dq_dma_body<D, NW, MK, BIAS>(p, blockIdx.x);
}

// ---------------------------------------------------------------------------
// dK/dV with asynchronous staging.  A workgroup owns NW * 32 keys (256 at
// D = 128, 128 at D <= 64) of one (batch, kv head) and one half of their
// (query tile, head) steps; wave w owns keys 32w .. 32w+31 outright.  Its K rows stay in registers (the B
// operand of S = Q K^T, natural orientation, a lane per key column); the
// workgroup's V rows sit in LDS.  Each step stages one 64-row query tile of
// one head (Q, dO, LSE*log2(e), Delta), worked through as two 32-row
// sub-tiles, by the asynchronous LDS copies of the
// forward into unpadded XOR-swizzled rows, the next step's during this one
// (double-buffered, one barrier per step).  dO^T and Q^T, the A operands of
// dV^T += dO^T P and dK^T += Q^T dS, are read straight from those row-major
// tiles with transposing LDS reads.  Rows past Sq are copied from the tile's
// first row (finite) and masked.
//
// At D = 128, 256 keys per workgroup let each staged query row serve twice
// the matrix work of a 128-key block (the copies into LDS are the kernel's
// costliest non-matrix work).  With fewer than 1024 blocks of 256 keys
// (dkdv_split, whatever the workgroup's own size), each
// block's steps are split between two workgroups, which keeps enough
// workgroups to balance the causal triangle (the halves are the two halves
// of the group's heads, or of the steps when the group is odd); each half
// writes its float32 sums to the workspace and dkdv_reduce_kernel adds the
// two halves, always half 0 + half 1, so reruns are bitwise identical.
// With more blocks one workgroup takes every step of its block and writes
// dK and dV directly.
// D <= 64: 4-wave workgroups of 128 keys (two or more share a compute unit,
// so one's per-step barrier does not idle all of its waves; three at D = 64,
// see dkdv_split_kernel); D = 128: 8 waves, 256 keys.
template <int D>
struct KvSplit {
  static constexpr int NW = D <= 64 ? 4 : 8;
  static constexpr int TKW = NW * 32;                  // keys per workgroup
  static constexpr int TQ = 64;                        // query rows per step (two 32-row sub-tiles)
  static constexpr int TILE = TQ * D * 2;              // one Q or dO tile (bytes)
  static constexpr int STAGE = 2 * TILE + 2 * TQ * 4;  // Q, dO, LSE*log2(e), Delta
  static constexpr int VB = TKW * D * 2;               // the V rows
  static constexpr int BYTES = 2 * STAGE + VB;
};

// MK: MK_FC (FULL, CAUSAL and TTT's step-0 keys) or MK_WIN.  SPLIT: two
// workgroups per key block, each writing float32 partial sums (see
// dkdv_split); without it one workgroup takes every step of its block and
// writes dK, dV.
template <int D, int MK, bool SPLIT, bool BIAS>
__device__ __forceinline__ void dkdv_split_body(const Params& p, int bid) {
  using L = KvSplit<D>;
  constexpr int NW = L::NW, TKW = L::TKW, TQ = L::TQ;
  // 32-wide d blocks of dK^T / dV^T; at D = 16 one block whose rows d >= 16
  // hold nothing real (their operands read real columns again; never written)
  constexpr int NJ = D / 16, NDB = D >= 32 ? D / 32 : 1;
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;         // rows per copy instruction
  constexpr int QINS = TQ / RPI;        // copy instructions per Q (or dO) tile
  // per copying wave per step (at D = 16 with 8 waves the 4 copies would take
  // 4 of them)
  constexpr int QLPW = 2 * QINS >= NW ? 2 * QINS / NW : 1;
  constexpr int VINS = TKW / RPI;       // copy instructions for the V rows
  constexpr int VLPW = VINS / NW;
  constexpr int ROW16 = 16 * 2 * D;     // bytes of 16 rows
  static_assert(D >= 16 && QLPW * NW >= 2 * QINS && QINS % QLPW == 0 && VLPW * NW == VINS &&
                kDkdvKeys % TKW == 0, "copy split");
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* const Vs = smem + 2 * L::STAGE;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hh = lane >> 5;

  // Block -> (batch, kv head, half of the steps) column and key-block rank.
  // Under TTT this kernel takes the step-0 keys (below L = Sq), which the
  // causal mask with the same shift and kv_valid describes; ttt_dkdv_kernel
  // takes the keys of the later steps.
  const int nkeys = walk_keys(p);
  const int nkt = (nkeys + TKW - 1) / TKW;
  int col, rank;
  map_block(bid, p.B * p.Hkv * (SPLIT ? 2 : 1), nkt, col, rank);
  const int half = SPLIT ? col & 1 : 0, bh = SPLIT ? col >> 1 : col;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  MaskB m = resolve_mask(p, b);
  set_instance_kind<MK>(m);
  m.Skv = nkeys;
  const int ka = rank * TKW, kbnd = min(nkeys, ka + TKW);
  const int kw = ka + wave * 32, kwe = min(nkeys, kw + 32);
  const int key = kw + l32;

  const bf16* Kg = static_cast<const bf16*>(p.k.ptr) + b * p.k.sb + hk * p.k.sh;
  const bf16* Vg = static_cast<const bf16*>(p.v.ptr) + b * p.v.sb + hk * p.v.sh;
  const int crow = lane / CPR, cslot = lane % CPR;

  // The workgroup's V rows; keys that are not real are copied from key 0
  // (finite values; their weights are masked to zero).
#pragma unroll
  for (int x = 0; x < VLPW; ++x) {
    const int ii = wave * VLPW + x;
    const int row = ii * RPI + crow;
    const int kk = ka + row;
    const int ch = 8 * (cslot ^ swz<D>(row));
    lds_dma16(Vg + (key_valid_nb(m, kk) ? (int64_t)kk * p.v.ss + ch : (int64_t)ch), Vs + ii * 1024);
  }
  // This wave's K rows as the B operand of S: lane (key, hh) holds
  // d = 16j + 8hh .. +8; keys that are not real hold zeros (and are masked).
  bf16x8 kreg[NJ];
  {
    const bool kok = key_valid_nb(m, key);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      kreg[j] = kok ? *reinterpret_cast<const bf16x8*>(Kg + (int64_t)key * p.k.ss + 16 * j + 8 * hh) : bf16x8{};
  }

  int qlo, qhi;
  query_hull(m, ka, kbnd, qlo, qhi);
  if (kbnd <= p.mask.frozen) qhi = qlo;   // every key frozen: no steps, zeros written
  const int t_first = qlo < qhi ? qlo / TQ : 0;
  const int t_last = qlo < qhi ? (qhi + TQ - 1) / TQ : 0;
  // The block's (query tile, head) steps with the group's heads inside, so
  // the workgroups sharing an XCD read the same tiles at about the same time.
  // With an even group each half takes half of the heads over every tile
  // (each Q/dO tile is then read by one half only, on one XCD); with an odd
  // one, half of the steps in the downward order.  Without SPLIT the one
  // workgroup takes them all.
  // Direction.  Under the causal triangle block r has nkt - r tiles of steps
  // and the blocks of an XCD start in rank order, so the compute unit that
  // finishes block r (of the first nkt / 2) is the one that next takes
  // about block nkt - 1 - r.  The first half of the ranks walk from the last
  // tile down, the second half from their diagonal up: at any moment the
  // workgroups of an XCD then read one of two tiles, and each Q/dO tile comes
  // from HBM about twice in all, where a downward walk started at each
  // workgroup's own time re-fetched it once per late starter.
  const int ntile = t_last - t_first;
  const bool by_head = SPLIT && (p.G & 1) == 0;
  const bool up = (by_head || !SPLIT) && m.kind == MASK_CAUSAL && 2 * rank >= nkt;   // CAUSAL, TTT
  const int hbeg = by_head ? half * (p.G / 2) : 0;
  const int hend = by_head ? hbeg + p.G / 2 : p.G;
  const int nall = ntile * p.G;
  const int s0 = by_head || half == 0 ? 0 : (nall + 1) / 2;
  const int nsteps = !SPLIT ? nall
                   : by_head ? ntile * (p.G / 2) : (half == 0 ? (nall + 1) / 2 : nall - (nall + 1) / 2);

  // Waves 0..NW/2-1 copy the Q rows, the others the dO rows (a run of QLPW
  // 1 KB copies each); LSE*log2(e) and Delta come through wave 0's registers.
  const int cidx0 = wave * QLPW;
  const bool stage_g = cidx0 >= QINS;
  const bf16* const Sbase = stage_g ? static_cast<const bf16*>(p.dout.ptr) + b * p.dout.sb
                                    : static_cast<const bf16*>(p.q.ptr) + b * p.q.sb;
  const int64_t ssh = stage_g ? p.dout.sh : p.q.sh;
  const int64_t sss = stage_g ? p.dout.ss : p.q.ss;
  int schunk[QLPW];
#pragma unroll
  for (int x = 0; x < QLPW; ++x) schunk[x] = 8 * (cslot ^ swz<D>((cidx0 % QINS + x) * RPI + crow));
  struct StepPos {
    int hs, q0;   // head slot in the group, first query row of the tile
  };
  const int qdir = up ? TQ : -TQ;
  auto advance = [&](StepPos& sp) __attribute__((always_inline)) {
    if (++sp.hs == hend) { sp.hs = hbeg; sp.q0 += qdir; }
  };
  // Whole tiles (every row below Sq) with a non-negative row stride take the
  // scalar-base form: per-lane byte offsets computed once, no vector
  // instructions per copy.
  unsigned qvoff[QLPW];
#pragma unroll
  for (int x = 0; x < QLPW; ++x) qvoff[x] = 2u * (unsigned)(((cidx0 % QINS + x) * RPI + crow) * (int)sss + schunk[x]);
  const unsigned lds_stage0 = lds_addr_of(smem) + (stage_g ? L::TILE : 0);
  const bool copier = cidx0 < 2 * QINS;   // this wave issues copies
  auto stage_rows = [&](const StepPos& sp, int buf) __attribute__((always_inline)) {
    if (!copier) return;
    const bf16* Sg = Sbase + (int64_t)(hk * p.G + sp.hs) * ssh + (int64_t)sp.q0 * sss;
    unsigned char* dst = smem + buf * L::STAGE + (stage_g ? L::TILE : 0);
    const bool whole = sp.q0 + TQ <= p.Sq;   // every row real: no per-lane select
    if (whole && sss >= 0) {
#pragma unroll
      for (int x = 0; x < QLPW; ++x)
        lds_dma16_s(Sg, qvoff[x], lds_stage0 + buf * L::STAGE + (cidx0 % QINS + x) * 1024);
      return;
    }
#pragma unroll
    for (int x = 0; x < QLPW; ++x) {
      const int ii = cidx0 % QINS + x;
      const int row = ii * RPI + crow;
      const bool ok = whole || sp.q0 + row < p.Sq;
      // rows past Sq are copied from the tile's first row (real, finite);
      // row * stride < 2^30 (strides are below 2^24 elements)
      lds_dma16(Sg + ((ok ? row * (int)sss : 0) + schunk[x]), dst + ii * 1024);
    }
  };
  float lrow = 0.f, drow = 0.f;
  auto fetch_rowvals = [&](const StepPos& sp) __attribute__((always_inline)) {
    if (tid < TQ) {
      const int q = sp.q0 + tid;
      const int64_t rb = ((int64_t)b * p.Hq + hk * p.G + sp.hs) * p.Sq;
      lrow = q < p.Sq ? p.lse2[rb + q] : 0.f;
      drow = q < p.Sq ? -p.delta[rb + q] : 0.f;   // staged as -Delta
    }
  };
  auto store_rowvals = [&](int buf) __attribute__((always_inline)) {
    float* Ls = reinterpret_cast<float*>(smem + buf * L::STAGE + 2 * L::TILE);
    if (tid < TQ) { Ls[tid] = lrow; Ls[TQ + tid] = drow; }
  };
  StepPos cur{by_head ? hbeg : s0 % p.G, (up ? t_first : t_last - 1 - (by_head ? 0 : s0 / p.G)) * TQ};
  StepPos nxt = cur;
  if (nsteps > 0) advance(nxt);
  if (nsteps > 0) {
    stage_rows(cur, 0);
    fetch_rowvals(cur);
  }
  wait_vmcnt<0>();
  if (nsteps > 0) store_rowvals(0);
  __syncthreads();

  int roff[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) roff[j] = swz_off<D>(l32, 16 * j + 8 * hh);
  const int tr_row = (lane & 15) >> 2;
  // (at D = 16 the lanes that would address columns 16..31 address real
  // columns instead; what they deliver lands in rows d >= 16 only)
  const int tr_col = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) & (D >= 32 ? 31 : D - 1);
  int toff[2][NDB];
#pragma unroll
  for (int c = 0; c < NDB; ++c) {
    toff[0][c] = swz_off<D>(4 * hh + tr_row, 32 * c + tr_col);
    toff[1][c] = swz_off<D>(4 * hh + tr_row + 8, 32 * c + tr_col);
  }
  const unsigned char* Vw = Vs + wave * 32 * 2 * D;

  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int c = 0; c < NDB; ++c) { dka[c] = f32x16{}; dva[c] = f32x16{}; }

  // BIAS: S starts from the scaled bias of this lane's key (the same for
  // every query row); otherwise from zero.
  const float kbias = BIAS && key < nkeys ? p.bias_s[(int64_t)b * p.vt_ss + key] : 0.f;

  // Rows from qfull on see every key of this wave's block (CAUSAL / FULL):
  // their tiles need no mask and no classification.
  int qfull = INT_MAX;
  if (kwe <= m.kvv && kw < kwe) {
    if (m.kind == MASK_FULL) qfull = 0;
    else if (m.kind == MASK_CAUSAL) qfull = kwe - 1 + m.shift;
  }
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) {
      stage_rows(nxt, buf ^ 1);
      fetch_rowvals(nxt);
    }
    const unsigned char* Qt = smem + buf * L::STAGE;
    const unsigned char* Gt = Qt + L::TILE;
    const float* Ls = reinterpret_cast<const float*>(Qt + 2 * L::TILE);
    const float* Ds = Ls + TQ;   // -Delta of the rows
    // 32-row sub-tiles; unrolled where registers allow (D <= 64), so one
    // sub-tile's products can overlap the other's exponentials
#pragma unroll(D <= 64 ? TQ / 32 : 1)
    for (int h = 0; h < TQ / 32; ++h) {
    const int qa = cur.q0 + 32 * h;
    int state = TILE_FULL;
    if (!(qa >= qfull && qa + 32 <= p.Sq)) {
      state = rect_state(m, kw, kwe, qa, min(p.Sq, qa + 32));
      if (state == TILE_FULL && qa + 32 > p.Sq) state = TILE_PART;   // rows past Sq
    }
    if (state != TILE_SKIP) {
      // At D = 64 the wave raises its issue priority while it forms S, dP,
      // P and dS, as the forward and dQ kernels do; at D = 128 and at
      // D <= 32 that was slower.
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
      // dP accumulates onto -Delta of each register's row (q = qa + 8*(i/4) +
      // 4*hh + i%4), so it comes out as dP - Delta.
      f32x16 s, dp;
      if constexpr (BIAS) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = kbias;
      } else {
        s = f32x16{};
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 d4 = *FA_LDS(const f32x4, Ds + 32 * h + 8 * g + 4 * hh);
#pragma unroll
        for (int u = 0; u < 4; ++u) dp[4 * g + u] = d4[u];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8 aq = *FA_LDS(const bf16x8, Qt + h * 32 * 2 * D + roff[j]);
        const bf16x8 ag = *FA_LDS(const bf16x8, Gt + h * 32 * 2 * D + roff[j]);
        s = mfma32(aq, kreg[j], s);
        dp = mfma32(ag, *FA_LDS(const bf16x8, Vw + roff[j]), dp);
      }
      // Per-register query rows: q = qa + 8*(i/4) + 4*hh + i%4.
      if (state == TILE_PART) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = qa + 8 * (i >> 2) + 4 * hh + (i & 3);
          s[i] = (allowed(m, qi, key) & (qi < p.Sq)) ? s[i] : -INFINITY;
        }
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float pe[8], de[8];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g = 2 * st + g2;
          const f32x4 l4 = *FA_LDS(const f32x4, Ls + 32 * h + 8 * g + 4 * hh);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * g + u;
            const float pr = exp2_fast(s[i] * p.scale_log2 - l4[u]);
            pe[4 * g2 + u] = pr;
            de[4 * g2 + u] = pr * dp[i];
          }
        }
        pb[st] = cat8(to_bf16x4(pe[0], pe[1], pe[2], pe[3]), to_bf16x4(pe[4], pe[5], pe[6], pe[7]));
        dsb[st] = cat8(to_bf16x4(de[0], de[1], de[2], de[3]), to_bf16x4(de[4], de[5], de[6], de[7]));
      }
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
      // dV^T += dO^T P,  dK^T += Q^T dS: A operands read transposed from the
      // row-major tiles (rows 16 st + (4 hh + r) and + 8, the order the score
      // registers hold the rows in).
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int rows = h * 32 * 2 * D + st * ROW16;
#pragma unroll
        for (int c = 0; c < NDB; ++c) {
          const bf16x8 ag = cat8(lds_read_tr4(reinterpret_cast<const bf16*>(Gt + rows + toff[0][c])),
                                 lds_read_tr4(reinterpret_cast<const bf16*>(Gt + rows + toff[1][c])));
          const bf16x8 aq = cat8(lds_read_tr4(reinterpret_cast<const bf16*>(Qt + rows + toff[0][c])),
                                 lds_read_tr4(reinterpret_cast<const bf16*>(Qt + rows + toff[1][c])));
          dva[c] = mfma32(ag, pb[st], dva[c]);
          dka[c] = mfma32(aq, dsb[st], dka[c]);
        }
      }
    }
    }
    if (more) store_rowvals(buf ^ 1);
    wait_vmcnt<0>();
    __syncthreads();
    cur = nxt;
    advance(nxt);
  }

  // Without SPLIT: dK = scale * dK^T sums, dV = dV^T sums, rounded to bf16;
  // lane (key, hh) holds d = 32c + 8g + 4hh + u.  Keys no query attends
  // hold exact zeros (every product added 0).
  if (key < p.mask.frozen) {   // a frozen key: written as exact zeros
#pragma unroll
    for (int c = 0; c < NDB; ++c) {
      dka[c] = f32x16{};
      dva[c] = f32x16{};
    }
  }
  if (!SPLIT) {
    if (key < nkeys) {
      bf16* DK = static_cast<bf16*>(const_cast<void*>(p.dk.ptr)) + b * p.dk.sb + hk * p.dk.sh + (int64_t)key * p.dk.ss;
      bf16* DV = static_cast<bf16*>(const_cast<void*>(p.dv.ptr)) + b * p.dv.sb + hk * p.dv.sh + (int64_t)key * p.dv.ss;
      const float sc = p.scale;
#pragma unroll
      for (int c = 0; c < NDB; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * c + 8 * g + 4 * hh;
          if (32 * c + 8 * g >= D) continue;   // rows d >= D of the block (D = 16)
          *reinterpret_cast<bf16x4*>(DK + d) = to_bf16x4(dka[c][4 * g] * sc, dka[c][4 * g + 1] * sc,
                                                         dka[c][4 * g + 2] * sc, dka[c][4 * g + 3] * sc);
          *reinterpret_cast<bf16x4*>(DV + d) = to_bf16x4(dva[c][4 * g], dva[c][4 * g + 1], dva[c][4 * g + 2],
                                                         dva[c][4 * g + 3]);
        }
    }
    return;
  }
  // This half's sums dK^T / dV^T as float32 rows of the workspace (unscaled);
  // lane (key, hh) holds d = 32c + 8g + 4hh + u.
  if (key < nkeys) {
    const int64_t n = (int64_t)p.B * p.Hkv * nkeys * D;
    const int64_t row = ((int64_t)bh * nkeys + key) * D;
    float* PK = p.dkv_part + (int64_t)half * 2 * n + row;
    float* PV = PK + n;
#pragma unroll
    for (int c = 0; c < NDB; ++c)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * c + 8 * g + 4 * hh;
        if (32 * c + 8 * g >= D) continue;   // rows d >= D of the block (D = 16)
        *reinterpret_cast<f32x4*>(PK + d) = f32x4{dka[c][4 * g], dka[c][4 * g + 1], dka[c][4 * g + 2], dka[c][4 * g + 3]};
        *reinterpret_cast<f32x4*>(PV + d) = f32x4{dva[c][4 * g], dva[c][4 * g + 1], dva[c][4 * g + 2], dva[c][4 * g + 3]};
      }
  }
}

// At D = 64 (without a key bias) the kernel fits 170 registers, so three
// waves share a SIMD: three 4-wave workgroups (49 KB of LDS each) per compute
// unit.  With a bias the extra registers would spill there.
template <int D, int MK, bool SPLIT, bool BIAS>
__global__ void __launch_bounds__(KvSplit<D>::NW * 64, D == 64 && !BIAS ? 3 : 2)
dkdv_split_kernel(Params p) {
  dkdv_split_body<D, MK, SPLIT, BIAS>(p, blockIdx.x);
}

// The two gradient kernels in one launch (dQ with the dK/dV kernel's wave
// count): blocks
// [0, nkv) are dkdv_split_kernel's workgroups, blocks [nkv_pad, gridDim) the
// dQ kernel's (nkv_pad is nkv rounded up to a multiple of 8, so the dQ blocks
// keep their XCD placement; the blocks in between do nothing).  Each block
// computes exactly what it computes in its own kernel, so the results are
// bitwise those of the two launches in turn; as the dK/dV workgroups drain,
// dQ workgroups take over their compute units instead of leaving them idle
// until the dK/dV launch ends.
template <int D, int MKKV, bool SPLIT, int MKQ, bool BIAS>
__global__ void __launch_bounds__(KvSplit<D>::NW * 64, 2)
grads_kernel(Params p, int nkv, int nkv_pad) {
  const int bid = blockIdx.x;
  if (bid < nkv_pad) {
    if (bid < nkv) dkdv_split_body<D, MKKV, SPLIT, BIAS>(p, bid);
    return;
  }
  dq_dma_body<D, KvSplit<D>::NW, MKQ, BIAS>(p, bid - nkv_pad);
}

// dK = scale * (half 0 + half 1), dV = half 0 + half 1, rounded to bf16; 8
// consecutive d of one key per thread.
template <int D>
__global__ void __launch_bounds__(256) dkdv_reduce_kernel(Params p) {
  const int nkeys = walk_keys(p);
  const int64_t n = (int64_t)p.B * p.Hkv * nkeys * D;
  const int64_t i8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i8 >= n) return;
  const int64_t row = i8 / D;
  const int d = (int)(i8 % D);
  const int key = (int)(row % nkeys);
  const int bh = (int)(row / nkeys);
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const float* P = p.dkv_part + i8;
  bf16* DK = static_cast<bf16*>(const_cast<void*>(p.dk.ptr)) + b * p.dk.sb + hk * p.dk.sh + (int64_t)key * p.dk.ss + d;
  bf16* DV = static_cast<bf16*>(const_cast<void*>(p.dv.ptr)) + b * p.dv.sb + hk * p.dv.sh + (int64_t)key * p.dv.ss + d;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(P + t * n);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(P + t * n + 4);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(P + 2 * n + t * n);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(P + 2 * n + t * n + 4);
    const float sc = t == 0 ? p.scale : 1.0f;
    const bf16x8 o = cat8(to_bf16x4((a0[0] + b0[0]) * sc, (a0[1] + b0[1]) * sc, (a0[2] + b0[2]) * sc, (a0[3] + b0[3]) * sc),
                          to_bf16x4((a1[0] + b1[0]) * sc, (a1[1] + b1[1]) * sc, (a1[2] + b1[2]) * sc, (a1[3] + b1[3]) * sc));
    *reinterpret_cast<bf16x8*>(t == 0 ? DK : DV) = o;
  }
}

// dK/dV of the TTT keys past step 0.  Key j = s*L + r (s >= 1, L = Sq)
// meets one query row, r, in each head of its group (when r < kv_valid):
//   dV_j = sum_h P_h dO_hr,  dK_j = scale * sum_h dS_h Q_hr,
//   P_h = exp2(scale log2(e) q_hr.k_j - LSE_hr log2(e)),  dS_h = P_h (dO_hr.v_j - Delta_hr),
// the heads summed in order (bitwise reproducible).  D/8 lanes per key, eight
// consecutive d each, the two dot products summed over the key's lanes by a
// butterfly (every lane ends with the same sum).  Consecutive key groups take
// the later steps of one row r, so its Q and dO rows are read together.
// Keys whose row is not below kv_valid get exact zeros.
template <int D>
__global__ void __launch_bounds__(256) ttt_dkdv_kernel(Params p) {
  constexpr int LPK = D / 8, KPB = 256 / LPK;
  const int L = p.Sq, nlate = p.Skv - p.Sq, nst = p.Skv / p.Sq - 1;
  const int64_t g = (int64_t)blockIdx.x * KPB + threadIdx.x / LPK;
  if (g >= (int64_t)p.B * p.Hkv * nlate) return;   // whole key groups leave together
  const int sub = threadIdx.x % LPK;
  const int bh = (int)(g / nlate), idx = (int)(g % nlate);
  const int r = idx / nst, j = (1 + idx % nst) * L + r;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const MaskB m = resolve_mask(p, b);
  const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.k.ptr) + b * p.k.sb +
                                                     hk * p.k.sh + (int64_t)j * p.k.ss + 8 * sub);
  const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.v.ptr) + b * p.v.sb +
                                                     hk * p.v.sh + (int64_t)j * p.v.ss + 8 * sub);
  float dk[8] = {}, dv[8] = {};
  const float kbias = p.bias_s ? p.bias_s[(int64_t)b * p.vt_ss + j] : 0.f;
  if (r < m.kvv) {
    for (int h = 0; h < p.G; ++h) {
      const int hq = hk * p.G + h;
      const bf16x8 q8 = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.q.ptr) + b * p.q.sb +
                                                         hq * p.q.sh + (int64_t)r * p.q.ss + 8 * sub);
      const bf16x8 g8 = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(p.dout.ptr) + b * p.dout.sb +
                                                         hq * p.dout.sh + (int64_t)r * p.dout.ss + 8 * sub);
      const int64_t row = ((int64_t)b * p.Hq + hq) * p.Sq + r;
      float sd = dot_bf16x8(q8, k8, 0.f), pd = dot_bf16x8(g8, v8, 0.f);
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1) {
        sd += __shfl_xor(sd, o, LPK);
        pd += __shfl_xor(pd, o, LPK);
      }
      const float pr = exp2_fast((sd + kbias) * p.scale_log2 - p.lse2[row]);
      const float ds = pr * (pd - p.delta[row]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dv[e] += pr * (float)g8[e];
        dk[e] += ds * (float)q8[e];
      }
    }
  }
  bf16* DK = static_cast<bf16*>(const_cast<void*>(p.dk.ptr)) + b * p.dk.sb + hk * p.dk.sh + (int64_t)j * p.dk.ss + 8 * sub;
  bf16* DV = static_cast<bf16*>(const_cast<void*>(p.dv.ptr)) + b * p.dv.sb + hk * p.dv.sh + (int64_t)j * p.dv.ss + 8 * sub;
  if (j < p.mask.frozen) {   // a frozen key: written as exact zeros
#pragma unroll
    for (int e = 0; e < 8; ++e) dk[e] = dv[e] = 0.f;
  }
  const float sc = p.scale;
  *reinterpret_cast<bf16x8*>(DK) = cat8(to_bf16x4(dk[0] * sc, dk[1] * sc, dk[2] * sc, dk[3] * sc),
                                        to_bf16x4(dk[4] * sc, dk[5] * sc, dk[6] * sc, dk[7] * sc));
  *reinterpret_cast<bf16x8*>(DV) = cat8(to_bf16x4(dv[0], dv[1], dv[2], dv[3]), to_bf16x4(dv[4], dv[5], dv[6], dv[7]));
}

template <typename K>
hipError_t set_lds(K k, int bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// After the dK/dV products of the step-0 keys: the reduction of the two
// halves' partial sums (split blocks) and, under TTT, the later steps' keys.
template <int D>
hipError_t launch_dkdv_rest(const Params& p, bool split, hipStream_t stream) {
  hipError_t e;
  const int nkeys = walk_keys(p);
  if (split) {
    const int64_t n8 = (int64_t)p.B * p.Hkv * nkeys * D / 8;
    hipLaunchKernelGGL(dkdv_reduce_kernel<D>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t nlate = (int64_t)p.B * p.Hkv * (p.Skv - nkeys);
  if (p.mask.kind == MASK_TTT && nlate > 0) {
    constexpr int KPB = 256 / (D / 8);
    hipLaunchKernelGGL(ttt_dkdv_kernel<D>, dim3((unsigned)((nlate + KPB - 1) / KPB)), dim3(256), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// dK/dV and dQ as one grads_kernel launch (workgroups of the dK/dV kernel's
// size: 8 waves at D = 128, 4 at D <= 64, where only split key blocks take
// it), when there are enough query rows for 8-wave dQ workgroups and both
// have work; sets `done`.  Otherwise leaves `done` false and launches
// nothing.
template <int D>
hipError_t launch_grads(const Params& p, hipStream_t stream, bool& done) {
  done = false;
  {
    using LD = KvSplit<D>;
    const int nkeys = walk_keys(p);
    const int64_t wg8 = (int64_t)p.B * p.Hq * ((p.Sq + 255) / 256);
    const int64_t ndq = (int64_t)p.B * p.Hq * ((p.Sq + LD::NW * 32 - 1) / (LD::NW * 32));
    const bool split = dkdv_split(p.B, p.Hkv, nkeys);
    const int64_t nkv = (int64_t)p.B * p.Hkv * (split ? 2 : 1) * ((nkeys + LD::TKW - 1) / LD::TKW);
    if (wg8 < 512 || nkv == 0) return hipSuccess;
    // D <= 64: only split key blocks (few of them, long dK/dV tails) gain from
    // sharing the launch with dQ; with many blocks the 8-wave dQ launched on
    // its own is faster than the 4-wave dQ the merged launch would take
    if (D <= 64 && !split) return hipSuccess;
    const int64_t nkv_pad = (nkv + 7) / 8 * 8;
    if (nkv_pad + ndq > INT_MAX) return hipSuccess;
    const int mk = mask_instance(p.mask.kind);
    auto pick = [&](auto bc) {
      constexpr bool BI = decltype(bc)::value;
      return mk == MK_WIN ? (split ? grads_kernel<D, MK_WIN, true, MK_WIN, BI> : grads_kernel<D, MK_WIN, false, MK_WIN, BI>)
           : mk == MK_TTT ? (split ? grads_kernel<D, MK_FC, true, MK_TTT, BI> : grads_kernel<D, MK_FC, false, MK_TTT, BI>)
                          : (split ? grads_kernel<D, MK_FC, true, MK_FC, BI> : grads_kernel<D, MK_FC, false, MK_FC, BI>);
    };
    auto k = p.bias_s ? pick(std::true_type{}) : pick(std::false_type{});
    const int lq = DqDma<D>::BYTES + (p.bias_s ? DqDma<D>::BIAS_BYTES : 0);
    const int lds = LD::BYTES > lq ? LD::BYTES : lq;
    hipError_t e;
    if ((e = set_lds(k, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)(nkv_pad + ndq)), dim3(LD::NW * 64), lds, stream, p, (int)nkv, (int)nkv_pad);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    done = true;
    return launch_dkdv_rest<D>(p, split, stream);
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_stage(const Params& p, int stage, hipStream_t stream) {
  hipError_t e;
  if (stage == STAGE_GRADS) {
    bool done = false;
    if ((e = launch_grads<D>(p, stream, done)) != hipSuccess || done) return e;
    if ((e = launch_stage<D>(p, STAGE_DKDV, stream)) != hipSuccess) return e;
    return launch_stage<D>(p, STAGE_DQ, stream);
  }
  const int64_t rows = (int64_t)p.B * p.Hq * p.Sq;
  if (stage == STAGE_DELTA && rows > 0) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL(delta_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the scaled key bias the dK/dV and dQ stages start their scores from
  if (stage == STAGE_DELTA && (e = launch_bias_scale(p, stream)) != hipSuccess) return e;
  if (stage == STAGE_DKDV) {
    using LD = KvSplit<D>;
    const int nkeys = walk_keys(p);
    const bool split = dkdv_split(p.B, p.Hkv, nkeys);
    const int64_t nblk = (int64_t)p.B * p.Hkv * (split ? 2 : 1) * ((nkeys + LD::TKW - 1) / LD::TKW);
    if (nblk > 0) {
      const bool win = p.mask.kind == MASK_WINDOW;
      auto pick = [&](auto bc) {
        constexpr bool BI = decltype(bc)::value;
        return split ? (win ? dkdv_split_kernel<D, MK_WIN, true, BI> : dkdv_split_kernel<D, MK_FC, true, BI>)
                     : (win ? dkdv_split_kernel<D, MK_WIN, false, BI> : dkdv_split_kernel<D, MK_FC, false, BI>);
      };
      auto k = p.bias_s ? pick(std::true_type{}) : pick(std::false_type{});
      if ((e = set_lds(k, LD::BYTES)) != hipSuccess) return e;
      hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(LD::NW * 64), LD::BYTES, stream, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if ((e = launch_dkdv_rest<D>(p, split, stream)) != hipSuccess) return e;
    } else if ((e = launch_dkdv_rest<D>(p, false, stream)) != hipSuccess) {
      return e;
    }
  }
  if (stage == STAGE_DQ && p.B > 0 && p.Sq > 0) {
    // 8-wave workgroups when there are enough to fill the chip twice over,
    // except at D = 64, and at D <= 32 under a causal, TTT or window mask:
    // there workgroups carry unequal work and 4-wave ones (several per
    // compute unit, as in the forward) balance it better; at D = 64 three of
    // them share a compute unit (the 48 KB ring), under FULL too.  At D <= 32
    // under FULL every workgroup is alike and the 8-wave one was faster.
    // Each wave's rows get the same arithmetic in either size, so results do
    // not depend on it (the one-launch backward's dQ blocks take the dK/dV
    // kernel's size).
    const bool small = D == 64 || (D <= 32 && p.mask.kind != MASK_FULL);
    const int64_t wg8 = small ? 0 : (int64_t)p.B * p.Hq * ((p.Sq + 255) / 256);
    const int mk = mask_instance(p.mask.kind);
    auto pick = [&](auto bc) {
      constexpr bool BI = decltype(bc)::value;
      return wg8 >= 512 ? (mk == MK_TTT ? dq_dma_kernel<D, 8, MK_TTT, BI>
                                        : (mk == MK_WIN ? dq_dma_kernel<D, 8, MK_WIN, BI> : dq_dma_kernel<D, 8, MK_FC, BI>))
                        : (mk == MK_TTT ? dq_dma_kernel<D, 4, MK_TTT, BI>
                                        : (mk == MK_WIN ? dq_dma_kernel<D, 4, MK_WIN, BI> : dq_dma_kernel<D, 4, MK_FC, BI>));
    };
    auto k = p.bias_s ? pick(std::true_type{}) : pick(std::false_type{});
    const int nw = wg8 >= 512 ? 8 : 4;
    const int64_t nblk = (int64_t)p.B * p.Hq * ((p.Sq + nw * 32 - 1) / (nw * 32));
    const int lds = DqDma<D>::BYTES + (p.bias_s ? DqDma<D>::BIAS_BYTES : 0);
    if ((e = set_lds(k, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(nw * 64), lds, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_bf16(const Params& p, int stage, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_stage<16>(p, stage, s);
    case 32: return launch_stage<32>(p, stage, s);
    case 64: return launch_stage<64>(p, stage, s);
    case 128: return launch_stage<128>(p, stage, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
