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
// Work split.  A workgroup owns NW*QB*32 query rows of one (batch, head); each
// wave owns QB blocks of 32 rows.  Keys stream through LDS in tiles of 64,
// double-buffered: tile t+1 is fetched into registers while tile t is used.
// Scores are computed transposed, S^T = K Q^T, so each lane owns one query
// column and 16 keys of it: the row max and row sum are in-lane reductions
// plus one cross-half swap, and the softmax scale, max and normaliser are one
// scalar per lane.  O^T = V^T P^T then takes P straight from the score
// registers (the key order inside each 16-key MFMA step is permuted the same
// way in both operands) and V^T straight from the row-major V tile with the
// transposing LDS read.
#include "fa_device.h"

namespace fa {
namespace {

constexpr int TK = 64;  // keys per LDS tile

template <int D>
struct FwdLds {
  static constexpr int KSTR = D + 8;                     // K row stride (elements)
  static constexpr int VSTR = D >= 64 ? D + 32 : D;      // V row stride (elements)
  static constexpr int KTILE = TK * KSTR;
  static constexpr int VTILE = TK * VSTR;
  static constexpr int BYTES = 2 * (KTILE + VTILE) * 2;  // two buffers, bf16
};

template <int D, int QB, int NW>
__global__ void __launch_bounds__(NW * 64)
fwd_kernel(Params p) {
  constexpr int NT = NW * 64;
  constexpr int TQ = NW * QB * 32;
  constexpr int DC = D / 8;                  // 16-byte chunks per row
  constexpr int CHUNKS = TK * DC;            // chunks per K (or V) tile
  constexpr int PER_T = (CHUNKS + NT - 1) / NT;
  constexpr int NDB = D >= 32 ? D / 32 : 1;  // 32-wide d blocks of O^T
  constexpr int NJ = D / 16;                 // 16-wide d steps of S^T
  using L = FwdLds<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* Ks = reinterpret_cast<bf16*>(smem);
  bf16* Vs = Ks + 2 * L::KTILE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  const int nq = (p.Sq + TQ - 1) / TQ;
  int col, rank;
  map_block(blockIdx.x, p.B * p.Hq, nq, col, rank);
  const int b = col / p.Hq, h = col % p.Hq, hk = h / p.G;
  const int qtile = p.mask.kind == MASK_FULL ? rank : nq - 1 - rank;
  const MaskB m = resolve_mask(p, b);

  const int qa = qtile * TQ, qb = min(p.Sq, qa + TQ);
  const int wa = qa + wave * QB * 32, wb = min(p.Sq, wa + QB * 32);

  const bf16* Qg = static_cast<const bf16*>(p.q.ptr) + b * p.q.sb + h * p.q.sh;
  const bf16* Kg = static_cast<const bf16*>(p.k.ptr) + b * p.k.sb + hk * p.k.sh;
  const bf16* Vg = static_cast<const bf16*>(p.v.ptr) + b * p.v.sb + hk * p.v.sh;

  // Q^T as the B operand: lane (q = l32, half hh) holds Q[q][16j + 8hh .. +8].
  bf16x8 qreg[QB][NJ];
#pragma unroll
  for (int qb_ = 0; qb_ < QB; ++qb_) {
    const int row = wa + qb_ * 32 + l32;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (row < p.Sq)
        qreg[qb_][j] = *reinterpret_cast<const bf16x8*>(Qg + (int64_t)row * p.q.ss + 16 * j + 8 * hh);
      else
        qreg[qb_][j] = bf16x8{};
    }
  }

  f32x16 acc[QB][NDB];
  float mrun[QB], lsum[QB];
#pragma unroll
  for (int qb_ = 0; qb_ < QB; ++qb_) {
    mrun[qb_] = kMaxInit;
    lsum[qb_] = 0.f;
#pragma unroll
    for (int c = 0; c < NDB; ++c) acc[qb_][c] = f32x16{};
  }

  // Stage one key tile into registers (zero rows for keys that are not real).
  i32x4 kst[PER_T], vst[PER_T];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + i * NT;
      const int r = c / DC, c8 = c % DC;
      const int key = t * TK + r;
      if (c < CHUNKS && key_valid(m, key)) {
        kst[i] = *reinterpret_cast<const i32x4*>(Kg + (int64_t)key * p.k.ss + 8 * c8);
        vst[i] = *reinterpret_cast<const i32x4*>(Vg + (int64_t)key * p.v.ss + 8 * c8);
      } else {
        kst[i] = i32x4{};
        vst[i] = i32x4{};
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + i * NT;
      if (c < CHUNKS) {
        const int r = c / DC, c8 = c % DC;
        lds_write16(Ks + buf * L::KTILE + r * L::KSTR + 8 * c8, kst[i]);
        lds_write16(Vs + buf * L::VTILE + r * L::VSTR + 8 * c8, vst[i]);
      }
    }
  };

  TileWalk walk;
  walk.start(m, qa, qb, TK);
  int buf = 0;
  if (walk.valid()) {
    fetch(walk.t);
    store(0);
  }
  __syncthreads();

  // Per-lane addressing inside a tile.
  const int tr_row = (lane & 15) >> 2;                 // row offset within a 4-key run
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const bool d_lane_ok = D >= 32 || ((lane >> 4) & 1) == 0;

  while (walk.valid()) {
    const int t = walk.t;
    TileWalk nxt = walk;
    nxt.next(m, qa, qb, TK);
    if (nxt.valid()) fetch(nxt.t);

    const int k0 = t * TK;
    const int state = tile_state(m, k0, TK, wa, wb);
    if (state != TILE_SKIP) {
      const bf16* Kt = Ks + buf * L::KTILE;
      const bf16* Vt = Vs + buf * L::VTILE;
      // S^T = K Q^T : 2 key blocks of 32, QB query blocks.
      f32x16 s[QB][2];
#pragma unroll
      for (int qb_ = 0; qb_ < QB; ++qb_) { s[qb_][0] = f32x16{}; s[qb_][1] = f32x16{}; }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = lds_read8(Kt + (32 * kb + l32) * L::KSTR + 16 * j + 8 * hh);
#pragma unroll
          for (int qb_ = 0; qb_ < QB; ++qb_) s[qb_][kb] = mfma32(a, qreg[qb_][j], s[qb_][kb]);
        }
      }
      if (state == TILE_PART) {
#pragma unroll
        for (int qb_ = 0; qb_ < QB; ++qb_) {
          const int qi = wa + qb_ * 32 + l32;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
              if (!allowed(m, qi, key)) s[qb_][kb][i] = -INFINITY;
            }
        }
      }
      // Online softmax, lazily rescaled.
      bf16x8 pb[QB][2][2];
#pragma unroll
      for (int qb_ = 0; qb_ < QB; ++qb_) {
        float mx = s[qb_][0][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[qb_][0][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[qb_][1][i]);
        mx = half_swap_max(mx) * p.scale_log2;
        if (__any(mx > mrun[qb_] + kRescaleSlack)) {
          const float mn = fmaxf(mrun[qb_], mx);
          const float alpha = exp2_fast(mrun[qb_] - mn);
          mrun[qb_] = mn;
          lsum[qb_] *= alpha;
#pragma unroll
          for (int c = 0; c < NDB; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[qb_][c][i] *= alpha;
        }
        const float mcur = mrun[qb_];
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            float e[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              e[u] = exp2_fast(s[qb_][kb][8 * st + u] * p.scale_log2 - mcur);
              ls += e[u];
            }
            const bf16x4 lo = to_bf16x4(e[0], e[1], e[2], e[3]);
            const bf16x4 hi = to_bf16x4(e[4], e[5], e[6], e[7]);
            pb[qb_][kb][st] = cat8(lo, hi);
          }
        lsum[qb_] += ls;
      }
      // O^T += V^T P^T.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int kbase = 32 * kb + 16 * st + 4 * hh + tr_row;
#pragma unroll
          for (int c = 0; c < NDB; ++c) {
            const int dcol = (D >= 32 ? 32 * c + tr_col : (tr_col & 15));
            bf16x8 a = cat8(lds_read_tr4(Vt + kbase * L::VSTR + dcol),
                            lds_read_tr4(Vt + (kbase + 8) * L::VSTR + dcol));
            if (!d_lane_ok) a = bf16x8{};
#pragma unroll
            for (int qb_ = 0; qb_ < QB; ++qb_) acc[qb_][c] = mfma32(a, pb[qb_][kb][st], acc[qb_][c]);
          }
        }
    }

    if (nxt.valid()) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    walk = nxt;
  }

  // Epilogue: O = acc / l, LSE = ln(sum exp(scaled scores)); empty rows -> 0.
  bf16* Og = static_cast<bf16*>(const_cast<void*>(p.o.ptr)) + b * p.o.sb + h * p.o.sh;
  float* Lg = p.lse + ((int64_t)b * p.Hq + h) * p.Sq;
#pragma unroll
  for (int qb_ = 0; qb_ < QB; ++qb_) {
    const int row = wa + qb_ * 32 + l32;
    const float lt = half_swap_sum(lsum[qb_]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    if (row < p.Sq) {
      if (hh == 0) Lg[row] = lt > 0.f ? (mrun[qb_] + log2_fast(lt)) * kLn2 : 0.f;
#pragma unroll
      for (int c = 0; c < NDB; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * c + 8 * g + 4 * hh;
          if (d < D) {
            const bf16x4 o = to_bf16x4(acc[qb_][c][4 * g] * inv, acc[qb_][c][4 * g + 1] * inv,
                                       acc[qb_][c][4 * g + 2] * inv, acc[qb_][c][4 * g + 3] * inv);
            *reinterpret_cast<bf16x4*>(Og + (int64_t)row * p.o.ss + d) = o;
          }
        }
    }
  }
}

template <int D, int QB, int NW>
hipError_t launch(const Params& p, hipStream_t stream) {
  constexpr int TQ = NW * QB * 32;
  const int nq = (p.Sq + TQ - 1) / TQ;
  const int64_t nblk = (int64_t)p.B * p.Hq * nq;
  if (nblk == 0) return hipSuccess;
  const int lds = FwdLds<D>::BYTES;
  auto k = fwd_kernel<D, QB, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(NW * 64), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const Params& p, hipStream_t s) {
  switch (p.D) {
    case 16: return launch<16, 2, 4>(p, s);
    case 32: return launch<32, 2, 4>(p, s);
    case 64: return launch<64, 2, 4>(p, s);
    case 128: return launch<128, 1, 8>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
