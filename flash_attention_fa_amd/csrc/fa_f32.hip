// fa_f32.hip - float32 forward and backward attention (the FA_F32 instance).
//
// Same mathematics, masks and saved state as the bf16 kernels (see
// fa_fwd.hip / fa_bwd.hip), computed in float32 end to end for callers that
// need fp32 accuracy (max abs error ~1e-6 against an exact reference, the
// strict-f32 mode of the ggml flash-attn-training playbook, section 1).
// One thread owns one query row (forward, dQ) or one key row (dK/dV); tiles
// of the other operand stream through LDS.  These are plain FMA kernels: the
// fp32 instance exists for accuracy, the bf16 MFMA kernels for speed.
#include "fa_device.h"

namespace fa {
namespace {

constexpr int F_ROWS = 64;  // rows per workgroup (one wave)
constexpr int F_TK = 32;    // keys (or queries) per LDS tile

template <int D>
__device__ __forceinline__ void load_rows(float* dst, const float* src, int64_t ss, int r0, int n,
                                          int rows_valid_end, const MaskB* mk, bool key_rows) {
  // Cooperative copy of n rows [r0, r0 + n) into LDS, zeros for rows that are
  // out of range (or not real keys when key_rows).
  for (int c = threadIdx.x; c < n * (D / 4); c += F_ROWS) {
    const int r = c / (D / 4), c4 = c % (D / 4);
    const int row = r0 + r;
    bool ok = row < rows_valid_end;
    if (key_rows && ok) ok = key_valid(*mk, row);
    f32x4 v = ok ? *reinterpret_cast<const f32x4*>(src + (int64_t)row * ss + 4 * c4) : f32x4{};
    *reinterpret_cast<f32x4*>(dst + r * D + 4 * c4) = v;
  }
}

template <int D>
__global__ void __launch_bounds__(F_ROWS) fwd_f32_kernel(Params p) {
  extern __shared__ __align__(16) float fsm[];
  float* Ks = fsm;
  float* Vs = Ks + F_TK * D;
  float* Qs = Vs + F_TK * D;
  const int nq = (p.Sq + F_ROWS - 1) / F_ROWS;
  const int qtile = blockIdx.x % nq;
  const int col = blockIdx.x / nq;
  const int b = col / p.Hq, h = col % p.Hq, hk = h / p.G;
  const MaskB m = resolve_mask(p, b);
  const int qa = qtile * F_ROWS, qb = min(p.Sq, qa + F_ROWS);
  const int i = qa + threadIdx.x;
  const float* Qg = static_cast<const float*>(p.q.ptr) + b * p.q.sb + h * p.q.sh;
  const float* Kg = static_cast<const float*>(p.k.ptr) + b * p.k.sb + hk * p.k.sh;
  const float* Vg = static_cast<const float*>(p.v.ptr) + b * p.v.sb + hk * p.v.sh;
  load_rows<D>(Qs, Qg, p.q.ss, qa, F_ROWS, p.Sq, &m, false);
  const float* Bg = p.mask.bias ? p.mask.bias + (int64_t)b * p.mask.bias_sb : nullptr;

  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float mrun = -INFINITY, l = 0.f;

  TileWalk walk;
  walk.start(m, qa, qb, F_TK);
  while (walk.valid()) {
    const int k0 = walk.t * F_TK;
    __syncthreads();
    load_rows<D>(Ks, Kg, p.k.ss, k0, F_TK, p.Skv, &m, true);
    load_rows<D>(Vs, Vg, p.v.ss, k0, F_TK, p.Skv, &m, true);
    __syncthreads();
    float sc[F_TK];
    float mt = -INFINITY;
    for (int j = 0; j < F_TK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(Qs[threadIdx.x * D + d], Ks[j * D + d], dot);
      const bool ok = allowed(m, i, k0 + j) && k0 + j < p.Skv;
      sc[j] = ok ? dot * p.scale_log2 + (Bg ? Bg[k0 + j] * kLog2e : 0.f) : -INFINITY;
      mt = fmaxf(mt, sc[j]);
    }
    const float mn = fmaxf(mrun, mt);
    if (mn > -INFINITY) {
      const float corr = mrun > -INFINITY ? exp2_fast(mrun - mn) : 0.f;
      l *= corr;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= corr;
      for (int j = 0; j < F_TK; ++j) {
        const float pj = exp2_fast(sc[j] - mn);
        l += pj;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(pj, Vs[j * D + d], o[d]);
      }
      mrun = mn;
    }
    walk.next(m, qa, qb, F_TK);
  }
  if (i < p.Sq) {
    float* Og = static_cast<float*>(const_cast<void*>(p.o.ptr)) + b * p.o.sb + h * p.o.sh + (int64_t)i * p.o.ss;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) Og[d] = o[d] * inv;
    p.lse[((int64_t)b * p.Hq + h) * p.Sq + i] = l > 0.f ? (mrun + log2_fast(l)) * kLn2 : 0.f;
  }
}

// Delta_i = sum_d dO_id O_id, one thread per row.
template <int D>
__global__ void __launch_bounds__(256) delta_f32_kernel(Params p) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= (int64_t)p.B * p.Hq * p.Sq) return;
  const int i = (int)(r % p.Sq);
  const int64_t bh = r / p.Sq;
  const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
  const float* orow = static_cast<const float*>(p.o.ptr) + b * p.o.sb + h * p.o.sh + (int64_t)i * p.o.ss;
  const float* grow = static_cast<const float*>(p.dout.ptr) + b * p.dout.sb + h * p.dout.sh + (int64_t)i * p.dout.ss;
  float acc = 0.f;
  for (int d = 0; d < D; ++d) acc = fmaf(orow[d], grow[d], acc);
  p.delta[r] = acc;
  p.lse2[r] = p.lse_in[r] * 1.4426950408889634f;
}

template <int D>
__global__ void __launch_bounds__(F_ROWS) dq_f32_kernel(Params p) {
  extern __shared__ __align__(16) float fsm[];
  float* Ks = fsm;
  float* Vs = Ks + F_TK * D;
  float* Qs = Vs + F_TK * D;
  float* Gs = Qs + F_ROWS * D;
  const int nq = (p.Sq + F_ROWS - 1) / F_ROWS;
  const int qtile = blockIdx.x % nq;
  const int col = blockIdx.x / nq;
  const int b = col / p.Hq, h = col % p.Hq, hk = h / p.G;
  const MaskB m = resolve_mask(p, b);
  const int qa = qtile * F_ROWS, qb = min(p.Sq, qa + F_ROWS);
  const int i = qa + threadIdx.x;
  const float* Qg = static_cast<const float*>(p.q.ptr) + b * p.q.sb + h * p.q.sh;
  const float* Gg = static_cast<const float*>(p.dout.ptr) + b * p.dout.sb + h * p.dout.sh;
  const float* Kg = static_cast<const float*>(p.k.ptr) + b * p.k.sb + hk * p.k.sh;
  const float* Vg = static_cast<const float*>(p.v.ptr) + b * p.v.sb + hk * p.v.sh;
  load_rows<D>(Qs, Qg, p.q.ss, qa, F_ROWS, p.Sq, &m, false);
  load_rows<D>(Gs, Gg, p.dout.ss, qa, F_ROWS, p.Sq, &m, false);
  const int64_t rb = ((int64_t)b * p.Hq + h) * p.Sq;
  const float* Bg = p.mask.bias ? p.mask.bias + (int64_t)b * p.mask.bias_sb : nullptr;
  float lse2 = 0.f, delta = 0.f;
  if (i < p.Sq) {
    lse2 = p.lse_in[rb + i] * 1.4426950408889634f;
    delta = p.delta[rb + i];
  }
  float dq[D];
#pragma unroll
  for (int d = 0; d < D; ++d) dq[d] = 0.f;
  TileWalk walk;
  walk.start(m, qa, qb, F_TK);
  while (walk.valid()) {
    const int k0 = walk.t * F_TK;
    __syncthreads();
    load_rows<D>(Ks, Kg, p.k.ss, k0, F_TK, p.Skv, &m, true);
    load_rows<D>(Vs, Vg, p.v.ss, k0, F_TK, p.Skv, &m, true);
    __syncthreads();
    for (int j = 0; j < F_TK; ++j) {
      if (!(allowed(m, i, k0 + j) && k0 + j < p.Skv)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(Qs[threadIdx.x * D + d], Ks[j * D + d], s);
        dp = fmaf(Gs[threadIdx.x * D + d], Vs[j * D + d], dp);
      }
      const float pr = exp2_fast(s * p.scale_log2 + (Bg ? Bg[k0 + j] * kLog2e : 0.f) - lse2);
      const float ds = pr * (dp - delta);
#pragma unroll
      for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, Ks[j * D + d], dq[d]);
    }
    walk.next(m, qa, qb, F_TK);
  }
  if (i < p.Sq) {
    float* Dg = static_cast<float*>(const_cast<void*>(p.dq.ptr)) + b * p.dq.sb + h * p.dq.sh + (int64_t)i * p.dq.ss;
#pragma unroll
    for (int d = 0; d < D; ++d) Dg[d] = dq[d] * p.scale;
  }
}

template <int D>
__global__ void __launch_bounds__(F_ROWS) dkdv_f32_kernel(Params p) {
  extern __shared__ __align__(16) float fsm[];
  float* Qs = fsm;
  float* Gs = Qs + F_TK * D;
  float* Ks = Gs + F_TK * D;
  float* Vs = Ks + F_ROWS * D;
  float* Ls = Vs + F_ROWS * D;
  float* Ds = Ls + F_TK;
  const int nk = (p.Skv + F_ROWS - 1) / F_ROWS;
  const int ktile = blockIdx.x % nk;
  const int col = blockIdx.x / nk;
  const int b = col / p.Hkv, hk = col % p.Hkv;
  const MaskB m = resolve_mask(p, b);
  const int ka = ktile * F_ROWS, kbnd = min(p.Skv, ka + F_ROWS);
  const int j = ka + threadIdx.x;
  const float* Kg = static_cast<const float*>(p.k.ptr) + b * p.k.sb + hk * p.k.sh;
  const float* Vg = static_cast<const float*>(p.v.ptr) + b * p.v.sb + hk * p.v.sh;
  load_rows<D>(Ks, Kg, p.k.ss, ka, F_ROWS, p.Skv, &m, true);
  load_rows<D>(Vs, Vg, p.v.ss, ka, F_ROWS, p.Skv, &m, true);
  float dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { dk[d] = 0.f; dv[d] = 0.f; }
  int qlo, qhi;
  query_hull(m, ka, kbnd, qlo, qhi);
  const bool real = j < p.Skv && key_valid(m, j);
  // this thread's key bias in log2 units (0 without one)
  const float kb2 = real && p.mask.bias ? p.mask.bias[(int64_t)b * p.mask.bias_sb + j] * kLog2e : 0.f;
  for (int hq = 0; hq < p.G; ++hq) {
    const int h = hk * p.G + hq;
    const float* Qg = static_cast<const float*>(p.q.ptr) + b * p.q.sb + h * p.q.sh;
    const float* Gg = static_cast<const float*>(p.dout.ptr) + b * p.dout.sb + h * p.dout.sh;
    const int64_t rb = ((int64_t)b * p.Hq + h) * p.Sq;
    for (int q0 = (qlo / F_TK) * F_TK; q0 < qhi; q0 += F_TK) {
      __syncthreads();
      load_rows<D>(Qs, Qg, p.q.ss, q0, F_TK, p.Sq, &m, false);
      load_rows<D>(Gs, Gg, p.dout.ss, q0, F_TK, p.Sq, &m, false);
      if (threadIdx.x < F_TK) {
        const int row = q0 + threadIdx.x;
        Ls[threadIdx.x] = row < p.Sq ? p.lse_in[rb + row] * 1.4426950408889634f : 0.f;
        Ds[threadIdx.x] = row < p.Sq ? p.delta[rb + row] : 0.f;
      }
      __syncthreads();
      if (!real) continue;
      for (int r = 0; r < F_TK; ++r) {
        const int i = q0 + r;
        if (i >= p.Sq || !allowed(m, i, j)) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          s = fmaf(Qs[r * D + d], Ks[threadIdx.x * D + d], s);
          dp = fmaf(Gs[r * D + d], Vs[threadIdx.x * D + d], dp);
        }
        const float pr = exp2_fast(s * p.scale_log2 + kb2 - Ls[r]);
        const float ds = pr * (dp - Ds[r]);
#pragma unroll
        for (int d = 0; d < D; ++d) {
          dv[d] = fmaf(pr, Gs[r * D + d], dv[d]);
          dk[d] = fmaf(ds, Qs[r * D + d], dk[d]);
        }
      }
    }
  }
  if (j < p.Skv) {
    float* DKg = static_cast<float*>(const_cast<void*>(p.dk.ptr)) + b * p.dk.sb + hk * p.dk.sh + (int64_t)j * p.dk.ss;
    float* DVg = static_cast<float*>(const_cast<void*>(p.dv.ptr)) + b * p.dv.sb + hk * p.dv.sh + (int64_t)j * p.dv.ss;
    const bool frozen = j < p.mask.frozen;   // written as exact zeros
#pragma unroll
    for (int d = 0; d < D; ++d) {
      DKg[d] = frozen ? 0.0f : dk[d] * p.scale;
      DVg[d] = frozen ? 0.0f : dv[d];
    }
  }
}

template <typename K>
hipError_t launch_dyn(K k, int64_t nblk, int lds, hipStream_t s, const Params& p) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3((unsigned)nblk), dim3(F_ROWS), lds, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t fwd_d(const Params& p, hipStream_t s) {
  const int64_t nblk = (int64_t)p.B * p.Hq * ((p.Sq + F_ROWS - 1) / F_ROWS);
  if (nblk == 0) return hipSuccess;
  return launch_dyn(fwd_f32_kernel<D>, nblk, (2 * F_TK + F_ROWS) * D * 4, s, p);
}

template <int D>
hipError_t bwd_d(const Params& p, int stage, hipStream_t s) {
  hipError_t e;
  const int64_t rows = (int64_t)p.B * p.Hq * p.Sq;
  if (stage == STAGE_DELTA && rows > 0) {
    hipLaunchKernelGGL(delta_f32_kernel<D>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t nq = (int64_t)p.B * p.Hq * ((p.Sq + F_ROWS - 1) / F_ROWS);
  if (stage == STAGE_DQ && nq > 0) {
    if ((e = launch_dyn(dq_f32_kernel<D>, nq, (2 * F_TK + 2 * F_ROWS) * D * 4, s, p)) != hipSuccess) return e;
  }
  const int64_t nk = (int64_t)p.B * p.Hkv * ((p.Skv + F_ROWS - 1) / F_ROWS);
  if (stage == STAGE_DKDV && nk > 0) {
    if ((e = launch_dyn(dkdv_f32_kernel<D>, nk, (2 * F_TK + 2 * F_ROWS) * D * 4 + 2 * F_TK * 4, s, p)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_fwd_f32(const Params& p, hipStream_t s) {
  switch (p.D) {
    case 16: return fwd_d<16>(p, s);
    case 32: return fwd_d<32>(p, s);
    case 64: return fwd_d<64>(p, s);
    case 128: return fwd_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_f32(const Params& p, int stage, hipStream_t s) {
  switch (p.D) {
    case 16: return bwd_d<16>(p, stage, s);
    case 32: return bwd_d<32>(p, stage, s);
    case 64: return bwd_d<64>(p, stage, s);
    case 128: return bwd_d<128>(p, stage, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
