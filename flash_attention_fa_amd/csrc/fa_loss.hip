// fa_loss.hip - soft-target log-softmax loss and its in-place gradient (fp32).
//
// The loss EAGLE3 training takes on the draft model's logits ("Flex Attention
// and Triton, Supporting Long Context Training in SpecForge", section
// In-place Gradient Calculation): for row i of N, with V logits x, soft
// targets t and mask weight w,
//   row_i = -w_i sum_v t_iv (x_iv - m_i - ln d_i),   loss = (1/N) sum_i row_i,
//   dloss/dx_iv = w_i / N (exp(x_iv - m_i) / d_i * tsum_i - t_iv),
// with m_i the row max, d_i = sum_v exp(x_iv - m_i) and tsum_i = sum_v t_iv.
//
// Both kernels are HBM-bound streams over the [N, V] matrices, one workgroup
// per row.  The forward reads x and t once: each thread keeps an online max
// and normaliser (the page's m and d) and the sums of t and t*x over its
// share of the row, so row_i = -w_i (sum t x - (m_i + ln d_i) tsum_i) needs
// no second pass.  The backward reads x and t once and writes the gradient
// over x.  Loads are 16 bytes per lane, consecutive lanes on consecutive
// chunks (rows that do not start on a 16-byte boundary take their first and
// last few elements one by one).  Row statistics are combined in a fixed tree (lanes by a butterfly,
// then the waves in order), and the mean is a separate one-workgroup sum in a
// fixed order, so reruns are bitwise identical.
#include <hip/hip_runtime.h>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kLossThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegHuge = -3.0e38f;   // finite start of the running max

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Online max / normaliser state of a share of a row: m is the max of the x
// seen (exact), d = sum exp(x - m), computed as 2^(x log2e - m log2e); st and
// sx are the sums of t and t * x.
struct RowStat {
  float m, d, st, sx;
};

__device__ __forceinline__ void add4(RowStat& r, const f32x4& x, const f32x4& t) {
  const float mn = fmaxf(r.m, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  const float mn2 = mn * kLog2e;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) s += exp2_hw(__builtin_fmaf(x[k], kLog2e, -mn2));
  r.d = __builtin_fmaf(r.d, exp2_hw((r.m - mn) * kLog2e), s);
  r.m = mn;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r.st += t[k];
    r.sx = __builtin_fmaf(t[k], x[k], r.sx);
  }
}

__device__ __forceinline__ void add1(RowStat& r, float x, float t) {
  const float mn = fmaxf(r.m, x);
  r.d = __builtin_fmaf(r.d, exp2_hw((r.m - mn) * kLog2e), exp2_hw(__builtin_fmaf(x, kLog2e, -mn * kLog2e)));
  r.m = mn;
  r.st += t;
  r.sx = __builtin_fmaf(t, x, r.sx);
}

__device__ __forceinline__ RowStat combine(const RowStat& a, const RowStat& b) {
  RowStat r;
  r.m = fmaxf(a.m, b.m);
  r.d = a.d * exp2_hw((a.m - r.m) * kLog2e) + b.d * exp2_hw((b.m - r.m) * kLog2e);
  r.st = a.st + b.st;
  r.sx = a.sx + b.sx;
  return r;
}

__device__ __forceinline__ RowStat shfl_xor(const RowStat& a, int off) {
  return RowStat{__shfl_xor(a.m, off), __shfl_xor(a.d, off), __shfl_xor(a.st, off), __shfl_xor(a.sx, off)};
}

// Walks one row of V floats of x and t with 16-byte loads where it can:
// the elements before x's first 16-byte boundary and after the last whole
// chunk go one by one (scalar(v)), the rest four at a time (vec(v), v a
// multiple of 4 past the head).  When t's row is aligned differently every
// element goes one by one.  Thread tid takes elements tid, tid + 256, ... of
// each part, so consecutive lanes read consecutive addresses.
template <typename Vec, typename Sca>
__device__ __forceinline__ void walk_row(const float* x, const float* t, int V, int tid, Vec vec, Sca sca) {
  const int hx = (int)((16 - (reinterpret_cast<uintptr_t>(x) & 15)) & 15) >> 2;
  const int ht = (int)((16 - (reinterpret_cast<uintptr_t>(t) & 15)) & 15) >> 2;
  if (hx != ht) {
    for (int v = tid; v < V; v += kLossThreads) sca(v);
    return;
  }
  const int h = hx < V ? hx : V;
  const int nc = (V - h) >> 2;
  if (tid < h) sca(tid);
#pragma unroll 4
  for (int c = tid; c < nc; c += kLossThreads) vec(h + 4 * c);
  const int v = h + 4 * nc + tid;
  if (v < V) sca(v);
}

__global__ void __launch_bounds__(kLossThreads) lsm_loss_fwd_kernel(LossParams p) {
  __shared__ RowStat part[kLossThreads / 64];
  const int i = blockIdx.x, tid = threadIdx.x;
  const float* x = p.x + (int64_t)i * p.x_ss;
  const float* t = p.t + (int64_t)i * p.t_ss;
  RowStat r{kNegHuge, 0.f, 0.f, 0.f};
  walk_row(
      x, t, p.V, tid,
      [&](int v) __attribute__((always_inline)) {
        add4(r, *reinterpret_cast<const f32x4*>(x + v), *reinterpret_cast<const f32x4*>(t + v));
      },
      [&](int v) __attribute__((always_inline)) { add1(r, x[v], t[v]); });
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) r = combine(r, shfl_xor(r, off));
  if ((tid & 63) == 0) part[tid >> 6] = r;
  __syncthreads();
  if (tid == 0) {
    RowStat a = part[0];
#pragma unroll
    for (int w = 1; w < kLossThreads / 64; ++w) a = combine(a, part[w]);
    const float lse = a.m + __builtin_amdgcn_logf(a.d) * kLn2;   // m + ln d
    const float wt = p.w ? p.w[i] : 1.0f;
    p.m[i] = a.m;
    p.d[i] = a.d;
    p.tsum[i] = a.st;
    p.row[i] = -wt * (a.sx - lse * a.st);
  }
}

// loss = (1/N) sum_i row_i: thread k sums rows k, k + 1024, ... in order,
// then a fixed tree over the threads.  N = 0 gives 0.
constexpr int kMeanThreads = 1024;
__global__ void __launch_bounds__(kMeanThreads) lsm_loss_mean_kernel(LossParams p) {
  __shared__ float s[kMeanThreads];
  const int tid = threadIdx.x;
  float a = 0.f;
  for (int i = tid; i < p.N; i += kMeanThreads) a += p.row[i];
  s[tid] = a;
  __syncthreads();
  for (int h = kMeanThreads / 2; h > 0; h >>= 1) {
    if (tid < h) s[tid] += s[tid + h];
    __syncthreads();
  }
  if (tid == 0) p.loss[0] = p.N > 0 ? s[0] / (float)p.N : 0.f;
}

// grad_iv = g w_i / N (exp(x_iv - m_i) / d_i * tsum_i - t_iv), over x.
__global__ void __launch_bounds__(kLossThreads) lsm_loss_bwd_kernel(LossParams p) {
  const int i = blockIdx.x, tid = threadIdx.x;
  float* x = p.x + (int64_t)i * p.x_ss;
  const float* t = p.t + (int64_t)i * p.t_ss;
  const float wt = p.w ? p.w[i] : 1.0f;
  const float coef = p.g[0] * wt / (float)p.N;
  const float m2 = p.m[i] * kLog2e;
  const float pd = p.tsum[i] / p.d[i];   // tsum_i / d_i
  walk_row(
      x, t, p.V, tid,
      [&](int v) __attribute__((always_inline)) {
        const f32x4 xv = *reinterpret_cast<const f32x4*>(x + v);
        const f32x4 tv = *reinterpret_cast<const f32x4*>(t + v);
        f32x4 gv;
#pragma unroll
        for (int k = 0; k < 4; ++k) gv[k] = coef * (exp2_hw(__builtin_fmaf(xv[k], kLog2e, -m2)) * pd - tv[k]);
        *reinterpret_cast<f32x4*>(x + v) = gv;
      },
      [&](int v) __attribute__((always_inline)) {
        x[v] = coef * (exp2_hw(__builtin_fmaf(x[v], kLog2e, -m2)) * pd - t[v]);
      });
}

}  // namespace

hipError_t launch_lsm_loss_fwd(const LossParams& p, hipStream_t s) {
  if (p.N > 0) {
    hipLaunchKernelGGL(lsm_loss_fwd_kernel, dim3((unsigned)p.N), dim3(kLossThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(lsm_loss_mean_kernel, dim3(1), dim3(kMeanThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_lsm_loss_bwd(const LossParams& p, hipStream_t s) {
  if (p.N == 0) return hipSuccess;
  hipLaunchKernelGGL(lsm_loss_bwd_kernel, dim3((unsigned)p.N), dim3(kLossThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
