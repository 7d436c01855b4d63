// lane_probe.hip - single-wave probes of the gfx950 building blocks that the
// attention kernels rely on (test infrastructure, built beside the library).
//
// Each probe calls one helper of fa_device.h the way the kernels call it and
// writes out what every lane received, so the GPU tests can hold it against
// the layout that header states:
//   probe_mfma  the operand and result lane maps of mfma32
//               (v_mfma_f32_32x32x16_bf16), accumulating onto a given C;
//   probe_tr    lds_read_tr4 (ds_read_b64_tr_b16) on a swizzled [64][D] tile
//               written at swz_off<D>, read back 4x16 block by block;
//   probe_swap  half_swap_max / half_swap_sum (v_permlane32_swap);
//   probe_dma   the landing slots of the asynchronous HBM->LDS copies, in
//               the per-lane address form (lds_dma16) and the scalar-base
//               form (lds_dma16_s).
// Every probe is one workgroup of one 64-lane wave; every global index is
// reduced into its buffer inside the kernel, so no input can take a probe out
// of bounds.
#include <hip/hip_runtime.h>

#include "fa_device.h"

using namespace fa;

namespace {

// A [32][16], B [16][32], C0 and C [32][32], all row-major.
__global__ __launch_bounds__(64) void probe_mfma_kernel(const bf16* A, const bf16* B, const float* C0,
                                                        float* C) {
  const int l = threadIdx.x;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = A[(l % 32) * 16 + 8 * (l / 32) + e];
    b[e] = B[(8 * (l / 32) + e) * 32 + l % 32];
  }
  f32x16 c;
  for (int i = 0; i < 16; ++i) c[i] = C0[(8 * (i / 4) + 4 * (l / 32) + i % 4) * 32 + l % 32];
  c = mfma32(a, b, c);
  for (int i = 0; i < 16; ++i) C[(8 * (i / 4) + 4 * (l / 32) + i % 4) * 32 + l % 32] = c[i];
}

// X [64][D] row-major; XT [D][64] receives what the transposing reads return.
// The tile is stored into LDS element by element at swz_off<D>; group g of 16
// lanes (lane r inside it) then reads block bi = 4 it + g, rows 4 kb .. 4 kb+3
// and columns 16 nb .. 16 nb+15, pointing at row 4 kb + r/4, column
// 16 nb + 4 (r%4).  By the stated map lane r receives column 16 nb + r of the
// four rows, which lands at XT[16 nb + r][4 kb + e].
template <int D>
__global__ __launch_bounds__(64) void probe_tr_kernel(const bf16* X, bf16* XT) {
  __shared__ __attribute__((aligned(16))) bf16 tile[64 * D];
  const int l = threadIdx.x;
  for (int i = l; i < 64 * D; i += 64) {
    const int r = i / D, e = i % D;
    *(bf16*)((unsigned char*)tile + swz_off<D>(r, e)) = X[i];
  }
  __syncthreads();
  const int g = l / 16, r = l % 16;
  constexpr int NB = 16 * (D / 16);  // 4x16 blocks in the tile
  for (int it = 0; it < NB / 4; ++it) {
    const int bi = 4 * it + g;
    const int kb = bi % 16, nb = bi / 16;
    const bf16* p = (const bf16*)((const unsigned char*)tile + swz_off<D>(4 * kb + r / 4, 16 * nb + 4 * (r % 4)));
    const bf16x4 v = lds_read_tr4(p);
    for (int e = 0; e < 4; ++e) XT[(16 * nb + r) * 64 + 4 * kb + e] = v[e];
  }
}

__global__ __launch_bounds__(64) void probe_swap_kernel(const float* x, float* mx, float* sm) {
  const int l = threadIdx.x;
  mx[l] = half_swap_max(x[l]);
  sm[l] = half_swap_sum(x[l]);
}

// g: n 16-byte chunks.  Copy 1 (per-lane address): lane l fetches chunk
// perm[l]; copy 2 (scalar base g, per-lane offset 16 perm[64 + l]).  Both land
// in LDS, one 1 KB block each, which the wave then writes out as it finds it.
__global__ __launch_bounds__(64) void probe_dma_kernel(const unsigned char* g, unsigned n, const unsigned* perm,
                                                       unsigned char* out) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2048];
  const int l = threadIdx.x;
  unsigned c1 = perm[l], c2 = perm[64 + l];
  if (c1 >= n) c1 = 0;
  if (c2 >= n) c2 = 0;
  lds_dma16(g + 16 * (size_t)c1, lds);
  lds_dma16_s(g, 16u * c2, lds_addr_of(lds + 1024));
  wait_vmcnt<0>();
  barrier_lds();
  const i32x4* src = (const i32x4*)lds;
  i32x4* dst = (i32x4*)out;
  dst[l] = src[l];
  dst[64 + l] = src[64 + l];
}

int status() { return (int)hipGetLastError(); }

}  // namespace

extern "C" {

int probe_mfma(const void* A, const void* B, const void* C0, void* C, hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(1), dim3(64), 0, s, (const bf16*)A, (const bf16*)B,
                     (const float*)C0, (float*)C);
  return status();
}

// D in {16, 32, 64, 128}; anything else is refused (returns -1, nothing runs).
int probe_tr(const void* X, void* XT, int D, hipStream_t s) {
  const bf16* x = (const bf16*)X;
  bf16* xt = (bf16*)XT;
  switch (D) {
    case 16: hipLaunchKernelGGL(probe_tr_kernel<16>, dim3(1), dim3(64), 0, s, x, xt); break;
    case 32: hipLaunchKernelGGL(probe_tr_kernel<32>, dim3(1), dim3(64), 0, s, x, xt); break;
    case 64: hipLaunchKernelGGL(probe_tr_kernel<64>, dim3(1), dim3(64), 0, s, x, xt); break;
    case 128: hipLaunchKernelGGL(probe_tr_kernel<128>, dim3(1), dim3(64), 0, s, x, xt); break;
    default: return -1;
  }
  return status();
}

int probe_swap(const void* x, void* mx, void* sm, hipStream_t s) {
  hipLaunchKernelGGL(probe_swap_kernel, dim3(1), dim3(64), 0, s, (const float*)x, (float*)mx, (float*)sm);
  return status();
}

// n >= 1 chunks at g; perm: 128 chunk indices; out: 2048 bytes.
int probe_dma(const void* g, unsigned n, const void* perm, void* out, hipStream_t s) {
  if (n == 0) return -1;
  hipLaunchKernelGGL(probe_dma_kernel, dim3(1), dim3(64), 0, s, (const unsigned char*)g, n,
                     (const unsigned*)perm, (unsigned char*)out);
  return status();
}

}  // extern "C"
