// fa_internal.h - parameters shared by the host dispatcher and the kernels.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace fa {

// A [B, H, S, D] tensor with unit D stride, strides in elements.
struct Tensor {
  const void* ptr;
  int64_t sb, sh, ss;
};

struct Mask {
  int kind;            // 0 FULL, 1 CAUSAL, 2 TTT, 3 WINDOW
  int shift;           // causal shift (negative: a prefix of -shift keys before the diagonal)
  const int* kv_valid; // device [B] or nullptr
  int wl, wr;          // WINDOW: keys allowed before / after the (shifted) diagonal
  int frozen;          // keys below it get dK = dV = 0, not computed
  const float* bias;   // key bias [B, Skv] (row stride bias_sb) or nullptr
  int64_t bias_sb;
};

// Keys per V^T tile of the forward workspace (the forward's key tile).
constexpr int kVtTile = 64;

// Everything a kernel needs.  Built once per call by the dispatcher.
struct Params {
  int B, Hq, Hkv, G, Sq, Skv, D;
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e): scores go through exp2
  Mask mask;
  Tensor q, k, v, o;   // o: forward output / backward input
  Tensor dout;         // backward: dO
  Tensor dq, dk, dv;   // backward outputs
  float* lse;          // forward output
  void* vt;            // forward workspace (bf16): V^T [B, Hkv, D, vt_ss]
  int64_t vt_ss;       // keys per V^T row: Skv rounded up to a whole key tile
  const float* lse_in; // backward input
  float* delta;        // backward workspace: Delta [B, Hq, Sq]
  float* lse2;         // backward workspace: LSE * log2(e) [B, Hq, Sq]
  float* dkv_part;     // backward workspace (bf16): two halves' float32
                       // sums [2][dK^T, dV^T][B, Hkv, Skv, D]
  float* bias_s;       // workspace (bf16, with a key bias): bias / scale,
                       // [B, vt_ss], zero past Skv; written by the pre-pass
                       // (forward) or the Delta stage (backward)
};

// The bf16 dK/dV kernel's split decision counts 256-key blocks (its
// workgroups own 256 keys at D = 128, 128 at D <= 64).  With fewer than 1024
// such blocks it splits each workgroup's query steps between two workgroups
// (so the causal triangle still balances over the chip), which then need
// float32 partial sums (per key) in the workspace and a reduction; with more,
// every workgroup takes all steps of its block and writes dK, dV itself.
constexpr int kDkdvKeys = 256;
inline bool dkdv_split(int B, int Hkv, int keys) {
  const int64_t nkt = ((int64_t)keys + kDkdvKeys - 1) / kDkdvKeys;
  return (int64_t)B * Hkv * nkt < 1024;
}

// Launchers (one translation unit per kernel family).  Each returns the
// hipError_t of its launches; shapes were validated by the dispatcher.
// Backward stages: Delta = rowsum(dO * O), then the dK/dV and dQ kernels
// (independent of each other once Delta exists).  STAGE_GRADS (bf16 only) is
// DKDV and DQ together, in one launch where their workgroups allow it.
enum { STAGE_DELTA = 0, STAGE_DKDV = 1, STAGE_DQ = 2, STAGE_GRADS = 3 };
// Soft-target log-softmax loss (fa_lsm_loss_fwd / _bwd), validated by the
// dispatcher.
struct LossParams {
  int N, V;
  float* x;              // logits [N, V] (backward: overwritten with the gradient)
  int64_t x_ss;
  const float* t;        // targets [N, V]
  int64_t t_ss;
  const float* w;        // row weights [N] or nullptr (all 1)
  float *m, *d, *tsum;   // per-row max, normaliser, target sum
  float* row;            // per-row loss term
  float* loss;           // [1] mean
  const float* g;        // [1] upstream gradient of the mean
};
hipError_t launch_lsm_loss_fwd(const LossParams& p, hipStream_t s);
hipError_t launch_lsm_loss_bwd(const LossParams& p, hipStream_t s);

hipError_t launch_fwd_bf16(const Params& p, hipStream_t s);
hipError_t launch_bwd_bf16(const Params& p, int stage, hipStream_t s);
hipError_t launch_fwd_f32(const Params& p, hipStream_t s);
hipError_t launch_bwd_f32(const Params& p, int stage, hipStream_t s);

}  // namespace fa
