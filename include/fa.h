/*
 * fa.h - C ABI of the MI355X (gfx950) fused training-attention library.
 *
 * The library computes exact scaled-dot-product attention and its gradient
 * without ever holding the S x S score matrix in device memory:
 *
 *   forward   O = softmax(scale * Q K^T + mask) V, saving only O and the
 *             per-row natural logsumexp LSE of the scaled, masked scores.
 *             ("Flex Attention and Triton, Supporting Long Context Training
 *             in SpecForge", section EAGLE3 Training, gives the formula;
 *             the ggml flash-attn-training playbook, section 1 "What
 *             exists", gives the saved state O + LSE.)
 *   backward  recomputes P from LSE, forms Delta = rowsum(dO * O) and writes
 *             dQ, dK, dV  (CS336 "Flash Attention (Triton)": the fused
 *             kernel computes what the explicit QK^T -> softmax -> PV chain
 *             computes; the playbook's section 1 asks for a bitwise
 *             deterministic backward with no floating-point atomics).
 *
 * Mask kinds (SpecForge page, section "Flex Attention"):
 *   FA_MASK_FULL    key j allowed iff j < kv_valid[b]
 *   FA_MASK_CAUSAL  key j allowed iff j <= i - causal_shift and j < kv_valid[b]
 *                   (top-left aligned when Sq != Skv)
 *   FA_MASK_TTT     EAGLE3 training-time-test: with L = Sq and Skv = n * L,
 *                   key j allowed iff
 *                     (j <= i - causal_shift and j < kv_valid[b])            or
 *                     (j >= L and (j - i) mod L == 0 and (j mod L) < kv_valid[b])
 *                   i.e. causal over the step-0 keys plus, for every later
 *                   step s, the key of step s at the query's own position.
 *   FA_MASK_WINDOW  a band of keys around the query position: key j allowed
 *                   iff i - causal_shift - window_left <= j
 *                       <= i - causal_shift + window_right  and j < kv_valid[b]
 *                   ((w - 1, 0) is a causal sliding window of w keys, (w, w)
 *                   a symmetric band; the ggml playbook, section "4.
 *                   Measurement discipline", names windowed self-attention
 *                   among the diffusion trainer's geometries without fixing
 *                   the window's form).
 *   Prefix (the rectangular-plus-causal mask a frozen KV prefix needs; the
 *   ggml playbook's per-trainer checklist names it for a trainer with a
 *   frozen KV prefix): FA_MASK_CAUSAL with causal_shift = -P, Skv = P + Sq,
 *   so every query sees keys [0, P) and the causal part behind them;
 *   frozen_keys = P then skips the gradients of the frozen prefix.
 *   A query row with no allowed key gets O = 0 and LSE = 0, and contributes
 *   no gradient; a key no query may attend gets dK = dV = 0 exactly (ggml
 *   playbook, "6. Trap list", items 8 and 9).
 *   The mask is the same for every head.  Grouped-query attention maps query
 *   head h to key/value head h / (Hq / Hkv).
 *
 * Layout.  Every tensor is a logical [B, H, S, D] array with unit stride in
 * D and arbitrary element strides for B, H and S (so BHSD and BSHD views both
 * work without a copy: the ggml playbook's "3. Per-trainer porting
 * checklist" requires the fused ops to accept non-contiguous q/k/v views,
 * since copying them to a contiguous layout spends the memory the fused
 * path saves).  LSE is a contiguous float32 [B, Hq, Sq] array.
 * All tensor pointers are device pointers.  Element type: FA_BF16 (bfloat16
 * storage, float32 accumulation; O, dQ, dK, dV rounded to nearest even) or
 * FA_F32 (float32 throughout).
 *
 * Ownership.  The caller owns every buffer, including the forward and
 * backward workspaces.  The library allocates no device memory, keeps no state between
 * calls, launches on the caller's stream and never synchronises the host.
 *
 * Errors.  All arguments are validated before anything is launched; on a
 * non-OK status nothing was launched and fa_last_error() describes why.
 * There is no fallback path of any kind (the ggml playbook, "2. The adoption
 * contract", item 2: an unsupported request must be a named hard error,
 * because a silent fallback to another implementation produces numbers that
 * look like a pass).
 *
 * Calling convention.  The problem statement of the path names two calls,
 * forward and backward, each taking its arguments and a stream.  Here both
 * also take a caller-owned workspace (pointer and size), because the library
 * allocates nothing: the backward's holds Delta and the dK/dV partial sums,
 * the forward's a transposed copy of V that the P.V product reads (one pass
 * over V, linear in Skv).  The *_workspace_bytes calls give the sizes.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,  /* NULL pointer, non-positive size, Hq % Hkv != 0,
                              TTT with Skv % Sq != 0, negative shift,
                              workspace too small, unit D stride violated */
  FA_ERR_UNSUPPORTED = 2,  /* D not in {16, 32, 64, 128}, unknown dtype/kind,
                              sequence stride of 2^24 elements or more */
  FA_ERR_ALIGNMENT = 3,    /* base pointer or B/H/S stride not 16-byte aligned */
  FA_ERR_ALIAS = 4,        /* an output's byte range overlaps an input's */
  FA_ERR_HIP = 5           /* no usable device, or a launch failed */
} fa_status;

typedef enum { FA_BF16 = 0, FA_F32 = 1 } fa_dtype;

typedef enum { FA_MASK_FULL = 0, FA_MASK_CAUSAL = 1, FA_MASK_TTT = 2, FA_MASK_WINDOW = 3 } fa_mask_kind;

/* One [B, H, S, D] tensor: base pointer and element strides (D stride = 1).
 * Any outer strides that are multiples of 16 bytes are accepted, so a BSHD
 * or otherwise strided view is passed as is (the ggml playbook, "3.
 * Per-trainer porting checklist": non-contiguous q/k/v views, no copies). */
typedef struct {
  void* data;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_s;
} fa_tensor;

/* The mask descriptor: which (query, key) pairs may attend, the same for
 * every head ("Flex Attention and Triton, Supporting Long Context Training in
 * SpecForge", section "Flex Attention": the causal, padding and suffix mask
 * functions, broadcast over heads, with per-batch sequence lengths; the
 * WINDOW and prefix forms are described above). */
typedef struct {
  int32_t kind;              /* fa_mask_kind */
  int32_t causal_shift;      /* used by CAUSAL, WINDOW and TTT's step-0 part; >= 0
                                for TTT, any value for CAUSAL and WINDOW (a negative
                                shift -P shows every query the first P keys before
                                the diagonal: CAUSAL with Skv = P + Sq is a causal
                                sequence behind a P-key prefix) */
  const int32_t* kv_valid;   /* device int32 [B] valid key count per batch
                                (clamped to [0, Skv] for FULL/CAUSAL/WINDOW and
                                to [0, Sq] for TTT), or NULL = all keys valid */
  int32_t window_left;       /* WINDOW only: >= 0 keys before the diagonal */
  int32_t window_right;      /* WINDOW only: >= 0 keys after the diagonal */
  int32_t frozen_keys;       /* >= 0: keys j < frozen_keys are frozen (a prefix
                                whose K/V are not trained): the backward writes
                                dK = dV = 0 there and does not compute them; the
                                forward and dQ are unchanged.  0 = none */
  const float* key_bias;     /* device float32 [B, Skv] or NULL: an additive mask
                                in per-key form (the ggml playbook, "3. Per-trainer
                                porting checklist": the fused ops take an additive
                                mask, broadcast where it has fewer dimensions).
                                key_bias[b * key_bias_stride_b + j] is added to the
                                scaled score of key j for every query row and head
                                of batch entry b, on top of the mask kind (a key
                                still needs the kind's permission); LSE includes
                                it.  Values are finite or -inf (-inf drops the key
                                for that batch entry); +inf and NaN give undefined
                                results.  An input only: the backward computes no
                                gradient for it.  4-byte aligned; the caller owns
                                it and must pass the same bias to fa_bwd. */
  int64_t key_bias_stride_b; /* >= 0, elements between batch rows of key_bias
                                (0: one row for every batch entry) */
} fa_mask_desc;

/* Forward arguments: the shapes, the softmax scale (1/sqrt(d_k) by default,
 * as in the SpecForge page's section "EAGLE3 Training"), Q, K, V and the
 * outputs.  Hkv < Hq is grouped-query attention and Sq != Skv is allowed (the
 * ggml playbook's "3. Per-trainer porting checklist" lists both among what
 * the fused ops must take). */
typedef struct {
  int32_t dtype;             /* fa_dtype */
  int32_t B, Hq, Hkv, Sq, Skv, D;
  float scale;               /* softmax scale; <= 0 selects 1/sqrt(D) */
  fa_tensor q;               /* in  [B, Hq,  Sq,  D] */
  fa_tensor k;               /* in  [B, Hkv, Skv, D] */
  fa_tensor v;               /* in  [B, Hkv, Skv, D] */
  fa_tensor o;               /* out [B, Hq,  Sq,  D] */
  float* lse;                /* out [B, Hq, Sq] float32, natural log */
  fa_mask_desc mask;
} fa_fwd_args;

/* Backward arguments: the forward's, plus its saved O and LSE and the
 * upstream gradient dO, and the three gradient outputs (the ggml playbook,
 * "1. What exists": the backward consumes the forward's O and LSE and
 * produces dQ, dK, dV). */
typedef struct {
  int32_t dtype;
  int32_t B, Hq, Hkv, Sq, Skv, D;
  float scale;               /* must equal the forward's */
  fa_tensor q, k, v;         /* in, as in the forward */
  fa_tensor o;               /* in  forward output O */
  fa_tensor dout;            /* in  upstream gradient dO [B, Hq, Sq, D] */
  const float* lse;          /* in  forward LSE [B, Hq, Sq] */
  fa_tensor dq;              /* out [B, Hq,  Sq,  D] */
  fa_tensor dk;              /* out [B, Hkv, Skv, D] (summed over the group) */
  fa_tensor dv;              /* out [B, Hkv, Skv, D] (summed over the group) */
  fa_mask_desc mask;         /* must equal the forward's */
} fa_bwd_args;

/* Bytes of device scratch fa_fwd needs for these arguments.  FA_BF16: one
 * transposed copy of V, bfloat16 [B, Hkv, D, Skv rounded up to 64], rounded
 * up to 256 bytes (the PV product, O^T = V^T P^T of CS336 "Flash Attention
 * (Triton)", contracts over keys; stored key-minor, V^T feeds the matrix
 * cores with plain 16-byte reads).  With a key_bias, FA_BF16 adds float32
 * [B, Skv rounded up to 64] (the bias divided by the scale, which the matrix
 * cores take as the initial value of each score), rounded up to 256 bytes.
 * FA_F32: 0.  Linear in Skv, never S x S.  Depends on args->mask.key_bias.
 * Returns 0 when args is NULL. */
size_t fa_fwd_workspace_bytes(const fa_fwd_args* args);

/* Forward: writes O and LSE.  `ws` is caller-owned device memory of at least
 * fa_fwd_workspace_bytes(args) bytes, 256-byte aligned (may be NULL when that
 * is 0); its contents on return are unspecified.  Asynchronous on `stream`
 * (0 = null stream). */
fa_status fa_fwd(const fa_fwd_args* args, void* ws, size_t ws_bytes, hipStream_t stream);

/* Forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results as fa_fwd, bitwise, with the workspace taken
 * from a static device array of FA_FWD_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device it runs on until the process ends.  The
 * caller still passes the inputs and outputs; the call itself allocates
 * nothing.  Shapes whose fa_fwd_workspace_bytes exceed the array are refused
 * with FA_ERR_UNSUPPORTED (before any launch).  Every call on one device
 * shares that device's array: calls that overlap in time on one device (on
 * different streams, or from different threads without ordering) race, and
 * must be ordered by the caller.  Nothing in the array needs to start at
 * zero (each call writes every element it reads). */
#define FA_FWD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fa_status fa_fwd_noalloc(const fa_fwd_args* args, hipStream_t stream);

/* Bytes of device scratch fa_bwd needs for these arguments.  It is linear
 * in the sequence lengths: the backward never holds the S x S score or
 * probability matrix, it rebuilds P tile by tile from the saved logsumexp
 * (CS336 "Flash Attention (Triton)", How it works: only O and the
 * logsumexp are kept for the backward).  The bytes: two float32
 * [B, Hq, Sq] arrays (Delta, and LSE in log2 units), each rounded up to 256
 * bytes, and for FA_BF16 the dK/dV kernel's float32 partial
 * sums, four [B, Hkv, Skv, D] arrays (two halves of each key block's query
 * steps, dK and dV; under FA_MASK_TTT only the Sq step-0 keys have them, so
 * Sq replaces Skv), rounded up to 256 bytes, and with a key_bias a float32
 * [B, Skv rounded up to 64] copy of it divided by the scale, rounded up to
 * 256 bytes; linear in Sq and Skv, never S x S.  Depends on args->mask.kind
 * and args->mask.key_bias.  Returns 0 when args is NULL. */
size_t fa_bwd_workspace_bytes(const fa_bwd_args* args);

/* Backward: writes dQ, dK, dV; bitwise identical on every rerun (fixed
 * reduction orders, no floating-point atomics).  `ws` is caller-owned device
 * memory of at least fa_bwd_workspace_bytes(args) bytes, 256-byte aligned. */
fa_status fa_bwd(const fa_bwd_args* args, void* ws, size_t ws_bytes,
                 hipStream_t stream);

/* The three stages of fa_bwd, in the order fa_bwd runs them. */
typedef enum {
  FA_BWD_DELTA = 0,  /* Delta_i = sum_d dO_id O_id into the workspace (the row
                        term of dS = P * (dP - Delta); CS336 "Flash Attention
                        (Triton)", backward pass), beside LSE_i * log2(e) */
  FA_BWD_DKDV = 1,   /* dK, dV: one workgroup per key block, summing over the
                        group's query heads in a fixed order */
  FA_BWD_DQ = 2      /* dQ: one workgroup per query block */
} fa_bwd_stage_id;

/* Runs one stage of fa_bwd with the same arguments, validation and workspace
 * (the ggml playbook, "4. Measurement discipline", attributes the fused
 * backward's cost kernel by kernel before changing any; this is the call
 * that lets a caller time or overlap the stages one by one).
 * DKDV and DQ read what a DELTA stage left in `ws` (on the same
 * stream, or ordered after it by the caller); given that, running DELTA,
 * DKDV, DQ in turn writes bitwise the same dQ, dK, dV as fa_bwd.  For callers
 * that overlap the two gradient kernels on separate streams or time them one
 * by one.  An unknown stage returns FA_ERR_INVALID_ARG. */
fa_status fa_bwd_stage(const fa_bwd_args* args, int stage, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Soft-target log-softmax loss, the loss EAGLE3 training takes after the
 * draft model's attention and LM head ("Flex Attention and Triton,
 * Supporting Long Context Training in SpecForge", section "In-place Gradient
 * Calculation").  For N rows (batch x positions) of V logits x, soft targets
 * t and per-row mask weights w:
 *
 *   m_i = max_v x_iv,  d_i = sum_v exp(x_iv - m_i),  tsum_i = sum_v t_iv
 *   row_i = -w_i * sum_v t_iv * (x_iv - m_i - ln d_i)
 *   loss  = (1/N) * sum_i row_i          (masked rows count in the mean)
 *   dloss/dx_iv = w_i / N * (exp(x_iv - m_i) / d_i * tsum_i - t_iv)
 *
 * The forward reads each row once (an online max and normaliser, as the
 * page's kernel keeps m and d) and saves m, d, tsum; the backward writes the
 * gradient, times the upstream gradient, over the logits in place (the
 * page's memory saving: no second [N, V] buffer).  All arithmetic is fp32.
 * The mean is a fixed-order sum, so reruns are bitwise identical. */
typedef struct {
  int32_t N;                 /* rows, >= 0 */
  int32_t V;                 /* vocabulary size (columns), >= 1 */
  float* logits;             /* [N, V], row stride logits_ss elements: read by the
                                forward; overwritten with the gradient by the
                                backward (in place) */
  int64_t logits_ss;
  const float* target;       /* [N, V] soft targets, row stride target_ss */
  int64_t target_ss;
  const float* mask;         /* [N] row weights w_i, or NULL for all 1 */
  float* m;                  /* [N] row max: forward writes, backward reads */
  float* d;                  /* [N] sum_v exp(x_iv - m_i): forward writes, backward reads */
  float* tsum;               /* [N] sum_v t_iv: forward writes, backward reads */
  float* row_loss;           /* [N] row_i: forward writes (backward ignores) */
  float* loss;               /* [1] the mean loss: forward writes (backward ignores) */
  const float* grad_loss;    /* [1] upstream gradient of loss: backward reads
                                (forward ignores) */
} fa_lsm_loss_args;

/* Forward of the loss: writes m, d, tsum, row_loss and loss.  All pointers
 * are device pointers, 4-byte aligned (else FA_ERR_ALIGNMENT); row strides
 * are at least V (rows that start 16-byte aligned, and whose logits and
 * target rows sit at the same offset from a 16-byte boundary, are read
 * with 16-byte loads; others element by element).  The
 * outputs must not overlap logits, target, mask or each other
 * (FA_ERR_ALIAS).  N = 0 writes loss = 0 and nothing else.  Validation runs
 * before any launch; asynchronous on `stream`. */
fa_status fa_lsm_loss_fwd(const fa_lsm_loss_args* args, hipStream_t stream);

/* Backward of the loss: overwrites logits with grad_loss[0] * dloss/dx, from
 * the m, d, tsum the forward wrote for these logits and targets (logits must
 * still hold the forward's values).  Same alignment and aliasing rules (m,
 * d, tsum and grad_loss must not overlap logits). */
fa_status fa_lsm_loss_bwd(const fa_lsm_loss_args* args, hipStream_t stream);

/* Text describing the last non-OK status returned on this thread
 * ("" if none).  The pointer stays valid until the thread's next call.
 * Every refusal names its reason here (the ggml playbook, "2. The adoption
 * contract", item 2: an unsupported case is reported as a named error, never
 * absorbed by a fallback). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
