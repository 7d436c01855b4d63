// fa_api.cpp - the C ABI: argument validation, dispatch, error text.
//
// Everything is validated before the first launch; a failing call launches
// nothing.  There is no fallback path: an unsupported request is an error
// (the ggml flash-attn-training playbook, section 2, item 2, explains why a
// silent fallback is worse than a hard error).
#include "../../include/fa.h"
#include "fa_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <unordered_map>

namespace {

thread_local std::string g_error;

fa_status fail(fa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return s;
}

struct Shape {
  int dtype, B, Hq, Hkv, Sq, Skv, D;
};

int elem_bytes(int dtype) { return dtype == FA_BF16 ? 2 : 4; }

// Byte range [lo, hi) spanned by a [n0, n1, n2, D] strided tensor.
struct Range {
  uintptr_t lo, hi;
  bool empty;
};

Range span(const fa_tensor& t, int n0, int n1, int n2, int D, int eb) {
  Range r{0, 0, true};
  if (n0 <= 0 || n1 <= 0 || n2 <= 0 || D <= 0) return r;
  int64_t lo = 0, hi = 0;
  const int64_t st[3] = {t.stride_b, t.stride_h, t.stride_s};
  const int64_t n[3] = {n0, n1, n2};
  for (int i = 0; i < 3; ++i) {
    int64_t ext = st[i] * (n[i] - 1);
    if (ext < 0) lo += ext; else hi += ext;
  }
  hi += D;
  r.lo = reinterpret_cast<uintptr_t>(t.data) + lo * eb;
  r.hi = reinterpret_cast<uintptr_t>(t.data) + hi * eb;
  r.empty = false;
  return r;
}

bool overlap(const Range& a, const Range& b) {
  return !a.empty && !b.empty && a.lo < b.hi && b.lo < a.hi;
}

fa_status check_shape(const Shape& s, const fa_mask_desc& m) {
  if (s.dtype != FA_BF16 && s.dtype != FA_F32)
    return fail(FA_ERR_UNSUPPORTED, "unknown dtype %d (expected FA_BF16=0 or FA_F32=1)", s.dtype);
  if (s.B < 0 || s.Sq < 0 || s.Skv < 0)
    return fail(FA_ERR_INVALID_ARG, "negative size: B=%d Sq=%d Skv=%d", s.B, s.Sq, s.Skv);
  if (s.Hq <= 0 || s.Hkv <= 0 || s.D <= 0)
    return fail(FA_ERR_INVALID_ARG, "non-positive size: Hq=%d Hkv=%d D=%d", s.Hq, s.Hkv, s.D);
  if (s.Hq % s.Hkv != 0)
    return fail(FA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", s.Hq, s.Hkv);
  if (s.D != 16 && s.D != 32 && s.D != 64 && s.D != 128)
    return fail(FA_ERR_UNSUPPORTED, "head dim D=%d not in {16, 32, 64, 128}", s.D);
  if (m.kind != FA_MASK_FULL && m.kind != FA_MASK_CAUSAL && m.kind != FA_MASK_TTT &&
      m.kind != FA_MASK_WINDOW)
    return fail(FA_ERR_UNSUPPORTED, "unknown mask kind %d", m.kind);
  if (m.kind == FA_MASK_WINDOW && (m.window_left < 0 || m.window_right < 0))
    return fail(FA_ERR_INVALID_ARG, "negative window (left %d, right %d)", m.window_left, m.window_right);
  if (m.causal_shift < 0 && m.kind == FA_MASK_TTT)
    return fail(FA_ERR_INVALID_ARG, "negative causal_shift %d with the TTT mask", m.causal_shift);
  if (m.frozen_keys < 0)
    return fail(FA_ERR_INVALID_ARG, "negative frozen_keys %d", m.frozen_keys);
  if (m.key_bias && s.B > 0 && s.Skv > 0) {
    if (reinterpret_cast<uintptr_t>(m.key_bias) % 4 != 0)
      return fail(FA_ERR_ALIGNMENT, "key_bias: pointer is not 4-byte aligned");
    if (m.key_bias_stride_b < 0)
      return fail(FA_ERR_INVALID_ARG, "key_bias_stride_b %lld is negative", (long long)m.key_bias_stride_b);
    if (m.key_bias_stride_b > (int64_t(1) << 40))
      return fail(FA_ERR_UNSUPPORTED, "key_bias_stride_b %lld is too large", (long long)m.key_bias_stride_b);
  }
  if (m.kind == FA_MASK_TTT) {
    if (s.Sq <= 0 && s.Skv != 0)
      return fail(FA_ERR_INVALID_ARG, "TTT mask needs Sq > 0 (Sq is the step length)");
    if (s.Sq > 0 && s.Skv % s.Sq != 0)
      return fail(FA_ERR_INVALID_ARG, "TTT mask needs Skv (%d) to be a multiple of Sq (%d)", s.Skv, s.Sq);
  }
  return FA_OK;
}

// Checks one tensor: non-null data (when non-empty), 16-byte alignment of the
// base pointer and of every outer stride, and, for outputs, that no two
// elements share an address.
fa_status check_tensor(const char* name, const fa_tensor& t, int n0, int n1, int n2,
                       int D, int eb, bool output) {
  if (n0 == 0 || n2 == 0) return FA_OK;  // empty: never touched
  if (t.data == nullptr) return fail(FA_ERR_INVALID_ARG, "%s: NULL data pointer", name);
  if (reinterpret_cast<uintptr_t>(t.data) % 16 != 0)
    return fail(FA_ERR_ALIGNMENT, "%s: base pointer %p is not 16-byte aligned", name, t.data);
  const int64_t st[3] = {t.stride_b, t.stride_h, t.stride_s};
  const int64_t n[3] = {n0, n1, n2};
  for (int i = 0; i < 3; ++i) {
    if (n[i] > 1 && (st[i] * eb) % 16 != 0)
      return fail(FA_ERR_ALIGNMENT, "%s: stride %d (%lld elements) is not a multiple of 16 bytes",
                  name, i, (long long)st[i]);
  }
  // The kernels address rows of one 64-row tile with 32-bit element offsets.
  if (std::llabs(t.stride_s) >= (int64_t(1) << 24))
    return fail(FA_ERR_UNSUPPORTED, "%s: sequence stride %lld elements is too large (limit 2^24)",
                name, (long long)t.stride_s);
  if (output) {
    // No self-overlap: sort the outer dims by |stride|; each stride must
    // cover the extent of everything below it.
    struct Dim { int64_t n, st; };
    Dim dims[3] = {{n[0], st[0]}, {n[1], st[1]}, {n[2], st[2]}};
    std::sort(dims, dims + 3, [](const Dim& a, const Dim& b) {
      return std::llabs(a.st) < std::llabs(b.st);
    });
    int64_t extent = D;
    for (const Dim& d : dims) {
      if (d.n <= 1) continue;
      if (std::llabs(d.st) < extent)
        return fail(FA_ERR_INVALID_ARG, "%s: output strides overlap (stride %lld < extent %lld)",
                    name, (long long)d.st, (long long)extent);
      extent = std::llabs(d.st) * d.n;
    }
  }
  return FA_OK;
}

fa_status check_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0)
    return fail(FA_ERR_HIP, "no HIP device available (%s)",
                e != hipSuccess ? hipGetErrorString(e) : "device count is 0");
  return FA_OK;
}

fa::Tensor tensor(const fa_tensor& t) { return {t.data, t.stride_b, t.stride_h, t.stride_s}; }

void fill_common(fa::Params& p, const Shape& s, float scale, const fa_mask_desc& m) {
  p.B = s.B; p.Hq = s.Hq; p.Hkv = s.Hkv; p.G = s.Hq / s.Hkv;
  p.Sq = s.Sq; p.Skv = s.Skv; p.D = s.D;
  p.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)s.D);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.mask.kind = m.kind;
  p.mask.shift = m.causal_shift;
  p.mask.kv_valid = m.kv_valid;
  p.mask.wl = m.kind == FA_MASK_WINDOW ? m.window_left : 0;
  p.mask.wr = m.kind == FA_MASK_WINDOW ? m.window_right : 0;
  p.mask.frozen = m.frozen_keys;
  p.mask.bias = s.B > 0 && s.Skv > 0 ? m.key_bias : nullptr;
  p.mask.bias_sb = m.key_bias_stride_b;
}

// The bytes the key bias spans (empty without one).
Range bias_span(const Shape& s, const fa_mask_desc& m) {
  if (!m.key_bias || s.B <= 0 || s.Skv <= 0) return Range{0, 0, true};
  const uintptr_t lo = reinterpret_cast<uintptr_t>(m.key_bias);
  return Range{lo, lo + ((uintptr_t)(s.B - 1) * (uintptr_t)m.key_bias_stride_b + (uintptr_t)s.Skv) * 4, false};
}

// One float32 [B, Hq, Sq] array, rounded up to 256 bytes.
size_t row_array_bytes(const Shape& s) {
  size_t n = (size_t)std::max(s.B, 0) * (size_t)std::max(s.Hq, 0) * (size_t)std::max(s.Sq, 0) * 4;
  return (n + 255) / 256 * 256;
}

// The dK/dV kernel's partial sums (bf16, when it splits its key blocks,
// fa::dkdv_split): two halves of float32 dK^T and dV^T,
// [2][2][B, Hkv, keys, D], rounded up to 256 bytes, over the keys the tile
// kernel owns (all Skv, or under TTT the Sq step-0 keys).
size_t part_bytes(const Shape& s, int kind) {
  if (s.dtype != FA_BF16) return 0;
  const int keys = kind == FA_MASK_TTT && s.Sq < s.Skv ? s.Sq : s.Skv;
  if (!fa::dkdv_split(std::max(s.B, 0), std::max(s.Hkv, 0), std::max(keys, 0))) return 0;
  size_t n = (size_t)4 * std::max(s.B, 0) * (size_t)std::max(s.Hkv, 0) * (size_t)std::max(keys, 0) *
             (size_t)s.D * 4;
  return (n + 255) / 256 * 256;
}

// Keys per row of the forward's V^T and of the scaled key-bias copy: Skv
// rounded up to a whole key tile.
int64_t vt_keys(const Shape& s) {
  return ((int64_t)std::max(s.Skv, 0) + fa::kVtTile - 1) / fa::kVtTile * fa::kVtTile;
}

// The key bias divided by the scale (bf16 kernels, with a key bias):
// float32 [B, vt_keys(s)], rounded up to 256 bytes.
size_t bias_copy_bytes(const Shape& s, const fa_mask_desc& m) {
  if (s.dtype != FA_BF16 || !m.key_bias || s.B <= 0 || s.Skv <= 0) return 0;
  size_t n = (size_t)s.B * (size_t)vt_keys(s) * 4;
  return (n + 255) / 256 * 256;
}

// Backward workspace: Delta, then LSE * log2(e) (both [B, Hq, Sq] float32),
// then the dK/dV partial sums, then the scaled key bias.
size_t delta_bytes(const Shape& s, const fa_mask_desc& m) {
  return 2 * row_array_bytes(s) + part_bytes(s, m.kind) + bias_copy_bytes(s, m);
}

// Forward workspace (bf16 only): V^T, bfloat16 [B, Hkv, D, vt_keys(s)], then
// the scaled key bias.
size_t vt_bytes(const Shape& s) {
  if (s.dtype != FA_BF16) return 0;
  size_t n = (size_t)std::max(s.B, 0) * (size_t)std::max(s.Hkv, 0) * (size_t)std::max(s.D, 0) *
             (size_t)vt_keys(s) * 2;
  return (n + 255) / 256 * 256;
}
size_t fwd_ws_bytes(const Shape& s, const fa_mask_desc& m) { return vt_bytes(s) + bias_copy_bytes(s, m); }

// A caller workspace of `need` bytes: present, large enough, 256-byte aligned.
fa_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return FA_OK;
  if (ws == nullptr) return fail(FA_ERR_INVALID_ARG, "workspace: NULL pointer (%zu bytes needed)", need);
  if (ws_bytes < need)
    return fail(FA_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(FA_ERR_ALIGNMENT, "workspace pointer %p is not 256-byte aligned", ws);
  return FA_OK;
}

// ---- the forward's allocation-free variant: a static scratch array ---------
// fa_fwd_noalloc takes its workspace (the forward's V^T copy) from this
// device array instead of the caller.  Each device the library runs on holds
// its own copy for the life of the process.  Host code never uses the
// array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocScratchBytes = FA_FWD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;   // device ordinal -> scratch's address there

fa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd_noalloc: no current device (%s)", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(FA_ERR_HIP, "fa_fwd_noalloc: the scratch array has no address on device %d (%s)", dev,
                  hipGetErrorString(e));
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return FA_OK;
}

// fa_fwd and fa_fwd_noalloc: validation, then the launches.  With
// static_ws the workspace is the scratch array (its size is ws_bytes; its
// address is looked up only once everything else is valid).
fa_status fwd_run(const fa_fwd_args* a, void* ws, size_t ws_bytes, hipStream_t stream, bool static_ws) {
  const char* fn = static_ws ? "fa_fwd_noalloc" : "fa_fwd";
  if (!a) return fail(FA_ERR_INVALID_ARG, "%s: args is NULL", fn);
  Shape s{a->dtype, a->B, a->Hq, a->Hkv, a->Sq, a->Skv, a->D};
  fa_status st = check_shape(s, a->mask);
  if (st != FA_OK) return st;
  const int eb = elem_bytes(s.dtype);
  if ((st = check_tensor("q", a->q, s.B, s.Hq, s.Sq, s.D, eb, false))) return st;
  if ((st = check_tensor("k", a->k, s.B, s.Hkv, s.Skv, s.D, eb, false))) return st;
  if ((st = check_tensor("v", a->v, s.B, s.Hkv, s.Skv, s.D, eb, false))) return st;
  if ((st = check_tensor("o", a->o, s.B, s.Hq, s.Sq, s.D, eb, true))) return st;
  const bool rows = s.B > 0 && s.Sq > 0;
  if (rows && a->lse == nullptr) return fail(FA_ERR_INVALID_ARG, "lse: NULL pointer");
  if (rows && reinterpret_cast<uintptr_t>(a->lse) % 4 != 0)
    return fail(FA_ERR_ALIGNMENT, "lse: pointer is not 4-byte aligned");
  // outputs must not overlap inputs or each other
  Range rq = span(a->q, s.B, s.Hq, s.Sq, s.D, eb), rk = span(a->k, s.B, s.Hkv, s.Skv, s.D, eb),
        rv = span(a->v, s.B, s.Hkv, s.Skv, s.D, eb), ro = span(a->o, s.B, s.Hq, s.Sq, s.D, eb);
  Range rl{reinterpret_cast<uintptr_t>(a->lse),
           reinterpret_cast<uintptr_t>(a->lse) + (size_t)s.B * s.Hq * s.Sq * 4, !rows};
  if (s.dtype == FA_BF16 && vt_keys(s) >= (int64_t(1) << 24))
    return fail(FA_ERR_UNSUPPORTED, "Skv=%d is too large (limit 2^24 - 64)", s.Skv);
  const size_t need = fwd_ws_bytes(s, a->mask);
  if (static_ws) {
    if (need > ws_bytes)
      return fail(FA_ERR_UNSUPPORTED,
                  "fa_fwd_noalloc: these shapes need %zu bytes of scratch (B*Hkv*D*Skv rounded up, bf16, "
                  "plus B*Skv floats with a key bias); "
                  "its static scratch holds %zu; call fa_fwd with a workspace instead", need, ws_bytes);
  } else if ((st = check_ws(ws, ws_bytes, need))) {
    return st;
  }
  // (the static scratch cannot overlap a caller's buffer: its address is never handed out)
  Range rw{reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + need, need == 0 || static_ws};
  for (const Range* in : {&rq, &rk, &rv}) {
    if (overlap(ro, *in)) return fail(FA_ERR_ALIAS, "o overlaps an input tensor");
    if (overlap(rl, *in)) return fail(FA_ERR_ALIAS, "lse overlaps an input tensor");
    if (overlap(rw, *in)) return fail(FA_ERR_ALIAS, "workspace overlaps an input tensor");
  }
  if (overlap(ro, rl)) return fail(FA_ERR_ALIAS, "o overlaps lse");
  if (overlap(rw, ro)) return fail(FA_ERR_ALIAS, "workspace overlaps o");
  if (overlap(rw, rl)) return fail(FA_ERR_ALIAS, "workspace overlaps lse");
  const Range rb = bias_span(s, a->mask);
  if (overlap(rb, ro) || overlap(rb, rl) || overlap(rb, rw))
    return fail(FA_ERR_ALIAS, "key_bias overlaps o, lse or the workspace");
  if (a->mask.kv_valid && reinterpret_cast<uintptr_t>(a->mask.kv_valid) % 4 != 0)
    return fail(FA_ERR_ALIGNMENT, "kv_valid: pointer is not 4-byte aligned");
  if (!rows) return FA_OK;  // nothing to compute
  if ((st = check_device())) return st;
  if (static_ws && need > 0 && (st = scratch_address(&ws))) return st;

  fa::Params p{};
  fill_common(p, s, a->scale, a->mask);
  p.q = tensor(a->q); p.k = tensor(a->k); p.v = tensor(a->v); p.o = tensor(a->o);
  p.lse = a->lse;
  p.vt = ws;
  p.vt_ss = vt_keys(s);
  p.bias_s = bias_copy_bytes(s, a->mask) ? reinterpret_cast<float*>(static_cast<char*>(ws) + vt_bytes(s)) : nullptr;
  hipError_t e = s.dtype == FA_BF16 ? fa::launch_fwd_bf16(p, stream) : fa::launch_fwd_f32(p, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s launch failed: %s", fn, hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

const char* fa_last_error(void) { return g_error.c_str(); }

size_t fa_fwd_workspace_bytes(const fa_fwd_args* a) {
  if (!a) return 0;
  Shape s{a->dtype, a->B, a->Hq, a->Hkv, a->Sq, a->Skv, a->D};
  return fwd_ws_bytes(s, a->mask);
}

fa_status fa_fwd(const fa_fwd_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_run(a, ws, ws_bytes, stream, false);
}

fa_status fa_fwd_noalloc(const fa_fwd_args* a, hipStream_t stream) {
  return fwd_run(a, nullptr, kNoAllocScratchBytes, stream, true);
}

size_t fa_bwd_workspace_bytes(const fa_bwd_args* a) {
  if (!a) return 0;
  Shape s{a->dtype, a->B, a->Hq, a->Hkv, a->Sq, a->Skv, a->D};
  return delta_bytes(s, a->mask);
}

// Validates a backward call and launches the requested stages in order.
static fa_status bwd_run(const fa_bwd_args* a, void* ws, size_t ws_bytes, hipStream_t stream,
                         int first_stage, int last_stage) {
  if (!a) return fail(FA_ERR_INVALID_ARG, "fa_bwd: args is NULL");
  Shape s{a->dtype, a->B, a->Hq, a->Hkv, a->Sq, a->Skv, a->D};
  fa_status st = check_shape(s, a->mask);
  if (st != FA_OK) return st;
  const int eb = elem_bytes(s.dtype);
  if ((st = check_tensor("q", a->q, s.B, s.Hq, s.Sq, s.D, eb, false))) return st;
  if ((st = check_tensor("k", a->k, s.B, s.Hkv, s.Skv, s.D, eb, false))) return st;
  if ((st = check_tensor("v", a->v, s.B, s.Hkv, s.Skv, s.D, eb, false))) return st;
  if ((st = check_tensor("o", a->o, s.B, s.Hq, s.Sq, s.D, eb, false))) return st;
  if ((st = check_tensor("dout", a->dout, s.B, s.Hq, s.Sq, s.D, eb, false))) return st;
  if ((st = check_tensor("dq", a->dq, s.B, s.Hq, s.Sq, s.D, eb, true))) return st;
  if ((st = check_tensor("dk", a->dk, s.B, s.Hkv, s.Skv, s.D, eb, true))) return st;
  if ((st = check_tensor("dv", a->dv, s.B, s.Hkv, s.Skv, s.D, eb, true))) return st;
  const bool rows = s.B > 0 && s.Sq > 0;
  if (rows && a->lse == nullptr) return fail(FA_ERR_INVALID_ARG, "lse: NULL pointer");
  if (rows && reinterpret_cast<uintptr_t>(a->lse) % 4 != 0)
    return fail(FA_ERR_ALIGNMENT, "lse: pointer is not 4-byte aligned");
  const size_t need = delta_bytes(s, a->mask);
  if ((st = check_ws(ws, ws_bytes, need))) return st;
  if (a->mask.kv_valid && reinterpret_cast<uintptr_t>(a->mask.kv_valid) % 4 != 0)
    return fail(FA_ERR_ALIGNMENT, "kv_valid: pointer is not 4-byte aligned");

  Range in[7] = {span(a->q, s.B, s.Hq, s.Sq, s.D, eb), span(a->k, s.B, s.Hkv, s.Skv, s.D, eb),
                 span(a->v, s.B, s.Hkv, s.Skv, s.D, eb), span(a->o, s.B, s.Hq, s.Sq, s.D, eb),
                 span(a->dout, s.B, s.Hq, s.Sq, s.D, eb),
                 {reinterpret_cast<uintptr_t>(a->lse),
                  reinterpret_cast<uintptr_t>(a->lse) + (size_t)s.B * s.Hq * s.Sq * 4, !rows},
                 bias_span(s, a->mask)};
  Range out[4] = {span(a->dq, s.B, s.Hq, s.Sq, s.D, eb), span(a->dk, s.B, s.Hkv, s.Skv, s.D, eb),
                  span(a->dv, s.B, s.Hkv, s.Skv, s.D, eb),
                  {reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + need, need == 0}};
  const char* out_names[4] = {"dq", "dk", "dv", "workspace"};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlap(out[i], in[j])) return fail(FA_ERR_ALIAS, "%s overlaps an input tensor", out_names[i]);
    for (int j = i + 1; j < 4; ++j)
      if (overlap(out[i], out[j]))
        return fail(FA_ERR_ALIAS, "%s overlaps %s", out_names[i], out_names[j]);
  }
  const bool keys = s.B > 0 && s.Skv > 0;
  if (!rows && !keys) return FA_OK;
  if ((st = check_device())) return st;

  fa::Params p{};
  fill_common(p, s, a->scale, a->mask);
  p.q = tensor(a->q); p.k = tensor(a->k); p.v = tensor(a->v); p.o = tensor(a->o);
  p.dout = tensor(a->dout); p.dq = tensor(a->dq); p.dk = tensor(a->dk); p.dv = tensor(a->dv);
  p.lse_in = a->lse;
  p.delta = static_cast<float*>(ws);
  p.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + row_array_bytes(s));
  p.dkv_part = part_bytes(s, a->mask.kind) ? reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * row_array_bytes(s))
                                            : nullptr;
  p.vt_ss = vt_keys(s);   // the row length of the scaled key-bias copy
  p.bias_s = bias_copy_bytes(s, a->mask)
                 ? reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * row_array_bytes(s) + part_bytes(s, a->mask.kind))
                 : nullptr;
  // The whole backward in bf16 runs the two gradient stages as one
  // (fa::STAGE_GRADS): the same workgroups, bitwise the same results.
  const bool whole = first_stage == fa::STAGE_DELTA && last_stage == fa::STAGE_DQ && s.dtype == FA_BF16;
  for (int stage = first_stage; stage <= last_stage; ++stage) {
    const int run = whole && stage == fa::STAGE_DKDV ? fa::STAGE_GRADS : stage;
    hipError_t e = s.dtype == FA_BF16 ? fa::launch_bwd_bf16(p, run, stream)
                                      : fa::launch_bwd_f32(p, run, stream);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_bwd launch failed: %s", hipGetErrorString(e));
    if (run == fa::STAGE_GRADS) break;
  }
  return FA_OK;
}

fa_status fa_bwd(const fa_bwd_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  return bwd_run(a, ws, ws_bytes, stream, fa::STAGE_DELTA, fa::STAGE_DQ);
}

fa_status fa_bwd_stage(const fa_bwd_args* a, int stage, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (stage != FA_BWD_DELTA && stage != FA_BWD_DKDV && stage != FA_BWD_DQ)
    return fail(FA_ERR_INVALID_ARG, "fa_bwd_stage: unknown stage %d", stage);
  return bwd_run(a, ws, ws_bytes, stream, stage, stage);
}

}  // extern "C"

// ---- soft-target log-softmax loss ------------------------------------------

namespace {

// Byte range of n floats at p (empty when n == 0 or p is null).
Range span_f(const void* p, int64_t n) {
  if (p == nullptr || n <= 0) return Range{0, 0, true};
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)n * 4, false};
}

// Checks shared by the loss forward and backward; fills the launch params.
fa_status check_loss(const fa_lsm_loss_args* a, bool backward, fa::LossParams& p) {
  const char* fn = backward ? "fa_lsm_loss_bwd" : "fa_lsm_loss_fwd";
  if (!a) return fail(FA_ERR_INVALID_ARG, "%s: args is NULL", fn);
  if (a->N < 0) return fail(FA_ERR_INVALID_ARG, "%s: negative N=%d", fn, a->N);
  if (a->V < 1) return fail(FA_ERR_INVALID_ARG, "%s: V=%d (needs at least one column)", fn, a->V);
  const int64_t N = a->N, V = a->V;
  if (N > 0) {
    if (!a->logits || !a->target) return fail(FA_ERR_INVALID_ARG, "%s: NULL logits or target", fn);
    if (!a->m || !a->d || !a->tsum) return fail(FA_ERR_INVALID_ARG, "%s: NULL m, d or tsum", fn);
    if (!backward && !a->row_loss) return fail(FA_ERR_INVALID_ARG, "%s: NULL row_loss", fn);
    if (backward && !a->grad_loss) return fail(FA_ERR_INVALID_ARG, "%s: NULL grad_loss", fn);
    if (a->logits_ss < V || a->target_ss < V)
      return fail(FA_ERR_INVALID_ARG, "%s: row stride below V (logits_ss %lld, target_ss %lld, V %d)", fn,
                  (long long)a->logits_ss, (long long)a->target_ss, a->V);
    if (reinterpret_cast<uintptr_t>(a->logits) % 4 || reinterpret_cast<uintptr_t>(a->target) % 4)
      return fail(FA_ERR_ALIGNMENT, "%s: logits and target must be 4-byte aligned", fn);
    if ((N - 1) * std::max(a->logits_ss, a->target_ss) + V >= (int64_t(1) << 40))
      return fail(FA_ERR_UNSUPPORTED, "%s: [N, V] matrices too large", fn);
  }
  if (!backward && !a->loss) return fail(FA_ERR_INVALID_ARG, "%s: NULL loss", fn);
  for (const void* q : {(const void*)a->mask, (const void*)a->m, (const void*)a->d, (const void*)a->tsum,
                        (const void*)a->row_loss, (const void*)a->loss, (const void*)a->grad_loss})
    if (reinterpret_cast<uintptr_t>(q) % 4)
      return fail(FA_ERR_ALIGNMENT, "%s: a per-row array or scalar is not 4-byte aligned", fn);
  const Range rx = N ? span_f(a->logits, (N - 1) * a->logits_ss + V) : Range{0, 0, true};
  const Range rt = N ? span_f(a->target, (N - 1) * a->target_ss + V) : Range{0, 0, true};
  const Range rw = span_f(a->mask, N), rm = span_f(a->m, N), rd = span_f(a->d, N), rs = span_f(a->tsum, N);
  if (!backward) {
    const Range rr = span_f(a->row_loss, N), rl = span_f(a->loss, 1);
    const Range outs[5] = {rm, rd, rs, rr, rl};
    for (int o = 0; o < 5; ++o) {
      if (overlap(outs[o], rx) || overlap(outs[o], rt) || overlap(outs[o], rw))
        return fail(FA_ERR_ALIAS, "%s: an output overlaps logits, target or mask", fn);
      for (int o2 = 0; o2 < o; ++o2)
        if (overlap(outs[o], outs[o2])) return fail(FA_ERR_ALIAS, "%s: two outputs overlap", fn);
    }
  } else {
    const Range rg = span_f(a->grad_loss, 1);
    for (const Range* in : {&rt, &rw, &rm, &rd, &rs, &rg})
      if (overlap(rx, *in)) return fail(FA_ERR_ALIAS, "%s: logits (the gradient's buffer) overlap an input", fn);
  }
  p = fa::LossParams{a->N, a->V, a->logits, a->logits_ss, a->target, a->target_ss, a->mask,
                     a->m, a->d, a->tsum, a->row_loss, a->loss, a->grad_loss};
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_lsm_loss_fwd(const fa_lsm_loss_args* a, hipStream_t stream) {
  fa::LossParams p{};
  fa_status st = check_loss(a, false, p);
  if (st != FA_OK) return st;
  if ((st = check_device())) return st;
  hipError_t e = fa::launch_lsm_loss_fwd(p, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_lsm_loss_fwd launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

fa_status fa_lsm_loss_bwd(const fa_lsm_loss_args* a, hipStream_t stream) {
  fa::LossParams p{};
  fa_status st = check_loss(a, true, p);
  if (st != FA_OK) return st;
  if (a->N == 0) return FA_OK;   // nothing to write
  if ((st = check_device())) return st;
  hipError_t e = fa::launch_lsm_loss_bwd(p, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_lsm_loss_bwd launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // extern "C"
