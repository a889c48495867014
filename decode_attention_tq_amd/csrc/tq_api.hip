// C ABI of the TurboQuant packed-KV library: argument validation (before any
// HIP call), workspace planning and kernel dispatch.
#include <math.h>

#include <mutex>

#include "tq_internal.h"

namespace tq {

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool is_fp16_exact(float v) { return (float)(_Float16)v == v; }

// Validates the descriptor itself; returns TQ_OK or an error code.
int check_cache(const tq_cache* c) {
  if (c == nullptr) return TQ_ERR_INVALID_ARGUMENT;
  if (c->role != TQ_KEYS && c->role != TQ_VALUES) return TQ_ERR_INVALID_ARGUMENT;
  if (c->bits < 2 || c->bits > 4) return TQ_ERR_UNSUPPORTED;
  if (c->qjl != 0 && c->qjl != 1) return TQ_ERR_INVALID_ARGUMENT;
  if (c->qjl && c->role != TQ_KEYS) return TQ_ERR_UNSUPPORTED;
  // head dimension 128 (the tuned kernels) or 64 / 256 (the generic ones, no QJL)
  if (c->d != 64 && c->d != kD && c->d != 256) return TQ_ERR_UNSUPPORTED;
  if (c->d != kD && c->qjl) return TQ_ERR_UNSUPPORTED;
  if (c->B <= 0 || c->H_kv <= 0 || c->T_cap <= 0) return TQ_ERR_INVALID_ARGUMENT;
  if (c->B > 65535 || c->H_kv > 65535) return TQ_ERR_UNSUPPORTED;
  if (c->role == TQ_VALUES && c->T_cap % kValueBlock != 0) return TQ_ERR_INVALID_ARGUMENT;
  if (c->block_table != nullptr) {
    // paged: power-of-two blocks of 32 .. 65536 tokens (a decode step never
    // crosses one), whole blocks per row, each array below 2 GiB (32-bit offsets)
    const int64_t bt = c->block_tokens;
    if (bt < 32 || bt > 65536 || (bt & (bt - 1)) != 0) return TQ_ERR_INVALID_ARGUMENT;
    if (c->T_cap % bt != 0 || c->n_blocks <= 0) return TQ_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)c->block_table & 3) != 0) return TQ_ERR_ALIGNMENT;
    if (c->n_blocks > ((int64_t)1 << 31) / (c->H_kv * bt)) return TQ_ERR_UNSUPPORTED;
    if (cache_rows(c) * (int64_t)c->d * c->bits / 8 >= (int64_t)1 << 31) return TQ_ERR_UNSUPPORTED;
  } else {
    // per-head byte ranges are addressed with 32-bit offsets
    if (c->T_cap * (int64_t)c->d * c->bits / 8 >= (int64_t)1 << 31) return TQ_ERR_UNSUPPORTED;
  }
  if (c->codes == nullptr || c->norms == nullptr || c->rot == nullptr) return TQ_ERR_INVALID_ARGUMENT;
  if (c->qjl && (c->qjl_signs == nullptr || c->qjl_gamma == nullptr || c->qjl_proj == nullptr))
    return TQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(c->codes) || !aligned16(c->norms) || !aligned16(c->rot)) return TQ_ERR_ALIGNMENT;
  if (c->qjl && (!aligned16(c->qjl_signs) || !aligned16(c->qjl_gamma) || !aligned16(c->qjl_proj)))
    return TQ_ERR_ALIGNMENT;
  const int L = 1 << c->bits;
  for (int i = 0; i < L; ++i) {
    if (!isfinite(c->centroids[i]) || !is_fp16_exact(c->centroids[i])) return TQ_ERR_INVALID_ARGUMENT;
    if (i > 0 && !(c->centroids[i] > c->centroids[i - 1])) return TQ_ERR_INVALID_ARGUMENT;
  }
  return TQ_OK;
}

// HIP error of the last failed device call made by an entry point on this thread.
thread_local hipError_t t_last_hip_error = hipSuccess;

// Status of a device call; the HIP error of a failure is kept for
// tq_last_hip_error.
int device_status(hipError_t e) {
  if (e == hipSuccess) return TQ_OK;
  t_last_hip_error = e;
  return TQ_ERR_DEVICE;
}

// Entry points check the launch error of their own kernels: an error left
// pending by an earlier, unrelated HIP call on this thread (one that did not
// poison the device) is cleared before they launch, so it is not reported as
// theirs. A device that did fault fails the launch itself.
void clear_pending_error() { (void)hipGetLastError(); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool plan_decode(int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int32_t n_split, int32_t qjl,
                 DecodePlan* p, int64_t M, int32_t d) {
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || T < 0 || n_split < 0 || M <= 0) return false;
  if (H_q % H_kv != 0) return false;
  const int64_t G = H_q / H_kv;
  if (G > 16) return false;
  p->B = B;
  p->H_q = H_q;
  p->H_kv = H_kv;
  p->T = T;
  p->M = M;
  p->G = (int32_t)G;
  p->wide = M * G > 8;
  p->Mt = (int32_t)(p->wide ? (M < 16 / G ? M : 16 / G) : M);
  p->nqt = (int32_t)((M + p->Mt - 1) / p->Mt);
  if (B * p->nqt > 65535) return false;   // grid z
  p->qjl = qjl ? 1 : 0;
  const int64_t Tp = T > 0 ? T : 1;
  const int64_t quantum = kChunkQuantum;
  int64_t target;
  if (n_split > 0) {
    target = n_split;
  } else {
    // about one workgroup per compute unit; a chunk keeps at least 2 quanta
    const int64_t units = B * H_kv * p->nqt;
    target = (kDecodeTargetWGs + units - 1) / units;
    const int64_t cap = (Tp + 2 * quantum - 1) / (2 * quantum);
    if (target > cap) target = cap;
    if (target < 1) target = 1;
  }
  int64_t chunk = (Tp + target - 1) / target;
  chunk = (chunk + quantum - 1) / quantum * quantum;
  p->chunk = (int32_t)chunk;
  p->n_split = (int32_t)((Tp + chunk - 1) / chunk);
  if (p->n_split > 1 && B * M * H_q * d / 256 >= INT32_MAX) return false;   // grid of the chunk merge
  size_t off = 0;
  p->off_ml = off;
  off = align256(off + (size_t)(B * M * H_q) * p->n_split * 2 * sizeof(float));
  p->off_acc = off;
  off = align256(off + (size_t)(B * M * H_q) * p->n_split * d * sizeof(float));
  p->bytes = off;
  return true;
}

bool plan_prefill_dense(int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int64_t M, int32_t n_split, DensePlan* p) {
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || T < 0 || n_split < 0 || M <= 1) return false;
  if (H_q % H_kv != 0) return false;
  const int64_t G = H_q / H_kv;
  if (G > 16 || M * G > (int64_t)1 << 30) return false;
  p->B = B;
  p->H_q = H_q;
  p->H_kv = H_kv;
  p->T = T;
  p->M = M;
  p->G = (int32_t)G;
  p->NC = (int32_t)(M * G);
  const int64_t waves = (p->NC + kDenseWaveCols - 1) / kDenseWaveCols;
  p->nwave = waves >= 4 ? 4 : (waves >= 2 ? 2 : 1);
  p->ncg = (int32_t)((p->NC + kDenseWaveCols * p->nwave - 1) / (kDenseWaveCols * p->nwave));
  if (B * p->ncg > 65535 || B * M > 65535) return false;   // grid z of the scan; rows
  if (B * M * H_q * kD / 256 >= INT32_MAX) return false;      // grid of the chunk merge (d threads a vector)
  const int64_t Tp = T > 0 ? T : 1;
  int64_t target;
  if (n_split > 0) {
    target = n_split;
  } else {
    // about two wavefronts per SIMD of a 256-CU part; chunks of at least 512 tokens
    const int64_t units = B * H_kv * p->ncg * p->nwave;
    target = (8 * kDecodeTargetWGs + units - 1) / units;
    const int64_t cap = (Tp + 511) / 512;
    if (target > cap) target = cap;
    if (target < 1) target = 1;
  }
  int64_t chunk = (Tp + target - 1) / target;
  chunk = (chunk + kStep - 1) / kStep * kStep;
  p->chunk = (int32_t)chunk;
  p->n_split = (int32_t)((Tp + chunk - 1) / chunk);
  size_t off = 0;
  p->off_ml = off;
  off = align256(off + (size_t)(B * M * H_q) * p->n_split * 2 * sizeof(float));
  p->off_acc = off;
  off = align256(off + (size_t)(B * M * H_q) * p->n_split * kD * sizeof(float));
  p->bytes = off;
  return true;
}

}  // namespace tq

using namespace tq;

extern "C" const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_ALIGNMENT: return "misaligned device pointer";
    case TQ_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case TQ_ERR_DEVICE: return "HIP device error";
    default: return "unknown status";
  }
}

extern "C" const char* tq_last_hip_error(void) { return hipGetErrorName(t_last_hip_error); }

extern "C" int32_t tq_decode_splits(int64_t B, int64_t H_kv, int64_t T, int32_t n_split) {
  DecodePlan p;
  if (!plan_decode(B, H_kv, H_kv, T, n_split, 0, &p)) return 0;
  return p.n_split;
}

extern "C" size_t tq_prefill_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t M, int64_t T,
                                             int32_t n_split, int32_t k_qjl) {
  // enough for every head dimension: the dense plan (d = 128) where it
  // applies, and the scan tiles' plan at the largest d that takes them (256
  // up to 8 (token, head) columns per KV head, else 128; d = 64 needs less)
  if (H_kv <= 0 || H_q % H_kv != 0 || M <= 0) return 0;
  size_t bytes = 0;
  if (use_dense_prefill(M, H_q / H_kv, k_qjl)) {
    DensePlan dp;
    if (!plan_prefill_dense(B, H_q, H_kv, T, M, n_split, &dp)) return 0;
    bytes = dp.bytes;
  }
  DecodePlan p;
  const int32_t dmax = M * (H_q / H_kv) <= 8 ? 256 : kD;
  if (plan_decode(B, H_q, H_kv, T, n_split, k_qjl, &p, M, dmax)) bytes = bytes > p.bytes ? bytes : p.bytes;
  return bytes;
}

extern "C" size_t tq_decode_workspace_bytes(int64_t B, int64_t H_q, int64_t H_kv, int64_t T,
                                            int32_t n_split, int32_t k_qjl) {
  DecodePlan p;   // (sized for the largest head dimension, 256)
  if (!plan_decode(B, H_q, H_kv, T, n_split, k_qjl, &p, 1, 256)) return 0;
  return p.bytes;
}

extern "C" int tq_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                              void* hip_stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 || workgroups <= 0 || workgroups > 65535)
    return TQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(src) || bytes % 16 != 0 || ((uintptr_t)sink & 3u) != 0) return TQ_ERR_ALIGNMENT;
  // each workgroup's slice is addressed with 32-bit offsets
  if ((bytes + (size_t)workgroups - 1) / (size_t)workgroups >= ((size_t)1 << 31)) return TQ_ERR_UNSUPPORTED;
  clear_pending_error();
  return device_status(launch_stream_read(src, bytes, sink, workgroups, (hipStream_t)hip_stream));
}

extern "C" int tq_quantize_kv(const void* x, int32_t x_dtype, int64_t B, int64_t T, int64_t H_kv,
                              int64_t stride_b, int64_t stride_t, int64_t stride_h,
                              const tq_cache* dst, int64_t t_offset, void* hip_stream) {
  int st = check_cache(dst);
  if (st != TQ_OK) return st;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_ERR_INVALID_ARGUMENT;
  if (B != dst->B || H_kv != dst->H_kv || T < 0 || t_offset < 0 || t_offset + T > dst->T_cap)
    return TQ_ERR_INVALID_ARGUMENT;
  if (T == 0) return TQ_OK;
  if (x == nullptr || stride_b < 0 || stride_t < 0 || stride_h < 0) return TQ_ERR_INVALID_ARGUMENT;
  const int64_t esz = x_dtype == TQ_F32 ? 4 : 2;
  const int64_t vec_align = 16 / esz;   // every row starts on a 16-byte boundary
  if (!aligned16(x) || stride_b % vec_align || stride_t % vec_align || stride_h % vec_align)
    return TQ_ERR_ALIGNMENT;
  clear_pending_error();
  if (dst->d != kD)
    return device_status(launch_quantize_generic(x, x_dtype, B, T, H_kv, stride_b, stride_t, stride_h, dst,
                                                 t_offset, nullptr, 0, (hipStream_t)hip_stream));
  return device_status(launch_quantize(x, x_dtype, B, T, H_kv, stride_b, stride_t, stride_h, dst, t_offset,
                                       (hipStream_t)hip_stream));
}

extern "C" int tq_append_kv(const void* k, const void* v, int32_t x_dtype, int64_t B, int64_t H_kv,
                            int64_t k_stride_b, int64_t k_stride_h, int64_t v_stride_b, int64_t v_stride_h,
                            const tq_cache* kc, const tq_cache* vc, int64_t t_offset, void* hip_stream) {
  int st = check_cache(kc);
  if (st != TQ_OK) return st;
  st = check_cache(vc);
  if (st != TQ_OK) return st;
  if (kc->role != TQ_KEYS || vc->role != TQ_VALUES) return TQ_ERR_INVALID_ARGUMENT;
  if (kc->d != vc->d) return TQ_ERR_INVALID_ARGUMENT;
  if (x_dtype != TQ_F32 && x_dtype != TQ_BF16) return TQ_ERR_INVALID_ARGUMENT;
  if (B != kc->B || B != vc->B || H_kv != kc->H_kv || H_kv != vc->H_kv) return TQ_ERR_INVALID_ARGUMENT;
  if (t_offset < 0 || t_offset >= kc->T_cap || t_offset >= vc->T_cap) return TQ_ERR_INVALID_ARGUMENT;
  if (k == nullptr || v == nullptr || k_stride_b < 0 || k_stride_h < 0 || v_stride_b < 0 || v_stride_h < 0)
    return TQ_ERR_INVALID_ARGUMENT;
  const int64_t vec_align = 16 / (x_dtype == TQ_F32 ? 4 : 2);   // every row starts on a 16-byte boundary
  if (!aligned16(k) || !aligned16(v) || k_stride_b % vec_align || k_stride_h % vec_align ||
      v_stride_b % vec_align || v_stride_h % vec_align)
    return TQ_ERR_ALIGNMENT;
  clear_pending_error();
  if (kc->d != kD) {
    const hipError_t e = launch_quantize_generic(k, x_dtype, B, 1, H_kv, k_stride_b, 0, k_stride_h, kc, t_offset,
                                                 nullptr, 0, (hipStream_t)hip_stream);
    if (e != hipSuccess) return device_status(e);
    return device_status(launch_quantize_generic(v, x_dtype, B, 1, H_kv, v_stride_b, 0, v_stride_h, vc, t_offset,
                                                 nullptr, 0, (hipStream_t)hip_stream));
  }
  return device_status(launch_append_kv(k, v, x_dtype, B, H_kv, k_stride_b, k_stride_h, v_stride_b, v_stride_h,
                                        kc, vc, t_offset, (hipStream_t)hip_stream));
}

extern "C" int tq_dequantize(const tq_cache* src, int64_t t0, int64_t t1, float* out, void* hip_stream) {
  int st = check_cache(src);
  if (st != TQ_OK) return st;
  if (t0 < 0 || t1 < t0 || t1 > src->T_cap) return TQ_ERR_INVALID_ARGUMENT;
  if (t1 == t0) return TQ_OK;
  if (out == nullptr) return TQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(out)) return TQ_ERR_ALIGNMENT;
  clear_pending_error();
  if (src->d != kD) return device_status(launch_dequantize_generic(src, t0, t1, out, (hipStream_t)hip_stream));
  return device_status(launch_dequantize(src, t0, t1, out, (hipStream_t)hip_stream));
}

namespace {

// Library-owned scratch of tq_decode_attention_noalloc: the context-chunk
// partials of one call. Each GPU the library runs on holds its own copy until
// the process ends; calls on one GPU share it (overlapping calls race).
static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on each device (the host-side name is only a
// stand-in for the symbol), looked up once per device with that device
// current.
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Address of the current device's scratch; nullptr with *err set on failure.
void* scratch_address(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Where the chunk partials go: the caller's workspace, or the library's scratch.
struct WorkspaceArg {
  void* ptr;
  size_t bytes;
  bool scratch;
};

// Shared validation and launch of decode (M = 1) and chunked causal attention.
int attention_call(const tq_cache* k, const tq_cache* v, const void* q, int32_t q_dtype, int64_t H_q, int64_t M,
                   const int32_t* ctx_lens, int64_t T, float scale, int32_t n_split, float* out, WorkspaceArg wsa,
                   void* hip_stream, const DecodeAppend* app = nullptr) {
  int st = check_cache(k);
  if (st != TQ_OK) return st;
  st = check_cache(v);
  if (st != TQ_OK) return st;
  if (k->role != TQ_KEYS || v->role != TQ_VALUES) return TQ_ERR_INVALID_ARGUMENT;
  if (k->B != v->B || k->H_kv != v->H_kv) return TQ_ERR_INVALID_ARGUMENT;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID_ARGUMENT;
  if (q == nullptr || out == nullptr || H_q <= 0 || T < 0 || n_split < 0 || M <= 0) return TQ_ERR_INVALID_ARGUMENT;
  if (T > k->T_cap || T > v->T_cap || T >= ((int64_t)1 << 30)) return TQ_ERR_INVALID_ARGUMENT;
  if (H_q % k->H_kv != 0) return TQ_ERR_INVALID_ARGUMENT;
  if (H_q / k->H_kv > 16 || H_q > 65535) return TQ_ERR_UNSUPPORTED;
  if (M > 65535) return TQ_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return TQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(out)) return TQ_ERR_ALIGNMENT;
  if (k->d != v->d) return TQ_ERR_INVALID_ARGUMENT;
  // The scan tiles take every head dimension except d = 256 with more than 8
  // (query token, head) columns per KV head: a decode with G > 8 there runs
  // the generic kernel (one launch, no workspace), and chunked prefill with
  // M * G > 8 is not offered. The dense prefill kernel is d = 128 only.
  const bool generic = k->d > kD && M * (H_q / k->H_kv) > 8;
  if (generic && M != 1) return TQ_ERR_UNSUPPORTED;
  const bool dense = k->d == kD && app == nullptr && use_dense_prefill(M, H_q / k->H_kv, k->qjl);
  DecodePlan p;
  DensePlan dp;
  if (generic) {
    p.bytes = 0;
  } else if (dense) {
    if (!plan_prefill_dense(k->B, H_q, k->H_kv, T, M, n_split, &dp)) return TQ_ERR_UNSUPPORTED;
    p.bytes = dp.bytes;
  } else if (!plan_decode(k->B, H_q, k->H_kv, T, n_split, k->qjl, &p, M, k->d)) {
    return TQ_ERR_UNSUPPORTED;
  }
  if (wsa.scratch) {
    if (p.bytes > (size_t)TQ_NOALLOC_SCRATCH_BYTES) return TQ_ERR_WORKSPACE_TOO_SMALL;
  } else if (!generic) {
    if (wsa.ptr == nullptr || wsa.bytes < p.bytes) return TQ_ERR_WORKSPACE_TOO_SMALL;
    if (((uintptr_t)wsa.ptr & 255u) != 0) return TQ_ERR_ALIGNMENT;
  }
  if (scale <= 0.f) scale = 1.0f / sqrtf((float)k->d);
  if (app != nullptr) {
    if (app->x_dtype != TQ_F32 && app->x_dtype != TQ_BF16) return TQ_ERR_INVALID_ARGUMENT;
    if (app->k == nullptr || app->v == nullptr || app->k_sb < 0 || app->k_sh < 0 || app->v_sb < 0 || app->v_sh < 0)
      return TQ_ERR_INVALID_ARGUMENT;
    const int64_t vec_align = 16 / (app->x_dtype == TQ_F32 ? 4 : 2);
    if (!aligned16(app->k) || !aligned16(app->v) || app->k_sb % vec_align || app->k_sh % vec_align ||
        app->v_sb % vec_align || app->v_sh % vec_align)
      return TQ_ERR_ALIGNMENT;
    // keys with a QJL sketch take the tiled quantize kernel, which writes one
    // position for all rows
    if (k->qjl && ctx_lens != nullptr) return TQ_ERR_UNSUPPORTED;
  }
  // every argument is valid from here on
  clear_pending_error();
  if (generic) {
    if (app != nullptr && (ctx_lens != nullptr || T > 0)) {
      // the new token of each row: at ctx_lens[b] - 1, or at T - 1 for every row
      const int64_t tk = ctx_lens != nullptr ? 0 : T - 1;
      hipError_t e = launch_quantize_generic(app->k, app->x_dtype, k->B, 1, k->H_kv, app->k_sb, 0, app->k_sh, k, tk,
                                             ctx_lens, T, (hipStream_t)hip_stream);
      if (e != hipSuccess) return device_status(e);
      e = launch_quantize_generic(app->v, app->x_dtype, k->B, 1, k->H_kv, app->v_sb, 0, app->v_sh, v, tk, ctx_lens, T,
                                  (hipStream_t)hip_stream);
      if (e != hipSuccess) return device_status(e);
    }
    return device_status(
        launch_decode_generic(k, v, q, q_dtype, H_q, ctx_lens, T, scale, out, (hipStream_t)hip_stream));
  }
  void* workspace = wsa.ptr;
  if (wsa.scratch) {
    hipError_t e = hipSuccess;
    workspace = scratch_address(&e);
    if (workspace == nullptr) return device_status(e);
  }
  if (app != nullptr) {
    // d = 128 keys without a QJL sketch: the decode kernel appends the token
    // in its prologue (one launch); otherwise an append launch first
    if (k->d == kD && !k->qjl)
      return device_status(launch_decode(p, k, v, q, q_dtype, ctx_lens, scale, out, workspace,
                                         (hipStream_t)hip_stream, app));
    if ((ctx_lens != nullptr || T > 0) && k->d == kD) {
      const hipError_t e = launch_append_kv(app->k, app->v, app->x_dtype, k->B, k->H_kv, app->k_sb, app->k_sh,
                                            app->v_sb, app->v_sh, k, v, T - 1, (hipStream_t)hip_stream, ctx_lens, T);
      if (e != hipSuccess) return device_status(e);
    } else if (ctx_lens != nullptr || T > 0) {
      // other head dimensions: the generic quantize, in its one-token mode
      const int64_t tk = ctx_lens != nullptr ? 0 : T - 1;
      hipError_t e = launch_quantize_generic(app->k, app->x_dtype, k->B, 1, k->H_kv, app->k_sb, 0, app->k_sh, k, tk,
                                             ctx_lens, T, (hipStream_t)hip_stream);
      if (e != hipSuccess) return device_status(e);
      e = launch_quantize_generic(app->v, app->x_dtype, k->B, 1, k->H_kv, app->v_sb, 0, app->v_sh, v, tk, ctx_lens, T,
                                  (hipStream_t)hip_stream);
      if (e != hipSuccess) return device_status(e);
    }
    return device_status(launch_decode(p, k, v, q, q_dtype, ctx_lens, scale, out, workspace,
                                       (hipStream_t)hip_stream));
  }
  if (dense)
    return device_status(launch_prefill_dense(dp, k, v, q, q_dtype, ctx_lens, scale, out, workspace,
                                              (hipStream_t)hip_stream));
  return device_status(launch_decode(p, k, v, q, q_dtype, ctx_lens, scale, out, workspace,
                                     (hipStream_t)hip_stream));
}

}  // namespace

extern "C" int tq_decode_attention(const tq_cache* k, const tq_cache* v, const void* q, int32_t q_dtype,
                                   int64_t H_q, const int32_t* ctx_lens, int64_t T, float scale,
                                   int32_t n_split, float* out, void* workspace, size_t workspace_bytes,
                                   void* hip_stream) {
  return attention_call(k, v, q, q_dtype, H_q, 1, ctx_lens, T, scale, n_split, out,
                        WorkspaceArg{workspace, workspace_bytes, false}, hip_stream);
}

extern "C" int tq_decode_attention_noalloc(const tq_cache* k, const tq_cache* v, const void* q, int32_t q_dtype,
                                           int64_t H_q, const int32_t* ctx_lens, int64_t T, float scale,
                                           int32_t n_split, float* out, void* hip_stream) {
  return attention_call(k, v, q, q_dtype, H_q, 1, ctx_lens, T, scale, n_split, out, WorkspaceArg{nullptr, 0, true},
                        hip_stream);
}

extern "C" int tq_decode_attention_append(const tq_cache* k, const tq_cache* v, const void* k_new, const void* v_new,
                                          int32_t new_dtype, int64_t k_stride_b, int64_t k_stride_h,
                                          int64_t v_stride_b, int64_t v_stride_h, const void* q, int32_t q_dtype,
                                          int64_t H_q, const int32_t* ctx_lens, int64_t T, float scale,
                                          int32_t n_split, float* out, void* workspace, size_t workspace_bytes,
                                          void* hip_stream) {
  DecodeAppend app;
  app.k = k_new;
  app.v = v_new;
  app.x_dtype = new_dtype;
  app.k_sb = k_stride_b;
  app.k_sh = k_stride_h;
  app.v_sb = v_stride_b;
  app.v_sh = v_stride_h;
  return attention_call(k, v, q, q_dtype, H_q, 1, ctx_lens, T, scale, n_split, out,
                        WorkspaceArg{workspace, workspace_bytes, false}, hip_stream, &app);
}

extern "C" int tq_prefill_attention(const tq_cache* k, const tq_cache* v, const void* q, int32_t q_dtype,
                                    int64_t H_q, int64_t M, const int32_t* ctx_lens, int64_t T, float scale,
                                    int32_t n_split, float* out, void* workspace, size_t workspace_bytes,
                                    void* hip_stream) {
  return attention_call(k, v, q, q_dtype, H_q, M, ctx_lens, T, scale, n_split, out,
                        WorkspaceArg{workspace, workspace_bytes, false}, hip_stream);
}
