// C ABI of the attention library: argument validation, kernel-family selection,
// workspace sizing and dispatch. Everything here runs on the host; nothing is
// enqueued until every check has passed. The contract is documented in
// include/sdpa.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/sdpa.h"
#include "kernels.h"

namespace {

using sdpa::Shape;

constexpr int64_t kMaxLen = int64_t(1) << 30;   // row indices are 32-bit inside the kernels
constexpr int64_t kMaxRows = int64_t(1) << 31;  // B*H*L rows, and workgroup counts
constexpr size_t kWsAlign = 256;
constexpr int64_t kMaxHeadBytes = (int64_t(1) << 31) - 1;

bool is_dtype(int d) { return d == SDPA_F32 || d == SDPA_F16 || d == SDPA_BF16; }

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool mul3(int64_t a, int64_t b, int64_t c, int64_t* out) {
  int64_t t;
  return !__builtin_mul_overflow(a, b, &t) && !__builtin_mul_overflow(t, c, out);
}

// Shape / dtype checks shared by every entry point.
sdpa_status_t check_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, int is_causal,
                          int dtype, int out_dtype) {
  if (!is_dtype(dtype) || !is_dtype(out_dtype)) return SDPA_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lkv < 1 || D < 1) return SDPA_ERR_SHAPE;
  if (Hq % Hkv != 0) return SDPA_ERR_SHAPE;
  if (D != 32 && D != 64 && D != 96 && D != 128 && D != 256) return SDPA_ERR_UNSUPPORTED;
  if (is_causal && Lq > Lkv) return SDPA_ERR_UNSUPPORTED;  // every query row must see a key
  if (out_dtype != dtype && out_dtype != SDPA_F32) return SDPA_ERR_UNSUPPORTED;
  if (Lq > kMaxLen || Lkv > kMaxLen) return SDPA_ERR_SHAPE;
  int64_t rq, rk, eq, ek;
  if (!mul3(B, Hq, Lq, &rq) || !mul3(B, Hkv, Lkv, &rk)) return SDPA_ERR_SHAPE;
  if (rq >= kMaxRows || rk >= kMaxRows) return SDPA_ERR_SHAPE;
  if (__builtin_mul_overflow(rq, D, &eq) || __builtin_mul_overflow(rk, D, &ek)) return SDPA_ERR_SHAPE;
  if (eq > (INT64_MAX >> 3) || ek > (INT64_MAX >> 3)) return SDPA_ERR_SHAPE;
  // One head's rows (plus a tile of slack) must be addressable with 32-bit byte offsets.
  const int64_t esz = dtype == SDPA_F32 ? 4 : 2;
  if ((Lq + 256) * D * esz > kMaxHeadBytes || (Lkv + 256) * D * esz > kMaxHeadBytes) return SDPA_ERR_SHAPE;
  return SDPA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int path_of(int64_t Hq, int64_t Hkv, int64_t Lq, int is_causal, int dtype) {
  if (dtype == SDPA_F32) return SDPA_PATH_FP32;
  return (Lq <= 8 && (Hq / Hkv) * Lq <= 32) ? SDPA_PATH_VECTOR : SDPA_PATH_TILED;
}

size_t delta_bytes(const Shape& s) { return align_up((size_t)(s.B * s.Hq * s.Lq) * sizeof(float)); }

size_t ws_bytes(int backward, const Shape& s, int path, bool causal) {
  if (!backward) {
    if (path == SDPA_PATH_VECTOR) return align_up(sdpa::vector_fwd_workspace(s));
    if (path == SDPA_PATH_TILED) return align_up(sdpa::tiled_fwd_workspace(s));  // key-split partials, small grids
    return 0;
  }
  // The vector backward forms Delta inside its kernel; the fp32 path keeps Delta and the
  // tiled path {LSE*log2e, -Delta} pairs per query row in the workspace.
  if (path == SDPA_PATH_VECTOR) return align_up(sdpa::vector_bwd_workspace(s));
  if (path == SDPA_PATH_TILED) return align_up(sdpa::tiled_bwd_workspace(s, causal));  // + split partials, small grids
  return delta_bytes(s);
}

sdpa_status_t device_status(hipError_t e) { return e == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE; }

// Mask arguments of the *_masked entry points; fills `m` for the kernels.
sdpa_status_t check_mask(int kind, const void* mask, int64_t sb, int64_t sh, int64_t sq, int64_t B, int64_t Hq,
                         int64_t Lq, int64_t Lkv, int is_causal, int dtype, sdpa::Mask* m) {
  *m = sdpa::kNoMask;
  if (kind == SDPA_MASK_NONE) return SDPA_OK;
  if (kind != SDPA_MASK_BOOL && kind != SDPA_MASK_ADDITIVE) return SDPA_ERR_VALUE;
  if (is_causal) return SDPA_ERR_UNSUPPORTED;
  if (!mask) return SDPA_ERR_NULL;
  if (sb < 0 || sh < 0 || sq < 0) return SDPA_ERR_SHAPE;
  // Largest element offset: (B-1)*sb + (Hq-1)*sh + (Lq-1)*sq + Lkv - 1, in int64.
  int64_t t0, t1, t2, last;
  if (__builtin_mul_overflow(B - 1, sb, &t0) || __builtin_mul_overflow(Hq - 1, sh, &t1) ||
      __builtin_mul_overflow(Lq - 1, sq, &t2) || __builtin_add_overflow(t0, t1, &last) ||
      __builtin_add_overflow(last, t2, &last) || __builtin_add_overflow(last, Lkv, &last) ||
      last > (INT64_MAX >> 3))
    return SDPA_ERR_SHAPE;
  const uintptr_t esz = kind == SDPA_MASK_BOOL ? 1 : (dtype == SDPA_F32 ? 4 : 2);
  if (((uintptr_t)mask & (esz - 1)) != 0) return SDPA_ERR_ALIGN;
  const bool vec4 = ((uintptr_t)mask % (4 * esz)) == 0 && sb % 4 == 0 && sh % 4 == 0 && sq % 4 == 0 && Lkv % 4 == 0;
  *m = sdpa::Mask{mask, kind == SDPA_MASK_BOOL ? sdpa::kMaskBool : sdpa::kMaskAdd, vec4 ? 1 : 0, sb, sh, sq};
  return SDPA_OK;
}

sdpa_status_t run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal, int mask_kind,
                      const void* mask_p, int64_t msb, int64_t msh, int64_t msq, const float* sinks,
                      sdpa_dtype_t dtype, sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  sdpa_status_t st = check_shape(B, Hq, Hkv, Lq, Lkv, D, is_causal, dtype, out_dtype);
  if (st != SDPA_OK) return st;
  if (!isfinite(scale)) return SDPA_ERR_VALUE;
  sdpa::Mask mask;
  st = check_mask(mask_kind, mask_p, msb, msh, msq, B, Hq, Lq, Lkv, is_causal, dtype, &mask);
  if (st != SDPA_OK) return st;
  if (!q || !k || !v || !o) return SDPA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return SDPA_ERR_ALIGN;
  if (((uintptr_t)sinks & 3u) != 0) return SDPA_ERR_ALIGN;
  const Shape s{B, Hq, Hkv, Lq, Lkv, D};
  const int path = path_of(Hq, Hkv, Lq, is_causal, dtype);
  const size_t need = ws_bytes(0, s, path, is_causal != 0);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return SDPA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return SDPA_ERR_ALIGN;
  }
  hipStream_t hs = (hipStream_t)stream;
  const bool causal = is_causal != 0;
  switch (path) {
    case SDPA_PATH_FP32:
      return device_status(sdpa::launch_fwd_f32(s, causal, mask, sinks, (const float*)q, (const float*)k,
                                                (const float*)v, (float*)o, lse, scale, hs));
    case SDPA_PATH_VECTOR:
      return device_status(sdpa::launch_fwd_vector(s, (sdpa::Dt)dtype, (sdpa::Dt)out_dtype, causal, mask, sinks, q, k,
                                                   v, o, lse, scale, workspace, hs));
    default:
      return device_status(sdpa::launch_fwd_tiled(s, (sdpa::Dt)dtype, (sdpa::Dt)out_dtype, causal, mask, sinks, q, k,
                                                  v, o, lse, scale, workspace, hs));
  }
}

}  // namespace

extern "C" {

int sdpa_select_path(int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, int is_causal, sdpa_dtype_t dtype) {
  if (check_shape(1, Hq, Hkv, Lq, Lkv, D, is_causal, dtype, dtype) != SDPA_OK) return -1;
  return path_of(Hq, Hkv, Lq, is_causal, dtype);
}

size_t sdpa_workspace_bytes(int backward, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D,
                            int is_causal, sdpa_dtype_t dtype) {
  if (check_shape(B, Hq, Hkv, Lq, Lkv, D, is_causal, dtype, dtype) != SDPA_OK) return (size_t)-1;
  const Shape s{B, Hq, Hkv, Lq, Lkv, D};
  return ws_bytes(backward, s, path_of(Hq, Hkv, Lq, is_causal, dtype), is_causal != 0);
}

sdpa_status_t sdpa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal,
                       sdpa_dtype_t dtype, sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return run_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lkv, D, scale, is_causal, SDPA_MASK_NONE, nullptr, 0, 0, 0, nullptr,
                 dtype, out_dtype, workspace, workspace_bytes, stream);
}

sdpa_status_t sdpa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                              int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal,
                              sdpa_mask_kind_t mask_kind, const void* mask, int64_t mask_stride_b,
                              int64_t mask_stride_h, int64_t mask_stride_q, const float* sinks, sdpa_dtype_t dtype,
                              sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return run_fwd(q, k, v, o, lse, B, Hq, Hkv, Lq, Lkv, D, scale, is_causal, mask_kind, mask, mask_stride_b,
                 mask_stride_h, mask_stride_q, sinks, dtype, out_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

sdpa_status_t run_bwd(int stages, const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                      int64_t Lkv, int64_t D, float scale, int is_causal, int mask_kind, const void* mask_p,
                      int64_t msb, int64_t msh, int64_t msq, const float* sinks, float* dsinks, sdpa_dtype_t dtype,
                      sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  sdpa_status_t st = check_shape(B, Hq, Hkv, Lq, Lkv, D, is_causal, dtype, out_dtype);
  if (st != SDPA_OK) return st;
  if (!isfinite(scale)) return SDPA_ERR_VALUE;
  sdpa::Mask mask;
  st = check_mask(mask_kind, mask_p, msb, msh, msq, B, Hq, Lq, Lkv, is_causal, dtype, &mask);
  if (st != SDPA_OK) return st;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return SDPA_ERR_NULL;
  if (sinks && !dsinks) return SDPA_ERR_NULL;
  if (((uintptr_t)sinks & 3u) != 0 || ((uintptr_t)dsinks & 3u) != 0) return SDPA_ERR_ALIGN;
  const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SDPA_ERR_ALIGN;
  const Shape s{B, Hq, Hkv, Lq, Lkv, D};
  const int path = path_of(Hq, Hkv, Lq, is_causal, dtype);
  const size_t need = ws_bytes(1, s, path, is_causal != 0);
  if (!workspace || workspace_bytes < need) return SDPA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return SDPA_ERR_ALIGN;
  hipStream_t hs = (hipStream_t)stream;
  const bool causal = is_causal != 0;
  float* delta = (float*)workspace;
  hipError_t e;
  // Where stage 0 leaves Delta_i (times dsign) for the sinks' gradient: element (bh * pitch + i) * es.
  const float* dl;
  int64_t pitch;
  int es;
  float dsign = 1.f;
  switch (path) {
    case SDPA_PATH_FP32:
      e = sdpa::launch_bwd_f32(s, causal, mask, (const float*)q, (const float*)k, (const float*)v, (const float*)o,
                               lse, (const float*)dO, (float*)dq, (float*)dk, (float*)dv, delta, scale, stages, hs);
      dl = delta, pitch = Lq, es = 1;
      break;
    case SDPA_PATH_VECTOR:
      e = sdpa::launch_bwd_vector(s, (sdpa::Dt)dtype, (sdpa::Dt)out_dtype, causal, mask, q, k, v, o, lse, dO, dq, dk,
                                  dv, workspace, scale, stages, hs);
      dl = (const float*)((const char*)workspace + sdpa::vector_bwd_delta_offset(s)), pitch = Lq, es = 1;
      break;
    default:
      e = sdpa::launch_bwd_tiled(s, (sdpa::Dt)dtype, (sdpa::Dt)out_dtype, causal, mask, q, k, v, o, lse, dO, dq, dk,
                                 dv, delta, scale, stages, hs);
      dl = delta + 1, pitch = sdpa::tiled_rowstat_stride(Lq), es = 2, dsign = -1.f;  // {LSE*log2e, -Delta} pairs
      break;
  }
  if (e == hipSuccess && sinks && (stages & sdpa::kStage1))
    e = sdpa::launch_sink_grad(s, lse, dl, pitch, es, dsign, sinks, dsinks, hs);
  return device_status(e);
}

}  // namespace

extern "C" {

sdpa_status_t sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                       void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv,
                       int64_t D, float scale, int is_causal, sdpa_dtype_t dtype, sdpa_dtype_t out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return run_bwd(sdpa::kStagesAll, q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lkv, D, scale, is_causal,
                 SDPA_MASK_NONE, nullptr, 0, 0, 0, nullptr, nullptr, dtype, out_dtype, workspace, workspace_bytes,
                 stream);
}

sdpa_status_t sdpa_bwd_masked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                              int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal,
                              sdpa_mask_kind_t mask_kind, const void* mask, int64_t mask_stride_b,
                              int64_t mask_stride_h, int64_t mask_stride_q, const float* sinks, float* dsinks,
                              sdpa_dtype_t dtype, sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return run_bwd(sdpa::kStagesAll, q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lkv, D, scale, is_causal,
                 mask_kind, mask, mask_stride_b, mask_stride_h, mask_stride_q, sinks, dsinks, dtype, out_dtype,
                 workspace, workspace_bytes, stream);
}

sdpa_status_t sdpa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                             int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal, sdpa_dtype_t dtype,
                             sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (stage != 0 && stage != 1) return SDPA_ERR_VALUE;
  return run_bwd(stage == 0 ? sdpa::kStage0 : sdpa::kStage1, q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lkv, D,
                 scale, is_causal, SDPA_MASK_NONE, nullptr, 0, 0, 0, nullptr, nullptr, dtype, out_dtype, workspace,
                 workspace_bytes, stream);
}

sdpa_status_t sdpa_bwd_masked_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dO, void* dq, void* dk, void* dv, int64_t B,
                                    int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, float scale,
                                    int is_causal, sdpa_mask_kind_t mask_kind, const void* mask,
                                    int64_t mask_stride_b, int64_t mask_stride_h, int64_t mask_stride_q,
                                    const float* sinks, float* dsinks, sdpa_dtype_t dtype, sdpa_dtype_t out_dtype,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (stage != 0 && stage != 1) return SDPA_ERR_VALUE;
  return run_bwd(stage == 0 ? sdpa::kStage0 : sdpa::kStage1, q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lkv, D,
                 scale, is_causal, mask_kind, mask, mask_stride_b, mask_stride_h, mask_stride_q, sinks, dsinks, dtype,
                 out_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- the backward without a workspace argument ------------------------------------------
// The fixed scratch of sdpa_bwd_noalloc. In host code `scratch` names a host-side stand-in,
// not device memory: the device address of each GPU's copy comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is used.
static __device__ __align__(256) uint8_t scratch[SDPA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, null until first looked up

// Device address of the current device's scratch, or null on failure.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

sdpa_status_t sdpa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                               int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal, sdpa_dtype_t dtype,
                               sdpa_dtype_t out_dtype, void* stream) {
  // Sizes first (a pure host check), so that an oversized call fails before any device call.
  sdpa_status_t st = check_shape(B, Hq, Hkv, Lq, Lkv, D, is_causal, dtype, out_dtype);
  if (st != SDPA_OK) return st;
  const size_t need = ws_bytes(1, Shape{B, Hq, Hkv, Lq, Lkv, D}, path_of(Hq, Hkv, Lq, is_causal, dtype),
                               is_causal != 0);
  if (need > SDPA_NOALLOC_SCRATCH_BYTES) return SDPA_ERR_WORKSPACE;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return SDPA_ERR_NULL;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return SDPA_ERR_DEVICE;
  return run_bwd(sdpa::kStagesAll, q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lkv, D, scale, is_causal,
                 SDPA_MASK_NONE, nullptr, 0, 0, 0, nullptr, nullptr, dtype, out_dtype, ws,
                 SDPA_NOALLOC_SCRATCH_BYTES, stream);
}

const char* sdpa_status_str(sdpa_status_t status) {
  switch (status) {
    case SDPA_OK: return "ok";
    case SDPA_ERR_NULL: return "a required pointer is NULL";
    case SDPA_ERR_SHAPE: return "invalid shape (size < 1, Hq not a multiple of Hkv, or too large)";
    case SDPA_ERR_UNSUPPORTED: return "unsupported combination (head dim, dtype, causal with Lq > Lkv or with a mask)";
    case SDPA_ERR_WORKSPACE: return "workspace missing or smaller than sdpa_workspace_bytes()";
    case SDPA_ERR_ALIGN: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case SDPA_ERR_DEVICE: return "HIP runtime rejected a kernel launch";
    case SDPA_ERR_VALUE: return "scale is not finite, or an invalid stage number or mask kind";
    default: return "unknown status";
  }
}

}  // extern "C"
