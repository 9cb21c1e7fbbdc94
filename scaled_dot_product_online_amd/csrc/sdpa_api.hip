// C ABI of the attention library: argument validation, kernel-family selection,
// workspace sizing and dispatch. Everything here runs on the host; nothing is
// enqueued until every check has passed. The contract is documented in
// include/sdpa.h.
#include <math.h>
#include <stdint.h>

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

size_t ws_bytes(int backward, const Shape& s, int path) {
  if (!backward) return path == SDPA_PATH_VECTOR ? align_up(sdpa::vector_fwd_workspace(s)) : 0;
  // The vector backward forms Delta inside its kernel; the fp32 path keeps Delta and the
  // tiled path {LSE*log2e, Delta} pairs per query row in the workspace.
  if (path == SDPA_PATH_VECTOR) return align_up(sdpa::vector_bwd_workspace(s));
  if (path == SDPA_PATH_TILED) return align_up((size_t)(s.B * s.Hq * sdpa::tiled_rowstat_stride(s.Lq)) * 8);
  return delta_bytes(s);
}

sdpa_status_t device_status(hipError_t e) { return e == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE; }

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
  return ws_bytes(backward, s, path_of(Hq, Hkv, Lq, is_causal, dtype));
}

sdpa_status_t sdpa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal,
                       sdpa_dtype_t dtype, sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  sdpa_status_t st = check_shape(B, Hq, Hkv, Lq, Lkv, D, is_causal, dtype, out_dtype);
  if (st != SDPA_OK) return st;
  if (!isfinite(scale)) return SDPA_ERR_VALUE;
  if (!q || !k || !v || !o) return SDPA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return SDPA_ERR_ALIGN;
  const Shape s{B, Hq, Hkv, Lq, Lkv, D};
  const int path = path_of(Hq, Hkv, Lq, is_causal, dtype);
  const size_t need = ws_bytes(0, s, path);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return SDPA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return SDPA_ERR_ALIGN;
  }
  hipStream_t hs = (hipStream_t)stream;
  const bool causal = is_causal != 0;
  switch (path) {
    case SDPA_PATH_FP32:
      return device_status(sdpa::launch_fwd_f32(s, causal, (const float*)q, (const float*)k, (const float*)v,
                                                (float*)o, lse, scale, hs));
    case SDPA_PATH_VECTOR:
      return device_status(sdpa::launch_fwd_vector(s, (sdpa::Dt)dtype, (sdpa::Dt)out_dtype, causal, q, k, v, o, lse, scale,
                                                   workspace, hs));
    default:
      return device_status(
          sdpa::launch_fwd_tiled(s, (sdpa::Dt)dtype, (sdpa::Dt)out_dtype, causal, q, k, v, o, lse, scale, hs));
  }
}

}  // extern "C"

namespace {

sdpa_status_t run_bwd(int stages, const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                      int64_t Lkv, int64_t D, float scale, int is_causal, sdpa_dtype_t dtype, sdpa_dtype_t out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  sdpa_status_t st = check_shape(B, Hq, Hkv, Lq, Lkv, D, is_causal, dtype, out_dtype);
  if (st != SDPA_OK) return st;
  if (!isfinite(scale)) return SDPA_ERR_VALUE;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return SDPA_ERR_NULL;
  const void* ptrs[] = {q, k, v, o, lse, dO, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SDPA_ERR_ALIGN;
  const Shape s{B, Hq, Hkv, Lq, Lkv, D};
  const int path = path_of(Hq, Hkv, Lq, is_causal, dtype);
  const size_t need = ws_bytes(1, s, path);
  if (!workspace || workspace_bytes < need) return SDPA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & (kWsAlign - 1)) != 0) return SDPA_ERR_ALIGN;
  hipStream_t hs = (hipStream_t)stream;
  const bool causal = is_causal != 0;
  float* delta = (float*)workspace;
  switch (path) {
    case SDPA_PATH_FP32:
      return device_status(sdpa::launch_bwd_f32(s, causal, (const float*)q, (const float*)k, (const float*)v,
                                                (const float*)o, lse, (const float*)dO, (float*)dq, (float*)dk,
                                                (float*)dv, delta, scale, stages, hs));
    case SDPA_PATH_VECTOR:
      return device_status(sdpa::launch_bwd_vector(s, (sdpa::Dt)dtype, (sdpa::Dt)out_dtype, causal, q, k, v, o, lse, dO, dq,
                                                   dk, dv, workspace, scale, stages, hs));
    default:
      return device_status(sdpa::launch_bwd_tiled(s, (sdpa::Dt)dtype, (sdpa::Dt)out_dtype, causal, q, k, v, o, lse,
                                                  dO, dq, dk, dv, delta, scale, stages, hs));
  }
}

}  // namespace

extern "C" {

sdpa_status_t sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                       void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv,
                       int64_t D, float scale, int is_causal, sdpa_dtype_t dtype, sdpa_dtype_t out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return run_bwd(sdpa::kStagesAll, q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lkv, D, scale, is_causal, dtype,
                 out_dtype, workspace, workspace_bytes, stream);
}

sdpa_status_t sdpa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                             int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal, sdpa_dtype_t dtype,
                             sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (stage != 0 && stage != 1) return SDPA_ERR_VALUE;
  return run_bwd(stage == 0 ? sdpa::kStage0 : sdpa::kStage1, q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lkv, D,
                 scale, is_causal, dtype, out_dtype, workspace, workspace_bytes, stream);
}

const char* sdpa_status_str(sdpa_status_t status) {
  switch (status) {
    case SDPA_OK: return "ok";
    case SDPA_ERR_NULL: return "a required pointer is NULL";
    case SDPA_ERR_SHAPE: return "invalid shape (size < 1, Hq not a multiple of Hkv, or too large)";
    case SDPA_ERR_UNSUPPORTED: return "unsupported combination (head dim, dtype, or causal with Lq != Lkv)";
    case SDPA_ERR_WORKSPACE: return "workspace missing or smaller than sdpa_workspace_bytes()";
    case SDPA_ERR_ALIGN: return "pointer not 16-byte aligned (workspace: 256-byte)";
    case SDPA_ERR_DEVICE: return "HIP runtime rejected a kernel launch";
    case SDPA_ERR_VALUE: return "scale is not finite";
    default: return "unknown status";
  }
}

}  // extern "C"
