// Internal launch interface between the C-ABI layer (sdpa_api.hip) and the
// kernel translation units. Shapes are validated by the caller; every launcher
// returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

enum Dt { kF32 = 0, kF16 = 1, kBF16 = 2 };

struct Shape {
  int64_t B, Hq, Hkv, Lq, Lkv, D;
};

// Backward stages (bit mask): stage 0 and stage 1 as documented for sdpa_bwd_stage.
enum { kStage0 = 1, kStage1 = 2, kStagesAll = 3 };

// Attention mask as the kernels read it (validated by the caller). Element (b, h, i, j)
// sits at p + b*sb + h*sh + i*sq + j elements; a stride of 0 broadcasts. kind: boolean
// bytes (nonzero keeps the key) or additive values in the operand type. A mask is never
// combined with causal masking. vec4: the base and every stride are multiples of 4
// elements (16 bytes for float32 masks) and Lkv is a multiple of 4, so 4 consecutive keys
// from a key index that is a multiple of 4 are one aligned load.
enum { kMaskNone = 0, kMaskBool = 1, kMaskAdd = 2 };
struct Mask {
  const void* p;
  int kind;
  int vec4;
  int64_t sb, sh, sq;
};
constexpr Mask kNoMask = {nullptr, kMaskNone, 0, 0, 0, 0};

// A boolean mask that varies only along keys (key padding: query and head strides 0).
__device__ __forceinline__ bool is_key_padding(const Mask& mask) {
  return mask.kind == kMaskBool && mask.sq == 0 && mask.sh == 0;
}
// A boolean mask that varies along queries, with aligned rows (vec4): the tiled forward and
// dQ kernels copy its block for each key tile into LDS with K and V (dynamic LDS, one byte
// per query row and key of a tile, two buffers) instead of reading it per score from global
// memory. Launchers and kernels decide it with this same test.
__host__ __device__ inline bool mask_staged(const Mask& m) { return m.kind == kMaskBool && m.sq != 0 && m.vec4; }
// For such a mask: this lane's key key0 + lane of batch b, nonzero when kept (lanes >= n
// and keys past the end read 0). A kernel loads the bytes of its next key tile one step
// ahead and tests them with __any() when it gets there.
__device__ __forceinline__ uint32_t key_kept(const Mask& mask, int b, int key0, int n, int Lkv, int lane) {
  const int key = key0 + lane;
  return (lane < n && key < Lkv) ? ((const uint8_t*)mask.p)[(int64_t)b * mask.sb + key] : 0u;
}

// dsinks[h] = -sum_{b,i} exp(sinks[h] - lse[b,h,i]) * Delta(b,h,i), where dsign * Delta(b,h,i)
// sits at delta[((b*Hq + h) * pitch + i) * es] (sink_grad.hip). One deterministic reduction
// per head.
hipError_t launch_sink_grad(const Shape& s, const float* lse, const float* delta, int64_t pitch, int es, float dsign,
                            const float* sinks, float* dsinks, hipStream_t st);


// Tiled forward, 16-bit operands (fwd_tiled.hip). When the (query block, head) grid is too
// small to fill the chip, the keys are split over tiled_fwd_splits(s) workgroups per block,
// which write unnormalised partials into `ws` (tiled_fwd_workspace(s) bytes:
// [nsplit][B*Hq*Lq][D] fp32, then [nsplit][B*Hq*Lq] (m, l) pairs) for launch_split_combine.
int tiled_fwd_splits(const Shape& s);
size_t tiled_fwd_workspace(const Shape& s);
hipError_t launch_fwd_tiled(const Shape& s, Dt dt, Dt out, bool causal, const Mask& mask, const float* sinks,
                            const void* q, const void* k, const void* v, void* o, float* lse, float scale, void* ws,
                            hipStream_t st);

// Tiled backward, 16-bit operands (bwd_tiled.hip). `ws` is the workspace of
// tiled_bwd_workspace(s, causal) bytes: first, per (b, hq), a row of tiled_rowstat_stride(Lq)
// {LSE*log2e, -Delta} fp32 pairs; then, on small grids, fp32 partials of dQ and of dK, dV.
inline int64_t tiled_rowstat_stride(int64_t Lq) { return (Lq + 63) / 64 * 64; }
size_t tiled_bwd_workspace(const Shape& s, bool causal);
hipError_t launch_bwd_tiled(const Shape& s, Dt dt, Dt out, bool causal, const Mask& mask, const void* q,
                            const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
                            void* dk, void* dv, float* ws, float scale, int stages, hipStream_t st);

// float32 path (fp32_path.hip).
hipError_t launch_fwd_f32(const Shape& s, bool causal, const Mask& mask, const float* sinks, const float* q,
                          const float* k, const float* v, float* o, float* lse, float scale, hipStream_t st);
hipError_t launch_bwd_f32(const Shape& s, bool causal, const Mask& mask, const float* q, const float* k,
                          const float* v, const float* o, const float* lse, const float* dO, float* dq, float* dk,
                          float* dv, float* delta, float scale, int stages, hipStream_t st);

// Merges `nsplit` key-split partials (layout above; m in log2 units of the scaled
// scores, O unnormalised) into o and lse; the per-head sinks, if any, join here, once
// (vector_path.hip).
hipError_t launch_split_combine(const Shape& s, Dt out, int nsplit, const float* part_o, const float* part_ml,
                                const float* sinks, void* o, float* lse, hipStream_t st);

// out[r, :] = scale * sum_s part[s, r, :] for `rows` rows of s.D elements, summed in split
// order, stored as `out` (vector_path.hip).
hipError_t launch_split_reduce(const Shape& s, Dt out, int nsplit, const float* part, void* out_ptr, int64_t rows,
                               float scale, hipStream_t st);

// Both reductions of a split dK/dV kernel in one launch: out_a from part_a with scale_a and
// out_b from part_b with scale_b, each as launch_split_reduce (vector_path.hip).
hipError_t launch_split_reduce_pair(const Shape& s, Dt out, int nsplit, const float* part_a, void* out_a,
                                    float scale_a, const float* part_b, void* out_b, float scale_b, int64_t rows,
                                    hipStream_t st);

// Short-query path (vector_path.hip).
int vector_num_splits(const Shape& s);
size_t vector_fwd_workspace(const Shape& s);
size_t vector_bwd_workspace(const Shape& s);
// Offset (bytes) in the vector backward's workspace of its Delta array [B*Hq*Lq] fp32.
size_t vector_bwd_delta_offset(const Shape& s);
hipError_t launch_fwd_vector(const Shape& s, Dt dt, Dt out, bool causal, const Mask& mask, const float* sinks,
                             const void* q, const void* k, const void* v, void* o, float* lse, float scale, void* ws,
                             hipStream_t st);
hipError_t launch_bwd_vector(const Shape& s, Dt dt, Dt out, bool causal, const Mask& mask, const void* q,
                             const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
                             void* dk, void* dv, void* ws, float scale, int stages, hipStream_t st);

}  // namespace sdpa
