// Backward pre-pass: Delta_i = sum_d dO[i,d] * O[i,d] for every query row.
//
// Delta is the row term of the softmax Jacobian, dS = P * (dP - Delta), that
// both backward kernels need (the backward work list of the MLX pull request
// "[Metal] Add Flash Attention VJP for training", author's reply: recompute the
// scores, load the logsumexp, form P, compute the gradients). It uses the O the
// caller passes in, i.e. exactly what the forward stored. HBM-bound: one read of
// O and dO, one fp32 write per row.
#include "device_common.h"
#include "kernels.h"

namespace sdpa {
namespace {

constexpr int kDeltaThreads = 256;

__device__ __forceinline__ void load8(const float* p, float* x) {
  const f32x4_t a = *(const f32x4_t*)p, b = *(const f32x4_t*)(p + 4);
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
template <typename T>
__device__ __forceinline__ void load8_16(const T* p, float* x) {
  const u32x4_t w = gload16B(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = lo_f32<T>(w[i]);
    x[2 * i + 1] = hi_f32<T>(w[i]);
  }
}
__device__ __forceinline__ void load8(const bf16_t* p, float* x) { load8_16<bf16_t>(p, x); }
__device__ __forceinline__ void load8(const f16_t* p, float* x) { load8_16<f16_t>(p, x); }

template <typename OT, typename DT, int D>
__global__ __launch_bounds__(kDeltaThreads) void delta_kernel(const OT* __restrict__ o, const DT* __restrict__ dO,
                                                              float* __restrict__ delta, int64_t rows) {
  // Threads per row, 8 elements each; a power of two for the shuffle reduction (D = 96:
  // 16 threads, the last 4 idle).
  constexpr int TPR = (D == 96) ? 16 : D / 8;
  const int64_t row = (int64_t)blockIdx.x * (kDeltaThreads / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows && part * 8 < D) {
    float a[8], b[8];
    load8(o + row * D + part * 8, a);
    load8(dO + row * D + part * 8, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(a[i], b[i], acc);
  }
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) delta[row] = acc;
}

template <typename OT, typename DT>
hipError_t launch_od(const Shape& s, const void* o, const void* dO, float* delta, hipStream_t st) {
  const int64_t rows = s.B * s.Hq * s.Lq;
  const int tpr = s.D == 96 ? 16 : (int)(s.D / 8);
  const int64_t rpb = kDeltaThreads / tpr;
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  switch (s.D) {
    case 32: hipLaunchKernelGGL((delta_kernel<OT, DT, 32>), grid, dim3(kDeltaThreads), 0, st, (const OT*)o, (const DT*)dO, delta, rows); break;
    case 64: hipLaunchKernelGGL((delta_kernel<OT, DT, 64>), grid, dim3(kDeltaThreads), 0, st, (const OT*)o, (const DT*)dO, delta, rows); break;
    case 96: hipLaunchKernelGGL((delta_kernel<OT, DT, 96>), grid, dim3(kDeltaThreads), 0, st, (const OT*)o, (const DT*)dO, delta, rows); break;
    case 128: hipLaunchKernelGGL((delta_kernel<OT, DT, 128>), grid, dim3(kDeltaThreads), 0, st, (const OT*)o, (const DT*)dO, delta, rows); break;
    case 256: hipLaunchKernelGGL((delta_kernel<OT, DT, 256>), grid, dim3(kDeltaThreads), 0, st, (const OT*)o, (const DT*)dO, delta, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Gradient of the sinks: dsinks[h] = -sum_{b,i} exp(sink_h - LSE_bhi) * Delta_bhi. The sink
// joins each row's softmax as a key with no value, so its dP is 0 and its dS is
// -P_sink * Delta (the backward work list of the MLX pull request, author's reply, applied
// to that extra column). One workgroup per query head sums its B*Lq rows in a fixed
// order: the result does not depend on scheduling.
__global__ __launch_bounds__(kDeltaThreads) void sink_grad_kernel(const float* __restrict__ lse,
                                                                  const float* __restrict__ delta, int64_t pitch,
                                                                  int es, const float* __restrict__ sinks,
                                                                  float* __restrict__ dsinks, int B, int Hq, int Lq) {
  const int h = blockIdx.x;
  const float sk = sinks[h];
  float acc = 0.f;
  if (sk > -INFINITY) {
    for (int64_t e = threadIdx.x; e < (int64_t)B * Lq; e += kDeltaThreads) {
      const int64_t bb = e / Lq, i = e - bb * Lq;
      const int64_t bh = bb * Hq + h;
      acc = fmaf(fast_exp2((sk - lse[bh * Lq + i]) * kLog2e), delta[(bh * pitch + i) * es], acc);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  __shared__ float part[kDeltaThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kDeltaThreads / 64; ++w) t += part[w];
    dsinks[h] = -t;
  }
}

}  // namespace

hipError_t launch_sink_grad(const Shape& s, const float* lse, const float* delta, int64_t pitch, int es,
                            const float* sinks, float* dsinks, hipStream_t st) {
  hipLaunchKernelGGL(sink_grad_kernel, dim3((unsigned)s.Hq), dim3(kDeltaThreads), 0, st, lse, delta, pitch, es, sinks,
                     dsinks, (int)s.B, (int)s.Hq, (int)s.Lq);
  return hipGetLastError();
}

hipError_t launch_delta(const Shape& s, Dt o_dt, Dt do_dt, const void* o, const void* dO, float* delta,
                        hipStream_t st) {
  if (do_dt == kF32) return launch_od<float, float>(s, o, dO, delta, st);
  if (do_dt == kBF16) return o_dt == kF32 ? launch_od<float, bf16_t>(s, o, dO, delta, st) : launch_od<bf16_t, bf16_t>(s, o, dO, delta, st);
  if (do_dt == kF16) return o_dt == kF32 ? launch_od<float, f16_t>(s, o, dO, delta, st) : launch_od<f16_t, f16_t>(s, o, dO, delta, st);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
