// Gradient of the per-head sinks from Delta_i = sum_d dO[i,d] * O[i,d], the row term of
// the softmax Jacobian, dS = P * (dP - Delta) (the backward work list of the MLX pull
// request "[Metal] Add Flash Attention VJP for training", author's reply: recompute the
// scores, load the logsumexp, form P, compute the gradients). Every backward forms Delta
// inside its first kernel, from the O the caller passes in, and leaves it in the
// workspace; this kernel reads it there.
#include "device_common.h"
#include "kernels.h"

namespace sdpa {
namespace {

constexpr int kDeltaThreads = 256;

// Gradient of the sinks: dsinks[h] = -sum_{b,i} exp(sink_h - LSE_bhi) * Delta_bhi. The sink
// joins each row's softmax as a key with no value, so its dP is 0 and its dS is
// -P_sink * Delta (the backward work list of the MLX pull request, author's reply, applied
// to that extra column). One workgroup per query head sums its B*Lq rows in a fixed
// order: the result does not depend on scheduling.
__global__ __launch_bounds__(kDeltaThreads) void sink_grad_kernel(const float* __restrict__ lse,
                                                                  const float* __restrict__ delta, int64_t pitch,
                                                                  int es, float dsign, const float* __restrict__ sinks,
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
    dsinks[h] = -dsign * t;  // the stored values are dsign * Delta
  }
}

}  // namespace

hipError_t launch_sink_grad(const Shape& s, const float* lse, const float* delta, int64_t pitch, int es, float dsign,
                            const float* sinks, float* dsinks, hipStream_t st) {
  hipLaunchKernelGGL(sink_grad_kernel, dim3((unsigned)s.Hq), dim3(kDeltaThreads), 0, st, lse, delta, pitch, es, dsign,
                     sinks, dsinks, (int)s.B, (int)s.Hq, (int)s.Lq);
  return hipGetLastError();
}

}  // namespace sdpa
