// float32 attention: forward, Delta pre-pass, dQ and dK/dV kernels on the vector ALUs.
//
// The float32 workloads on the pages are small (PyTensor issue "PERF: detect
// scaled-dot-product-attention pattern ...", "Reproducer + metrics": B=8, H=8,
// S=128, D=64) and their stated accuracy is 1e-5 ("Acceptance criteria"), so this
// path keeps every product and sum in fp32 and runs on the VALUs: R lanes share one
// row, each holding a W-element slice (W = 2 at D = 32 and 4 at D = 64 and 128: short
// per-lane chains and a large grid for these small shapes; W = 8 at D = 256, where R = 32
// is the most a row's lane sum takes; R = 8 lanes of 12 at D = 96 so that R stays a power
// of two). It follows the same online softmax (exp2 domain) and the same two-kernel
// backward without atomics as the 16-bit path (MLX pull request "[Metal] Add Flash
// Attention VJP for training", "Implementation Notes").
#include "device_common.h"
#include "kernels.h"

namespace sdpa {
namespace {

constexpr int kF32Threads = 256;
constexpr int kF32BN = 32;  // rows of the streamed operand per LDS tile

// Sum over the R (a power of two, <= 32) lanes of a row: a butterfly that adds the partner
// lane's value at distance 1, 2, 4, ... (lane ^ d). Distances 1 and 2 are DPP quad
// permutes on the vector ALU; 4, 8 and 16 are ds_swizzle in its bit-mask mode (and 0x1f,
// xor d), which needs no address register.
template <int R>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(R >= 1 && R <= 32 && (R & (R - 1)) == 0, "lanes per row: a power of two up to 32");
  if constexpr (R >= 2) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  if constexpr (R >= 4) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  if constexpr (R >= 8) x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (4 << 10) | 0x1F));
  if constexpr (R >= 16) x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (8 << 10) | 0x1F));
  if constexpr (R >= 32) x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (16 << 10) | 0x1F));
  return x;
}

// LDS tile of kF32BN rows: slice s of a row starts at s*(W+1) so that the R lanes
// of a row (reading different slices of the same row) hit different banks.
template <int D>
struct F32Tile {
  static constexpr int R = D == 96 ? 8 : D == 256 ? 32 : D == 32 ? 16 : D / 4;  // lanes per row
  static constexpr int W = D / R;                   // elements of a lane's slice
  static constexpr int SP = W + 1;                  // slice pitch in LDS
  static constexpr int PITCH = R * SP;
  static constexpr int ELEMS = kF32BN * PITCH;
  __device__ static int idx(int row, int d) { return row * PITCH + (d / W) * SP + d % W; }
};

// One kF32BN-row tile of a row-major [L, D] matrix in the registers of the workgroup's
// threads (16-byte loads; rows >= L read as zero), so that the next tile's global loads
// are in flight while the current tile is consumed from LDS.
// Keys (or queries) of a tile unrolled in the backward loops: all of them, so that the
// lane reductions of different keys overlap; 4 with a mask, whose loads and offsets would
// not fit the registers with every key in flight.
template <bool HAS_MASK>
constexpr int unroll_keys() {
  return HAS_MASK ? 4 : kF32BN;
}

template <int D>
struct F32Stage {
  static constexpr int N4 = kF32BN * D / 4 / kF32Threads;  // 16-byte pieces per thread
  static_assert(kF32BN * D / 4 % kF32Threads == 0, "whole 16-byte pieces per thread");
  f32x4_t x[N4];
  __device__ __forceinline__ void load(const float* src, int r0, int L) {
#pragma unroll
    for (int i = 0; i < N4; ++i) {
      const int e4 = (int)threadIdx.x + i * kF32Threads, r = e4 / (D / 4), c = (e4 % (D / 4)) * 4;
      x[i] = (r0 + r < L) ? *(const f32x4_t*)(src + (int64_t)(r0 + r) * D + c) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }
  }
  __device__ __forceinline__ void store(float* lds) const {
#pragma unroll
    for (int i = 0; i < N4; ++i) {
      const int e4 = (int)threadIdx.x + i * kF32Threads, r = e4 / (D / 4), c = (e4 % (D / 4)) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) lds[F32Tile<D>::idx(r, c + j)] = x[i][j];
    }
  }
};

template <int D>
__device__ __forceinline__ float dot_slice(const float* x, const float* lds, int row, int slice) {
  const float* p = lds + row * F32Tile<D>::PITCH + slice * F32Tile<D>::SP;
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < F32Tile<D>::W; ++e) acc = fmaf(x[e], p[e], acc);
  return acc;
}

template <int D, bool CAUSAL, bool HAS_MASK>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                               const float* __restrict__ v, float* __restrict__ o,
                                                               float* __restrict__ lse, int Hq, int G, int Lq,
                                                               int Lkv, int n_qblk, float scale_log2, Mask mask,
                                                               const float* __restrict__ sinks) {
  using TL = F32Tile<D>;
  constexpr int R = TL::R, ROWS = kF32Threads / R;
  __shared__ float k_lds[TL::ELEMS];
  __shared__ float v_lds[TL::ELEMS];
  const int bh = blockIdx.x / n_qblk, qblk = blockIdx.x - bh * n_qblk;
  const int b = bh / Hq, hq = bh - b * Hq, Hkv = Hq / G, hk = hq / G;
  const int slice = threadIdx.x % R, qrow = qblk * ROWS + threadIdx.x / R;
  const float* kh = k + (int64_t)(b * Hkv + hk) * Lkv * D;
  const float* vh = v + (int64_t)(b * Hkv + hk) * Lkv * D;
  float qv[TL::W], acc[TL::W];
#pragma unroll
  for (int e = 0; e < TL::W; ++e) {
    qv[e] = (qrow < Lq) ? q[((int64_t)bh * Lq + qrow) * D + slice * TL::W + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f, lc = 0.f;  // row max, row sum and its compensation
  if (sinks != nullptr && sinks[hq] > -INFINITY) {  // the sink: a first key with no value
    m = sinks[hq] * kLog2e;
    l = 1.f;
  }
  const int64_t mrow =
      HAS_MASK ? (int64_t)b * mask.sb + (int64_t)hq * mask.sh + (int64_t)min(qrow, Lq - 1) * mask.sq : 0;
  const int co = Lkv - Lq;  // causal offset: key j visible to query i iff j <= i + co
  const int kv_end = CAUSAL ? min(Lkv, qblk * ROWS + ROWS + co) : Lkv;
  F32Stage<D> ks, vs;
  ks.load(kh, 0, Lkv);
  vs.load(vh, 0, Lkv);
  for (int t0 = 0; t0 < kv_end; t0 += kF32BN) {
    __syncthreads();
    ks.store(k_lds);
    vs.store(v_lds);
    __syncthreads();
    if (t0 + kF32BN < kv_end) {  // the next tile streams in while this one is consumed
      ks.load(kh, t0 + kF32BN, Lkv);
      vs.load(vh, t0 + kF32BN, Lkv);
    }
    float s[kF32BN];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      float x = row_sum<R>(dot_slice<D>(qv, k_lds, j, slice)) * scale_log2;
      const int key = t0 + j;
      if (HAS_MASK && key < Lkv) x += mask_bias_log2<float>(mask.p, mask.kind, mrow + key);
      if (key >= Lkv || (CAUSAL && key > qrow + co)) x = -INFINITY;
      s[j] = x;
      tmax = fmaxf(tmax, x);
    }
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    l *= alpha;
    lc *= alpha;
#pragma unroll
    for (int e = 0; e < TL::W; ++e) acc[e] *= alpha;
    float tsum = 0.f;  // the tile's probabilities, added to the row sum once
#pragma unroll
    for (int j = 0; j < kF32BN; ++j) {
      const float p = fast_exp2(s[j] - m_use);
      tsum += p;
      const float* vr = v_lds + j * TL::PITCH + slice * TL::SP;
#pragma unroll
      for (int e = 0; e < TL::W; ++e) acc[e] = fmaf(p, vr[e], acc[e]);
    }
    kahan_add(l, lc, tsum);
  }
  if (qrow < Lq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < TL::W; ++e) o[((int64_t)bh * Lq + qrow) * D + slice * TL::W + e] = acc[e] * inv;
    if (lse != nullptr && slice == 0) lse[(int64_t)bh * Lq + qrow] = (m + fast_log2(l)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool HAS_MASK>
__global__ __launch_bounds__(kF32Threads) void dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                              const float* __restrict__ v, const float* __restrict__ lse,
                                                              const float* __restrict__ dO,
                                                              const float* __restrict__ o, float* __restrict__ delta,
                                                              float* __restrict__ dq, int Hq, int G, int Lq, int Lkv,
                                                              int n_qblk, float scale_log2, float scale, Mask mask) {
  using TL = F32Tile<D>;
  constexpr int R = TL::R, ROWS = kF32Threads / R;
  constexpr int kUnrollKeys = unroll_keys<HAS_MASK>();
  __shared__ float k_lds[TL::ELEMS];
  __shared__ float v_lds[TL::ELEMS];
  const int bh = blockIdx.x / n_qblk, qblk = blockIdx.x - bh * n_qblk;
  const int b = bh / Hq, hq = bh - b * Hq, Hkv = Hq / G, hk = hq / G;
  const int slice = threadIdx.x % R, qrow = qblk * ROWS + threadIdx.x / R;
  const float* kh = k + (int64_t)(b * Hkv + hk) * Lkv * D;
  const float* vh = v + (int64_t)(b * Hkv + hk) * Lkv * D;
  const bool valid = qrow < Lq;
  const int64_t roff = ((int64_t)bh * Lq + (valid ? qrow : 0)) * D + slice * TL::W;
  float qv[TL::W], dov[TL::W], acc[TL::W];
  float dpart = 0.f;  // this lane's share of Delta = sum_d dO * O, from the O the caller passes in
#pragma unroll
  for (int e = 0; e < TL::W; ++e) {
    qv[e] = valid ? q[roff + e] : 0.f;
    dov[e] = valid ? dO[roff + e] : 0.f;
    dpart = fmaf(dov[e], valid ? o[roff + e] : 0.f, dpart);
    acc[e] = 0.f;
  }
  float lse2 = valid ? lse[(int64_t)bh * Lq + qrow] * kLog2e : 0.f;
  if (HAS_MASK && lse2 == -INFINITY) lse2 = INFINITY;  // a masked row with no key: P = 0
  const float dlt = row_sum<R>(dpart);
  if (valid && slice == 0) delta[(int64_t)bh * Lq + qrow] = dlt;  // for the dK/dV kernel and the sinks' gradient
  const int64_t mrow =
      HAS_MASK ? (int64_t)b * mask.sb + (int64_t)hq * mask.sh + (int64_t)min(qrow, Lq - 1) * mask.sq : 0;
  const int co = Lkv - Lq;  // causal offset: key j visible to query i iff j <= i + co
  const int kv_end = CAUSAL ? min(Lkv, qblk * ROWS + ROWS + co) : Lkv;
  F32Stage<D> ks, vs;
  ks.load(kh, 0, Lkv);
  vs.load(vh, 0, Lkv);
  for (int t0 = 0; t0 < kv_end; t0 += kF32BN) {
    __syncthreads();
    ks.store(k_lds);
    vs.store(v_lds);
    __syncthreads();
    if (t0 + kF32BN < kv_end) {
      ks.load(kh, t0 + kF32BN, Lkv);
      vs.load(vh, t0 + kF32BN, Lkv);
    }
#pragma unroll(kUnrollKeys)
    for (int j = 0; j < kF32BN; ++j) {
      const float sv = row_sum<R>(dot_slice<D>(qv, k_lds, j, slice));
      const float dp = row_sum<R>(dot_slice<D>(dov, v_lds, j, slice));
      const int key = t0 + j;
      const float nb = HAS_MASK && key < Lkv ? mask_bias_log2<float>(mask.p, mask.kind, mrow + key) - lse2 : -lse2;
      float p = exp2_le1(fmaf(sv, scale_log2, nb));
      if (key >= Lkv || (CAUSAL && key > qrow + co)) p = 0.f;
      const float ds = p * (dp - dlt);
      const float* kr = k_lds + j * TL::PITCH + slice * TL::SP;
#pragma unroll
      for (int e = 0; e < TL::W; ++e) acc[e] = fmaf(ds, kr[e], acc[e]);
    }
  }
  if (valid) {
#pragma unroll
    for (int e = 0; e < TL::W; ++e) dq[roff + e] = acc[e] * scale;
  }
}

template <int D, bool CAUSAL, bool HAS_MASK>
__global__ __launch_bounds__(kF32Threads) void dkv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                               const float* __restrict__ v,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ dO,
                                                               const float* __restrict__ delta, float* __restrict__ dk,
                                                               float* __restrict__ dv, int Hq, int G, int Lq, int Lkv,
                                                               int n_kblk, float scale_log2, float scale, Mask mask) {
  using TL = F32Tile<D>;
  constexpr int R = TL::R, ROWS = kF32Threads / R;
  constexpr int kUnrollKeys = unroll_keys<HAS_MASK>();
  __shared__ float q_lds[TL::ELEMS];
  __shared__ float do_lds[TL::ELEMS];
  __shared__ float lse_lds[kF32BN];
  __shared__ float dl_lds[kF32BN];
  const int bhk = blockIdx.x / n_kblk, kblk = blockIdx.x - bhk * n_kblk;
  const int Hkv = Hq / G, b = bhk / Hkv, hk = bhk - b * Hkv;
  const int slice = threadIdx.x % R, krow = kblk * ROWS + threadIdx.x / R;
  const bool valid = krow < Lkv;
  const int64_t roff = ((int64_t)bhk * Lkv + (valid ? krow : 0)) * D + slice * TL::W;
  float kv_[TL::W], vv[TL::W], dka[TL::W], dva[TL::W];
#pragma unroll
  for (int e = 0; e < TL::W; ++e) {
    kv_[e] = valid ? k[roff + e] : 0.f;
    vv[e] = valid ? v[roff + e] : 0.f;
    dka[e] = 0.f;
    dva[e] = 0.f;
  }
  // Causal: queries below the first key of this block never see it.
  const int co = Lkv - Lq;  // causal offset: key j visible to query i iff j <= i + co
  const int q_begin = CAUSAL ? (max(0, kblk * ROWS - co) / kF32BN) * kF32BN : 0;
  // (head, query tile) pairs, heads outer; each pair's tiles are loaded into registers
  // while the previous pair is consumed.
  const int ntq = q_begin < Lq ? (Lq - q_begin + kF32BN - 1) / kF32BN : 0;
  F32Stage<D> qs, dos;
  float l2n = 0.f, dln = 0.f;  // LSE*log2e and Delta of query threadIdx.x of the loaded tile
  auto load = [&](int it) {
    const int t0 = q_begin + (it % ntq) * kF32BN;
    const int64_t qbase = (int64_t)(b * Hq + hk * G + it / ntq) * Lq;
    qs.load(q + qbase * D, t0, Lq);
    dos.load(dO + qbase * D, t0, Lq);
    if (threadIdx.x < kF32BN) {
      const int i = t0 + threadIdx.x;
      l2n = (i < Lq) ? lse[qbase + i] * kLog2e : 0.f;
      dln = (i < Lq) ? delta[qbase + i] : 0.f;
    }
  };
  if (ntq > 0) load(0);
  for (int it = 0; it < G * ntq; ++it) {
    const int gi = it / ntq, hq = hk * G + gi, t0 = q_begin + (it % ntq) * kF32BN;
    {
      __syncthreads();
      qs.store(q_lds);
      dos.store(do_lds);
      if (threadIdx.x < kF32BN) {
        lse_lds[threadIdx.x] = (HAS_MASK && l2n == -INFINITY) ? INFINITY : l2n;  // no key: P = 0
        dl_lds[threadIdx.x] = dln;
      }
      __syncthreads();
      if (it + 1 < G * ntq) load(it + 1);
#pragma unroll(kUnrollKeys)
      for (int j = 0; j < kF32BN; ++j) {
        const int i = t0 + j;
        const float sv = row_sum<R>(dot_slice<D>(kv_, q_lds, j, slice));
        const float dp = row_sum<R>(dot_slice<D>(vv, do_lds, j, slice));
        float nb = -lse_lds[j];
        if constexpr (HAS_MASK)
          nb += mask_bias_log2<float>(mask.p, mask.kind,
                                      (int64_t)b * mask.sb + (int64_t)hq * mask.sh +
                                          (int64_t)min(i, Lq - 1) * mask.sq + min(krow, Lkv - 1));
        float p = exp2_le1(fmaf(sv, scale_log2, nb));
        if (i >= Lq || (CAUSAL && krow > i + co)) p = 0.f;
        const float ds = p * (dp - dl_lds[j]);
        const float* qr = q_lds + j * TL::PITCH + slice * TL::SP;
        const float* dr = do_lds + j * TL::PITCH + slice * TL::SP;
#pragma unroll
        for (int e = 0; e < TL::W; ++e) {
          dva[e] = fmaf(p, dr[e], dva[e]);
          dka[e] = fmaf(ds, qr[e], dka[e]);
        }
      }
    }
  }
  if (valid) {
#pragma unroll
    for (int e = 0; e < TL::W; ++e) {
      dk[roff + e] = dka[e] * scale;
      dv[roff + e] = dva[e];
    }
  }
}

template <int D, bool C, bool M>
hipError_t fwd_typed(const Shape& s, const Mask& mask, const float* sinks, const float* q, const float* k,
                     const float* v, float* o, float* lse, float scale, hipStream_t st) {
  constexpr int ROWS = kF32Threads / F32Tile<D>::R;
  const int n_qblk = (int)((s.Lq + ROWS - 1) / ROWS);
  hipLaunchKernelGGL((fwd_f32_kernel<D, C, M>), dim3(n_qblk * s.B * s.Hq), dim3(kF32Threads), 0, st, q, k, v, o,
                     lse, (int)s.Hq, (int)(s.Hq / s.Hkv), (int)s.Lq, (int)s.Lkv, n_qblk,
                     (float)((double)scale * 1.4426950408889634), mask, sinks);
  return hipGetLastError();
}

template <int D, bool C, bool M>
hipError_t bwd_typed(const Shape& s, const Mask& mask, const float* q, const float* k, const float* v, const float* o,
                     const float* lse, const float* dO, float* delta, float* dq, float* dk, float* dv,
                     float scale, int stages, hipStream_t st) {
  constexpr int ROWS = kF32Threads / F32Tile<D>::R;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  if (stages & kStage0) {
    const int n_qblk = (int)((s.Lq + ROWS - 1) / ROWS);
    hipLaunchKernelGGL((dq_f32_kernel<D, C, M>), dim3(n_qblk * s.B * s.Hq), dim3(kF32Threads), 0, st, q, k, v, lse,
                       dO, o, delta, dq, (int)s.Hq, (int)(s.Hq / s.Hkv), (int)s.Lq, (int)s.Lkv, n_qblk, scale_log2,
                       scale, mask);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(stages & kStage1)) return hipSuccess;
  const int n_kblk = (int)((s.Lkv + ROWS - 1) / ROWS);
  hipLaunchKernelGGL((dkv_f32_kernel<D, C, M>), dim3(n_kblk * s.B * s.Hkv), dim3(kF32Threads), 0, st, q, k, v, lse,
                     dO, delta, dk, dv, (int)s.Hq, (int)(s.Hq / s.Hkv), (int)s.Lq, (int)s.Lkv, n_kblk, scale_log2,
                     scale, mask);
  return hipGetLastError();
}

template <int D>
hipError_t fwd_mode(const Shape& s, bool causal, const Mask& mask, const float* sinks, const float* q, const float* k,
                    const float* v, float* o, float* lse, float scale, hipStream_t st) {
  if (causal) return fwd_typed<D, true, false>(s, mask, sinks, q, k, v, o, lse, scale, st);
  if (mask.kind != kMaskNone) return fwd_typed<D, false, true>(s, mask, sinks, q, k, v, o, lse, scale, st);
  return fwd_typed<D, false, false>(s, mask, sinks, q, k, v, o, lse, scale, st);
}

template <int D>
hipError_t bwd_mode(const Shape& s, bool causal, const Mask& mask, const float* q, const float* k, const float* v, const float* o,
                    const float* lse, const float* dO, float* delta, float* dq, float* dk, float* dv,
                    float scale, int stages, hipStream_t st) {
  if (causal) return bwd_typed<D, true, false>(s, mask, q, k, v, o, lse, dO, delta, dq, dk, dv, scale, stages, st);
  if (mask.kind != kMaskNone)
    return bwd_typed<D, false, true>(s, mask, q, k, v, o, lse, dO, delta, dq, dk, dv, scale, stages, st);
  return bwd_typed<D, false, false>(s, mask, q, k, v, o, lse, dO, delta, dq, dk, dv, scale, stages, st);
}

}  // namespace

hipError_t launch_fwd_f32(const Shape& s, bool causal, const Mask& mask, const float* sinks, const float* q,
                          const float* k, const float* v, float* o, float* lse, float scale, hipStream_t st) {
  switch (s.D) {
    case 32: return fwd_mode<32>(s, causal, mask, sinks, q, k, v, o, lse, scale, st);
    case 64: return fwd_mode<64>(s, causal, mask, sinks, q, k, v, o, lse, scale, st);
    case 96: return fwd_mode<96>(s, causal, mask, sinks, q, k, v, o, lse, scale, st);
    case 128: return fwd_mode<128>(s, causal, mask, sinks, q, k, v, o, lse, scale, st);
    case 256: return fwd_mode<256>(s, causal, mask, sinks, q, k, v, o, lse, scale, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_f32(const Shape& s, bool causal, const Mask& mask, const float* q, const float* k,
                          const float* v, const float* o, const float* lse, const float* dO, float* dq, float* dk,
                          float* dv, float* delta, float scale, int stages, hipStream_t st) {
  switch (s.D) {
    case 32: return bwd_mode<32>(s, causal, mask, q, k, v, o, lse, dO, delta, dq, dk, dv, scale, stages, st);
    case 64: return bwd_mode<64>(s, causal, mask, q, k, v, o, lse, dO, delta, dq, dk, dv, scale, stages, st);
    case 96: return bwd_mode<96>(s, causal, mask, q, k, v, o, lse, dO, delta, dq, dk, dv, scale, stages, st);
    case 128: return bwd_mode<128>(s, causal, mask, q, k, v, o, lse, dO, delta, dq, dk, dv, scale, stages, st);
    case 256: return bwd_mode<256>(s, causal, mask, q, k, v, o, lse, dO, delta, dq, dk, dv, scale, stages, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdpa
