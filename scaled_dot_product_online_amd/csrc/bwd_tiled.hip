// Two-kernel backward of scaled-dot-product attention for 16-bit operands (gfx950).
//
// Gradients of sum(O * dO) (MLX pull request "[Metal] Add Flash Attention VJP for
// training", "Implementation Notes": a dQ kernel whose outer loop runs over KV
// blocks, and a dK/dV kernel in which each wave owns its key rows exclusively, so
// that the query heads of a GQA group need no atomics; the probabilities are
// recomputed from the forward's logsumexp, P = exp2(S*scale*log2e - LSE*log2e),
// with the exponent clamped above at 0):
//
//   dP = dO V^T,  Delta_i = sum_d dO_id O_id,  dS = P * (dP - Delta),
//   dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO.
//
// Kernel 1 (dq_kernel): one workgroup = 4 waves x 32 query rows of one (b, hq).
//   It first forms Delta for its rows from O and dO and stores it for kernel 2,
//   then streams K/V tiles of 64 keys through LDS. Like the forward it works on
//   transposed scores (S^T = K Q^T, dP^T = V dO^T) so that each lane owns one
//   query row; dQ^T += K^T dS^T reads K^T with the LDS transpose read.
// Kernel 2 (dkv_kernel): one workgroup = 4 waves x 32 key rows of one (b, hk);
//   the waves keep K and V of their rows in registers and accumulate dK and dV
//   while streaming Q/dO tiles of 64 queries of every query head of the group.
//   Scores are computed as S = Q K^T (lane owns one key column), which puts P
//   and dS directly in the B-operand layout of dV^T += dO^T P and
//   dK^T += Q^T dS; dO^T and Q^T are read with the LDS transpose read.
#include "device_common.h"
#include "kernels.h"

namespace sdpa {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------------
// dQ (+ Delta)
// ---------------------------------------------------------------------------------
constexpr int kDqBM = 128;  // query rows per workgroup
constexpr int kDqBN = 64;   // keys per tile

template <int D>
struct DqTile {
  static constexpr int KP = D + 8;  // 16-byte skew
  static constexpr int VP = D + 8;
  static constexpr int CPR = D / 8;
  static constexpr int RPP = kThreads / CPR;
  static constexpr int PASSES = kDqBN / RPP;
};

template <typename OutT>
__device__ __forceinline__ void load_out8(const OutT* p, float* x);
template <>
__device__ __forceinline__ void load_out8<float>(const float* p, float* x) {
  const f32x4_t a = *(const f32x4_t*)p, b = *(const f32x4_t*)(p + 4);
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
template <>
__device__ __forceinline__ void load_out8<bf16_t>(const bf16_t* p, float* x) {
  const u32x4_t w = gload16B(p);
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = lo_f32<bf16_t>(w[i]);
    x[2 * i + 1] = hi_f32<bf16_t>(w[i]);
  }
}
template <>
__device__ __forceinline__ void load_out8<f16_t>(const f16_t* p, float* x) {
  const u32x4_t w = gload16B(p);
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = lo_f32<f16_t>(w[i]);
    x[2 * i + 1] = hi_f32<f16_t>(w[i]);
  }
}

template <typename T, int D, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(kThreads, 1) void dq_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, const OutT* __restrict__ o,
                                                         const float* __restrict__ lse,
                                                         const uint16_t* __restrict__ dO, OutT* __restrict__ dq,
                                                         float* __restrict__ delta, int Hq, int G, int Lq, int Lkv,
                                                         int n_qblk, int n_bh, float scale_log2, float scale) {
  using TL = DqTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kDqBN * TL::KP];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kDqBN * TL::VP];

  int qblk = blockIdx.x / n_bh;
  const int bh = blockIdx.x - qblk * n_bh;
  if (CAUSAL) qblk = n_qblk - 1 - qblk;
  const int b = bh / Hq, hq = bh - b * Hq;
  const int hk = hq / G, Hkv = Hq / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int q0 = qblk * kDqBM + wave * 32;
  const int qrow = q0 + n;
  const bool row_ok = qrow < Lq;
  const int64_t row_off = ((int64_t)bh * Lq + (row_ok ? qrow : 0)) * D;

  const int64_t kvoff = (int64_t)(b * Hkv + hk) * Lkv * D;
  const uint16_t* kh = k + kvoff;
  const uint16_t* vh = v + kvoff;

  // Q^T and dO^T B operands; Delta from the stored O (this lane's half of the row).
  u32x4_t qop[D / 16], doop[D / 16];
  float dpart = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const int d0 = 16 * c + 8 * g;
    if (row_ok) {
      qop[c] = gload16B(q + row_off + d0);
      doop[c] = gload16B(dO + row_off + d0);
      float ov[8];
      load_out8<OutT>(o + row_off + d0, ov);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dpart = fmaf(lo_f32<T>(doop[c][w]), ov[2 * w], dpart);
        dpart = fmaf(hi_f32<T>(doop[c][w]), ov[2 * w + 1], dpart);
      }
    } else {
      qop[c] = (u32x4_t){0u, 0u, 0u, 0u};
      doop[c] = (u32x4_t){0u, 0u, 0u, 0u};
    }
  }
  const float dlt = half_swap_sum(dpart);
  const float lse2 = row_ok ? lse[(int64_t)bh * Lq + qrow] * kLog2e : 0.f;
  if (row_ok && g == 0) delta[(int64_t)bh * Lq + qrow] = dlt;

  f32x16_t acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int kv_end = CAUSAL ? min(Lkv, qblk * kDqBM + kDqBM) : Lkv;
  const int ntiles = (kv_end + kDqBN - 1) / kDqBN;
  const int ld_row = tid / TL::CPR, ld_col = (tid % TL::CPR) * 8;
  u32x4_t kbuf[TL::PASSES], vbuf[TL::PASSES];
  auto fetch = [&](int t) {
#pragma unroll
    for (int p = 0; p < TL::PASSES; ++p) {
      const int r = t * kDqBN + p * TL::RPP + ld_row;
      if (r < Lkv) {
        kbuf[p] = gload16B(kh + (int64_t)r * D + ld_col);
        vbuf[p] = gload16B(vh + (int64_t)r * D + ld_col);
      } else {
        kbuf[p] = (u32x4_t){0u, 0u, 0u, 0u};
        vbuf[p] = (u32x4_t){0u, 0u, 0u, 0u};
      }
    }
  };
  const int G16 = lane >> 4, L16 = lane & 15;
  fetch(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < TL::PASSES; ++p) {
      const int r = p * TL::RPP + ld_row;
      lds_write16B(k_lds + r * TL::KP + ld_col, kbuf[p]);
      lds_write16B(v_lds + r * TL::VP + ld_col, vbuf[p]);
    }
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);
    const int kt0 = t * kDqBN;
    if (CAUSAL && kt0 > q0 + 31) continue;

    f32x16_t s[kDqBN / 32], dp[kDqBN / 32];
#pragma unroll
    for (int kb = 0; kb < kDqBN / 32; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = 0.f;
        dp[kb][i] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        s[kb] = mfma32<T>(lds_read16B(k_lds + (kb * 32 + n) * TL::KP + 16 * c + 8 * g), qop[c], s[kb]);
        dp[kb] = mfma32<T>(lds_read16B(v_lds + (kb * 32 + n) * TL::VP + 16 * c + 8 * g), doop[c], dp[kb]);
      }
    }
    const bool need_mask = (kt0 + kDqBN > Lkv) || (CAUSAL && kt0 + kDqBN - 1 > q0);
    u32x4_t dsop[kDqBN / 16];
#pragma unroll
    for (int kb = 0; kb < kDqBN / 32; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * c2 + e;
          float p = fast_exp2(fminf(s[kb][i] * scale_log2 - lse2, 0.f));
          if (need_mask) {
            const int key = kt0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key >= Lkv || (CAUSAL && key > qrow)) p = 0.f;
          }
          ds[e] = p * (dp[kb][i] - dlt);
        }
        dsop[kb * 2 + c2] = (u32x4_t){pack2<T>(ds[0], ds[1]), pack2<T>(ds[2], ds[3]), pack2<T>(ds[4], ds[5]),
                                      pack2<T>(ds[6], ds[7])};
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + 16 * (G16 & 1) + 4 * (L16 & 3);
#pragma unroll
      for (int kb = 0; kb < kDqBN / 32; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int row = kb * 32 + 16 * c2 + 4 * g + (L16 >> 2);
          const u32x2_t lo = lds_read_tr16(k_lds + row * TL::KP + col);
          const u32x2_t hi = lds_read_tr16(k_lds + (row + 8) * TL::KP + col);
          acc[db] = mfma32<T>((u32x4_t){lo[0], lo[1], hi[0], hi[1]}, dsop[kb * 2 + c2], acc[db]);
        }
    }
  }
  if (row_ok) {
    OutT* out = dq + row_off;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        Store4<OutT>::run(out + db * 32 + 8 * r4 + 4 * g, acc[db][4 * r4] * scale, acc[db][4 * r4 + 1] * scale,
                          acc[db][4 * r4 + 2] * scale, acc[db][4 * r4 + 3] * scale);
  }
}

// ---------------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------------
constexpr int kKvBN = 128;  // key rows per workgroup (32 per wave)
constexpr int kKvBM = 64;   // queries per tile

template <int D>
struct KvTile {
  static constexpr int QP = D + 8;
  static constexpr int CPR = D / 8;
  static constexpr int RPP = kThreads / CPR;
  static constexpr int PASSES = kKvBM / RPP;
};

template <typename T, int D, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(kThreads, 1) void dkv_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ lse,
                                                          const uint16_t* __restrict__ dO,
                                                          const float* __restrict__ delta, OutT* __restrict__ dk,
                                                          OutT* __restrict__ dv, int Hq, int G, int Lq, int Lkv,
                                                          int n_kblk, int n_bhk, float scale_log2, float scale) {
  using TL = KvTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kKvBM * TL::QP];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[kKvBM * TL::QP];
  __shared__ __attribute__((aligned(16))) float lse_lds[kKvBM];
  __shared__ __attribute__((aligned(16))) float dl_lds[kKvBM];

  // Key block 0 sees the most causal queries; low block ids are dispatched first.
  const int kblk = blockIdx.x / n_bhk;
  const int bhk = blockIdx.x - kblk * n_bhk;
  const int Hkv = Hq / G, b = bhk / Hkv, hk = bhk - b * Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int kw0 = kblk * kKvBN + wave * 32;  // first key of this wave
  const int krow = kw0 + n;
  const bool key_ok = krow < Lkv;
  const int64_t krow_off = ((int64_t)bhk * Lkv + (key_ok ? krow : 0)) * D;

  // K^T and V^T as B operands: lane (n, g) holds row krow, d = 16c + 8g .. +7.
  u32x4_t kop[D / 16], vop[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    kop[c] = key_ok ? gload16B(k + krow_off + 16 * c + 8 * g) : (u32x4_t){0u, 0u, 0u, 0u};
    vop[c] = key_ok ? gload16B(v + krow_off + 16 * c + 8 * g) : (u32x4_t){0u, 0u, 0u, 0u};
  }
  f32x16_t dka[D / 32], dva[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[db][i] = 0.f;
      dva[db][i] = 0.f;
    }

  const int q_begin = CAUSAL ? (kblk * kKvBN / kKvBM) * kKvBM : 0;
  const int ntiles = (Lq - q_begin + kKvBM - 1) / kKvBM;
  const int total = G * ntiles;  // (head, query tile) pairs, head-major
  const int ld_row = tid / TL::CPR, ld_col = (tid % TL::CPR) * 8;
  u32x4_t qbuf[TL::PASSES], dbuf[TL::PASSES];
  float side = 0.f;  // threads 0..63 carry LSE*log2e, 64..127 carry Delta
  auto fetch = [&](int it) {
    const int gi = it / ntiles, t0 = q_begin + (it - gi * ntiles) * kKvBM;
    const int64_t base = (int64_t)(b * Hq + hk * G + gi) * Lq;
#pragma unroll
    for (int p = 0; p < TL::PASSES; ++p) {
      const int r = t0 + p * TL::RPP + ld_row;
      if (r < Lq) {
        qbuf[p] = gload16B(q + (base + r) * D + ld_col);
        dbuf[p] = gload16B(dO + (base + r) * D + ld_col);
      } else {
        qbuf[p] = (u32x4_t){0u, 0u, 0u, 0u};
        dbuf[p] = (u32x4_t){0u, 0u, 0u, 0u};
      }
    }
    if (tid < 2 * kKvBM) {
      const int r = t0 + (tid & (kKvBM - 1));
      side = (r < Lq) ? (tid < kKvBM ? lse[base + r] * kLog2e : delta[base + r]) : 0.f;
    }
  };
  const int G16 = lane >> 4, L16 = lane & 15;
  if (total > 0) fetch(0);
  for (int it = 0; it < total; ++it) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < TL::PASSES; ++p) {
      const int r = p * TL::RPP + ld_row;
      lds_write16B(q_lds + r * TL::QP + ld_col, qbuf[p]);
      lds_write16B(do_lds + r * TL::QP + ld_col, dbuf[p]);
    }
    if (tid < kKvBM)
      lse_lds[tid] = side;
    else if (tid < 2 * kKvBM)
      dl_lds[tid - kKvBM] = side;
    __syncthreads();
    const int t0 = q_begin + (it % ntiles) * kKvBM;
    if (it + 1 < total) fetch(it + 1);
    if (CAUSAL && t0 + kKvBM - 1 < kw0) continue;  // every query of the tile precedes this wave's keys

    const bool need_mask = (t0 + kKvBM > Lq) || (CAUSAL && t0 < kw0 + 31);
    u32x4_t pop[kKvBM / 16], dsop[kKvBM / 16];
#pragma unroll
    for (int qb = 0; qb < kKvBM / 32; ++qb) {
      f32x16_t s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        s = mfma32<T>(lds_read16B(q_lds + (qb * 32 + n) * TL::QP + 16 * c + 8 * g), kop[c], s);
        dp = mfma32<T>(lds_read16B(do_lds + (qb * 32 + n) * TL::QP + 16 * c + 8 * g), vop[c], dp);
      }
      // Lane (n, g) holds queries qb*32 + 8*(i/4) + 4g + (i%4) of key krow.
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        float pv[8], dsv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int qi0 = qb * 32 + 16 * c2 + 8 * h + 4 * g;
          const f32x4_t l4 = *(const f32x4_t*)(lse_lds + qi0);
          const f32x4_t d4 = *(const f32x4_t*)(dl_lds + qi0);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 8 * c2 + 4 * h + j;
            float p = fast_exp2(fminf(s[i] * scale_log2 - l4[j], 0.f));
            if (need_mask) {
              const int qi = t0 + qi0 + j;
              if (qi >= Lq || (CAUSAL && krow > qi)) p = 0.f;
            }
            pv[4 * h + j] = p;
            dsv[4 * h + j] = p * (dp[i] - d4[j]);
          }
        }
        pop[qb * 2 + c2] = (u32x4_t){pack2<T>(pv[0], pv[1]), pack2<T>(pv[2], pv[3]), pack2<T>(pv[4], pv[5]),
                                     pack2<T>(pv[6], pv[7])};
        dsop[qb * 2 + c2] = (u32x4_t){pack2<T>(dsv[0], dsv[1]), pack2<T>(dsv[2], dsv[3]),
                                      pack2<T>(dsv[4], dsv[5]), pack2<T>(dsv[6], dsv[7])};
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS (A operands transposed out of LDS).
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + 16 * (G16 & 1) + 4 * (L16 & 3);
#pragma unroll
      for (int qb = 0; qb < kKvBM / 32; ++qb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int row = qb * 32 + 16 * c2 + 4 * g + (L16 >> 2);
          const u32x2_t dlo = lds_read_tr16(do_lds + row * TL::QP + col);
          const u32x2_t dhi = lds_read_tr16(do_lds + (row + 8) * TL::QP + col);
          dva[db] = mfma32<T>((u32x4_t){dlo[0], dlo[1], dhi[0], dhi[1]}, pop[qb * 2 + c2], dva[db]);
          const u32x2_t qlo = lds_read_tr16(q_lds + row * TL::QP + col);
          const u32x2_t qhi = lds_read_tr16(q_lds + (row + 8) * TL::QP + col);
          dka[db] = mfma32<T>((u32x4_t){qlo[0], qlo[1], qhi[0], qhi[1]}, dsop[qb * 2 + c2], dka[db]);
        }
    }
  }
  if (key_ok) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + 8 * r4 + 4 * g;
        Store4<OutT>::run(dk + krow_off + d, dka[db][4 * r4] * scale, dka[db][4 * r4 + 1] * scale,
                          dka[db][4 * r4 + 2] * scale, dka[db][4 * r4 + 3] * scale);
        Store4<OutT>::run(dv + krow_off + d, dva[db][4 * r4], dva[db][4 * r4 + 1], dva[db][4 * r4 + 2],
                          dva[db][4 * r4 + 3]);
      }
  }
}

template <typename T, int D, bool C, typename OutT>
hipError_t launch_typed(const Shape& s, const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, void* dq, void* dk, void* dv, float* delta, float scale, int stages,
                        hipStream_t st) {
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  const int G = (int)(s.Hq / s.Hkv);
  if (stages & kStage0) {
    const int n_qblk = (int)((s.Lq + kDqBM - 1) / kDqBM);
    const int n_bh = (int)(s.B * s.Hq);
    hipLaunchKernelGGL((dq_kernel<T, D, C, OutT>), dim3(n_qblk * n_bh), dim3(kThreads), 0, st, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, (const OutT*)o, lse, (const uint16_t*)dO, (OutT*)dq,
                       delta, (int)s.Hq, G, (int)s.Lq, (int)s.Lkv, n_qblk, n_bh, scale_log2, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(stages & kStage1)) return hipSuccess;
  const int n_kblk = (int)((s.Lkv + kKvBN - 1) / kKvBN);
  const int n_bhk = (int)(s.B * s.Hkv);
  hipLaunchKernelGGL((dkv_kernel<T, D, C, OutT>), dim3(n_kblk * n_bhk), dim3(kThreads), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, lse, (const uint16_t*)dO, (const float*)delta,
                     (OutT*)dk, (OutT*)dv, (int)s.Hq, G, (int)s.Lq, (int)s.Lkv, n_kblk, n_bhk, scale_log2, scale);
  return hipGetLastError();
}

template <typename T, typename OutT>
hipError_t launch_d(const Shape& s, bool causal, const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dO, void* dq, void* dk, void* dv, float* delta, float scale,
                    int stages, hipStream_t st) {
#define SDPA_BWD_CASE(DV)                                                                                          \
  case DV:                                                                                                         \
    return causal ? launch_typed<T, DV, true, OutT>(s, q, k, v, o, lse, dO, dq, dk, dv, delta, scale, stages, st) \
                  : launch_typed<T, DV, false, OutT>(s, q, k, v, o, lse, dO, dq, dk, dv, delta, scale, stages, st);
  switch (s.D) {
    SDPA_BWD_CASE(32)
    SDPA_BWD_CASE(64)
    SDPA_BWD_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef SDPA_BWD_CASE
}

}  // namespace

hipError_t launch_bwd_tiled(const Shape& s, Dt dt, Dt out, bool causal, const void* q, const void* k, const void* v,
                            const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                            float* delta, float scale, int stages, hipStream_t st) {
  if (dt == kBF16)
    return out == kF32 ? launch_d<bf16_t, float>(s, causal, q, k, v, o, lse, dO, dq, dk, dv, delta, scale, stages, st)
                       : launch_d<bf16_t, bf16_t>(s, causal, q, k, v, o, lse, dO, dq, dk, dv, delta, scale, stages, st);
  if (dt == kF16)
    return out == kF32 ? launch_d<f16_t, float>(s, causal, q, k, v, o, lse, dO, dq, dk, dv, delta, scale, stages, st)
                       : launch_d<f16_t, f16_t>(s, causal, q, k, v, o, lse, dO, dq, dk, dv, delta, scale, stages, st);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
