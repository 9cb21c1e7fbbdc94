// Tiled forward of scaled-dot-product attention for 16-bit operands on gfx950.
//
// Computes O = softmax((Q K^T) * scale [+ causal]) V and the per-row logsumexp
// (definition: PyTensor issue "PERF: detect scaled-dot-product-attention pattern
// and lower to mx.fast.scaled_dot_product_attention", section "Sketch"; the
// logsumexp is the forward's cached "second output", MLX pull request "[Metal]
// Add Flash Attention VJP for training", section "Key Features"). Softmax is
// evaluated online over key tiles in the exp2 domain with fp32 state (same pull
// request, "Implementation Notes": log2 domain, fp32 accumulators).
//
// Work decomposition: one workgroup = 4 waves = 128 query rows of one
// (batch, query head); each wave owns 32 rows. Key/value tiles of 64 rows are
// staged through LDS (register-prefetched one tile ahead) and shared by the 4
// waves.
//
// Orientation: the scores are computed transposed, S^T = K Q^T, so that in the
// 32x32 accumulator each lane holds 16 scores of ONE query row (lanes l and
// l+32 split the 32 keys of a block). Row max / row sum then need one
// half-wave exchange, the rescale factor is per lane, and the probabilities
// already sit in the B-operand layout of O^T += V^T P^T. V^T is read from the
// row-major V tile with the LDS transpose read.
#include "device_common.h"
#include "kernels.h"

namespace sdpa {
namespace {

constexpr int kFwdBM = 128;  // query rows per workgroup
constexpr int kFwdBN = 64;   // keys per tile
constexpr int kFwdThreads = 256;

template <int D>
struct FwdTile {
  static constexpr int KP = D + 8;    // K tile row pitch (elements): 16-byte skew, conflict-free 16-byte row reads
  static constexpr int VP = D + 16;   // V tile row pitch: 32-byte skew, conflict-free transposed reads
  static constexpr int CPR = D / 8;   // 16-byte chunks per row
  static constexpr int RPP = kFwdThreads / CPR;  // rows staged per pass
  static constexpr int PASSES = kFwdBN / RPP;
  static_assert(PASSES >= 1 && kFwdBN % RPP == 0, "tile staging");
};

template <typename T, int D, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_tiled_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    OutT* __restrict__ o, float* __restrict__ lse, int Hq, int G, int Lq, int Lkv, int n_qblk, int n_bh,
    float scale_log2) {
  using TL = FwdTile<D>;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kFwdBN * TL::KP];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kFwdBN * TL::VP];

  int qblk = blockIdx.x / n_bh;
  const int bh = blockIdx.x - qblk * n_bh;
  if (CAUSAL) qblk = n_qblk - 1 - qblk;  // longest causal rows are dispatched first
  const int b = bh / Hq, hq = bh - b * Hq;
  const int hk = hq / G, Hkv = Hq / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int q0 = qblk * kFwdBM + wave * 32;
  const int qrow = q0 + n;

  const uint16_t* qh = q + (int64_t)bh * Lq * D;
  const int64_t kvoff = (int64_t)(b * Hkv + hk) * Lkv * D;
  const uint16_t* kh = k + kvoff;
  const uint16_t* vh = v + kvoff;

  // Q^T as the B operand: lane (n, g) holds Q[qrow][16c + 8g .. +7].
  u32x4_t qop[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    qop[c] = (qrow < Lq) ? gload16B(qh + (int64_t)qrow * D + 16 * c + 8 * g) : (u32x4_t){0u, 0u, 0u, 0u};

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -INFINITY;  // running row max of the log2-domain scores
  float lsum = 0.f;     // this lane's share of the running row sum

  const int kv_end = CAUSAL ? min(Lkv, qblk * kFwdBM + kFwdBM) : Lkv;
  const int ntiles = (kv_end + kFwdBN - 1) / kFwdBN;

  const int ld_row = tid / TL::CPR, ld_col = (tid % TL::CPR) * 8;
  u32x4_t kbuf[TL::PASSES], vbuf[TL::PASSES];
  auto fetch = [&](int t) {
#pragma unroll
    for (int p = 0; p < TL::PASSES; ++p) {
      const int r = t * kFwdBN + p * TL::RPP + ld_row;
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
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int p = 0; p < TL::PASSES; ++p) {
      const int r = p * TL::RPP + ld_row;
      lds_write16B(k_lds + r * TL::KP + ld_col, kbuf[p]);
      lds_write16B(v_lds + r * TL::VP + ld_col, vbuf[p]);
    }
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);  // next tile's global loads overlap this tile's math

    const int kt0 = t * kFwdBN;
    if (CAUSAL && kt0 > q0 + 31) continue;  // tile entirely above this wave's diagonal

    // S^T = K Q^T: 32 keys x 32 queries per accumulator block.
    f32x16_t s[kFwdBN / 32];
#pragma unroll
    for (int kb = 0; kb < kFwdBN / 32; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4_t a = lds_read16B(k_lds + (kb * 32 + n) * TL::KP + 16 * c + 8 * g);
        s[kb] = mfma32<T>(a, qop[c], s[kb]);
      }
    }

    // Scale into the log2 domain, mask, and take the tile's row max.
    const bool need_mask = (kt0 + kFwdBN > Lkv) || (CAUSAL && kt0 + kFwdBN - 1 > q0);
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kFwdBN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[kb][i] * scale_log2;
        if (need_mask) {
          const int key = kt0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= Lkv || (CAUSAL && key > qrow)) x = -INFINITY;
        }
        s[kb][i] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = half_swap_max(tmax);
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // P = 2^(t - m), rounded to the operand type for the P.V product.
    u32x4_t pop[kFwdBN / 16];
#pragma unroll
    for (int kb = 0; kb < kFwdBN / 32; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(s[kb][8 * c2 + e] - m_use);
          lsum += p[e];
        }
        pop[kb * 2 + c2] = (u32x4_t){pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]), pack2<T>(p[4], p[5]),
                                     pack2<T>(p[6], p[7])};
      }

    // O^T += V^T P^T. B operand chunk (kb, c2) covers keys kb*32 + 16*c2 + {4g..4g+3, 8+4g..8+4g+3};
    // the A operand reads the same keys of V transposed.
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int col = db * 32 + 16 * (G16 & 1) + 4 * (L16 & 3);
#pragma unroll
      for (int kb = 0; kb < kFwdBN / 32; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int row = kb * 32 + 16 * c2 + 4 * g + (L16 >> 2);
          const u32x2_t lo = lds_read_tr16(v_lds + row * TL::VP + col);
          const u32x2_t hi = lds_read_tr16(v_lds + (row + 8) * TL::VP + col);
          oacc[db] = mfma32<T>((u32x4_t){lo[0], lo[1], hi[0], hi[1]}, pop[kb * 2 + c2], oacc[db]);
        }
    }
  }

  const float l = half_swap_sum(lsum);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (qrow < Lq) {
    OutT* orow = o + ((int64_t)bh * Lq + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        Store4<OutT>::run(orow + db * 32 + 8 * r4 + 4 * g, oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv,
                          oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
    if (lse != nullptr && g == 0) lse[(int64_t)bh * Lq + qrow] = (m + fast_log2(l)) * kLn2;
  }
}

template <typename T, int D, bool C, typename OutT>
hipError_t launch_typed(const Shape& s, const void* q, const void* k, const void* v, void* o, float* lse, float scale,
                        hipStream_t st) {
  const int n_qblk = (int)((s.Lq + kFwdBM - 1) / kFwdBM);
  const int n_bh = (int)(s.B * s.Hq);
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  hipLaunchKernelGGL((fwd_tiled_kernel<T, D, C, OutT>), dim3(n_qblk * n_bh), dim3(kFwdThreads), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (OutT*)o, lse, (int)s.Hq,
                     (int)(s.Hq / s.Hkv), (int)s.Lq, (int)s.Lkv, n_qblk, n_bh, scale_log2);
  return hipGetLastError();
}

template <typename T, typename OutT>
hipError_t launch_d(const Shape& s, bool causal, const void* q, const void* k, const void* v, void* o, float* lse,
                    float scale, hipStream_t st) {
  switch (s.D) {
    case 32:
      return causal ? launch_typed<T, 32, true, OutT>(s, q, k, v, o, lse, scale, st)
                    : launch_typed<T, 32, false, OutT>(s, q, k, v, o, lse, scale, st);
    case 64:
      return causal ? launch_typed<T, 64, true, OutT>(s, q, k, v, o, lse, scale, st)
                    : launch_typed<T, 64, false, OutT>(s, q, k, v, o, lse, scale, st);
    case 128:
      return causal ? launch_typed<T, 128, true, OutT>(s, q, k, v, o, lse, scale, st)
                    : launch_typed<T, 128, false, OutT>(s, q, k, v, o, lse, scale, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd_tiled(const Shape& s, Dt dt, Dt out, bool causal, const void* q, const void* k, const void* v,
                            void* o, float* lse, float scale, hipStream_t st) {
  if (dt == kBF16)
    return out == kF32 ? launch_d<bf16_t, float>(s, causal, q, k, v, o, lse, scale, st)
                       : launch_d<bf16_t, bf16_t>(s, causal, q, k, v, o, lse, scale, st);
  if (dt == kF16)
    return out == kF32 ? launch_d<f16_t, float>(s, causal, q, k, v, o, lse, scale, st)
                       : launch_d<f16_t, f16_t>(s, causal, q, k, v, o, lse, scale, st);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
