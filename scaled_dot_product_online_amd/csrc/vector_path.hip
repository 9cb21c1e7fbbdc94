// Short-query attention (Lq <= 8) for 16-bit operands on gfx950.
//
// The MLX pull request "[Metal] Add Flash Attention VJP for training"
// ("Implementation Notes", vector VJP for L <= 8, fp32 accumulators) treats short
// queries separately: the work is one pass over K and V, so the kernels are sized
// for HBM bandwidth, not for the matrix cores. Here the G*Lq (<= 32) query rows of
// a GQA group are packed into the 32 rows of one MFMA block (they are contiguous
// in BHLD memory: head hk*G + r/Lq, query r%Lq is row hk*G*Lq + r), and the keys
// of each (b, hk) are split across workgroups so that the few groups still fill
// the chip.
//
// Forward:  vec_fwd_kernel  — split s, wave w streams its own contiguous segment of
//                            the split in 32-key tiles with an online softmax;
//                            the 4 waves merge in LDS; the split writes
//                            (O_unnormalised, m, l) partials, or the final O and
//                            logsumexp when there is one split.
//           vec_combine_kernel — merges the splits' partials per row:
//                            m* = max m_s, l* = sum l_s 2^(m_s-m*),
//                            O = sum O_s 2^(m_s-m*) / l*, LSE = (m* + log2 l*) ln 2.
// Backward: vec_bwd_kernel  — split s, wave w owns 32 keys per step exclusively:
//                            P from the logsumexp, dP, dS; dV = P^T dO and
//                            dK = scale dS^T Q are complete for those keys (all
//                            query rows of the group are resident) and are stored
//                            directly; dS is also transposed through LDS into
//                            dQ^T += K^T dS^T, summed over the split's keys.
//           vec_dq_reduce_kernel — dQ = scale * sum_s dQ_s.
#include "device_common.h"
#include "kernels.h"

namespace sdpa {
namespace {

constexpr int kThreads = 256;  // combine and reduction kernels
// Waves per workgroup of the two streaming kernels: 4, or 2 at D = 256, where a wave's
// K/V ring (two 32-key slots of K and V) takes 64 KiB of LDS.
template <int D>
constexpr int vec_waves() {
  return D == 256 ? 2 : 4;
}
int vec_waves_of(int64_t D) { return D == 256 ? 2 : 4; }

struct SplitPlan {
  int nsplit;
  int64_t split_len;  // keys per split, a multiple of (waves per workgroup) * kVecKeys
};

int64_t rows_total(const Shape& s) { return s.B * s.Hq * s.Lq; }

// ---------------------------------------------------------------------------------
// Forward split
// ---------------------------------------------------------------------------------
// One workgroup of 4 waves (2 at D = 256) per CU (the plan sizes the grid to the CU count). Each wave
// streams its own contiguous key segment in 32-key steps: K and V tiles go straight from
// HBM into a two-slot LDS ring owned by the wave (direct buffer-to-LDS loads with the
// non-temporal policy: K and V are read exactly once), so the wave only waits on its own
// loads and never on the other waves until the final merge. The tiles use the same
// swizzled layout and read patterns as the tiled forward.
constexpr int kVecKeys = 32;  // keys per step
constexpr int kVecRing = 2;   // LDS slots per wave

SplitPlan plan(const Shape& s) {
  const int64_t groups = s.B * s.Hkv * ((s.Hq / s.Hkv * s.Lq + 31) / 32);
  const int64_t unit = vec_waves_of(s.D) * kVecKeys;  // one step per wave
  const int64_t units = (s.Lkv + unit - 1) / unit;
  int64_t want = (256 + groups - 1) / groups;  // about one workgroup per CU
  if (want < 1) want = 1;
  if (want > units) want = units;
  const int64_t len = ((s.Lkv + want - 1) / want + unit - 1) / unit * unit;
  return SplitPlan{(int)((s.Lkv + len - 1) / len), len};
}

template <typename T, int D, bool CAUSAL, bool HAS_MASK, typename OutT>
__global__ __launch_bounds__(64 * vec_waves<D>(), 1) void vec_fwd_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v, OutT* __restrict__ o,
                                                              float* __restrict__ lse, float* __restrict__ part_o,
                                                              float* __restrict__ part_ml, int Hq, int G, int Lq,
                                                              int Lkv, int nsplit, int split_len, int n_rb,
                                                              int64_t total_rows, float scale_log2, Mask mask,
                                                              const float* __restrict__ sinks) {
  using TL = SwzTile<D>;
  constexpr int kWaves = vec_waves<D>();
  constexpr int TILE = kVecKeys * TL::RB;         // bytes of one K or V tile
  constexpr int WAVE_LDS = kVecRing * 2 * TILE;   // [slot][K, V]
  constexpr int NDMA = 2 * kVecKeys * TL::CPR / 64;  // buffer-to-LDS loads per step (K and V)
  static_assert(kWaves * 32 * D * 4 <= kWaves * WAVE_LDS, "merge scratch must fit in the tile LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kWaves * WAVE_LDS];
  __shared__ float mrg_m[kWaves][32];
  __shared__ float mrg_l[kWaves][32];

  const int split = blockIdx.x % nsplit;
  const int rb = (blockIdx.x / nsplit) % n_rb;
  const int bhk = blockIdx.x / (nsplit * n_rb);
  const int Hkv = Hq / G, b = bhk / Hkv, hk = bhk - b * Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int n = lane & 31, g = lane >> 5;
  const int rows = G * Lq;
  const int64_t row0 = (int64_t)b * Hq * Lq + (int64_t)hk * G * Lq;  // first packed row of the group
  const int64_t kv0 = (int64_t)bhk * Lkv;

  // Q^T as the B operand: lane (n, g) holds packed row rb*32 + n, d = 16c + 8g .. +7
  // (rows past the group's G*Lq read as zero).
  const rsrc_t rq = make_rsrc(q + (row0 + rb * 32) * D, (uint32_t)max(0, rows - rb * 32) * D * 2);
  // The scale's sign is folded into Q (see q_sign), so scores are only scaled by a factor > 0.
  u32x4_t qop[D / 16];
  const QSign qs = q_sign(scale_log2);
  scale_log2 = qs.scale_log2;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) qop[c] = qs.apply(buf_load16(rq, (uint32_t)((n * D + 16 * c + 8 * g) * 2)));
#pragma unroll
  for (int c = 0; c < D / 16; ++c) settle(qop[c]);

  // Causal (sequences aligned at their ends): packed row r is query r % Lq of its head
  // and sees keys up to (r % Lq) + Lkv - Lq.
  const int qlim = CAUSAL ? (rb * 32 + n) % Lq + (Lkv - Lq) : Lkv;
  // With a mask: element offset of packed row rb*32 + n (head hk*G + row / Lq, query
  // row % Lq; rows past the group clamped into range, their outputs are not stored).
  int64_t mrow = 0;
  if constexpr (HAS_MASK) {
    const int r = min(rb * 32 + n, rows - 1);
    mrow = (int64_t)b * mask.sb + (int64_t)(hk * G + r / Lq) * mask.sh + (int64_t)(r % Lq) * mask.sq;
  }
  // This wave's key tiles: the split's 32-key tiles [s0, kb1) taken round-robin by the
  // waves, so that a workgroup's waves stream adjacent tiles (one front in HBM per
  // workgroup rather than one per wave).
  const int s0 = split * split_len;
  const int kb1 = min(s0 + split_len, Lkv);
  const int ntile = kb1 > s0 ? (kb1 - s0 + kVecKeys - 1) / kVecKeys : 0;
  const int steps = ntile > wave ? (ntile - wave + kWaves - 1) / kWaves : 0;
  auto tile0 = [&](int st) { return s0 + (st * kWaves + wave) * kVecKeys; };

  // Ring of 2 K slots and 2 V slots per wave. The K slot of step st is refilled with
  // step st + 2 as soon as S^T of step st has been read out of it, and the V slot as soon
  // as P V has: each tile is requested about two steps before it is used.
  uint8_t* my = lds + wave * WAVE_LDS;
  const uint16_t* kbase = k + kv0 * D;
  const uint16_t* vbase = v + kv0 * D;
  auto kslot = [&](int st) { return my + (st & 1) * 2 * TILE; };
  auto vslot = [&](int st) { return my + (st & 1) * 2 * TILE + TILE; };
  const typename TL::template DmaPlan<kVecKeys, 1> dma(0, lane);
  auto fill_k = [&](int st) {
    dma.template fill<kCacheStream, false>(srd_rows<D>(kbase, Lkv, tile0(st)), kslot(st), 0);
  };
  auto fill_v = [&](int st) {
    dma.template fill<kCacheStream, false>(srd_rows<D>(vbase, Lkv, tile0(st)), vslot(st), 0);
  };

  const int G16 = lane >> 4, L16 = lane & 15;
  const int vrow = 4 * g + (L16 >> 2);
  const int vx = 2 * (G16 & 1) + ((L16 & 3) >> 1);
  const int xk = g ^ TL::f(n), xv = vx ^ TL::f(vrow), xv8 = vx ^ TL::f(vrow + 8);
  const int srow = n * TL::RB, vrow_b = vrow * TL::RB + 8 * (L16 & 1);

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -INFINITY, lsum = 0.f, lcomp = 0.f;  // row max, row sum and its compensation

  for (int st = 0; st < 2 && st < steps; ++st) {
    fill_k(st);
    fill_v(st);
  }
  for (int st = 0; st < steps; ++st) {
    // Loads in flight, oldest first: K(st), V(st), then K(st+1), V(st+1) if issued.
    if (st + 1 < steps)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint8_t* kt = kslot(st);
    const uint8_t* vt = vslot(st);
    const int t0 = tile0(st);

    // S^T = K Q^T: lane holds keys t0 + 8*(i/4) + 4g + i%4 of packed row n.
    f32x16_t s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      s = mfma32<T>(*(const u32x4_t*)(kt + srow + ((2 * c) ^ xk) * 16), qop[c], s);
    if (st + 2 < steps) {  // the K reads above have returned (S^T depends on them)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      fill_k(st + 2);
    }
    // Wave-uniform: the segment ends inside this step, or (causal) some row's last
    // visible key co + (row % Lq) lies inside it.
    if (t0 + kVecKeys > kb1 || (CAUSAL && t0 + kVecKeys - 1 > Lkv - Lq)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = t0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (key >= kb1 || (CAUSAL && key > qlim)) s[i] = -INFINITY;
      }
    }
    float bias[16];
    if constexpr (HAS_MASK) {  // keys t0 + 8*i4 + 4g + 0..3 (past the end: clamped, and already -inf)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int key0 = t0 + 8 * i4 + 4 * g;
        if (mask.vec4 && key0 < Lkv) {
          mask_bias4_log2<T>(mask.p, mask.kind, mrow + key0, bias + 4 * i4);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            bias[4 * i4 + j] = mask_bias_log2<T>(mask.p, mask.kind, mrow + min(key0 + j, Lkv - 1));
        }
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (HAS_MASK)  // scale and the mask's bias, keys past the segment stay -inf
        s[i] = fmaf(s[i], scale_log2, bias[i]);
      else
        s[i] *= scale_log2;
      tmax = fmaxf(tmax, s[i]);
    }
    tmax = half_swap_max(tmax);
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    lsum *= alpha;
    lcomp *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    u32x4_t pop[2];
    float tsum = 0.f;  // the step's probabilities, added to the row sum once
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(s[8 * c2 + e] - m_use);
        tsum += p[e];
      }
      pop[c2] = (u32x4_t){pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]), pack2<T>(p[4], p[5]), pack2<T>(p[6], p[7])};
    }
    kahan_add(lsum, lcomp, tsum);
    // O^T += V^T P^T; B operand chunk c2 covers keys t0 + 16*c2 + {4g..4g+3, 8+4g..8+4g+3}.
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const uint8_t* vb = vt + 16 * c2 * TL::RB + vrow_b;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x2_t lo = lds_read_tr16((const uint16_t*)(vb + ((4 * db) ^ xv) * 16));
        const u32x2_t hi = lds_read_tr16((const uint16_t*)(vb + 8 * TL::RB + ((4 * db) ^ xv8) * 16));
        oacc[db] = mfma32<T>((u32x4_t){lo[0], lo[1], hi[0], hi[1]}, pop[c2], oacc[db]);
      }
    }
    if (st + 2 < steps) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      fill_v(st + 2);
    }
  }
  const float l = half_swap_sum(lsum);

  // Merge the 4 waves: scratch O_w (fp32, [32 rows][D]) reuses the tile LDS. Every wave's
  // loads have landed (vmcnt(0) on its last step) before the barrier.
  __syncthreads();
  float* mrg_o = (float*)lds;
  if (g == 0) {
    mrg_m[wave][n] = m;
    mrg_l[wave][n] = l;
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *(f32x4_t*)(mrg_o + (wave * 32 + n) * D + db * 32 + 8 * r4 + 4 * g) =
          (f32x4_t){oacc[db][4 * r4], oacc[db][4 * r4 + 1], oacc[db][4 * r4 + 2], oacc[db][4 * r4 + 3]};
  __syncthreads();
  // TPM = 2 * kWaves threads per row, 4 columns at a time.
  constexpr int TPM = 2 * kWaves;
  const int mr = tid / TPM, part = tid % TPM;
  const int rr = rb * 32 + mr;
  // The sink joins the row here when there is one split, else in the combine kernel.
  const float sk =
      (nsplit == 1 && sinks != nullptr && rr < rows) ? sinks[hk * G + rr / Lq] * kLog2e : -INFINITY;
  float mw[kWaves], M = sk;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = mrg_m[w][mr];
    M = fmaxf(M, mw[w]);
  }
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float sc[kWaves], L = sk > -INFINITY ? fast_exp2(sk - Mu) : 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    sc[w] = fast_exp2(mw[w] - Mu);
    L += mrg_l[w][mr] * sc[w];
  }
  if (rr < rows) {
    const int64_t grow = row0 + rr;
    if (nsplit == 1) {
      const float inv = L > 0.f ? 1.f / L : 0.f;
      for (int d = part * 4; d < D; d += 4 * TPM) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float a = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) a += mrg_o[(w * 32 + mr) * D + d + j] * sc[w];
          x[j] = a * inv;
        }
        Store4<OutT>::run(o + grow * D + d, x[0], x[1], x[2], x[3]);
      }
      if (lse != nullptr && part == 0) lse[grow] = (M + fast_log2(L)) * kLn2;
    } else {
      float* pod = part_o + ((int64_t)split * total_rows + grow) * D;  // [split][row][D]
      for (int d = part * 4; d < D; d += 4 * TPM) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float a = 0.f;
#pragma unroll
          for (int w = 0; w < kWaves; ++w) a += mrg_o[(w * 32 + mr) * D + d + j] * sc[w];
          x[j] = a;
        }
        *(f32x4_t*)(pod + d) = (f32x4_t){x[0], x[1], x[2], x[3]};
      }
      if (part == 0) {
        part_ml[((int64_t)split * total_rows + grow) * 2 + 0] = M;
        part_ml[((int64_t)split * total_rows + grow) * 2 + 1] = L;
      }
    }
  }
}

template <int D, typename OutT>
__global__ __launch_bounds__(kThreads) void vec_combine_kernel(const float* __restrict__ part_o,
                                                               const float* __restrict__ part_ml,
                                                               OutT* __restrict__ o, float* __restrict__ lse,
                                                               int64_t total_rows, int nsplit,
                                                               const float* __restrict__ sinks, int Hq, int Lq) {
  constexpr int TPR = D / 4;            // threads per row, 4 columns each
  constexpr int RPB = kThreads / TPR;  // rows per block (D = 96: 10 rows, 16 threads idle)
  if ((int)threadIdx.x >= RPB * TPR) return;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 4;
  if (row >= total_rows) return;
  // The sink of the row's query head: one more term of the denominator, with no value.
  const float sk = sinks != nullptr ? sinks[(row / Lq) % Hq] * kLog2e : -INFINITY;
  float M = sk;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[((int64_t)s * total_rows + row) * 2]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float L = sk > -INFINITY ? fast_exp2(sk - Mu) : 0.f, x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const int64_t pr = (int64_t)s * total_rows + row;
    const float w = fast_exp2(part_ml[pr * 2] - Mu);
    L += part_ml[pr * 2 + 1] * w;
    const f32x4_t a = *(const f32x4_t*)(part_o + pr * D + c);
    x0 += a[0] * w;
    x1 += a[1] * w;
    x2 += a[2] * w;
    x3 += a[3] * w;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  Store4<OutT>::run(o + row * D + c, x0 * inv, x1 * inv, x2 * inv, x3 * inv);
  if (lse != nullptr && c == 0) lse[row] = (M + fast_log2(L)) * kLn2;
}

// ---------------------------------------------------------------------------------
// Backward split
// ---------------------------------------------------------------------------------
// Same streaming layout as the forward: one workgroup of 4 waves per CU, each wave with
// its own key segment and a two-slot LDS ring of K and V tiles fed by non-temporal
// buffer-to-LDS loads. Q and dO of the group's 32 packed rows are staged once in
// swizzled tiles; every LDS read uses the conflict-free patterns of the tiled forward
// (16-byte rows for the S / dP operands, transposed reads for Q^T, dO^T and K^T).
// At D = 256 (2 waves) the rings and the Q/dO tiles fill the whole 160 KiB of LDS, so
// the dS^T scratch lives in the step's V tile once dP has consumed it, the per-row
// statistics are kept in registers, and dV/dK are formed in two halves of d after the
// dQ update, each staged as soon as it is complete.
template <typename T, int D, bool CAUSAL, bool HAS_MASK, typename OutT>
__global__ __launch_bounds__(64 * vec_waves<D>(), 1) void vec_bwd_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              const OutT* __restrict__ o,
                                                              const float* __restrict__ lse,
                                                              const uint16_t* __restrict__ dO, OutT* __restrict__ dk,
                                                              OutT* __restrict__ dv, float* __restrict__ dq_part,
                                                              int Hq, int G, int Lq, int Lkv, int nsplit,
                                                              int split_len, int64_t total_rows, float scale_log2,
                                                              float scale, Mask mask, float* __restrict__ delta_out) {
  using TL = SwzTile<D>;
  constexpr int kWaves = vec_waves<D>();
  constexpr int kWgThreads = 64 * kWaves;
  constexpr bool kTight = D == 256;              // scratch in the V tile, statistics in registers
  constexpr int TILE = kVecKeys * TL::RB;        // bytes of one 32-row tile
  constexpr int WAVE_LDS = kVecRing * 2 * TILE;  // [slot][K, V]
  constexpr int NDMA = 2 * kVecKeys * TL::CPR / 64;
  constexpr int DSP = 32 + 16;                   // dS^T scratch pitch (elements)
  static_assert(kWaves * 32 * D * 4 <= kWaves * WAVE_LDS, "dQ reduction scratch must fit in the ring LDS");
  static_assert(!kTight || 32 * DSP * 2 <= TILE, "dS^T scratch must fit in a V tile");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kWaves * WAVE_LDS];
  __shared__ __attribute__((aligned(1024))) uint8_t qd_lds[2 * TILE];  // Q tile, dO tile
  __shared__ __attribute__((aligned(16))) uint16_t ds_lds[kTight ? 1 : kWaves][kTight ? 8 : 32 * DSP];
  // Per packed row r: LSE*log2e, Delta, and (causal) the last key it sees. At D = 256 these
  // are staged in the ring before its first fill and then held in registers.
  __shared__ __attribute__((aligned(16))) float stat_lds[kTight ? 4 : 3 * 32];
  float* lse_lds = kTight ? (float*)lds : stat_lds;
  float* dl_lds = lse_lds + 32;
  int* lim_lds = (int*)(lse_lds + 64);

  const int split = blockIdx.x % nsplit;
  const int bhk = blockIdx.x / nsplit;
  const int Hkv = Hq / G, b = bhk / Hkv, hk = bhk - b * Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int n = lane & 31, g = lane >> 5;
  const int rows = G * Lq;
  const int64_t row0 = (int64_t)b * Hq * Lq + (int64_t)hk * G * Lq;
  const int64_t kv0 = (int64_t)bhk * Lkv;

  // Stage Q and dO of the group's rows (rows past G*Lq arrive as zeros); Delta and
  // LSE*log2e per row.
  {
    const srd_t rq = make_srd(q + row0 * D, (uint32_t)rows * D * 2);
    const srd_t rdo = make_srd(dO + row0 * D, (uint32_t)rows * D * 2);
    TL::template dma_fill<32>(rq, qd_lds, 0, wave, kWaves, lane);
    TL::template dma_fill<32>(rdo, qd_lds + TILE, 0, wave, kWaves, lane);
    constexpr int TPR = kWgThreads / 32;  // Delta: threads per row
    const int r = tid / TPR, part = tid % TPR;
    float acc = 0.f;
    if (r < rows) {
      for (int d = part; d < D; d += TPR) acc = fmaf(load_f32(o + (row0 + r) * D + d), to_f32<T>(dO[(row0 + r) * D + d]), acc);
    }
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (part == 0) {
      dl_lds[r] = acc;
      const float l2 = (r < rows) ? lse[row0 + r] * kLog2e : 0.f;
      lse_lds[r] = (HAS_MASK && l2 == -INFINITY) ? INFINITY : l2;  // a masked row with no key: P = 0
      lim_lds[r] = CAUSAL ? r % Lq + (Lkv - Lq) : Lkv;
      if (delta_out != nullptr && split == 0 && r < rows) delta_out[row0 + r] = acc;  // for the sinks' gradient
    }
    wait_vmem();
    __syncthreads();
  }
  // D = 256: this lane's rows 8i + 4g + j (i = 2*c2 + h below) move to registers before
  // the ring, which holds them, is filled.
  f32x4_t l4r[4], d4r[4];
  i32x4_t lim4r[4];
  if constexpr (kTight) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l4r[i] = *(const f32x4_t*)(lse_lds + 8 * i + 4 * g);
      d4r[i] = *(const f32x4_t*)(dl_lds + 8 * i + 4 * g);
      lim4r[i] = *(const i32x4_t*)(lim_lds + 8 * i + 4 * g);
    }
    __syncthreads();
  }
  const uint8_t* qt = qd_lds;
  const uint8_t* dt = qd_lds + TILE;

  // Key tiles taken round-robin by the waves, as in the forward.
  const int s0 = split * split_len;
  const int kb1 = min(s0 + split_len, Lkv);
  const int ntile = kb1 > s0 ? (kb1 - s0 + kVecKeys - 1) / kVecKeys : 0;
  const int steps = ntile > wave ? (ntile - wave + kWaves - 1) / kWaves : 0;
  auto tile0 = [&](int st) { return s0 + (st * kWaves + wave) * kVecKeys; };
  uint8_t* my = lds + wave * WAVE_LDS;
  const uint16_t* kbase = k + kv0 * D;
  const uint16_t* vbase = v + kv0 * D;
  const typename TL::template DmaPlan<kVecKeys, 1> dma(0, lane);
  auto fill = [&](int st) {
    uint8_t* slot = my + (st % kVecRing) * 2 * TILE;
    dma.template fill<kCacheStream, false>(srd_rows<D>(kbase, Lkv, tile0(st)), slot, 0);
    dma.template fill<kCacheStream, false>(srd_rows<D>(vbase, Lkv, tile0(st)), slot + TILE, 0);
  };

  // LDS geometry (as in the tiled forward): 16-byte reads of row n, chunk 2c + g; transposed
  // reads of rows 16*c2 + 4g + L16/4 (+8), chunk 4*db + vx, byte 8*(L16&1).
  const int G16 = lane >> 4, L16 = lane & 15;
  const int trow = 4 * g + (L16 >> 2);
  const int vx = 2 * (G16 & 1) + ((L16 & 3) >> 1);
  const int xs = g ^ TL::f(n), xt = vx ^ TL::f(trow), xt8 = vx ^ TL::f(trow + 8);
  const int srow = n * TL::RB, trow_b = trow * TL::RB + 8 * (L16 & 1);
  auto rd16 = [&](const uint8_t* t, int c) { return *(const u32x4_t*)(t + srow + ((2 * c) ^ xs) * 16); };
  // A operand of 32 rows (d) x 16 k (rows 16*c2 + ... of the tile), d block db.
  auto rdtr = [&](const uint8_t* t, int c2, int db) {
    const uint8_t* base = t + 16 * c2 * TL::RB + trow_b;
    const u32x2_t lo = lds_read_tr16((const uint16_t*)(base + ((4 * db) ^ xt) * 16));
    const u32x2_t hi = lds_read_tr16((const uint16_t*)(base + 8 * TL::RB + ((4 * db) ^ xt8) * 16));
    return (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
  };

  f32x16_t dqa[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[db][i] = 0.f;

  if (steps > 0) fill(0);
  for (int st = 0; st < steps; ++st) {
    if (st + 1 < steps) {
      fill(st + 1);  // the slot of step st - 1: this wave's reads of it have completed
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const uint8_t* kt = my + (st % kVecRing) * 2 * TILE;
    const uint8_t* vt = kt + TILE;
    uint16_t* dsw = kTight ? (uint16_t*)const_cast<uint8_t*>(vt) : ds_lds[wave];  // V is consumed once dP is formed
    const int t0 = tile0(st);
    const int key = t0 + n;  // this lane's key column
    // A mask that varies only along keys (query and head strides 0) has one bias per lane.
    float kbias = 0.f;
    if constexpr (HAS_MASK)
      if (mask.sq == 0 && mask.sh == 0)
        kbias = mask_bias_log2<T>(mask.p, mask.kind, (int64_t)b * mask.sb + min(key, Lkv - 1));
    // S = Q K^T and dP = dO V^T: rows = packed query rows, columns = this wave's 32 keys.
    f32x16_t s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = 0.f;
      dp[i] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      s = mfma32<T>(rd16(qt, c), rd16(kt, c), s);
      dp = mfma32<T>(rd16(dt, c), rd16(vt, c), dp);
    }
    u32x4_t pop[2], dsop[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      float pv[8], dsv[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r0 = 16 * c2 + 8 * h + 4 * g;
        f32x4_t l4, d4;
        i32x4_t lim4;
        if constexpr (kTight) {
          l4 = l4r[2 * c2 + h];
          d4 = d4r[2 * c2 + h];
          lim4 = lim4r[2 * c2 + h];
        } else {
          l4 = *(const f32x4_t*)(lse_lds + r0);
          d4 = *(const f32x4_t*)(dl_lds + r0);
          lim4 = *(const i32x4_t*)(lim_lds + r0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 8 * c2 + 4 * h + j;
          float nb = -l4[j];
          if constexpr (HAS_MASK) {  // bias of (packed row r0 + j, key), both clamped into range
            if (mask.sq == 0 && mask.sh == 0) {
              nb += kbias;
            } else {
              const int r = min(r0 + j, rows - 1);
              nb += mask_bias_log2<T>(mask.p, mask.kind,
                                      (int64_t)b * mask.sb + (int64_t)(hk * G + r / Lq) * mask.sh +
                                          (int64_t)(r % Lq) * mask.sq + min(key, Lkv - 1));
            }
          }
          float p = exp2_le1(fmaf(s[i], scale_log2, nb));
          if (r0 + j >= rows || key >= kb1 || (CAUSAL && key > lim4[j])) p = 0.f;
          pv[4 * h + j] = p;
          dsv[4 * h + j] = p * (dp[i] - d4[j]);
        }
      }
      pop[c2] = (u32x4_t){pack2<T>(pv[0], pv[1]), pack2<T>(pv[2], pv[3]), pack2<T>(pv[4], pv[5]), pack2<T>(pv[6], pv[7])};
      dsop[c2] = (u32x4_t){pack2<T>(dsv[0], dsv[1]), pack2<T>(dsv[2], dsv[3]), pack2<T>(dsv[4], dsv[5]),
                           pack2<T>(dsv[6], dsv[7])};
      // dS^T scratch, row = key n, columns = query rows (4 consecutive rows per dword pair).
      *(u32x2_t*)(dsw + n * DSP + 16 * c2 + 4 * g) = (u32x2_t){dsop[c2][0], dsop[c2][1]};
      *(u32x2_t*)(dsw + n * DSP + 16 * c2 + 8 + 4 * g) = (u32x2_t){dsop[c2][2], dsop[c2][3]};
    }
    // dV^T = dO^T P and dK^T = Q^T dS for this wave's keys (complete: all rows are here),
    // d blocks [hh * DBH, (hh + 1) * DBH).
    constexpr int NH = kTight ? 2 : 1, DBH = D / 32 / NH;
    auto dkv_products = [&](int hh, f32x16_t* dva, f32x16_t* dka) {
#pragma unroll
      for (int j = 0; j < DBH; ++j) {
        const int db = hh * DBH + j;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          dva[j][i] = 0.f;
          dka[j][i] = 0.f;
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          dva[j] = mfma32<T>(rdtr(dt, c2, db), pop[c2], dva[j]);
          dka[j] = mfma32<T>(rdtr(qt, c2, db), dsop[c2], dka[j]);
        }
      }
    };
    // fp32 outputs: stored straight from the accumulators.
    auto store_f32 = [&](int hh, const f32x16_t* dva, const f32x16_t* dka) {
      if (key < kb1) {
        const int64_t kro = (kv0 + key) * D;
#pragma unroll
        for (int j = 0; j < DBH; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d = (hh * DBH + j) * 32 + 8 * r4 + 4 * g;
            Store4<OutT>::run(dk + kro + d, dka[j][4 * r4] * scale, dka[j][4 * r4 + 1] * scale,
                              dka[j][4 * r4 + 2] * scale, dka[j][4 * r4 + 3] * scale);
            Store4<OutT>::run(dv + kro + d, dva[j][4 * r4], dva[j][4 * r4 + 1], dva[j][4 * r4 + 2],
                              dva[j][4 * r4 + 3]);
          }
      }
    };
    // 16-bit outputs: dV and dK rows are staged in this step's V and K slots (consumed by
    // then), swizzled like the input tiles, and written as whole rows below.
    uint8_t* vs = const_cast<uint8_t*>(vt);
    uint8_t* ks = const_cast<uint8_t*>(kt);
    auto stage16 = [&](int hh, const f32x16_t* dva, const f32x16_t* dka) {
#pragma unroll
      for (int j = 0; j < DBH; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int o = TL::off(n, 4 * (hh * DBH + j) + r4) + 8 * g;  // row key, d = db*32 + 8*r4 + 4g .. +3
          *(u32x2_t*)(vs + o) = (u32x2_t){pack2<OutT>(dva[j][4 * r4], dva[j][4 * r4 + 1]),
                                          pack2<OutT>(dva[j][4 * r4 + 2], dva[j][4 * r4 + 3])};
          *(u32x2_t*)(ks + o) =
              (u32x2_t){pack2<OutT>(dka[j][4 * r4] * scale, dka[j][4 * r4 + 1] * scale),
                        pack2<OutT>(dka[j][4 * r4 + 2] * scale, dka[j][4 * r4 + 3] * scale)};
        }
    };
    // dQ^T += K^T dS^T over this wave's 32 keys; A and B use the same transposed-read rows,
    // so their k slots pair the same keys. Needs the dS^T scratch visible across lanes.
    auto dq_update = [&]() {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int krow = 16 * c2 + trow;
        const u32x2_t blo = lds_read_tr16(dsw + krow * DSP + 16 * (G16 & 1) + 4 * (L16 & 3));
        const u32x2_t bhi = lds_read_tr16(dsw + (krow + 8) * DSP + 16 * (G16 & 1) + 4 * (L16 & 3));
        const u32x4_t bop = (u32x4_t){blo[0], blo[1], bhi[0], bhi[1]};
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dqa[db] = mfma32<T>(rdtr(kt, c2, db), bop, dqa[db]);
      }
    };
    if constexpr (!kTight) {
      f32x16_t dva[DBH], dka[DBH];
      dkv_products(0, dva, dka);
      if constexpr (sizeof(OutT) == 4) store_f32(0, dva, dka);
      wave_sync();  // the dS^T scratch written above is read across lanes below
      dq_update();
      if constexpr (sizeof(OutT) == 2) stage16(0, dva, dka);
    } else {
      // The dS^T scratch and the staged rows share the V slot: the dQ update reads the
      // scratch (and K) before any row is staged.
      wave_sync();
      dq_update();
      wave_sync();  // every lane's scratch and K reads are done before the slots are overwritten
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        f32x16_t dva[DBH], dka[DBH];
        dkv_products(hh, dva, dka);
        if constexpr (sizeof(OutT) == 4)
          store_f32(hh, dva, dka);
        else
          stage16(hh, dva, dka);
      }
    }
    if constexpr (sizeof(OutT) == 2) {
      wave_sync();
      // 64 lanes store 64 consecutive 16-byte chunks of the [kVecKeys, D] tile per step
      // (1 KiB per instruction, non-temporal: written once).
      static_assert(kVecKeys * TL::CPR % 64 == 0, "whole 64-lane store steps");
#pragma unroll
      for (int i = 0; i < kVecKeys * TL::CPR / 64; ++i) {
        const int r = (64 * i + lane) / TL::CPR, c = (64 * i + lane) % TL::CPR;
        if (t0 + r < kb1) {
          const int64_t go = (kv0 + t0 + r) * D + 8 * c;
          __builtin_nontemporal_store(*(const u32x4_t*)(vs + TL::off(r, c)), (u32x4_t*)(dv + go));
          __builtin_nontemporal_store(*(const u32x4_t*)(ks + TL::off(r, c)), (u32x4_t*)(dk + go));
        }
      }
    }
    wave_sync();  // the scratch and slots are rewritten by the next steps
  }
  // Sum the waves' dQ^T (lane (n, g) holds row n, d = db*32 + 8*(i/4) + 4g + i%4).
  __syncthreads();
  float* red = (float*)lds;  // kWaves * 32 * D floats
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *(f32x4_t*)(red + (wave * 32 + n) * D + db * 32 + 8 * r4 + 4 * g) =
          (f32x4_t){dqa[db][4 * r4], dqa[db][4 * r4 + 1], dqa[db][4 * r4 + 2], dqa[db][4 * r4 + 3]};
  __syncthreads();
  for (int e = tid; e < 32 * (D / 4); e += kWgThreads) {
    const int r = e / (D / 4), c = (e % (D / 4)) * 4;
    if (r >= rows) continue;
    f32x4_t a = *(const f32x4_t*)(red + r * D + c);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const f32x4_t x = *(const f32x4_t*)(red + (w * 32 + r) * D + c);
      a[0] += x[0];
      a[1] += x[1];
      a[2] += x[2];
      a[3] += x[3];
    }
    *(f32x4_t*)(dq_part + ((int64_t)split * total_rows + row0 + r) * D + c) = a;
  }
}

template <int D, typename OutT>
__global__ __launch_bounds__(kThreads) void vec_dq_reduce_kernel(const float* __restrict__ dq_part,
                                                                 OutT* __restrict__ dq, int64_t total_rows,
                                                                 int nsplit, float scale) {
  const int64_t e4 = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // one group of 4 columns
  if (e4 >= total_rows * (D / 4)) return;
  float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const f32x4_t a = *(const f32x4_t*)(dq_part + (int64_t)s * total_rows * D + e4 * 4);
    x0 += a[0];
    x1 += a[1];
    x2 += a[2];
    x3 += a[3];
  }
  Store4<OutT>::run(dq + e4 * 4, x0 * scale, x1 * scale, x2 * scale, x3 * scale);
}

// Two such reductions in one launch (the dK and dV partials of a split dK/dV kernel):
// workgroups [0, nb) take (part_a, out_a, scale_a), the rest (part_b, out_b, scale_b), each
// over n4 groups of 4 columns, summed in split order as above.
template <typename OutT>
__global__ __launch_bounds__(kThreads) void vec_pair_reduce_kernel(const float* __restrict__ part_a,
                                                                   OutT* __restrict__ out_a, float scale_a,
                                                                   const float* __restrict__ part_b,
                                                                   OutT* __restrict__ out_b, float scale_b,
                                                                   int64_t n4, int nb, int nsplit) {
  const bool second = (int)blockIdx.x >= nb;
  const float* part = second ? part_b : part_a;
  OutT* out = second ? out_b : out_a;
  const float scale = second ? scale_b : scale_a;
  const int64_t e4 = (int64_t)(blockIdx.x - (second ? nb : 0)) * kThreads + threadIdx.x;
  if (e4 >= n4) return;
  float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const f32x4_t a = *(const f32x4_t*)(part + (int64_t)sp * n4 * 4 + e4 * 4);
    x0 += a[0];
    x1 += a[1];
    x2 += a[2];
    x3 += a[3];
  }
  Store4<OutT>::run(out + e4 * 4, x0 * scale, x1 * scale, x2 * scale, x3 * scale);
}

// The combine kernel over `nsplit` partials [nsplit][B*Hq*Lq][D] and (m, l) pairs.
template <int D, typename OutT>
hipError_t combine_typed(const Shape& s, int nsplit, const float* part_o, const float* part_ml, const float* sinks,
                         void* o, float* lse, hipStream_t st) {
  const int64_t tr = rows_total(s);
  constexpr int RPB = kThreads / (D / 4);
  hipLaunchKernelGGL((vec_combine_kernel<D, OutT>), dim3((unsigned)((tr + RPB - 1) / RPB)), dim3(kThreads), 0, st,
                     part_o, part_ml, (OutT*)o, lse, tr, nsplit, sinks, (int)s.Hq, (int)s.Lq);
  return hipGetLastError();
}

template <typename T, int D, typename OutT>
hipError_t fwd_typed(const Shape& s, bool causal, const Mask& mask, const float* sinks, const void* q, const void* k,
                     const void* v, void* o, float* lse, float scale, void* ws, hipStream_t st) {
  const SplitPlan pl = plan(s);
  const int G = (int)(s.Hq / s.Hkv);
  const int n_rb = (int)((G * s.Lq + 31) / 32);
  const int64_t tr = rows_total(s);
  float* part_o = (float*)ws;
  float* part_ml = part_o + (int64_t)pl.nsplit * tr * D;
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  auto kern = causal                     ? vec_fwd_kernel<T, D, true, false, OutT>
              : mask.kind != kMaskNone ? vec_fwd_kernel<T, D, false, true, OutT>
                                         : vec_fwd_kernel<T, D, false, false, OutT>;
  hipLaunchKernelGGL(kern, dim3(pl.nsplit * n_rb * s.B * s.Hkv), dim3(64 * vec_waves<D>()), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (OutT*)o, lse, part_o, part_ml, (int)s.Hq, G, (int)s.Lq,
                     (int)s.Lkv, pl.nsplit, (int)pl.split_len, n_rb, tr, scale_log2, mask, sinks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nsplit == 1) return e;
  return combine_typed<D, OutT>(s, pl.nsplit, part_o, part_ml, sinks, o, lse, st);
}

template <typename T, int D, typename OutT>
hipError_t bwd_typed(const Shape& s, bool causal, const Mask& mask, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv, void* ws,
                     float scale, int stages, hipStream_t st) {
  const SplitPlan pl = plan(s);
  const int G = (int)(s.Hq / s.Hkv);
  const int64_t tr = rows_total(s);
  float* dq_part = (float*)ws;
  float* delta = (float*)((char*)ws + vector_bwd_delta_offset(s));
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  if (stages & kStage0) {
    auto kern = causal                     ? vec_bwd_kernel<T, D, true, false, OutT>
                : mask.kind != kMaskNone ? vec_bwd_kernel<T, D, false, true, OutT>
                                           : vec_bwd_kernel<T, D, false, false, OutT>;
    hipLaunchKernelGGL(kern, dim3(pl.nsplit * s.B * s.Hkv), dim3(64 * vec_waves<D>()), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const OutT*)o, lse,
                       (const uint16_t*)dO, (OutT*)dk, (OutT*)dv, dq_part, (int)s.Hq, G, (int)s.Lq, (int)s.Lkv,
                       pl.nsplit, (int)pl.split_len, tr, scale_log2, scale, mask, delta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(stages & kStage1)) return hipSuccess;
  const int64_t n4 = tr * (D / 4);
  hipLaunchKernelGGL((vec_dq_reduce_kernel<D, OutT>), dim3((unsigned)((n4 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, (const float*)dq_part, (OutT*)dq, tr, pl.nsplit, scale);
  return hipGetLastError();
}

}  // namespace

int vector_num_splits(const Shape& s) { return plan(s).nsplit; }

size_t vector_fwd_workspace(const Shape& s) {
  const SplitPlan pl = plan(s);
  if (pl.nsplit == 1) return 0;
  return (size_t)pl.nsplit * (size_t)rows_total(s) * (size_t)(s.D + 2) * sizeof(float);
}

// dQ partials [nsplit][B*Hq*Lq][D], then (256-byte aligned) Delta [B*Hq*Lq].
size_t vector_bwd_delta_offset(const Shape& s) {
  const size_t part = (size_t)plan(s).nsplit * (size_t)rows_total(s) * (size_t)s.D * sizeof(float);
  return (part + 255) / 256 * 256;
}

size_t vector_bwd_workspace(const Shape& s) {
  return vector_bwd_delta_offset(s) + (size_t)rows_total(s) * sizeof(float);
}

#define SDPA_VEC_DISPATCH(FN, ...)                                                                          \
  switch (s.D) {                                                                                            \
    case 32: return dt == kBF16 ? (out == kF32 ? FN<bf16_t, 32, float>(__VA_ARGS__) : FN<bf16_t, 32, bf16_t>(__VA_ARGS__)) \
                                : (out == kF32 ? FN<f16_t, 32, float>(__VA_ARGS__) : FN<f16_t, 32, f16_t>(__VA_ARGS__));   \
    case 64: return dt == kBF16 ? (out == kF32 ? FN<bf16_t, 64, float>(__VA_ARGS__) : FN<bf16_t, 64, bf16_t>(__VA_ARGS__)) \
                                : (out == kF32 ? FN<f16_t, 64, float>(__VA_ARGS__) : FN<f16_t, 64, f16_t>(__VA_ARGS__));   \
    case 96: return dt == kBF16 ? (out == kF32 ? FN<bf16_t, 96, float>(__VA_ARGS__) : FN<bf16_t, 96, bf16_t>(__VA_ARGS__)) \
                                : (out == kF32 ? FN<f16_t, 96, float>(__VA_ARGS__) : FN<f16_t, 96, f16_t>(__VA_ARGS__));   \
    case 128: return dt == kBF16 ? (out == kF32 ? FN<bf16_t, 128, float>(__VA_ARGS__) : FN<bf16_t, 128, bf16_t>(__VA_ARGS__)) \
                                 : (out == kF32 ? FN<f16_t, 128, float>(__VA_ARGS__) : FN<f16_t, 128, f16_t>(__VA_ARGS__));   \
    case 256: return dt == kBF16 ? (out == kF32 ? FN<bf16_t, 256, float>(__VA_ARGS__) : FN<bf16_t, 256, bf16_t>(__VA_ARGS__)) \
                                 : (out == kF32 ? FN<f16_t, 256, float>(__VA_ARGS__) : FN<f16_t, 256, f16_t>(__VA_ARGS__));   \
    default: return hipErrorInvalidValue;                                                                   \
  }

hipError_t launch_split_combine(const Shape& s, Dt out, int nsplit, const float* part_o, const float* part_ml,
                                const float* sinks, void* o, float* lse, hipStream_t st) {
#define SDPA_COMBINE(DD)                                                                                   \
  case DD:                                                                                                 \
    return out == kF32    ? combine_typed<DD, float>(s, nsplit, part_o, part_ml, sinks, o, lse, st)         \
           : out == kBF16 ? combine_typed<DD, bf16_t>(s, nsplit, part_o, part_ml, sinks, o, lse, st)        \
                          : combine_typed<DD, f16_t>(s, nsplit, part_o, part_ml, sinks, o, lse, st);
  switch (s.D) {
    SDPA_COMBINE(32)
    SDPA_COMBINE(64)
    SDPA_COMBINE(96)
    SDPA_COMBINE(128)
    SDPA_COMBINE(256)
    default: return hipErrorInvalidValue;
  }
#undef SDPA_COMBINE
}

hipError_t launch_split_reduce_pair(const Shape& s, Dt out, int nsplit, const float* part_a, void* out_a,
                                    float scale_a, const float* part_b, void* out_b, float scale_b, int64_t rows,
                                    hipStream_t st) {
  const int64_t n4 = rows * (s.D / 4);
  const int nb = (int)((n4 + kThreads - 1) / kThreads);
  const dim3 grid((unsigned)(2 * nb));
  if (out == kF32)
    hipLaunchKernelGGL((vec_pair_reduce_kernel<float>), grid, dim3(kThreads), 0, st, part_a, (float*)out_a, scale_a,
                       part_b, (float*)out_b, scale_b, n4, nb, nsplit);
  else if (out == kBF16)
    hipLaunchKernelGGL((vec_pair_reduce_kernel<bf16_t>), grid, dim3(kThreads), 0, st, part_a, (bf16_t*)out_a,
                       scale_a, part_b, (bf16_t*)out_b, scale_b, n4, nb, nsplit);
  else
    hipLaunchKernelGGL((vec_pair_reduce_kernel<f16_t>), grid, dim3(kThreads), 0, st, part_a, (f16_t*)out_a,
                       scale_a, part_b, (f16_t*)out_b, scale_b, n4, nb, nsplit);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const Shape& s, Dt out, int nsplit, const float* part, void* out_ptr, int64_t rows,
                               float scale, hipStream_t st) {
  const int64_t n4 = rows * (s.D / 4);
  const dim3 grid((unsigned)((n4 + kThreads - 1) / kThreads));
#define SDPA_REDUCE(DD)                                                                                          \
  case DD:                                                                                                       \
    if (out == kF32)                                                                                             \
      hipLaunchKernelGGL((vec_dq_reduce_kernel<DD, float>), grid, dim3(kThreads), 0, st, part, (float*)out_ptr, \
                         rows, nsplit, scale);                                                                   \
    else if (out == kBF16)                                                                                       \
      hipLaunchKernelGGL((vec_dq_reduce_kernel<DD, bf16_t>), grid, dim3(kThreads), 0, st, part,                 \
                         (bf16_t*)out_ptr, rows, nsplit, scale);                                                 \
    else                                                                                                         \
      hipLaunchKernelGGL((vec_dq_reduce_kernel<DD, f16_t>), grid, dim3(kThreads), 0, st, part, (f16_t*)out_ptr, \
                         rows, nsplit, scale);                                                                   \
    return hipGetLastError();
  switch (s.D) {
    SDPA_REDUCE(32)
    SDPA_REDUCE(64)
    SDPA_REDUCE(96)
    SDPA_REDUCE(128)
    SDPA_REDUCE(256)
    default: return hipErrorInvalidValue;
  }
#undef SDPA_REDUCE
}

hipError_t launch_fwd_vector(const Shape& s, Dt dt, Dt out, bool causal, const Mask& mask, const float* sinks,
                             const void* q, const void* k, const void* v, void* o, float* lse, float scale, void* ws,
                             hipStream_t st) {
  if (dt != kBF16 && dt != kF16) return hipErrorInvalidValue;
  SDPA_VEC_DISPATCH(fwd_typed, s, causal, mask, sinks, q, k, v, o, lse, scale, ws, st)
}

hipError_t launch_bwd_vector(const Shape& s, Dt dt, Dt out, bool causal, const Mask& mask, const void* q,
                             const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
                             void* dk, void* dv, void* ws, float scale, int stages, hipStream_t st) {
  if (dt != kBF16 && dt != kF16) return hipErrorInvalidValue;
  SDPA_VEC_DISPATCH(bwd_typed, s, causal, mask, q, k, v, o, lse, dO, dq, dk, dv, ws, scale, stages, st)
}

}  // namespace sdpa
