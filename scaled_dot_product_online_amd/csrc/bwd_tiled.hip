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
//   It first forms Delta for its rows from O and dO and stores {LSE*log2e, -Delta}
//   per query in the workspace for kernel 2, then streams K/V tiles of 64 keys
//   through double-buffered, swizzled LDS filled by direct buffer-to-LDS loads. Like the forward it works on
//   transposed scores (S^T = K Q^T, dP^T = V dO^T) so that each lane owns one
//   query row; dQ^T += K^T dS^T reads K^T with the LDS transpose read.
//   At D = 256 stage 0 runs dq16_kernel instead: 8 waves x 16 query rows on 16x16x32
//   tiles and 32-key tiles, which fits two waves per SIMD.
// Kernel 2 (dkv_kernel): one workgroup = 8 waves x 16 key rows of one (b, hk);
//   the waves keep K and V of their rows in registers and accumulate dK and dV
//   while streaming Q/dO tiles of 64 queries (128 at D <= 64 without a mask) of every
//   query head of the group. At D = 256 the workgroup's K rows sit in LDS instead and
//   the query tiles are 32 rows, which fits two waves per SIMD.
//   Scores are computed as S = Q K^T on 16x16x32 tiles (lane owns one key
//   column), which puts P and dS directly in the B-operand layout of
//   dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T are read with the LDS
//   transpose read.
// Small grids (fewer workgroups than the chip holds at once): kernel 1 splits its key
//   tiles and kernel 2 its (query head, query tile) sequence over several workgroups,
//   which write fp32 partials of dQ (resp. dK and dV); a reduction kernel sums them in a
//   fixed order (deterministic) and applies the scale.
#include "device_common.h"
#include "kernels.h"

namespace sdpa {
namespace {

constexpr int kThreads = 256;

template <typename OutT>
__device__ __forceinline__ void load_out8(rsrc_t r, uint32_t elem, float* x);
template <>
__device__ __forceinline__ void load_out8<float>(rsrc_t r, uint32_t elem, float* x) {
  const u32x4_t a = buf_load16(r, elem * 4), b = buf_load16(r, elem * 4 + 16);
  for (int i = 0; i < 4; ++i) {
    x[i] = __uint_as_float(a[i]);
    x[4 + i] = __uint_as_float(b[i]);
  }
}
template <typename T16>
__device__ __forceinline__ void load_out8_16(rsrc_t r, uint32_t elem, float* x) {
  const u32x4_t w = buf_load16(r, elem * 2);
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = lo_f32<T16>(w[i]);
    x[2 * i + 1] = hi_f32<T16>(w[i]);
  }
}
template <>
__device__ __forceinline__ void load_out8<bf16_t>(rsrc_t r, uint32_t elem, float* x) {
  load_out8_16<bf16_t>(r, elem, x);
}
template <>
__device__ __forceinline__ void load_out8<f16_t>(rsrc_t r, uint32_t elem, float* x) {
  load_out8_16<f16_t>(r, elem, x);
}

// ---------------------------------------------------------------------------------
// Stage 0: dQ, plus the per-query {LSE*log2e, -Delta} pairs for stage 1
// ---------------------------------------------------------------------------------
constexpr int kDqBM = 128;  // query rows per workgroup
// Keys per tile: 64; 32 at D = 256 (dq16_kernel below; 32-row waves there would hold 256
// registers of resident Q/dO operands and dQ accumulators, one wave per SIMD); 128 at
// D <= 64 without a mask (1-3% faster measured; slower with a mask).
template <int D, bool HAS_MASK>
constexpr int dq_bn() {
  return D == 256 ? 32 : (D <= 64 && !HAS_MASK) ? 128 : 64;
}

// The dQ kernel stages a mask through LDS (mask_staged) at D <= 96.
template <int D>
__host__ __device__ inline bool dq_mask_staged(const Mask& m) {
  return D <= 96 && mask_staged(m);
}

// D <= 128 (D = 256 runs dq16_kernel).
template <typename T, int D, bool CAUSAL, bool HAS_MASK, typename OutT>
__global__ __launch_bounds__(kThreads, 2) void dq_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, const OutT* __restrict__ o,
                                                         const float* __restrict__ lse,
                                                         const uint16_t* __restrict__ dO, OutT* __restrict__ dq,
                                                         f32x2_t* __restrict__ rowstat, int Hq, int G, int Lq,
                                                         int Lkv, int n_qblk, int n_bh, int lq_pad,
                                                         float scale_log2, float scale, Mask mask, int nsplit,
                                                         int split_tiles, float* __restrict__ dq_part) {
  static_assert(D <= 128, "D = 256 runs dq16_kernel");
  using TL = SwzTile<D>;
  constexpr int kDqBN = dq_bn<D, HAS_MASK>();
  constexpr int TILE = kDqBN * TL::RB;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * 2 * TILE];  // [buffer][K, V]

  // Work id: query block major, then key split, then (b, hq) (as the forward).
  const int wid = xcd_remap(blockIdx.x, n_qblk * n_bh * nsplit, G);
  int qblk = wid / (n_bh * nsplit);
  const int rest = wid - qblk * (n_bh * nsplit);
  const int split = rest / n_bh;
  const int bh = rest - split * n_bh;
  if (CAUSAL) qblk = n_qblk - 1 - qblk;
  const int b = bh / Hq, hq = bh - b * Hq;
  const int hk = hq / G, Hkv = Hq / G;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 31, g = lane >> 5;
  const int q0 = qblk * kDqBM + wave * 32;
  const int qrow = q0 + n;

  const int64_t kvoff = (int64_t)(b * Hkv + hk) * Lkv * D;
  const int64_t qoff = (int64_t)bh * Lq * D;
  const rsrc_t rq = make_rsrc(q + qoff, (uint32_t)Lq * D * 2);
  const rsrc_t rdo = make_rsrc(dO + qoff, (uint32_t)Lq * D * 2);
  const rsrc_t ro = make_rsrc(o + qoff, (uint32_t)Lq * D * (uint32_t)sizeof(OutT));

  // Q^T and dO^T B operands; Delta from the stored O over this lane's half of the row.
  u32x4_t qop[D / 16], doop[D / 16];
  float dpart = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const uint32_t e = (uint32_t)(qrow * D + 16 * c + 8 * g);
    qop[c] = buf_load16(rq, e * 2);
    doop[c] = buf_load16(rdo, e * 2);
    float ov[8];
    load_out8<OutT>(ro, e, ov);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dpart = fmaf(lo_f32<T>(doop[c][w]), ov[2 * w], dpart);
      dpart = fmaf(hi_f32<T>(doop[c][w]), ov[2 * w + 1], dpart);
    }
  }
  const float dlt = half_swap_sum(dpart);
#pragma unroll
  for (int c = 0; c < D / 16; ++c) settle(qop[c]);
  const bool row_ok = qrow < Lq;
  float lse2 = row_ok ? lse[(int64_t)bh * Lq + qrow] * kLog2e : 0.f;
  // A masked row that sees no key (LSE = -inf) has P = 0: +inf makes every exponent -inf.
  if (HAS_MASK && lse2 == -INFINITY) lse2 = INFINITY;
  const int64_t mrow =
      HAS_MASK ? (int64_t)b * mask.sb + (int64_t)hq * mask.sh + (int64_t)min(qrow, Lq - 1) * mask.sq : 0;
  // -Delta: the dK/dV kernel starts its dP accumulators from it.
  if (row_ok && g == 0 && split == 0) rowstat[(int64_t)bh * lq_pad + qrow] = (f32x2_t){lse2, -dlt};
  f32x16_t ndlt;  // -Delta of this lane's query in every element (the dP chains' start)
#pragma unroll
  for (int i = 0; i < 16; ++i) ndlt[i] = -dlt;

  f32x16_t acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int co = Lkv - Lq;  // causal offset: key j visible to query i iff j <= i + co
  const int kv_end = CAUSAL ? min(Lkv, qblk * kDqBM + kDqBM + co) : Lkv;
  const int ntiles = (kv_end + kDqBN - 1) / kDqBN;
  const int t_lo = split * split_tiles, t_hi = min(ntiles, t_lo + split_tiles);  // this split's key tiles
  const int key_lim = CAUSAL ? min(Lkv, qrow + 1 + co) : Lkv;
  const int G16 = lane >> 4, L16 = lane & 15;
  const int fk0 = TL::f(n);
  const int trow = 4 * g + (L16 >> 2);
  const int ft0 = TL::f(trow), ft80 = TL::f(trow + 8);  // swizzle of the two rows each transposed read pair uses
  const int tx = 2 * (G16 & 1) + ((L16 & 3) >> 1);
  constexpr int NKB = kDqBN / 32;  // 32-key blocks per tile
  constexpr int NC = D / 16;       // 16-wide steps of the S / dP contraction over d

  // One key tile. As in the dK/dV kernel, each stage's LDS reads are issued one stage
  // ahead of the matrix-core instructions that use them, behind scheduling fences.
  // Key padding (a boolean mask that varies only along keys): tiles whose keys are all
  // padding are skipped, and the others take each key's keep flag from a ballot of the
  // mask bytes, which are read a tile ahead (no per-score mask loads).
  const bool pad = HAS_MASK && is_key_padding(mask);
  // A boolean mask that varies along queries (mask_staged), at D <= 96: its block for each
  // key tile (the workgroup's 128 query rows, the tile's keys, one byte each) is copied into
  // dynamic LDS with K and V, double-buffered, and read from there. (At D = 128 the masked
  // kernel already holds 256 registers and the staged path would spill.)
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_mask[];
  constexpr int MBLK = kDqBM * kDqBN;
  const bool mstage = HAS_MASK && dq_mask_staged<D>(mask);
  auto tile = [&](bool masked, const uint8_t* kt, const uint8_t* vt, int kt0, uint64_t keep) {
    // Lane constants made opaque per tile, so that the compiler rebuilds the LDS addresses
    // derived from them inside the loop instead of keeping each one live across it.
    // Chunk 2c + g of row n sits at (2c ^ (g ^ f(n))); chunk 4db + tx of row r at (4db ^ (tx ^ f(r))).
    int xs = g ^ fk0, xt = tx ^ ft0, xt8 = tx ^ ft80, klim = key_lim - 4 * g, srow = n * TL::RB,
        trow_b = trow * TL::RB + 8 * (L16 & 1);
    asm volatile("" : "+v"(xs), "+v"(xt), "+v"(xt8), "+v"(klim), "+v"(srow), "+v"(trow_b));
    // Stage c of the S / dP products of 32-key block kb.
    auto load_s = [&](int kb, int c, u32x4_t* kv) {
      const int off = kb * 32 * TL::RB + srow + ((2 * c) ^ xs) * 16;
      kv[0] = *(const u32x4_t*)(kt + off);
      kv[1] = *(const u32x4_t*)(vt + off);
    };
    // dQ stage c2 of block kb: keys kb*32 + 16*c2 + {4g..4g+3, 8+4g..8+4g+3}, all d blocks.
    auto load_q = [&](int kb, int c2, u32x2_t* tb) {
      const uint8_t* krow_p = kt + (kb * 32 + 16 * c2) * TL::RB + trow_b;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        tb[2 * db] = lds_read_tr16((const uint16_t*)(krow_p + ((4 * db) ^ xt) * 16));
        tb[2 * db + 1] = lds_read_tr16((const uint16_t*)(krow_p + 8 * TL::RB + ((4 * db) ^ xt8) * 16));
      }
    };

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T for keys kb*32 .. +31 (lane owns query qrow and 16
      // of the keys).
      // K/V operands read SD - 1 = 1 stage ahead (two stages ahead measured no faster with
      // two waves per SIMD).
      constexpr int SD = 2;
      u32x4_t kv[SD][2];
#pragma unroll
      for (int c = 0; c < SD - 1; ++c) load_s(kb, c, kv[c]);
      sched_fence();
      f32x16_t s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
      u32x2_t tb[2][D / 16];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + SD - 1 < NC) load_s(kb, c + SD - 1, kv[(c + SD - 1) % SD]);
        else if (c + SD - 1 == NC) load_q(kb, 0, tb[0]);
        s = mfma32<T>(kv[c % SD][0], qop[c], s);
        // Without a mask the dP chain starts from -Delta (a block kept across the loop), so
        // that dS = P * dP needs no subtraction per score.
        dp = mfma32<T>(kv[c % SD][1], doop[c], (!HAS_MASK && c == 0) ? ndlt : dp);
        sched_fence();
      }
      // dS^T as B operands, one per 16-key half c2. Only the softmax is duplicated for
      // the masked case (a wave-uniform branch), so both paths share the same registers.
      u32x4_t dsop[2];
      // PAD: bits 8r + j of lm keep key kt0 + kb*32 + 8r + 4g + j (the lane's element 4r + j).
      const uint32_t lm = (uint32_t)(keep >> (32 * kb)) >> (4 * g);
      auto softmax = [&](auto edge_tag, auto pad_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        constexpr bool PAD = decltype(pad_tag)::value;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          float ds[8];
          // The mask's bias of keys kt0 + kb*32 + 8*(2*c2 + h) + 4g + 0..3 (element e = 4h + j).
          float bias[8];
          if constexpr (HAS_MASK && !PAD) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int key0 = kt0 + kb * 32 + 8 * (2 * c2 + h) + 4 * g;
              if (D <= 96 && mstage) {  // this lane's row of the tile's staged block
                const uint8_t* mblk = lds_mask + ((kt0 / kDqBN) & 1) * MBLK + (wave * 32 + n) * kDqBN + 4 * g;
                mask_bias4_bool_word(*(const uint32_t*)(mblk + kb * 32 + 8 * (2 * c2 + h)), bias + 4 * h);
                if constexpr (EDGE) {  // keys past the end (the last tile only)
#pragma unroll
                  for (int j = 0; j < 4; ++j)
                    if (key0 + j >= Lkv) bias[4 * h + j] = -INFINITY;
                }
              } else if (mask.vec4 && key0 < Lkv) {
                mask_bias4_log2<T>(mask.p, mask.kind, mrow + key0, bias + 4 * h);
              } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  bias[4 * h + j] =
                      key0 + j < Lkv ? mask_bias_log2<T>(mask.p, mask.kind, mrow + key0 + j) : -INFINITY;
              }
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = 8 * c2 + e;
            float nb = -lse2;
            if constexpr (HAS_MASK && !PAD) nb = bias[e] - lse2;
            float p = exp2_le1(fmaf(s[i], scale_log2, nb));
            if constexpr (EDGE)  // key kt0 + kb*32 + 8*(i/4) + (i%4) + 4g below key_lim
              p = kt0 + kb * 32 + 8 * (i >> 2) + (i & 3) < klim ? p : 0.f;
            if constexpr (PAD) p = ((lm >> (8 * (i >> 2) + (i & 3))) & 1u) ? p : 0.f;
            ds[e] = HAS_MASK ? p * (dp[i] - dlt) : p * dp[i];
          }
          dsop[c2] = (u32x4_t){pack2<T>(ds[0], ds[1]), pack2<T>(ds[2], ds[3]), pack2<T>(ds[4], ds[5]),
                               pack2<T>(ds[6], ds[7])};
        }
      };
      if (HAS_MASK && pad)  // no causal mask with a mask; keys past the end have no bit
        softmax(std::false_type{}, std::true_type{});
      else if (masked)
        softmax(std::true_type{}, std::false_type{});
      else
        softmax(std::false_type{}, std::false_type{});
      sched_fence();
      // dQ^T += K^T dS^T.
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        if (c2 == 0) load_q(kb, 1, tb[1]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const u32x2_t lo = tb[c2][2 * db], hi = tb[c2][2 * db + 1];
          acc[db] = mfma32<T>((u32x4_t){lo[0], lo[1], hi[0], hi[1]}, dsop[c2], acc[db]);
        }
        sched_fence();
      }
    }
  };

  const uint16_t* kbase = k + kvoff;
  const uint16_t* vbase = v + kvoff;
  const typename TL::template DmaPlan<kDqBN, 4> dma(wave, lane);
  auto stage_mask = [&](int t) {  // 16 bytes per lane, kDqBN / 16 lanes per row
    constexpr int LPR = kDqBN / 16, RPI = 64 / LPR;
    const int kt0 = t * kDqBN, r0 = qblk * kDqBM;
    const int64_t e0 = (int64_t)b * mask.sb + (int64_t)hq * mask.sh + (int64_t)r0 * mask.sq + kt0;
    const int64_t nel = (int64_t)(Lq - 1 - r0) * mask.sq + (Lkv - kt0);  // through row Lq - 1, key Lkv - 1
    const srd_t rm = make_srd((const uint8_t*)mask.p + e0, (uint32_t)min(nel, (int64_t)0xffffffffll));
    uint8_t* mb = lds_mask + (t & 1) * MBLK;
    for (int i = wave; i < kDqBM / RPI; i += 4) {
      const int r = i * RPI + lane / LPR;
      dma16(rm, mb + 1024 * i, (uint32_t)(r * mask.sq + (lane % LPR) * 16));
    }
  };
  if (t_lo < t_hi) {
    uint8_t* b0 = lds + (t_lo & 1) * 2 * TILE;
    dma.fill(srd_rows<D>(kbase, Lkv, t_lo * kDqBN), b0, wave);
    dma.fill(srd_rows<D>(vbase, Lkv, t_lo * kDqBN), b0 + TILE, wave);
    if (mstage) stage_mask(t_lo);
  }
  uint32_t kept_next = pad && t_lo < t_hi ? key_kept(mask, b, t_lo * kDqBN, kDqBN, Lkv, lane) : 1u;
  for (int t = t_lo; t < t_hi; ++t) {
    wait_vmem();
    __syncthreads();
    if (t + 1 < t_hi) {
      uint8_t* nb = lds + ((t + 1) & 1) * 2 * TILE;
      dma.fill(srd_rows<D>(kbase, Lkv, (t + 1) * kDqBN), nb, wave);
      dma.fill(srd_rows<D>(vbase, Lkv, (t + 1) * kDqBN), nb + TILE, wave);
      if (mstage) stage_mask(t + 1);
    }
    const uint32_t kept = kept_next;
    if (pad && t + 1 < t_hi) kept_next = key_kept(mask, b, (t + 1) * kDqBN, kDqBN, Lkv, lane);
    const uint8_t* kt = lds + (t & 1) * 2 * TILE;
    const uint8_t* vt = kt + TILE;
    const int kt0 = t * kDqBN;
    if (CAUSAL && kt0 > q0 + 31 + co) continue;
    const uint64_t keep = pad ? __ballot(kept != 0u) : 0;  // bit j: key kt0 + j kept
    if (pad && keep == 0) continue;                           // every key of the tile is padding
    tile((kt0 + kDqBN > Lkv) || (CAUSAL && kt0 + kDqBN - 1 > q0 + co), kt, vt, kt0, keep);  // wave-uniform flag
  }
  if (dq_part != nullptr) {  // one key split: fp32 partial of dQ / scale, [split][b*Hq*Lq + hq*Lq + q]
    if (row_ok) {
      float* po = dq_part + (((int64_t)split * n_bh + bh) * Lq + qrow) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4_t*)(po + db * 32 + 8 * r4 + 4 * g) =
              (f32x4_t){acc[db][4 * r4], acc[db][4 * r4 + 1], acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]};
    }
    return;
  }
  if (row_ok) {
    OutT* out = dq + qoff + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        Store4<OutT>::run(out + db * 32 + 8 * r4 + 4 * g, acc[db][4 * r4] * scale, acc[db][4 * r4 + 1] * scale,
                          acc[db][4 * r4 + 2] * scale, acc[db][4 * r4 + 3] * scale);
  }
}

// Stage 0 at D = 256 on 16-row waves: one workgroup = 8 waves x 16 query rows of one
// (b, hq), 16x16x32 matrix-core tiles, 32-key K/V tiles. The resident Q^T/dO^T operands
// (64 registers) and dQ^T accumulators (64) then leave room for two waves per SIMD, where
// the 32-row kernel's 256 registers of operands and accumulators allow one; each wave reads
// the whole K/V tile for 16 rows instead of 32 (twice the LDS reads per FLOP). Orientation
// as the dK/dV kernel's: S^T = K Q^T puts four keys of one query in each lane, which is the
// B-operand layout of dQ^T += K^T dS^T; K^T comes from the LDS transpose read.
constexpr int kDq16Waves = 8;
template <typename T, int D, bool CAUSAL, bool HAS_MASK, typename OutT>
__global__ __launch_bounds__(64 * kDq16Waves, 1) void dq16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const OutT* __restrict__ o, const float* __restrict__ lse, const uint16_t* __restrict__ dO,
    OutT* __restrict__ dq, f32x2_t* __restrict__ rowstat, int Hq, int G, int Lq, int Lkv, int n_qblk, int n_bh,
    int lq_pad, float scale_log2, float scale, Mask mask, int nsplit, int split_tiles, float* __restrict__ dq_part) {
  static_assert(kDq16Waves * 16 == kDqBM, "8 waves of 16 rows make the 128-row query block");
  using TL = SwzTile<D, 16>;
  constexpr int BN = 32;  // keys per tile: two 16-key blocks
  constexpr int TILE = BN * TL::RB;
  constexpr int NC = D / 32;  // 32-wide steps of the S / dP contraction over d
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * 2 * TILE];  // [buffer][K, V]

  // Work id: query block major, then key split, then (b, hq) (as the 32-row kernel).
  const int wid = xcd_remap(blockIdx.x, n_qblk * n_bh * nsplit, G);
  int qblk = wid / (n_bh * nsplit);
  const int rest = wid - qblk * (n_bh * nsplit);
  const int split = rest / n_bh;
  const int bh = rest - split * n_bh;
  if (CAUSAL) qblk = n_qblk - 1 - qblk;
  const int b = bh / Hq, hq = bh - b * Hq;
  const int hk = hq / G, Hkv = Hq / G;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n16 = lane & 15, q4 = lane >> 4;
  const int q0 = qblk * kDqBM + wave * 16;  // wave-uniform
  const int qrow = q0 + n16;

  const int64_t kvoff = (int64_t)(b * Hkv + hk) * Lkv * D;
  const int64_t qoff = (int64_t)bh * Lq * D;
  const rsrc_t rq = make_rsrc(q + qoff, (uint32_t)Lq * D * 2);
  const rsrc_t rdo = make_rsrc(dO + qoff, (uint32_t)Lq * D * 2);
  const rsrc_t ro = make_rsrc(o + qoff, (uint32_t)Lq * D * (uint32_t)sizeof(OutT));

  // Q^T and dO^T B operands: lane (n16, q4) holds row qrow, d = 32c + 8*q4 .. +7. Delta from
  // the stored O over this lane's quarter of the row, then summed over the four lanes.
  u32x4_t qop[NC], doop[NC];
  float dpart = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t e = (uint32_t)(qrow * D + 32 * c + 8 * q4);
    qop[c] = buf_load16(rq, e * 2);
    doop[c] = buf_load16(rdo, e * 2);
    float ov[8];
    load_out8<OutT>(ro, e, ov);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dpart = fmaf(lo_f32<T>(doop[c][w]), ov[2 * w], dpart);
      dpart = fmaf(hi_f32<T>(doop[c][w]), ov[2 * w + 1], dpart);
    }
  }
  dpart += __shfl_xor(dpart, 16);
  const float dlt = dpart + __shfl_xor(dpart, 32);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    settle(qop[c]);
    settle(doop[c]);
  }
  const bool row_ok = qrow < Lq;
  float lse2 = row_ok ? lse[(int64_t)bh * Lq + qrow] * kLog2e : 0.f;
  // A masked row that sees no key (LSE = -inf) has P = 0: +inf makes every exponent -inf.
  if (HAS_MASK && lse2 == -INFINITY) lse2 = INFINITY;
  const int64_t mrow =
      HAS_MASK ? (int64_t)b * mask.sb + (int64_t)hq * mask.sh + (int64_t)min(qrow, Lq - 1) * mask.sq : 0;
  // -Delta: the dK/dV kernel starts its dP accumulators from it.
  if (row_ok && q4 == 0 && split == 0) rowstat[(int64_t)bh * lq_pad + qrow] = (f32x2_t){lse2, -dlt};
  const f32x4_t ndlt = {-dlt, -dlt, -dlt, -dlt};  // the dP chains' start without a mask (as in dq_kernel)

  // dQ^T block db: lane (n16, q4) holds d = 16*db + 4*q4 + i of query qrow.
  f32x4_t acc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[db][i] = 0.f;

  const int co = Lkv - Lq;  // causal offset: key j visible to query i iff j <= i + co
  const int kv_end = CAUSAL ? min(Lkv, qblk * kDqBM + kDqBM + co) : Lkv;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int t_lo = split * split_tiles, t_hi = min(ntiles, t_lo + split_tiles);  // this split's key tiles
  const int key_lim = CAUSAL ? min(Lkv, qrow + 1 + co) : Lkv;
  const int L16 = lane & 15;
  const int fa0 = TL::f(n16);            // 16-byte reads: row kb*16 + n16 (f depends on the row mod 8)
  const int trow = 4 * q4 + (L16 >> 2);  // transposed reads: rows trow and trow + 16
  const int ft0 = TL::f(trow);
  const int tcol = 8 * (L16 & 1);  // byte within the 16-byte chunk
  const int tch = (L16 & 3) >> 1;  // chunk 2*db + tch

  // One key tile. Stage c of the S / dP products reads its K/V operands one stage ahead.
  // Chunk indices past 15 (d >= 128) keep bit 4 under the XOR with f < 16, so each address
  // is a lane term plus a constant.
  auto tile = [&](bool masked, const uint8_t* kt, const uint8_t* vt, int kt0) {
    // Lane constants made opaque per tile, so that the compiler rebuilds the LDS addresses
    // derived from them inside the loop instead of keeping each one live across it.
    int fa = fa0, ft = ft0, srow = n16 * TL::RB, trow_b = trow * TL::RB + tcol, q4x = q4, tchx = tch,
        klim = key_lim - 4 * q4;
    asm volatile("" : "+v"(fa), "+v"(ft), "+v"(srow), "+v"(trow_b), "+v"(q4x), "+v"(tchx), "+v"(klim));
    auto load_s = [&](int c, u32x4_t* kv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int off = kb * 16 * TL::RB + srow + ((4 * (c & 3) + q4x) ^ fa) * 16 + (c >> 2) * 256;
        kv[2 * kb] = *(const u32x4_t*)(kt + off);
        kv[2 * kb + 1] = *(const u32x4_t*)(vt + off);
      }
    };
    // dQ A operands of d block db: K^T rows (keys) 4*q4 + 0..3 and 16 + 4*q4 + 0..3.
    auto load_q = [&](int db, u32x2_t* tb) {
      const int off = trow_b + ((2 * (db & 7) + tchx) ^ ft) * 16 + (db >> 3) * 256;
      tb[0] = lds_read_tr16((const uint16_t*)(kt + off));
      tb[1] = lds_read_tr16((const uint16_t*)(kt + off + 16 * TL::RB));
    };
    u32x4_t kv[2][4];
    load_s(0, kv[0]);
    sched_fence();
    f32x4_t s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[kb][i] = 0.f;
        dp[kb][i] = 0.f;
      }
    u32x2_t tb[2][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + 1 < NC) load_s(c + 1, kv[(c + 1) & 1]);
      else load_q(0, tb[0]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = mfma16<T>(kv[c & 1][2 * kb], qop[c], s[kb]);
        dp[kb] = mfma16<T>(kv[c & 1][2 * kb + 1], doop[c], (!HAS_MASK && c == 0) ? ndlt : dp[kb]);
      }
      sched_fence();
    }
    // dS^T as the B operand: keys 4*q4 + 0..3 (block 0) then 16 + 4*q4 + 0..3 (block 1).
    u32x4_t dsop;
    auto softmax = [&](auto edge_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
      float ds[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float bias[4];
        if constexpr (HAS_MASK) {
          const int key0 = kt0 + kb * 16 + 4 * q4;
          if (mask.vec4 && key0 < Lkv) {
            mask_bias4_log2<T>(mask.p, mask.kind, mrow + key0, bias);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              bias[j] = key0 + j < Lkv ? mask_bias_log2<T>(mask.p, mask.kind, mrow + key0 + j) : -INFINITY;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float nb = -lse2;
          if constexpr (HAS_MASK) nb = bias[j] - lse2;
          float p = exp2_le1(fmaf(s[kb][j], scale_log2, nb));
          if constexpr (EDGE)  // key kt0 + kb*16 + 4*q4 + j below key_lim
            p = kt0 + kb * 16 + j < klim ? p : 0.f;
          ds[4 * kb + j] = HAS_MASK ? p * (dp[kb][j] - dlt) : p * dp[kb][j];
        }
      }
      dsop = (u32x4_t){pack2<T>(ds[0], ds[1]), pack2<T>(ds[2], ds[3]), pack2<T>(ds[4], ds[5]), pack2<T>(ds[6], ds[7])};
    };
    if (masked)
      softmax(std::true_type{});
    else
      softmax(std::false_type{});
    sched_fence();
    // dQ^T += K^T dS^T, one 16-wide d block per step, reads one step ahead.
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      if (db + 1 < D / 16) load_q(db + 1, tb[(db + 1) & 1]);
      const u32x2_t lo = tb[db & 1][0], hi = tb[db & 1][1];
      acc[db] = mfma16<T>((u32x4_t){lo[0], lo[1], hi[0], hi[1]}, dsop, acc[db]);
      sched_fence();
    }
  };

  const uint16_t* kbase = k + kvoff;
  const uint16_t* vbase = v + kvoff;
  const typename TL::template DmaPlan<BN, kDq16Waves> dma(wave, lane);
  if (t_lo < t_hi) {
    uint8_t* b0 = lds + (t_lo & 1) * 2 * TILE;
    dma.fill(srd_rows<D>(kbase, Lkv, t_lo * BN), b0, wave);
    dma.fill(srd_rows<D>(vbase, Lkv, t_lo * BN), b0 + TILE, wave);
  }
  // Key padding: tiles whose keys are all padding are skipped (mask bytes read a tile ahead).
  const bool pad = HAS_MASK && is_key_padding(mask);
  uint32_t kept_next = pad && t_lo < t_hi ? key_kept(mask, b, t_lo * BN, BN, Lkv, lane) : 1u;
  for (int t = t_lo; t < t_hi; ++t) {
    wait_vmem();
    __syncthreads();
    if (t + 1 < t_hi) {
      uint8_t* nb = lds + ((t + 1) & 1) * 2 * TILE;
      dma.fill(srd_rows<D>(kbase, Lkv, (t + 1) * BN), nb, wave);
      dma.fill(srd_rows<D>(vbase, Lkv, (t + 1) * BN), nb + TILE, wave);
    }
    const uint32_t kept = kept_next;
    if (pad && t + 1 < t_hi) kept_next = key_kept(mask, b, (t + 1) * BN, BN, Lkv, lane);
    const uint8_t* kt = lds + (t & 1) * 2 * TILE;
    const uint8_t* vt = kt + TILE;
    const int kt0 = t * BN;
    if (CAUSAL && kt0 > q0 + 15 + co) continue;  // tile entirely above this wave's diagonal
    if (pad && !__any(kept != 0u)) continue;     // every key of the tile is padding
    tile((kt0 + BN > Lkv) || (CAUSAL && kt0 + BN - 1 > q0 + co), kt, vt, kt0);  // wave-uniform flag
  }
  if (dq_part != nullptr) {  // one key split: fp32 partial of dQ / scale, [split][b*Hq*Lq + hq*Lq + q]
    if (row_ok) {
      float* po = dq_part + (((int64_t)split * n_bh + bh) * Lq + qrow) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) *(f32x4_t*)(po + db * 16 + 4 * q4) = acc[db];
    }
    return;
  }
  if (row_ok) {
    OutT* out = dq + qoff + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      Store4<OutT>::run(out + db * 16 + 4 * q4, acc[db][0] * scale, acc[db][1] * scale, acc[db][2] * scale,
                        acc[db][3] * scale);
  }
}

// ---------------------------------------------------------------------------------
// Stage 1: dK, dV
// ---------------------------------------------------------------------------------
// One workgroup = 8 waves x 16 key rows = 128 keys of one (b, hk), two waves per SIMD.
// Each wave keeps K and V of its 16 keys as B operands and the dK^T, dV^T accumulators in
// registers (16x16x32 matrix-core tiles keep that state at 96 registers per lane for
// D = 128), and streams Q/dO tiles of 64 queries (128 at D <= 64 without a mask, see
// kv_bm) of every query head of the group.
// At D = 256 that state would be 192 registers, too many for two waves per SIMD beside the
// scores and operand staging: there the workgroup's 128 K rows are copied into LDS once
// (64 KiB) and each wave reads its K^T operands from there per contraction step, the query
// tiles are 32 rows, and the wave keeps V and the accumulators (160 registers). Against 4
// waves of 16 keys at one wave per SIMD with K in registers: 28-38% faster, one more LDS
// read per step.
template <int D>
constexpr int kv_waves() {
  return 8;
}
template <int D>
constexpr bool kv_k_lds() {
  return D == 256;
}
constexpr int kKvBM = 64;  // queries per tile (the split count's unit)
// Queries per tile of an instantiation: 128 at D <= 64 without a mask (the per-tile costs
// over twice the products), 32 at D = 256, else kKvBM.
template <int D, bool HAS_MASK>
constexpr int kv_bm() {
  return D == 256 ? 32 : (D <= 64 && !HAS_MASK) ? 128 : kKvBM;
}

// SPLIT: one of several workgroups that share a key block's (head, query tile) sequence
// and write fp32 partials (a separate instantiation, so that the unsplit kernel is unchanged).
template <typename T, int D, bool CAUSAL, bool HAS_MASK, typename OutT, bool SPLIT>
__global__ __launch_bounds__(64 * kv_waves<D>(), 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkv_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            const uint16_t* __restrict__ dO,
                                                            const f32x2_t* __restrict__ rowstat,
                                                            OutT* __restrict__ dk, OutT* __restrict__ dv, int Hq,
                                                            int G, int Lq, int Lkv, int n_kblk, int n_bhk,
                                                            int lq_pad, float scale_log2, float scale, Mask mask,
                                                            int nsplit, float* __restrict__ dk_part,
                                                            float* __restrict__ dv_part) {
  using TL = SwzTile<D, 16>;
  constexpr int kKvWaves = kv_waves<D>();
  constexpr int kKvBN = 16 * kKvWaves;  // key rows per workgroup
  constexpr int BM = kv_bm<D, HAS_MASK>();
  constexpr int QB = BM / 16, NCC = BM / 32, PPC = QB / 2;  // 16-query blocks, 32-query chunks, pairs
  constexpr int TILE = BM * TL::RB;
  constexpr int STAT = BM * 8;       // {LSE*log2e, -Delta} of the tile's queries
  // A mask that varies along queries, with aligned rows (vec4), is copied tile by tile into
  // LDS with Q and dO: the tile's BM query rows of the workgroup's keys, row-major, 16-bit
  // elements at most. Read from global memory per score instead, a lane (one key) walks
  // down a column of the mask.
  constexpr int MT = HAS_MASK ? BM * kKvBN * 2 : 0;
  constexpr int BUF = 2 * TILE + STAT + MT;  // one buffer: Q tile, dO tile, stats, mask block
  constexpr bool KLDS = kv_k_lds<D>();
  constexpr int KT = KLDS ? kKvBN * TL::RB : 0;  // the workgroup's K rows (KLDS)
  __shared__ __attribute__((aligned(1024))) uint8_t lds_all[KT + 2 * BUF];
  uint8_t* const lds = lds_all + KT;

  // Low block ids carry the key blocks that see the most causal queries (dispatched
  // first), then the split, then the KV group. With n_bhk a multiple of 8, dispatch
  // id % 8 == bhk % 8: each XCD keeps to its own KV groups.
  const int nsp = SPLIT ? nsplit : 1;
  const int kblk = blockIdx.x / (n_bhk * nsp);
  const int rest = blockIdx.x - kblk * (n_bhk * nsp);
  const int split = SPLIT ? rest / n_bhk : 0;
  const int bhk = rest - split * n_bhk;
  const int Hkv = Hq / G, b = bhk / Hkv, hk = bhk - b * Hkv;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n16 = lane & 15, q4 = lane >> 4;
  const int kw0 = kblk * kKvBN + wave * 16;  // first key of this wave
  const int krow = kw0 + n16;

  // K^T and V^T as B operands: lane (n16, q4) holds row krow, d = 32c + 8*q4 .. +7.
  const int64_t kvoff = (int64_t)bhk * Lkv * D;
  const rsrc_t rk = make_rsrc(k + kvoff, (uint32_t)Lkv * D * 2);
  const rsrc_t rv = make_rsrc(v + kvoff, (uint32_t)Lkv * D * 2);
  u32x4_t kop[KLDS ? 1 : D / 32], vop[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    const uint32_t e = (uint32_t)(krow * D + 32 * c + 8 * q4) * 2;
    if constexpr (!KLDS) kop[c] = buf_load16(rk, e);
    vop[c] = buf_load16(rv, e);
  }
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    if constexpr (!KLDS) settle(kop[c]);
    settle(vop[c]);
  }
  if constexpr (KLDS) {  // the K rows of the workgroup, copied once (waited with the first tile)
    const typename TL::template DmaPlan<kKvBN, kKvWaves> kdma(wave, lane);
    kdma.fill(srd_rows<D>(k + kvoff, Lkv, kblk * kKvBN), lds_all, wave);
  }
  // dK^T, dV^T: block db holds d = 16*db + 4*q4 + i of key krow.
  f32x4_t dka[D / 16], dva[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dka[db][i] = 0.f;
      dva[db][i] = 0.f;
    }

  const int co = Lkv - Lq;  // causal offset: key j visible to query i iff j <= i + co
  const int q_begin = CAUSAL ? (max(0, kblk * kKvBN - co) / BM) * BM : 0;
  const int ntiles = (Lq - q_begin + BM - 1) / BM;
  // (head, query tile) pairs, query tiles from the last one backward and the G heads of
  // each tile together: every workgroup of a KV group starts at the same (last) tile, so
  // the workgroups that run at once stream the same Q / dO tiles and share them in L2.
  const int total = G * ntiles;
  auto tile_of = [&](int it) { return q_begin + (ntiles - 1 - it / G) * BM; };
  // This split's part of the sequence (all of it without splits).
  const int per = SPLIT ? (total + nsplit - 1) / nsplit : total;
  const int it_lo = SPLIT ? min(total, split * per) : 0, it_hi = SPLIT ? min(total, it_lo + per) : total;
  const int L16 = lane & 15;
  const int fa0 = TL::f(n16);            // 16-byte reads: row qm*16 + n16
  const int trow = 4 * q4 + (L16 >> 2);  // transposed reads: rows 32c' + trow (+16)
  const int ft0 = TL::f(trow);
  const int tcol = 8 * (L16 & 1);  // byte within the 16-byte chunk
  const int tch = (L16 & 3) >> 1;  // chunk 2*db + tch
  const typename TL::template DmaPlan<BM, kKvWaves> dma(wave, lane);
  const bool mtile = HAS_MASK && mask.sq != 0 && mask.vec4;
  auto issue = [&](int it, uint8_t* buf) {
    const int gi = it % G, t0 = tile_of(it);
    const int64_t head = (int64_t)(b * Hq + hk * G + gi);
    dma.fill(srd_rows<D>(q + head * Lq * D, Lq, t0), buf, wave);
    dma.fill(srd_rows<D>(dO + head * Lq * D, Lq, t0), buf + TILE, wave);
    if (wave == kKvWaves - 1 && lane < STAT / 16) {
      const srd_t rs = make_srd(rowstat + head * lq_pad + t0, (uint32_t)(Lq - t0) * 8);
      dma16(rs, buf + 2 * TILE, (uint32_t)(16 * lane));
    }
    if constexpr (HAS_MASK) {
      if (mtile) {
        const int es = mask.kind == kMaskBool ? 1 : 2;
        const int lpr = kKvBN * es / 16, rpi = 64 / lpr;  // lanes per row, rows per 1 KiB copy
        const int64_t e0 = (int64_t)b * mask.sb + (int64_t)(hk * G + gi) * mask.sh + (int64_t)t0 * mask.sq +
                           (int64_t)kblk * kKvBN;
        // Elements from e0 through key Lkv - 1 of query row Lq - 1: rows past the end (and
        // keys past the end in the last row) arrive as zeros.
        const int64_t nel = (int64_t)(Lq - 1 - t0) * mask.sq + (Lkv - kblk * kKvBN);
        const srd_t rm =
            make_srd((const uint8_t*)mask.p + e0 * es, (uint32_t)min(nel * es, (int64_t)0xffffffffll));
        for (int i = wave; i < BM / rpi; i += kKvWaves) {
          const int r = i * rpi + lane / lpr;
          dma16(rm, buf + 2 * TILE + STAT + 1024 * i, (uint32_t)(r * mask.sq * es + (lane % lpr) * 16));
        }
      }
    }
  };
  constexpr int NC = D / 32;       // 32-wide steps of the S / dP contraction over d
  constexpr int NCS = NCC * (D / 32);  // stages of the dV / dK products: (c', pair of 16-wide d blocks)

  // One query tile. The LDS operand reads of each stage are issued one stage ahead of the
  // matrix-core instructions that use them; sched_fence() keeps the compiler from sinking
  // them back next to their uses.
  // With a mask: element offset of (this tile's query head, query 0, key krow); rows are
  // added per query (clamped into range: out-of-range entries are zeroed by the edge test).
  const int64_t mkey = HAS_MASK ? (int64_t)b * mask.sb + (int64_t)min(krow, Lkv - 1) : 0;
  // A key-padding mask that removes all 16 keys of this wave leaves dK = dV = 0: no tile work.
  const bool wave_keys = !(HAS_MASK && is_key_padding(mask)) || __any(key_kept(mask, b, kw0, 16, Lkv, lane) != 0u);
  // One that removes every key of the workgroup: no tile is streamed at all (every wave
  // takes the same decision, so no barrier is left unmatched); dK = dV = 0 is written below.
  bool wg_keys = true;
  if constexpr (HAS_MASK) {
    if (is_key_padding(mask)) {
      uint32_t kk = 0u;
#pragma unroll
      for (int r = 0; r < kKvBN / 64; ++r) kk |= key_kept(mask, b, kblk * kKvBN + 64 * r, 64, Lkv, lane);
      wg_keys = __any(kk != 0u);
    }
  }
  const int it_end = wg_keys ? it_hi : it_lo;
  auto tile = [&](bool masked, const uint8_t* qt, const uint8_t* dt, const f32x4_t* st, int t0, int hq, float kbias) {
    // Lane constants made opaque per tile, so that the compiler recomputes the LDS
    // addresses derived from them inside the loop instead of keeping each one live.
    int fa = fa0, ft = ft0, q4x4 = 4 * q4;
    asm volatile("" : "+v"(fa), "+v"(ft), "+v"(q4x4));
    // Stage a of the S / dP products: d step c = a / PPC, query blocks 2*(a % PPC) + 0, 1.
    auto load_a = [&](int a, u32x4_t* qa, u32x4_t* da, u32x4_t& ka) {
      const int c = a / PPC;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int off = ((2 * (a % PPC) + h) * 16 + n16) * TL::RB + ((4 * c + q4) ^ fa) * 16;
        qa[h] = *(const u32x4_t*)(qt + off);
        da[h] = *(const u32x4_t*)(dt + off);
      }
      // K^T operand of step c: row wave*16 + n16 of the K rows, whose swizzle equals that
      // of row n16 (it depends on the row's low 3 bits).
      if constexpr (KLDS)
        if (a % PPC == 0) ka = *(const u32x4_t*)(lds_all + (wave * 16 + n16) * TL::RB + ((4 * c + q4) ^ fa) * 16);
    };
    auto load_c = [&](int si, u32x2_t* tb) {
      const int cc = si / (D / 32), dbp = si % (D / 32);
      const int r0 = (32 * cc + trow) * TL::RB + tcol;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int co = r0 + ((2 * (2 * dbp + e) + tch) ^ ft) * 16;
        tb[4 * e + 0] = lds_read_tr16((const uint16_t*)(dt + co));
        tb[4 * e + 1] = lds_read_tr16((const uint16_t*)(dt + co + 16 * TL::RB));
        tb[4 * e + 2] = lds_read_tr16((const uint16_t*)(qt + co));
        tb[4 * e + 3] = lds_read_tr16((const uint16_t*)(qt + co + 16 * TL::RB));
      }
    };

    // Row statistics of this lane's queries qm*16 + 4*q4 + j: {LSE*log2e, -Delta} pairs, held
    // in registers over the tile at 64 queries, read from LDS where they are used at 128.
    constexpr bool kStatRegs = QB <= 4 && !KLDS;
    f32x4_t sreg[kStatRegs ? 2 * QB : 1];
    if constexpr (kStatRegs) {
#pragma unroll
      for (int i = 0; i < 2 * QB; ++i) sreg[i] = st[((i >> 1) * 16 + 4 * q4) / 2 + (i & 1)];
    }
    auto stat = [&](int qm, int half) {
      if constexpr (kStatRegs)
        return sreg[2 * qm + half];
      else
        return st[(qm * 16 + 4 * q4) / 2 + half];
    };
    u32x4_t qa[2][2], da[2][2], ka[2];
    load_a(0, qa[0], da[0], ka[0]);
    sched_fence();

    // S = Q K^T and dP - Delta = dO V^T - Delta (Delta enters as the accumulator's start)
    // in 16-query blocks qm: lane (n16, q4) holds queries qm*16 + 4*q4 + j of key krow.
    f32x4_t s[QB], dp[QB];
#pragma unroll
    for (int qm = 0; qm < QB; ++qm) {
      const f32x4_t sa = stat(qm, 0), sb = stat(qm, 1);
      s[qm] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      dp[qm] = (f32x4_t){sa[1], sa[3], sb[1], sb[3]};
    }
    u32x2_t tb[2][8];
#pragma unroll
    for (int a = 0; a < PPC * NC; ++a) {
      if (a + 1 < PPC * NC) load_a(a + 1, qa[(a + 1) & 1], da[(a + 1) & 1], ka[((a + 1) / PPC) & 1]);
      else load_c(0, tb[0]);
      const int c = a / PPC;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qm = 2 * (a % PPC) + h;
        s[qm] = mfma16<T>(qa[a & 1][h], KLDS ? ka[c & 1] : kop[KLDS ? 0 : c], s[qm]);
        dp[qm] = mfma16<T>(da[a & 1][h], vop[c], dp[qm]);
      }
      sched_fence();
    }

    // P and dS as B operands; chunk c' (32 queries): e = 0..3 -> block 2c', e = 4..7 -> block 2c'+1.
    // Only the softmax is duplicated for the masked case (a wave-uniform branch), so
    // both paths share the same registers.
    u32x4_t pop[NCC], dsop[NCC];
    // MK: 0 = no mask, a mask constant along queries (kbias) or one read per score; 1 / 2 = a
    // boolean / additive mask block in LDS (this lane's column: key wave*16 + n16).
    const uint8_t* mb = qt + 2 * TILE + STAT;
    const int mcol = wave * 16 + n16;
    auto softmax = [&](auto edge_tag, auto mk_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
      constexpr int MK = decltype(mk_tag)::value;
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        float pv[8], dsv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int qm = 2 * cc + h;
          const f32x4_t sa = stat(qm, 0), sb = stat(qm, 1);
          const float l2[4] = {sa[0], sa[2], sb[0], sb[2]};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float nb = -l2[j];
            if constexpr (HAS_MASK && MK == 1) {  // bias of (query t0 + qm*16 + 4*q4 + j, key krow)
              nb += mb[(qm * 16 + 4 * q4 + j) * kKvBN + mcol] ? 0.f : -INFINITY;
            } else if constexpr (HAS_MASK && MK == 2) {
              nb += to_f32<T>(((const uint16_t*)mb)[(qm * 16 + 4 * q4 + j) * kKvBN + mcol]) * kLog2e;
            } else if constexpr (HAS_MASK) {
              if (mask.sq == 0) {
                nb += kbias;
              } else {
                const int qi = min(t0 + qm * 16 + 4 * q4 + j, Lq - 1);
                nb += mask_bias_log2<T>(mask.p, mask.kind, mkey + (int64_t)hq * mask.sh + (int64_t)qi * mask.sq);
              }
            }
            float p = exp2_le1(fmaf(s[qm][j], scale_log2, nb));
            if constexpr (EDGE) {  // query t0 + qm*16 + j + 4*q4 exists and, if causal, sees key krow
              const int u = t0 + qm * 16 + j + co;  // wave-uniform part
              p = (q4x4 < Lq + co - u && (!CAUSAL || q4x4 - krow >= -u)) ? p : 0.f;
            }
            pv[4 * h + j] = p;
            dsv[4 * h + j] = p * dp[qm][j];
          }
        }
        pop[cc] = (u32x4_t){pack2<T>(pv[0], pv[1]), pack2<T>(pv[2], pv[3]), pack2<T>(pv[4], pv[5]),
                            pack2<T>(pv[6], pv[7])};
        dsop[cc] = (u32x4_t){pack2<T>(dsv[0], dsv[1]), pack2<T>(dsv[2], dsv[3]), pack2<T>(dsv[4], dsv[5]),
                             pack2<T>(dsv[6], dsv[7])};
      }
    };
    auto run_softmax = [&](auto edge_tag) {
      if constexpr (HAS_MASK) {
        if (mtile && mask.kind == kMaskBool) {
          softmax(edge_tag, std::integral_constant<int, 1>{});
          return;
        }
        if (mtile) {
          softmax(edge_tag, std::integral_constant<int, 2>{});
          return;
        }
      }
      softmax(edge_tag, std::integral_constant<int, 0>{});
    };
    if (masked)
      run_softmax(std::true_type{});
    else
      run_softmax(std::false_type{});
    sched_fence();

    // dV^T += dO^T P and dK^T += Q^T dS: A operands transposed out of LDS, rows
    // 32c' + 4*q4 + 0..3 (first read) and + 16 (second read), columns 16*db + L16.
#pragma unroll
    for (int si = 0; si < NCS; ++si) {
      if (si + 1 < NCS) load_c(si + 1, tb[(si + 1) & 1]);
      const int cc = si / (D / 32), dbp = si % (D / 32);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int db = 2 * dbp + e;
        const u32x2_t* b = tb[si & 1] + 4 * e;
        dva[db] = mfma16<T>((u32x4_t){b[0][0], b[0][1], b[1][0], b[1][1]}, pop[cc], dva[db]);
        dka[db] = mfma16<T>((u32x4_t){b[2][0], b[2][1], b[3][0], b[3][1]}, dsop[cc], dka[db]);
      }
      sched_fence();
    }
  };

  // A mask that does not vary along queries (key padding, or a per-head key bias) has one
  // bias per lane (its key) and query head. It is read one step ahead, before that step's
  // tile copies are issued, and taken into a register right after the step's copy wait:
  // read inside the step, its wait would also cover the next tile's copies, which the
  // wait counter orders before it.
  const bool kbias_step = HAS_MASK && mask.sq == 0;
  auto kbias_of = [&](int it) {
    return mask_bias_log2<T>(mask.p, mask.kind, mkey + (int64_t)(hk * G + it % G) * mask.sh);
  };
  float kbias_next = 0.f;
  if (kbias_step && it_lo < it_end) kbias_next = kbias_of(it_lo);
  if (it_lo < it_end) issue(it_lo, lds + (it_lo & 1) * BUF);
  for (int it = it_lo; it < it_end; ++it) {
    wait_vmem();
    __syncthreads();
    float kbias = 0.f;
    if constexpr (HAS_MASK) {
      kbias = kbias_next;
      asm volatile("" : "+v"(kbias));  // the load's wait here, with nothing else in flight
      if (kbias_step && it + 1 < it_end) kbias_next = kbias_of(it + 1);
    }
    if (it + 1 < it_end) issue(it + 1, lds + ((it + 1) & 1) * BUF);
    const uint8_t* qt = lds + (it & 1) * BUF;
    const uint8_t* dt = qt + TILE;
    const f32x4_t* st = (const f32x4_t*)(qt + 2 * TILE);
    const int t0 = tile_of(it);
    if (CAUSAL && t0 + BM - 1 + co < kw0) continue;  // no query of the tile sees this wave's keys
    if (!wave_keys) continue;
    tile((t0 + BM > Lq) || (CAUSAL && t0 + co < kw0 + 15), qt, dt, st, t0, hk * G + it % G, kbias);  // wave-uniform flag
  }
  if constexpr (KLDS) wait_vmem();  // the K copy, when no tile waited for it
  if constexpr (SPLIT) {  // one split: fp32 partials of dK / scale and dV, [split][b*Hkv*Lkv + hk*Lkv + key]
    if (krow < Lkv) {
      const int64_t po = ((int64_t)split * n_bhk + bhk) * Lkv * D + (int64_t)krow * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const int d = db * 16 + 4 * q4;
        *(f32x4_t*)(dk_part + po + d) = dka[db];
        *(f32x4_t*)(dv_part + po + d) = dva[db];
      }
    }
    return;
  }
  if (krow < Lkv) {
    const int64_t ko = kvoff + (int64_t)krow * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int d = db * 16 + 4 * q4;
      Store4<OutT>::run(dk + ko + d, dka[db][0] * scale, dka[db][1] * scale, dka[db][2] * scale, dka[db][3] * scale);
      Store4<OutT>::run(dv + ko + d, dva[db][0], dva[db][1], dva[db][2], dva[db][3]);
    }
  }
}

// Splits of the two kernels (small grids only), at most 16. dQ: enough workgroups for one
// per CU, at least 4 key tiles per split on average; under a causal mask also at least one
// split per 2048 keys (the longest row block sets the kernel's span), but no more than for
// two workgroups per CU. dK/dV (one workgroup per CU): enough for one per CU, at least 8
// (head, 64-query tile) steps per split; two per CU under a causal mask whose triangle spans
// most of the keys (2 Lq > Lkv), where the key blocks near the end see few query tiles and
// about half of the split workgroups have little work. (Measured on 8 and 16 heads of
// 1024-4096 queries at D = 64-256 and GQA 8:1 at 1024 queries against 4096 keys: a second
// workgroup per CU gains less than the fp32 partials and their reduction cost, except in those
// two causal cases.)
int split_count(int64_t work, int64_t target, int64_t steps, int64_t min_steps) {
  if (work >= target) return 1;
  int64_t n = (target + work - 1) / work;
  if (n > steps / min_steps) n = steps / min_steps;
  if (n > 16) n = 16;
  return n < 1 ? 1 : (int)n;
}
int dq_splits(const Shape& s, bool causal) {
  const int64_t bn = s.D == 256 ? 32 : 64;
  const int64_t work = (s.Lq + kDqBM - 1) / kDqBM * s.B * s.Hq, steps = (s.Lkv + bn - 1) / bn;
  const int n = split_count(work, 256, steps, 4);
  if (!causal) return n;
  return min(split_count(work, 2 * 256, steps, 4), max(n, (int)((s.Lkv + 2047) / 2048)));
}
int dkv_splits(const Shape& s, bool causal) {
  const int64_t bn = 128;  // 8 waves x 16 keys
  const bool triangle = causal && 2 * s.Lq > s.Lkv;
  return split_count((s.Lkv + bn - 1) / bn * s.B * s.Hkv, (triangle ? 2 : 1) * 256,
                     (s.Hq / s.Hkv) * ((s.Lq + kKvBM - 1) / kKvBM), 8);
}
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
// Workspace: {LSE*log2e, -Delta} pairs, then (split grids) the dQ partials, then the dK and
// dV partials.
size_t rowstat_bytes(const Shape& s) { return align256((size_t)(s.B * s.Hq * tiled_rowstat_stride(s.Lq)) * 8); }
size_t dq_part_bytes(const Shape& s, bool causal) {
  const int n = dq_splits(s, causal);
  return n > 1 ? align256((size_t)n * (size_t)(s.B * s.Hq * s.Lq * s.D) * 4) : 0;
}
size_t dkv_part_bytes(const Shape& s, bool causal) {  // each of dK, dV
  const int n = dkv_splits(s, causal);
  return n > 1 ? align256((size_t)n * (size_t)(s.B * s.Hkv * s.Lkv * s.D) * 4) : 0;
}

template <typename T, int D, bool C, bool M, typename OutT>
hipError_t launch_typed(const Shape& s, Dt out, const Mask& mask, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv, float* ws,
                        float scale, int stages, hipStream_t st) {
  f32x2_t* rowstat = (f32x2_t*)ws;  // [B*Hq][lq_pad] {LSE*log2e, -Delta}
  const int lq_pad = (int)tiled_rowstat_stride(s.Lq);
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  const int G = (int)(s.Hq / s.Hkv);
  char* parts = (char*)ws + rowstat_bytes(s);
  if (stages & kStage0) {
    const int n_qblk = (int)((s.Lq + kDqBM - 1) / kDqBM);
    const int n_bh = (int)(s.B * s.Hq);
    const int nsplit = dq_splits(s, C);
    constexpr int BN = dq_bn<D, M>();
    const int nt = (int)((s.Lkv + BN - 1) / BN);
    float* dq_part = nsplit > 1 ? (float*)parts : nullptr;
    if constexpr (D == 256)
      hipLaunchKernelGGL((dq16_kernel<T, D, C, M, OutT>), dim3(n_qblk * n_bh * nsplit), dim3(64 * kDq16Waves), 0,
                         st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const OutT*)o, lse,
                         (const uint16_t*)dO, (OutT*)dq, rowstat, (int)s.Hq, G, (int)s.Lq, (int)s.Lkv, n_qblk, n_bh,
                         lq_pad, scale_log2, scale, mask, nsplit, (nt + nsplit - 1) / nsplit, dq_part);
    else
      hipLaunchKernelGGL((dq_kernel<T, D, C, M, OutT>), dim3(n_qblk * n_bh * nsplit), dim3(kThreads),
                         (M && dq_mask_staged<D>(mask)) ? 2 * (size_t)kDqBM * BN : 0, st,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const OutT*)o, lse,
                         (const uint16_t*)dO, (OutT*)dq, rowstat, (int)s.Hq, G, (int)s.Lq, (int)s.Lkv, n_qblk, n_bh,
                         lq_pad, scale_log2, scale, mask, nsplit, (nt + nsplit - 1) / nsplit, dq_part);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && nsplit > 1) e = launch_split_reduce(s, out, nsplit, dq_part, dq, s.B * s.Hq * s.Lq, scale, st);
    if (e != hipSuccess) return e;
  }
  if (!(stages & kStage1)) return hipSuccess;
  constexpr int kKvBN = 16 * kv_waves<D>();
  const int n_kblk = (int)((s.Lkv + kKvBN - 1) / kKvBN);
  const int n_bhk = (int)(s.B * s.Hkv);
  const int nsplit = dkv_splits(s, C);
  float* dk_part = nsplit > 1 ? (float*)(parts + dq_part_bytes(s, C)) : nullptr;
  float* dv_part = nsplit > 1 ? (float*)(parts + dq_part_bytes(s, C) + dkv_part_bytes(s, C)) : nullptr;
  auto kern = nsplit > 1 ? dkv_kernel<T, D, C, M, OutT, true> : dkv_kernel<T, D, C, M, OutT, false>;
  hipLaunchKernelGGL(kern, dim3(n_kblk * n_bhk * nsplit), dim3(64 * kv_waves<D>()), 0, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dO, (const f32x2_t*)rowstat, (OutT*)dk,
                     (OutT*)dv, (int)s.Hq, G, (int)s.Lq, (int)s.Lkv, n_kblk, n_bhk, lq_pad, scale_log2, scale, mask,
                     nsplit, dk_part, dv_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  return launch_split_reduce_pair(s, out, nsplit, dk_part, dk, scale, dv_part, dv, 1.f, s.B * s.Hkv * s.Lkv, st);
}

template <typename T, int D, typename OutT>
hipError_t launch_mode(const Shape& s, Dt out, bool causal, const Mask& mask, const void* q, const void* k,
                       const void* v, const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                       float* ws, float scale, int stages, hipStream_t st) {
  if (causal)
    return launch_typed<T, D, true, false, OutT>(s, out, mask, q, k, v, o, lse, dO, dq, dk, dv, ws, scale, stages,
                                                 st);
  if (mask.kind != kMaskNone)
    return launch_typed<T, D, false, true, OutT>(s, out, mask, q, k, v, o, lse, dO, dq, dk, dv, ws, scale, stages,
                                                 st);
  return launch_typed<T, D, false, false, OutT>(s, out, mask, q, k, v, o, lse, dO, dq, dk, dv, ws, scale, stages,
                                                st);
}

template <typename T, typename OutT>
hipError_t launch_d(const Shape& s, Dt out, bool causal, const Mask& mask, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv, float* ws,
                    float scale, int stages, hipStream_t st) {
#define SDPA_BWD_D(DD) \
  case DD: return launch_mode<T, DD, OutT>(s, out, causal, mask, q, k, v, o, lse, dO, dq, dk, dv, ws, scale, stages, st);
  switch (s.D) {
    SDPA_BWD_D(32)
    SDPA_BWD_D(64)
    SDPA_BWD_D(96)
    SDPA_BWD_D(128)
    SDPA_BWD_D(256)
    default: return hipErrorInvalidValue;
  }
#undef SDPA_BWD_D
}

}  // namespace

size_t tiled_bwd_workspace(const Shape& s, bool causal) {
  return rowstat_bytes(s) + dq_part_bytes(s, causal) + 2 * dkv_part_bytes(s, causal);
}

hipError_t launch_bwd_tiled(const Shape& s, Dt dt, Dt out, bool causal, const Mask& mask, const void* q,
                            const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
                            void* dk, void* dv, float* ws, float scale, int stages, hipStream_t st) {
  if (dt == kBF16)
    return out == kF32
               ? launch_d<bf16_t, float>(s, out, causal, mask, q, k, v, o, lse, dO, dq, dk, dv, ws, scale, stages, st)
               : launch_d<bf16_t, bf16_t>(s, out, causal, mask, q, k, v, o, lse, dO, dq, dk, dv, ws, scale, stages,
                                          st);
  if (dt == kF16)
    return out == kF32
               ? launch_d<f16_t, float>(s, out, causal, mask, q, k, v, o, lse, dO, dq, dk, dv, ws, scale, stages, st)
               : launch_d<f16_t, f16_t>(s, out, causal, mask, q, k, v, o, lse, dO, dq, dk, dv, ws, scale, stages, st);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
