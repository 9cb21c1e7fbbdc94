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
// Work decomposition: one workgroup = 4 waves = 128 query rows of one (batch, query head)
// (8 waves = 256 rows at D = 128 without a mask); each wave owns 32 rows. Key/value tiles
// of 64 rows (32 at D = 256, 128 at D <= 64 and D = 128 without a mask) are copied into LDS
// by direct buffer-to-LDS loads (range-checked, so rows past the end arrive as zeros),
// double-buffered so that tile t+1 streams in while tile t is consumed, and shared by the
// workgroup's waves. Tiles are stored
// unpadded with an XOR swizzle of 16-byte chunks (SwzTile) that keeps both read patterns
// conflict-free.
//
// Orientation: the scores are computed transposed, S^T = K Q^T, so that in the
// 32x32 accumulator each lane holds 16 scores of ONE query row (lanes l and
// l+32 split the 32 keys of a block). Row max / row sum then need one
// half-wave exchange, the rescale factor is per lane, and the probabilities
// already sit in the B-operand layout of O^T += V^T P^T. V^T is read from the
// row-major V tile with the LDS transpose read.
//
// Small grids: when there are fewer (query block, head) workgroups than two per CU (one
// head of a few thousand queries, say), the keys are split into contiguous ranges of whole
// tiles handled by separate workgroups. Each writes its rows' unnormalised O, reference
// maximum m and row sum l (fp32), and a combine kernel merges the splits exactly as the
// online softmax merges tiles: m* = max m_s, O = sum O_s 2^(m_s - m*) / sum l_s 2^(m_s - m*).
//
// Masks and sinks (MASKED instantiations; the sink is a runtime pointer): the mask's
// bias enters every score in the log2 domain before the row maximum, and a row's sink
// logit seeds the reference maximum and the row sum as if it were a first key with no
// value (the drop-in semantics that mps-flash-sdpa 0.1.0, "When MFA Dispatches vs.
// Falls Back", and the MLX pull request, "Limitations", leave to the unfused path).
#include "device_common.h"
#include "kernels.h"

namespace sdpa {
namespace {

// Keys per tile: 64, or 32 at D = 256, where the O accumulators alone take 128 registers
// per lane and a 64-key score block would not fit beside them. Every head dim runs two
// waves per SIMD: at D = 256 that leaves 256 registers per lane for 128 of accumulators
// and 64 of Q operands (the masked instantiation spills a few registers; measured 16-29%
// faster than one wave per SIMD).
// Without a mask, D <= 64 and D = 128 take 128-key tiles: the per-tile costs (barrier, row
// maximum, rescale test, copy issue) over twice the products (2-8% faster measured at
// D <= 64; with a mask the larger tile ran slower). At D = 128 two 128-key K/V buffers take
// 128 KiB of LDS, so the workgroup grows to 8 waves (256 rows) for two waves per SIMD, with
// K operands one stage ahead and the LDS address lane constants rebuilt per tile (256
// registers, no spills): 4-6% faster without the causal mask, level with it.
template <int D, bool MASKED>
constexpr int fwd_bn() {
  return D == 256 ? 32 : ((D <= 64 || D == 128) && !MASKED) ? 128 : 64;
}
// Waves per workgroup: 8 (256 query rows, one workgroup per CU) for unmasked D = 128 with
// its 128-key tiles (two 64 KiB K/V buffers), else 4 (two workgroups per CU).
template <int D, bool MASKED>
constexpr int fwd_waves() {
  return (D == 128 && !MASKED) ? 8 : 4;
}

template <typename T, int D, bool CAUSAL, bool MASKED, typename OutT>
__global__ __launch_bounds__((64 * fwd_waves<D, MASKED>()), (8 / fwd_waves<D, MASKED>())) void fwd_tiled_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    OutT* __restrict__ o, float* __restrict__ lse, int Hq, int G, int Lq, int Lkv, int n_qblk, int n_bh,
    float scale_log2, Mask mask, const float* __restrict__ sinks, int nsplit, int split_tiles,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  using TL = SwzTile<D>;
  constexpr int kFwdBN = fwd_bn<D, MASKED>();
  constexpr int W = fwd_waves<D, MASKED>();
  constexpr int kFwdBM = 32 * W;  // query rows per workgroup
  constexpr int TILE = kFwdBN * TL::RB;  // bytes of one K or V tile
  // [buffer][K, V] tiles; buffer t & 1 holds key tile t while tile t + 1 streams into the other.
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * 2 * TILE];

  // Work id: query block major (longest causal rows first), then key split, then (b, hq)
  // with the G heads of a KV group adjacent and co-located on one XCD.
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
  const int q0 = qblk * kFwdBM + wave * 32;  // wave-uniform
  const int qrow = q0 + n;

  const int64_t kvoff = (int64_t)(b * Hkv + hk) * Lkv * D;
  const rsrc_t rq = make_rsrc(q + (int64_t)bh * Lq * D, (uint32_t)Lq * D * 2);

  // Q^T as the B operand: lane (n, g) holds Q[qrow][16c + 8g .. +7] (rows past Lq read as zero).
  // The scale is folded into Q's sign: the kernel only ever multiplies scores by a positive
  // factor, so that the row maximum and the -inf of masked keys are taken on scaled scores.
  u32x4_t qop[D / 16];
  const QSign qs = q_sign(scale_log2);
  scale_log2 = qs.scale_log2;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) qop[c] = qs.apply(buf_load16(rq, (uint32_t)((qrow * D + 16 * c + 8 * g) * 2)));
#pragma unroll
  for (int c = 0; c < D / 16; ++c) settle(qop[c]);

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -INFINITY;  // reference row max of the log2-domain scores (see kRescaleSlack)
  float lsum = 0.f;     // this lane's share of the running row sum
  float lcomp = 0.f;    // its compensation term (kahan_add)
  if (sinks != nullptr) {  // the sink: a first "key" of score sink*log2e and no value
    const float sk = sinks[hq] * kLog2e;
    if (sk > -INFINITY) {
      m = sk;
      lsum = g == 0 ? 1.f : 0.f;
    }
  }
  // With a mask the scores are moved to the log2 domain (scale and bias) before the row
  // maximum, and the remaining steps take them with unit scale.
  const float sl2 = MASKED ? 1.f : scale_log2;
  const int64_t mrow = MASKED ? (int64_t)b * mask.sb + (int64_t)hq * mask.sh + (int64_t)min(qrow, Lq - 1) * mask.sq : 0;

  // Causal: key j is visible to query i iff j <= i + co, co = Lkv - Lq >= 0 (sequences
  // aligned at their ends; co = 0 when the lengths are equal).
  const int co = Lkv - Lq;
  const int kv_end = CAUSAL ? min(Lkv, qblk * kFwdBM + kFwdBM + co) : Lkv;
  const int ntiles = (kv_end + kFwdBN - 1) / kFwdBN;
  // This workgroup's key tiles: all of them, or one split's range (empty for a causal block
  // that ends before the split begins).
  const int t_lo = split * split_tiles, t_hi = min(ntiles, t_lo + split_tiles);
  const int key_lim = CAUSAL ? min(Lkv, qrow + 1 + co) : Lkv;  // keys >= key_lim are masked for this row

  // Per-lane LDS offsets. K rows (16-byte reads): row kb*32 + n, chunk 2c + g.
  // V^T (transposed 8-byte reads): row kb*32 + 16*c2 + 4g + L16/4 (+8), column chunk
  // 4*db + 2*(G16&1) + (L16&3)/2, byte 8*(L16&1) within the chunk.
  const int G16 = lane >> 4, L16 = lane & 15;
  const int fk = TL::f(n);
  const int vrow = 4 * g + (L16 >> 2);
  const int fv = TL::f(vrow), fv8 = TL::f(vrow + 8);  // swizzle of the two rows each transposed read pair uses
  const int vx = 2 * (G16 & 1) + ((L16 & 3) >> 1);

  const uint16_t* kbase = k + kvoff;
  const uint16_t* vbase = v + kvoff;
  const typename TL::template DmaPlan<kFwdBN, W> dma(wave, lane);
  // A boolean mask that varies along queries (mask_staged): the block of the workgroup's
  // query rows and the tile's keys is copied into dynamic LDS ([buffer][row][key], one
  // byte each) with K and V, 16 bytes per lane; rows past Lq arrive as zeros.
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_mask[];
  constexpr int MBLK = kFwdBM * kFwdBN;  // bytes of one buffer's mask block
  const bool mstage = MASKED && mask_staged(mask);
  auto stage_mask = [&](int t) {
    constexpr int LPR = kFwdBN / 16, RPI = 64 / LPR;  // lanes per row, rows per 1 KiB copy
    const int kt0 = t * kFwdBN, r0 = qblk * kFwdBM;
    const int64_t e0 = (int64_t)b * mask.sb + (int64_t)hq * mask.sh + (int64_t)r0 * mask.sq + kt0;
    const int64_t nel = (int64_t)(Lq - 1 - r0) * mask.sq + (Lkv - kt0);  // through row Lq - 1, key Lkv - 1
    const srd_t rm = make_srd((const uint8_t*)mask.p + e0, (uint32_t)min(nel, (int64_t)0xffffffffll));
    uint8_t* mb = lds_mask + (t & 1) * MBLK;
    for (int i = wave; i < kFwdBM / RPI; i += W) {
      const int r = i * RPI + lane / LPR;
      dma16(rm, mb + 1024 * i, (uint32_t)(r * mask.sq + (lane % LPR) * 16));
    }
  };
  if (t_lo < t_hi) {
    uint8_t* b0 = lds + (t_lo & 1) * 2 * TILE;
    dma.fill(srd_rows<D>(kbase, Lkv, t_lo * kFwdBN), b0, wave);
    dma.fill(srd_rows<D>(vbase, Lkv, t_lo * kFwdBN), b0 + TILE, wave);
    if (mstage) stage_mask(t_lo);
  }
  // Key padding: a tile whose keys are all padding adds nothing and is skipped; its mask
  // bytes are read one tile ahead.
  const bool pad = MASKED && is_key_padding(mask);
  uint32_t kept_next = pad && t_lo < t_hi ? key_kept(mask, b, t_lo * kFwdBN, kFwdBN, Lkv, lane) : 1u;
  for (int t = t_lo; t < t_hi; ++t) {
    wait_vmem();
    __syncthreads();  // tile t is in LDS; every wave has finished tile t - 1
    if (t + 1 < t_hi) {
      uint8_t* nb = lds + ((t + 1) & 1) * 2 * TILE;
      dma.fill(srd_rows<D>(kbase, Lkv, (t + 1) * kFwdBN), nb, wave);
      dma.fill(srd_rows<D>(vbase, Lkv, (t + 1) * kFwdBN), nb + TILE, wave);
      if (mstage) stage_mask(t + 1);
    }
    const uint32_t kept = kept_next;
    if (pad && t + 1 < t_hi) kept_next = key_kept(mask, b, (t + 1) * kFwdBN, kFwdBN, Lkv, lane);
    const uint8_t* kt = lds + (t & 1) * 2 * TILE;
    const uint8_t* vt = kt + TILE;
    const int kt0 = t * kFwdBN;
    if (CAUSAL && kt0 > q0 + 31 + co) continue;  // tile entirely above this wave's diagonal
    if (pad && !__any(kept != 0u)) continue;  // every key of the tile is padding

    // At D = 256 (two waves per SIMD, 128 registers of O accumulators) and with 128-key tiles
    // at D = 128 (128 registers of scores) the lane constants of the LDS addresses are made
    // opaque per tile, so that the compiler rebuilds each stage's address inside the loop
    // instead of keeping all of them live across it.
    int fkx = fk, fvx = fv, fv8x = fv8, nrow = n * TL::RB;
    if constexpr (D == 256 || (D == 128 && kFwdBN == 128)) asm volatile("" : "+v"(fkx), "+v"(fvx), "+v"(fv8x), "+v"(nrow));
    // S^T = K Q^T: 32 keys x 32 queries per accumulator block.
    f32x16_t s[kFwdBN / 32];
#pragma unroll
    for (int kb = 0; kb < kFwdBN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    // K operands are read KD - 1 stages of the contraction ahead of the matrix-core
    // instructions that use them (two, or one at D = 256 and with 128-key tiles at D = 128,
    // for registers), behind scheduling fences.
    constexpr int KD = (D == 256 || (D == 128 && kFwdBN == 128)) ? 2 : 3;
    u32x4_t ka[KD][kFwdBN / 32];
    // Chunk 2c + g of row n sits at chunk (2c + g) ^ f(n); f < 16, so for c >= 8 (D = 256)
    // that is 16 + ((2(c - 8) + g) ^ f(n)): eight lane-dependent offsets and constants.
    static_assert(D / 16 <= 16, "chunk index split assumes at most 32 chunks per row");
    auto load_k = [&](int c, u32x4_t* a) {
#pragma unroll
      for (int kb = 0; kb < kFwdBN / 32; ++kb)
        a[kb] = *(const u32x4_t*)(kt + kb * 32 * TL::RB + nrow + ((2 * (c & 7) + g) ^ fkx) * 16 + (c >> 3) * 256);
    };
#pragma unroll
    for (int c = 0; c < KD - 1; ++c) load_k(c, ka[c]);
    sched_fence();
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      if (c + KD - 1 < D / 16) load_k(c + KD - 1, ka[(c + KD - 1) % KD]);
#pragma unroll
      for (int kb = 0; kb < kFwdBN / 32; ++kb) s[kb] = mfma32<T>(ka[c % KD][kb], qop[c], s[kb]);
      sched_fence();
    }

    if (MASKED && D <= 128 && pad) {
      // Key padding: the keep flags of the tile's keys are already in registers (one byte per
      // lane, read a tile ahead); a ballot gathers them, bit j for key kt0 + j (keys past
      // the end read as dropped), and each score takes its key's bit. (At D = 256 the
      // general path below, which spills fewer registers there.)
      const uint64_t keep = __ballot(kept != 0u);
#pragma unroll
      for (int kb = 0; kb < kFwdBN / 32; ++kb) {
        // Bits 8r + j of lm: key kt0 + kb*32 + 8r + 4g + j, the lane's element 4r + j.
        const uint32_t lm = (uint32_t)(keep >> (32 * kb)) >> (4 * g);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kb][i] = ((lm >> (8 * (i >> 2) + (i & 3))) & 1u) ? s[kb][i] * scale_log2 : -INFINITY;
      }
    } else if (MASKED && D <= 128 && mstage) {  // a staged boolean mask: as below, the flags from LDS
      const uint8_t* mrow_l = lds_mask + (t & 1) * MBLK + (wave * 32 + n) * kFwdBN + 4 * g;  // this lane's row
#pragma unroll
      for (int kb = 0; kb < kFwdBN / 32; ++kb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {  // keys key0 .. key0 + 3
          const int key0 = kt0 + kb * 32 + 8 * i4 + 4 * g;
          float bias[4];
          mask_bias4_bool_word(*(const uint32_t*)(mrow_l + kb * 32 + 8 * i4), bias);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            s[kb][4 * i4 + j] = key0 + j < Lkv ? fmaf(s[kb][4 * i4 + j], scale_log2, bias[j]) : -INFINITY;
        }
    } else if constexpr (MASKED) {  // every tile: s <- s*scale*log2e + bias, keys past the end -inf
#pragma unroll
      for (int kb = 0; kb < kFwdBN / 32; ++kb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {  // keys key0 .. key0 + 3
          const int key0 = kt0 + kb * 32 + 8 * i4 + 4 * g;
          float bias[4];
          if (D == 256 && mstage) {  // (at D = 256 the branch inside the loop spills fewer registers)
            mask_bias4_bool_word(
                *(const uint32_t*)(lds_mask + (t & 1) * MBLK + (wave * 32 + n) * kFwdBN + kb * 32 + 8 * i4 + 4 * g),
                bias);
          } else if (mask.vec4 && key0 < Lkv) {
            mask_bias4_log2<T>(mask.p, mask.kind, mrow + key0, bias);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              bias[j] = key0 + j < Lkv ? mask_bias_log2<T>(mask.p, mask.kind, mrow + key0 + j) : -INFINITY;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
            s[kb][4 * i4 + j] = key0 + j < Lkv ? fmaf(s[kb][4 * i4 + j], scale_log2, bias[j]) : -INFINITY;
        }
    } else if ((kt0 + kFwdBN > Lkv) || (CAUSAL && kt0 + kFwdBN - 1 > q0 + co)) {
      // Mask (only tiles that reach past the diagonal or the end), then the row max on raw scores.
#pragma unroll
      for (int kb = 0; kb < kFwdBN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          s[kb][i] = key < key_lim ? s[kb][i] : -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kFwdBN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[kb][i]);
    tmax = half_swap_max(tmax) * sl2;
    // Raise the reference max only past the slack; rescale O when any row of the wave moved.
    const bool grow = tmax > m + kRescaleSlack;
    if (__any(grow)) {
      const float m_new = grow ? tmax : m;
      // A row that did not move keeps its scale: its m may still be -inf (a mask, or a key
      // split that starts past the row's causal limit), where m - m_new would be NaN.
      const float alpha = grow ? fast_exp2(m - m_new) : 1.f;
      m = m_new;
      lsum *= alpha;
      lcomp *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    const float neg_m = (m == -INFINITY) ? 0.f : -m;

    // P = 2^(s*scale*log2e - m), rounded to the operand type, then O^T += V^T P^T.
    // B operand chunk (kb, c2) covers keys kb*32 + 16*c2 + {4g..4g+3, 8+4g..8+4g+3}.
    // The tile's probabilities are summed first and added to the row sum once, with
    // compensation: added one by one, over millions of keys each term falls near the
    // sum's rounding step.
    float tsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < kFwdBN / 32; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(s[kb][8 * c2 + e], sl2, neg_m));
          tsum += p[e];
        }
        const u32x4_t pop = (u32x4_t){pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]), pack2<T>(p[4], p[5]),
                                      pack2<T>(p[6], p[7])};
        const uint8_t* vrow_p = vt + (kb * 32 + 16 * c2 + vrow) * TL::RB + 8 * (L16 & 1);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int ch = 4 * db + vx;
          const u32x2_t lo = lds_read_tr16((const uint16_t*)(vrow_p + (ch ^ fvx) * 16));
          const u32x2_t hi = lds_read_tr16((const uint16_t*)(vrow_p + 8 * TL::RB + (ch ^ fv8x) * 16));
          oacc[db] = mfma32<T>((u32x4_t){lo[0], lo[1], hi[0], hi[1]}, pop, oacc[db]);
        }
      }
    kahan_add(lsum, lcomp, tsum);
  }

  const float l = half_swap_sum(lsum);
  // The epilogue's lane indices, rebuilt here from the lane count of the (full) execution
  // mask rather than kept in registers across the key loop (at D = 256 they would spill).
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int ge = lane_e >> 5, qre = q0 + (lane_e & 31);
  if (part_o != nullptr) {  // one key split: unnormalised partials [split][b*Hq*Lq + hq*Lq + q]
    if (qre < Lq) {
      const int64_t prow = ((int64_t)split * n_bh + bh) * Lq + qre;
      float* po = part_o + prow * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4_t*)(po + db * 32 + 8 * r4 + 4 * ge) =
              (f32x4_t){oacc[db][4 * r4], oacc[db][4 * r4 + 1], oacc[db][4 * r4 + 2], oacc[db][4 * r4 + 3]};
      if (ge == 0) *(f32x2_t*)(part_ml + prow * 2) = (f32x2_t){m, l};
    }
    return;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (qre < Lq) {
    OutT* orow = o + ((int64_t)bh * Lq + qre) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        Store4<OutT>::run(orow + db * 32 + 8 * r4 + 4 * ge, oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv,
                          oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
    if (lse != nullptr && ge == 0) lse[(int64_t)bh * Lq + qre] = (m + fast_log2(l)) * kLn2;
  }
}

template <typename T, int D, bool C, bool M, typename OutT>
hipError_t launch_typed(const Shape& s, Dt out, const Mask& mask, const float* sinks, const void* q, const void* k,
                        const void* v, void* o, float* lse, float scale, void* ws, hipStream_t st) {
  constexpr int BMW = 32 * fwd_waves<D, M>();
  const int n_qblk = (int)((s.Lq + BMW - 1) / BMW);
  const int n_bh = (int)(s.B * s.Hq);
  const float scale_log2 = (float)((double)scale * 1.4426950408889634);
  constexpr int BN = fwd_bn<D, M>();
  const int nt = (int)((s.Lkv + BN - 1) / BN);
  const int nsplit = tiled_fwd_splits(s);
  const int split_tiles = (nt + nsplit - 1) / nsplit;
  float* part_o = nsplit > 1 ? (float*)ws : nullptr;
  float* part_ml = nsplit > 1 ? part_o + (int64_t)nsplit * s.B * s.Hq * s.Lq * s.D : nullptr;
  // With key splits the sink joins in the combine kernel, once per row.
  const size_t mshm = (M && mask_staged(mask)) ? 2 * (size_t)BMW * BN : 0;  // staged mask blocks
  hipLaunchKernelGGL((fwd_tiled_kernel<T, D, C, M, OutT>), dim3(n_qblk * n_bh * nsplit), dim3(BMW * 2), mshm, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (OutT*)o, lse, (int)s.Hq,
                     (int)(s.Hq / s.Hkv), (int)s.Lq, (int)s.Lkv, n_qblk, n_bh, scale_log2, mask,
                     nsplit > 1 ? nullptr : sinks, nsplit, split_tiles, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  return launch_split_combine(s, out, nsplit, part_o, part_ml, sinks, o, lse, st);
}

template <typename T, int D, typename OutT>
hipError_t launch_mode(const Shape& s, Dt out, bool causal, const Mask& mask, const float* sinks, const void* q,
                       const void* k, const void* v, void* o, float* lse, float scale, void* ws, hipStream_t st) {
  if (causal) return launch_typed<T, D, true, false, OutT>(s, out, mask, sinks, q, k, v, o, lse, scale, ws, st);
  if (mask.kind != kMaskNone)
    return launch_typed<T, D, false, true, OutT>(s, out, mask, sinks, q, k, v, o, lse, scale, ws, st);
  return launch_typed<T, D, false, false, OutT>(s, out, mask, sinks, q, k, v, o, lse, scale, ws, st);
}

template <typename T, typename OutT>
hipError_t launch_d(const Shape& s, Dt out, bool causal, const Mask& mask, const float* sinks, const void* q,
                    const void* k, const void* v, void* o, float* lse, float scale, void* ws, hipStream_t st) {
  switch (s.D) {
    case 32: return launch_mode<T, 32, OutT>(s, out, causal, mask, sinks, q, k, v, o, lse, scale, ws, st);
    case 64: return launch_mode<T, 64, OutT>(s, out, causal, mask, sinks, q, k, v, o, lse, scale, ws, st);
    case 96: return launch_mode<T, 96, OutT>(s, out, causal, mask, sinks, q, k, v, o, lse, scale, ws, st);
    case 128: return launch_mode<T, 128, OutT>(s, out, causal, mask, sinks, q, k, v, o, lse, scale, ws, st);
    case 256: return launch_mode<T, 256, OutT>(s, out, causal, mask, sinks, q, k, v, o, lse, scale, ws, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Key splits (small grids only): enough workgroups for one per CU (256 CUs), counted in the
// workgroups the unmasked instantiation launches (256 query rows at D = 128, 128 otherwise),
// and for two per CU at D = 256; each split keeps at least 4 key tiles of 64 keys on average
// (counted in 64-key tiles whatever the instantiation's tile, so that the count, and the
// workspace, do not depend on the mask); at most 16 splits. At D <= 96 a second 4-wave
// workgroup per CU gains less than its fp32 partials and their combine cost (measured on 8
// and 16 heads of 1024-4096 queries, fp16 D = 64: 8 heads of 2048 take 22 us with two splits
// against 26 us with four); at D = 256 the longer tiles make the second one pay.
int tiled_fwd_splits(const Shape& s) {
  const int64_t bn = s.D == 256 ? 32 : 64;
  const int64_t rows = s.D == 128 ? 256 : 128;
  const int64_t work = (s.Lq + rows - 1) / rows * s.B * s.Hq;
  const int64_t target = s.D == 256 ? 2 * 256 : 256;
  if (work >= target) return 1;
  const int64_t nt = (s.Lkv + bn - 1) / bn;
  int64_t n = (target + work - 1) / work;
  if (n > nt / 4) n = nt / 4;
  if (n > 16) n = 16;
  return n < 1 ? 1 : (int)n;
}

size_t tiled_fwd_workspace(const Shape& s) {
  const int n = tiled_fwd_splits(s);
  if (n == 1) return 0;
  return (size_t)n * (size_t)(s.B * s.Hq * s.Lq) * (size_t)(s.D + 2) * sizeof(float);
}

hipError_t launch_fwd_tiled(const Shape& s, Dt dt, Dt out, bool causal, const Mask& mask, const float* sinks,
                            const void* q, const void* k, const void* v, void* o, float* lse, float scale, void* ws,
                            hipStream_t st) {
  if (dt == kBF16)
    return out == kF32 ? launch_d<bf16_t, float>(s, out, causal, mask, sinks, q, k, v, o, lse, scale, ws, st)
                       : launch_d<bf16_t, bf16_t>(s, out, causal, mask, sinks, q, k, v, o, lse, scale, ws, st);
  if (dt == kF16)
    return out == kF32 ? launch_d<f16_t, float>(s, out, causal, mask, sinks, q, k, v, o, lse, scale, ws, st)
                       : launch_d<f16_t, f16_t>(s, out, causal, mask, sinks, q, k, v, o, lse, scale, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
