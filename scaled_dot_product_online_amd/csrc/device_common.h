// Device helpers shared by the attention kernels (gfx950 / CDNA4 only).
//
// Matrix-core conventions used throughout (confirmed on gfx950 hardware with
// integer-valued operands):
//   v_mfma_f32_32x32x16_{bf16,f16}: lane l supplies row/column (l % 32) and the
//   8 consecutive k values 8*(l/32) .. 8*(l/32)+7 of its A row / B column;
//   accumulator element i of lane l is C[8*(i/4) + 4*(l/32) + (i%4)][l % 32].
//   ds_read_b64_tr_b16: within each group of 16 lanes, lane L reads 4 16-bit
//   elements at its own address; the result in lane i is element (i % 4) of
//   the addresses given by lanes 4*r + i/4, r = 0..3 — i.e. when lanes 4r..4r+3
//   address row r of a 4 x 16 block, lane i receives column i.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sdpa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Storage types. 16-bit operands travel as raw bits; the tag selects arithmetic.
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- MFMA -------------------------------------------------------------------
template <typename T> __device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c);
template <> __device__ __forceinline__ f32x16_t mfma32<bf16_t>(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16_t mfma32<f16_t>(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

template <typename T> __device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c);
template <> __device__ __forceinline__ f32x4_t mfma16<bf16_t>(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4_t mfma16<f16_t>(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

// ---- conversions --------------------------------------------------------------
// Two fp32 values -> one dword of two 16-bit values (round to nearest even);
// `lo` lands in bits 0..15.
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) {
  bf16x2_t r = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}
template <> __device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi) {
  f16x2_t r = __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}
template <typename T> __device__ __forceinline__ float to_f32(uint16_t bits);
template <> __device__ __forceinline__ float to_f32<bf16_t>(uint16_t bits) {
  return __uint_as_float(((uint32_t)bits) << 16);
}
template <> __device__ __forceinline__ float to_f32<f16_t>(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}
// Low / high 16-bit element of a dword as fp32.
template <typename T> __device__ __forceinline__ float lo_f32(uint32_t w) { return to_f32<T>((uint16_t)(w & 0xffffu)); }
template <typename T> __device__ __forceinline__ float hi_f32(uint32_t w) { return to_f32<T>((uint16_t)(w >> 16)); }

// ---- exp2 / log2 (hardware v_exp_f32 / v_log_f32) --------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
// exp2(min(x, 0)): the backward's probabilities with the exponent clamped above at 0, as
// exp2(x) clamped to [0, 1] (equal, since exp2 is increasing and exp2(0) = 1), which the
// compiler folds into the clamp bit of v_exp_f32 instead of a separate v_min_f32.
__device__ __forceinline__ float exp2_le1(float x) { return __builtin_amdgcn_fmed3f(fast_exp2(x), 0.f, 1.f); }

// ---- half-wave exchange: lanes l and l^32 ------------------------------------------
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; feeding x twice leaves {own, partner} in each lane.
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- online softmax ------------------------------------------------------------------
// A row's reference maximum (log2 domain) is raised only when a tile's maximum
// exceeds it by more than this many binades, so probabilities are bounded by
// 2^kRescaleSlack and the O rescale is skipped for most tiles.
constexpr float kRescaleSlack = 8.0f;

// ---- the sign of the scale ---------------------------------------------------------------
// The forward kernels take the row maximum of the scaled scores by scaling the maximum of
// the raw ones, and mask keys with -inf before scaling. Both need a factor > 0. A negative
// scale is therefore applied as |scale| to Q with its sign bits flipped, and a zero scale
// as 1 to Q = 0: either way each score is exactly scale * (Q K^T) (a sign flip of 16-bit
// operands is exact, and the fp32 sums are symmetric under it), every masked key stays
// -inf, and the kernel's multiplier is positive.
struct QSign {
  float scale_log2;  // the factor the kernel uses, > 0
  uint32_t keep, flip;
  __device__ __forceinline__ u32x4_t apply(u32x4_t x) const {
    return (u32x4_t){(x[0] & keep) ^ flip, (x[1] & keep) ^ flip, (x[2] & keep) ^ flip, (x[3] & keep) ^ flip};
  }
};
__device__ __forceinline__ QSign q_sign(float scale_log2) {
  if (scale_log2 == 0.f) return QSign{1.f, 0u, 0u};
  if (scale_log2 < 0.f) return QSign{-scale_log2, ~0u, 0x80008000u};
  return QSign{scale_log2, ~0u, 0u};
}

// ---- dispatch order ------------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Map dispatch id i to a work id so that, within every run of 8*chunk dispatch
// ids, XCD x receives the `chunk` consecutive work ids x*chunk .. x*chunk+chunk-1
// (e.g. the query heads of one GQA group, which share K and V). Ids past the
// last full run map to themselves.
__device__ __forceinline__ int xcd_remap(int i, int n, int chunk) {
  const int run = 8 * chunk;
  if (chunk <= 1 || i >= (n / run) * run) return i;
  const int base = (i / run) * run, r = i - base;
  return base + (r & 7) * chunk + (r >> 3);
}

// ---- LDS -------------------------------------------------------------------------
#define SDPA_LDS(ptr) ((__attribute__((address_space(3))) void*)(ptr))

// Transposed read of 4 16-bit elements (see the header comment), as two dwords.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}
__device__ __forceinline__ u32x4_t lds_read16B(const uint16_t* p) { return *(const u32x4_t*)p; }
__device__ __forceinline__ void lds_write16B(uint16_t* p, u32x4_t v) { *(u32x4_t*)p = v; }

// ---- buffer resources (range-checked loads: offsets at or past `bytes` read as zero) ----
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family buffer descriptor flags (raw, 32-bit dwords)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
// 16 bytes at byte offset `off` into registers.
__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// Cache policy of a buffer load: kCacheDefault, or kCacheStream (non-temporal) for data
// read exactly once, which measured 7.1-7.3 TB/s against 5.9-6.1 TB/s for default loads
// in a pure read stream on MI355X.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;
// Buffer descriptor in scalar registers for the buffer-to-LDS loads: base address, no
// stride, `bytes` records (offsets past the end read as zero), same flags as make_rsrc.
// Every word goes through readfirstlane, so the descriptor is wave-uniform even where the
// compiler cannot prove the inputs uniform.
typedef u32x4_t srd_t;
__device__ __forceinline__ srd_t make_srd(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return (srd_t){(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), (uint32_t)kRsrcWord3};
}
// Direct buffer-to-LDS load of 16 bytes per lane: lane i writes lds_base + 16*i (M0 holds
// the wave-uniform LDS base).
//  - dma16: the compiler's intrinsic. The compiler tracks it as an LDS store and, before
//    the next LDS read, waits for every such load still in flight. Used by the tiled
//    kernels, which hand tiles between waves through barriers; there the early wait
//    measured faster (8% on the dK/dV kernel) than the untracked form.
//  - dma16_untracked: the same instruction as inline assembly, invisible to that
//    tracking, for a wave's private LDS ring: it waits for its own loads with
//    s_waitcnt vmcnt(n), so the next tile keeps streaming while this one is consumed.
template <int CPOL = kCacheDefault>
__device__ __forceinline__ void dma16(srd_t r, void* lds_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)r[1] << 32) | r[0]), (short)0, (int)r[2],
                                        kRsrcWord3),
      (__attribute__((address_space(3))) void*)lds_base, 16, (int)off, 0, 0, CPOL);
}
template <int CPOL = kCacheDefault>
__device__ __forceinline__ void dma16_untracked(srd_t r, void* lds_base, uint32_t off) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base);
  if constexpr (CPOL == kCacheStream)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(m0), "v"(off), "s"(r)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(off), "s"(r)
                 : "memory", "m0");
}
// Waits for every vector memory operation of the wave, buffer-to-LDS loads included.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Orders the LDS accesses of one wave: everything before completes and is visible to
// the wave's lanes before anything after it (a wave-scope fence around a wave barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
// Marks a loaded register as consumed here, so that the compiler waits for the load once,
// before a loop, instead of placing an s_waitcnt vmcnt(n) for it inside the loop, where
// the count would also cover tile loads in flight that it does not track.
__device__ __forceinline__ void settle(u32x4_t& x) { asm volatile("" : "+v"(x)); }
// Scheduling fence: the compiler moves no instruction across it.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// Compensated addition, sum += x, carrying each addition's rounding error in c (Kahan's
// summation, 1965): the error of a running sum stays a few ulps however many similar
// terms are added. Both sum and c are rescaled together when the sum is.
__device__ __forceinline__ void kahan_add(float& sum, float& c, float x) {
  const float y = x - c;
  const float t = sum + y;
  c = (t - sum) - y;
  sum = t;
}
// Wave index as a scalar (lets the compiler keep per-wave quantities uniform).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// ---- swizzled LDS tiles ---------------------------------------------------------------
// A tile of rows of D 16-bit elements, rows stored back to back (no padding); the 16-byte
// chunk c of row r is stored at chunk position c ^ f(r), f(r) < D/8. The LDS has 64
// four-byte banks (256 bytes per clock). Measured on gfx950 (a lane pair that reads one
// bank only costs a cycle when both lanes sit in the same phase), ds_read_b128 serves a
// wave in four phases of 16 lanes, {0-3, 12-15, 20-27}, {4-11, 16-19, 28-31} and the same
// two sets plus 32, and ds_read_b64_tr_b16 in two phases, lanes 0-31 and 32-63; f makes
// the 16 (b128) or 32 (tr) lanes of every phase touch 64 distinct banks. Two read
// geometries are supported (M = the matrix-core tile edge the kernel uses):
//  M = 32 (32x32x16 tiles): lane l reads chunk 2c + l/32 of row l%32, and transposed
//    reads of an aligned group of 4 chunks in 4 consecutive rows;
//  M = 16 (16x16x32 tiles): lane l reads chunk 4c + l/16 of row l%16, and transposed
//    reads of an aligned pair of chunks in 8 consecutive rows.
template <int D, int M = 32>
struct SwzTile {
  static constexpr int RB = D * 2;   // row bytes
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  __device__ __forceinline__ static int f(int r) {
    if (M == 32) {
      if (CPR >= 16) return 4 * (r & 3) + ((r >> 2) & 3);      // 256-byte rows: one row per bank window
      if (CPR == 8) return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);  // 128-byte rows: two rows per window
      return (r >> 2) & 3;  // 64-byte rows: four rows per window; also 192-byte rows (D = 96)
    }
    if (CPR >= 16) return 2 * (r & 7);
    if (CPR == 8) return 2 * ((r >> 1) & 3);
    return 2 * ((r >> 2) & 1);  // 64- and 192-byte rows
  }
  __device__ __forceinline__ static int off(int r, int c) { return r * RB + ((c ^ f(r)) << 4); }
  // LDS DMA of rows [g0, g0 + ROWS) of a range-checked row-major [rows, D] resource
  // (rows past its end arrive as zeros). The `waves` waves of the workgroup split the
  // 1 KiB slices; `w` is this wave.
  template <int ROWS, int CPOL = kCacheDefault, bool TRACKED = true>
  __device__ __forceinline__ static void dma_fill(srd_t src, uint8_t* lds, int g0, int w, int waves, int lane) {
    constexpr int SLICES = ROWS * CPR / 64;
    static_assert(ROWS * CPR % 64 == 0, "tile must be a whole number of 1 KiB slices");
    for (int j = w; j < SLICES; j += waves) {
      const int pc_lin = 64 * j + lane;
      const int r = pc_lin / CPR, pc = pc_lin % CPR;
      const uint32_t off = (uint32_t)(((g0 + r) * D + (pc ^ f(r)) * 8) * 2);
      if constexpr (TRACKED)
        dma16<CPOL>(src, lds + 1024 * j, off);
      else
        dma16_untracked<CPOL>(src, lds + 1024 * j, off);
    }
  }
  // The same copy for a kernel that fills many tiles: wave w of WAVES computes the
  // source offsets of its slices once (they do not depend on the tile's first row), and
  // each tile's first row goes into the buffer resource instead (srd_rows), so a tile
  // costs no vector ALU work; rows past the tensor's end still arrive as zeros.
  template <int ROWS, int WAVES>
  struct DmaPlan {
    static constexpr int SLICES = ROWS * CPR / 64;
    static constexpr int NS = (SLICES + WAVES - 1) / WAVES;  // slices of one wave (at most)
    static_assert(ROWS * CPR % 64 == 0, "tile must be a whole number of 1 KiB slices");
    uint32_t off[NS];
    __device__ __forceinline__ DmaPlan(int w, int lane) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int pc_lin = 64 * (w + s * WAVES) + lane;
        const int r = pc_lin / CPR, pc = pc_lin % CPR;
        off[s] = (uint32_t)((r * D + (pc ^ f(r)) * 8) * 2);
      }
    }
    template <int CPOL = kCacheDefault, bool TRACKED = true>
    __device__ __forceinline__ void fill(srd_t src, uint8_t* lds, int w) const {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int j = w + s * WAVES;
        if (SLICES % WAVES != 0 && j >= SLICES) break;
        if constexpr (TRACKED)
          dma16<CPOL>(src, lds + 1024 * j, off[s]);
        else
          dma16_untracked<CPOL>(src, lds + 1024 * j, off[s]);
      }
    }
  };
};

// Buffer resource of rows [g0, rows) of a row-major [rows, D] 16-bit tensor at `base`
// (no records when g0 >= rows): a tile's copy with DmaPlan addresses its rows from here.
template <int D>
__device__ __forceinline__ srd_t srd_rows(const uint16_t* base, int rows, int g0) {
  return make_srd(base + (int64_t)g0 * D, (uint32_t)max(0, rows - g0) * (uint32_t)(D * 2));
}

// ---- global ------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t gload16B(const void* p) { return *(const u32x4_t*)p; }
__device__ __forceinline__ void gstore16B(void* p, u32x4_t v) { *(u32x4_t*)p = v; }
__device__ __forceinline__ void gstore8B(void* p, u32x2_t v) { *(u32x2_t*)p = v; }

// Store 4 consecutive fp32 results as OutT (16-bit tag types or float).
template <typename OutT> struct Store4;
template <> struct Store4<float> {
  __device__ __forceinline__ static void run(float* p, float a, float b, float c, float d) {
    *(f32x4_t*)p = (f32x4_t){a, b, c, d};
  }
};
template <> struct Store4<bf16_t> {
  __device__ __forceinline__ static void run(bf16_t* p, float a, float b, float c, float d) {
    gstore8B(p, (u32x2_t){pack2<bf16_t>(a, b), pack2<bf16_t>(c, d)});
  }
};
template <> struct Store4<f16_t> {
  __device__ __forceinline__ static void run(f16_t* p, float a, float b, float c, float d) {
    gstore8B(p, (u32x2_t){pack2<f16_t>(a, b), pack2<f16_t>(c, d)});
  }
};

// Load one element of an output-typed array as fp32.
__device__ __forceinline__ float load_f32(const float* p) { return *p; }

// The mask's additive bias in log2 units for element `off`: 0 or -inf for a boolean mask,
// value * log2(e) for an additive one (operand type T: a 16-bit tag type or float).
template <typename T>
__device__ __forceinline__ float mask_bias_log2(const void* p, int kind, int64_t off) {
  if (kind == 1) return ((const uint8_t*)p)[off] ? 0.f : -INFINITY;
  if constexpr (sizeof(T) == 4)
    return ((const float*)p)[off] * kLog2e;
  else
    return to_f32<T>(((const uint16_t*)p)[off]) * kLog2e;
}
// The same for the 4 consecutive keys at element offset `off`, with one aligned load
// (off a multiple of 4, and the mask's vec4 property). 16-bit operand types only.
template <typename T>
__device__ __forceinline__ void mask_bias4_log2(const void* p, int kind, int64_t off, float* b) {
  if (kind == 1) {
    const uint32_t w = *(const uint32_t*)((const uint8_t*)p + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = ((w >> (8 * j)) & 0xffu) ? 0.f : -INFINITY;
  } else {
    const u32x2_t w = *(const u32x2_t*)((const uint16_t*)p + off);
    b[0] = lo_f32<T>(w[0]) * kLog2e;
    b[1] = hi_f32<T>(w[0]) * kLog2e;
    b[2] = lo_f32<T>(w[1]) * kLog2e;
    b[3] = hi_f32<T>(w[1]) * kLog2e;
  }
}
// The biases of 4 boolean mask bytes held in one word (byte j: key j), in log2 units.
__device__ __forceinline__ void mask_bias4_bool_word(uint32_t w, float* b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = ((w >> (8 * j)) & 0xffu) ? 0.f : -INFINITY;
}
__device__ __forceinline__ float load_f32(const bf16_t* p) { return to_f32<bf16_t>(p->bits); }

__device__ __forceinline__ float load_f32(const f16_t* p) { return to_f32<f16_t>(p->bits); }

}  // namespace sdpa
