/*
 * sdpa.h — fused scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libsdpa_mi355x.so. The library computes
 *
 *     O = softmax((Q K^T) * scale [+ causal mask]) V
 *
 * and its gradients, with grouped-query attention (GQA). The forward is the
 * definition in the PyTensor issue "PERF: detect scaled-dot-product-attention
 * pattern and lower to mx.fast.scaled_dot_product_attention" (section "Sketch":
 * scores (Q K^T) * scale, row-max subtraction, exponentials normalised by their
 * row sum, times V); causal masking and the [B, H, S, D] layout follow
 * mps-flash-sdpa 0.1.0 ("Quick Start"); GQA, causal masking, the logsumexp that
 * the forward caches and the backward consumes, and the two-kernel backward
 * without atomics follow the MLX pull request "[Metal] Add Flash Attention VJP
 * for training" ("Implementation Notes", "Key Features", "Limitations").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout      Row-major "BHLD", head dimension innermost, fully contiguous:
 *               q, o, dO, dq : [B, Hq,  Lq,  D]
 *               k, v, dk, dv : [B, Hkv, Lkv, D]
 *               lse          : [B, Hq,  Lq]   float32, natural log
 *             Query head h reads key/value head h / (Hq / Hkv).
 * Masking     is_causal != 0 keeps key j for query i iff j <= i + (Lkv - Lq): the
 *             query and key sequences are aligned at their ends, so the last query
 *             sees every key (new queries against a key/value cache); with Lq == Lkv
 *             this is j <= i. It requires Lq <= Lkv, so that every query row sees a
 *             key. The pages list unequal query and key lengths only as a test edge
 *             case (MLX pull request, "Test Plan"); the end alignment is this
 *             library's reading. Boolean and additive masks and attention sinks
 *             are taken by sdpa_fwd_masked / sdpa_bwd_masked below. No dropout.
 * Precision   dtype is the operand type of q, k, v, dO (SDPA_F32, SDPA_F16 or
 *             SDPA_BF16). Products accumulate in float32. out_dtype is the type
 *             of o, dq, dk, dv and must be dtype or SDPA_F32 (with SDPA_F32
 *             operands it must be SDPA_F32).
 * Pointers    Device memory owned by the caller. Every tensor base must be
 *             16-byte aligned. Outputs must not alias inputs or each other.
 *             The library never allocates, frees, retains a pointer after the
 *             call returns, or synchronises; work is enqueued on `stream`
 *             (a hipStream_t; NULL means the default stream). It enqueues kernel
 *             launches only (no memory sets or copies), so the calls can be
 *             captured in a HIP graph and replayed.
 * Workspace   Caller-owned device scratch of at least sdpa_workspace_bytes(...)
 *             bytes (may be NULL when that is 0), 256-byte aligned. Its contents
 *             on entry do not matter. Calls that share a workspace must be
 *             ordered on one stream.
 * Errors      Arguments are validated before anything is enqueued. A failed
 *             validation returns a non-zero status and touches no memory. A
 *             launch failure returns SDPA_ERR_DEVICE. Faults inside a kernel
 *             surface at the caller's next synchronisation, as for any stream
 *             operation. All outputs are fully overwritten (dk and dv are not
 *             accumulated into).
 * Scale       Any finite value, including 0 (every visible key weighs the same) and
 *             negative values; a non-finite scale is SDPA_ERR_VALUE.
 * Threads     No mutable global state (except the fixed scratch of
 *             sdpa_bwd_noalloc, below); calls are thread-safe.
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SDPA_F32 = 0, SDPA_F16 = 1, SDPA_BF16 = 2 } sdpa_dtype_t;

typedef enum {
  SDPA_OK = 0,
  SDPA_ERR_NULL = 1,        /* a required pointer is NULL                              */
  SDPA_ERR_SHAPE = 2,       /* a size < 1, Hq % Hkv != 0, counts overflow, or one head's
                               (L + 256) * D elements exceed 2 GiB                     */
  SDPA_ERR_UNSUPPORTED = 3, /* D not in {32,64,96,128,256}, causal with Lq > Lkv or with a
                               mask, bad dtype                                          */
  SDPA_ERR_WORKSPACE = 4,   /* workspace smaller than sdpa_workspace_bytes()            */
  SDPA_ERR_ALIGN = 5,       /* a base pointer is not 16-byte (workspace: 256) aligned   */
  SDPA_ERR_DEVICE = 6,      /* the HIP runtime rejected a launch                        */
  SDPA_ERR_VALUE = 7        /* scale not finite, invalid stage number or mask kind      */
} sdpa_status_t;

/* Kernel families, as returned by sdpa_select_path(). */
enum {
  SDPA_PATH_TILED = 0,  /* 16-bit operands, otherwise: MFMA tiles, online softmax         */
  SDPA_PATH_VECTOR = 1, /* 16-bit, Lq <= 8 and (Hq/Hkv)*Lq <= 32: one pass over split keys */
  SDPA_PATH_FP32 = 2    /* float32 operands                                               */
};

/*
 * Which kernel family a call with these sizes runs (a pure host function).
 * The short-query cutoff is the MLX pull request's vector VJP condition
 * (L <= 8, "Implementation Notes"), read as the query length (causal or not), and
 * limited to groups whose (Hq / Hkv) * Lq query rows fit one 32-row matrix block.
 * Returns one of SDPA_PATH_*, or -1 if the combination is unsupported.
 */
int sdpa_select_path(int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, int is_causal, sdpa_dtype_t dtype);

/*
 * Bytes of workspace sdpa_fwd (backward = 0) or sdpa_bwd (backward = 1) needs
 * for these sizes; 0 if none. Pure host function. The workspace is caller-owned
 * device memory that the library uses in place and never allocates itself, as the
 * pages' kernels take the caller's tensors' buffers directly (mps-flash-sdpa 0.1.0,
 * "How It Works": zero-copy buffer handoff to the kernels). Returns (size_t)-1 when the
 * sizes are invalid. The forward needs one on the short-query path, and on the
 * tiled path when its grid of (query block, head) pairs is too small to give every
 * compute unit a workgroup (two at D = 256): there the keys are split over several
 * workgroups whose fp32 partials (unnormalised O, running max, row sum) the
 * workspace holds until a second kernel merges them. The backward always needs one
 * (per-row statistics that its first stage leaves for the second); on small grids
 * it also holds the fp32 partials of dQ, dK and dV of split kernels, which a
 * reduction sums in a fixed order.
 */
size_t sdpa_workspace_bytes(int backward, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv,
                            int64_t D, int is_causal, sdpa_dtype_t dtype);

/*
 * Forward: o = softmax((q k^T) * scale [+ causal]) v, and, when lse != NULL,
 * lse[b, h, i] = log(sum_j exp(scale * q_i . k_j)) over the unmasked keys
 * (the "second output" that the backward needs: MPS SDPA issue, section
 * "Problem - Unused second output tensor"; pass NULL when no backward follows
 * and it is not computed).
 *
 *   q, k, v    inputs in dtype (layouts above)
 *   o          output in out_dtype, [B, Hq, Lq, D]
 *   lse        optional output, float32 [B, Hq, Lq]
 *   scale      multiplies the scores before the softmax (usually 1/sqrt(D))
 */
sdpa_status_t sdpa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal,
                       sdpa_dtype_t dtype, sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Backward of sdpa_fwd for the upstream gradient dO: writes dq, dk, dv (the
 * gradients of sum(O * dO) with respect to q, k, v). `o` and `lse` must be
 * exactly what sdpa_fwd wrote for the same q, k, v, scale and is_causal; lse is
 * required (the MLX pull request, "Limitations": the VJP needs the forward's
 * logsumexp). dk and dv sum the contributions of all query heads of a group.
 *
 *   q, k, v, dO   inputs in dtype;  o in out_dtype;  lse float32
 *   dq, dk, dv    outputs in out_dtype
 */
sdpa_status_t sdpa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                       void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv,
                       int64_t D, float scale, int is_causal, sdpa_dtype_t dtype, sdpa_dtype_t out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward as two stream-ordered stages; sdpa_bwd(...) is stage 0 followed
 * by stage 1 with the same arguments. Stage 1 must be enqueued after stage 0 on
 * the same stream with the same workspace, which carries state between them.
 *   tiled and fp32 paths: stage 0 writes dq (and Delta_i = sum_d dO_id O_id
 *                         into the workspace); stage 1 writes dk and dv.
 *   vector path:          stage 0 writes dk, dv and per-split dq partials (in
 *                         the workspace); stage 1 reduces them into dq.
 * Arguments, validation and errors are those of sdpa_bwd; `stage` must be 0 or 1
 * (else SDPA_ERR_VALUE). Useful to time or schedule the two halves separately.
 */
sdpa_status_t sdpa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                             int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal, sdpa_dtype_t dtype,
                             sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention masks and sinks
 * -------------------------
 * The pages name float masks, boolean masks with False entries and attention sinks
 * only as cases that fused paths hand back to unfused attention (mps-flash-sdpa
 * 0.1.0, "When MFA Dispatches vs. Falls Back"; MLX pull request, "Limitations"), and
 * place a mask as a term added to the scaled scores before the softmax (PyTensor
 * issue, "Important guards in the matcher"). This library reads them as PyTorch's
 * scaled_dot_product_attention does:
 *
 *   s_ij  = scale * q_i . k_j + bias_ij       (bias_ij = 0 / -inf for a boolean mask)
 *   LSE_i = log(exp(sink_h) + sum_j exp(s_ij))  (no sink term when sinks is NULL)
 *   o_i   = sum_j exp(s_ij - LSE_i) v_j
 *
 *   mask_kind   SDPA_MASK_NONE: no mask (mask and its strides are ignored);
 *               SDPA_MASK_BOOL: uint8 elements, nonzero = the key takes part;
 *               SDPA_MASK_ADDITIVE: elements of `dtype` added to the scaled scores
 *               (finite or -inf; +inf and NaN are not allowed and not checked).
 *   mask        device memory; element (b, h, i, j) of query head h is
 *                 mask[b * mask_stride_b + h * mask_stride_h + i * mask_stride_q + j]
 *               (strides in elements, >= 0; 0 broadcasts that dimension; keys are
 *               contiguous). Additive masks are aligned to their element size.
 *   sinks       NULL, or float32 [Hq] on the device: one logit per query head in the
 *               units of the scaled scores; -inf means no sink for that head.
 *
 * A mask cannot be combined with is_causal != 0 (SDPA_ERR_UNSUPPORTED). A row that
 * sees no key and has no sink gets o = 0 and lse = -inf, and contributes no gradient.
 * The mask is a constant: no gradient is formed for it.
 */
typedef enum { SDPA_MASK_NONE = 0, SDPA_MASK_BOOL = 1, SDPA_MASK_ADDITIVE = 2 } sdpa_mask_kind_t;

/*
 * sdpa_fwd with a mask and/or sinks (definitions above). Other arguments, the
 * workspace (sdpa_workspace_bytes with the same sizes) and errors as for sdpa_fwd;
 * additionally SDPA_ERR_VALUE for an unknown mask_kind, SDPA_ERR_NULL for a missing
 * mask, SDPA_ERR_SHAPE for a negative stride or an element offset that overflows, and
 * SDPA_ERR_ALIGN for a misaligned additive mask.
 */
sdpa_status_t sdpa_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                              int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal,
                              sdpa_mask_kind_t mask_kind, const void* mask, int64_t mask_stride_b,
                              int64_t mask_stride_h, int64_t mask_stride_q, const float* sinks, sdpa_dtype_t dtype,
                              sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_bwd with a mask and/or sinks: `o` and `lse` must be what sdpa_fwd_masked wrote
 * with the same mask and sinks. With sinks != NULL, dsinks (float32 [Hq], device,
 * required then) receives the gradient of sum(O * dO) with respect to the sinks,
 *   dsinks[h] = -sum_{b,i} exp(sinks[h] - lse[b,h,i]) * sum_d dO[b,h,i,d] o[b,h,i,d],
 * summed in a fixed order (deterministic). Other arguments and errors as for sdpa_bwd
 * and sdpa_fwd_masked.
 */
sdpa_status_t sdpa_bwd_masked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                              int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal,
                              sdpa_mask_kind_t mask_kind, const void* mask, int64_t mask_stride_b,
                              int64_t mask_stride_h, int64_t mask_stride_q, const float* sinks, float* dsinks,
                              sdpa_dtype_t dtype, sdpa_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * sdpa_bwd_masked as two stream-ordered stages, as sdpa_bwd_stage is for sdpa_bwd (same
 * stage contents; dsinks is written by stage 1, from what stage 0 left in the workspace).
 * `stage` must be 0 or 1 (else SDPA_ERR_VALUE).
 */
sdpa_status_t sdpa_bwd_masked_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dO, void* dq, void* dk, void* dv, int64_t B,
                                    int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lkv, int64_t D, float scale,
                                    int is_causal, sdpa_mask_kind_t mask_kind, const void* mask,
                                    int64_t mask_stride_b, int64_t mask_stride_h, int64_t mask_stride_q,
                                    const float* sinks, float* dsinks, sdpa_dtype_t dtype, sdpa_dtype_t out_dtype,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code being captured into a HIP graph, serving loops that must not call
 * hipMalloc, harnesses that forbid it). The scratch that sdpa_bwd keeps in the
 * caller's workspace lives instead in a fixed array of SDPA_NOALLOC_SCRATCH_BYTES
 * (64 MiB) inside the library, one per GPU, held until the process ends. The call
 * allocates and frees nothing. Arguments, results and errors are those of sdpa_bwd,
 * plus SDPA_ERR_WORKSPACE when sdpa_workspace_bytes(1, ...) for these sizes exceeds
 * the array (the bf16 GQA shape B=4, Hq=32, Hkv=4, L=4096, D=128 needs 4 MiB), and
 * SDPA_ERR_DEVICE when the array's address cannot be obtained on the current device.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents
 * (nothing in it needs to start at zero): calls on one GPU that may overlap, on
 * different streams or from different threads, race on it and must be ordered by the
 * caller.
 */
#define SDPA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
sdpa_status_t sdpa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dO, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                               int64_t Lq, int64_t Lkv, int64_t D, float scale, int is_causal, sdpa_dtype_t dtype,
                               sdpa_dtype_t out_dtype, void* stream);

/* Static string naming a status code. Never NULL. */
const char* sdpa_status_str(sdpa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H */
