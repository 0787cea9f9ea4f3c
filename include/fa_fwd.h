/*
 * fa_fwd.h -- C ABI of the MI355X (gfx950) FlashAttention forward library.
 *
 * Operation.  For every batch b and head h, with S = scale * Q K^T (N x N):
 *
 *     O   = softmax(S) V                      (row-wise softmax)
 *     lse = log(sum_j exp(S_ij))              (natural log, per query row i)
 *
 * optionally under the causal mask (query i sees key j iff j <= i).  This is
 * the attention formula of the systems-analysis.info page "FlashAttention (PL)",
 * section "Problematyka standardowego mechanizmu uwagi", and of the
 * chipfoundryservices glossary entry "Flash Attention", "Standard attention"
 * paragraph; ``scale`` is the 1/sqrt(d_k) factor.  The causal mask is the
 * optional mask of the robocikowo.com "Flash Attention" page, and lse is the
 * per-row logsumexp L that page says the backward pass recomputes from.
 * The computation is tiled with an online softmax (glossary, "Tiling
 * Algorithm" steps 1-6): the N x N score matrix never leaves the chip and the
 * library needs no memory besides its arguments.
 *
 * Layout.  q, k, v and o are dense row-major [B][H][N][d] arrays (d fastest,
 * no padding); lse is a dense [B][H][N] float array.  N is both the query and
 * the key length.
 *
 * Memory and streams.  Every pointer is a device pointer owned by the caller;
 * the library never allocates, frees or synchronises.  The one thing it keeps
 * between calls is a per-device, per-kernel cache of two read-only launch
 * facts (how many workgroups of the kernel fit on the device at once, and the
 * compute units per XCD), filled by the first call on a device.  It decides
 * only the order in which workgroups are dealt to compute units, never a
 * result, and it is written with atomic stores, so all entry points are
 * re-entrant and thread-safe.  ``stream`` is a hipStream_t
 * (NULL = the default stream); the work is enqueued on it and the call
 * returns without waiting.  o and lse must not overlap q, k, v or each other.
 * Results are bitwise reproducible for equal inputs, shape and device.
 *
 * Errors.  Arguments are checked before anything is launched; on a failed
 * check nothing is enqueued and the status says why.  A failure reported by
 * the HIP runtime at launch returns FA_ERR_HIP.  Faults that happen while the
 * kernel runs surface at the caller's next synchronisation, as with any HIP
 * kernel.  Inputs are assumed finite.
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* B, H or N < 1, H_kv < 1 or not dividing H, or an element count overflows int64/int32 indexing */
  FA_ERR_UNSUPPORTED = 3, /* d not in {64, 128, 256}, or unknown dtype */
  FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  FA_ERR_SCALE = 5,       /* scale not finite, or an fp8 descale not finite and > 0 */
  FA_ERR_HIP = 6,         /* the HIP runtime rejected the launch */
  FA_ERR_SCRATCH = 7      /* fa_fwd_split_noalloc: the call needs more than the library's fixed scratch */
} fa_status;

typedef enum {
  FA_F32 = 0,       /* q, k, v, o are float32 (products use a three-term bf16 split) */
  FA_BF16 = 1,      /* q, k, v, o are bfloat16 */
  FA_FP8_E4M3 = 2   /* q, k, v are OCP e4m3fn bytes with unit descales; o is bfloat16 */
} fa_dtype;

/*
 * fa_fwd -- exact attention forward, O and lse as described above.
 *   q, k, v : inputs, element type given by dtype, [B][H][N][d]
 *   o       : output, same element type as the inputs (bfloat16 for FA_FP8_E4M3)
 *   lse     : output, float32 [B][H][N]
 *   scale   : any finite value multiplying Q K^T (usually 1/sqrt(d))
 *   causal  : 0 = no mask, nonzero = query i sees keys j <= i
 *   dtype   : a fa_dtype value
 *   stream  : hipStream_t to enqueue on
 * FA_FP8_E4M3 here is fa_fwd_fp8 with all three descales equal to 1.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t N, int64_t d,
                 float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_fp8 -- the same operation on FP8 inputs with per-tensor scales
 * (the FP8 forward the pages attribute to FlashAttention-3: systems-analysis
 * page section "FlashAttention-3 (2024)", glossary "Flash Attention 3
 * (Hopper)" paragraph, dexblog.ro table row on data types).
 *   q8, k8, v8 : OCP e4m3fn bytes [B][H][N][d]; the value of an element is
 *                e4m3(x8) * x_descale
 *   o_bf16     : bfloat16 output [B][H][N][d]
 *   lse        : float32 [B][H][N], natural-log logsumexp of the scaled,
 *                dequantised scores
 *   *_descale  : finite and > 0, else FA_ERR_SCALE
 * Softmax statistics and both products accumulate in float32.  The softmax
 * probabilities, taken against an exponent base that may trail the row
 * maximum by up to 2 (log2 units), so at most 2^2, are pre-scaled by 2^6 (at
 * most 256 then) and rounded to e4m3 for the P V product; the row sum uses
 * them unrounded, so the factor cancels in O / l, and L removes it.
 */
fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     float q_descale, float k_descale, float v_descale,
                     int causal, void* stream);

/*
 * fa_fwd_gqa -- grouped-query attention: the H query heads are split into
 * H_kv consecutive groups of G = H / H_kv heads and every query head h of
 * group h / G attends over K/V head h / G (multi-query attention is
 * H_kv = 1; H_kv = H is fa_fwd).  Otherwise the same operation, arguments,
 * errors and guarantees as fa_fwd.  The pages name Multi-Query Attention
 * among the architectures FlashAttention-2 extended its support to
 * (systems-analysis.info "FlashAttention (PL)", section "FlashAttention-2
 * (2023)"); grouped-query attention is read as its general case.
 *   q, o   : [B][H][N][d]
 *   k, v   : [B][H_kv][N][d]
 *   lse    : float32 [B][H][N]
 *   H_kv   : >= 1 and dividing H, else FA_ERR_SHAPE
 */
fa_status fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                     float scale, int causal, int dtype, void* stream);

/* fa_fwd_gqa on FP8 inputs with per-tensor descales, as fa_fwd_fp8. */
fa_status fa_fwd_gqa_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse,
                         int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d, float scale,
                         float q_descale, float k_descale, float v_descale,
                         int causal, void* stream);

/*
 * fa_fwd_alibi -- fa_fwd with ALiBi linear biases: the score of query i and
 * key j of head h is scale * q_i . k_j - slopes[h] * |i - j| (under the
 * causal mask, -slopes[h] * (i - j)).  The robocikowo.com "Flash Attention"
 * page says such masks need kernel variants; the bias form is the usual
 * ALiBi one.
 *   slopes : device float32 [H], finite, 4-byte aligned (FA_ERR_ALIGN), not NULL
 * Every dtype and head dim of fa_fwd except FA_F32 at d = 256
 * (FA_ERR_UNSUPPORTED).  Otherwise as fa_fwd.
 */
fa_status fa_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse, const float* slopes,
                       int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype,
                       void* stream);

/*
 * fa_fwd_alibi on FP8 inputs with per-tensor descales, as fa_fwd_fp8: the
 * score is scale * q_descale * k_descale * q8_i . k8_j - slopes[h] * |i - j|.
 */
fa_status fa_fwd_alibi_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse,
                           const float* slopes, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                           float q_descale, float k_descale, float v_descale, int causal, void* stream);

/*
 * fa_fwd_blocksparse -- fa_fwd restricted to the allowed blocks of a block
 * mask: the scores of query block I and key block J (128 x 128 elements,
 * the last blocks ragged) are computed only if
 *     block_mask[b * mask_stride_b + h * mask_stride_h + I * nb + J] != 0,
 * nb = ceil(N / 128), and are -inf otherwise; the causal mask applies on top.
 * Disallowed blocks are never loaded.  A row with no allowed key gets O = 0
 * and lse = -inf.  (The pages name block-sparse patterns among the masks that
 * need kernel variants, and FlashMask in their literature.)
 *   block_mask    : device bytes, nb x nb per (batch, head), not NULL
 *   mask_stride_b : bytes between batches' masks (0: one mask for all batches), >= 0
 *   mask_stride_h : bytes between heads' masks (0: one mask for all heads), >= 0
 * Every dtype and head dim of fa_fwd except FA_F32 at d = 256
 * (FA_ERR_UNSUPPORTED).  Otherwise as fa_fwd.
 */
fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                             const uint8_t* block_mask, int64_t mask_stride_b, int64_t mask_stride_h,
                             int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype,
                             void* stream);

/* fa_fwd_blocksparse on FP8 inputs with per-tensor descales, as fa_fwd_fp8. */
fa_status fa_fwd_blocksparse_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse,
                                 const uint8_t* block_mask, int64_t mask_stride_b, int64_t mask_stride_h,
                                 int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                 float q_descale, float k_descale, float v_descale, int causal, void* stream);

/*
 * fa_plan -- the launch fa_fwd / fa_fwd_fp8 (and their grouped-query
 * forms, whose grid does not depend on H_kv) would make for this problem,
 * without launching anything.  Any output pointer may be NULL.
 *   block_rows / block_cols : queries per workgroup (B_r) and keys per K/V tile (B_c)
 *   workgroups, threads     : grid size and threads per workgroup
 *   lds_bytes               : LDS per workgroup
 *   kv_tiles                : total K/V tiles the grid streams (fully masked causal tiles excluded)
 * Returns the status fa_fwd would return for the same shape/dtype checks.
 */
fa_status fa_plan(int64_t B, int64_t H, int64_t N, int64_t d, int causal, int dtype,
                  int* block_rows, int* block_cols, int64_t* workgroups, int* threads,
                  int* lds_bytes, int64_t* kv_tiles);

/* Human-readable name of a status code (static string; never NULL). */
const char* fa_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int fa_version(void);

/*
 * Diagnostic timeline of the last forward launch through fa_fwd, fa_fwd_fp8,
 * fa_fwd_gqa or fa_fwd_gqa_fp8 on the current device (a measurement aid, not
 * part of the attention computation).  Only a library built with
 * -DFA_TIMELINE (python -m exact_io_aware_48_amd.build --timeline, a separate
 * file) records it; any other build returns FA_ERR_UNSUPPORTED and touches
 * nothing.  Per workgroup id w, six 64-bit words at dst[6w .. 6w+5]: the
 * 100 MHz s_memrealtime stamps at entry, after its Q and first K/V tiles,
 * after the main loop, and after the O store, then (XCC_ID << 32 | HW_ID) and
 * (row block << 32 | batch*head).  bytes: how much to copy (at most 2 MiB);
 * dst is host memory owned by the caller.  Synchronous with the device.
 * FA_ERR_NULL for a NULL dst, FA_ERR_SHAPE for a size out of range.
 */
fa_status fa_timeline_read(void* dst, int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
