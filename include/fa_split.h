/*
 * fa_split.h -- C ABI of split-KV (decode-shaped) attention and the
 * logsumexp merge of attention partials, for MI355X (gfx950).
 *
 * Operation.  N_q queries that are the last N_q positions of a sequence of
 * N_k >= N_q keys: for batch b and query head h (K/V head h / (H / H_kv)),
 *
 *     O   = softmax(S) V,   lse = log(sum_j exp(S_ij)),   S = scale * Q K^T,
 *
 * where under the causal mask query i (0-based among the N_q) sees keys
 * j <= N_k - N_q + i (N_q = N_k is the square mask of fa_fwd).  The key
 * range is split over workgroups; each split writes a partial (O_s
 * normalised over its keys, L_s its logsumexp) and a merge forms
 *
 *     L = log(sum_s exp(L_s)),   O = sum_s exp(L_s - L) O_s,
 *
 * which is the exact softmax over all keys.  The pages name sequence
 * parallelism among FlashAttention-2's changes (systems-analysis.info
 * "FlashAttention (PL)", section "FlashAttention-2 (2023)") and cite decoding
 * work (FlashDecoding++) in its literature list; they give no formula, so
 * this is the attention definition of fa_fwd.h over the keys each query sees.
 *
 * Layout.  q, o: dense [B][H][N_q][d]; k, v: [B][H_kv][N_k][d]; lse:
 * float32 [B][H][N_q].  Memory, streams, re-entrancy and errors as in
 * fa_fwd.h.  The result depends on the number of splits only through
 * rounding; for a fixed split count it is bitwise reproducible.
 */
#ifndef FA_SPLIT_H
#define FA_SPLIT_H

#include <stdint.h>

#include "fa_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_fwd_split_plan -- the split count fa_fwd_split (dtype FA_BF16) or
 * fa_fwd_split_fp8 (dtype FA_FP8_E4M3) would use and the workspace it needs
 * (splits * B * H * N_q * (d + 1) * 4 bytes), without launching anything.
 * num_splits = 0 lets the library choose (about two workgroups per compute
 * unit of the current device, at least four key tiles per split: 32 keys at
 * d = 128 and 256 in bf16, else 64); a positive value asks for that many
 * splits, fewer when the key tiles run out.  splits and workspace_bytes may
 * be NULL.  Checks as fa_fwd_split (FA_ERR_SHAPE also for num_splits < 0;
 * FA_ERR_UNSUPPORTED for a dtype other than those two).
 */
fa_status fa_fwd_split_plan(int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d,
                            int num_splits, int dtype, int* splits, int64_t* workspace_bytes);

/*
 * fa_fwd_split -- O and lse as above, by split-KV partials and their merge
 * (two launches).
 *   q          : bfloat16 [B][H][N_q][d]
 *   k, v       : bfloat16 [B][H_kv][N_k][d]
 *   o          : bfloat16 output [B][H][N_q][d]
 *   lse        : float32 output [B][H][N_q]
 *   workspace  : device memory of the size fa_fwd_split_plan reports for the
 *                same arguments; holds the partials (fp32 O_s, then L_s)
 *   N_q, N_k   : 1 <= N_q <= N_k, else FA_ERR_SHAPE
 *   d          : 64, 128 or 256; dtype must be FA_BF16 (else FA_ERR_UNSUPPORTED)
 *   scale      : any finite value; causal as described above
 *   num_splits : as for fa_fwd_split_plan
 * Every pointer must be 16-byte aligned.
 */
fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                       int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d,
                       float scale, int causal, int num_splits, int dtype, void* stream);

/*
 * fa_fwd_split_fp8 -- fa_fwd_split on FP8 inputs with per-tensor scales, as
 * fa_fwd_fp8 is the forward on them (the FP8 forward the pages attribute to
 * FlashAttention-3: systems-analysis page section "FlashAttention-3 (2024)",
 * glossary "Flash Attention 3 (Hopper)" paragraph, dexblog.ro table row on
 * data types); for decoding this is an fp8 K/V cache, half the bytes of the
 * bf16 stream the split pass is bound by.
 *   q8         : OCP e4m3fn bytes [B][H][N_q][d]
 *   k8, v8     : OCP e4m3fn bytes [B][H_kv][N_k][d]; the value of an element
 *                is e4m3(x8) * x_descale
 *   o_bf16     : bfloat16 output [B][H][N_q][d]
 *   lse        : float32 output [B][H][N_q], natural-log logsumexp of the
 *                scaled, dequantised scores
 *   workspace  : the size fa_fwd_split_plan reports with dtype FA_FP8_E4M3
 *   *_descale  : finite and > 0, else FA_ERR_SCALE
 * Shapes, splits, the causal rule and the other errors as fa_fwd_split.
 * Products and softmax statistics accumulate in float32, and the
 * probabilities enter the P V product as in fa_fwd_fp8 (pre-scaled by 2^6,
 * rounded to e4m3; the row sums use them unrounded).
 */
fa_status fa_fwd_split_fp8(const void* q8, const void* k8, const void* v8, void* o_bf16, float* lse, void* workspace,
                           int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, float scale,
                           float q_descale, float k_descale, float v_descale, int causal, int num_splits,
                           void* stream);

/*
 * fa_fwd_split_noalloc -- fa_fwd_split without a workspace argument, for
 * callers that cannot allocate device memory (code being captured into a HIP
 * graph, serving loops that must not call the allocator, harnesses that forbid
 * it).  The partials go to a fixed array inside the library instead:
 * fa_split_scratch_bytes() bytes (32 MiB) on each GPU the library runs on,
 * held until the process ends.  A call whose partials (the workspace size
 * fa_fwd_split_plan reports for the same arguments) exceed that returns
 * FA_ERR_SCRATCH before launching anything.  The call itself allocates and
 * frees nothing.
 * Every call on one GPU uses that GPU's one array: calls that can overlap on
 * the same GPU (on different streams, or from different threads without
 * ordering) race on it and must be serialised by the caller.  Calls on
 * different GPUs do not interfere.  Arguments, results, errors and the split
 * count are those of fa_fwd_split; for the same split count the result is
 * bitwise the same.
 */
fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                               int64_t H, int64_t H_kv, int64_t N_q, int64_t N_k, int64_t d, float scale,
                               int causal, int num_splits, int dtype, void* stream);

/* fa_split_scratch_bytes -- the size of fa_fwd_split_noalloc's fixed array, in bytes. */
int64_t fa_split_scratch_bytes(void);

/*
 * fa_lse_merge -- the merge alone, for partials made elsewhere (for example
 * one per device of a sequence-parallel split):
 *   o_parts   : float32 [num_parts][rows][d], each part normalised over its keys
 *   lse_parts : float32 [num_parts][rows]; -inf marks a part the row does not see
 *               (its O part is then ignored)
 *   o         : output [rows][d], bfloat16 (out_dtype FA_BF16) or float32 (FA_F32)
 *   lse       : float32 output [rows]; -inf (and O = 0) for a row no part sees
 * 1 <= num_parts, 1 <= rows, 1 <= d <= 4096, else FA_ERR_SHAPE.
 */
fa_status fa_lse_merge(const float* o_parts, const float* lse_parts, int64_t num_parts, int64_t rows,
                       int64_t d, void* o, float* lse, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_SPLIT_H */
