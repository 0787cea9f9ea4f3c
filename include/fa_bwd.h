/*
 * fa_bwd.h -- C ABI of the MI355X (gfx950) FlashAttention backward.
 *
 * Operation.  For every batch b and query head h (K/V head g = h / (H / H_kv)),
 * with S = scale * Q K^T under the optional causal mask, P = softmax(S) and the
 * forward's O = P V, the gradients of the scalar sum(dO * O):
 *
 *     dV_g = sum over the group's heads of  P^T dO
 *     dP   = dO V^T,   D_i = sum_d dO_id O_id,   dS = P * (dP - D)   (row-broadcast D)
 *     dQ   = scale * dS K
 *     dK_g = sum over the group's heads of  scale * dS^T Q
 *
 * The robocikowo.com "Flash Attention" page says the backward pass rebuilds
 * the attention matrix from the saved output O and the per-row logsumexp L
 * instead of storing it; P is recomputed here as exp(S - L) tile by tile and
 * never written to memory.  The formulas are the chain rule of the forward
 * definition (systems-analysis.info "FlashAttention (PL)", section
 * "Problematyka standardowego mechanizmu uwagi").
 *
 * Layout.  q, o, dout, dq: dense row-major [B][H][N][d]; k, v, dk, dv:
 * [B][H_kv][N][d]; lse: float32 [B][H][N] (natural log, as fa_fwd writes it).
 *
 * Memory and streams.  Every pointer is a device pointer owned by the caller;
 * the library allocates, frees and synchronises nothing; like fa_fwd it keeps
 * only a per-device cache of read-only launch facts (see fa_fwd.h).
 * ``workspace`` holds fa_bwd_workspace_size() bytes of per-row statistics
 * (and partial sums) that the call writes and then reads; its contents
 * before and after the call carry no meaning for the caller.  The work is
 * enqueued on ``stream`` (a hipStream_t, NULL = default) and the call
 * returns without waiting.
 * Outputs and workspace must not overlap each other or any input.  Results
 * are bitwise reproducible for equal inputs, shape and device (no atomics).
 *
 * Errors.  As in fa_fwd.h: arguments are checked before anything is
 * enqueued; FA_ERR_HIP reports a launch the runtime rejected.
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#include <stdint.h>

#include "fa_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_bwd_workspace_size -- bytes of workspace fa_bwd needs: the per-row
 * statistics, 512 * B * H * ceil(N / 64), and with grouped query heads
 * (H_kv < H) room for partial dK and dV sums, 8 * B * H * N * d (a small
 * causal grid splits each group's query heads over several workgroups and
 * adds their shares afterwards).  FA_ERR_NULL if bytes is NULL; the shape
 * checks of fa_bwd otherwise.
 */
fa_status fa_bwd_workspace_size(int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d, int64_t* bytes);

/*
 * fa_bwd -- dQ, dK and dV of exact attention, recomputing P from q, k and lse.
 *   q, k, v   : the forward's inputs, bfloat16 (dtype must be FA_BF16)
 *   o         : the forward's output O, bfloat16 [B][H][N][d]
 *   dout      : upstream gradient dO, bfloat16 [B][H][N][d]
 *   lse       : the forward's logsumexp, float32 [B][H][N]
 *   workspace : device memory of fa_bwd_workspace_size(B, H, H_kv, N, d) bytes
 *   dq        : output, float32 [B][H][N][d]
 *   dk, dv    : outputs, float32 [B][H_kv][N][d] (each K/V head's sum over its group)
 *   H_kv      : K/V heads, >= 1 and dividing H (H_kv = H: one K/V head per head)
 *   d         : 64, 128 or 256, else FA_ERR_UNSUPPORTED
 *   scale     : finite, the value the forward used
 *   causal    : 0 = no mask, nonzero = query i sees keys j <= i (as in the forward)
 * Every pointer must be 16-byte aligned (FA_ERR_ALIGN).  The statistics D are
 * formed from the given O, so o must be the forward's output for these
 * inputs; lse likewise.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* workspace, float* dq, float* dk, float* dv,
                 int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                 float scale, int causal, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
