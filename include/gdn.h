/*
 * gdn.h -- C ABI of the Gated DeltaNet prefill scan (part of the same library as moe.h).
 *
 * "Optimizing on-device inference for Apple Silicon", section "Prefill > Keep recurrent
 * state on chip": during prefill a Gated DeltaNet layer scans the prompt in order and
 * carries a recurrent state matrix; the state and its gate are 32-bit floats, query and
 * key activations bfloat16.  The pages print no update formula; the one implemented is
 * the gated delta rule (Yang, Kautz and Hatamizadeh, "Gated Delta Networks", ICLR 2025),
 * per value head h and token t:
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * S is d_v x d_k with one row per value channel; value head h reads key head
 * h / (n_vheads / n_kheads).  The state stays in registers for the whole scan (one
 * 16-lane group per row) and is written back once at the end.
 *
 * Conventions are those of moe.h: device pointers, caller-owned memory, work enqueued
 * on `stream` without host synchronisation, status codes from moe_status.
 */
#ifndef MOE_GDN_MI355X_H
#define MOE_GDN_MI355X_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Scan T tokens of one layer, starting from the state in `state` and leaving the state
 * after token T-1 there (so a long prompt can be scanned in chunks, the state carried
 * from one call to the next; section "Prefill > Bound temporary memory with prompt
 * chunking").
 *   T          tokens, >= 0 (0: nothing is enqueued, the state is unchanged)
 *   n_kheads   key/query heads >= 1; n_vheads value heads, a multiple of n_kheads, <= 4096
 *   d_k, d_v   head widths; both must be 128
 *   q, k       bf16 [T][n_kheads][128], 16-byte aligned
 *   v          bf16 [T][n_vheads][128], 16-byte aligned
 *   alpha      float32 [T][n_vheads]: the decay gate (in [0, 1] for the intended use;
 *              0 clears the state before the token's write), 4-byte aligned
 *   beta       float32 [T][n_vheads]: the write strength, 4-byte aligned
 *   state      float32 [n_vheads][128][128] (row j = value channel j), read and
 *              written in place, 16-byte aligned
 *   out        bf16 [T][n_vheads][128], o_t rounded to nearest even, 2-byte aligned
 * out and state may overlap neither an input nor each other (MOE_ERR_ALIAS).
 * Returns MOE_ERR_TOKENS (T < 0), MOE_ERR_SHAPE, MOE_ERR_NULL, MOE_ERR_ALIGN,
 * MOE_ERR_DEVICE (current device not gfx950) or MOE_ERR_HIP, before enqueueing anything
 * except for MOE_ERR_HIP. */
moe_status moe_gdn_scan(int32_t T, int32_t n_kheads, int32_t n_vheads, int32_t d_k, int32_t d_v,
                        const void *q, const void *k, const void *v, const float *alpha,
                        const float *beta, float *state, void *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
