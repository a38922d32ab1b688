/*
 * mla_tree_mask.h -- C ABI of the device-side builder of the tree visibility mask that
 * mla_verify_attn reads (custom_mask + mask_indptr), from the draft trees' parent pointers.
 *
 * Sources:
 *  - "From Capture Safety to MoE Ceiling", section "Phase 2e: The Occupancy Epiphany and the
 *    3-6x Speedup": the serving loop built the draft tree and then the mask on the host, about
 *    0.18 ms per step for the mask alone; this entry point builds it on the device, inside the
 *    same stream and graph as the attention, with no host round trip.
 *  - "From Capture Safety to MoE Ceiling", section "The Architecture of Capture Safety": the
 *    kernel reads the raw custom_mask through mask_indptr offsets.
 *  - "The Custom sm_120 Verify Kernel", section "The Debugging Gauntlet" (bug 2): a request's
 *    mask row is prefix + q_len bytes, prefix columns first, then the draft columns.
 *
 * Visibility (the usual tree-attention rule): for draft token i of request b, every prefix
 * column is visible, and draft column j is visible iff j is i or an ancestor of i.
 *
 * Conventions are those of mla_verify.h: device pointers on the current device, caller-owned
 * buffers, host-side argument checks returning a negative mla_verify_status before any HIP
 * call, asynchronous on `stream`, graph-capturable (the launch shape depends on B and q_len
 * only; every length is read on the device), no global state.
 */
#ifndef MLA_TREE_MASK_H
#define MLA_TREE_MASK_H

#include "mla_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bits of the device status word written by mla_verify_tree_mask (0: valid input, all written). */
#define MLA_TREE_BAD_PARENT 1 /* an entry of parents lies outside [-1, i): it was read as -1 */
#define MLA_TREE_CAPACITY 2   /* the masks need more than mask_capacity (or 2^31 - 1) bytes */

#define MLA_TREE_MAX_QLEN 4096 /* largest q_len the builder accepts */
#define MLA_TREE_MAX_B 65535   /* largest B the builder accepts */

/*
 * Build custom_mask and mask_indptr for B requests of q_len draft tokens each.
 *
 *  parents       int32 [B * q_len]: parents[b*q_len + i] is the index (0 .. q_len-1, inside
 *                request b) of draft token i's parent, or -1 for a root. A parent must precede
 *                its child; several roots are allowed. An entry outside [-1, i) sets
 *                MLA_TREE_BAD_PARENT and is read as -1.
 *  kv_indptr     int32 [B + 1], as in mla_verify_attn: P_b = max(0, kv_indptr[b+1] - kv_indptr[b]).
 *  B, q_len      requests and draft tokens per request: 1 <= B <= MLA_TREE_MAX_B,
 *                1 <= q_len <= MLA_TREE_MAX_QLEN.
 *  custom_mask   uint8 [mask_capacity], written: request b's q_len rows of L_b = P_b + q_len bytes
 *                (1 = visible, 0 = not) start at mask_indptr[b], requests back to back from 0.
 *  mask_capacity bytes available at custom_mask (>= 0).
 *  mask_indptr   int32 [B + 1], written: exclusive running sum of q_len * L_b, from 0. When the
 *                total exceeds min(mask_capacity, 2^31 - 1) every entry past that limit is
 *                clamped to it, MLA_TREE_CAPACITY is set and the requests that do not fit are not
 *                written (their bytes keep their old contents).
 *  status        int32 [1], written with the MLA_TREE_* bits above (0 when all is well). Reading
 *                it needs no host synchronisation on the call's stream: it is ordered like any
 *                other output.
 *  stream        HIP stream the two kernels (offsets + checks, then the fill) are enqueued on.
 *
 * Returns MLA_VERIFY_OK, MLA_VERIFY_ERR_NULL (a pointer is NULL), MLA_VERIFY_ERR_SHAPE (B or
 * q_len out of range, mask_capacity < 0) or MLA_VERIFY_ERR_LAUNCH.
 */
int mla_verify_tree_mask(const int32_t *parents, const int32_t *kv_indptr, int B, int q_len,
                         uint8_t *custom_mask, int64_t mask_capacity, int32_t *mask_indptr,
                         int32_t *status, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_TREE_MASK_H */
