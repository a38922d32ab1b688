/*
 * mla_kv_compact.h -- C ABI of the KV compaction step: copy each request's prefix rows of the
 * paged MLA KV pool into one contiguous run of slots and rewrite its indices.
 *
 * Sources:
 *  - "The Art of Knowing When to Stop: Deferring Tier 1 Defrag", section "The Decision: Why
 *    Tier 1 Defrag Gets Deferred": Tier 1 would physically move KV rows in device memory so a
 *    request's cache is compact, and update the indices; it was designed and then deferred.
 *  - "From Capture Safety to MoE Ceiling", section "Tier 0 Defrag: The Art of Knowing When to
 *    Stop": the Tier 0 remedy only keeps the allocator's free list sorted, so new allocations come
 *    out contiguous; rows already scattered stay where they are. This call moves those rows into
 *    a contiguous run the caller took from that free list.
 *
 * Per row the work is one 1152-byte read and one 1152-byte write; the step is bound by HBM.
 *
 * Conventions are those of mla_verify.h: device pointers on the current device, caller-owned
 * buffers, host-side argument checks returning a negative mla_verify_status before any HIP
 * call, asynchronous on `stream`, graph-capturable (the launch shape depends on B only), no
 * global state.
 */
#ifndef MLA_KV_COMPACT_H
#define MLA_KV_COMPACT_H

#include "mla_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bits of the device status word written by mla_verify_kv_compact (0: every row moved). */
#define MLA_COMPACT_BAD_DST 1 /* a request's destination run leaves [0, N): that request is untouched */
#define MLA_COMPACT_BAD_SRC 2 /* a source slot lies outside [0, N): that row is not moved */

#define MLA_COMPACT_MAX_B 4096 /* largest B the compaction accepts */

/*
 * For each request b with P_b = max(0, kv_indptr[b+1] - kv_indptr[b]) and j < P_b:
 *   kv_pool[dst_start[b] + j, :] = kv_pool[kv_indices[kv_indptr[b] + j], :]   (all 576 values)
 *   new_kv_indices[kv_indptr[b] + j] = dst_start[b] + j
 *
 *  kv_pool        bf16 [N, 576], read and written in place; 16-byte aligned.
 *  N              pool rows, 1 <= N <= 2^31 - 1.
 *  kv_indptr      int32 [B + 1], as in mla_verify_attn (kv_indptr[0] need not be 0).
 *  kv_indices     int32: the prefix slots, read.
 *  dst_start      int32 [B]: first slot of request b's destination run.
 *  B              requests, 1 <= B <= MLA_COMPACT_MAX_B.
 *  new_kv_indices int32, written at the same positions as kv_indices (entries outside every
 *                 request's range are not touched); must not overlap kv_indices.
 *  status         int32 [1], written with the MLA_COMPACT_* bits above.
 *  stream         HIP stream the two kernels (checks, then the copy) are enqueued on.
 *
 * The destination runs must not overlap each other or any source slot of the same call (the
 * free list hands out slots no live row uses); otherwise the result is undefined. A request
 * whose run leaves the pool keeps its rows and its indices (new_kv_indices = kv_indices there);
 * a row whose source slot is outside the pool is not copied and keeps its index.
 *
 * Returns MLA_VERIFY_OK, MLA_VERIFY_ERR_NULL (a pointer is NULL), MLA_VERIFY_ERR_SHAPE (B or N
 * out of range, kv_pool not 16-byte aligned) or MLA_VERIFY_ERR_LAUNCH.
 */
int mla_verify_kv_compact(void *kv_pool, int64_t N, const int32_t *kv_indptr,
                          const int32_t *kv_indices, const int32_t *dst_start, int B,
                          int32_t *new_kv_indices, int32_t *status, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_KV_COMPACT_H */
