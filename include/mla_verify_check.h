/*
 * mla_verify_check.h -- C ABI of the capture-safe validate mode: a device-side cross-check of the
 * verify attention against a simple per-row GPU reference, with the errors written to a device
 * report and no host synchronisation.
 *
 * Sources:
 *  - "The Custom sm_120 Verify Kernel", section "The Integration Challenge": a validate mode ran the
 *    reference attention and the custom kernel side by side, compared and logged their outputs and
 *    served the reference's result; section "The Debugging Gauntlet" (bug 1) and "From Capture
 *    Safety to MoE Ceiling", section "The Leap of Faith": that comparison synchronised with the host
 *    (and allocated), so it broke graph capture and could only run eagerly.
 *  - "The Custom sm_120 Verify Kernel", section "Building the Custom Kernel": the baseline there was a
 *    naive kernel, one block per head. The reference here is that plain per-row form, in fp32,
 *    written independently of the fast path.
 *
 * Difference from the pages' mode: the output is the fast path's (the reference only checks it),
 * and the comparison result stays on the device for the caller to read whenever it likes.
 *
 * Conventions are those of mla_verify.h: device pointers on the current device, caller-owned
 * buffers, host-side argument checks returning a negative mla_verify_status before any HIP call,
 * asynchronous on `stream`, graph-capturable (the launch shape depends on (B, q_len, H,
 * sample_stride) only; the report is cleared by a kernel, not a memset), no global state.
 */
#ifndef MLA_VERIFY_CHECK_H
#define MLA_VERIFY_CHECK_H

#include "mla_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Words of the report written by the check (float [MLA_VERIFY_REPORT_WORDS]). */
#define MLA_VERIFY_REPORT_MAX_OUT 0  /* max |out - ref| over the checked rows' 512 values */
#define MLA_VERIFY_REPORT_MAX_LSE 1  /* max |lse - ref_lse| over the checked rows with finite LSE */
#define MLA_VERIFY_REPORT_ROWS 2     /* number of rows checked */
#define MLA_VERIFY_REPORT_BAD 3      /* checked rows with a non-finite output value or whose -inf LSE
                                        pattern differs from the reference */
#define MLA_VERIFY_REPORT_WORDS 4

/*
 * Recompute the rows r = 0, sample_stride, 2*sample_stride, ... of the flattened (b, token, head)
 * index (r = (b*q_len + i)*H + h) with a plain per-row reference and compare them with `out` and
 * `lse` as they stand on `stream` when the check runs (so it checks whatever wrote them earlier on
 * the stream: mla_verify_attn, the balanced form or anything else).
 *
 * The reference: each checked row's columns are cut into 64 pieces; for each piece, a first pass
 * over its visible columns takes the max of the scaled scores and a second pass turns each score
 * into exp(s - max) (fp32, not rounded) and accumulates the value rows and the sum; a merge kernel
 * combines the pieces (max, then exp-weighted sums), forms out_ref = acc / sum and lse_ref =
 * max + ln(sum) and compares. Columns, slots and the mask follow mla_verify_attn exactly. The cost
 * grows with the checked rows times their lengths (every checked row reads its KV rows three
 * times); choose sample_stride accordingly.
 *
 *  (inputs)      as mla_verify_attn: q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices,
 *                out_cache_loc, custom_mask, mask_indptr, B, q_len, H, scale.
 *  out, lse      the outputs to check (read only).
 *  sample_stride >= 1; 1 checks every row.
 *  workspace     device scratch of mla_verify_attn_check_workspace_size(B, q_len, H, sample_stride)
 *                bytes or more, 256-byte aligned; contents unspecified before and after.
 *  report        float [MLA_VERIFY_REPORT_WORDS], device memory, overwritten (cleared first).
 *
 * Returns MLA_VERIFY_OK, MLA_VERIFY_ERR_NULL, MLA_VERIFY_ERR_SHAPE (as mla_verify_attn, or
 * sample_stride < 1), MLA_VERIFY_ERR_WORKSPACE or MLA_VERIFY_ERR_LAUNCH.
 */
size_t mla_verify_attn_check_workspace_size(int B, int q_len, int H, int sample_stride);

int mla_verify_attn_check(const void *q_nope, const void *q_rope, const void *kv_pool, int64_t N,
                          const int32_t *kv_indptr, const int32_t *kv_indices,
                          const int32_t *out_cache_loc, const uint8_t *custom_mask,
                          const int32_t *mask_indptr, int B, int q_len, int H, float scale,
                          const void *out, const float *lse, int sample_stride, void *workspace,
                          size_t workspace_bytes, float *report, hipStream_t stream);

/*
 * Validate mode in one call: mla_verify_attn (same arguments) followed by mla_verify_attn_check on
 * its output, both using `workspace` (the attention's partials are dead once its combine has run).
 * The workspace must hold mla_verify_attn_validate_workspace_size(B, q_len, H, nsplit,
 * sample_stride) bytes (the larger of the two needs; 0 for arguments out of range). out and lse
 * hold the fast path's result; the report says how far it is from the reference. Returns the first
 * non-OK status of the two.
 */
size_t mla_verify_attn_validate_workspace_size(int B, int q_len, int H, int nsplit, int sample_stride);

int mla_verify_attn_validate(const void *q_nope, const void *q_rope, const void *kv_pool, int64_t N,
                             const int32_t *kv_indptr, const int32_t *kv_indices,
                             const int32_t *out_cache_loc, const uint8_t *custom_mask,
                             const int32_t *mask_indptr, int B, int q_len, int H, float scale,
                             int nsplit, void *workspace, size_t workspace_bytes, void *out,
                             float *lse, int sample_stride, float *report, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_CHECK_H */
