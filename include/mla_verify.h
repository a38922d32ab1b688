/*
 * mla_verify.h -- C ABI of the MI355X (gfx950) tree-verify attention over an MLA paged KV cache.
 *
 * One call computes, for every request b, draft token i and head h, softmax attention of the
 * query [q_nope | q_rope] (576 values) over the request's columns: its prefix tokens followed by
 * its q_len draft tokens, each a 576-wide bf16 row of the KV pool (512 latent values, which are
 * also the value vector, then 64 rope values), restricted to the columns the tree mask makes
 * visible. It runs as a split-KV flash-decode: nsplit partials per request, each holding online
 * softmax statistics of one contiguous column slice, then a log-sum-exp combine.
 *
 * Sources (the pages this interface is built from):
 *  - "From Capture Safety to MoE Ceiling" (magik.net llmopt seg_66/chunk_3), section
 *    "The Architecture of Capture Safety": a fixed NSPLIT with chunk bounds computed on the
 *    device from the actual KV length and cheap early exit of empty splits; prefix slots read
 *    from kv_indices and draft slots from out_cache_loc, chosen by position relative to the
 *    prefix length (no host-side concatenation); the raw custom_mask with mask_indptr offsets
 *    indexed inline; a workspace allocated outside the step; no host synchronisation,
 *    allocation or copy inside the step, so the step can be captured into a graph.
 *  - "The Custom sm_120 Verify Kernel" (magik.net llmopt seg_66/chunk_2), section "Building
 *    the Custom Kernel": per-split partial softmax statistics in global scratch and a second
 *    reduction kernel; section "The Debugging Gauntlet": draft columns come after the prefix
 *    columns and a mask row is prefix + q_len bytes wide; only the first B mask offsets matter.
 *
 * Conventions for every entry point:
 *  - Device pointers refer to memory of the current HIP device; host scalars are passed by value.
 *  - The caller owns every buffer (the no-alloc call's static scratch aside). The library never
 *    allocates, frees, copies through the host or synchronises; it only enqueues kernels on
 *    `stream` (NULL = the default stream).
 *  - Argument errors are detected on the host and returned as a negative status before any HIP
 *    call is made. A failed kernel launch returns MLA_VERIFY_ERR_LAUNCH.
 *  - The call is asynchronous and can be captured into a hipGraph: the launch configuration
 *    depends only on (B, q_len, H, nsplit), and every length is read on the device.
 *  - Apart from the static scratch of mla_verify_attn_balanced_noalloc there is no global mutable
 *    state: calls on different streams with different workspaces may run concurrently.
 */
#ifndef MLA_VERIFY_H
#define MLA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_VERIFY_OK = 0,
    MLA_VERIFY_ERR_NULL = -1,      /* a required pointer is NULL */
    MLA_VERIFY_ERR_SHAPE = -2,     /* B, q_len, H or N out of range, or scale not finite and > 0 */
    MLA_VERIFY_ERR_NSPLIT = -3,    /* nsplit outside [1, MLA_VERIFY_MAX_NSPLIT] */
    MLA_VERIFY_ERR_WORKSPACE = -4, /* workspace NULL, misaligned or smaller than required */
    MLA_VERIFY_ERR_LAUNCH = -5,    /* the HIP runtime refused a kernel launch */
    MLA_VERIFY_ERR_SCRATCH = -6    /* the sizes need more than the static scratch of the no-alloc call */
} mla_verify_status;

#define MLA_VERIFY_LATENT 512          /* latent (value) width of a KV row */
#define MLA_VERIFY_ROPE 64             /* rope width of a KV row */
#define MLA_VERIFY_ROW 576             /* bf16 values per KV pool row (1152 bytes) */
#define MLA_VERIFY_MAX_NSPLIT 1024
#define MLA_VERIFY_WORKSPACE_ALIGN 256 /* required alignment of the workspace pointer */
#define MLA_VERIFY_MAX_UNITS 4096      /* largest `units` of the balanced entry points */
#define MLA_VERIFY_BALANCED_MAX_B 4096 /* largest B of the balanced entry points */
#define MLA_VERIFY_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20) /* static scratch per device (no-alloc call) */

/*
 * Bytes of workspace mla_verify_attn needs for these sizes ("From Capture Safety to MoE
 * Ceiling", "The Architecture of Capture Safety": the workspace is allocated once, outside
 * the step). It holds one partial per (request, split, draft token, head): the running max,
 * the sum and a power-of-two scale (a 16-byte record), the 512-wide accumulator (512 fp16
 * values) and the top record (8 bytes).
 * Returns 0 when an argument is out of range (B, q_len, H < 1; nsplit outside [1, 1024]).
 */
size_t mla_verify_attn_workspace_size(int B, int q_len, int H, int nsplit);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char *mla_verify_status_string(int status);

/*
 * Tree-verify attention for B requests (sources above).
 *
 *  q_nope        bf16 [B, q_len, H, 512], dense row-major: latent part of each query.
 *  q_rope        bf16 [B, q_len, H, 64], dense row-major: rope part of each query.
 *  kv_pool       bf16 [N, 576], dense row-major: one row per token slot (page size 1);
 *                columns [0, 512) are the latent (key and value), [512, 576) the rope (key).
 *  N             number of pool rows. A slot outside [0, N) is clamped into range, so no read
 *                leaves the pool; the result of a row that reads such a slot is unspecified.
 *  kv_indptr     int32 [B + 1]: the prefix of request b is kv_indices[kv_indptr[b] ..
 *                kv_indptr[b+1]); prefix length P_b = kv_indptr[b+1] - kv_indptr[b] >= 0.
 *                kv_indptr[0] need not be 0. A negative P_b is treated as 0.
 *  kv_indices    int32: prefix slots. May be NULL only if every P_b is 0.
 *  out_cache_loc int32 [B * q_len]: slot of draft token t of request b at b*q_len + t.
 *  custom_mask   uint8: for request b, q_len rows of L_b = P_b + q_len bytes starting at
 *                mask_indptr[b]; byte custom_mask[mask_indptr[b] + i*L_b + c] != 0 makes
 *                column c (prefix columns first, then draft columns) visible to draft token i.
 *  mask_indptr   int32, at least B entries (a CSR array of B + 1 is accepted; entry B is
 *                never read): start offset of each request's mask.
 *  B, q_len, H   requests, draft tokens per request, query heads; all >= 1.
 *  scale         multiplies the 576-wide dot product before the softmax (finite, > 0).
 *  nsplit        number of contiguous column splits per request, in [1, 1024]. Split s covers
 *                columns [s*chunk, min(L_b, (s+1)*chunk)) with chunk = ceil(L_b / nsplit)
 *                rounded up to a multiple of 32; splits past L_b exit at once.
 *  workspace     device scratch of at least mla_verify_attn_workspace_size(B, q_len, H, nsplit)
 *                bytes, aligned to 256 bytes. No initialisation is needed; its contents after
 *                the call are unspecified. Calls that share a workspace must be ordered (same
 *                stream, or synchronised).
 *  out           bf16 [B, q_len, H, 512]: softmax-weighted sum of the visible latent rows,
 *                rounded to nearest even. A row with no visible column gets zeros.
 *  lse           fp32 [B, q_len, H]: natural-log log-sum-exp of the visible scaled scores
 *                (-inf for a row with no visible column).
 *  stream        HIP stream the two kernels are enqueued on.
 *
 * Returns MLA_VERIFY_OK or a negative mla_verify_status. Behaviour is undefined when a device
 * array is shorter than described above (for example a mask shorter than its offsets imply).
 */
int mla_verify_attn(const void *q_nope, const void *q_rope, const void *kv_pool, int64_t N,
                    const int32_t *kv_indptr, const int32_t *kv_indices,
                    const int32_t *out_cache_loc, const uint8_t *custom_mask,
                    const int32_t *mask_indptr, int B, int q_len, int H, float scale, int nsplit,
                    void *workspace, size_t workspace_bytes, void *out, float *lse,
                    hipStream_t stream);

/*
 * The two phases of mla_verify_attn as separate calls (same arguments and rules as above).
 * mla_verify_attn == mla_verify_attn_partial followed by mla_verify_attn_combine on one stream.
 *
 * mla_verify_attn_partial runs the split kernel ("The Custom sm_120 Verify Kernel", section
 * "Building the Custom Kernel": each block takes one contiguous column slice and writes partial
 * online-softmax statistics to global scratch) and leaves the nsplit partials in `workspace`.
 * mla_verify_attn_combine runs the reduction kernel of the same section on those partials and
 * writes out and lse. Between the two calls the workspace holds, for every (b, s, i, h), the
 * split's running max m (base-2 units of the scaled score, -inf for an empty or fully masked
 * split), its sum l of 2^(score*log2(e) - m), its 512-wide accumulator A (every probability
 * rounded to bf16 before it multiplies a value row, as the matrix cores take it, summed in fp32)
 * stored as fp16 values of A * 2^-e, with e chosen per row so that the largest |A| * 2^-e lies in
 * [2^14, 2^15) (one rounding to 11 significant bits, no overflow for any finite A), and its top
 * record: the exact probability p of the split's largest visible score (same base as l) and the
 * pool slot (already clamped into [0, N)) of that column's 576-wide row. Laid out as
 * float4 ml[B][nsplit][q_len*H] = {m, l, 2^e, 0}, then fp16 acc[B][nsplit][q_len*H][512], then
 * int32x2 top[B][nsplit][q_len*H] = {bits of p, slot}, each region starting at a 256-byte
 * boundary. The combine adds w_s (p - bf16(p)) times the first 512 values of pool row `slot`
 * for every split whose p w_s is at least 1/32 of the row's final sum (exact probability restored
 * for the columns that dominate a row). It reads those rows from `kv_pool` (clamping the slot into
 * [0, N) again, so no read leaves the pool whatever the workspace holds); kv_pool and N must be
 * the ones the partial call used, and its rows must be unchanged in between. A caller may move the
 * partials to another buffer or device between the two calls as long as the combine is given the
 * same pool contents. Calls with the same (B, q_len, H, nsplit) must be used for both.
 */
int mla_verify_attn_partial(const void *q_nope, const void *q_rope, const void *kv_pool, int64_t N,
                            const int32_t *kv_indptr, const int32_t *kv_indices,
                            const int32_t *out_cache_loc, const uint8_t *custom_mask,
                            const int32_t *mask_indptr, int B, int q_len, int H, float scale,
                            int nsplit, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

int mla_verify_attn_combine(const void *workspace, size_t workspace_bytes, const void *kv_pool,
                            int64_t N, int B, int q_len, int H, int nsplit, void *out, float *lse,
                            hipStream_t stream);

/*
 * Balanced partition of the same computation. The per-request splits above give every request
 * nsplit splits whatever its length, so in a ragged batch the short requests' workgroups finish
 * early while the long ones' run on, and every split writes a partial. Here `units` is a split
 * budget for the whole batch (B <= units <= MLA_VERIFY_MAX_UNITS). Request b has T_b =
 * ceil(L_b / 32) column tiles; the device takes the smallest split size C (in tiles) with
 * sum_b ceil(T_b / C) <= units, gives request b n_b = ceil(T_b / C) splits and cuts its tiles
 * evenly: split s covers tiles [floor(s T_b / n_b), floor((s+1) T_b / n_b)) (columns clipped to
 * L_b). The largest split is as small as any such partition allows, so a fixed grid of
 * units * ceil(q_len * H / 128) workgroups is filled with near-equal work; budget left over by the
 * rounding exits at once. Sources: "From Capture Safety to MoE Ceiling", section "The Architecture
 * of Capture Safety" (a fixed grid with chunk bounds computed on the device from the actual lengths)
 * and section "The Occupancy Calculation" (the split count is chosen to fill every SM); "The Custom
 * sm_120 Verify Kernel", section "Building the Custom Kernel" (per-split partials and a second
 * reduction kernel).
 *
 * Arguments and rules are those of mla_verify_attn, with `units` in place of nsplit (the launch
 * shape depends on (B, q_len, H, units) only; a multiple of 8 keeps the XCDs equally loaded) and
 * B <= MLA_VERIFY_BALANCED_MAX_B. units outside [B, MLA_VERIFY_MAX_UNITS] returns
 * MLA_VERIFY_ERR_NSPLIT. The result equals mla_verify_attn's up to rounding order; with units = B
 * every request gets one split and the result is bit-identical to mla_verify_attn with nsplit = 1.
 *
 * The workspace holds the plan (split_info int32x4 [units]: {request, first column, end column, 0}
 * of each split, {-1, 0, 0, 0} if unused; then split_start int32 [B + 1]: the running sum of n_b),
 * then float4 ml [units][q_len*H], fp16 acc [units][q_len*H][512] and int32x2 top
 * [units][q_len*H] partials as described for mla_verify_attn_partial (split split_start[b] + s of
 * request b at block split_start[b] + s), each region 256-byte aligned.
 * mla_verify_attn_balanced_partial writes the plan and the partials (for B <= 64 the partial
 * kernel's workgroups compute the plan themselves; larger batches get it from a one-wave kernel
 * launched first, with the same result); mla_verify_attn_balanced_combine reads both.
 * mla_verify_attn_balanced_workspace_size returns 0 for arguments out of range.
 */
size_t mla_verify_attn_balanced_workspace_size(int B, int q_len, int H, int units);

int mla_verify_attn_balanced(const void *q_nope, const void *q_rope, const void *kv_pool, int64_t N,
                             const int32_t *kv_indptr, const int32_t *kv_indices,
                             const int32_t *out_cache_loc, const uint8_t *custom_mask,
                             const int32_t *mask_indptr, int B, int q_len, int H, float scale, int units,
                             void *workspace, size_t workspace_bytes, void *out, float *lse,
                             hipStream_t stream);

int mla_verify_attn_balanced_partial(const void *q_nope, const void *q_rope, const void *kv_pool,
                                     int64_t N, const int32_t *kv_indptr, const int32_t *kv_indices,
                                     const int32_t *out_cache_loc, const uint8_t *custom_mask,
                                     const int32_t *mask_indptr, int B, int q_len, int H, float scale,
                                     int units, void *workspace, size_t workspace_bytes,
                                     hipStream_t stream);

int mla_verify_attn_balanced_combine(const void *workspace, size_t workspace_bytes, const void *kv_pool,
                                     int64_t N, int B, int q_len, int H, int units, void *out, float *lse,
                                     hipStream_t stream);

/*
 * mla_verify_attn_balanced without a workspace argument, for callers that cannot allocate device
 * memory: code under hipGraph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, rules and result as mla_verify_attn_balanced (the same kernels run), with the
 * workspace taken from a static device array of MLA_VERIFY_NOALLOC_SCRATCH_BYTES (128 MiB) that the
 * library defines. Every device the library's code is loaded on holds its own copy of that array
 * until the process ends. The first call on a device (the current one) resolves the array's address
 * there, once, and keeps it; no call allocates, frees or copies memory. Nothing in the array needs
 * initialising: each call rewrites the plan and the partials it reads.
 *
 * Sizes whose balanced workspace (mla_verify_attn_balanced_workspace_size) exceeds the array return
 * MLA_VERIFY_ERR_SCRATCH before any HIP call; a device whose copy of the array cannot be resolved
 * returns MLA_VERIFY_ERR_LAUNCH.
 *
 * All calls on one device share that device's array: two calls whose kernels can overlap (on
 * different streams, or on one stream while a graph containing another such call runs) race on it
 * and their results are undefined. Order them on one stream or synchronise in between.
 */
int mla_verify_attn_balanced_noalloc(const void *q_nope, const void *q_rope, const void *kv_pool, int64_t N,
                                     const int32_t *kv_indptr, const int32_t *kv_indices,
                                     const int32_t *out_cache_loc, const uint8_t *custom_mask,
                                     const int32_t *mask_indptr, int B, int q_len, int H, float scale,
                                     int units, void *out, float *lse, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H */
