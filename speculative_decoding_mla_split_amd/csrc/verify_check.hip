// Capture-safe validate mode for the verify attention (gfx950): a plain per-row fp32 reference,
// run on the device after the fast path, that writes how far the fast path's out/lse are from it
// into a device report. Nothing goes through the host, so the whole thing can sit in a graph.
//
//   report_clear_kernel     zeroes the report (a kernel, so graph replays never carry a memset node).
//   ref_piece_kernel        grid (checked rows, 64 pieces): every sample_stride-th row of the
//                           flattened (b, token, head) index is cut into 64 column pieces, one
//                           workgroup of 256 threads each (a 185k-column row in one workgroup took
//                           ~46 ms, latency-bound). The query sits in LDS as fp32. Pass 1: each
//                           thread scores its columns (a full 576-wide dot product per column straight
//                           from the pool row) and the workgroup takes the max over the visible ones.
//                           Pass 2, 256 columns at a time: each thread turns one column's score into
//                           exp(s - max) and parks it with the column's slot in LDS; then thread t
//                           accumulates output values 2t and 2t+1 over the parked columns. The piece's
//                           (max, sum, 512 accumulators) go to the workspace.
//   ref_merge_check_kernel  one workgroup per checked row: merges its pieces, out_ref = acc / sum,
//                           lse_ref = max + ln(sum); the row's largest |out - out_ref| and
//                           |lse - lse_ref| go into the report with atomic max (non-negative floats
//                           order like their bit patterns), the row count and the count of bad rows
//                           with atomic adds.
//
// The reference is written from the definition of the operation, independently of the fast path:
// no MFMA, no bf16 rounding of probabilities, exact exp, fp32 throughout, and no shared helpers with
// the fast kernels.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "mla_verify_check.h"

namespace {

constexpr int kRefThreads = 256;
constexpr int kRowBytes = MLA_VERIFY_ROW * 2;
constexpr int kLatent = MLA_VERIFY_LATENT;
constexpr int kRope = MLA_VERIFY_ROPE;
constexpr int kPieces = 64;  // pieces per checked row, each its own workgroup

__global__ void report_clear_kernel(float* __restrict__ report) {
  if (threadIdx.x < MLA_VERIFY_REPORT_WORDS) report[threadIdx.x] = 0.0f;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// scale * (q . K_row) over the 576 values of one pool row.
__device__ __forceinline__ float row_score(const float* q, const uint8_t* __restrict__ row, float scale) {
  float acc = 0.0f;
  const uint4* r = reinterpret_cast<const uint4*>(row);
#pragma unroll 4
  for (int k = 0; k < kRowBytes / 16; ++k) {
    const uint4 v = r[k];
    const float* qk = q + 8 * k;
    acc += qk[0] * bf16_lo(v.x) + qk[1] * bf16_hi(v.x) + qk[2] * bf16_lo(v.y) + qk[3] * bf16_hi(v.y) +
           qk[4] * bf16_lo(v.z) + qk[5] * bf16_hi(v.z) + qk[6] * bf16_lo(v.w) + qk[7] * bf16_hi(v.w);
  }
  return scale * acc;
}

__device__ __forceinline__ float block_max(float x, float* red) {
  for (int d = 32; d >= 1; d >>= 1) x = fmaxf(x, __shfl_xor(x, d, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = red[0];
  for (int w = 1; w < kRefThreads / 64; ++w) m = fmaxf(m, red[w]);
  return m;
}

__device__ __forceinline__ float block_sum(float x, float* red) {
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float s = 0.0f;
  for (int w = 0; w < kRefThreads / 64; ++w) s += red[w];
  return s;
}

// Pass over one piece [c_lo, c_hi) of a checked row: max of the visible scaled scores, then
// exp(s - max), their sum and the weighted sum of the value rows (values 2t, 2t + 1 per thread).
// Writes the piece's (max, sum) and 512 accumulators.
__global__ void __launch_bounds__(kRefThreads)
ref_piece_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
                 const uint8_t* __restrict__ kv_pool, int N, const int32_t* __restrict__ kv_indptr,
                 const int32_t* __restrict__ kv_indices, const int32_t* __restrict__ out_cache_loc,
                 const uint8_t* __restrict__ custom_mask, const int32_t* __restrict__ mask_indptr, int q_len,
                 int H, float scale, int sample_stride, float2* __restrict__ piece_ml,
                 float* __restrict__ piece_acc) {
  __shared__ float q[kLatent + kRope];
  __shared__ float p_park[kRefThreads];
  __shared__ int slot_park[kRefThreads];
  __shared__ float red[kRefThreads / 64];
  const int t = threadIdx.x;
  const long long k = blockIdx.x;                 // checked row number
  const long long row = k * sample_stride;        // (b * q_len + i) * H + h
  const int R = q_len * H;
  const int b = (int)(row / R), i = (int)((row % R) / H);

  for (int d = t; d < kLatent + kRope; d += kRefThreads)
    q[d] = __uint_as_float((uint32_t)(d < kLatent ? q_nope[row * kLatent + d] : q_rope[row * kRope + d - kLatent])
                           << 16);
  const int kv_start = kv_indptr[b];
  const int P = max(kv_indptr[b + 1] - kv_start, 0);
  const int L = P + q_len;
  const int chunk = (L + kPieces - 1) / kPieces;
  const int c_lo = min(L, (int)blockIdx.y * chunk), c_hi = min(L, c_lo + chunk);
  const uint8_t* mask_row = custom_mask + (size_t)mask_indptr[b] + (size_t)i * L;
  auto slot_of = [&](int c) {
    const int s = c < P ? kv_indices[kv_start + c] : out_cache_loc[(size_t)b * q_len + (c - P)];
    return min(max(s, 0), N - 1);
  };
  __syncthreads();

  float m = -INFINITY;
  for (int c = c_lo + t; c < c_hi; c += kRefThreads)
    if (mask_row[c]) m = fmaxf(m, row_score(q, kv_pool + (size_t)slot_of(c) * kRowBytes, scale));
  m = block_max(m, red);

  float acc0 = 0.0f, acc1 = 0.0f, l_part = 0.0f;
  if (m != -INFINITY) {
    for (int c0 = c_lo; c0 < c_hi; c0 += kRefThreads) {
      const int c = c0 + t;
      float p = 0.0f;
      int s = 0;
      if (c < c_hi && mask_row[c]) {
        s = slot_of(c);
        p = expf(row_score(q, kv_pool + (size_t)s * kRowBytes, scale) - m);
      }
      l_part += p;
      __syncthreads();  // the previous chunk's parked values are no longer read
      p_park[t] = p;
      slot_park[t] = s;
      __syncthreads();
      const int n = min(kRefThreads, c_hi - c0);
      for (int j = 0; j < n; ++j) {
        const float pj = p_park[j];
        if (pj != 0.0f) {
          const uint32_t v = *reinterpret_cast<const uint32_t*>(kv_pool + (size_t)slot_park[j] * kRowBytes + 4 * t);
          acc0 += pj * bf16_lo(v);
          acc1 += pj * bf16_hi(v);
        }
      }
    }
  }
  const float l = block_sum(l_part, red);
  const size_t piece = (size_t)k * kPieces + blockIdx.y;
  reinterpret_cast<float2*>(piece_acc + piece * kLatent)[t] = make_float2(acc0, acc1);
  if (t == 0) piece_ml[piece] = make_float2(m, l);
}

// Merge a checked row's pieces (max M, sum = sum_p exp(m_p - M) l_p, likewise the accumulators),
// form out_ref and lse_ref, compare with the fast path's out and lse and fold the row into the
// report.
__global__ void __launch_bounds__(kRefThreads)
ref_merge_check_kernel(const float2* __restrict__ piece_ml, const float* __restrict__ piece_acc, int sample_stride,
                       const uint16_t* __restrict__ out, const float* __restrict__ lse, float* __restrict__ report) {
  __shared__ float red[kRefThreads / 64];
  const int t = threadIdx.x;
  const long long k = blockIdx.x;
  const long long row = k * sample_stride;
  const float2* ml = piece_ml + (size_t)k * kPieces;
  float M = -INFINITY;
  for (int p = 0; p < kPieces; ++p) M = fmaxf(M, ml[p].x);
  const bool empty = M == -INFINITY;
  float l = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
  if (!empty) {
    for (int p = 0; p < kPieces; ++p) {
      const float2 st = ml[p];
      if (st.x == -INFINITY) continue;  // a piece with no visible column
      const float w = expf(st.x - M);
      l += w * st.y;
      const float2 a = reinterpret_cast<const float2*>(piece_acc + ((size_t)k * kPieces + p) * kLatent)[t];
      acc0 += w * a.x;
      acc1 += w * a.y;
    }
  }
  const float ref0 = empty ? 0.0f : acc0 / l, ref1 = empty ? 0.0f : acc1 / l;
  const uint32_t o = *reinterpret_cast<const uint32_t*>(out + row * kLatent + 2 * t);
  const float o0 = bf16_lo(o), o1 = bf16_hi(o);
  const bool finite = isfinite(o0) && isfinite(o1);
  const float d = finite ? fmaxf(fabsf(o0 - ref0), fabsf(o1 - ref1)) : 0.0f;
  const float d_max = block_max(d, red);
  const float bad_out = block_max(finite ? 0.0f : 1.0f, red);
  if (t == 0) {
    const float ref_lse = empty ? -INFINITY : M + logf(l);
    const float got = lse[row];
    bool bad = bad_out != 0.0f;
    float d_lse = 0.0f;
    if (empty)
      bad = bad || got != -INFINITY;
    else if (isfinite(got))
      d_lse = fabsf(got - ref_lse);
    else
      bad = true;
    atomicMax(reinterpret_cast<int*>(report + MLA_VERIFY_REPORT_MAX_OUT), __float_as_int(d_max));
    atomicMax(reinterpret_cast<int*>(report + MLA_VERIFY_REPORT_MAX_LSE), __float_as_int(d_lse));
    atomicAdd(report + MLA_VERIFY_REPORT_ROWS, 1.0f);
    if (bad) atomicAdd(report + MLA_VERIFY_REPORT_BAD, 1.0f);
  }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool sizes_ok(int B, int q_len, int H) {
  if (B < 1 || q_len < 1 || H < 1) return false;
  const long long rows = (long long)q_len * H;
  return rows <= (1LL << 24) && (long long)B * rows <= (1LL << 30);
}

long long checked_rows(int B, int q_len, int H, int sample_stride) {
  const long long rows = (long long)B * q_len * H;
  return (rows + sample_stride - 1) / sample_stride;
}

}  // namespace

extern "C" size_t mla_verify_attn_check_workspace_size(int B, int q_len, int H, int sample_stride) {
  if (!sizes_ok(B, q_len, H) || sample_stride < 1) return 0;
  const size_t pieces = (size_t)checked_rows(B, q_len, H, sample_stride) * kPieces;
  return align_up(pieces * sizeof(float2), MLA_VERIFY_WORKSPACE_ALIGN) +
         align_up(pieces * kLatent * sizeof(float), MLA_VERIFY_WORKSPACE_ALIGN);
}

extern "C" int mla_verify_attn_check(const void* q_nope, const void* q_rope, const void* kv_pool, int64_t N,
                                     const int32_t* kv_indptr, const int32_t* kv_indices,
                                     const int32_t* out_cache_loc, const uint8_t* custom_mask,
                                     const int32_t* mask_indptr, int B, int q_len, int H, float scale,
                                     const void* out, const float* lse, int sample_stride, void* workspace,
                                     size_t workspace_bytes, float* report, hipStream_t stream) {
  if (!q_nope || !q_rope || !kv_pool || !kv_indptr || !out_cache_loc || !custom_mask || !mask_indptr || !out ||
      !lse || !report)
    return MLA_VERIFY_ERR_NULL;
  if (!sizes_ok(B, q_len, H) || N < 1 || N > INT32_MAX || !(scale > 0.0f) || !isfinite(scale) || sample_stride < 1)
    return MLA_VERIFY_ERR_SHAPE;
  const long long checked = checked_rows(B, q_len, H, sample_stride);
  if (checked > INT32_MAX) return MLA_VERIFY_ERR_SHAPE;
  const size_t need = mla_verify_attn_check_workspace_size(B, q_len, H, sample_stride);
  if (!workspace || ((uintptr_t)workspace % MLA_VERIFY_WORKSPACE_ALIGN) != 0 || workspace_bytes < need)
    return MLA_VERIFY_ERR_WORKSPACE;
  float2* piece_ml = static_cast<float2*>(workspace);
  float* piece_acc = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                              align_up((size_t)checked * kPieces * sizeof(float2),
                                                       MLA_VERIFY_WORKSPACE_ALIGN));
  hipLaunchKernelGGL(report_clear_kernel, dim3(1), dim3(64), 0, stream, report);
  if (hipGetLastError() != hipSuccess) return MLA_VERIFY_ERR_LAUNCH;
  hipLaunchKernelGGL(ref_piece_kernel, dim3((unsigned)checked, kPieces), dim3(kRefThreads), 0, stream,
                     static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope),
                     static_cast<const uint8_t*>(kv_pool), (int)N, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                     mask_indptr, q_len, H, scale, sample_stride, piece_ml, piece_acc);
  if (hipGetLastError() != hipSuccess) return MLA_VERIFY_ERR_LAUNCH;
  hipLaunchKernelGGL(ref_merge_check_kernel, dim3((unsigned)checked), dim3(kRefThreads), 0, stream,
                     (const float2*)piece_ml, (const float*)piece_acc, sample_stride,
                     static_cast<const uint16_t*>(out), lse, report);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

extern "C" size_t mla_verify_attn_validate_workspace_size(int B, int q_len, int H, int nsplit, int sample_stride) {
  const size_t a = mla_verify_attn_workspace_size(B, q_len, H, nsplit);
  const size_t c = mla_verify_attn_check_workspace_size(B, q_len, H, sample_stride);
  return (a == 0 || c == 0) ? 0 : (a > c ? a : c);
}

extern "C" int mla_verify_attn_validate(const void* q_nope, const void* q_rope, const void* kv_pool, int64_t N,
                                        const int32_t* kv_indptr, const int32_t* kv_indices,
                                        const int32_t* out_cache_loc, const uint8_t* custom_mask,
                                        const int32_t* mask_indptr, int B, int q_len, int H, float scale,
                                        int nsplit, void* workspace, size_t workspace_bytes, void* out, float* lse,
                                        int sample_stride, float* report, hipStream_t stream) {
  if (!report) return MLA_VERIFY_ERR_NULL;
  if (sample_stride < 1) return MLA_VERIFY_ERR_SHAPE;
  if (workspace_bytes < mla_verify_attn_check_workspace_size(B, q_len, H, sample_stride))
    return MLA_VERIFY_ERR_WORKSPACE;
  // the attention's partials are dead once its combine has run, so the check reuses the workspace
  const int rc = mla_verify_attn(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                                 mask_indptr, B, q_len, H, scale, nsplit, workspace, workspace_bytes, out, lse, stream);
  if (rc != MLA_VERIFY_OK) return rc;
  return mla_verify_attn_check(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                               mask_indptr, B, q_len, H, scale, out, lse, sample_stride, workspace, workspace_bytes,
                               report, stream);
}
