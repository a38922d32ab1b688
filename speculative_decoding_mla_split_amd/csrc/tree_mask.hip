// Device-side builder of the tree visibility mask read by the verify attention (gfx950).
//
// The serving loop of "From Capture Safety to MoE Ceiling" (section "Phase 2e: The Occupancy
// Epiphany and the 3-6x Speedup") built the mask on the host for every step. Here it is one or two
// small kernels on the caller's stream, capturable with the attention:
//
//   tree_fused_kernel    small batches (B <= 1024, B * q_len <= 8192), one launch: each workgroup
//                        sums the mask sizes before its request itself, then fills like
//                        tree_fill_kernel; workgroup (0, 0) also writes the status word.
//   tree_offsets_kernel  larger batches, one workgroup: mask_indptr as the running sum of
//                        q_len * (P_b + q_len) (64-bit, clamped to the capacity), the parent
//                        checks and the status word; then
//   tree_fill_kernel     grid (X, B): request b's rows, 16 bytes per lane per step over aligned
//                        16-byte chunks of the output. A chunk that lies inside one row's prefix
//                        columns is a single 16-byte store of ones; other chunks compute each
//                        byte (prefix column: 1; draft column j of row i: walk i's ancestors, held
//                        in LDS, down to j) and store whole when the chunk is inside the request,
//                        byte by byte at the request's two ends.
//
// The mask layout follows "The Custom sm_120 Verify Kernel", section "The Debugging Gauntlet"
// (rows of prefix + q_len bytes, prefix columns first).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mla_tree_mask.h"

namespace {

constexpr int kOffsetThreads = 1024;
constexpr int kFillThreads = 256;
constexpr int kFillBlocksTarget = 1024;  // workgroups of one fill launch (spread over the requests)
constexpr int kFusedMaxB = 1024;          // single-launch form up to this many requests ...
constexpr int kFusedMaxParents = 8192;    // ... and this many parent entries (checked by one workgroup)

__device__ __forceinline__ long long prefix_len(const int32_t* kv_indptr, int b) {
  const long long p = (long long)kv_indptr[b + 1] - (long long)kv_indptr[b];
  return p > 0 ? p : 0;
}

__global__ __launch_bounds__(kOffsetThreads) void tree_offsets_kernel(const int32_t* __restrict__ parents,
                                                                      const int32_t* __restrict__ kv_indptr,
                                                                      int B, int q_len, long long limit,
                                                                      int32_t* __restrict__ mask_indptr,
                                                                      int32_t* __restrict__ status) {
  __shared__ long long wave_tot[kOffsetThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long carry = 0;  // bytes of all requests before the current chunk of kOffsetThreads
  if (tid == 0) mask_indptr[0] = 0;
  for (int b0 = 0; b0 < B; b0 += kOffsetThreads) {
    const int b = b0 + tid;
    long long x = b < B ? (long long)q_len * (prefix_len(kv_indptr, b) + q_len) : 0;
    // inclusive scan: within the wave, then over the wave totals
    for (int d = 1; d < 64; d <<= 1) {
      const long long y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    long long before = 0, chunk_tot = 0;
    for (int w = 0; w < kOffsetThreads / 64; ++w) {
      const long long t = wave_tot[w];
      if (w < wave) before += t;
      chunk_tot += t;
    }
    const long long end = carry + before + x;
    if (b < B) mask_indptr[b + 1] = (int32_t)(end < limit ? end : limit);
    carry += chunk_tot;
    __syncthreads();  // wave_tot is rewritten by the next chunk
  }
  int bad = 0;
  const long long n = (long long)B * q_len;
  for (long long k = tid; k < n; k += kOffsetThreads) {
    const int i = (int)(k % q_len);
    const int p = parents[k];
    bad |= (p < -1 || p >= i);
  }
  bad = __syncthreads_or(bad);
  if (tid == 0) *status = (bad ? MLA_TREE_BAD_PARENT : 0) | (carry > limit ? MLA_TREE_CAPACITY : 0);
}

// 1 if draft node j is node i or one of its ancestors. par[k] lies in [-1, k) for every k, so the
// walk strictly descends and ends.
__device__ __forceinline__ uint32_t ancestor_or_self(const int* par, int i, int j) {
  if (j > i) return 0;
  int k = i;
  while (k > j) k = par[k];
  return k == j ? 1u : 0u;
}

// Writes request b's q_len rows of P + q_len bytes at custom_mask[start, end); this workgroup
// takes the 16-byte chunks blockIdx.x, blockIdx.x + gridDim.x, ... of them.
__device__ __forceinline__ void fill_request(const int32_t* __restrict__ parents, int b, int q_len, long long P,
                                             long long start, long long end, uint8_t* __restrict__ custom_mask,
                                             int* par) {
  const long long L = P + q_len;
  for (int k = threadIdx.x; k < q_len; k += kFillThreads) {
    const int p = parents[(long long)b * q_len + k];
    par[k] = (p < -1 || p >= k) ? -1 : p;
  }
  __syncthreads();

  const uintptr_t a_lo = reinterpret_cast<uintptr_t>(custom_mask) + (uintptr_t)start;
  const uintptr_t a_hi = reinterpret_cast<uintptr_t>(custom_mask) + (uintptr_t)end;
  const uintptr_t c_lo = a_lo & ~(uintptr_t)15;
  const long long n_chunks = (long long)((a_hi - c_lo + 15) >> 4);
  for (long long k = (long long)blockIdx.x * kFillThreads + threadIdx.x; k < n_chunks;
       k += (long long)gridDim.x * kFillThreads) {
    const uintptr_t ca = c_lo + ((uintptr_t)k << 4);
    const uintptr_t first = ca > a_lo ? ca : a_lo;
    const uintptr_t last = ca + 16 < a_hi ? ca + 16 : a_hi;
    // the request fits in 2^31 - 1 bytes, so its offsets and row length fit 32 bits
    const uint32_t r = (uint32_t)(first - a_lo);
    uint32_t i = r / (uint32_t)L, c = r - i * (uint32_t)L;
    const bool whole = first == ca && last == ca + 16;
    if (whole && (long long)c + 15 < P) {  // sixteen prefix columns of one row
      *reinterpret_cast<uint4*>(ca) = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
      continue;
    }
    uint32_t w[4] = {0, 0, 0, 0};
    for (int q = (int)(first - ca); q < (int)(last - ca); ++q) {
      const uint32_t v = (long long)c < P ? 1u : ancestor_or_self(par, (int)i, (int)((long long)c - P));
      w[q >> 2] |= v << (8 * (q & 3));
      if (++c == (uint32_t)L) {
        c = 0;
        ++i;
      }
    }
    if (whole) {
      *reinterpret_cast<uint4*>(ca) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      for (int q = (int)(first - ca); q < (int)(last - ca); ++q)
        *reinterpret_cast<uint8_t*>(ca + q) = (uint8_t)(w[q >> 2] >> (8 * (q & 3)));
    }
  }
}

__global__ __launch_bounds__(kFillThreads) void tree_fill_kernel(const int32_t* __restrict__ parents,
                                                                 const int32_t* __restrict__ kv_indptr,
                                                                 int q_len, uint8_t* __restrict__ custom_mask,
                                                                 const int32_t* __restrict__ mask_indptr) {
  __shared__ int par[MLA_TREE_MAX_QLEN];
  const int b = blockIdx.y;
  const long long P = prefix_len(kv_indptr, b);
  const long long start = mask_indptr[b], end = mask_indptr[b + 1];
  if (end - start != (long long)q_len * (P + q_len)) return;  // did not fit the capacity: left unwritten
  fill_request(parents, b, q_len, P, start, end, custom_mask, par);
}

__device__ __forceinline__ long long block_sum(long long x, long long* red) {
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  __syncthreads();  // red may still be read by an earlier call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  long long t = 0;
  for (int w = 0; w < kFillThreads / 64; ++w) t += red[w];
  return t;
}

// Single-launch form for small batches: every workgroup sums the mask sizes of the requests before
// its own, workgroup (0, b) writes mask_indptr[b + 1], and workgroup (0, 0) also checks every parent
// and the capacity and writes the status word.
__global__ __launch_bounds__(kFillThreads) void tree_fused_kernel(const int32_t* __restrict__ parents,
                                                                  const int32_t* __restrict__ kv_indptr, int B,
                                                                  int q_len, long long limit,
                                                                  uint8_t* __restrict__ custom_mask,
                                                                  int32_t* __restrict__ mask_indptr,
                                                                  int32_t* __restrict__ status) {
  __shared__ int par[MLA_TREE_MAX_QLEN];
  __shared__ long long red[kFillThreads / 64];
  const int b = blockIdx.y;
  long long part = 0;
  for (int k = threadIdx.x; k < b; k += kFillThreads) part += (long long)q_len * (prefix_len(kv_indptr, k) + q_len);
  const long long start = block_sum(part, red);
  const long long P = prefix_len(kv_indptr, b);
  const long long end = start + (long long)q_len * (P + q_len);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    mask_indptr[b + 1] = (int32_t)(end < limit ? end : limit);
    if (b == 0) mask_indptr[0] = 0;
  }
  if (blockIdx.x == 0 && b == 0) {
    long long tot = 0;
    int bad = 0;
    for (int k = threadIdx.x; k < B; k += kFillThreads) tot += (long long)q_len * (prefix_len(kv_indptr, k) + q_len);
    for (int k = threadIdx.x; k < B * q_len; k += kFillThreads) {
      const int p = parents[k];
      bad |= (p < -1 || p >= k % q_len);
    }
    tot = block_sum(tot, red);
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) *status = (bad ? MLA_TREE_BAD_PARENT : 0) | (tot > limit ? MLA_TREE_CAPACITY : 0);
  }
  if (end > limit) return;  // does not fit the capacity: left unwritten
  fill_request(parents, b, q_len, P, start, end, custom_mask, par);
}

}  // namespace

extern "C" int mla_verify_tree_mask(const int32_t* parents, const int32_t* kv_indptr, int B, int q_len,
                                    uint8_t* custom_mask, int64_t mask_capacity, int32_t* mask_indptr,
                                    int32_t* status, hipStream_t stream) {
  if (!parents || !kv_indptr || !custom_mask || !mask_indptr || !status) return MLA_VERIFY_ERR_NULL;
  if (B < 1 || B > MLA_TREE_MAX_B || q_len < 1 || q_len > MLA_TREE_MAX_QLEN || mask_capacity < 0)
    return MLA_VERIFY_ERR_SHAPE;
  const long long limit = mask_capacity < INT32_MAX ? mask_capacity : INT32_MAX;
  const int x = (kFillBlocksTarget + B - 1) / B;
  if (B <= kFusedMaxB && (long long)B * q_len <= kFusedMaxParents) {
    hipLaunchKernelGGL(tree_fused_kernel, dim3(x, B), dim3(kFillThreads), 0, stream, parents, kv_indptr, B, q_len,
                       limit, custom_mask, mask_indptr, status);
    return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
  }
  hipLaunchKernelGGL(tree_offsets_kernel, dim3(1), dim3(kOffsetThreads), 0, stream, parents, kv_indptr, B, q_len,
                     limit, mask_indptr, status);
  if (hipGetLastError() != hipSuccess) return MLA_VERIFY_ERR_LAUNCH;
  hipLaunchKernelGGL(tree_fill_kernel, dim3(x, B), dim3(kFillThreads), 0, stream, parents, kv_indptr, q_len,
                     custom_mask, mask_indptr);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}
