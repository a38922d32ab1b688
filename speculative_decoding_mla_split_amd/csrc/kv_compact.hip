// KV compaction for the paged MLA cache (gfx950): move each request's prefix rows into one
// contiguous run of slots and rewrite its indices -- the relocation step that "The Art of Knowing
// When to Stop: Deferring Tier 1 Defrag" (section "The Decision: Why Tier 1 Defrag Gets Deferred")
// designs and defers.
//
//   kv_compact_check_kernel  one workgroup: checks every destination run against the pool and
//                            writes the status word.
//   kv_compact_kernel        one wave of resident workgroups striding over the concatenated prefix
//                            rows of all requests (so ragged batches spread evenly). A wave moves 8 rows per
//                            step: lanes 0-7 resolve one row each (request by binary search over
//                            the running sum of prefix lengths held in LDS, source and destination
//                            slot, new index), then every lane moves nine 16-byte pieces of those
//                            8 x 1152 bytes, all nine loads issued before the first store. Loads and
//                            stores are non-temporal: each byte is touched once.
//
// The work is one read and one write of each 1152-byte row: bound by HBM bandwidth.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mla_kv_compact.h"

namespace {

constexpr int kCheckThreads = 1024;
constexpr int kCopyThreads = 256;
constexpr int kCopyWaves = kCopyThreads / 64;
constexpr int kCopyBlocksFallback = 2048;  // grid when the occupancy query fails
constexpr int kRowBytes = MLA_VERIFY_ROW * 2;
constexpr int kPiecesPerRow = kRowBytes / 16;  // 72 sixteen-byte pieces
constexpr int kRowsPerStep = 8;
constexpr int kPiecesPerLane = kRowsPerStep * kPiecesPerRow / 64;  // 9
static_assert(kRowsPerStep * kPiecesPerRow % 64 == 0, "a step is a whole number of pieces per lane");

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte piece, kept in VGPRs

__device__ __forceinline__ long long prefix_len(const int32_t* kv_indptr, int b) {
  const long long p = (long long)kv_indptr[b + 1] - (long long)kv_indptr[b];
  return p > 0 ? p : 0;
}

__device__ __forceinline__ bool run_fits(long long d0, long long P, long long N) {
  return P == 0 || (d0 >= 0 && d0 + P <= N);
}

__global__ __launch_bounds__(kCheckThreads) void kv_compact_check_kernel(const int32_t* __restrict__ kv_indptr,
                                                                         const int32_t* __restrict__ dst_start,
                                                                         int B, long long N,
                                                                         int32_t* __restrict__ status) {
  int bad = 0;
  for (int b = threadIdx.x; b < B; b += kCheckThreads)
    bad |= !run_fits(dst_start[b], prefix_len(kv_indptr, b), N);
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) *status = bad ? MLA_COMPACT_BAD_DST : 0;
}

__global__ __launch_bounds__(kCopyThreads) void kv_compact_kernel(uint8_t* __restrict__ pool, long long N,
                                                                  const int32_t* __restrict__ kv_indptr,
                                                                  const int32_t* __restrict__ kv_indices,
                                                                  const int32_t* __restrict__ dst_start, int B,
                                                                  int32_t* __restrict__ new_kv_indices,
                                                                  int32_t* __restrict__ status) {
  extern __shared__ long long first_row[];  // [B + 1]: running sum of the prefix lengths
  __shared__ long long wave_tot[kCopyWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long carry = 0;
  if (tid == 0) first_row[0] = 0;
  for (int b0 = 0; b0 < B; b0 += kCopyThreads) {
    const int b = b0 + tid;
    long long x = b < B ? prefix_len(kv_indptr, b) : 0;
    for (int d = 1; d < 64; d <<= 1) {
      const long long y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    long long before = 0, chunk_tot = 0;
    for (int w = 0; w < kCopyWaves; ++w) {
      const long long t = wave_tot[w];
      if (w < wave) before += t;
      chunk_tot += t;
    }
    if (b < B) first_row[b + 1] = carry + before + x;
    carry += chunk_tot;
    __syncthreads();
  }
  const long long total = first_row[B];

  for (long long v0 = ((long long)blockIdx.x * kCopyWaves + wave) * kRowsPerStep; v0 < total;
       v0 += (long long)gridDim.x * kCopyWaves * kRowsPerStep) {
    // lanes 0..7: one row each
    int src = -1, dst = -1;
    if (lane < kRowsPerStep && v0 + lane < total) {
      const long long v = v0 + lane;
      int lo = 0, hi = B;  // the last b with first_row[b] <= v (requests with P_b = 0 are skipped)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (first_row[mid] <= v) lo = mid; else hi = mid;
      }
      const int b = lo;
      const long long j = v - first_row[b];
      const long long t = (long long)kv_indptr[b] + j;
      const int s = kv_indices[t];
      const long long d0 = dst_start[b];
      int keep = s;
      if (run_fits(d0, prefix_len(kv_indptr, b), N)) {
        if (s >= 0 && s < N) {
          src = s;
          dst = (int)(d0 + j);
          keep = dst;
        } else {
          atomicOr(status, MLA_COMPACT_BAD_SRC);
        }
      }
      new_kv_indices[t] = keep;
    }
    // Every lane loads all nine pieces (a row that is not moved reads row 0 instead, which always
    // exists), so the loads stay unconditional and in registers; only the stores are predicated.
    u32x4 piece[kPiecesPerLane];
    int dst_of[kPiecesPerLane], part_of[kPiecesPerLane];
#pragma unroll
    for (int q = 0; q < kPiecesPerLane; ++q) {
      const int p = lane + 64 * q;
      const int r = p / kPiecesPerRow;
      part_of[q] = p - r * kPiecesPerRow;
      const int s = __shfl(src, r, 64);
      dst_of[q] = __shfl(dst, r, 64);
      piece[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pool + (size_t)(s >= 0 ? s : 0) * kRowBytes) +
                                            part_of[q]);
    }
#pragma unroll
    for (int q = 0; q < kPiecesPerLane; ++q)
      if (dst_of[q] >= 0)
        __builtin_nontemporal_store(piece[q], reinterpret_cast<u32x4*>(pool + (size_t)dst_of[q] * kRowBytes) + part_of[q]);
  }
}

}  // namespace

extern "C" int mla_verify_kv_compact(void* kv_pool, int64_t N, const int32_t* kv_indptr, const int32_t* kv_indices,
                                     const int32_t* dst_start, int B, int32_t* new_kv_indices, int32_t* status,
                                     hipStream_t stream) {
  if (!kv_pool || !kv_indptr || !kv_indices || !dst_start || !new_kv_indices || !status) return MLA_VERIFY_ERR_NULL;
  if (B < 1 || B > MLA_COMPACT_MAX_B || N < 1 || N > INT32_MAX || ((uintptr_t)kv_pool & 15) != 0)
    return MLA_VERIFY_ERR_SHAPE;
  hipLaunchKernelGGL(kv_compact_check_kernel, dim3(1), dim3(kCheckThreads), 0, stream, kv_indptr, dst_start, B,
                     (long long)N, status);
  if (hipGetLastError() != hipSuccess) return MLA_VERIFY_ERR_LAUNCH;
  // One wave of resident workgroups (the grid-stride loop spreads the rows evenly); a larger grid
  // leaves a partly filled last wave of workgroups that costs as much as a full one.
  const size_t lds = (B + 1) * sizeof(long long);
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kv_compact_kernel, kCopyThreads, lds) != hipSuccess) {
    (void)hipGetLastError();  // a failed query must not read as a failed launch below
    cus = per_cu = 0;
  }
  const int grid = (cus > 0 && per_cu > 0) ? cus * per_cu : kCopyBlocksFallback;
  hipLaunchKernelGGL(kv_compact_kernel, dim3(grid), dim3(kCopyThreads), lds, stream,
                     static_cast<uint8_t*>(kv_pool), (long long)N, kv_indptr, kv_indices, dst_start, B,
                     new_kv_indices, status);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}
