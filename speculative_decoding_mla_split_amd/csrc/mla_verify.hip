// Tree-verify attention over an MLA paged KV cache for MI355X (gfx950, CDNA4).
//
// Split-KV flash-decode in two kernels ("The Custom sm_120 Verify Kernel", section "Building the
// Custom Kernel": every workgroup handles one contiguous column slice and writes partial online
// softmax statistics to global scratch; a second kernel combines the partials):
//
//   verify_partial_kernel  one workgroup per (request, split, 128-row tile). The 576-wide bf16 KV
//                          rows of the split are gathered through the two index arrays straight
//                          into LDS with 16-byte direct-to-LDS loads (three-deep ring of 32-row
//                          tiles), shared by all 128 query rows (4 waves x 32 rows). QK^T and PV
//                          run on 32x32x16 bf16 MFMA with fp32 accumulation; the mask lookup and
//                          online softmax happen in registers between the two.
//   verify_combine_kernel  one wave per query row: log-sum-exp combine of the nsplit partials into
//                          the bf16 output and the fp32 natural-log LSE.
//
// Layout conventions of the partial kernel (per wave, 32 query rows r, columns c of one tile):
//   S^T[c][r] = K[c][:] . Q[r][:]  (A = K from LDS, B = Q resident in VGPRs)
//   O^T[e][r] += V^T[e][c] . P^T[c][r]  (A = V^T via ds_read_b64_tr_b16, B = P^T from registers)
// so each lane holds one query row (lane % 32) for both S^T and O^T, and the softmax statistics and
// the rescale factor never leave the lane (only the lane pair l, l^32 shares a row).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "mla_verify.h"

namespace {

constexpr int kLatent = MLA_VERIFY_LATENT;
constexpr int kRope = MLA_VERIFY_ROPE;
constexpr int kRowBytes = MLA_VERIFY_ROW * 2;  // 1152
constexpr int kChunks = kRowBytes / 16;        // 72 sixteen-byte chunks per KV row
constexpr int kTile = 32;                      // KV columns per LDS tile
constexpr int kPairs = 2;                      // wave pairs per workgroup
constexpr int kWaves = 2 * kPairs;
constexpr int kRowsPerPair = 32;
constexpr int kRowsPerWG = kPairs * kRowsPerPair;        // 64
constexpr int kBufs = 3;                                 // LDS ring depth
constexpr int kTileBytes = kTile * kRowBytes;            // 36864
constexpr int kLoaders = 4;                              // waves that gather KV rows
constexpr int kRowsPerLoader = kTile / kLoaders;         // 8
constexpr int kLoadsPerWave = kRowsPerLoader * kChunks / 64;  // 9 direct-to-LDS loads
constexpr int kHalfSteps = (kLatent + kRope) / 32;       // 18 k-steps of 16 per half of the row
constexpr int kHalfEBlocks = kLatent / 64;               // 8 blocks of 32 output columns per half
constexpr int kXchgBytes = 64 * 16 * 4;                  // one wave's 32x32 fp32 partial scores
constexpr int kMaskPairs = 2;                            // token pairs of mask bits prefetched
constexpr float kRescaleSlack = 8.0f;                    // lazy rescale threshold (log2 units)

static_assert(kRowsPerLoader * kChunks % 64 == 0, "loader must tile whole wave instructions");
static_assert(kWaves >= kLoaders, "not enough waves to gather a tile");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// XOR swizzle of the 16-byte chunks of an LDS KV row: chunk k of tile row c is stored at chunk
// k ^ swz(c). It spreads the 32-row K-operand reads and the 8-row transposed V reads over all
// LDS banks; the XOR only touches chunk bits 1-2, so a chunk stays inside its aligned group of 8.
__device__ __forceinline__ int swz(int c) { return ((c >> 1) & 3) << 1; }

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

struct Split {
  int b, s, rt;
  bool valid;
};

// Workgroup id -> (request, split, row tile). Consecutive ids are dispatched round-robin over the
// 8 XCDs; this mapping gives each XCD a contiguous range of units, so the row tiles of one split
// (which read the same KV rows) run on the same XCD and share its L2.
__device__ __forceinline__ Split decode_unit(int B, int nsplit, int n_rt) {
  const int units = B * nsplit * n_rt;
  const int per_xcd = (units + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  Split sp;
  sp.valid = u < units;
  sp.rt = u % n_rt;
  sp.s = (u / n_rt) % nsplit;
  sp.b = u / (n_rt * nsplit);
  return sp;
}

// Partial kernel. Wave pair p owns 32 query rows; its wave h (0/1) holds the query values of the
// row half d in [288h, 288h + 288) and the output columns e in [256h, 256h + 256). Per 32-column
// tile each wave computes the partial scores of its half, the pair swaps them through LDS, both
// waves run the same online softmax on the summed scores, and each updates its output half.
__global__ void __launch_bounds__(kWaves * 64, 1)
verify_partial_kernel(const __bf16* __restrict__ q_nope, const __bf16* __restrict__ q_rope,
                      const uint8_t* __restrict__ kv_pool, int N,
                      const int32_t* __restrict__ kv_indptr, const int32_t* __restrict__ kv_indices,
                      const int32_t* __restrict__ out_cache_loc,
                      const uint8_t* __restrict__ custom_mask,
                      const int32_t* __restrict__ mask_indptr, int B, int q_len, int H,
                      float scale_log2, int nsplit, int n_rt, float2* __restrict__ ws_ml,
                      float* __restrict__ ws_acc) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_kv[kBufs * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_x[kWaves * kXchgBytes];

  const int lane = threadIdx.x & 63;
  const int w = wave_uniform(threadIdx.x >> 6);
  const int pr_id = w >> 1, hf = w & 1;
  const Split sp = decode_unit(B, nsplit, n_rt);
  if (!sp.valid) return;
  const int b = sp.b, s = sp.s;
  const int R = q_len * H;

  // ---- split bounds from the actual lengths (empty splits leave at once)
  const int kv_start = kv_indptr[b];
  const int P = max(kv_indptr[b + 1] - kv_start, 0);
  const int L = P + q_len;
  int chunk = (L + nsplit - 1) / nsplit;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  const int c_begin = s * chunk;
  const int c_end = min(L, c_begin + chunk);

  const int g = lane >> 5;  // k-group of the MFMA operands
  const int row0 = sp.rt * kRowsPerWG + pr_id * kRowsPerPair;
  const int my_row = row0 + (lane & 31);
  const bool row_ok = my_row < R;
  const size_t part = ((size_t)b * nsplit + s) * R;

  if (c_begin >= c_end) {
    if (row_ok && g == 0 && hf == 0) ws_ml[part + my_row] = make_float2(-INFINITY, 0.0f);
    return;
  }
  const bool pair_has_rows = row0 < R;

  // ---- this wave's half of the query row as MFMA B operands: k-step ks holds
  // Q[row][288 hf + 16 ks + 8 g .. +8] (rows past R load row R-1 and are zeroed)
  bf16x8 q[kHalfSteps];
  {
    const int q_row = min(my_row, R - 1);
    const bf16x8* qn = reinterpret_cast<const bf16x8*>(q_nope + ((size_t)b * R + q_row) * kLatent);
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(q_rope + ((size_t)b * R + q_row) * kRope);
#pragma unroll
    for (int ks = 0; ks < kHalfSteps; ++ks) {
      const int chunk8 = 36 * hf + 2 * ks + g;  // 8-value chunk of the 576-wide row
      const bf16x8 v = chunk8 < kLatent / 8 ? qn[chunk8] : qr[chunk8 - kLatent / 8];
      q[ks] = row_ok ? v : bf16x8{};
    }
  }

  // ---- gather: loader wave w (< 4) loads tile rows [8w, 8w+8); instruction j of the 9 covers LDS
  // chunks [64j, 64j+64) of those rows, lane t -> chunk p = 64j+t of row p/72, read from logical
  // chunk (p % 72) ^ swz(p / 72) of that row (swz(8w + rho) == swz(rho)).
  const bool loader = w < kLoaders;
  auto load_slot = [&](int tile_c0) -> int {
    int c = min(tile_c0 + (w % kLoaders) * kRowsPerLoader + (lane & 7), c_end - 1);
    int slot = c < P ? kv_indices[kv_start + c] : out_cache_loc[(size_t)b * q_len + (c - P)];
    return min(max(slot, 0), N - 1);
  };
  auto issue_kv = [&](int slotv, int buf) {
    uint8_t* dst = lds_kv + buf * kTileBytes + w * kRowsPerLoader * kRowBytes;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // keep the per-lane offsets inside the loop (register pressure)
#pragma unroll
    for (int j = 0; j < kLoadsPerWave; ++j) {
      const int lo = (64 * j) / kChunks;
      const int boundary = kChunks * (lo + 1) - 64 * j;
      const int s_lo = __builtin_amdgcn_readlane(slotv, lo);
      const int s_hi = __builtin_amdgcn_readlane(slotv, lo + 1 < 8 ? lo + 1 : 7);
      const bool first = ln < boundary;
      const int slot = first ? s_lo : s_hi;
      const int pc = first ? 64 * j + ln - kChunks * lo : 64 * j + ln - kChunks * (lo + 1);
      const int off = (pc ^ swz(first ? lo : lo + 1)) * 16;
      const uint8_t* src = kv_pool + (size_t)(uint32_t)slot * kRowBytes + off;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + j * 1024), 16, 0, 0);
    }
  };

  // ---- tree-mask bits: the pair's rows span tokens [tok_first, tok_last]; one byte load per lane
  // covers two tokens x 32 columns and a ballot turns it into two 32-bit visibility words.
  const size_t mask_base = (size_t)mask_indptr[b];
  const int tok_first = row0 / H;
  const int tok_last = (min(row0 + kRowsPerPair, R) - 1) / H;
  const int my_tok = my_row / H;
  const int my_pair = (my_tok - tok_first) >> 1, my_half = (my_tok - tok_first) & 1;
  const int n_tok_pairs = pair_has_rows ? (tok_last - tok_first + 2) >> 1 : 0;
  auto mask_byte = [&](int tile_c0, int tp) -> int {
    const int t = tok_first + 2 * tp + g;
    const int c = tile_c0 + (lane & 31);
    int v = 0;
    if (t <= tok_last && c < c_end) v = custom_mask[mask_base + (size_t)t * L + c];
    return v;
  };
  auto mask_bits = [&](int byte_val, int tp, uint32_t cur) -> uint32_t {
    const uint64_t bal = __ballot(byte_val != 0);
    const uint32_t word = my_half ? (uint32_t)(bal >> 32) : (uint32_t)bal;
    return my_pair == tp ? word : cur;
  };

  // ---- online softmax state (per lane: its row; identical in both waves of the pair)
  f32x16 oacc[kHalfEBlocks];
#pragma unroll
  for (int eb = 0; eb < kHalfEBlocks; ++eb) oacc[eb] = f32x16{};
  float m_ref = -INFINITY;  // reference max in log2 units (may lag the true max by < slack)
  float l_lane = 0.0f;

  // K-operand reads: lane reads tile row (lane & 31), logical chunk 36 hf + 2ks + g, i.e. physical
  // chunk 8(ks/4) + 36 hf + ((2(ks%4) + g) ^ swz(row)) (36 hf is a multiple of 4 but not of 8,
  // so it is added outside the XOR only for hf = 0; hf = 1 handles the odd group below).
  const int k_row = lane & 31;
  // transposed V reads: the 16-lane group G reads tile rows 16kk + 8m + 4(G/2) + (k16/4), m = 0, 1,
  // latent columns 32eb + 16(G%2) + 4(k16%4) .. +3; physical chunk 8(eb/2) + ((4(eb%2) + vc) ^ swz).
  const int k16 = lane & 15, G = lane >> 4;
  const int v_row = 4 * (G >> 1) + (k16 >> 2);
  const int v_chunk = 2 * (G & 1) + ((k16 & 3) >> 1);
  int v_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    v_off[par] = v_row * kRowBytes + (((4 * par + v_chunk) ^ swz(v_row)) * 16) + (k16 & 1) * 8;
  uint8_t* const x_mine = lds_x + w * kXchgBytes + lane * 16;
  const uint8_t* const x_other = lds_x + (w ^ 1) * kXchgBytes + lane * 16;

  const int ntiles = (c_end - c_begin + kTile - 1) / kTile;

  // ---- prologue: KV of tiles 0 and 1 in flight, slots of tile 2 and mask bytes of tile 0 loaded
  int slot_c = 0;
  int mbyte_cur[kMaskPairs], mbyte_nxt[kMaskPairs];
#pragma unroll
  for (int tp = 0; tp < kMaskPairs; ++tp) mbyte_cur[tp] = tp < n_tok_pairs ? mask_byte(c_begin, tp) : 0;
  if (loader) {
    const int slot_a = load_slot(c_begin);
    const int slot_b = load_slot(c_begin + kTile);
    issue_kv(slot_a, 0);
    if (ntiles > 1) issue_kv(slot_b, 1);
    slot_c = load_slot(c_begin + 2 * kTile);
  }

  for (int t = 0; t < ntiles; ++t) {
    const int tile_c0 = c_begin + t * kTile;
    // wait until this wave's loads of tile t have landed: only tile t+1's 9 loads may remain
    if (loader && t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt((kLoadsPerWave & 0xF) | (0x7 << 4) | (0xF << 8));
    } else {
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
    }
    __syncthreads();  // tile t is in LDS; buffer (t+2)%3 and the score exchange are free again

    // prefetch: mask bytes of tile t+1, KV rows of tile t+2, slots of tile t+3
#pragma unroll
    for (int tp = 0; tp < kMaskPairs; ++tp)
      mbyte_nxt[tp] = (tp < n_tok_pairs && t + 1 < ntiles) ? mask_byte(tile_c0 + kTile, tp) : 0;
    int slot_d = 0;
    if (loader) {
      if (t + 2 < ntiles) issue_kv(slot_c, (t + 2) % kBufs);
      slot_d = load_slot(tile_c0 + 3 * kTile);
    }

    const uint8_t* kb = lds_kv + (t % kBufs) * kTileBytes;
    // partial scores S^T = K[:, half] . Q[:, half]^T
    f32x16 sacc = {};
    if (pair_has_rows) {
      const uint8_t* krow = kb + k_row * kRowBytes;
      const int ksw = swz(k_row);
#pragma unroll
      for (int ks = 0; ks < kHalfSteps; ++ks) {
        const int logical = 36 * hf + 2 * ks + g;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + ((logical ^ ksw) * 16));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[ks], sacc, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<f32x4*>(x_mine + k * 1024) = f32x4{sacc[4 * k], sacc[4 * k + 1], sacc[4 * k + 2], sacc[4 * k + 3]};
    }
    __syncthreads();  // both halves of every pair's scores are in LDS

    if (pair_has_rows) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(x_other + k * 1024);
        // the same addition order in both waves keeps their softmax states bit-identical
#pragma unroll
        for (int j = 0; j < 4; ++j) sacc[4 * k + j] = hf ? o[j] + sacc[4 * k + j] : sacc[4 * k + j] + o[j];
      }
      // visibility word of this lane's row for the 32 columns of the tile
      uint32_t bits = 0;
#pragma unroll
      for (int tp = 0; tp < kMaskPairs; ++tp) bits = mask_bits(mbyte_cur[tp], tp, bits);
      for (int tp = kMaskPairs; tp < n_tok_pairs; ++tp) bits = mask_bits(mask_byte(tile_c0, tp), tp, bits);

      // mask + online softmax; element i of sacc is column 8(i/4) + 4g + i%4 of the tile
      float v[16];
      float mx = -INFINITY;
      const uint32_t bsh = bits >> (4 * g);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        v[i] = ((bsh >> (8 * (i >> 2) + (i & 3))) & 1u) ? sacc[i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, v[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool need = mx > m_ref + kRescaleSlack;
      if (__any(need)) {
        const float new_ref = need ? mx : m_ref;
        const float alpha = !need ? 1.0f : (m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - new_ref));
#pragma unroll
        for (int eb = 0; eb < kHalfEBlocks; ++eb) oacc[eb] *= alpha;
        l_lane *= alpha;
        m_ref = new_ref;
      }
      const float base = m_ref == -INFINITY ? 0.0f : m_ref;
      bf16x8 pb[2];
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(v[i] - base);
        psum += p;
        pb[i >> 3][i & 7] = (__bf16)p;
      }
      l_lane += psum;

      // O^T[e half] += V^T . P^T; k-step kk covers tile columns [16kk, 16kk+16) permuted as
      // logical k = 8g + j  <->  column 16kk + 4g + j (j < 4), 16kk + 8 + 4g + (j - 4) (j >= 4)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int eb = 0; eb < kHalfEBlocks; ++eb) {
          const int geb = kHalfEBlocks * hf + eb;  // global block of 32 output columns
          const uint8_t* p0 = kb + v_off[geb & 1] + 128 * (geb >> 1) + 16 * kk * kRowBytes;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * kRowBytes));
          const bf16x4 lo4 = __builtin_bit_cast(bf16x4, lo), hi4 = __builtin_bit_cast(bf16x4, hi);
          const bf16x8 a = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          oacc[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], oacc[eb], 0, 0, 0);
        }
      }
    }

    // rotate the prefetch registers
#pragma unroll
    for (int tp = 0; tp < kMaskPairs; ++tp) mbyte_cur[tp] = mbyte_nxt[tp];
    slot_c = slot_d;
  }

  // ---- partial write: (m_ref, l) and this wave's half of the unnormalised accumulator
  const float l_row = l_lane + __shfl_xor(l_lane, 32);
  if (row_ok) {
    float* dst = ws_acc + (part + my_row) * kLatent + 256 * hf;
#pragma unroll
    for (int eb = 0; eb < kHalfEBlocks; ++eb) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 val = {oacc[eb][4 * a], oacc[eb][4 * a + 1], oacc[eb][4 * a + 2], oacc[eb][4 * a + 3]};
        *reinterpret_cast<f32x4*>(dst + 32 * eb + 8 * a + 4 * g) = val;
      }
    }
    if (g == 0 && hf == 0) ws_ml[part + my_row] = make_float2(m_ref, l_row);
  }
}

// One wave per query row (b, r): weights w_s = 2^(m_s - M) over the non-empty partials,
// out = sum w_s acc_s / sum w_s l_s, lse = (M + log2 sum w_s l_s) * ln 2.
__global__ void __launch_bounds__(256)
verify_combine_kernel(const float2* __restrict__ ws_ml, const float* __restrict__ ws_acc, int B, int R,
                      int nsplit, __bf16* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);  // global row index b*R + r
  if (row >= (long)B * R) return;
  const long b = row / R, r = row % R;
  const float2* ml = ws_ml + (size_t)b * nsplit * R + r;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[(size_t)s * R].x);
  bf16x8* o = reinterpret_cast<bf16x8*>(out + (size_t)row * kLatent + lane * 8);
  if (M == -INFINITY) {
    *o = bf16x8{};
    if (lane == 0) lse[row] = -INFINITY;
    return;
  }
  float acc[8] = {};
  float den = 0.0f;
  for (int s = 0; s < nsplit; ++s) {
    const float2 st = ml[(size_t)s * R];
    if (st.x == -INFINITY) continue;  // empty or fully masked split: weight 0, accumulator unused
    const float wgt = exp2f(st.x - M);
    den += wgt * st.y;
    const f32x4* src = reinterpret_cast<const f32x4*>(ws_acc + ((size_t)(b * nsplit + s) * R + r) * kLatent + lane * 8);
    const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[k] += wgt * x0[k];
      acc[4 + k] += wgt * x1[k];
    }
  }
  const float inv = 1.0f / den;
  bf16x8 res;
#pragma unroll
  for (int k = 0; k < 8; ++k) res[k] = (__bf16)(acc[k] * inv);
  *o = res;
  if (lane == 0) lse[row] = (M + log2f(den)) * 0.69314718055994530942f;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WorkspaceLayout {
  size_t ml_bytes, acc_bytes;
};

WorkspaceLayout workspace_layout(int B, int q_len, int H, int nsplit) {
  const size_t rows = (size_t)B * nsplit * q_len * H;
  return {align_up(rows * sizeof(float2), MLA_VERIFY_WORKSPACE_ALIGN),
          align_up(rows * kLatent * sizeof(float), MLA_VERIFY_WORKSPACE_ALIGN)};
}

bool sizes_ok(int B, int q_len, int H) {
  if (B < 1 || q_len < 1 || H < 1) return false;
  const long long rows = (long long)q_len * H;
  return rows <= (1LL << 24) && (long long)B * rows <= (1LL << 30);
}

}  // namespace

extern "C" size_t mla_verify_attn_workspace_size(int B, int q_len, int H, int nsplit) {
  if (!sizes_ok(B, q_len, H) || nsplit < 1 || nsplit > MLA_VERIFY_MAX_NSPLIT) return 0;
  const WorkspaceLayout lay = workspace_layout(B, q_len, H, nsplit);
  return lay.ml_bytes + lay.acc_bytes;
}

extern "C" const char* mla_verify_status_string(int status) {
  switch (status) {
    case MLA_VERIFY_OK: return "ok";
    case MLA_VERIFY_ERR_NULL: return "a required pointer is NULL";
    case MLA_VERIFY_ERR_SHAPE: return "B, q_len, H or N out of range, or scale not finite";
    case MLA_VERIFY_ERR_NSPLIT: return "nsplit outside [1, 1024]";
    case MLA_VERIFY_ERR_WORKSPACE: return "workspace NULL, misaligned or too small";
    case MLA_VERIFY_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

namespace {

struct Launch {
  float2* ws_ml;
  float* ws_acc;
  int R;
};

int check_common(int B, int q_len, int H, int nsplit, const void* workspace, size_t workspace_bytes) {
  if (!sizes_ok(B, q_len, H)) return MLA_VERIFY_ERR_SHAPE;
  if (nsplit < 1 || nsplit > MLA_VERIFY_MAX_NSPLIT) return MLA_VERIFY_ERR_NSPLIT;
  const size_t need = mla_verify_attn_workspace_size(B, q_len, H, nsplit);
  if (!workspace || ((uintptr_t)workspace % MLA_VERIFY_WORKSPACE_ALIGN) != 0 || workspace_bytes < need)
    return MLA_VERIFY_ERR_WORKSPACE;
  return MLA_VERIFY_OK;
}

Launch split_workspace(void* workspace, int B, int q_len, int H, int nsplit) {
  const WorkspaceLayout lay = workspace_layout(B, q_len, H, nsplit);
  return {static_cast<float2*>(workspace),
          reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + lay.ml_bytes), q_len * H};
}

int launch_partial(const void* q_nope, const void* q_rope, const void* kv_pool, int64_t N,
                   const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* out_cache_loc,
                   const uint8_t* custom_mask, const int32_t* mask_indptr, int B, int q_len, int H,
                   float scale, int nsplit, const Launch& ws, hipStream_t stream) {
  const int n_rt = (ws.R + kRowsPerWG - 1) / kRowsPerWG;
  const long long units = (long long)B * nsplit * n_rt;
  const long long grid = (units + 7) / 8 * 8;
  if (grid > INT32_MAX) return MLA_VERIFY_ERR_SHAPE;
  const float scale_log2 = scale * 1.44269504088896340736f;
  hipLaunchKernelGGL(verify_partial_kernel, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream,
                     static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(q_rope),
                     static_cast<const uint8_t*>(kv_pool), (int)N, kv_indptr, kv_indices, out_cache_loc,
                     custom_mask, mask_indptr, B, q_len, H, scale_log2, nsplit, n_rt, ws.ws_ml, ws.ws_acc);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

int launch_combine(const Launch& ws, int B, int nsplit, void* out, float* lse, hipStream_t stream) {
  const long long crows = (long long)B * ws.R;
  hipLaunchKernelGGL(verify_combine_kernel, dim3((unsigned)((crows + 3) / 4)), dim3(256), 0, stream, ws.ws_ml,
                     ws.ws_acc, B, ws.R, nsplit, static_cast<__bf16*>(out), lse);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

bool inputs_null(const void* q_nope, const void* q_rope, const void* kv_pool, const int32_t* kv_indptr,
                 const int32_t* out_cache_loc, const uint8_t* custom_mask, const int32_t* mask_indptr) {
  return !q_nope || !q_rope || !kv_pool || !kv_indptr || !out_cache_loc || !custom_mask || !mask_indptr;
}

}  // namespace

extern "C" int mla_verify_attn_partial(const void* q_nope, const void* q_rope, const void* kv_pool, int64_t N,
                                       const int32_t* kv_indptr, const int32_t* kv_indices,
                                       const int32_t* out_cache_loc, const uint8_t* custom_mask,
                                       const int32_t* mask_indptr, int B, int q_len, int H, float scale,
                                       int nsplit, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (inputs_null(q_nope, q_rope, kv_pool, kv_indptr, out_cache_loc, custom_mask, mask_indptr))
    return MLA_VERIFY_ERR_NULL;
  if (!sizes_ok(B, q_len, H) || N < 1 || N > INT32_MAX || !isfinite(scale)) return MLA_VERIFY_ERR_SHAPE;
  const int rc = check_common(B, q_len, H, nsplit, workspace, workspace_bytes);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_partial(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                        B, q_len, H, scale, nsplit, split_workspace(workspace, B, q_len, H, nsplit), stream);
}

extern "C" int mla_verify_attn_combine(const void* workspace, size_t workspace_bytes, int B, int q_len, int H,
                                       int nsplit, void* out, float* lse, hipStream_t stream) {
  if (!out || !lse) return MLA_VERIFY_ERR_NULL;
  const int rc = check_common(B, q_len, H, nsplit, workspace, workspace_bytes);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_combine(split_workspace(const_cast<void*>(workspace), B, q_len, H, nsplit), B, nsplit, out, lse,
                        stream);
}

extern "C" int mla_verify_attn(const void* q_nope, const void* q_rope, const void* kv_pool, int64_t N,
                               const int32_t* kv_indptr, const int32_t* kv_indices,
                               const int32_t* out_cache_loc, const uint8_t* custom_mask,
                               const int32_t* mask_indptr, int B, int q_len, int H, float scale,
                               int nsplit, void* workspace, size_t workspace_bytes, void* out, float* lse,
                               hipStream_t stream) {
  if (inputs_null(q_nope, q_rope, kv_pool, kv_indptr, out_cache_loc, custom_mask, mask_indptr) || !out || !lse)
    return MLA_VERIFY_ERR_NULL;
  if (!sizes_ok(B, q_len, H) || N < 1 || N > INT32_MAX || !isfinite(scale)) return MLA_VERIFY_ERR_SHAPE;
  int rc = check_common(B, q_len, H, nsplit, workspace, workspace_bytes);
  if (rc != MLA_VERIFY_OK) return rc;
  const Launch ws = split_workspace(workspace, B, q_len, H, nsplit);
  rc = launch_partial(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr, B,
                      q_len, H, scale, nsplit, ws, stream);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_combine(ws, B, nsplit, out, lse, stream);
}
