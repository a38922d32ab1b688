// Tree-verify attention over an MLA paged KV cache for MI355X (gfx950, CDNA4).
//
// Split-KV flash-decode in two kernels ("The Custom sm_120 Verify Kernel", section "Building the
// Custom Kernel": every workgroup handles one contiguous column slice and writes partial online
// softmax statistics to global scratch; a second kernel combines the partials):
//
//   verify_partial_kernel  one workgroup per (request, split, 128-row tile). The 576-wide bf16 KV
//                          rows of the split are gathered through the two index arrays straight
//                          into LDS with 16-byte direct-to-LDS loads (three-deep ring of 32-row
//                          tiles), shared by all 128 query rows (4 waves x 32 rows). QK^T and
//                          PV run on 32x32x16 bf16 MFMA with fp32 accumulation; the mask lookup
//                          and the softmax of one tile run in registers between the score
//                          products of the next.
//   verify_combine_kernel  log-sum-exp combine of each query row's partials into the bf16 output
//                          and the fp32 natural-log LSE (one, four or, below 512 rows, a quarter
//                          row per workgroup).
//
// Layout conventions of the partial kernel (per MFMA block of 32 query rows r, columns c of one
// tile):
//   S^T[c][r] = K[c][:] . Q[r][:]  (A = K from LDS, B = Q resident in VGPRs)
//   O^T[e][r] += V^T[e][c] . P^T[c][r]  (A = V^T via ds_read_b64_tr_b16, B = P^T from registers)
// so each lane holds one query row (lane % 32) for both S^T and O^T, and the softmax statistics
// never leave the lane (only the lane pair l, l^32 shares a row). A wave scores its block over the
// whole row and accumulates the block's whole 512-wide output, so the four waves exchange nothing
// but the KV tiles they load together.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "mla_verify.h"

namespace {

constexpr int kLatent = MLA_VERIFY_LATENT;
constexpr int kRope = MLA_VERIFY_ROPE;
constexpr int kRowBytes = MLA_VERIFY_ROW * 2;  // 1152
constexpr int kChunks = kRowBytes / 16;        // 72 sixteen-byte chunks per KV row
constexpr int kTile = 32;                      // KV columns per LDS tile
constexpr int kWaves = 4;                      // waves per workgroup, one 32-row block each
constexpr int kBlockRows = 32;                 // query rows per MFMA block (one lane per row)
constexpr int kRowsPerWG = kWaves * kBlockRows;          // 128
constexpr int kBufs = 3;                                 // LDS ring depth
// LDS tile layout. Loader wave w owns tile rows [8w, 8w+8) in region w; a region holds 9 groups
// (16-byte chunks 8j .. 8j+7 of all its 8 rows, 128 bytes per row), so one direct-to-LDS
// instruction fills one group. Regions are 9344 bytes apart (9216 + 128): the 128-byte shift
// puts row c and row c+8 on opposite halves of the 64 LDS banks.
constexpr int kGroupBytes = 1024;
constexpr int kRegionBytes = 9 * kGroupBytes + 128;      // 9344
constexpr int kTileBytes = 4 * kRegionBytes;             // 37376
constexpr int kLoaders = 4;                              // waves that gather KV rows
constexpr int kRowsPerLoader = kTile / kLoaders;         // 8
constexpr int kLoadsPerWave = kRowsPerLoader * kChunks / 64;  // 9 direct-to-LDS loads
constexpr int kSteps = (kLatent + kRope) / 16;           // 36 k-steps of 16 over the 576-wide row
constexpr int kRegSteps = kLatent / 16;                  // 32 of them (the latent part) keep Q in VGPRs
constexpr int kQRopeBytes = (kSteps - kRegSteps) * 64 * 16;  // a wave's rope Q operands in LDS (4 KB)
constexpr int kEBlocks = kLatent / 32;                   // 16 blocks of 32 output columns
constexpr float kHeadroom = 64.0f;  // scores may exceed a row's reference max by this (log2 units)
// Per-tile metadata of one wave, all through byte-granular direct-to-LDS loads (each byte lands
// zero-extended in its own dword): load 0 carries the 4 bytes of each of the 8 slot indices of the
// rows this wave gathers (lanes 0-31) and the 32 mask bytes of the first token of the wave's row
// block (lanes 32-63); extra load k carries two more tokens (1 + 2k, 2 + 2k). A 32-row block
// spans 1 token for H >= 32, so most configurations need a single metadata load per tile.
constexpr int kMetaExtra = 2;                    // extra mask loads at most (block tokens <= 5)
constexpr int kMetaTokens = 1 + 2 * kMetaExtra;  // block tokens whose mask bytes ride in LDS
constexpr int kMetaBytes = 256 * (1 + kMetaExtra);
constexpr int kMetaStages = 8;                   // per-wave ring of per-tile metadata
constexpr int kLdsBytes = kBufs * kTileBytes + kWaves * (kMetaStages * kMetaBytes + kQRopeBytes);

static_assert(kRowsPerLoader * kChunks % 64 == 0, "loader must tile whole wave instructions");
static_assert(kWaves == kLoaders, "every wave gathers a share of each tile");
static_assert(kLdsBytes + 64 <= 160 * 1024, "LDS budget of one CU");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = B .. E-1, so code that branches on
// the index (which softmax piece or load goes between which matrix products) is resolved while
// compiling rather than left to the optimiser after unrolling.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// XOR swizzle inside a group: logical chunk k of tile row c sits in slot (k % 8) ^ swz(c) of group
// k / 8, with swz a permutation of the three low bits of the row (bit 1 of c drives bit 2 of the
// slot). Bank of a 16-byte slot (64 banks of 4 bytes): 8 ((c / 8 + c) & 1) + ((k % 8) ^ swz(c)) in
// units of 4 banks, the first term from the 128-byte row stride and the regions' 128-byte shift.
//  - K operand reads (16 B per lane, 16 lanes a cycle: one chunk of 16 consecutive rows) hit 16
//    different slots for any swz that is a bijection of c % 8.
//  - V^T operand reads (ds_read_b64_tr_b16, 32 lanes a cycle: chunks 4 eb .. 4 eb + 3 of rows
//    c0 .. c0 + 3, c0 % 4 == 0) need rows c0 and c0 + 2 (same half of the banks) in disjoint slot
//    sets, i.e. swz(c0) ^ swz(c0 + 2) with bit 2 set. Plain c & 7 put both rows on the same four
//    slots: a 2-way conflict on every V read, 4.38e7 conflict cycles per launch at the ragged 185k
//    batch, two per read.
__host__ __device__ constexpr int swz(int c) { return (c & 1) | ((c >> 1 & 1) << 2) | ((c >> 2 & 1) << 1); }

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Byte offset, inside a tile buffer, of logical 16-byte chunk k of tile row c.
__host__ __device__ constexpr int tile_offset(int c, int k) {
  return (c / 8) * kRegionBytes + (k / 8) * kGroupBytes + (c % 8) * 128 + (((k % 8) ^ swz(c)) * 16);
}

// Per-lane parts of the MFMA operand addresses inside a tile, and the parts common to a wave.
// K operand of k-step ks: logical chunk 2 (ks % 4) + g of tile row lane % 32, at k_lane_offset(lane,
// ks % 4) + k_step_offset(ks). V^T operand of output block eb and k-step kk (two transposed 8-byte
// reads, m = 0, 1): the 16-lane group G reads tile rows 16 kk + 8m + 4 (G / 2) + (k16 / 4), latent
// columns 32 eb + 16 (G % 2) + 4 (k16 % 4) .. +3, i.e. logical chunk 4 eb + 2 (G % 2) + (k16 % 4) / 2,
// at v_lane_offset(lane, eb % 2) + v_step_offset(kk, eb, m).
__host__ __device__ constexpr int k_lane_offset(int lane, int b4) { return tile_offset(lane & 31, 2 * b4 + (lane >> 5)); }
__host__ __device__ constexpr int k_step_offset(int ks) { return kGroupBytes * (ks / 4); }
__host__ __device__ constexpr int v_lane_offset(int lane, int half) {
  const int k16 = lane & 15, G = lane >> 4;
  return tile_offset(4 * (G >> 1) + (k16 >> 2), 4 * half + 2 * (G & 1) + ((k16 & 3) >> 1)) + (k16 & 1) * 8;
}
__host__ __device__ constexpr int v_step_offset(int kk, int eb, int m) {
  return 2 * kk * kRegionBytes + kGroupBytes * (eb >> 1) + m * kRegionBytes;
}

// Build-time proof that the operand reads meet no LDS bank conflict, on the bank model of gfx950
// (64 banks of 4 bytes; a 16-byte-per-lane read is served 16 lanes a cycle, a transposed 8-byte read
// 32 lanes a cycle): within each group of lanes served together, no two lanes touch the same bank.
constexpr bool k_reads_conflict_free() {
  for (int ks = 0; ks < kSteps; ++ks)
    for (int l0 = 0; l0 < 64; l0 += 16) {
      bool used[16] = {};
      for (int lane = l0; lane < l0 + 16; ++lane) {
        const int bank16 = ((k_lane_offset(lane, ks % 4) + k_step_offset(ks)) / 16) % 16;
        if (used[bank16]) return false;
        used[bank16] = true;
      }
    }
  return true;
}
constexpr bool v_reads_conflict_free() {
  for (int kk = 0; kk < 2; ++kk)
    for (int eb = 0; eb < kLatent / 32; ++eb)
      for (int m = 0; m < 2; ++m)
        for (int l0 = 0; l0 < 64; l0 += 32) {
          bool used[32] = {};
          for (int lane = l0; lane < l0 + 32; ++lane) {
            const int bank8 = ((v_lane_offset(lane, eb & 1) + v_step_offset(kk, eb, m)) / 8) % 32;
            if (used[bank8]) return false;
            used[bank8] = true;
          }
        }
  return true;
}
static_assert(k_reads_conflict_free(), "K operand reads of the tile layout meet a bank conflict");
static_assert(v_reads_conflict_free(), "transposed V operand reads of the tile layout meet a bank conflict");

// Workgroup barrier for LDS traffic only: waits for this wave's LDS reads and writes, then
// s_barrier. Unlike __syncthreads() it does not drain the vector-memory counter, so direct-to-LDS
// loads of later tiles stay in flight across it (their completion is awaited explicitly with
// s_waitcnt vmcnt before the barrier that publishes them). The "memory" clobber keeps the compiler
// from moving memory accesses across it.
// Direct-to-LDS loads (LDS address = m0 + size * lane; the probed placement on gfx950, sub-dword
// sizes zero-extended into a dword). Written as inline asm so the compiler does not pair them with
// the blanket "wait for every direct-to-LDS load" it would otherwise put in front of each LDS read;
// the kernel waits for them explicitly with s_waitcnt vmcnt. The compiler sets m0 itself before
// any instruction that needs it, so overwriting it here is safe.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)reinterpret_cast<uintptr_t>((lds_void*)p));
}
// Group j of a loader wave's region: global src + 128j -> LDS lds + 1024j (+ 16 * lane). The
// immediate offset is added to both addresses, so m0 is set to lds + 896j. Two address forms: a
// 64-bit address per lane (any pool size), or the pool base in SGPRs plus a 32-bit byte offset per
// lane (pools up to 4 GiB). The second sends half the address bits per instruction, and the
// gather-bound loop is measurably faster with it (ragged 185k batch: 808 -> 797 us).
template <int J>
__device__ __forceinline__ void dma_group(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(g),
               "s"(lds + 896 * J), "i"(128 * J)
               : "memory", "m0");
}
template <int J>
__device__ __forceinline__ void dma_group(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %3 offset:%2" ::"v"(voff),
               "s"(lds + 896 * J), "i"(128 * J), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_u8(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Row max / row sum over the lane pair (l, l ^ 32) through v_permlane32_swap, without an LDS round
// trip. The swap exchanges one wave half of its two operands with the other, so afterwards every
// lane holds its own value and its partner's, one in each result; max and (commutative) addition
// of the two give the same bits in both lanes of the pair.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct Split {
  int b, s, rt;
  bool valid;
};

// Workgroup id -> (request, split, row tile). Consecutive workgroup ids are dispatched round-robin
// over the 8 XCDs. Split sigma = b * nsplit + s goes to XCD sigma % 8 and all its row tiles stay on
// that XCD (they read the same KV rows, so the re-reads hit its L2), while consecutive splits, and
// thus every request, are spread evenly over the XCDs. The grid is 8 * ceil(B * nsplit / 8) * n_rt.
__device__ __forceinline__ Split decode_unit(int B, int nsplit, int n_rt) {
  const int xcd = (int)(blockIdx.x % 8), k = (int)(blockIdx.x / 8);
  const int sigma = xcd + 8 * (k / n_rt);
  Split sp;
  sp.valid = sigma < B * nsplit;
  sp.rt = k % n_rt;
  sp.s = sigma % nsplit;
  sp.b = sigma / nsplit;
  return sp;
}

// Per-wave constants of the partial kernel (request/split bounds, lane roles, LDS offsets).
struct Ctx {
  size_t mask_base;
  int N, b, q_len, kv_start, P, L, c_end;
  int lane, g;
  int loader_row0;
  int tok_first, tok_last, my_pair, my_half, n_tok_pairs;
  bool uniform_token;  // the wave's 32 rows all belong to one draft token (wave-uniform)
  int n_meta;  // metadata loads per tile of this wave: 1 + extra mask loads (wave-uniform)
  float scale_log2;
};

// Metadata loads of one tile into a wave's ring stage m (x.n_meta instructions; PART > 0 is a no-op
// beyond that). Token i of the block lands at m + 128(i + 1) + 4c for column tile_c0 + c; byte j
// of the slot of gather row r at m + 16r + 4j. Addresses are clamped to valid ones.
template <int PART>
__device__ __forceinline__ void issue_meta_part(const Ctx& x, const int32_t* kv_indices, const int32_t* out_cache_loc,
                                                const uint8_t* custom_mask, int tile_c0, uint8_t* m) {
  static_assert(PART >= 0 && PART <= kMetaExtra, "metadata part");
  const int c = min(tile_c0 + (x.lane & 31), x.c_end - 1);
  const uint8_t* mask_row = custom_mask + x.mask_base + c;
  if constexpr (PART == 0) {
    const int cr = min(tile_c0 + x.loader_row0 + ((x.lane & 31) >> 2), x.c_end - 1);
    const int32_t* slot = cr < x.P ? kv_indices + x.kv_start + cr : out_cache_loc + (size_t)x.b * x.q_len + (cr - x.P);
    const uint8_t* src = x.g ? mask_row + (size_t)x.tok_first * x.L
                             : reinterpret_cast<const uint8_t*>(slot) + (x.lane & 3);
    dma_u8(src, lds_addr(m));
  } else {
    if (PART <= x.n_meta - 1) {
      const int t = min(x.tok_first + 2 * PART - 1 + x.g, x.tok_last);
      dma_u8(mask_row + (size_t)t * x.L, lds_addr(m + 256 * PART));
    }
  }
}
__device__ __forceinline__ void issue_meta(const Ctx& x, const int32_t* kv_indices, const int32_t* out_cache_loc,
                                           const uint8_t* custom_mask, int tile_c0, uint8_t* m) {
  issue_meta_part<0>(x, kv_indices, out_cache_loc, custom_mask, tile_c0, m);
  issue_meta_part<1>(x, kv_indices, out_cache_loc, custom_mask, tile_c0, m);
  issue_meta_part<2>(x, kv_indices, out_cache_loc, custom_mask, tile_c0, m);
}
static_assert(kMetaExtra == 2, "issue_meta issues every part");

// Row gather of one tile, split so the 9 loads can be interleaved with MFMA work. Lane t serves row
// t / 8 and slot t % 8 of every group of this wave's region (region loader_row0 / 8 of the tile
// buffer): group j moves logical chunk 8j + ((t % 8) ^ swz(t / 8)) of that row, so the row address is
// computed once and the 9 loads differ only by an immediate offset.
// kWide: 64-bit addresses (src); otherwise base + voff with voff < 2^32 (the host takes the narrow
// form only for pools of at most 2^32 bytes).
struct KvGather {
  const uint8_t* src;
  const uint8_t* base;
  uint32_t voff;
  uint32_t m0;
};
template <bool kWide, int J>
__device__ __forceinline__ void kv_gather_group(const KvGather& k) {
  if constexpr (kWide)
    dma_group<J>(k.src, k.m0);
  else
    dma_group<J>(k.base, k.voff, k.m0);
}
// The four slot bytes of the gather row this lane serves (one per dword in the metadata ring).
__device__ __forceinline__ u32x4 kv_slot_bytes(const Ctx& x, const uint8_t* slots) {
  return *reinterpret_cast<const u32x4*>(slots + 16 * (x.lane >> 3));
}
__device__ __forceinline__ KvGather kv_gather_build(const Ctx& x, const uint8_t* kv_pool, u32x4 sb, uint8_t* dst) {
  const int rho = x.lane >> 3, p = x.lane & 7;
  const int raw_slot = (int)(sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24));
  const int slot = min(max(raw_slot, 0), x.N - 1);
  KvGather k;
  k.voff = (uint32_t)slot * kRowBytes + ((p ^ swz(rho)) * 16);
  k.src = kv_pool + (size_t)(uint32_t)slot * kRowBytes + ((p ^ swz(rho)) * 16);
  k.base = kv_pool;
  k.m0 = lds_addr(dst + (x.loader_row0 / 8) * kRegionBytes);
  return k;
}
__device__ __forceinline__ KvGather kv_gather_setup(const Ctx& x, const uint8_t* kv_pool, const uint8_t* slots,
                                                    uint8_t* dst) {
  return kv_gather_build(x, kv_pool, kv_slot_bytes(x, slots), dst);
}
template <bool kWide, int J0, int J1>
__device__ __forceinline__ void kv_gather_groups(const KvGather& k) {
  if constexpr (J0 < J1) {
    kv_gather_group<kWide, J0>(k);
    kv_gather_groups<kWide, J0 + 1, J1>(k);
  }
}
template <bool kWide>
__device__ __forceinline__ void issue_kv(const Ctx& x, const uint8_t* kv_pool, const uint8_t* slots, uint8_t* dst) {
  kv_gather_groups<kWide, 0, 9>(kv_gather_setup(x, kv_pool, slots, dst));
}

// Visibility word of this lane's row for columns tile_c0 .. tile_c0+31 (bit c <-> tile_c0 + c).
__device__ __forceinline__ uint32_t mask_word(const Ctx& x, const uint8_t* custom_mask, const uint8_t* m, int tile_c0) {
  uint32_t bits = 0;
  const bool col_ok = tile_c0 + (x.lane & 31) < x.c_end;
  if (x.tok_last - x.tok_first < kMetaTokens) {  // wave-uniform: every token of the block is in LDS
#pragma unroll
    for (int tp = 0; tp < (kMetaTokens + 1) / 2; ++tp) {
      if (tp < x.n_tok_pairs) {
        const int i = 2 * tp + x.g;  // token of this lane half within the block
        const bool ok = col_ok && x.tok_first + i <= x.tok_last;
        const int byte_val = *reinterpret_cast<const int*>(m + 128 * (min(i, kMetaTokens - 1) + 1) + 4 * (x.lane & 31));
        const uint64_t bal = __ballot(ok && byte_val != 0);
        const uint32_t word = x.my_half ? (uint32_t)(bal >> 32) : (uint32_t)bal;
        bits = x.my_pair == tp ? word : bits;
      }
    }
  } else {  // blocks of more than kMetaTokens tokens (H < 8): read every byte directly
    for (int tp = 0; tp < x.n_tok_pairs; ++tp) {
      const int t = x.tok_first + 2 * tp + x.g;
      const bool ok = col_ok && t <= x.tok_last;
      const int byte_val = ok ? custom_mask[x.mask_base + (size_t)t * x.L + tile_c0 + (x.lane & 31)] : 0;
      const uint64_t bal = __ballot(byte_val != 0);
      const uint32_t word = x.my_half ? (uint32_t)(bal >> 32) : (uint32_t)bal;
      bits = x.my_pair == tp ? word : bits;
    }
  }
  return bits;
}

// Global inputs of the partial kernel that the per-tile steps read.
struct Glob {
  const uint8_t* kv_pool;
  const int32_t* kv_indices;
  const int32_t* out_cache_loc;
  const uint8_t* custom_mask;
};

// LDS areas of one wave: the shared tile ring, its private metadata ring and its rope query operands
// (k-step 32 + j of lane l at q_rope + 1024 j + 16 l).
struct Bufs {
  uint8_t* kv;
  uint8_t* meta;
  const uint8_t* q_rope;
};

// Running softmax state of the lane's query row over one split (see tile_iter).
struct RowStats {
  float m_ref;     // reference max (base-2 units of the scaled score), fixed once set
  float l_lane;    // the lane's share of the row sum of 2^(score - m_ref)
  float best_raw;  // the lane's largest visible raw score (element index in its low bits)
  int best_col;    // and its column
  bool over;       // a score exceeded m_ref + kHeadroom
};

// The score product S^T = K . Q^T of a tile accumulates in VGPRs through inline assembly. With the
// 256 output accumulators in AGPRs, the compiler's own form of this product takes its accumulator in
// AGPRs as well and so moves an output block out to VGPRs and back around every tile (48 register
// moves per tile); this hipcc crashes on its option that selects the VGPR form. What the compiler
// does not see through the asm: (1) a product that adds onto the previous product's result (the
// same registers, the same instruction) needs no wait states, the matrix core forwards it; (2) a
// vector instruction may read the accumulator only some 20 wait states after the last product,
// which the loop guarantees by reading a score block one PV phase (32 products) after it was
// finished, and qk_settle() provides where a read follows at once. The K operand registers are
// written by LDS reads, whose completion the compiler tracks through the asm operands as for any
// other instruction.
__device__ __forceinline__ void qk_first(f32x16& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "v"(q));
}
__device__ __forceinline__ void qk_next(f32x16& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "v"(q));
}
__device__ __forceinline__ void qk_settle(f32x16& s) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s)); }

// Query (B) operand of k-step ks: the latent k-steps live in VGPRs, the four rope k-steps in LDS
// (freeing 16 VGPRs the pipelined loop needs).
template <int KS>
__device__ __forceinline__ bf16x8 q_operand(const bf16x8 (&q)[kRegSteps], const Bufs& bf, int lane) {
  if constexpr (KS < kRegSteps)
    return q[KS];
  else
    return *reinterpret_cast<const bf16x8*>(bf.q_rope + 1024 * (KS - kRegSteps) + 16 * lane);
}

// K operand of k-step ks (logical chunk 2ks + g of tile row lane & 31) at kb + k_off[ks % 4] +
// 1024 (ks / 4); the four per-lane offsets do not change from tile to tile.
__device__ __forceinline__ bf16x8 load_k(const uint8_t* kb, const int (&k_off)[4], int ks) {
  return *reinterpret_cast<const bf16x8*>(kb + k_off[ks % 4] + k_step_offset(ks));
}

// V^T operand of output block eb (latent columns [32 eb, 32 eb + 32)) and k-step kk (tile columns
// [16 kk, 16 kk + 16), permuted as the probabilities are): two transposed 8-byte reads, rows
// 16 kk + 8m + v_row of latent chunk 4 eb + v_chunk (see run_split for v_off).
__device__ __forceinline__ bf16x8 load_v(const uint8_t* kb, const int (&v_off)[2], int kk, int eb) {
  const uint8_t* p0 = kb + v_off[eb & 1] + v_step_offset(kk, eb, 0);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(kb + v_off[eb & 1] + v_step_offset(kk, eb, 1)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Visibility word of the lane's row for columns tile_c0 .. tile_c0 + 31 when all 32 rows of the
// block belong to one draft token (H a multiple of 32): every lane reads the mask byte of column
// lane % 32 from the metadata ring and one compare gives the whole word.
__device__ __forceinline__ int mask_byte_uniform(const Ctx& x, const uint8_t* m) {
  return *reinterpret_cast<const int*>(m + 128 + 4 * (x.lane & 31));
}
__device__ __forceinline__ uint32_t mask_word_uniform(const Ctx& x, int byte_val, int tile_c0) {
  const bool col_ok = tile_c0 + (x.lane & 31) < x.c_end;
  return (uint32_t)__ballot(col_ok && byte_val != 0);
}

// One pipelined tile step of one wave (the wave owns query rows 32w .. 32w+31 of the row tile: the
// whole 576-wide query row in VGPRs, the whole 512-wide output row in AGPRs). Step t:
//   1. the score product of tile t+1 (36 products into s_nxt, K from ring slot (t+1) % 3), and
//      between its products the softmax of tile t on s_cur: mask, maximum, reference, the
//      numerators 2^(score - m_ref) rounded to bf16 for the PV product, and their exact sum; the
//      row loads of tile t+2 go out between the first nine products, the metadata loads of tile
//      t+4 under the last ones (products 27-35 carry no softmax piece; between the PV products
//      their address arithmetic cost ~0.7% more at the ragged 185k batch);
//   2. the PV product of tile t (32 products, V^T from ring slot t % 3, two transposed reads per
//      V operand, each feeding one product);
//   3. the wave waits for its row loads of tile t+2, then the workgroup barrier: after it, tile
//      t+2 is in LDS for every wave, and every wave is done with ring slot t % 3, which the next
//      step's row loads (tile t+3) refill.
// No other synchronisation: the waves share the tile ring and nothing else. A vector instruction
// issued between matrix products runs in the products' shadow only at about two per product (a
// measured property of gfx950 with one wave per SIMD), so the softmax is spread over the 36 score
// products a few instructions at a time, each group pinned in place by a scheduling barrier.
template <bool kWide>
__device__ __forceinline__ void tile_iter(const Ctx& x_in, int t, int c_begin, const Glob& gl, const Bufs& bf,
                                          const bf16x8 (&q)[kRegSteps], const int (&k_off)[4], const int (&v_off)[2],
                                          f32x16 (&oacc)[kEBlocks], f32x16& s_cur, f32x16& s_nxt, RowStats& st) {
  const int tile_c0 = c_begin + t * kTile;
  // The metadata, mask and gather addresses derive from the lane's role; hiding those inputs behind
  // an empty asm makes the compiler rebuild the addresses in each step as short-lived values instead
  // of hoisting a dozen 64-bit addresses out of the loop (which does not fit the registers).
  Ctx x = x_in;
  asm volatile("" : "+v"(x.lane), "+v"(x.g), "+v"(x.my_pair), "+v"(x.my_half));
  const uint8_t* __restrict__ kb_cur = bf.kv + (t % kBufs) * kTileBytes;
  const uint8_t* __restrict__ kb_nxt = bf.kv + ((t + 1) % kBufs) * kTileBytes;
  const uint8_t* meta_cur = bf.meta + (t % kMetaStages) * kMetaBytes;
  uint8_t* const meta_dst = bf.meta + ((t + 4) % kMetaStages) * kMetaBytes;
  const int meta_c0 = tile_c0 + 4 * kTile;
  KvGather gat;

  // The LDS reads that feed scalar decisions (this tile's mask byte, the slots of the rows gathered
  // next) go out before the K operand reads, so the waits for them never drain the reads behind.
  const int mask_byte = x.uniform_token ? mask_byte_uniform(x, meta_cur) : 0;
  const u32x4 sb = kv_slot_bytes(x, bf.meta + ((t + 2) % kMetaStages) * kMetaBytes);

  // ---- softmax pieces of tile t (s_cur), spread over the score products of tile t+1
  uint32_t bits = 0;
  bool all_vis = false;
  float raw = -INFINITY;
  float base = 0.0f;
  float p_even = 0.0f;
  bf16x8 pb[2];
  float psum = 0.0f;
  // Each piece ends with an empty asm on what it produced: the matrix products are volatile asm too,
  // so no piece can be moved (by the IR optimiser, which ignores scheduling barriers) away from the
  // products it is meant to run under.
  // (fmaxf on values the compiler cannot see the origin of would canonicalise every input first)
  auto pin = [](float& v) { asm volatile("" : "+v"(v)); };
  auto max3 = [](float a, float b, float c) {
    float r;
    asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
  };
  auto piece = [&](auto kc) {
    constexpr int ks = decltype(kc)::value;
    if constexpr (ks == 0) {
      bits = x.uniform_token ? mask_word_uniform(x, mask_byte, tile_c0) : mask_word(x, gl.custom_mask, meta_cur, tile_c0);
      all_vis = __all(bits == 0xFFFFFFFFu);
    } else if constexpr (ks >= 1 && ks <= 4) {  // element index into the low 4 mantissa bits
#pragma unroll
      for (int i = 4 * (ks - 1); i < 4 * ks; ++i)
        s_cur[i] = __uint_as_float((__float_as_uint(s_cur[i]) & ~15u) | (uint32_t)i);
      asm volatile("" : "+v"(s_cur));  // in place: the masked branch below then needs no copies
    } else if constexpr (ks == 5) {
      if (!all_vis) {  // a tile with hidden columns (draft tiles, arbitrary masks): masked scores are -inf
        const uint32_t bsh = bits >> (4 * x.g);
#pragma unroll
        for (int i = 0; i < 16; ++i) s_cur[i] = ((bsh >> (8 * (i >> 2) + (i & 3))) & 1u) ? s_cur[i] : -INFINITY;
      }
      asm volatile("" : "+v"(s_cur));
    } else if constexpr (ks == 6) {
      raw = max3(max3(s_cur[0], s_cur[1], s_cur[2]), s_cur[3], s_cur[4]);
    } else if constexpr (ks == 7) {
      raw = max3(max3(raw, s_cur[5], s_cur[6]), s_cur[7], s_cur[8]);
    } else if constexpr (ks == 8) {
      raw = max3(max3(raw, s_cur[9], s_cur[10]), s_cur[11], s_cur[12]);
    } else if constexpr (ks == 9) {
      raw = max3(max3(raw, s_cur[13], s_cur[14]), s_cur[15], s_cur[15]);
      // the lane's best visible score so far and its column (an earlier tile keeps a tie)
      const int col = (int)(__float_as_uint(raw) & 15u);
      st.best_col = raw > st.best_raw ? tile_c0 + 8 * (col >> 2) + 4 * x.g + (col & 3) : st.best_col;
      st.best_raw = fmaxf(st.best_raw, raw);
    } else if constexpr (ks == 10) {
      const float mx = pair_max(raw) * x.scale_log2;
      st.m_ref = st.m_ref == -INFINITY ? mx : st.m_ref;
      st.over = st.over || mx > st.m_ref + kHeadroom;
      base = st.m_ref == -INFINITY ? 0.0f : st.m_ref;
      pin(base);
    } else if constexpr (ks >= 11 && ks < 27) {  // one numerator per product (2^-inf = 0 when masked)
      constexpr int i = ks - 11;
      float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[i], x.scale_log2, -base));
      pin(pv);
      if constexpr ((i & 1) == 0) {
        p_even = pv;
      } else {
        const bf16x2 pk = __builtin_convertvector(f32x2{p_even, pv}, bf16x2);
        pb[i >> 3][(i - 1) & 7] = pk[0];
        pb[i >> 3][i & 7] = pk[1];
        psum += p_even + pv;
      }
    } else if constexpr (ks == 27) {
      st.l_lane += psum;
    }
  };

  // ---- 1. score product of tile t+1 with the softmax of tile t between its products (the LDS reads
  // of the mask byte and of the gathered rows' slots went out first, see above)
  constexpr int kKAhead = 2;
  bf16x8 kf[kKAhead + 1];
#pragma unroll
  for (int ks = 0; ks < kKAhead; ++ks) kf[ks] = load_k(kb_nxt, k_off, ks);
  piece(std::integral_constant<int, 0>{});  // the first mask and index work covers the first K reads' latency
  gat = kv_gather_build(x, gl.kv_pool, sb, bf.kv + ((t + 2) % kBufs) * kTileBytes);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 qr[kSteps - kRegSteps];  // rope query operands, read from LDS kKAhead k-steps ahead
  static_for<0, kSteps>([&](auto kc) {
    constexpr int ks = decltype(kc)::value;
    if constexpr (ks + kKAhead < kSteps) {
      kf[(ks + kKAhead) % (kKAhead + 1)] = load_k(kb_nxt, k_off, ks + kKAhead);
      if constexpr (ks + kKAhead >= kRegSteps) qr[ks + kKAhead - kRegSteps] = q_operand<ks + kKAhead>(q, bf, x.lane);
    }
    if constexpr (ks == 0)
      qk_first(s_nxt, kf[0], q[0]);
    else if constexpr (ks < kRegSteps)
      qk_next(s_nxt, kf[ks % (kKAhead + 1)], q[ks]);
    else
      qk_next(s_nxt, kf[ks % (kKAhead + 1)], qr[ks - kRegSteps]);
    if constexpr (ks + 1 < 28) piece(std::integral_constant<int, ks + 1>{});
    // the row loads of tile t+2, one after each of the first nine products: they need most of the
    // step to land (a CU's gathers of one tile complete about 3000 cycles after the first is issued,
    // wherever in the step they go; nine back to back before the first product cost more issue time)
    if constexpr (ks >= 0 && ks <= 8) kv_gather_group<kWide, ks>(gat);
    // the metadata loads of tile t+4 under the last score products, which carry no softmax piece
    if constexpr (ks == 27) issue_meta_part<0>(x, gl.kv_indices, gl.out_cache_loc, gl.custom_mask, meta_c0, meta_dst);
    if constexpr (ks == 30) issue_meta_part<1>(x, gl.kv_indices, gl.out_cache_loc, gl.custom_mask, meta_c0, meta_dst);
    if constexpr (ks == 33) issue_meta_part<2>(x, gl.kv_indices, gl.out_cache_loc, gl.custom_mask, meta_c0, meta_dst);

    __builtin_amdgcn_sched_barrier(0);
  });

  // ---- 2. PV product of tile t: O^T[eb] += V^T(kk, eb) . P^T(kk); V operands two ahead
  constexpr int kVAhead = 2;
  bf16x8 vf[kVAhead + 1];
#pragma unroll
  for (int f = 0; f < kVAhead; ++f) vf[f] = load_v(kb_cur, v_off, f >> 4, f & 15);
  static_for<0, 2 * kEBlocks>([&](auto fc) {
    constexpr int f = decltype(fc)::value;
    if constexpr (f + kVAhead < 2 * kEBlocks)
      vf[(f + kVAhead) % (kVAhead + 1)] = load_v(kb_cur, v_off, (f + kVAhead) >> 4, (f + kVAhead) & 15);
    __builtin_amdgcn_sched_barrier(0);
    oacc[f & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[f % (kVAhead + 1)], pb[f >> 4], oacc[f & 15], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  });

  // ---- 3. this wave's row loads of tile t+2 have landed (the metadata loads issued after them may
  // still be in flight: loads retire in order), then the barrier
  if (x.n_meta == 1)
    __builtin_amdgcn_s_waitcnt(1 | (0x7 << 4) | (0xF << 8));
  else if (x.n_meta == 2)
    __builtin_amdgcn_s_waitcnt(2 | (0x7 << 4) | (0xF << 8));
  else
    __builtin_amdgcn_s_waitcnt(3 | (0x7 << 4) | (0xF << 8));
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // The score block of tile t+1 stays allocated to the end of the step. The compiler takes an asm
  // product as finished when it is issued, but the matrix core writes its result some 30 cycles
  // later; in the last step, where that block is never read, the compiler would otherwise hand its
  // registers to the PV phase's addresses and operands right after the last product, and the late
  // write would clobber them.
  asm volatile("" : "+v"(s_nxt));
}

// Partial kernel body. Wave w owns query rows 32w .. 32w+31 of the row tile: it scores them against
// every column of the split, runs their softmax and accumulates their 512-wide outputs; the four
// waves share only the ring of KV tiles they gather together.
//
// Vector-memory pipeline: everything a tile needs arrives through direct-to-LDS loads, so no loaded
// register is waited on inside the loop. Step t issues the 9 row loads of tile t+2 and the n_meta
// metadata loads of tile t+4 and waits for the row loads before its barrier, so tile t+2 (and, in
// order, the metadata of tile t+3) is in LDS for everyone after it. The prologue issues the metadata
// of tiles 0-3 and the rows of tiles 0 and 1, waits for both tiles and scores tile 0.
// Prefetches past the split read clamped, valid addresses into buffers that are never read.
// Inputs of the partial kernels that every split reads.
struct PartialArgs {
  const __bf16* q_nope;
  const __bf16* q_rope;
  const uint8_t* kv_pool;
  int N;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* out_cache_loc;
  const uint8_t* custom_mask;
  const int32_t* mask_indptr;
  int B, q_len, H;
  float scale_log2;
  float4* ws_ml;
  uint16_t* ws_acc;
  int2* ws_top;
};

// The partial kernels' LDS.
struct PartialLds {
  uint8_t* kv;
  uint8_t* meta;
  uint8_t* q_rope;
  int* over;
};

// A wave whose 32 rows all lie past R (the fourth wave at R = 72, the last two of a 64-row remainder)
// has nothing to score, but the tile ring is filled by all four waves and every step ends in a
// workgroup barrier. Such a wave keeps its share of the pipeline, step for step as tile_iter and
// run_split do it: the same metadata and row loads, the same waits and the same barriers (one after
// the prologue, one per tile, two for the rerun decision), and skips the products and the softmax.
// It reports no overflow and follows the others into a second pass if one of them asks for it.
template <bool kWide>
__device__ __forceinline__ void run_loads_only(const Ctx& x, int c_begin, int ntiles, const Glob& gl, const Bufs& bf,
                                            int* lds_over, int w) {
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      issue_meta(x, gl.kv_indices, gl.out_cache_loc, gl.custom_mask, c_begin + k * kTile, bf.meta + k * kMetaBytes);
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
    issue_kv<kWide>(x, gl.kv_pool, bf.meta, bf.kv);
    issue_kv<kWide>(x, gl.kv_pool, bf.meta + kMetaBytes, bf.kv + kTileBytes);
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
    lds_barrier();
    for (int t = 0; t < ntiles; ++t) {
      issue_kv<kWide>(x, gl.kv_pool, bf.meta + ((t + 2) % kMetaStages) * kMetaBytes,
                      bf.kv + ((t + 2) % kBufs) * kTileBytes);
      issue_meta(x, gl.kv_indices, gl.out_cache_loc, gl.custom_mask, c_begin + (t + 4) * kTile,
                 bf.meta + ((t + 4) % kMetaStages) * kMetaBytes);
      // the row loads have landed; the x.n_meta metadata loads behind them may still be in flight
      if (x.n_meta == 1)
        __builtin_amdgcn_s_waitcnt(1 | (0x7 << 4) | (0xF << 8));
      else if (x.n_meta == 2)
        __builtin_amdgcn_s_waitcnt(2 | (0x7 << 4) | (0xF << 8));
      else
        __builtin_amdgcn_s_waitcnt(3 | (0x7 << 4) | (0xF << 8));
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)
    if ((threadIdx.x & 63) == 0) lds_over[w] = 0;
    lds_barrier();
    int any_over = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) any_over |= lds_over[k];
    lds_barrier();
    if (!any_over) break;
  }
}

// Where request b's inputs start: kv_indptr[b], its prefix length and mask_indptr[b].
struct Request {
  int kv_start, P;
  int mask_base;
};
__device__ __forceinline__ Request load_request(const PartialArgs& a, int b) {
  Request r;
  r.kv_start = a.kv_indptr[b];
  r.P = max(a.kv_indptr[b + 1] - r.kv_start, 0);
  r.mask_base = a.mask_indptr[b];
  return r;
}

// Columns [c_begin, c_end) (c_begin < c_end) of request b for the 128 query rows of row tile rt:
// writes the (m, l, 2^e) records and fp16 accumulator partials of those rows at partial row offset `part`.
template <bool kWide>
__device__ __forceinline__ void run_split(const PartialArgs& a, const PartialLds& lds, int b, const Request& rq,
                                          int c_begin, int c_end, int rt, size_t part) {
  const __bf16* __restrict__ q_nope = a.q_nope;
  const __bf16* __restrict__ q_rope = a.q_rope;
  const uint8_t* __restrict__ kv_pool = a.kv_pool;
  const int32_t* __restrict__ kv_indices = a.kv_indices;
  const int32_t* __restrict__ out_cache_loc = a.out_cache_loc;
  const uint8_t* __restrict__ custom_mask = a.custom_mask;
  float4* __restrict__ ws_ml = a.ws_ml;
  uint16_t* __restrict__ ws_acc = a.ws_acc;
  const int H = a.H, q_len = a.q_len;
  const int lane = threadIdx.x & 63;
  const int w = wave_uniform(threadIdx.x >> 6);
  const int R = q_len * H;
  const int kv_start = rq.kv_start;
  const int P = rq.P;
  const int L = P + q_len;

  const int g = lane >> 5;  // k-group of the MFMA operands
  const int own_row0 = rt * kRowsPerWG + w * kBlockRows;
  const int own_row = own_row0 + (lane & 31);
  if (c_begin >= c_end) {
    if (own_row < R && g == 0) ws_ml[part + own_row] = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
    return;
  }

  Ctx x;
  x.mask_base = (size_t)rq.mask_base;
  x.N = a.N;
  x.b = b;
  x.q_len = q_len;
  x.kv_start = kv_start;
  x.P = P;
  x.L = L;
  x.c_end = c_end;
  x.lane = lane;
  x.g = g;
  x.loader_row0 = (w % kLoaders) * kRowsPerLoader;
  // tokens of the wave's rows (a block past R uses the last token: valid, never stored)
  x.tok_first = min(own_row0, R - 1) / H;
  x.tok_last = (min(own_row0 + kBlockRows, R) - 1) / H;
  x.uniform_token = x.tok_first == x.tok_last;
  const int my_tok_ix = min(own_row, R - 1) / H - x.tok_first;
  x.my_pair = my_tok_ix >> 1;
  x.my_half = my_tok_ix & 1;
  x.n_tok_pairs = (x.tok_last - x.tok_first + 2) >> 1;
  // metadata loads per tile: the first carries token 0, each extra one two more tokens
  x.n_meta = 1 + min((x.tok_last - x.tok_first + 1) / 2, kMetaExtra);
  x.scale_log2 = a.scale_log2;
  uint8_t* const meta = lds.meta + w * kMetaStages * kMetaBytes;
  uint8_t* const q_lds = lds.q_rope + w * kQRopeBytes;
  uint8_t* const lds_kv = lds.kv;
  const Bufs bf = {lds_kv, meta, q_lds};
  const Glob gl = {kv_pool, kv_indices, out_cache_loc, custom_mask};
  if (own_row0 >= R) {  // wave-uniform: only padding rows
    run_loads_only<kWide>(x, c_begin, (c_end - c_begin + kTile - 1) / kTile, gl, bf, lds.over, w);
    return;
  }

  // ---- the metadata of the first four tiles, then the wave's query rows: the latent k-steps as MFMA
  // B operands in registers (k-step ks holds Q[row][16 ks + 8 g .. +8]), the rope k-steps straight
  // to LDS. Rows past R repeat row R-1 (their results are never written; a copy of a real row
  // cannot set the rerun flag unless that row does). All of it is in flight at once and one wait
  // in the prologue covers it; issued before the query registers are live, the metadata loads have
  // their addresses at hand, not in spill slots whose reloads would each wait for every load.
  issue_meta(x, kv_indices, out_cache_loc, custom_mask, c_begin, meta);
  issue_meta(x, kv_indices, out_cache_loc, custom_mask, c_begin + kTile, meta + kMetaBytes);
  issue_meta(x, kv_indices, out_cache_loc, custom_mask, c_begin + 2 * kTile, meta + 2 * kMetaBytes);
  issue_meta(x, kv_indices, out_cache_loc, custom_mask, c_begin + 3 * kTile, meta + 3 * kMetaBytes);
  bf16x8 q[kRegSteps];
  {
    const int q_row = min(own_row, R - 1);
    const bf16x8* qn = reinterpret_cast<const bf16x8*>(q_nope + ((size_t)b * R + q_row) * kLatent);
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(q_rope + ((size_t)b * R + q_row) * kRope);
#pragma unroll
    for (int j = 0; j < kSteps - kRegSteps; ++j) dma_group<0>(qr + 2 * j + g, lds_addr(q_lds + 1024 * j));
#pragma unroll
    for (int ks = 0; ks < kRegSteps; ++ks) q[ks] = qn[2 * ks + g];
  }


  // per-lane LDS offsets inside a tile, the same for every tile (k_lane_offset, v_lane_offset)
  int k_off[4], v_off[2];
#pragma unroll
  for (int b4 = 0; b4 < 4; ++b4) k_off[b4] = k_lane_offset(lane, b4);
  v_off[0] = v_lane_offset(lane, 0);
  v_off[1] = v_lane_offset(lane, 1);

  const int ntiles = (c_end - c_begin + kTile - 1) / kTile;
  f32x16 oacc[kEBlocks];
  RowStats st;
  st.m_ref = -INFINITY;
  int* const lds_over = lds.over;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int eb = 0; eb < kEBlocks; ++eb) oacc[eb] = f32x16{};
    const float m_fixed = st.m_ref;  // pass 1: each row's true max over the split (set below)
    st.m_ref = pass == 0 ? -INFINITY : m_fixed;
    st.l_lane = 0.0f;
    st.best_raw = -INFINITY;
    st.best_col = 0;
    st.over = false;

    // ---- prologue: the metadata of tiles 0-3 (issued above for the first pass), the rows of tiles 0
    // and 1 (both tiles' addresses formed before either tile's loads go out, so no spill reload and
    // its wait falls between them), then the scores of tile 0
    if (pass > 0) {
      issue_meta(x, kv_indices, out_cache_loc, custom_mask, c_begin, meta);
      issue_meta(x, kv_indices, out_cache_loc, custom_mask, c_begin + kTile, meta + kMetaBytes);
      issue_meta(x, kv_indices, out_cache_loc, custom_mask, c_begin + 2 * kTile, meta + 2 * kMetaBytes);
      issue_meta(x, kv_indices, out_cache_loc, custom_mask, c_begin + 3 * kTile, meta + 3 * kMetaBytes);
    }
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0): query rows and metadata
#pragma unroll
    for (int ks = 0; ks < kRegSteps; ++ks) asm volatile("" ::"v"(q[ks]));  // query rows ready here
    {
      const KvGather g0 = kv_gather_setup(x, kv_pool, meta, lds_kv);
      const KvGather g1 = kv_gather_setup(x, kv_pool, meta + kMetaBytes, lds_kv + kTileBytes);
      kv_gather_groups<kWide, 0, 9>(g0);
      kv_gather_groups<kWide, 0, 9>(g1);
    }
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0): tiles 0 and 1
    lds_barrier();
    f32x16 s_a, s_b;
    {
      bf16x8 kf[4];
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) kf[ks] = load_k(lds_kv, k_off, ks);
      static_for<0, kSteps>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if constexpr (ks + 3 < kSteps) kf[(ks + 3) % 4] = load_k(lds_kv, k_off, ks + 3);
        if constexpr (ks == 0)
          qk_first(s_a, kf[0], q[0]);
        else
          qk_next(s_a, kf[ks % 4], q_operand<ks>(q, bf, lane));
        __builtin_amdgcn_sched_barrier(0);
      });
      qk_settle(s_a);
    }
    // ---- the tile loop, two steps per trip so the two score blocks trade roles without copies
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      tile_iter<kWide>(x, t, c_begin, gl, bf, q, k_off, v_off, oacc, s_a, s_b, st);
      tile_iter<kWide>(x, t + 1, c_begin, gl, bf, q, k_off, v_off, oacc, s_b, s_a, st);
    }
    if (t < ntiles) tile_iter<kWide>(x, t, c_begin, gl, bf, q, k_off, v_off, oacc, s_a, s_b, st);
    // the last steps prefetched rows past the split; let them land before LDS is reused
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0)

    // a score above its row's reference + headroom anywhere in the workgroup: rerun the split
    // with every row's reference at its true max (the second pass cannot overflow)
    if (lane == 0) lds_over[w] = __any(st.over) ? 1 : 0;
    lds_barrier();
    int any_over = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) any_over |= lds_over[k];
    lds_barrier();
    if (!any_over) break;
    st.m_ref = pair_max(st.best_raw) * x.scale_log2;  // the row's true max over the split
  }

  // ---- the row's top probability. Each visible column entered the PV product with its probability
  // rounded to bf16 (the sum l took the exact values). For the row's largest one (the same fma +
  // exp2 as in the tile, so the same value) the exact probability and the pool slot of its value
  // row go to the top record; the combine adds back what the rounding dropped, (p - bf16(p)) times
  // that value row, where the column matters against the row's final sum. Without that, a row
  // dominated by one column whose score came after the reference tile is off by up to 2^-9 of that
  // column's values. The lane pair first agrees on the row's best column.
  {
    const auto rs = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.best_raw), __float_as_uint(st.best_raw),
                                                     false, false);
    const auto cs = __builtin_amdgcn_permlane32_swap((unsigned)st.best_col, (unsigned)st.best_col, false, false);
    const float ra = __uint_as_float(rs[0]), rb = __uint_as_float(rs[1]);
    const int ca = (int)cs[0], cb = (int)cs[1];
    const bool take_b = rb > ra || (rb == ra && cb < ca);
    const float top = take_b ? rb : ra;
    const int col = take_b ? cb : ca;
    if (own_row < R && g == 0) {
      const float base = st.m_ref == -INFINITY ? 0.0f : st.m_ref;
      const float p = top == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(__builtin_fmaf(top, x.scale_log2, -base));
      int slot = col < P ? kv_indices[kv_start + col] : out_cache_loc[(size_t)b * q_len + (col - P)];
      slot = min(max(slot, 0), a.N - 1);
      a.ws_top[part + own_row] = make_int2(__float_as_int(p), slot);
    }
  }

  // ---- partial write: (m_ref, l, 2^e) and the row's 512-wide accumulator times 2^-e in fp16, with e
  // taken from the row's largest |value| so that it lands in [2^14, 2^15): one rounding to 11
  // significant bits and no overflow whatever the values' range (half the bytes of fp32 partials).
  const float l_row = pair_sum(st.l_lane);
  float amax = 0.0f;
#pragma unroll
  for (int eb = 0; eb < kEBlocks; ++eb) {
#pragma unroll
    for (int j = 0; j < 16; j += 2)
      asm volatile("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(amax) : "v"(amax), "v"(oacc[eb][j]), "v"(oacc[eb][j + 1]));
  }
  amax = pair_max(amax);
  // amax = f 2^fe with f in [0.5, 1): the scale 2^(15 - fe) puts it in [2^14, 2^15); capped so that
  // the factor stays a normal float (rows below 2^-111 then keep smaller values, still exact in range)
  const int fe = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 15;
  const int sh = min(15 - fe, 126);
  const float up = __builtin_amdgcn_ldexpf(1.0f, sh);
  {
    // rows past R (the last block's padding) convert and swap like the others, unstored: the lane
    // swap runs with the whole wave active
    uint16_t* dst = ws_acc + (part + min(own_row, R - 1)) * kLatent;
#pragma unroll
    for (int eb = 0; eb < kEBlocks; ++eb) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        // values 8m .. 8m+3 are columns 32 eb + 16 m + 4 g + (0..3), values 8m+4 .. 8m+7 columns
        // 32 eb + 16 m + 8 + 4 g + (0..3); one swap with the partner lane (g = 1 - g) leaves lane g
        // with columns 32 eb + 16 m + 8 g + (0..7), stored as one 16-byte write
        uint32_t lo[2], hi[2];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const f16x2 a = __builtin_convertvector(
              (f32x2){oacc[eb][8 * m + 2 * d] * up, oacc[eb][8 * m + 2 * d + 1] * up}, f16x2);
          const f16x2 c = __builtin_convertvector(
              (f32x2){oacc[eb][8 * m + 4 + 2 * d] * up, oacc[eb][8 * m + 4 + 2 * d + 1] * up}, f16x2);
          const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a),
                                                          __builtin_bit_cast(uint32_t, c), false, false);
          lo[d] = r[0];
          hi[d] = r[1];
        }
        if (own_row < R)
          *reinterpret_cast<u32x4*>(dst + 32 * eb + 16 * m + 8 * g) = (u32x4){lo[0], lo[1], hi[0], hi[1]};
      }
    }
  }
  if (own_row < R && g == 0)
    ws_ml[part + own_row] = make_float4(st.m_ref, l_row, __builtin_amdgcn_ldexpf(1.0f, -sh), 0.0f);
}

#define PARTIAL_LDS_DECL                                                          \
  __shared__ __attribute__((aligned(16))) uint8_t lds_kv[kBufs * kTileBytes];     \
  __shared__ __attribute__((aligned(16))) uint8_t lds_meta[kWaves * kMetaStages * kMetaBytes]; \
  __shared__ __attribute__((aligned(16))) uint8_t lds_qrope[kWaves * kQRopeBytes]; \
  __shared__ int lds_over[kWaves];                                                \
  const PartialLds lds = {lds_kv, lds_meta, lds_qrope, lds_over};

// Per-request splits: workgroup -> (request b, split s, row tile) by decode_unit; split s of request
// b covers columns [s*chunk, min(L_b, (s+1)*chunk)) with chunk = ceil(L_b / nsplit) rounded up to the
// tile, and writes partial row block (b*nsplit + s)*R. An empty split writes (m = -inf, l = 0).
template <bool kWide>
__global__ void __launch_bounds__(kWaves * 64, 1)
verify_partial_kernel(const __bf16* __restrict__ q_nope, const __bf16* __restrict__ q_rope,
                      const uint8_t* __restrict__ kv_pool, int N,
                      const int32_t* __restrict__ kv_indptr, const int32_t* __restrict__ kv_indices,
                      const int32_t* __restrict__ out_cache_loc,
                      const uint8_t* __restrict__ custom_mask,
                      const int32_t* __restrict__ mask_indptr, int B, int q_len, int H,
                      float scale_log2, int nsplit, int n_rt, float4* __restrict__ ws_ml,
                      uint16_t* __restrict__ ws_acc, int2* __restrict__ ws_top) {
  PARTIAL_LDS_DECL
  const PartialArgs a = {q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                         B, q_len, H, scale_log2, ws_ml, ws_acc, ws_top};
  const Split sp = decode_unit(a.B, nsplit, n_rt);
  if (!sp.valid) return;
  const int b = sp.b, s = sp.s;
  const int R = a.q_len * a.H;
  // split bounds from the actual lengths (empty splits leave at once)
  const Request rq = load_request(a, b);
  const int L = rq.P + a.q_len;
  int chunk = (L + nsplit - 1) / nsplit;
  chunk = (chunk + kTile - 1) / kTile * kTile;
  const int c_begin = s * chunk;
  const int c_end = min(L, c_begin + chunk);
  const size_t part = ((size_t)b * nsplit + s) * R;
  run_split<kWide>(a, lds, b, rq, c_begin, c_end, sp.rt, part);
}

// ---- Balanced partition of the batch. Request b has T_b = ceil(L_b / 32) column tiles. With a
// budget of `units` splits for the whole batch (units >= B), the plan takes the smallest split size C
// (in tiles) for which sum_b ceil(T_b / C) <= units, gives request b n_b = ceil(T_b / C) splits and
// cuts its tiles evenly: split s covers tiles [floor(s T_b / n_b), floor((s+1) T_b / n_b)). This
// minimises the largest split, so a ragged batch spreads over a fixed grid in near-equal pieces
// (a short request gets one split, a long one many) instead of nsplit splits per request. Splits are
// numbered request after request: split_start[b] = sum_{b' < b} n_b', and the partial of split
// split_start[b] + s is partial row block (split_start[b] + s) * R. Splits never straddle requests, so
// a workgroup keeps one request's query rows, exactly like the per-request kernel.
// One wave computes the plan (the batch is small and the search is a few dozen steps, so wave
// reductions without workgroup barriers are the quickest form).
constexpr int kPlanThreads = 64;

__device__ __forceinline__ long long wave_sum(long long x) {
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

// split_info [units] = {request, first column, end column, 0} ({-1, 0, 0, 0} for unused splits) and
// split_start [B + 1]. A split's workgroups read their whole assignment with one load.
__global__ void __launch_bounds__(kPlanThreads)
verify_plan_kernel(const int32_t* __restrict__ kv_indptr, int B, int q_len, int units,
                   int* __restrict__ split_start, int4* __restrict__ split_info) {
  __shared__ int tiles[MLA_VERIFY_BALANCED_MAX_B];
  __shared__ int lens[MLA_VERIFY_BALANCED_MAX_B];
  __shared__ int start_s[MLA_VERIFY_BALANCED_MAX_B + 1];
  const int lane = threadIdx.x;
  int tmax = 1;
  for (int b = lane; b < B; b += kPlanThreads) {
    const long long L = max((long long)kv_indptr[b + 1] - (long long)kv_indptr[b], 0LL) + q_len;
    const int t = (int)((L + kTile - 1) / kTile);
    tiles[b] = t;
    lens[b] = (int)L;
    tmax = max(tmax, t);
  }
  for (int d = 32; d >= 1; d >>= 1) tmax = max(tmax, __shfl_xor(tmax, d, 64));
  __syncthreads();
  // smallest C in [1, tmax] with sum ceil(T_b / C) <= units (C = tmax gives B splits, and B <= units)
  unsigned lo = 1, hi = (unsigned)tmax;
  while (lo < hi) {
    const unsigned mid = (lo + hi) / 2;
    long long cnt = 0;  // 64-bit: with C = 1 the count is the batch's whole tile total
    for (int b = lane; b < B; b += kPlanThreads) cnt += ((unsigned)tiles[b] + mid - 1) / mid;
    if (wave_sum(cnt) <= units) hi = mid; else lo = mid + 1;
  }
  const unsigned C = lo;
  // split_start: running sum of n_b = ceil(T_b / C)
  int carry = 0;
  if (lane == 0) start_s[0] = 0;
  for (int b0 = 0; b0 < B; b0 += kPlanThreads) {
    const int b = b0 + lane;
    int x = b < B ? (int)(((unsigned)tiles[b] + C - 1) / C) : 0;
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (b < B) start_s[b + 1] = carry + x;
    carry += __shfl(x, 63, 64);
  }
  __syncthreads();
  for (int b = lane; b <= B; b += kPlanThreads) split_start[b] = start_s[b];
  for (int j = lane; j < units; j += kPlanThreads) {
    int l = 0, h = B;  // the last b with start_s[b] <= j
    while (h - l > 1) {
      const int mid = (l + h) >> 1;
      if (start_s[mid] <= j) l = mid; else h = mid;
    }
    if (j < start_s[B]) {
      const int s = j - start_s[l], n = start_s[l + 1] - start_s[l];
      const long long T = tiles[l];
      const int c0 = (int)((long long)s * T / n) * kTile;
      const int c1 = min(lens[l], (int)((long long)(s + 1) * T / n) * kTile);
      split_info[j] = make_int4(l, c0, c1, 0);
    } else {
      split_info[j] = make_int4(-1, 0, 0, 0);
    }
  }
}

// Wave-wide sum / max of 32-bit values as a wave-uniform result, and an inclusive prefix sum over the
// 64 lanes: DPP moves inside each 16-lane row (rotations for the reductions, shifts that bring in 0
// for the scan), then the four row results through readlane, with no LDS round trip.
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);  // row_ror:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x122, 0xF, 0xF, false);  // row_ror:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x121, 0xF, 0xF, false);  // row_ror:1
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x122, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x121, 0xF, 0xF, false));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_incl_scan_i32(int x, int lane) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// The same plan for batches of at most 64 requests, computed by one wave inside the partial kernel
// (lane b holds request b) for split j alone: {request, first column, end column, 0}, or
// {-1, 0, 0, 0} when the plan leaves split j unused. Every wave of every workgroup computes it (a few
// search steps of wave reductions, cheaper than a separate launch in front of the kernel). The
// result is the same C, n_b and ranges as verify_plan_kernel's: the count function is monotone in C,
// so searching a narrower interval that contains the smallest feasible C finds the same one, here
// [ceil(total / units), ceil(total / (units - B))] (below the first bound the count exceeds
// total / C > units; at the second it is at most total / C + B <= units), capped by the largest T_b.
// Counts are 32-bit while every T_b < 2^25 (64 requests then total under 2^31 tiles); longer
// requests (prefixes beyond 2^30 columns) take a 64-bit search over [1, max T_b]. Lanes b < B return
// their request's running split count in *start_incl. The lane of request b also loads mask_indptr[b]
// with its lengths, so the split's request bounds (*rq) cost no further round trip to memory.
constexpr int kFusedPlanMaxB = 64;
__device__ __forceinline__ int4 plan_split_wave(const int32_t* __restrict__ kv_indptr,
                                                const int32_t* __restrict__ mask_indptr, int B, int q_len, int units,
                                                int j, int lane, int* start_incl, Request* rq) {
  int T = 0, Lb = 0, k0 = 0, m0 = 0;
  if (lane < B) {
    k0 = kv_indptr[lane];
    m0 = mask_indptr[lane];
    const long long L = max((long long)kv_indptr[lane + 1] - (long long)k0, 0LL) + q_len;
    T = (int)((L + kTile - 1) / kTile);
    Lb = (int)L;
  }
  const int tmax = max(wave_max_i32(T), 1);
  unsigned C;
  if (tmax < (1 << 25)) {
    const int total = wave_sum_i32(T);
    int lo = max((total + units - 1) / units, 1);
    int hi = units > B ? min(tmax, (total + (units - B) - 1) / (units - B)) : tmax;
    lo = min(lo, hi);
    while (lo < hi) {  // wave-uniform bounds: a scalar loop
      const int mid = (lo + hi) >> 1;
      const int cnt = wave_sum_i32((int)(((unsigned)T + (unsigned)mid - 1) / (unsigned)mid));
      if (cnt <= units) hi = mid; else lo = mid + 1;
    }
    C = (unsigned)lo;
  } else {
    unsigned lo = 1, hi = (unsigned)tmax;
    while (lo < hi) {
      const unsigned mid = (lo + hi) / 2;
      const long long cnt = (long long)(((unsigned)T + mid - 1) / mid);
      if (wave_sum(cnt) <= units) hi = mid; else lo = mid + 1;
    }
    C = lo;
  }
  const int n = lane < B ? (int)(((unsigned)T + C - 1) / C) : 0;
  const int incl = wave_incl_scan_i32(n, lane);
  const int excl = incl - n;
  *start_incl = incl;
  const unsigned long long own = __ballot(lane < B && excl <= j && j < incl);
  if (own == 0) return make_int4(-1, 0, 0, 0);
  const int l = __ffsll((long long)own) - 1;
  const int s_l = j - __builtin_amdgcn_readlane(excl, l), n_l = __builtin_amdgcn_readlane(n, l);
  const long long T_l = __builtin_amdgcn_readlane(T, l);
  const int L_l = __builtin_amdgcn_readlane(Lb, l);
  rq->kv_start = __builtin_amdgcn_readlane(k0, l);
  rq->P = L_l - q_len;
  rq->mask_base = __builtin_amdgcn_readlane(m0, l);
  const int c0 = (int)((long long)s_l * T_l / n_l) * kTile;
  const int c1 = min(L_l, (int)((long long)(s_l + 1) * T_l / n_l) * kTile);
  return make_int4(l, c0, c1, 0);
}

// Workgroup -> (split j, row tile): split j on XCD j % 8 with all its row tiles (they read the same KV
// rows). The grid is 8 * ceil(units / 8) * n_rt; splits the plan leaves unused exit at once. With
// fused_plan (B <= kFusedPlanMaxB) the workgroups compute their split themselves and write the plan
// records (split_info[j] by split j's first row tile, split_start by workgroup 0); otherwise they
// read split_info, which verify_plan_kernel wrote.
template <bool kWide>
__global__ void __launch_bounds__(kWaves * 64, 1)
verify_partial_balanced_kernel(const __bf16* __restrict__ q_nope, const __bf16* __restrict__ q_rope,
                               const uint8_t* __restrict__ kv_pool, int N,
                               const int32_t* __restrict__ kv_indptr, const int32_t* __restrict__ kv_indices,
                               const int32_t* __restrict__ out_cache_loc,
                               const uint8_t* __restrict__ custom_mask,
                               const int32_t* __restrict__ mask_indptr, int B, int q_len, int H,
                               float scale_log2, int units, int n_rt, int fused_plan, int4* __restrict__ split_info,
                               int* __restrict__ split_start, float4* __restrict__ ws_ml,
                               uint16_t* __restrict__ ws_acc, int2* __restrict__ ws_top) {
  PARTIAL_LDS_DECL
  const PartialArgs a = {q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                         B, q_len, H, scale_log2, ws_ml, ws_acc, ws_top};
  const int xcd = (int)(blockIdx.x % 8), k = (int)(blockIdx.x / 8);
  const int j = xcd + 8 * (k / n_rt), rt = k % n_rt;
  if (j >= units) return;
  int4 info;  // {request, first column, end column}
  Request rq;
  if (fused_plan) {
    const int lane = threadIdx.x & 63;
    int incl;
    info = plan_split_wave(kv_indptr, mask_indptr, B, q_len, units, j, lane, &incl, &rq);
    if (threadIdx.x < 64) {
      if (rt == 0 && lane == 0) split_info[j] = info;
      if (blockIdx.x == 0) {
        if (lane == 0) split_start[0] = 0;
        if (lane < B) split_start[lane + 1] = incl;
      }
    }
    info = make_int4(wave_uniform(info.x), wave_uniform(info.y), wave_uniform(info.z), 0);
    if (info.x < 0) return;
    rq = {wave_uniform(rq.kv_start), wave_uniform(rq.P), wave_uniform(rq.mask_base)};
  } else {
    info = split_info[j];
    if (info.x < 0) return;
    rq = load_request(a, info.x);
  }
  const int b = info.x, c_begin = info.y, c_end = info.z;
  run_split<kWide>(a, lds, b, rq, c_begin, c_end, rt, (size_t)j * (q_len * H));
}

// Adds one split's partial to a combine lane's 8 columns: weight 2^(m - M) on the sum l, and on the
// 8 stored fp16 values (the accumulator times 2^-e) the weight times 2^e (st = {m, l, 2^e, 0}). An
// empty or fully masked split (m = -inf) adds nothing and its data is not used.
__device__ __forceinline__ void add_partial(const float4& st, const u32x4& x, float M, f32x4& acc0, f32x4& acc1,
                                            float& den) {
  const bool live = st.x != -INFINITY;
  const float wgt = live ? __builtin_amdgcn_exp2f(st.x - M) : 0.0f;
  den += live ? wgt * st.y : 0.0f;
  const float wv = wgt * st.z;
  const f16x8 h = __builtin_bit_cast(f16x8, x);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    acc0[k] += live ? wv * (float)h[k] : 0.0f;
    acc1[k] += live ? wv * (float)h[4 + k] : 0.0f;
  }
}

// kWaves waves per query row (b, r): weights w_s = 2^(m_s - M) over the non-empty partials,
// out = sum w_s acc_s / sum w_s l_s, lse = (M + log2 sum w_s l_s) * ln 2, with acc_s read as its
// stored fp16 values times 2^e_s. One wave per row (4 rows
// per workgroup) suits many rows (the ragged 185k batch, 4096 rows); more waves per row keep the chip
// busy when there are few rows and many splits (72 rows x 256 splits with one wave each left most
// CUs idle and walked 256 splits serially: 95 us, against 11 us with sixteen waves; the quarter-row
// kernel below takes that case now). The kernel is
// bound by memory round trips, so it keeps them few:
//  1. lane k of wave w reads the (m, l, 2^e) record and top record of split w*64 + k (and the maxima of
//     splits further on): the row max M;
//  2. lane k owns output columns [8k, 8k+8); wave w takes splits w, w + kWaves, ..., 4 at a time,
//     every record and accumulator load of a batch issued together (an empty
//     split's accumulator was never written: it is read, then discarded by a select);
//  3. the sum is reduced over the row's waves; each wave adds back, for its own splits whose top
//     column holds at least 1/32 of the row's sum, w_s (p - bf16(p)) times that column's value row
//     (the partial kernels rounded p to bf16 for the PV product; a column below that share moves the
//     output by under 2^-14 of its value row), from the records it read in step 1; waves 1.. hand
//     their accumulators to wave 0 through LDS.
// kBalanced: the partials of request b are blocks split_start[b] .. split_start[b+1] - 1 (the plan);
// otherwise the nsplit blocks b * nsplit .. b * nsplit + nsplit - 1.
template <int kWaves>
constexpr int combine_block_waves() { return kWaves == 1 ? 4 : kWaves; }

template <bool kBalanced, int kWaves>
__global__ void __launch_bounds__(combine_block_waves<kWaves>() * 64)
verify_combine_kernel(const float4* __restrict__ ws_ml, const uint16_t* __restrict__ ws_acc,
                      const int2* __restrict__ ws_top, const uint8_t* __restrict__ kv_pool, int N, int B, int R,
                      int nsplit_or_units, const int* __restrict__ split_start, __bf16* __restrict__ out,
                      float* __restrict__ lse) {
  constexpr int kRed = kWaves > 1 ? kWaves : 2;
  __shared__ float red_m[kRed];
  __shared__ f32x4 red_acc[kRed - 1][2][64];
  __shared__ float red_den[kRed];
  const int lane = threadIdx.x & 63;
  const int w = kWaves == 1 ? 0 : (int)(threadIdx.x >> 6);  // wave of the row
  const long row = kWaves == 1 ? (long)blockIdx.x * 4 + (threadIdx.x >> 6) : (long)blockIdx.x;
  if (row >= (long)B * R) return;  // only the one-wave form has a partial last workgroup
  const long b = row / R, r = row % R;
  size_t first;
  int nsplit;
  if constexpr (kBalanced) {
    first = (size_t)split_start[b];
    nsplit = split_start[b + 1] - split_start[b];
  } else {
    nsplit = nsplit_or_units;
    first = (size_t)b * nsplit;
  }
  const float4* ml = ws_ml + first * R + r;
  const int2* top = ws_top + first * R + r;
  // 1. split w*64 + lane: (m, l, 2^e) and top records in registers; the max over every split
  const int s_own = w * 64 + lane;
  const float4 st_own = s_own < nsplit ? ml[(size_t)s_own * R] : make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
  const int2 top_own = s_own < nsplit ? top[(size_t)s_own * R] : make_int2(0, 0);
  float M = st_own.x;
  for (int s = s_own + kWaves * 64; s < nsplit; s += kWaves * 64) M = fmaxf(M, ml[(size_t)s * R].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if constexpr (kWaves > 1) {
    if (lane == 0) red_m[w] = M;
    __syncthreads();
    M = red_m[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) M = fmaxf(M, red_m[k]);
  }
  bf16x8* o = reinterpret_cast<bf16x8*>(out + (size_t)row * kLatent + lane * 8);
  if (M == -INFINITY) {
    if (w == 0) {
      *o = bf16x8{};
      if (lane == 0) lse[row] = -INFINITY;
    }
    return;
  }
  // 2. weighted accumulators and sum over this wave's splits
  f32x4 acc0 = {}, acc1 = {};
  float den = 0.0f;
  const uint16_t* base = ws_acc + (first * R + r) * kLatent + lane * 8;
  const size_t split_stride = (size_t)R * kLatent;
  constexpr int kU = 4;  // splits per batch (8 measured slower: the registers cut occupancy to 3 waves)
  for (int s0 = w; s0 < nsplit; s0 += kWaves * kU) {
    float4 st[kU];
    u32x4 x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = s0 + kWaves * u;
      const bool valid = s < nsplit;
      st[u] = valid ? ml[(size_t)s * R] : make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
      x[u] = *reinterpret_cast<const u32x4*>(base + (size_t)(valid ? s : 0) * split_stride);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) add_partial(st[u], x[u], M, acc0, acc1, den);
  }
  // 3. the row's sum, then the exact top probabilities of this wave's splits
  float den_row = den;
  if constexpr (kWaves > 1) {
    if (lane == 0) red_den[w] = den;
    __syncthreads();
    den_row = red_den[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) den_row += red_den[k];
  }
  for (int s = s_own; s - lane < nsplit; s += kWaves * 64) {  // wave-uniform bound
    float4 st = st_own;
    int2 t = top_own;
    if (s != s_own && s < nsplit) {  // splits past the first 64 kWaves (rare): read their records
      st = ml[(size_t)s * R];
      t = top[(size_t)s * R];
    }
    const bool live = s < nsplit && st.x != -INFINITY;
    const float p = __int_as_float(t.x);
    const float wgt = live ? __builtin_amdgcn_exp2f(st.x - M) : 0.0f;  // the weight the accumulator got
    const bool take = live && 32.0f * (p * wgt) >= den_row;
    const float coef = wgt * (p - (float)(__bf16)p);
    uint64_t pick = __ballot(take);
    while (pick) {
      const int k = __ffsll((long long)pick) - 1;
      pick &= pick - 1;
      const float c = __shfl(coef, k, 64);
      const int slot = min(max(__shfl(t.y, k, 64), 0), N - 1);  // clamped again: any workspace stays in the pool
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(kv_pool + (size_t)slot * kRowBytes + lane * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc0[q] += c * (float)v[q];
        acc1[q] += c * (float)v[4 + q];
      }
    }
  }
  if constexpr (kWaves > 1) {
    if (w > 0) {
      red_acc[w - 1][0][lane] = acc0;
      red_acc[w - 1][1][lane] = acc1;
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int k = 0; k < kWaves - 1; ++k) {
      acc0 += red_acc[k][0][lane];
      acc1 += red_acc[k][1][lane];
    }
  }
  const float inv = 1.0f / den_row;
  bf16x8 res;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    res[k] = (__bf16)(acc0[k] * inv);
    res[4 + k] = (__bf16)(acc1[k] * inv);
  }
  *o = res;
  if (lane == 0) lse[row] = (M + log2f(den_row)) * 0.69314718055994530942f;
}

// Few rows: the same combine with four workgroups per row, one per 128-column quarter of the
// output, so the pass over the partials spreads over four times as many CUs (72 rows x 256 splits
// with one workgroup per row read their 38 MB from 72 CUs at ~2.8 TB/s). Lane (sq, cl) = (lane / 16,
// lane % 16) takes columns [128 qc + 8 cl, +8) of the splits s = sq (mod 4) of its wave; the four lane
// groups are summed by shuffles before the top-probability corrections and the cross-wave sum.
constexpr int kQuarterWaves = 8;
template <bool kBalanced>
__global__ void __launch_bounds__(kQuarterWaves * 64)
verify_combine_quarter_kernel(const float4* __restrict__ ws_ml, const uint16_t* __restrict__ ws_acc,
                              const int2* __restrict__ ws_top, const uint8_t* __restrict__ kv_pool, int N, int B,
                              int R, int nsplit_or_units,
                              const int* __restrict__ split_start, __bf16* __restrict__ out,
                              float* __restrict__ lse) {
  __shared__ float red_m[kQuarterWaves];
  __shared__ float red_den[kQuarterWaves];
  __shared__ f32x4 red_acc[kQuarterWaves - 1][2][16];
  const int lane = threadIdx.x & 63;
  const int w = (int)(threadIdx.x >> 6);
  const int sq = lane >> 4, cl = lane & 15;
  const long row = (long)(blockIdx.x >> 2);
  const int qc = (int)(blockIdx.x & 3);
  if (row >= (long)B * R) return;
  const long b = row / R, r = row % R;
  size_t first;
  int nsplit;
  if constexpr (kBalanced) {
    first = (size_t)split_start[b];
    nsplit = split_start[b + 1] - split_start[b];
  } else {
    nsplit = nsplit_or_units;
    first = (size_t)b * nsplit;
  }
  const float4* ml = ws_ml + first * R + r;
  const int2* top = ws_top + first * R + r;
  // 1. split w*64 + lane: (m, l, 2^e) and top records in registers; the max over every split
  const int s_own = w * 64 + lane;
  const float4 st_own = s_own < nsplit ? ml[(size_t)s_own * R] : make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
  const int2 top_own = s_own < nsplit ? top[(size_t)s_own * R] : make_int2(0, 0);
  float M = st_own.x;
  for (int s = s_own + kQuarterWaves * 64; s < nsplit; s += kQuarterWaves * 64) M = fmaxf(M, ml[(size_t)s * R].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red_m[w] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int k = 1; k < kQuarterWaves; ++k) M = fmaxf(M, red_m[k]);
  const int col0 = 128 * qc + 8 * cl;
  bf16x8* o = reinterpret_cast<bf16x8*>(out + (size_t)row * kLatent + col0);
  if (M == -INFINITY) {
    if (w == 0 && sq == 0) {
      *o = bf16x8{};
      if (cl == 0 && qc == 0) lse[row] = -INFINITY;
    }
    return;
  }
  // 2. weighted accumulators and sum over this lane group's splits
  f32x4 acc0 = {}, acc1 = {};
  float den = 0.0f;
  const uint16_t* base = ws_acc + (first * R + r) * kLatent + col0;
  const size_t split_stride = (size_t)R * kLatent;
  constexpr int kU = 4;
  constexpr int kStride = 4 * kQuarterWaves;  // splits between consecutive ones of a lane group
  for (int s0 = 4 * w + sq; s0 < nsplit; s0 += kStride * kU) {
    float4 st[kU];
    u32x4 x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = s0 + kStride * u;
      const bool valid = s < nsplit;
      st[u] = valid ? ml[(size_t)s * R] : make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
      x[u] = *reinterpret_cast<const u32x4*>(base + (size_t)(valid ? s : 0) * split_stride);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) add_partial(st[u], x[u], M, acc0, acc1, den);
  }
  // the four lane groups of the wave: every lane ends with the wave's sums for its columns
#pragma unroll
  for (int d = 16; d <= 32; d <<= 1) {
    den += __shfl_xor(den, d);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc0[k] += __shfl_xor(acc0[k], d);
      acc1[k] += __shfl_xor(acc1[k], d);
    }
  }
  // 3. the row's sum, then the exact top probabilities of this wave's splits (every lane group adds
  // them to its identical copy; only group 0's is kept)
  if (lane == 0) red_den[w] = den;
  __syncthreads();
  float den_row = red_den[0];
#pragma unroll
  for (int k = 1; k < kQuarterWaves; ++k) den_row += red_den[k];
  for (int s = s_own; s - lane < nsplit; s += kQuarterWaves * 64) {  // wave-uniform bound
    float4 st = st_own;
    int2 t = top_own;
    if (s != s_own && s < nsplit) {
      st = ml[(size_t)s * R];
      t = top[(size_t)s * R];
    }
    const bool live = s < nsplit && st.x != -INFINITY;
    const float p = __int_as_float(t.x);
    const float wgt = live ? __builtin_amdgcn_exp2f(st.x - M) : 0.0f;
    const bool take = live && 32.0f * (p * wgt) >= den_row;
    const float coef = wgt * (p - (float)(__bf16)p);
    uint64_t pick = __ballot(take);
    while (pick) {
      const int k = __ffsll((long long)pick) - 1;
      pick &= pick - 1;
      const float c = __shfl(coef, k, 64);
      const int slot = min(max(__shfl(t.y, k, 64), 0), N - 1);
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(kv_pool + (size_t)slot * kRowBytes + 2 * col0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc0[q] += c * (float)v[q];
        acc1[q] += c * (float)v[4 + q];
      }
    }
  }
  if (w > 0 && sq == 0) {
    red_acc[w - 1][0][cl] = acc0;
    red_acc[w - 1][1][cl] = acc1;
  }
  __syncthreads();
  if (w != 0 || sq != 0) return;
#pragma unroll
  for (int k = 0; k < kQuarterWaves - 1; ++k) {
    acc0 += red_acc[k][0][cl];
    acc1 += red_acc[k][1][cl];
  }
  const float inv = 1.0f / den_row;
  bf16x8 res;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    res[k] = (__bf16)(acc0[k] * inv);
    res[4 + k] = (__bf16)(acc1[k] * inv);
  }
  *o = res;
  if (cl == 0 && qc == 0) lse[row] = (M + log2f(den_row)) * 0.69314718055994530942f;
}

// Row counts at which the combine uses one wave per row, else four, else eight per
// quarter row (enough waves to fill 256 CUs either way).
constexpr long long kCombineManyRows = 2048;
constexpr long long kCombineFewRows = 512;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Per partial row: {m, l, 2^e, 0}, the 512 accumulators times 2^-e in fp16, and the top record
// {exact top probability (float bits), pool slot of its value row}; each region 256-byte aligned.
struct WorkspaceLayout {
  size_t ml_bytes, acc_bytes, top_bytes;
};

WorkspaceLayout workspace_layout(int B, int q_len, int H, int nsplit) {
  const size_t rows = (size_t)B * nsplit * q_len * H;
  return {align_up(rows * sizeof(float4), MLA_VERIFY_WORKSPACE_ALIGN),
          align_up(rows * kLatent * sizeof(uint16_t), MLA_VERIFY_WORKSPACE_ALIGN),
          align_up(rows * sizeof(int2), MLA_VERIFY_WORKSPACE_ALIGN)};
}

bool sizes_ok(int B, int q_len, int H) {
  if (B < 1 || q_len < 1 || H < 1) return false;
  const long long rows = (long long)q_len * H;
  return rows <= (1LL << 24) && (long long)B * rows <= (1LL << 30);
}

// Balanced workspace: the plan (split_info int32x4 [units], split_start int32 [B + 1]), then (m, l, 2^e),
// accumulators and top records for `units` partial row blocks, each region 256-byte aligned.
struct BalancedLayout {
  size_t plan_bytes, ml_bytes, acc_bytes, top_bytes;
};

BalancedLayout balanced_layout(int B, int q_len, int H, int units) {
  const size_t rows = (size_t)units * q_len * H;
  return {align_up((size_t)units * sizeof(int4) + (size_t)(B + 1) * sizeof(int), MLA_VERIFY_WORKSPACE_ALIGN),
          align_up(rows * sizeof(float4), MLA_VERIFY_WORKSPACE_ALIGN),
          align_up(rows * kLatent * sizeof(uint16_t), MLA_VERIFY_WORKSPACE_ALIGN),
          align_up(rows * sizeof(int2), MLA_VERIFY_WORKSPACE_ALIGN)};
}

bool balanced_sizes_ok(int B, int q_len, int H, int units) {
  return sizes_ok(B, q_len, H) && B <= MLA_VERIFY_BALANCED_MAX_B && units >= B && units <= MLA_VERIFY_MAX_UNITS &&
         (long long)units * q_len * H <= (1LL << 30);
}

}  // namespace

extern "C" size_t mla_verify_attn_workspace_size(int B, int q_len, int H, int nsplit) {
  if (!sizes_ok(B, q_len, H) || nsplit < 1 || nsplit > MLA_VERIFY_MAX_NSPLIT) return 0;
  const WorkspaceLayout lay = workspace_layout(B, q_len, H, nsplit);
  return lay.ml_bytes + lay.acc_bytes + lay.top_bytes;
}

extern "C" size_t mla_verify_attn_balanced_workspace_size(int B, int q_len, int H, int units) {
  if (!balanced_sizes_ok(B, q_len, H, units)) return 0;
  const BalancedLayout lay = balanced_layout(B, q_len, H, units);
  return lay.plan_bytes + lay.ml_bytes + lay.acc_bytes + lay.top_bytes;
}

extern "C" const char* mla_verify_status_string(int status) {
  switch (status) {
    case MLA_VERIFY_OK: return "ok";
    case MLA_VERIFY_ERR_NULL: return "a required pointer is NULL";
    case MLA_VERIFY_ERR_SHAPE: return "B, q_len, H or N out of range, or scale not finite and positive";
    case MLA_VERIFY_ERR_NSPLIT: return "nsplit outside [1, 1024]";
    case MLA_VERIFY_ERR_WORKSPACE: return "workspace NULL, misaligned or too small";
    case MLA_VERIFY_ERR_LAUNCH: return "kernel launch failed";
    case MLA_VERIFY_ERR_SCRATCH: return "sizes need more workspace than the no-alloc call's static scratch holds";
    default: return "unknown status";
  }
}

namespace {

struct Launch {
  float4* ws_ml;
  uint16_t* ws_acc;
  int2* ws_top;
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
  uint8_t* w = static_cast<uint8_t*>(workspace);
  return {reinterpret_cast<float4*>(w), reinterpret_cast<uint16_t*>(w + lay.ml_bytes),
          reinterpret_cast<int2*>(w + lay.ml_bytes + lay.acc_bytes), q_len * H};
}

// The partial kernels gather rows with 32-bit byte offsets from the pool base when every offset they
// form (at most N * 1152 - 1 including the immediate) fits in 32 bits, with 64-bit addresses otherwise.
bool narrow_pool(int64_t N) { return (uint64_t)N * kRowBytes <= (uint64_t(1) << 32); }

int launch_partial(const void* q_nope, const void* q_rope, const void* kv_pool, int64_t N,
                   const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* out_cache_loc,
                   const uint8_t* custom_mask, const int32_t* mask_indptr, int B, int q_len, int H,
                   float scale, int nsplit, const Launch& ws, hipStream_t stream) {
  const int n_rt = (ws.R + kRowsPerWG - 1) / kRowsPerWG;
  const long long grid = ((long long)B * nsplit + 7) / 8 * 8 * n_rt;
  if (grid > INT32_MAX) return MLA_VERIFY_ERR_SHAPE;
  const PartialArgs a = {static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(q_rope),
                         static_cast<const uint8_t*>(kv_pool), (int)N, kv_indptr, kv_indices, out_cache_loc,
                         custom_mask, mask_indptr, B, q_len, H, scale * 1.44269504088896340736f,
                         ws.ws_ml, ws.ws_acc, ws.ws_top};
  hipLaunchKernelGGL(narrow_pool(N) ? verify_partial_kernel<false> : verify_partial_kernel<true>, dim3((unsigned)grid),
                     dim3(kWaves * 64), 0, stream, a.q_nope, a.q_rope,
                     a.kv_pool, a.N, a.kv_indptr, a.kv_indices, a.out_cache_loc, a.custom_mask, a.mask_indptr, a.B,
                     a.q_len, a.H, a.scale_log2, nsplit, n_rt, a.ws_ml, a.ws_acc, a.ws_top);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

int launch_combine(const Launch& ws, const void* kv_pool, int64_t N, int B, int nsplit, void* out, float* lse,
                   hipStream_t stream) {
  const uint8_t* pool = static_cast<const uint8_t*>(kv_pool);
  const long long crows = (long long)B * ws.R;
  if (crows >= kCombineManyRows)
    hipLaunchKernelGGL((verify_combine_kernel<false, 1>), dim3((unsigned)((crows + 3) / 4)), dim3(256), 0, stream,
                       ws.ws_ml, ws.ws_acc, ws.ws_top, pool, (int)N, B, ws.R, nsplit, nullptr, static_cast<__bf16*>(out), lse);
  else if (crows >= kCombineFewRows)
    hipLaunchKernelGGL((verify_combine_kernel<false, 4>), dim3((unsigned)crows), dim3(256), 0, stream, ws.ws_ml,
                       ws.ws_acc, ws.ws_top, pool, (int)N, B, ws.R, nsplit, nullptr, static_cast<__bf16*>(out), lse);
  else
    hipLaunchKernelGGL((verify_combine_quarter_kernel<false>), dim3((unsigned)(4 * crows)), dim3(kQuarterWaves * 64), 0,
                       stream, ws.ws_ml, ws.ws_acc, ws.ws_top, pool, (int)N, B, ws.R, nsplit, nullptr, static_cast<__bf16*>(out),
                       lse);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

struct BalancedLaunch {
  int* split_start;
  int4* split_info;
  float4* ws_ml;
  uint16_t* ws_acc;
  int2* ws_top;
  int R;
};

int check_balanced(int B, int q_len, int H, int units, const void* workspace, size_t workspace_bytes) {
  if (!sizes_ok(B, q_len, H) || B > MLA_VERIFY_BALANCED_MAX_B) return MLA_VERIFY_ERR_SHAPE;
  if (units < B || units > MLA_VERIFY_MAX_UNITS) return MLA_VERIFY_ERR_NSPLIT;
  if (!balanced_sizes_ok(B, q_len, H, units)) return MLA_VERIFY_ERR_SHAPE;
  const size_t need = mla_verify_attn_balanced_workspace_size(B, q_len, H, units);
  if (!workspace || ((uintptr_t)workspace % MLA_VERIFY_WORKSPACE_ALIGN) != 0 || workspace_bytes < need)
    return MLA_VERIFY_ERR_WORKSPACE;
  return MLA_VERIFY_OK;
}

BalancedLaunch balanced_workspace(void* workspace, int B, int q_len, int H, int units) {
  const BalancedLayout lay = balanced_layout(B, q_len, H, units);
  uint8_t* w = static_cast<uint8_t*>(workspace);
  return {reinterpret_cast<int*>(w + (size_t)units * sizeof(int4)), reinterpret_cast<int4*>(w),
          reinterpret_cast<float4*>(w + lay.plan_bytes), reinterpret_cast<uint16_t*>(w + lay.plan_bytes + lay.ml_bytes),
          reinterpret_cast<int2*>(w + lay.plan_bytes + lay.ml_bytes + lay.acc_bytes), q_len * H};
}

int launch_balanced_partial(const void* q_nope, const void* q_rope, const void* kv_pool, int64_t N,
                            const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* out_cache_loc,
                            const uint8_t* custom_mask, const int32_t* mask_indptr, int B, int q_len, int H,
                            float scale, int units, const BalancedLaunch& ws, hipStream_t stream) {
  const int n_rt = (ws.R + kRowsPerWG - 1) / kRowsPerWG;
  const long long grid = ((long long)units + 7) / 8 * 8 * n_rt;
  if (grid > INT32_MAX) return MLA_VERIFY_ERR_SHAPE;
  const int fused = B <= kFusedPlanMaxB ? 1 : 0;
  if (!fused) {
    hipLaunchKernelGGL(verify_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, kv_indptr, B, q_len, units,
                       ws.split_start, ws.split_info);
    if (hipGetLastError() != hipSuccess) return MLA_VERIFY_ERR_LAUNCH;
  }
  hipLaunchKernelGGL(narrow_pool(N) ? verify_partial_balanced_kernel<false> : verify_partial_balanced_kernel<true>,
                     dim3((unsigned)grid), dim3(kWaves * 64), 0, stream,
                     static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(q_rope),
                     static_cast<const uint8_t*>(kv_pool), (int)N, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                     mask_indptr, B, q_len, H, scale * 1.44269504088896340736f, units, n_rt, fused,
                     (int4*)ws.split_info, (int*)ws.split_start, ws.ws_ml, ws.ws_acc, ws.ws_top);
  return hipGetLastError() == hipSuccess ? MLA_VERIFY_OK : MLA_VERIFY_ERR_LAUNCH;
}

int launch_balanced_combine(const BalancedLaunch& ws, const void* kv_pool, int64_t N, int B, int units, void* out,
                            float* lse, hipStream_t stream) {
  const uint8_t* pool = static_cast<const uint8_t*>(kv_pool);
  const long long crows = (long long)B * ws.R;
  if (crows >= kCombineManyRows)
    hipLaunchKernelGGL((verify_combine_kernel<true, 1>), dim3((unsigned)((crows + 3) / 4)), dim3(256), 0, stream,
                       ws.ws_ml, ws.ws_acc, ws.ws_top, pool, (int)N, B, ws.R, units, (const int*)ws.split_start, static_cast<__bf16*>(out), lse);
  else if (crows >= kCombineFewRows)
    hipLaunchKernelGGL((verify_combine_kernel<true, 4>), dim3((unsigned)crows), dim3(256), 0, stream, ws.ws_ml,
                       ws.ws_acc, ws.ws_top, pool, (int)N, B, ws.R, units, (const int*)ws.split_start, static_cast<__bf16*>(out), lse);
  else
    hipLaunchKernelGGL((verify_combine_quarter_kernel<true>), dim3((unsigned)(4 * crows)), dim3(kQuarterWaves * 64), 0,
                       stream, ws.ws_ml, ws.ws_acc, ws.ws_top, pool, (int)N, B, ws.R, units, (const int*)ws.split_start,
                       static_cast<__bf16*>(out), lse);
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
  if (!sizes_ok(B, q_len, H) || N < 1 || N > INT32_MAX || !(scale > 0.0f) || !isfinite(scale))
    return MLA_VERIFY_ERR_SHAPE;
  const int rc = check_common(B, q_len, H, nsplit, workspace, workspace_bytes);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_partial(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr,
                        B, q_len, H, scale, nsplit, split_workspace(workspace, B, q_len, H, nsplit), stream);
}

extern "C" int mla_verify_attn_combine(const void* workspace, size_t workspace_bytes, const void* kv_pool, int64_t N,
                                       int B, int q_len, int H, int nsplit, void* out, float* lse,
                                       hipStream_t stream) {
  if (!out || !lse || !kv_pool) return MLA_VERIFY_ERR_NULL;
  if (N < 1 || N > INT32_MAX) return MLA_VERIFY_ERR_SHAPE;
  const int rc = check_common(B, q_len, H, nsplit, workspace, workspace_bytes);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_combine(split_workspace(const_cast<void*>(workspace), B, q_len, H, nsplit), kv_pool, N, B, nsplit,
                        out, lse, stream);
}

extern "C" int mla_verify_attn(const void* q_nope, const void* q_rope, const void* kv_pool, int64_t N,
                               const int32_t* kv_indptr, const int32_t* kv_indices,
                               const int32_t* out_cache_loc, const uint8_t* custom_mask,
                               const int32_t* mask_indptr, int B, int q_len, int H, float scale,
                               int nsplit, void* workspace, size_t workspace_bytes, void* out, float* lse,
                               hipStream_t stream) {
  if (inputs_null(q_nope, q_rope, kv_pool, kv_indptr, out_cache_loc, custom_mask, mask_indptr) || !out || !lse)
    return MLA_VERIFY_ERR_NULL;
  if (!sizes_ok(B, q_len, H) || N < 1 || N > INT32_MAX || !(scale > 0.0f) || !isfinite(scale))
    return MLA_VERIFY_ERR_SHAPE;
  int rc = check_common(B, q_len, H, nsplit, workspace, workspace_bytes);
  if (rc != MLA_VERIFY_OK) return rc;
  const Launch ws = split_workspace(workspace, B, q_len, H, nsplit);
  rc = launch_partial(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr, B,
                      q_len, H, scale, nsplit, ws, stream);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_combine(ws, kv_pool, N, B, nsplit, out, lse, stream);
}

extern "C" int mla_verify_attn_balanced_partial(const void* q_nope, const void* q_rope, const void* kv_pool,
                                                int64_t N, const int32_t* kv_indptr, const int32_t* kv_indices,
                                                const int32_t* out_cache_loc, const uint8_t* custom_mask,
                                                const int32_t* mask_indptr, int B, int q_len, int H, float scale,
                                                int units, void* workspace, size_t workspace_bytes,
                                                hipStream_t stream) {
  if (inputs_null(q_nope, q_rope, kv_pool, kv_indptr, out_cache_loc, custom_mask, mask_indptr))
    return MLA_VERIFY_ERR_NULL;
  if (!sizes_ok(B, q_len, H) || N < 1 || N > INT32_MAX || !(scale > 0.0f) || !isfinite(scale))
    return MLA_VERIFY_ERR_SHAPE;
  const int rc = check_balanced(B, q_len, H, units, workspace, workspace_bytes);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_balanced_partial(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                                 mask_indptr, B, q_len, H, scale, units,
                                 balanced_workspace(workspace, B, q_len, H, units), stream);
}

extern "C" int mla_verify_attn_balanced_combine(const void* workspace, size_t workspace_bytes, const void* kv_pool,
                                                int64_t N, int B, int q_len, int H, int units, void* out, float* lse,
                                                hipStream_t stream) {
  if (!out || !lse || !kv_pool) return MLA_VERIFY_ERR_NULL;
  if (N < 1 || N > INT32_MAX) return MLA_VERIFY_ERR_SHAPE;
  const int rc = check_balanced(B, q_len, H, units, workspace, workspace_bytes);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_balanced_combine(balanced_workspace(const_cast<void*>(workspace), B, q_len, H, units), kv_pool, N, B,
                                 units, out, lse, stream);
}

extern "C" int mla_verify_attn_balanced(const void* q_nope, const void* q_rope, const void* kv_pool, int64_t N,
                                        const int32_t* kv_indptr, const int32_t* kv_indices,
                                        const int32_t* out_cache_loc, const uint8_t* custom_mask,
                                        const int32_t* mask_indptr, int B, int q_len, int H, float scale, int units,
                                        void* workspace, size_t workspace_bytes, void* out, float* lse,
                                        hipStream_t stream) {
  if (inputs_null(q_nope, q_rope, kv_pool, kv_indptr, out_cache_loc, custom_mask, mask_indptr) || !out || !lse)
    return MLA_VERIFY_ERR_NULL;
  if (!sizes_ok(B, q_len, H) || N < 1 || N > INT32_MAX || !(scale > 0.0f) || !isfinite(scale))
    return MLA_VERIFY_ERR_SHAPE;
  int rc = check_balanced(B, q_len, H, units, workspace, workspace_bytes);
  if (rc != MLA_VERIFY_OK) return rc;
  const BalancedLaunch ws = balanced_workspace(workspace, B, q_len, H, units);
  rc = launch_balanced_partial(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                               mask_indptr, B, q_len, H, scale, units, ws, stream);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_balanced_combine(ws, kv_pool, N, B, units, out, lse, stream);
}

// ---- the entry point that allocates nothing: mla_verify_attn_balanced on a static workspace

// The workspace of mla_verify_attn_balanced_noalloc. Each device the code object is loaded on has
// its own copy. In host code this name is a host-side stand-in, never a device address: the
// kernels get the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[MLA_VERIFY_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's copy of `scratch`, resolved on the first call there.
int scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_VERIFY_ERR_LAUNCH;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_VERIFY_ERR_LAUNCH;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return MLA_VERIFY_OK;
}

}  // namespace

extern "C" int mla_verify_attn_balanced_noalloc(const void* q_nope, const void* q_rope, const void* kv_pool,
                                                int64_t N, const int32_t* kv_indptr, const int32_t* kv_indices,
                                                const int32_t* out_cache_loc, const uint8_t* custom_mask,
                                                const int32_t* mask_indptr, int B, int q_len, int H, float scale,
                                                int units, void* out, float* lse, hipStream_t stream) {
  if (inputs_null(q_nope, q_rope, kv_pool, kv_indptr, out_cache_loc, custom_mask, mask_indptr) || !out || !lse)
    return MLA_VERIFY_ERR_NULL;
  if (!sizes_ok(B, q_len, H) || N < 1 || N > INT32_MAX || !(scale > 0.0f) || !isfinite(scale))
    return MLA_VERIFY_ERR_SHAPE;
  if (B > MLA_VERIFY_BALANCED_MAX_B) return MLA_VERIFY_ERR_SHAPE;
  if (units < B || units > MLA_VERIFY_MAX_UNITS) return MLA_VERIFY_ERR_NSPLIT;
  if (!balanced_sizes_ok(B, q_len, H, units)) return MLA_VERIFY_ERR_SHAPE;
  const size_t need = mla_verify_attn_balanced_workspace_size(B, q_len, H, units);
  if (need > MLA_VERIFY_NOALLOC_SCRATCH_BYTES) return MLA_VERIFY_ERR_SCRATCH;
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc != MLA_VERIFY_OK) return rc;
  const BalancedLaunch lw = balanced_workspace(ws, B, q_len, H, units);
  rc = launch_balanced_partial(q_nope, q_rope, kv_pool, N, kv_indptr, kv_indices, out_cache_loc, custom_mask,
                               mask_indptr, B, q_len, H, scale, units, lw, stream);
  if (rc != MLA_VERIFY_OK) return rc;
  return launch_balanced_combine(lw, kv_pool, N, B, units, out, lse, stream);
}
