// Device code for the paged KV-cache decode path on gfx950 (CDNA4).
//
// Work decomposition
//   A workgroup of NW wavefronts (64 lanes each) owns one (sequence, KV head)
//   pair -- and, in the split pass, one partition of that sequence's context.
//   The pair's query group (G = Hq / Hkv <= 16 query heads) is served by one
//   read of each K/V row, which is what makes grouped-query decode cheap
//   (nanoserve write-up, "What I built": one fused kernel walking the block
//   table with an online softmax).  Inside the workgroup the context is cut
//   into 16-token subtiles (one subtile never straddles a block, since block
//   sizes are multiples of 16); wave w takes tiles of NS subtiles round-robin
//   and keeps up to DEPTH of them in flight.
//
// Per subtile, per wave
//   * K rows: lane l loads 16 contiguous bytes of token (l % 16), dims
//     8*(l/16) + 32m .. +8.  That is exactly the A-operand layout of
//     v_mfma_f32_16x16x32_f16, so S^T = K Q^T is D/32 MFMAs with the query
//     group as the 16-wide B operand (zero-padded past G).  The result holds,
//     in lane l, the logits of head (l % 16) for tokens 4*(l/16) + 0..3.
//   * Online softmax in the exp2 domain (scale * log2 e folded into one fp32
//     multiply): the tile maximum per head needs one in-lane max and two
//     cross-lane exchanges; the running output is rescaled once per tile.
//   * P V: the probabilities already sit in the B-operand layout of
//     v_mfma_f32_16x16x16_f16 (k = token, column = head).  P is split into an
//     fp16 high part and an fp16 remainder and both are multiplied in, so the
//     product carries ~22 bits of P (plain fp16 P would cost up to 2^-11
//     relative error per weight, more than the fp16 output can absorb).  V
//     must be the transposed A operand (row = dim, k = token), so each
//     subtile of V goes through LDS: written row-major as loaded (masked
//     positions written as zeros, so a NaN in an unused slot never meets a
//     zero weight), read back with gfx950's transposing LDS read.
//   * Partial results of the NW waves merge through LDS at the end.
//
// All accumulation is fp32.  Positions past the context, or in a block whose
// id is outside [0, num_blocks), are excluded by select (never by a multiply
// with zero).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;
// Ticket counters of the fused step, one per 128-byte line: the tickets of
// different (sequence, KV head) pairs never contend for one line (measured:
// B=8 x 4096 with 16 partitions per pair, 12.0 -> 10.5 us).
constexpr int kCounterStride = 32;
constexpr float kLn2 = 0.69314718055994530942f;

// Merge groups of the fused step.  In the launches with more than
// kFlatMerge partitions per (sequence, KV head), a pair with more than that
// many merges in two levels: its np partitions form ng
// groups of gs consecutive partitions (the last may be smaller); the last
// workgroup of a group to take its ticket merges the group and stores the
// result in its own partition's row, and the last workgroup of all merges
// the group results.  Words 0-1 of the pair's counter line are one 64-bit
// ticket word holding a w-bit count per group, so a single atomic tells a
// workgroup both whether it closes its group and whether it closes the pair.
// Word kGroupRowWord + k carries group k's result row (partition + 1) from
// its merger to the pair's.  About 8 partitions per group, at most 16 groups
// (fewer when the counts would not fit 64 bits).
constexpr int kFlatMerge = 32;
constexpr int kMaxMergeGroups = 16;
constexpr int kGroupRowWord = 2;
struct MergeGroups {
  int ng;  // groups
  int gs;  // partitions per group (the last group: np - (ng - 1) * gs)
  int w;   // bits per group count in the ticket word
};
__host__ __device__ inline MergeGroups merge_groups(int np) {
  if (np <= kFlatMerge) return MergeGroups{1, np, 32 - __builtin_clz((unsigned)(np | 1))};
  int ng = (np + 7) / 8 < kMaxMergeGroups ? (np + 7) / 8 : kMaxMergeGroups;
  for (;; --ng) {
    const int gs = (np + ng - 1) / ng;
    const int n = (np + gs - 1) / gs;  // groups in use (none empty)
    const int w = 32 - __builtin_clz((unsigned)gs);  // counts 0 .. gs
    if (n * w <= 64 || n == 1) return MergeGroups{n, gs, w};
  }
}

struct AttnParams {
  const f16* q;
  const f16* k_pool;
  const f16* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  f16* out;             // unsplit: [B, Hq, D]
  float* partial_out;   // split:   [B, Hq, P_max, D]
  float* partial_lse;   // split:   [B, Hq, P_max]
  int32_t B, Hq, Hkv, G;
  int32_t block_size, num_blocks, max_blocks;
  int32_t partition_size, max_partitions;
  int32_t spb_shift;    // log2(block_size / 16) when a power of two, else -1
  int32_t part_shift;   // log2(partition_size) when a power of two, else -1
  int32_t bs_shift;     // log2(block_size) when a power of two, else -1
  float scale_log2;     // softmax scale * log2(e)
  // fused decode step only
  f16* k_pool_w;        // the pools, writable (the step's append)
  f16* v_pool_w;
  const f16* k_new;     // [B, Hkv, D] the step's new token per sequence
  const f16* v_new;
  const int64_t* slot_mapping;  // [B] or null (no append)
  int32_t* counters;    // [B, Hkv, kCounterStride] ticket words and group rows (8-byte
                        // aligned), zero between calls
  float* lse_out;       // [B, Hq] or null
};

struct ReduceParams {
  f16* out;
  float* lse_out;
  const float* partial_out;
  const float* partial_lse;
  const int32_t* context_lens;
  int32_t Hq, partition_size, max_partitions;
  int32_t B;
};

struct AppendParams {
  f16* k_pool;
  f16* v_pool;
  const f16* k_new;
  const f16* v_new;
  const int64_t* slot_mapping;
  int64_t num_slots;    // num_blocks * block_size
  int32_t num_tokens, Hkv, D;
};

__device__ __forceinline__ f16x8 zero8() {
  f16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (f16)0.0f;
  return z;
}

__device__ __forceinline__ f32x4 zero4f() {
  f32x4 z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = 0.0f;
  return z;
}

// x / d and x % d for x >= 0, with a shift when d is a power of two
// (sh = log2 d, else -1).
__device__ __forceinline__ int div_sh(int x, int d, int sh) { return sh >= 0 ? x >> sh : x / d; }
__device__ __forceinline__ int mod_sh(int x, int d, int sh) {
  return sh >= 0 ? x & ((1 << sh) - 1) : x % d;
}

// The value of lane l ^ 8 within each 16-lane row (a DPP row rotation by 8:
// a VALU move, no LDS round trip).
__device__ __forceinline__ float row_xor8(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

// 1 / x for a positive normal x (v_rcp_f32, within 1 ulp); 0 for x <= 0.
__device__ __forceinline__ float recip_or_zero(float x) {
  return x > 0.0f ? __builtin_amdgcn_rcpf(x) : 0.0f;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// Device-coherent 16-byte and 4-byte accesses for the fused step's partials
// (workgroups of one (sequence, KV head) may run on different XCDs, whose L2s
// are not coherent with each other): raw buffer instructions with the sc1
// cache-policy bit, which write through to, and read from, the device's
// coherence point.  Buffer accesses are also range-checked by the hardware:
// reads past the resource's end return 0, writes past it are dropped.
//
// Hand-off encoding.  A partial word is stored bit-inverted, and an all-zero
// word means "not written yet": the workspace rests at zero between calls
// (a zeroed buffer is ready to use), and a stored word is zero only for the
// all-ones pattern, which no computed value has (NaNs from fp16 inputs or
// from invalid operations carry other payloads; it is mapped to a quiet NaN
// anyway).  32-bit words are single-copy atomic, so a row some of whose
// words are still zero is seen as not written.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCoherent = 16;  // sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void store_coherent4(__amdgpu_buffer_rsrc_t rs, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kCoherent);
}
__device__ __forceinline__ void store_coherent1(__amdgpu_buffer_rsrc_t rs, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), rs, off, 0, kCoherent);
}
// Loads return through a bit cast to a float vector: element reads straight
// from the builtin's integer-vector result were narrowed to the wrong dword
// by this compiler.
__device__ __forceinline__ f32x4 load_coherent4(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCoherent));
}
__device__ __forceinline__ float load_coherent1(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kCoherent));
}
// Encode a value for the hand-off (never the all-zero word), and back.
__device__ __forceinline__ float encode_partial(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  return __builtin_bit_cast(float, u == 0xFFFFFFFFu ? ~0x7FC00000u : ~u);
}
__device__ __forceinline__ float decode_partial(float w) {
  return __builtin_bit_cast(float, ~__builtin_bit_cast(unsigned, w));
}
__device__ __forceinline__ bool is_written(float w) { return __builtin_bit_cast(unsigned, w) != 0u; }
__device__ __forceinline__ bool row_written(f32x4 x, float l) {
  return is_written(x[0]) && is_written(x[1]) && is_written(x[2]) && is_written(x[3]) &&
         is_written(l);
}

// Streaming loads through buffer resources.  A load past the resource's
// range reads zeros without a memory access, so a masked-out row (a subtile
// past the context, a block id out of range, a tile past the wave's last)
// is a load with an empty resource rather than a branch around the load.
// Every path through the decode loop then issues the same loads in the same
// order, which keeps the compiler's in-order wait counts exact: a wait for
// one tile never has to drain the tiles requested after it.
// A byte offset past every resource it is used with (each spans < 2^30
// bytes), with room for small immediate offsets on top.
constexpr int kOutOfRange = 0x40000000;

__device__ __forceinline__ f32x4 load_b128(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}
__device__ __forceinline__ f16x8 load_rows16(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f16x8, load_b128(rs, off));
}
// Eight query values; `sign` is 0x80008000 to negate them (flipping fp16
// sign bits is exact), else 0.  Lanes whose column holds no query head read
// past the resource and get zeros.
__device__ __forceinline__ f16x8 load_q16(__amdgpu_buffer_rsrc_t rs, int off, unsigned sign) {
  u32x4 w = __builtin_bit_cast(u32x4, load_b128(rs, off));
  w ^= sign;
  return __builtin_bit_cast(f16x8, w);
}

// LDS bytes one wave uses: V staging during the loop, merge buffers after.
template <int D, int NS>
struct AttnSmem {
  static constexpr int kRow = D + 4;                   // halves; 8-B aligned rows
  static constexpr int kStageHalves = NS * 16 * kRow;
  static constexpr int kMergeFloats = (D / 4) * 64 + 32;
  static constexpr int kWaveBytes =
      (kStageHalves * 2 > kMergeFloats * 4 ? kStageHalves * 2 : kMergeFloats * 4);
};

// The running maximum used as the softmax reference moves only when a tile's
// maximum exceeds it by more than this (log2 units), so probabilities stay
// <= 2^8 and the accumulators are rescaled only a few times per sequence.
constexpr float kRescaleLog2 = 8.0f;

// K and V registers of one tile (NS subtiles of 16 tokens) of one wave.
template <int D, int NS>
struct KVTile {
  f16x8 k[NS][D / 32];
  f16x8 v[NS][D / 32];
  int okmask;  // bit j: subtile j was loaded (valid block id, inside the range)
  int s0;
  int new_phys;  // block id of subtile s_new when the tile holds it, else -1
  bool full;   // every position of the tile is attended: no masking needed
};

// Physical block ids of the NS subtiles starting at subtile s0, one per lane
// (lanes 0..NS-1; 0 at or past subtile `limit`, where the caller masks the
// subtile anyway).  One vector load per wave through the resource of the
// sequence's table row (max_blocks * 4 bytes).
template <int NS>
__device__ __forceinline__ int load_block_ids(__amdgpu_buffer_rsrc_t bt_rs, int s0, int limit,
                                              int spb, int spb_shift, int lane) {
  const int s = s0 + (lane & (NS - 1));
  const int blk = spb_shift >= 0 ? (s >> spb_shift) : (s / spb);
  const int off = (lane < NS && s < limit) ? blk * 4 : kOutOfRange;
  return __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(bt_rs, off, 0, 0));
}

// Block ids of a tile's subtiles either as one register (lane j holds
// subtile j's id, from load_block_ids) or as wave-uniform scalars.
template <int NS>
struct ScalarIds {
  int v[NS];
};
__device__ __forceinline__ int block_id_of(int ids, int j) {
  return __builtin_amdgcn_readlane(ids, j);
}
template <int NS>
__device__ __forceinline__ int block_id_of(const ScalarIds<NS>& ids, int j) {
  return ids.v[j];
}

// Issue the K/V loads of one tile.  A subtile past sub_end, or in a block
// whose id is outside [0, num_blocks), is loaded through an empty resource
// (zeros, no memory access) and masked out.  Each subtile's resource starts
// at its first token's row of head kvh and spans the subtile (16 tokens x
// all heads); lane_off_b is the lane's fixed byte offset in it.
template <int D, int NS, typename Ids>
__device__ __forceinline__ void load_kv_tile(KVTile<D, NS>& T, const AttnParams& a,
                                             const Ids& ids, int s0, int sub_end, int t_end,
                                             int spb, int spb_shift, int64_t tok_stride, int kvh,
                                             int lane_off_b, int s_new = -1) {
  constexpr int KC = D / 32;
  const int sub_bytes = 32 * (int)tok_stride;
  T.s0 = s0;
  int okm = 0;
  int new_phys = -1;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int phys = block_id_of(ids, j);
    new_phys = s0 + j == s_new ? phys : new_phys;
    const bool ok = s0 + j < sub_end && phys >= 0 && phys < a.num_blocks;
    okm |= (ok ? 1 : 0) << j;
    const int s = s0 + j;
    const int sib = spb_shift >= 0 ? (s & (spb - 1)) : (s % spb);
    const int64_t blk_off =
        ((int64_t)(ok ? phys : 0) * a.block_size + sib * 16) * tok_stride + (int64_t)kvh * D;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(a.k_pool + blk_off, ok ? sub_bytes : 0);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(a.v_pool + blk_off, ok ? sub_bytes : 0);
#pragma unroll
    for (int m = 0; m < KC; ++m) {
      T.k[j][m] = load_rows16(kr, lane_off_b + 64 * m);
      T.v[j][m] = load_rows16(vr, lane_off_b + 64 * m);
    }
  }
  T.okmask = okm;
  T.new_phys = new_phys;
  T.full = okm == (1 << NS) - 1 && ((s0 + NS) << 4) <= t_end;
}

// Decode-path K/V loads: whole 128-byte lines per instruction, non-temporal.
// Eight consecutive lanes (sixteen at head_dim 128) read one token's head row
// of D halves in 16-byte chunks, so one wave-wide load covers 64 / (D / 8)
// whole rows (1 KiB).  Measured with a read-only probe of this machine layout
// (B=32 x 4096 at head_dim 64, random block tables, 64 MiB per launch): 16
// rows x 64 bytes per instruction -- the MFMA operand layout -- read in
// 13.5 us; whole rows per instruction with the non-temporal bit in 11.9 us
// (either change alone: 13.2 and 13.8 us).  The rows are then staged in LDS
// and read back in the MFMA layouts: K with 16-byte reads, V with the
// transposing read.  In LDS a row's chunk slot s holds chunk s ^ (row & 7),
// so the eight rows one 8-lane group of a K read touches hit distinct banks;
// the swizzle is applied on the load side (each lane loads the chunk its
// slot holds), which keeps each LDS write a plain 1 KiB contiguous store.
template <int D>
struct LineMap {
  static constexpr int kChunksPerRow = D / 8;          // 16-byte chunks of a head row
  static constexpr int kRowsPerLoad = 64 / kChunksPerRow;
  static constexpr int kLoads = D / 32;                // wave loads per 16-row subtile
  // row (within the subtile) and global chunk of lane's load m
  static __device__ __forceinline__ int row(int lane, int m) {
    return kRowsPerLoad * m + lane / kChunksPerRow;
  }
  static __device__ __forceinline__ int chunk(int lane, int m) {
    return (lane % kChunksPerRow) ^ (row(lane, m) & 7);
  }
};

template <int D, int NS>
struct LineSmem {
  static constexpr int kSubBytes = 16 * D * 2;           // one subtile of K (or V)
  static constexpr int kStageBytes = 2 * NS * kSubBytes;  // K subtiles, then V subtiles
  static constexpr int kMergeBytes = ((D / 4) * 64 + 32) * 4;  // the waves' merge
  static constexpr int kWaveBytes = kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes;
};

constexpr int kNonTemporal = 2;  // cache-policy bit of the streaming K/V loads

__device__ __forceinline__ f16x8 load_line16(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(
      f16x8, __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0,
                                                                              kNonTemporal)));
}

// Issue the K/V loads of one tile in the line layout above.  Each subtile's
// resource starts at its first token's row of head kvh and ends right after
// the head row of its last attended token, so rows past the context (and
// every row of a subtile past sub_end or in a block whose id is outside
// [0, num_blocks)) read as zeros without a memory access: V needs no
// masking, K's logits are masked by select.  lane_off[m] is the lane's byte
// offset of load m in a resource.
template <int D, int NS, typename Ids>
__device__ __forceinline__ void load_kv_lines(KVTile<D, NS>& T, const AttnParams& a,
                                              const Ids& ids, int s0, int sub_end, int t_end,
                                              int spb, int spb_shift, int64_t tok_stride,
                                              int kvh, const int (&lane_off)[D / 32],
                                              int s_new) {
  constexpr int KC = D / 32;
  T.s0 = s0;
  int okm = 0;
  int new_phys = -1;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int phys = block_id_of(ids, j);
    new_phys = s0 + j == s_new ? phys : new_phys;
    const bool ok = s0 + j < sub_end && phys >= 0 && phys < a.num_blocks;
    okm |= (ok ? 1 : 0) << j;
    const int s = s0 + j;
    const int sib = spb_shift >= 0 ? (s & (spb - 1)) : (s % spb);
    const int nvalid = ok ? min(16, t_end - (s << 4)) : 0;  // >= 1 when ok
    const int bytes = ok ? ((nvalid - 1) * (int)tok_stride + D) * 2 : 0;
    const int64_t blk_off =
        ((int64_t)(ok ? phys : 0) * a.block_size + sib * 16) * tok_stride + (int64_t)kvh * D;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(a.k_pool + blk_off, bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(a.v_pool + blk_off, bytes);
#pragma unroll
    for (int m = 0; m < KC; ++m) {
      T.k[j][m] = load_line16(kr, lane_off[m]);
      T.v[j][m] = load_line16(vr, lane_off[m]);
    }
  }
  T.okmask = okm;
  T.new_phys = new_phys;
  T.full = okm == (1 << NS) - 1 && ((s0 + NS) << 4) <= t_end;
}

// Online-softmax state of one wave: reference maximum (log2 domain) per head
// column, and the O^T and weight-sum accumulators (MFMA layout: lane
// (quad, g) holds rows 4*quad + v of column g).
template <int D>
struct SoftmaxState {
  f32x4 o[D / 16];
  f32x4 lsum;  // row 0 of column g = sum of the column's weights
  float m;
};

// Maximum over the two lanes l and l^16, then over l^32 (gfx950 row swaps).
__device__ __forceinline__ float max_across_quads(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// QK^T, online-softmax update and PV for one loaded tile.
//   DUAL (G <= 8): MFMA columns 0..7 carry the query heads with P rounded to
//   fp16, columns 8..15 the same heads with the fp16 remainder P - fp16(P),
//   so one PV MFMA per 16 dims takes both parts; the two column halves are
//   summed once at the end.  Otherwise (G <= 16) each part has its own MFMA.
//   Tiles where every position is attended skip all masking.
//   c = |scale| * log2(e) > 0 (a negative scale is folded into q; a zero
//   scale is raised to the smallest normal float, which keeps masked logits
//   at -inf and rounds every weight of a uniform softmax to exactly 1).
//   ones: the A operand with row 0 all ones, so one more MFMA per part sums
//   the weights of every column (no per-value VALU adds).
//   rem_mul: with DUAL, -1 in the remainder columns, else 0 (selects P or
//   P - fp16(P) with one exact fused multiply-add); without DUAL, -1 (the
//   remainder's multiplier).  Opaque to the compiler, so the remainder stays
//   one mixed-precision FMA rather than a convert, a subtract and a convert.
//   SUB: position (s_new, tok_new) takes K/V from kn/vn (the fused step's new
//   token, which this launch also writes to the pool) when `slot` is the
//   position's slot in the table: T.new_phys * block_size + new_off.
template <int D, int NS, bool DUAL, bool SUB>
__device__ __forceinline__ void consume_tile(KVTile<D, NS>& T, SoftmaxState<D>& st,
                                             const f16x8 (&qb)[D / 32], f16* stage, float c,
                                             int t_end, int lane, f16x4 ones, float rem_mul,
                                             int s_new, int tok_new, int64_t slot, int new_off,
                                             int block_size,
                                             const f16x8 (&kn)[D / 32],
                                             const f16x8 (&vn)[D / 32]) {
  constexpr int KC = D / 32;
  constexpr int NDB = D / 16;
  const int g = lane & 15;
  const int quad = lane >> 4;
  using LM = LineMap<D>;
  using LS = LineSmem<D, NS>;
  if (SUB && T.new_phys >= 0 && (int64_t)T.new_phys * block_size + new_off == slot) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
      for (int m = 0; m < KC; ++m) {
        const bool mine = T.s0 + j == s_new && LM::row(lane, m) == tok_new;
        T.k[j][m] = mine ? kn[m] : T.k[j][m];
        T.v[j][m] = mine ? vn[m] : T.v[j][m];
      }
    }
  }

  // K and V of the tile to LDS as loaded: load m of subtile j is 1 KiB of
  // whole rows, lane l's chunk at byte 16 l.
  unsigned char* kst = reinterpret_cast<unsigned char*>(stage);
  unsigned char* vst = kst + NS * LS::kSubBytes;
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int m = 0; m < KC; ++m) {
      *reinterpret_cast<f16x8*>(kst + j * LS::kSubBytes + m * 1024 + 16 * lane) = T.k[j][m];
      *reinterpret_cast<f16x8*>(vst + j * LS::kSubBytes + m * 1024 + 16 * lane) = T.v[j][m];
    }
  asm volatile("" ::: "memory");

  // raw logits S^T[token][column]; K in the A layout: lane l holds token
  // l % 16, dims 8 (l / 16) + 32 m .. + 8 (chunk l / 16 + 4 m, swizzled).
  f32x4 sc[NS];
  {
    const int t = lane & 15;
    const unsigned char* krow = kst + t * (D * 2);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      f32x4 acc = zero4f();
#pragma unroll
      for (int m = 0; m < KC; ++m) {
        const int ch = ((lane >> 4) + 4 * m) ^ (t & 7);
        const f16x8 kk =
            *reinterpret_cast<const f16x8*>(krow + j * LS::kSubBytes + 16 * ch);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kk, qb[m], acc, 0, 0, 0);
      }
      sc[j] = acc;
    }
  }
  if (!T.full) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = ((T.s0 + j) << 4) + 4 * quad + v;
        sc[j][v] = (((T.okmask >> j) & 1) && tok < t_end) ? sc[j][v] : -INFINITY;
      }
    }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) tmax = fmaxf(tmax, sc[j][v]);
  tmax = max_across_quads(tmax);
  const float tmax_s = tmax * c;  // c > 0: -inf stays -inf
  const bool grow = tmax_s > st.m + kRescaleLog2;
  if (__any(grow)) {
    const float m_new = grow ? tmax_s : st.m;
    const float alpha = fast_exp2(st.m - m_new);  // 1 where unchanged, 0 from -inf
    st.m = m_new;
    st.lsum *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i) st.o[i] *= alpha;
  }
  const float neg_m = (st.m == -INFINITY) ? 0.0f : -st.m;

  f16x4 ph[NS], pl[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    float pv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pv[v] = fast_exp2(fmaf(sc[j][v], c, neg_m));  // masked: exp2(-inf) = 0
    }
#pragma unroll
    for (int v = 0; v < 4; v += 2) {
      const f16 h0 = (f16)pv[v], h1 = (f16)pv[v + 1];
      if (DUAL) {
        ph[j][v] = (f16)fmaf((float)h0, rem_mul, pv[v]);
        ph[j][v + 1] = (f16)fmaf((float)h1, rem_mul, pv[v + 1]);
      } else {
        ph[j][v] = h0;
        ph[j][v + 1] = h1;
        pl[j][v] = (f16)fmaf((float)h0, rem_mul, pv[v]);
        pl[j][v + 1] = (f16)fmaf((float)h1, rem_mul, pv[v + 1]);
      }
    }
  }

  // V^T operand by transposing LDS reads: within each 16-lane group, lane i
  // of ds_read_b64_tr_b16 receives element (i % 4) of the 8-byte chunks that
  // lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4 point at.  Lane j of quad q points
  // at V[4q + j/4][16 db + 4 (j%4) ..], so lane (q, i) receives
  // V[4q + k][16 db + i] for k = 0..3: the A operand of the 16x16x16 MFMA.
  // Without DUAL both parts of P go into one 16x16x32 MFMA: its lane (q, i)
  // holds k = 8q .. 8q + 7, taken as the lane's 4 tokens' high parts then
  // their remainders (B), against the same 4 V values twice (A).  Rows past
  // the context were loaded as zeros, so a zero weight never meets a NaN.
  const int vr = 4 * quad + (g >> 2);
  const unsigned char* vrow = vst + vr * (D * 2) + 8 * (g & 1);
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const f16x8 pb = __builtin_shufflevector(ph[j], pl[j], 0, 1, 2, 3, 4, 5, 6, 7);
    if (DUAL)
      st.lsum = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, ph[j], st.lsum, 0, 0, 0);
    else
      st.lsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_shufflevector(ones, ones, 0, 1, 2, 3, 4, 5, 6, 7), pb, st.lsum, 0, 0, 0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      const int ch = (2 * db + ((g & 3) >> 1)) ^ (vr & 7);
      const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vrow + j * LS::kSubBytes + 16 * ch));
      const f16x4 va = __builtin_bit_cast(f16x4, raw);
      if (DUAL)
        st.o[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, ph[j], st.o[db], 0, 0, 0);
      else
        st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_shufflevector(va, va, 0, 1, 2, 3, 0, 1, 2, 3), pb, st.o[db], 0, 0, 0);
    }
  }
  asm volatile("" ::: "memory");  // next tile's LDS writes stay after these reads
}

// Merge of the NW waves' partial results through LDS; calls emit(db, acc, L,
// M) for the column blocks this wave finalises.
template <int D, int NW, typename Emit>
__device__ __forceinline__ void merge_waves_impl(const SoftmaxState<D>& st, float l_tot,
                                                 unsigned char* smem, int wave_bytes, int wave,
                                                 int lane, Emit& emit) {
  constexpr int NDB = D / 16;
  const int g = lane & 15;
  const int quad = lane >> 4;
  __syncthreads();  // every wave is done with its staging area
  float* mine = reinterpret_cast<float*>(smem + wave * wave_bytes);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 4; ++v) mine[(db * 4 + v) * 64 + lane] = st.o[db][v];
  if (quad == 0) {
    mine[NDB * 4 * 64 + g] = st.m;
    mine[NDB * 4 * 64 + 16 + g] = l_tot;
  }
  __syncthreads();

  for (int db = wave; db < NDB; db += NW) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* theirs = reinterpret_cast<const float*>(smem + w * wave_bytes);
      M = fmaxf(M, theirs[NDB * 4 * 64 + g]);
    }
    const float mu = (M == -INFINITY) ? 0.0f : M;
    float L = 0.0f;
    f32x4 acc = zero4f();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* theirs = reinterpret_cast<const float*>(smem + w * wave_bytes);
      const float e = fast_exp2(theirs[NDB * 4 * 64 + g] - mu);
      L += e * theirs[NDB * 4 * 64 + 16 + g];
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += e * theirs[(db * 4 + v) * 64 + lane];
    }
    emit(db, acc, L, M);
  }
}

constexpr int kMergeSlots = 512;  // >= 16 heads x 128/4 dims
constexpr int kMergeRowsInFlight = 8;  // the merge's largest batch of partition rows per thread
// One-level fused-step launches with at most this many partitions per pair
// take MODE 4: each merging thread takes every partition of its (head,
// 4 dims) in one batch and writes the output itself, with no LDS staging and
// no barrier (measured faster at 4 partitions, slower at 8, and slower
// everywhere when both merges share one instantiation).
constexpr int kDirectMergeItems = 4;
// The merger's wait for the other workgroups' rows is bounded in time: a
// workspace that breaks its contract (rows reset under a running writer, a
// stale counter) costs at most this long and gives wrong numbers, never a
// stalled queue.  Legitimate waits end within microseconds (every writer has
// started and waits on nothing).  s_memrealtime counts at 100 MHz: 20 ms.
constexpr long long kSpinTicks = 2000000;

// Streaming LSE merge of one thread's items (grp, grp + ngroups, ... of the
// n items; item q is partial row rowtbl[q], or row0 + q without the table)
// for head hh, dims 4cc..4cc+3, into (M, L, acc), BATCH rows in flight.
// Item q_own is the merging workgroup's own partial (own_x, own_l), not read.
template <int D, int BATCH>
__device__ __forceinline__ void merge_rows(__amdgpu_buffer_rsrc_t po_rs,
                                           __amdgpu_buffer_rsrc_t pl_rs, int Pm, int n,
                                           int q_own, const int* rowtbl, bool use_tbl, int row0,
                                           int grp, int ngroups, int hh, int cc, f32x4 own_x,
                                           float own_l, float& M, float& L, f32x4& acc) {
  for (int q0 = grp; q0 < n; q0 += BATCH * ngroups) {
    // Straight-line code for the common case: every row of the batch is
    // requested at once (items past n, the merger's own, and rows outside
    // [0, Pm) through an out-of-range offset: zeros, no memory access),
    // checked with one vector test, and merged with selects.  Rows not
    // written yet are requested again in a wave-uniform loop, the only
    // branch.
    int xo[BATCH], lo[BATCH];
    f32x4 x[BATCH];
    float l[BATCH];
    bool ok[BATCH], other[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int q = q0 + j * ngroups;
      other[j] = q < n && q != q_own;
      // rows of the table come from other workgroups (checked); the others
      // are partitions of this launch
      const int r = use_tbl ? rowtbl[other[j] ? q : 0] : row0 + q;
      const bool in = other[j] && (!use_tbl || (r >= 0 && r < Pm));
      xo[j] = in ? ((hh * Pm + r) * D + 4 * cc) * 4 : kOutOfRange;
      lo[j] = in ? (hh * Pm + r) * 4 : kOutOfRange;
      x[j] = load_coherent4(po_rs, xo[j]);
      l[j] = load_coherent1(pl_rs, lo[j]);
    }
    bool all_ok = true;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      ok[j] = !other[j] || row_written(x[j], l[j]);
      all_ok = all_ok && ok[j];
    }
    const long long t_spin = __all(all_ok) ? 0 : (long long)__builtin_amdgcn_s_memrealtime();
    while (!__all(all_ok) &&
           (long long)__builtin_amdgcn_s_memrealtime() - t_spin < kSpinTicks) {
      __builtin_amdgcn_s_sleep(1);
      asm volatile("" ::: "memory");
      // Every re-request is issued before any is waited for (one memory
      // round trip per poll, not one per row); rows already seen go through
      // the out-of-range offset.
      f32x4 nx[BATCH];
      float nl[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        nx[j] = load_coherent4(po_rs, ok[j] ? kOutOfRange : xo[j]);
        nl[j] = load_coherent1(pl_rs, ok[j] ? kOutOfRange : lo[j]);
      }
      all_ok = true;
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
#pragma unroll
        for (int v = 0; v < 4; ++v) x[j][v] = ok[j] ? x[j][v] : nx[j][v];
        l[j] = ok[j] ? l[j] : nl[j];
        ok[j] = !other[j] || row_written(x[j], l[j]);
        all_ok = all_ok && ok[j];
      }
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int q = q0 + j * ngroups;
      const bool mine = q == q_own;
      f32x4 xd;
#pragma unroll
      for (int v = 0; v < 4; ++v) xd[v] = decode_partial(x[j][v]);
      const float lq = q < n ? (mine ? own_l : decode_partial(l[j])) : -INFINITY;
      const f32x4 xq = mine ? own_x : (other[j] ? xd : zero4f());
      const float Mn = fmaxf(M, lq);
      const float mu = Mn == -INFINITY ? 0.0f : Mn;
      const float sa = fast_exp2((M - mu) * kLog2e);  // 1 while M holds; 0 from -inf
      const float sb = fast_exp2((lq - mu) * kLog2e);  // 0 for items past n
      acc = acc * sa + xq * sb;
      L = L * sa + sb;
      M = Mn;
    }
  }
}

// The direct merge of n <= NO + 1 partitions (one level, no table): only the
// other partitions' rows are requested, NO at once; the merge then takes the
// items in partition order, the own partial at its place.
template <int D, int NO>
__device__ __forceinline__ void merge_direct_others(__amdgpu_buffer_rsrc_t po_rs,
                                                    __amdgpu_buffer_rsrc_t pl_rs, int Pm, int n,
                                                    int q_own, int hh, int cc, f32x4 own_x,
                                                    float own_l, float& M, float& L,
                                                    f32x4& acc) {
  int xo[NO], lo[NO];
  f32x4 x[NO];
  float l[NO];
  bool ok[NO], other[NO];
#pragma unroll
  for (int j = 0; j < NO; ++j) {
    const int q = j < q_own ? j : j + 1;
    other[j] = q < n;
    xo[j] = other[j] ? ((hh * Pm + q) * D + 4 * cc) * 4 : kOutOfRange;
    lo[j] = other[j] ? (hh * Pm + q) * 4 : kOutOfRange;
    x[j] = load_coherent4(po_rs, xo[j]);
    l[j] = load_coherent1(pl_rs, lo[j]);
  }
  bool all_ok = true;
#pragma unroll
  for (int j = 0; j < NO; ++j) {
    ok[j] = !other[j] || row_written(x[j], l[j]);
    all_ok = all_ok && ok[j];
  }
  const long long t_spin = __all(all_ok) ? 0 : (long long)__builtin_amdgcn_s_memrealtime();
  while (!__all(all_ok) &&
         (long long)__builtin_amdgcn_s_memrealtime() - t_spin < kSpinTicks) {
    __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
    f32x4 nx[NO];
    float nl[NO];
#pragma unroll
    for (int j = 0; j < NO; ++j) {
      nx[j] = load_coherent4(po_rs, ok[j] ? kOutOfRange : xo[j]);
      nl[j] = load_coherent1(pl_rs, ok[j] ? kOutOfRange : lo[j]);
    }
    all_ok = true;
#pragma unroll
    for (int j = 0; j < NO; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) x[j][v] = ok[j] ? x[j][v] : nx[j][v];
      l[j] = ok[j] ? l[j] : nl[j];
      ok[j] = !other[j] || row_written(x[j], l[j]);
      all_ok = all_ok && ok[j];
    }
  }
#pragma unroll
  for (int q = 0; q <= NO; ++q) {
    const bool mine = q == q_own;
    const int j = q < q_own ? q : (q > 0 ? q - 1 : 0);
    f32x4 xd;
#pragma unroll
    for (int v = 0; v < 4; ++v) xd[v] = decode_partial(x[j][v]);
    const float lq = q < n ? (mine ? own_l : decode_partial(l[j])) : -INFINITY;
    const f32x4 xq = mine ? own_x : (q < n ? xd : zero4f());
    const float Mn = fmaxf(M, lq);
    const float mu = Mn == -INFINITY ? 0.0f : Mn;
    const float sa = fast_exp2((M - mu) * kLog2e);
    const float sb = fast_exp2((lq - mu) * kLog2e);
    acc = acc * sa + xq * sb;
    L = L * sa + sb;
    M = Mn;
  }
}

// The ticket word of (b, kvh) (words 0-1 of its counter line).
__device__ __forceinline__ unsigned long long* step_ticket_word(const AttnParams& a, int b,
                                                                int kvh) {
  return reinterpret_cast<unsigned long long*>(a.counters +
                                               ((size_t)b * a.Hkv + kvh) * kCounterStride);
}
// Partition p's ticket: the ticket word before its own count is added.
// The groups are worked out here and again once the ticket is back, so that
// nothing of them stays live across the K/V loop.
// Launches with one level count in the word's low half only.
template <bool TWO>
__device__ __forceinline__ unsigned long long take_step_ticket(const AttnParams& a, int b,
                                                               int kvh, int np, int p) {
  if (!TWO)
    return __hip_atomic_fetch_add(reinterpret_cast<unsigned*>(step_ticket_word(a, b, kvh)), 1u,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const MergeGroups mg = merge_groups(np);
  return __hip_atomic_fetch_add(step_ticket_word(a, b, kvh), 1ull << (mg.w * (p / mg.gs)),
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// What partition p does once its ticket is back (thread 0): 0 stores its
// partial; 1 merges its group and stores the result in its own row (whose
// index it then publishes); 2 merges its group and then the pair (the pair's
// last ticket: the ticket word goes back to zero at once, every ticket of
// this launch being taken).
template <bool TWO>
__device__ __forceinline__ int step_merge_role(const AttnParams& a, int b, int kvh, int np,
                                               int p, unsigned long long ticket) {
  if (!TWO) {
    if ((unsigned)ticket != (unsigned)(np - 1)) return 0;
    __hip_atomic_store(reinterpret_cast<unsigned*>(step_ticket_word(a, b, kvh)), 0u,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return 2;
  }
  asm volatile("" : "+s"(np));  // recomputed, not kept from the ticket's request
  const MergeGroups mg = merge_groups(np);
  const int k = p / mg.gs;
  const int gk = min(mg.gs, np - k * mg.gs);
  const unsigned long long mask = (1ull << mg.w) - 1;
  if ((int)((ticket >> (mg.w * k)) & mask) != gk - 1) return 0;
  unsigned long long full = 0;
  for (int j = 0; j < mg.ng; ++j)
    full += (unsigned long long)min(mg.gs, np - j * mg.gs) << (mg.w * j);
  if (ticket + (1ull << (mg.w * k)) == full) {
    __hip_atomic_store(step_ticket_word(a, b, kvh), 0ull, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    return 2;
  }
  __hip_atomic_store(a.counters + ((size_t)b * a.Hkv + kvh) * kCounterStride + kGroupRowWord + k,
                     p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 1;
}

// The merges of the fused step by partition p of (b, kvh), whose role (1 or
// 2, step_merge_role) says which: its group's, and for role 2 then the
// pair's, over the group results (the group mergers' rows, polled from the
// counter line; its own group's result stays in LDS).  With one group the
// group's merge is the pair's.
// Each merge covers n items (item q_own is the workgroup's own partial, in
// LDS at `own`), every other item's row polled until none of its words is
// still unwritten and set back to unwritten for the next launch once read.
// Threads cover (head, 4 dims) x item groups with a streaming LSE merge, and
// the item groups combine through LDS; with DIRECT (one level, at most
// kDirectMergeItems items), one thread takes every item of its (head,
// 4 dims) and writes the result itself.  Results do not depend on which
// workgroups merge: items are merged in partition, then group, order.
// The waits end: the workgroups whose rows are read took their tickets
// before this one took its last, so they are running and wait on nothing.
template <int D, int NW, bool TWO, bool DIRECT = false>
__device__ void merge_step_partitions(const AttnParams& a, int b, int kvh, int np, int p,
                                      int role, float* own /* [16][D] o, then [16] lse */,
                                      float* msm /* 6 * kMergeSlots floats */,
                                      int* rowtbl /* kMaxMergeGroups */) {
  static_assert(!(TWO && DIRECT), "the direct merge is one-level");
  constexpr int NT = NW * 64;
  constexpr int TPR = D / 4;
  const int t = threadIdx.x;
  const int G = a.G;
  const int Pm = a.max_partitions;
  const size_t head0 = (size_t)b * a.Hq + kvh * G;
  const __amdgpu_buffer_rsrc_t po_rs = buffer_rsrc(a.partial_out + head0 * Pm * D, G * Pm * D * 4);
  const __amdgpu_buffer_rsrc_t pl_rs = buffer_rsrc(a.partial_lse + head0 * Pm, G * Pm * 4);
  if (TWO) asm volatile("" : "+s"(np));  // recomputed, not kept from the ticket's request
  const MergeGroups mg = TWO ? merge_groups(np) : MergeGroups{1, np, 0};
  const int k = TWO ? p / mg.gs : 0;
  const int lo = k * mg.gs;
  int32_t* rows_w = a.counters + ((size_t)b * a.Hkv + kvh) * kCounterStride + kGroupRowWord;

  // The first merge: the whole pair (one group), or this workgroup's group.
  // out: 0 the step's output, 1 the group result into this partition's row,
  // 2 the group result into LDS (then the merge of the groups).
  const bool flat = !TWO || mg.ng == 1;
  int n = flat ? np : min(mg.gs, np - lo);
  int q_own = flat ? p : p - lo;
  int row0 = flat ? 0 : lo;
  bool use_tbl = false;
  int out = flat ? 0 : role;

  // Pair merger: request the other groups' result rows now, so they arrive
  // with the first batch of its group's rows.
  int rid = 0;
  if (TWO && out == 2 && t < mg.ng && t != k)
    rid = __hip_atomic_load(rows_w + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  const int per_group = G * TPR;
  const int ngroups = !DIRECT && per_group <= NT ? NT / per_group : 1;
  const int nslots = per_group * ngroups;
  const f32x4 unwritten4 = zero4f();
  for (;;) {
    auto row_of = [&](int q) { return TWO && use_tbl ? rowtbl[q] : row0 + q; };
    // The merged value of (hh, cc): the step's output, the group's result
    // into this partition's row, or the group's result into LDS.
    auto finish = [&](int hh, int cc, float M, float L, f32x4 acc) {
      const float inv = recip_or_zero(L);
      if (!TWO || out == 0) {
        const int h = kvh * G + hh;
        f16x4 o;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = (f16)(acc[v] * inv);
        *reinterpret_cast<f16x4*>(a.out + ((size_t)b * a.Hq + h) * D + 4 * cc) = o;
        if (a.lse_out != nullptr && cc == 0)
          a.lse_out[(size_t)b * a.Hq + h] = L > 0.0f ? M + logf(L) : -INFINITY;
      } else {
        // the group's result as a partial: normalised o and its lse
        f32x4 x;
#pragma unroll
        for (int v = 0; v < 4; ++v) x[v] = acc[v] * inv;
        const float lse = L > 0.0f ? M + logf(L) : -INFINITY;
        if (out == 2) {
          *reinterpret_cast<f32x4*>(own + hh * D + 4 * cc) = x;
          if (cc == 0) own[16 * D + hh] = lse;
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) x[v] = encode_partial(x[v]);
          store_coherent4(po_rs, ((hh * Pm + p) * D + 4 * cc) * 4, x);
          if (cc == 0) store_coherent1(pl_rs, (hh * Pm + p) * 4, encode_partial(lse));
        }
      }
    };
    for (int slot = t; slot < nslots; slot += NT) {
      const int grp = slot / per_group;
      const int hc = slot % per_group;
      const int hh = hc / TPR;
      const int cc = hc % TPR;
      const f32x4 own_x = *reinterpret_cast<const f32x4*>(own + hh * D + 4 * cc);
      const float own_l = own[16 * D + hh];
      float M = -INFINITY, L = 0.0f;
      f32x4 acc = zero4f();
      if constexpr (DIRECT) {
        merge_direct_others<D, kDirectMergeItems - 1>(po_rs, pl_rs, Pm, n, q_own, hh, cc,
                                                      own_x, own_l, M, L, acc);
        // Back to "not written" for the next launch.  The threads that read
        // a head's lse words are TPR consecutive lanes of one wave, all past
        // their loads here, so its first lane resets them.
        for (int q = 0; q < n; ++q) {
          if (q == q_own) continue;
          store_coherent4(po_rs, ((hh * Pm + row0 + q) * D + 4 * cc) * 4, unwritten4);
          if (cc == 0) store_coherent1(pl_rs, (hh * Pm + row0 + q) * 4, 0.0f);
        }
        finish(hh, cc, M, L, acc);
      } else {
        // rows in flight per thread: its share of the items, 2 to 8
        const int rows = (n + ngroups - 1) / ngroups;
        if (rows <= 2)
          merge_rows<D, 2>(po_rs, pl_rs, Pm, n, q_own, rowtbl, TWO && use_tbl, row0, grp,
                           ngroups, hh, cc, own_x, own_l, M, L, acc);
        else if (rows <= 4)
          merge_rows<D, 4>(po_rs, pl_rs, Pm, n, q_own, rowtbl, TWO && use_tbl, row0, grp,
                           ngroups, hh, cc, own_x, own_l, M, L, acc);
        else
          merge_rows<D, kMergeRowsInFlight>(po_rs, pl_rs, Pm, n, q_own, rowtbl, TWO && use_tbl,
                                            row0, grp, ngroups, hh, cc, own_x, own_l, M, L, acc);
        // Back to "not written" for the next launch: this thread's data words
        // as soon as its last slot's rows are read (no load of this merge
        // follows them then, and loads and stores count down one in-order
        // counter); the lse words, which every thread of a head reads, after
        // the barrier below.
        if (slot + NT >= nslots) {
          for (int s2 = t; s2 <= slot; s2 += NT) {
            const int g2 = s2 / per_group;
            const int h2 = (s2 % per_group) / TPR;
            const int c2 = (s2 % per_group) % TPR;
            for (int q = g2; q < n; q += ngroups) {
              const int r = row_of(q);
              if (q != q_own && (!use_tbl || (r >= 0 && r < Pm)))
                store_coherent4(po_rs, ((h2 * Pm + r) * D + 4 * c2) * 4, unwritten4);
            }
          }
        }
        float* rr = msm + 6 * slot;
        rr[0] = M;
        rr[1] = L;
        rr[2] = acc[0];
        rr[3] = acc[1];
        rr[4] = acc[2];
        rr[5] = acc[3];
      }
    }
    if constexpr (DIRECT) return;
    __syncthreads();
    for (int i = t; i < G * n; i += NT) {
      const int q = i % n;
      const int r = row_of(q);
      if (q != q_own && (!use_tbl || (r >= 0 && r < Pm)))
        store_coherent1(pl_rs, ((i / n) * Pm + r) * 4, 0.0f);
    }
    for (int hc = t; hc < per_group; hc += NT) {
      float M = -INFINITY;
      for (int gi = 0; gi < ngroups; ++gi) M = fmaxf(M, msm[6 * (gi * per_group + hc)]);
      const float mu = M == -INFINITY ? 0.0f : M;
      float L = 0.0f;
      f32x4 acc = zero4f();
      for (int gi = 0; gi < ngroups; ++gi) {
        const float* rr = msm + 6 * (gi * per_group + hc);
        const float e = fast_exp2((rr[0] - mu) * kLog2e);
        L += e * rr[1];
        acc[0] += e * rr[2];
        acc[1] += e * rr[3];
        acc[2] += e * rr[4];
        acc[3] += e * rr[5];
      }
      finish(hc / TPR, hc % TPR, M, L, acc);
    }
    if (!TWO || out != 2) return;

    // The group results' rows; the words go back to zero for the next launch.
    if (t < mg.ng) {
      if (t == k) {
        rowtbl[t] = p;
      } else {
        const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
        while (rid == 0 && (long long)__builtin_amdgcn_s_memrealtime() - t0 < kSpinTicks) {
          __builtin_amdgcn_s_sleep(1);
          rid = __hip_atomic_load(rows_w + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __hip_atomic_store(rows_w + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        rowtbl[t] = rid - 1;  // -1 after a broken contract: read as zeros, never written
      }
    }
    __syncthreads();  // own holds the group's result; rowtbl is complete
    n = mg.ng;
    q_own = k;
    row0 = 0;
    use_tbl = true;
    out = 0;
  }
}

// MODE 0: unsplit decode (one workgroup per (sequence, KV head), fp16 out).
// MODE 1: split pass (one workgroup per partition, fp32 partials + lse).
// MODE 2: fused decode step: the split pass plus, in the same launch, the
//         step's cache write and the LSE merge of each (sequence, KV head)
//         by one of its workgroups.
// MODE 3: MODE 2 with the two-level merge (merge_groups), for launches with
//         more than kFlatMerge partitions per pair.
// MODE 4: MODE 2 with the direct merge, for launches with at most
//         kDirectMergeItems partitions per pair.
//
// Fused-step hand-off.  Each workgroup of a (b, kvh) with more than one
// partition takes a ticket from the pair's counter early (its latency hides
// under the K/V stream); the one holding the last ticket merges.  The others
// store their partials with device-coherent stores and exit without waiting.
// The merger keeps its own partial in LDS and polls the others' rows, which
// hold a zero word until written (the merger sets them back after reading,
// and resets the counter), so no store->flag->load round trips sit on the
// kernel's tail.
// One work item -- (sequence b, KV head kvh, partition p; p = 0 unsplit) --
// of the attention kernels.  Every thread of the workgroup calls it with the
// same item; smem is the workgroup's NW * AttnSmem<D, NS>::kWaveBytes bytes.
template <int D, int NS, int NW, int DEPTH, int MODE, bool DUAL>
__device__ __forceinline__ void attn_item(const AttnParams& a, const int b, const int kvh,
                                          const int p, unsigned char* smem) {
  constexpr int KC = D / 32;   // QK MFMAs (16x16x32) per subtile
  constexpr int NDB = D / 16;  // PV MFMA column blocks (16 dims each)
  constexpr bool SPLIT = MODE >= 1;
  constexpr bool STEP = MODE >= 2;
  constexpr bool TWO = MODE == 3;
  constexpr bool DIRECT = MODE == 4;
  using SM = LineSmem<D, NS>;
  using LM = LineMap<D>;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15;     // MFMA column
  const int quad = lane >> 4;  // 0..3
  const int head_col = DUAL ? (g & 7) : g;  // query head (within the group) of this column
  const int Hkv = a.Hkv;

  const int spb = a.block_size >> 4;  // subtiles per block
  const int spb_shift = a.spb_shift;
  const int64_t tok_stride = (int64_t)Hkv * D;
  int lane_off[KC];
#pragma unroll
  for (int m = 0; m < KC; ++m)
    lane_off[m] = (LM::row(lane, m) * (int)tok_stride + 8 * LM::chunk(lane, m)) * 2;
  const int32_t* bt_row = a.block_tables + (size_t)b * a.max_blocks;
  const __amdgpu_buffer_rsrc_t bt_rs = buffer_rsrc(bt_row, a.max_blocks * 4);
  constexpr int TSTEP = NW * NS;  // subtiles between a wave's consecutive tiles

  // The block ids of the wave's first DEPTH tiles do not depend on the
  // context length: any entry of the table row is a valid read, and ids past
  // the context are masked once the length is known.  They are scalar loads
  // (measured 1.3-1.8% faster than vector loads in the split pass, and
  // 1.7-3.8% in the fused step once its tile is one subtile).
  const int t_begin = SPLIT ? p * a.partition_size : 0;
  const int sub_begin = t_begin >> 4;
  const int s_first = sub_begin + wave * NS;
  ScalarIds<NS> ids0[DEPTH];
  int ids[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int s = s_first + i * TSTEP + j;
      const int blk = spb_shift >= 0 ? (s >> spb_shift) : (s / spb);
      ids0[i].v[j] = bt_row[blk < a.max_blocks ? blk : a.max_blocks - 1];
    }

  // Fused step: the new token's slot, requested before the length so that
  // one round trip brings both (the owner of the new token must not wait for
  // it after the length is known).
  const int64_t slot_in = STEP && a.slot_mapping != nullptr ? a.slot_mapping[b] : -1;
  const int cap = a.max_blocks * a.block_size;
  int ctx = a.context_lens[b];
  // Left alone, the compiler sinks the id loads past the early exit below,
  // so their round trip would start only once the length has arrived.  In
  // the fused step, naming them beside the length keeps the requests
  // together (0.5-1% faster; the split pass measured no gain).
  if constexpr (STEP) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) asm volatile("" : : "s"(ids0[i].v[j]), "s"(ctx));
  }
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  int t_end = ctx;
  if (SPLIT) {
    // the fused step's partition 0 of an empty sequence still writes zeros
    if (t_begin >= ctx && !(STEP && ctx == 0 && p == 0)) {
      if (!STEP && threadIdx.x < a.G)
        a.partial_lse[((size_t)b * a.Hq + kvh * a.G + threadIdx.x) * a.max_partitions + p] =
            -INFINITY;
      return;
    }
    t_end = min(ctx, t_begin + a.partition_size);
  }
  const int sub_end = (t_end + 15) >> 4;
  const int n_parts =
      STEP ? div_sh(ctx + a.partition_size - 1, a.partition_size, a.part_shift) : 1;

  // Fused step: the workgroup owning position ctx-1 (partition 0 if ctx = 0)
  // writes the new token's K/V row of its head into the pool (at the end of
  // the kernel), and takes that position's K/V from k_new/v_new instead of
  // the pool when the slot is the position's slot in the block table (so the
  // launch never reads its own write).  That block id comes with the tile
  // that holds the position; nothing here waits for a load after the length.
  const bool owns_new = STEP && a.slot_mapping != nullptr &&
                        p == (ctx > 0 ? div_sh(ctx - 1, a.partition_size, a.part_shift) : 0);
  const int64_t slot = owns_new ? slot_in : -1;
  int s_new = -1, tok_new = -1, new_off = 0;
  f16x8 kn[KC], vn[KC];
  const size_t new_row = ((size_t)b * Hkv + kvh) * D;
  if (owns_new) {
    if (ctx > 0) {
      const int pos = ctx - 1;
      new_off = mod_sh(pos, a.block_size, a.bs_shift);
      s_new = pos >> 4;
      tok_new = pos & 15;
    }
    // A branch around these loads sits before the K/V loop, where it costs
    // the loop's wait counts nothing (loading them through empty resources
    // in every workgroup measured slower).
    // in the line layout of the K/V loads (load m of this lane)
#pragma unroll
    for (int m = 0; m < KC; ++m) {
      kn[m] = *reinterpret_cast<const f16x8*>(a.k_new + new_row + 8 * LM::chunk(lane, m));
      vn[m] = *reinterpret_cast<const f16x8*>(a.v_new + new_row + 8 * LM::chunk(lane, m));
    }
  } else {
#pragma unroll
    for (int m = 0; m < KC; ++m) {
      kn[m] = zero8();
      vn[m] = zero8();
    }
  }

  // The query group as the B operand (lane l holds q[head of column l%16]
  // [8*(l/16) + 32m ..]).
  // A negative scale is folded into q (negating fp16 is exact), so the
  // kernel works with c = |scale| * log2(e).
  const bool neg_scale = a.scale_log2 < 0.0f;
  const float c = fmaxf(neg_scale ? -a.scale_log2 : a.scale_log2, 1.17549435e-38f);
  f16x8 qb[KC];
  {
    // the group's G query rows; columns past G read zeros
    const __amdgpu_buffer_rsrc_t q_rs =
        buffer_rsrc(a.q + ((size_t)b * a.Hq + kvh * a.G) * D, a.G * D * 2);
    const unsigned sign = neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int m = 0; m < KC; ++m)
      qb[m] = load_q16(q_rs, (head_col * D + 8 * quad + 32 * m) * 2, sign);
  }
  f16x4 ones;
#pragma unroll
  for (int i = 0; i < 4; ++i) ones[i] = (f16)(g == 0 ? 1.0f : 0.0f);
  float rem_mul = DUAL ? (g >= 8 ? -1.0f : 0.0f) : -1.0f;
  asm volatile("" : "+v"(rem_mul));

  SoftmaxState<D> st;
#pragma unroll
  for (int i = 0; i < NDB; ++i) st.o[i] = zero4f();
  st.lsum = zero4f();
  st.m = -INFINITY;
  f16* stage = reinterpret_cast<f16*>(smem + wave * SM::kWaveBytes);

  // DEPTH-slot software pipeline over the wave's tiles: up to DEPTH tiles of
  // K/V are in flight while one is consumed.  The block ids of tile u+DEPTH
  // are requested right after the K/V of tile u, so the in-order wait for
  // them only ever waits for tiles already consumed.  The loop runs while a
  // tile remains to be requested, and every iteration issues the same loads
  // (past the wave's last tile through empty resources: no memory access), so
  // the waits inside it stay partial.  The tiles still in flight after it are
  // consumed with no further requests: requests past the end would still
  // return through the memory pipeline, and the code after the loop waits for
  // all of them (0.15-0.5 us per step measured).
  const int n_tiles = s_first < sub_end ? (sub_end - s_first + TSTEP - 1) / TSTEP : 0;
  KVTile<D, NS> buf[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) {
    load_kv_lines<D, NS>(buf[i], a, ids0[i], s_first + i * TSTEP, sub_end, t_end, spb,
                         spb_shift, tok_stride, kvh, lane_off, s_new);
    ids[i] = load_block_ids<NS>(bt_rs, s_first + (i + DEPTH) * TSTEP, sub_end, spb, spb_shift,
                                lane);
  }
  // Fused step: the ticket (issued after the first K/V requests; waited for
  // only at the end).
  unsigned long long ticket = 0;
  if (STEP && n_parts > 1 && threadIdx.x == 0) ticket = take_step_ticket<TWO>(a, b, kvh, n_parts, p);
  int u0 = 0;
  for (; u0 + DEPTH < n_tiles; u0 += DEPTH) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      const int u = u0 + i;
      consume_tile<D, NS, DUAL, STEP>(buf[i], st, qb, stage, c, t_end, lane, ones, rem_mul,
                                      s_new, tok_new, slot, new_off, a.block_size, kn, vn);
      load_kv_lines<D, NS>(buf[i], a, ids[i], s_first + (u + DEPTH) * TSTEP, sub_end, t_end,
                           spb, spb_shift, tok_stride, kvh, lane_off, s_new);
      ids[i] = load_block_ids<NS>(bt_rs, s_first + (u + 2 * DEPTH) * TSTEP, sub_end, spb,
                                  spb_shift, lane);
    }
  }
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    if (u0 + i < n_tiles)
      consume_tile<D, NS, DUAL, STEP>(buf[i], st, qb, stage, c, t_end, lane, ones, rem_mul,
                                      s_new, tok_new, slot, new_off, a.block_size, kn, vn);

  // DUAL: fold the remainder columns (8..15) into the head columns (0..7).
  if (DUAL) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) st.o[db][v] += row_xor8(st.o[db][v]);
    st.lsum[0] += row_xor8(st.lsum[0]);
  }
  // Weight sum of this lane's column: row 0, held by the quad-0 lane (the
  // wave merge reads it from those lanes only).
  const float l_tot = NW == 1 ? __shfl(st.lsum[0], g) : st.lsum[0];

  // Fused step: publish whether and what this workgroup merges (its ticket
  // closes its group, or the pair), before the barriers of the wave merge.
  __shared__ int s_merge;
  __shared__ __attribute__((aligned(16))) float own[STEP ? 16 * D + 16 : 4];
  if (STEP && n_parts > 1 && threadIdx.x == 0)
    s_merge = step_merge_role<TWO>(a, b, kvh, n_parts, p, ticket);
  if (NW == 1 && STEP) __syncthreads();

  // Fused step: the append of the new token's row of this head (after the
  // ticket is read: the wait for it would otherwise include these stores).
  if (owns_new && slot >= 0 && slot < (int64_t)a.num_blocks * a.block_size) {
    // lanes 0 .. D/8-1 hold the row's chunks 0 .. D/8-1 in load 0 (row 0, no swizzle)
    if (wave == 0 && lane < LM::kChunksPerRow) {
      *reinterpret_cast<f16x8*>(a.k_pool_w + (slot * Hkv + kvh) * D + 8 * lane) = kn[0];
      *reinterpret_cast<f16x8*>(a.v_pool_w + (slot * Hkv + kvh) * D + 8 * lane) = vn[0];
    }
  }

  // Final value for column block db of this lane's head.
  const bool emits = (DUAL ? g < 8 : true) && head_col < a.G;
  auto emit = [&](int db, f32x4 acc, float L, float M) {
    if (!emits) return;
    const int h = kvh * a.G + head_col;
    const float inv = recip_or_zero(L);
    const int d0 = 16 * db + 4 * quad;
    if (SPLIT && !(STEP && n_parts <= 1)) {
      f32x4 r;
#pragma unroll
      for (int v = 0; v < 4; ++v) r[v] = acc[v] * inv;
      const float lse_v = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
      if (STEP) {
        if (s_merge) {
          *reinterpret_cast<f32x4*>(own + head_col * D + d0) = r;
          if (db == 0 && quad == 0) own[16 * D + head_col] = lse_v;
        } else {
          const size_t head0 = (size_t)b * a.Hq + kvh * a.G;
          const int Pm = a.max_partitions;
          const __amdgpu_buffer_rsrc_t po_rs =
              buffer_rsrc(a.partial_out + head0 * Pm * D, a.G * Pm * D * 4);
          const __amdgpu_buffer_rsrc_t pl_rs =
              buffer_rsrc(a.partial_lse + head0 * Pm, a.G * Pm * 4);
#pragma unroll
          for (int v = 0; v < 4; ++v) r[v] = encode_partial(r[v]);
          store_coherent4(po_rs, ((head_col * Pm + p) * D + d0) * 4, r);
          if (db == 0 && quad == 0)
            store_coherent1(pl_rs, (head_col * Pm + p) * 4, encode_partial(lse_v));
        }
      } else {
        float* dst = a.partial_out + (((size_t)b * a.Hq + h) * a.max_partitions + p) * D + d0;
        *reinterpret_cast<f32x4*>(dst) = r;
        if (db == 0 && quad == 0)
          a.partial_lse[((size_t)b * a.Hq + h) * a.max_partitions + p] = lse_v;
      }
    } else {
      f16x4 r;
#pragma unroll
      for (int v = 0; v < 4; ++v) r[v] = (f16)(acc[v] * inv);
      *reinterpret_cast<f16x4*>(a.out + ((size_t)b * a.Hq + h) * D + d0) = r;
      if (STEP && a.lse_out != nullptr && db == 0 && quad == 0)
        a.lse_out[(size_t)b * a.Hq + h] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
  };

  if (NW == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) emit(db, st.o[db], l_tot, st.m);
  } else {
    merge_waves_impl<D, NW>(st, l_tot, smem, SM::kWaveBytes, wave, lane, emit);
  }
  if (!STEP || n_parts <= 1 || !s_merge) return;
  __syncthreads();  // the merger's own partial is complete in LDS
  __shared__ float msm[DIRECT ? 4 : 6 * kMergeSlots];
  __shared__ int rowtbl[kMaxMergeGroups];
  merge_step_partitions<D, NW, TWO, DIRECT>(a, b, kvh, n_parts, p, s_merge, own, msm, rowtbl);
}

// Direct grid.  Unsplit decode: one workgroup per (sequence, KV head),
// blockIdx.x = b * Hkv + kvh.  Partitioned passes: a 3-D grid (KV head,
// partition, sequence), so the item needs no division.
template <int D, int NS, int NW, int DEPTH, int MODE, bool DUAL>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const AttnParams a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[NW * LineSmem<D, NS>::kWaveBytes];
  if constexpr (MODE >= 1)
    attn_item<D, NS, NW, DEPTH, MODE, DUAL>(a, blockIdx.z, blockIdx.x, blockIdx.y, smem);
  else
    attn_item<D, NS, NW, DEPTH, MODE, DUAL>(a, blockIdx.x / a.Hkv, blockIdx.x % a.Hkv, 0, smem);
}

// Compact grid for the split pass and the fused step when most of the
// B x Hkv x max_partitions grid would be empty (ragged lengths, a wide
// table): a fixed number of workgroups each scans the batch's partition
// counts into LDS and loops over its share of the non-empty items only.  An
// empty workgroup still costs a dispatch (~1.3 ns each on MI355X), which
// dominates a skewed batch's launch otherwise.
constexpr int kCompactMaxB = 4096;

// Largest b in [0, B) with prefix[b] <= idx (prefix non-decreasing,
// prefix[0] = 0 <= idx); two ballots over 64 lanes, B <= 4096.
__device__ __forceinline__ int find_sequence(const int* prefix, int B, int idx, int lane) {
  const int step = (B + 63) >> 6;
  int c = lane * step;
  int k = __popcll(__ballot(c < B && prefix[c] <= idx));
  const int lo = (k - 1) * step;
  c = lo + lane;
  k = __popcll(__ballot(lane < step && c < B && prefix[c] <= idx));
  return lo + k - 1;
}

template <int D, int NS, int NW, int DEPTH, int MODE, bool DUAL>
__global__ __launch_bounds__(NW * 64) void attn_compact_kernel(const AttnParams a) {
  static_assert(MODE >= 1, "the compact grid is for the partitioned passes");
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) unsigned char smem[NW * LineSmem<D, NS>::kWaveBytes];
  __shared__ int prefix[kCompactMaxB + 1];
  __shared__ int wave_sum[NW];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int B = a.B;
  const int cap = a.max_blocks * a.block_size;

  // items of sequence b: its non-empty partitions (the fused step gives an
  // empty sequence one, which writes its zero output)
  const int per = (B + NT - 1) / NT;
  const int j0 = min(B, t * per), j1 = min(B, j0 + per);
  int local = 0;
  for (int j = j0; j < j1; ++j) {
    int ctx = a.context_lens[j];
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    int n = (ctx + a.partition_size - 1) / a.partition_size;
    if (MODE >= 2 && n == 0) n = 1;
    prefix[j] = n;  // the count for now; each thread touches its own indices only
    local += n;
  }
  // exclusive scan of the per-thread sums across the workgroup
  int incl = local;
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int base = incl - local;
  for (int w = 0; w < wave; ++w) base += wave_sum[w];
  int run = base;
  for (int j = j0; j < j1; ++j) {
    const int n = prefix[j];
    prefix[j] = run;
    run += n;
  }
  __syncthreads();
  if (t == 0) {
    int total = 0;
    for (int w = 0; w < NW; ++w) total += wave_sum[w];
    prefix[B] = total;
  }
  __syncthreads();
  const int total_items = prefix[B] * a.Hkv;

  // split pass: partitions at or past the context get lse = -inf
  if (MODE == 1) {
    for (int b = blockIdx.x; b < B; b += gridDim.x) {
      const int n = prefix[b + 1] - prefix[b];
      const int spare = a.max_partitions - n;
      for (int e = t; e < a.Hq * spare; e += NT)
        a.partial_lse[((size_t)b * a.Hq + e / spare) * a.max_partitions + n + e % spare] =
            -INFINITY;
    }
  }
  for (int i = blockIdx.x; i < total_items; i += gridDim.x) {
    const int idx = i / a.Hkv;
    const int b = find_sequence(prefix, B, idx, lane);
    attn_item<D, NS, NW, DEPTH, MODE, DUAL>(a, b, i % a.Hkv, idx - prefix[b], smem);
    __syncthreads();  // LDS is reused by the next item
  }
}

// LSE-weighted merge of the valid partitions of one (sequence, query head).
// One 256-thread workgroup per pair: the partition weights exp(lse_p - max)
// are computed once into LDS, then thread (row r, column c) accumulates
// partitions r, r + ROWS, ... of its 4 dims with 16-byte loads, so ROWS
// partitions are in flight at a time; rows are summed through LDS at the end.
// The first 256 log-sum-exps and the first ROWS partition rows are requested
// together with the context length (every index below max_partitions is a
// valid read), so a call with few partitions costs one memory round trip.
template <int D>
__global__ __launch_bounds__(256) void split_reduce_kernel(const ReduceParams a) {
  constexpr int TPR = D / 4;         // threads per partition row (4 dims each)
  constexpr int ROWS = 256 / TPR;    // partitions in flight (16 for D=64)
  constexpr int CHUNK = 2048;        // weights staged per pass
  __shared__ float w[CHUNK];
  __shared__ f32x4 red[ROWS][TPR];
  __shared__ float wave_part[4];

  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int r = t / TPR;
  const int c = t % TPR;
  const int Pm = a.max_partitions;
  const float* lse = a.partial_lse + (size_t)bh * Pm;
  const float* po = a.partial_out + (size_t)bh * Pm * D + 4 * c;

  const float lse_t = t < Pm ? lse[t] : -INFINITY;
  const f32x4 x_r = r < Pm ? *reinterpret_cast<const f32x4*>(po + (size_t)r * D) : zero4f();
  const int cap = Pm * a.partition_size;
  int ctx = a.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  const int np = (ctx + a.partition_size - 1) / a.partition_size;

  float M = t < np ? lse_t : -INFINITY;
  for (int i = t + 256; i < np; i += 256) M = fmaxf(M, lse[i]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh));
  if (lane == 0) wave_part[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(wave_part[0], wave_part[1]), fmaxf(wave_part[2], wave_part[3]));

  f32x4 acc = zero4f();
  float L = 0.0f;
  if (M != -INFINITY) {
    const float M2 = M * kLog2e;
    for (int base = 0; base < np; base += CHUNK) {
      const int n = min(CHUNK, np - base);
      __syncthreads();  // previous chunk's weights are consumed
      for (int i = t; i < n; i += 256) {
        const float li = (base == 0 && i == t) ? lse_t : lse[base + i];
        const float e = fast_exp2(fmaf(li, kLog2e, -M2));
        w[i] = e;
        L += e;
      }
      __syncthreads();
      int i = r;
      if (base == 0) {
        if (r < n) acc += w[r] * x_r;
        i = r + ROWS;
      }
#pragma unroll 4
      for (; i < n; i += ROWS) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(po + (size_t)(base + i) * D);
        acc += w[i] * x;
      }
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) L += __shfl_xor(L, sh);
  __syncthreads();
  if (lane == 0) wave_part[wave] = L;
  red[r][c] = acc;
  __syncthreads();
  if (t < TPR) {
    L = wave_part[0] + wave_part[1] + wave_part[2] + wave_part[3];
    f32x4 sum = zero4f();
#pragma unroll
    for (int i = 0; i < ROWS; ++i) sum += red[i][t];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    f16x4 o;
#pragma unroll
    for (int v = 0; v < 4; ++v) o[v] = (f16)(sum[v] * inv);
    *reinterpret_cast<f16x4*>(a.out + (size_t)bh * D + 4 * t) = o;
    if (a.lse_out != nullptr && t == 0) a.lse_out[bh] = L > 0.0f ? M + logf(L) : -INFINITY;
  }
}

// The same merge for many (row, head) pairs with few partitions each (chunk
// rows of a split prefill, large decode batches): D/4 threads per pair, 4
// dims each, so a workgroup merges 256/(D/4) pairs.  Each thread streams its
// pair's partitions with the LSE update, four rows in flight; a -inf lse
// weighs its (finite) row by zero.
template <int D>
__global__ __launch_bounds__(256) void split_reduce_rows_kernel(const ReduceParams a) {
  constexpr int TPR = D / 4;
  constexpr int RPW = 256 / TPR;
  const int t = threadIdx.x;
  const int64_t bh = (int64_t)blockIdx.x * RPW + t / TPR;
  const int c = t % TPR;
  if (bh >= (int64_t)a.B * a.Hq) return;
  const int b = (int)(bh / a.Hq);
  const int Pm = a.max_partitions;
  const int cap = Pm * a.partition_size;
  int ctx = a.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  const int np = (ctx + a.partition_size - 1) / a.partition_size;
  const float* lse = a.partial_lse + bh * Pm;
  const float* po = a.partial_out + bh * Pm * D + 4 * c;
  float M = -INFINITY, L = 0.0f;
  f32x4 acc = zero4f();
  for (int q0 = 0; q0 < np; q0 += 4) {
    float l[4];
    f32x4 x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = q0 + j < np;
      l[j] = in ? lse[q0 + j] : -INFINITY;
      x[j] = in ? *reinterpret_cast<const f32x4*>(po + (size_t)(q0 + j) * D) : zero4f();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float Mn = fmaxf(M, l[j]);
      const float mu = Mn == -INFINITY ? 0.0f : Mn;
      const float sa = fast_exp2((M - mu) * kLog2e);  // 1 while M holds; 0 from -inf
      const float sb = fast_exp2((l[j] - mu) * kLog2e);
      acc = acc * sa + x[j] * sb;
      L = L * sa + sb;
      M = Mn;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  f16x4 o;
#pragma unroll
  for (int v = 0; v < 4; ++v) o[v] = (f16)(acc[v] * inv);
  *reinterpret_cast<f16x4*>(a.out + (size_t)bh * D + 4 * c) = o;
  if (a.lse_out != nullptr && c == 0) a.lse_out[bh] = L > 0.0f ? M + logf(L) : -INFINITY;
}

// Bit-exact scatter of new K/V rows: one thread per 16-byte chunk of one
// (token, KV head) row, K and V both.
__global__ __launch_bounds__(256) void append_kernel(const AppendParams a) {
  const int chunks = a.D >> 3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.num_tokens * a.Hkv * chunks;
  if (idx >= total) return;
  const int c = (int)(idx % chunks);
  const int64_t rest = idx / chunks;
  const int h = (int)(rest % a.Hkv);
  const int64_t n = rest / a.Hkv;
  // The new rows are read together with their slot (not after it).
  const int64_t src = (n * a.Hkv + h) * a.D + 8 * c;
  const uint4 kx = *reinterpret_cast<const uint4*>(a.k_new + src);
  const uint4 vx = *reinterpret_cast<const uint4*>(a.v_new + src);
  const int64_t slot = a.slot_mapping[n];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t dst = (slot * a.Hkv + h) * a.D + 8 * c;
  *reinterpret_cast<uint4*>(a.k_pool + dst) = kx;
  *reinterpret_cast<uint4*>(a.v_pool + dst) = vx;
}

}  // namespace pkv
