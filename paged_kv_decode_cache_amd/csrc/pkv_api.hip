// C ABI of libpkv.so: argument validation (before any HIP call), launch
// configuration, and launches on the caller's stream.  No allocation, no
// synchronisation, no device reads on the host.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "pkv.h"
#include "pkv_kernels.hpp"
#include "pkv_prefill.hpp"
#include "pkv_q8.hpp"

namespace {

using pkv::AppendParams;
using pkv::AttnParams;
using pkv::ReduceParams;

constexpr int kVersion = 100;  // 0.1.0

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool head_dim_ok(int32_t d) { return d == 64 || d == 128; }

bool block_size_ok(int32_t bs) { return bs >= 16 && bs <= 256 && bs % 16 == 0; }

// Launch shape: waves per workgroup, 16-token subtiles per tile, tiles in
// flight per wave.  Defaults (measured on MI355X): the unsplit pass has one
// workgroup per (sequence, KV head) and uses 8 waves; the partitioned passes
// use 4 (one partition each).  At head_dim 64 the split pass loads 2
// subtiles per tile and the fused step 1 (its last tile's compute is exposed
// before the hand-off).  A call may override any of them through a
// pkv_launch_config (the _ex entry points); nothing is kept between calls.
struct Shape {
  int waves, subtiles, depth;
};

Shape default_shape(int mode, int head_dim) {
  Shape s;
  s.waves = mode == 0 ? 8 : 4;
  s.subtiles = head_dim == 64 && mode != 2 ? 2 : 1;
  s.depth = 2;
  return s;
}

bool config_ok(const pkv_launch_config* c) {
  if (!c) return true;
  const int w = c->waves_per_group, t = c->subtiles_per_tile, d = c->tiles_in_flight;
  return (w == 0 || w == 1 || w == 2 || w == 4 || w == 8) &&
         (t == 0 || t == 1 || t == 2 || t == 4) && (d == 0 || d == 2 || d == 4) &&
         c->grid >= 0 && c->grid <= 2;
}

Shape pick_shape(int mode, int head_dim, const pkv_launch_config* c) {
  Shape s = default_shape(mode, head_dim);
  if (c) {
    if (c->waves_per_group) s.waves = c->waves_per_group;
    if (c->subtiles_per_tile) s.subtiles = c->subtiles_per_tile;
    if (c->tiles_in_flight) s.depth = c->tiles_in_flight;
  }
  // register budget: at most 8 subtiles of K/V in flight per wave at
  // head_dim 64 and 4 at head_dim 128
  const int max_inflight = head_dim == 64 ? 8 : 4;
  if (head_dim == 128 && s.subtiles > 2) s.subtiles = 2;
  if (s.subtiles * s.depth > max_inflight) s.depth = 2;
  if (s.subtiles * s.depth > max_inflight) s.subtiles = max_inflight / 2;
  return s;
}

// MODE: 0 unsplit decode, 1 split pass, 2 and 3 fused decode step.  The grid of
// the partitioned passes is (Hkv, max_partitions, B); of the unsplit pass
// (B * Hkv).
dim3 attn_grid(const AttnParams& p, int mode) {
  if (mode == 0) return dim3((unsigned)(p.B * p.Hkv));
  return dim3((unsigned)p.Hkv, (unsigned)p.max_partitions, (unsigned)p.B);
}

template <int D, int NS, int NW, int DEPTH, int MODE>
void launch_attn_inst(const AttnParams& p, hipStream_t st) {
  // Groups of up to 8 query heads put the fp16 remainder of P in the spare
  // MFMA columns (one PV MFMA per 16 dims instead of two).
  const dim3 grid = attn_grid(p, MODE);
  if (p.G <= 8)
    hipLaunchKernelGGL((pkv::attn_kernel<D, NS, NW, DEPTH, MODE, true>), grid, dim3(NW * 64), 0,
                       st, p);
  else
    hipLaunchKernelGGL((pkv::attn_kernel<D, NS, NW, DEPTH, MODE, false>), grid, dim3(NW * 64),
                       0, st, p);
}

template <int D, int NS, int DEPTH, int MODE>
void launch_attn_nw(const AttnParams& p, int waves, hipStream_t st) {
  switch (waves) {
    case 1: launch_attn_inst<D, NS, 1, DEPTH, MODE>(p, st); break;
    case 2: launch_attn_inst<D, NS, 2, DEPTH, MODE>(p, st); break;
    case 4: launch_attn_inst<D, NS, 4, DEPTH, MODE>(p, st); break;
    default: launch_attn_inst<D, NS, 8, DEPTH, MODE>(p, st); break;
  }
}

template <int D, int MODE>
void launch_attn_shape(const AttnParams& p, Shape s, hipStream_t st) {
  const int w = s.waves;
  if (s.depth == 4) {
    if (s.subtiles == 1) launch_attn_nw<D, 1, 4, MODE>(p, w, st);
    else if constexpr (D == 64) launch_attn_nw<D, 2, 4, MODE>(p, w, st);
    else launch_attn_nw<D, 1, 4, MODE>(p, w, st);
  } else {
    if (s.subtiles == 1) launch_attn_nw<D, 1, 2, MODE>(p, w, st);
    else if (s.subtiles == 2) launch_attn_nw<D, 2, 2, MODE>(p, w, st);
    else if constexpr (D == 64) launch_attn_nw<D, 4, 2, MODE>(p, w, st);
    else launch_attn_nw<D, 2, 2, MODE>(p, w, st);
  }
}

// log2(v) when v is a positive power of two, else -1.
int log2_or_neg(int64_t v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int sh = 0;
  while ((int64_t(1) << sh) < v) ++sh;
  return sh;
}

int spb_shift_of(int32_t block_size) {
  const int spb = block_size / 16;
  if (spb & (spb - 1)) return -1;
  int sh = 0;
  while ((1 << sh) < spb) ++sh;
  return sh;
}

// Grid of the partitioned passes: direct (a workgroup per sequence x KV head
// x partition) or compact (a fixed number of workgroups looping over the
// non-empty partitions; attn_compact_kernel).  Auto picks compact when the
// direct grid would exceed kCompactAbove workgroups (ragged batches with a
// wide table are mostly empty partitions, each a workgroup dispatch), or
// when a dimension exceeds the direct grid's limits.  The compact kernel is built for the default shape only; a call
// with another shape stays direct.
constexpr int64_t kCompactAbove = 8192;
constexpr int kCompactGroups = 2048;
constexpr int64_t kMaxGridYZ = 65535;

template <int D, int NS, int MODE>
void launch_compact(const AttnParams& p, int64_t wgs, hipStream_t st) {
  const unsigned g = (unsigned)(wgs < kCompactGroups ? wgs : kCompactGroups);
  if (p.G <= 8)
    hipLaunchKernelGGL((pkv::attn_compact_kernel<D, NS, 4, 2, MODE, true>), dim3(g), dim3(256),
                       0, st, p);
  else
    hipLaunchKernelGGL((pkv::attn_compact_kernel<D, NS, 4, 2, MODE, false>), dim3(g), dim3(256),
                       0, st, p);
}

// The fused steps (fp16 and 8-bit) take 8 waves when the grid is at most
// one workgroup per CU and a pair has at least 8 partitions: few workgroups
// then stream the context, twice the waves keep twice the requests in
// flight, and the merge spreads its rows over twice the threads.  Same-box
// A/B of the fp16 step, 4 -> 8 waves (us): B=1 x 4096 P=256 8.4 -> 7.6,
// B=8 x 4096 P=256 9.4 -> 9.0, B=8 x 4096 P=512 9.7-10.2 -> 8.9-9.3,
// B=8 x 2048 P=256 7.9 -> 7.5, B=1 x 2048 P=256 7.3 -> 6.9.  With 4
// partitions it was level or slower (B=32 x 1024 P=256 7.7 -> 8.0,
// B=8 x 512 P=128 5.6 -> 5.9, B=32 x 4096 P=1024 15.2 -> 15.65), and with
// more workgroups than CUs 4 waves stay faster.
constexpr int64_t kStepWideMergeMaxGrid = 256;
constexpr int kStepWideMinPartitions = 8;
bool step_wide_merge(int head_dim, int64_t grid, int max_partitions, int /*group*/) {
  return head_dim == 64 && grid <= kStepWideMergeMaxGrid &&
         max_partitions >= kStepWideMinPartitions;
}

// MODE: 0 unsplit, 1 split pass, 2 fused step; the fused step's launches
// with more than kFlatMerge partitions per pair take MODE 3 (the two-level
// merge), those with at most kDirectMergeItems MODE 4 (the direct merge),
// the others keep the one-level code with the merge through LDS.  Each is
// its own instantiation: merge code a launch does not use still costs the
// kernel registers and time.
template <int MODE>
int launch_attn(const AttnParams& p, int head_dim, const pkv_launch_config* cfg,
                hipStream_t st) {
  if constexpr (MODE == 2) {
    if (p.max_partitions > pkv::kFlatMerge) return launch_attn<3>(p, head_dim, cfg, st);
    if (p.max_partitions <= pkv::kDirectMergeItems) return launch_attn<4>(p, head_dim, cfg, st);
  }
  constexpr int SHAPE_MODE = MODE >= 2 ? 2 : MODE;
  Shape s = pick_shape(SHAPE_MODE, head_dim, cfg);
  if constexpr (MODE >= 1) {
    Shape d = default_shape(SHAPE_MODE, head_dim);
    if constexpr (MODE >= 2) {
      const int64_t grid = (int64_t)p.B * p.Hkv * p.max_partitions;
      if (step_wide_merge(head_dim, grid, p.max_partitions, p.G)) {
        d.waves = 8;
        if (!cfg || cfg->waves_per_group == 0) s.waves = 8;
      }
    }
    const int64_t wgs = (int64_t)p.B * p.Hkv * p.max_partitions;
    const int mode = cfg ? cfg->grid : 0;
    const bool same_shape =
        s.waves == d.waves && s.subtiles == d.subtiles && s.depth == d.depth;
    const bool direct_fits = p.max_partitions <= kMaxGridYZ && p.B <= kMaxGridYZ;
    if (p.B <= pkv::kCompactMaxB && same_shape &&
        (mode == 2 || (mode == 0 && wgs > kCompactAbove) || !direct_fits)) {
      if (head_dim == 64)
        launch_compact<64, MODE >= 2 ? 1 : 2, MODE>(p, wgs, st);
      else
        launch_compact<128, 1, MODE>(p, wgs, st);
      return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
    }
    if (!direct_fits) return PKV_ERR_UNSUPPORTED;
  }
  if (head_dim == 64)
    launch_attn_shape<64, MODE>(p, s, st);
  else
    launch_attn_shape<128, MODE>(p, s, st);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

// Checks shared by both attention passes.  Returns PKV_OK or an error code.
int check_attn_common(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                      float scale) {
  if (B < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PKV_ERR_INVALID_ARG;
  if (!k_pool || !v_pool || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return PKV_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PKV_ERR_UNSUPPORTED;
  if (num_q_heads / num_kv_heads > 16) return PKV_ERR_UNSUPPORTED;
  // positions per sequence must fit in int32
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;  // empty per-sequence arrays may be null
  if (!q || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

// Chunked prefill: NCT column tiles of 16 (query row, head) pairs; fewer at
// head_dim 128 (register budget of the accumulators).  A launch with fewer
// workgroups than the chip has CUs (short chunks, few sequences) gives each
// 8 waves, so each streams its context in half the time; larger launches
// use 4 (measured on MI355X: 56 vs 78 us at 8 x 64-row chunks over 4K
// contexts, 186 vs 201 us at 8 x 512).
constexpr int kComputeUnits = 256;

template <int D, bool SPLIT>
int launch_prefill(const pkv::PrefillParams& p, int64_t grid, hipStream_t st) {
  constexpr int NCT = D == 64 ? 4 : 2;
  if (grid < kComputeUnits)
    hipLaunchKernelGGL((pkv::prefill_kernel<D, NCT, 8, 2, SPLIT>), dim3((unsigned)grid),
                       dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((pkv::prefill_kernel<D, NCT, 4, 2, SPLIT>), dim3((unsigned)grid),
                       dim3(256), 0, st, p);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

// 8-bit decode: unsplit (8 waves), split pass or fused step (4 waves, or 8
// under the rules of launch_q8), 2 tiles in flight; 2 subtiles per tile at
// head_dim 64 (1 at 128).  Unlike the fp16 step, the 4-wave 8-bit step takes
// 2 as well: a wave's range is half the bytes, so one subtile per tile
// leaves it more round trips per range (at its best partition size:
// B=8 x 4096 11.1 -> 10.7 us, B=32 x 2048 11.5 -> 10.95 us, B=128 x 8192
// 70.1 -> 69.2 us, B=32 x 4096 15.3 -> 15.2 us).  8-wave launches (step
// or split pass) take 1: with 2, the step at B=4 x 32768 was 0.4 us
// slower, at B=1 x 32768 0.4 us faster and at B=1 x 131072 level, and the
// direct-merge step at B=128 x 4096 37.6 -> 45.2 us.
// MODE: 0 unsplit, 1 split pass, 2 fused decode step (3 with the two-level
// merge, 4 with the direct merge).
template <int D, int NW, int MODE>
void launch_q8_nw(const pkv::Q8Params& p, int64_t grid, hipStream_t st) {
  constexpr int NS = D == 64 && (MODE == 0 || NW == 4) ? 2 : 1;
  if (p.a.G <= 8)
    hipLaunchKernelGGL((pkv::attn_q8_kernel<D, NS, NW, 2, MODE, true>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, st, p);
  else
    hipLaunchKernelGGL((pkv::attn_q8_kernel<D, NS, NW, 2, MODE, false>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, st, p);
}

// The fused step takes 8 waves where the fp16 step does (step_wide_merge),
// and always with the direct merge (MODE 4): its loop is latency-bound, and
// two waves per SIMD at 4 partitions per pair beat 8 partitions of 4-wave
// workgroups (same-box A/B, us: B=32 x 4096 at P=1024 15.25-15.43 ->
// 13.56-13.79, B=32 x 2048 at P=512 11.28 -> 10.29-10.36, B=8 x 1024 at
// P=512 10.12-10.15 -> 9.42-9.65, B=128 x 4096 at P=1024 level).  The fp16
// step keeps 4 waves there (15.2 -> 15.65 us at B=32 x 4096).
template <int D, int MODE>
int launch_q8(const pkv::Q8Params& p, int64_t grid, hipStream_t st) {
  if constexpr (MODE == 2) {
    if (p.a.max_partitions > pkv::kFlatMerge) return launch_q8<D, 3>(p, grid, st);
    if (p.a.max_partitions <= pkv::kDirectMergeItems) return launch_q8<D, 4>(p, grid, st);
  }
  if constexpr (MODE >= 2 && D == 64) {
    if (MODE == 4 || step_wide_merge(D, grid, p.a.max_partitions, p.a.G))
      launch_q8_nw<D, 8, MODE>(p, grid, st);
    else
      launch_q8_nw<D, 4, MODE>(p, grid, st);
  } else if constexpr (MODE == 1 && D == 64) {
    // The split pass likewise takes 8 waves (one subtile) at partitions of
    // 1024 positions or more on at most one workgroup per CU: same-box A/B
    // in both orders, us: B=32 x 4096 at P=1024 12.1 -> 10.35 (its best
    // partition size now; 10.8-11.2 at P=512 with 4 waves), B=4 x 32768
    // 10.8 -> 10.3-10.8.  Shorter partitions and larger grids keep 4 waves
    // (8 was 0.05-0.13 us slower at B=1 x 4096, B=1 x 32768 and B=8 x 4096,
    // and 1.7 us slower at B=128 x 8192).
    if (grid <= kStepWideMergeMaxGrid && p.a.partition_size >= 1024)
      launch_q8_nw<D, 8, MODE>(p, grid, st);
    else
      launch_q8_nw<D, 4, MODE>(p, grid, st);
  } else {
    launch_q8_nw<D, MODE >= 1 ? 4 : 8, MODE>(p, grid, st);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int fill_q8(pkv::Q8Params& p, const void* q, const void* k_codes, const void* v_codes,
            const float* k_scales, const float* v_scales, const int32_t* block_tables,
            const int32_t* context_lens, int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
            int32_t head_dim, int32_t block_size, int32_t num_blocks,
            int32_t max_blocks_per_seq, float scale) {
  int rc = check_attn_common(q, k_codes, v_codes, block_tables, context_lens, B, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                             scale);
  if (rc != PKV_OK) return rc;
  if (!k_scales || !v_scales || !aligned(k_scales, 16) || !aligned(v_scales, 16))
    return PKV_ERR_INVALID_ARG;
  p = {};
  p.a.q = static_cast<const pkv::f16*>(q);
  p.a.block_tables = block_tables;
  p.a.context_lens = context_lens;
  p.a.Hq = num_q_heads;
  p.a.Hkv = num_kv_heads;
  p.a.G = num_q_heads / num_kv_heads;
  p.a.block_size = block_size;
  p.a.num_blocks = num_blocks;
  p.a.max_blocks = max_blocks_per_seq;
  p.a.spb_shift = spb_shift_of(block_size);
  p.a.bs_shift = log2_or_neg(block_size);
  p.a.part_shift = log2_or_neg(p.a.partition_size);
  p.a.scale_log2 = scale * pkv::kLog2e;
  p.k_codes = static_cast<const int8_t*>(k_codes);
  p.v_codes = static_cast<const int8_t*>(v_codes);
  p.k_scales = k_scales;
  p.v_scales = v_scales;
  return PKV_OK;
}

// Argument checks of the fused step that do not involve its workspace
// (decided on the host, before any HIP call).
int check_step(const void* out, const float* lse_out, const void* q, const void* k_pool,
               const void* v_pool, const void* k_new, const void* v_new,
               const int64_t* slot_mapping, const int32_t* block_tables,
               const int32_t* context_lens, int32_t B, int32_t num_q_heads,
               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
               int32_t max_blocks_per_seq, int32_t partition_size, int32_t max_partitions,
               float scale) {
  int rc = check_attn_common(q, k_pool, v_pool, block_tables, context_lens, B, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                             scale);
  if (rc != PKV_OK) return rc;
  if (partition_size <= 0 || max_partitions <= 0 || partition_size % block_size != 0)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size < (int64_t)max_blocks_per_seq * block_size)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!out || !aligned(out, 16) || (lse_out && !aligned(lse_out, 4))) return PKV_ERR_INVALID_ARG;
  if (slot_mapping) {
    if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16) ||
        !aligned(slot_mapping, 8))
      return PKV_ERR_INVALID_ARG;
  }
  const int64_t cells = (int64_t)B * num_kv_heads * max_partitions;
  if (cells > INT32_MAX) return PKV_ERR_INVALID_ARG;
  // one buffer resource spans a pair's partials; its byte offsets, and the
  // out-of-range offset the merge uses for rows it skips (2^30), must not meet
  if ((int64_t)(num_q_heads / num_kv_heads) * max_partitions * head_dim * 4 >= (1 << 30))
    return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

int launch_step(void* out, float* lse_out, void* k_pool, void* v_pool, const void* q,
                const void* k_new, const void* v_new, const int64_t* slot_mapping,
                const int32_t* block_tables, const int32_t* context_lens, float* partial_out,
                float* partial_lse, int32_t* counters, int32_t B, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                int32_t max_blocks_per_seq, int32_t partition_size, int32_t max_partitions,
                float scale, const pkv_launch_config* config, hipStream_t st) {
  AttnParams p = {};
  p.q = static_cast<const pkv::f16*>(q);
  p.k_pool = static_cast<const pkv::f16*>(k_pool);
  p.v_pool = static_cast<const pkv::f16*>(v_pool);
  p.k_pool_w = static_cast<pkv::f16*>(k_pool);
  p.v_pool_w = static_cast<pkv::f16*>(v_pool);
  p.k_new = static_cast<const pkv::f16*>(k_new);
  p.v_new = static_cast<const pkv::f16*>(v_new);
  p.slot_mapping = slot_mapping;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = static_cast<pkv::f16*>(out);
  p.lse_out = lse_out;
  p.partial_out = partial_out;
  p.partial_lse = partial_lse;
  p.counters = counters;
  p.B = B;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.G = num_q_heads / num_kv_heads;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.partition_size = partition_size;
  p.max_partitions = max_partitions;
  p.spb_shift = spb_shift_of(block_size);
  p.bs_shift = log2_or_neg(block_size);
  p.part_shift = log2_or_neg(partition_size);
  p.scale_log2 = scale * pkv::kLog2e;
  return launch_attn<2>(p, head_dim, config, st);
}

// ---- paged_decode_step_noalloc: the fused step on a static scratch -------
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the step's workspace
// (partials, their lse, ticket counters) lives in this file-scope device
// array instead of a caller buffer.  Each GPU the library runs on holds its
// own copy until the process ends.  Its rest state is all zero, which every
// call leaves (as the workspace contract of paged_decode_step).
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchLayout {
  size_t partial_out, partial_lse, counters;
};

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// Byte offsets of the workspace parts in the scratch; false if they do not fit.
bool scratch_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t Pm,
                    ScratchLayout* L) {
  const size_t po = round256((size_t)B * Hq * Pm * D * 4);
  const size_t pl = round256((size_t)B * Hq * Pm * 4);
  const size_t ct = round256((size_t)B * Hkv * pkv::kCounterStride * 4);
  L->partial_out = 0;
  L->partial_lse = po;
  L->counters = po + pl;
  return po + pl + ct <= kScratchBytes;
}

__global__ __launch_bounds__(256) void zero_scratch_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The scratch's device address on the current device (the array's name is a
// host-side stand-in, never passed to a kernel).  Resolved once per device
// with that device current, and cleared once there by a fill kernel on the
// caller's stream (ordered before the caller's step; a memset node is never
// recorded into a graph the caller may be capturing).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch[kMaxDevices] = {};

int device_scratch(unsigned char** out, hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return PKV_ERR_LAUNCH;
    hipLaunchKernelGGL(zero_scratch_kernel, dim3(1024), dim3(256), 0, st,
                       static_cast<uint4*>(ptr), kScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
    g_scratch[dev] = static_cast<unsigned char*>(ptr);
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_NO_SPACE: return "no space: not enough free cache blocks";
    case PKV_ERR_SCRATCH:
      return "the call needs more than paged_decode_step_noalloc's static scratch holds";
    default: return "unknown status";
  }
}

int pkv_version(void) { return kVersion; }

int kv_cache_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                    const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                    int32_t block_size, int32_t num_kv_heads, int32_t head_dim, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!k_pool || !v_pool || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return PKV_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;  // empty per-token arrays may be null
  if (!k_new || !v_new || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 8))
    return PKV_ERR_INVALID_ARG;

  AppendParams p;
  p.k_pool = static_cast<pkv::f16*>(k_pool);
  p.v_pool = static_cast<pkv::f16*>(v_pool);
  p.k_new = static_cast<const pkv::f16*>(k_new);
  p.v_new = static_cast<const pkv::f16*>(v_new);
  p.slot_mapping = slot_mapping;
  p.num_slots = (int64_t)num_blocks * block_size;
  p.num_tokens = num_tokens;
  p.Hkv = num_kv_heads;
  p.D = head_dim;
  const int64_t threads = (int64_t)num_tokens * num_kv_heads * (head_dim / 8);
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(pkv::append_kernel, dim3((unsigned)grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_attention_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                           float scale, void* stream) {
  return paged_attention_decode_ex(out, q, k_pool, v_pool, block_tables, context_lens, B,
                                   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                   max_blocks_per_seq, scale, nullptr, stream);
}

int paged_attention_decode_ex(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, float scale,
                              const pkv_launch_config* config, void* stream) {
  if (!config_ok(config)) return PKV_ERR_INVALID_ARG;
  int rc = check_attn_common(q, k_pool, v_pool, block_tables, context_lens, B, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                             scale);
  if (rc != PKV_OK) return rc;
  if (B == 0) return PKV_OK;
  if (!out || !aligned(out, 16)) return PKV_ERR_INVALID_ARG;
  const int64_t grid = (int64_t)B * num_kv_heads;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;

  AttnParams p = {};
  p.q = static_cast<const pkv::f16*>(q);
  p.k_pool = static_cast<const pkv::f16*>(k_pool);
  p.v_pool = static_cast<const pkv::f16*>(v_pool);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = static_cast<pkv::f16*>(out);
  p.B = B;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.G = num_q_heads / num_kv_heads;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.partition_size = max_blocks_per_seq * block_size;
  p.max_partitions = 1;
  p.spb_shift = spb_shift_of(block_size);
  p.bs_shift = log2_or_neg(block_size);
  p.part_shift = log2_or_neg(p.partition_size);
  p.scale_log2 = scale * pkv::kLog2e;
  return launch_attn<0>(p, head_dim, config, static_cast<hipStream_t>(stream));
}

int paged_attention_decode_split(float* partial_out, float* partial_lse, const void* q,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t partition_size,
                                 int32_t max_partitions, float scale, void* stream) {
  return paged_attention_decode_split_ex(partial_out, partial_lse, q, k_pool, v_pool,
                                         block_tables, context_lens, B, num_q_heads,
                                         num_kv_heads, head_dim, block_size, num_blocks,
                                         max_blocks_per_seq, partition_size, max_partitions,
                                         scale, nullptr, stream);
}

int paged_attention_decode_split_ex(float* partial_out, float* partial_lse, const void* q,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t max_blocks_per_seq, int32_t partition_size,
                                    int32_t max_partitions, float scale,
                                    const pkv_launch_config* config, void* stream) {
  if (!config_ok(config)) return PKV_ERR_INVALID_ARG;
  int rc = check_attn_common(q, k_pool, v_pool, block_tables, context_lens, B, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                             scale);
  if (rc != PKV_OK) return rc;
  if (partition_size <= 0 || max_partitions <= 0 || partition_size % block_size != 0)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size < (int64_t)max_blocks_per_seq * block_size)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!partial_out || !partial_lse || !aligned(partial_out, 16) || !aligned(partial_lse, 4))
    return PKV_ERR_INVALID_ARG;
  const int64_t grid = (int64_t)B * num_kv_heads * max_partitions;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;

  AttnParams p = {};
  p.q = static_cast<const pkv::f16*>(q);
  p.k_pool = static_cast<const pkv::f16*>(k_pool);
  p.v_pool = static_cast<const pkv::f16*>(v_pool);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.partial_out = partial_out;
  p.partial_lse = partial_lse;
  p.B = B;
  p.Hq = num_q_heads;
  p.Hkv = num_kv_heads;
  p.G = num_q_heads / num_kv_heads;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.partition_size = partition_size;
  p.max_partitions = max_partitions;
  p.spb_shift = spb_shift_of(block_size);
  p.bs_shift = log2_or_neg(block_size);
  p.part_shift = log2_or_neg(p.partition_size);
  p.scale_log2 = scale * pkv::kLog2e;
  return launch_attn<1>(p, head_dim, config, static_cast<hipStream_t>(stream));
}

int paged_decode_step(void* out, float* lse_out, void* k_pool, void* v_pool, const void* q,
                      const void* k_new, const void* v_new, const int64_t* slot_mapping,
                      const int32_t* block_tables, const int32_t* context_lens,
                      float* partial_out, float* partial_lse, int32_t* counters, int32_t B,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                      int32_t partition_size, int32_t max_partitions, float scale,
                      void* stream) {
  return paged_decode_step_ex(out, lse_out, k_pool, v_pool, q, k_new, v_new, slot_mapping,
                              block_tables, context_lens, partial_out, partial_lse, counters, B,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                              max_blocks_per_seq, partition_size, max_partitions, scale,
                              nullptr, stream);
}

int paged_decode_step_ex(void* out, float* lse_out, void* k_pool, void* v_pool, const void* q,
                         const void* k_new, const void* v_new, const int64_t* slot_mapping,
                         const int32_t* block_tables, const int32_t* context_lens,
                         float* partial_out, float* partial_lse, int32_t* counters, int32_t B,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t partition_size, int32_t max_partitions, float scale,
                         const pkv_launch_config* config, void* stream) {
  if (!config_ok(config)) return PKV_ERR_INVALID_ARG;
  int rc = check_step(out, lse_out, q, k_pool, v_pool, k_new, v_new, slot_mapping, block_tables,
                      context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size,
                      num_blocks, max_blocks_per_seq, partition_size, max_partitions, scale);
  if (rc != PKV_OK || B == 0) return rc;
  if (!partial_out || !partial_lse || !counters) return PKV_ERR_INVALID_ARG;
  if (!aligned(partial_out, 16) || !aligned(partial_lse, 4) || !aligned(counters, 8))
    return PKV_ERR_INVALID_ARG;
  return launch_step(out, lse_out, k_pool, v_pool, q, k_new, v_new, slot_mapping, block_tables,
                     context_lens, partial_out, partial_lse, counters, B, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     partition_size, max_partitions, scale, config,
                     static_cast<hipStream_t>(stream));
}

int paged_decode_step_noalloc(void* out, float* lse_out, void* k_pool, void* v_pool,
                              const void* q, const void* k_new, const void* v_new,
                              const int64_t* slot_mapping, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t B, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t partition_size, int32_t max_partitions, float scale,
                              void* stream) {
  int rc = check_step(out, lse_out, q, k_pool, v_pool, k_new, v_new, slot_mapping, block_tables,
                      context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size,
                      num_blocks, max_blocks_per_seq, partition_size, max_partitions, scale);
  if (rc != PKV_OK || B == 0) return rc;
  ScratchLayout L;
  if (!scratch_layout(B, num_q_heads, num_kv_heads, head_dim, max_partitions, &L))
    return PKV_ERR_SCRATCH;
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned char* base = nullptr;
  rc = device_scratch(&base, st);
  if (rc != PKV_OK) return rc;
  return launch_step(out, lse_out, k_pool, v_pool, q, k_new, v_new, slot_mapping, block_tables,
                     context_lens, reinterpret_cast<float*>(base + L.partial_out),
                     reinterpret_cast<float*>(base + L.partial_lse),
                     reinterpret_cast<int32_t*>(base + L.counters), B, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     partition_size, max_partitions, scale, nullptr, st);
}

int paged_attention_prefill(void* out, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* query_start, int32_t B, int32_t max_query_len,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            float scale, void* stream) {
  int rc = check_attn_common(q, k_pool, v_pool, block_tables, context_lens, B, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                             scale);
  if (rc != PKV_OK) return rc;
  if (max_query_len < 0) return PKV_ERR_INVALID_ARG;
  if (B == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !query_start || !aligned(out, 16) || !aligned(query_start, 4))
    return PKV_ERR_INVALID_ARG;
  const int G = num_q_heads / num_kv_heads;
  const int rows = pkv::prefill_rows_per_tile(head_dim == 64 ? 4 : 2, G);
  const int64_t q_tiles = (max_query_len + rows - 1) / rows;
  const int64_t grid = (int64_t)B * num_kv_heads * q_tiles;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;

  pkv::PrefillParams p = {};
  p.a.q = static_cast<const pkv::f16*>(q);
  p.a.k_pool = static_cast<const pkv::f16*>(k_pool);
  p.a.v_pool = static_cast<const pkv::f16*>(v_pool);
  p.a.block_tables = block_tables;
  p.a.context_lens = context_lens;
  p.a.out = static_cast<pkv::f16*>(out);
  p.a.Hq = num_q_heads;
  p.a.Hkv = num_kv_heads;
  p.a.G = G;
  p.a.block_size = block_size;
  p.a.num_blocks = num_blocks;
  p.a.max_blocks = max_blocks_per_seq;
  p.a.spb_shift = spb_shift_of(block_size);
  p.a.bs_shift = log2_or_neg(block_size);
  p.a.part_shift = log2_or_neg(p.a.partition_size);
  p.a.scale_log2 = scale * pkv::kLog2e;
  p.query_start = query_start;
  p.max_q = max_query_len;
  p.q_tiles = (int32_t)q_tiles;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return head_dim == 64 ? launch_prefill<64, false>(p, grid, st)
                        : launch_prefill<128, false>(p, grid, st);
}

int paged_attention_prefill_split(float* partial_out, float* partial_lse,
                                  int32_t* row_context_lens, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* query_start,
                                  int32_t B, int32_t max_query_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, int32_t max_blocks_per_seq,
                                  int32_t partition_size, int32_t max_partitions, float scale,
                                  void* stream) {
  int rc = check_attn_common(q, k_pool, v_pool, block_tables, context_lens, B, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                             scale);
  if (rc != PKV_OK) return rc;
  if (max_query_len < 0) return PKV_ERR_INVALID_ARG;
  if (partition_size <= 0 || max_partitions <= 0 || partition_size % block_size != 0)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size < (int64_t)max_blocks_per_seq * block_size)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (B == 0 || max_query_len == 0) return PKV_OK;
  if (!partial_out || !partial_lse || !row_context_lens || !query_start ||
      !aligned(partial_out, 16) || !aligned(partial_lse, 4) || !aligned(row_context_lens, 4) ||
      !aligned(query_start, 4))
    return PKV_ERR_INVALID_ARG;
  const int G = num_q_heads / num_kv_heads;
  const int rows = pkv::prefill_rows_per_tile(head_dim == 64 ? 4 : 2, G);
  const int64_t q_tiles = (max_query_len + rows - 1) / rows;
  const int64_t grid = (int64_t)B * num_kv_heads * q_tiles * max_partitions;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;

  pkv::PrefillParams p = {};
  p.a.q = static_cast<const pkv::f16*>(q);
  p.a.k_pool = static_cast<const pkv::f16*>(k_pool);
  p.a.v_pool = static_cast<const pkv::f16*>(v_pool);
  p.a.block_tables = block_tables;
  p.a.context_lens = context_lens;
  p.a.partial_out = partial_out;
  p.a.partial_lse = partial_lse;
  p.a.Hq = num_q_heads;
  p.a.Hkv = num_kv_heads;
  p.a.G = G;
  p.a.block_size = block_size;
  p.a.num_blocks = num_blocks;
  p.a.max_blocks = max_blocks_per_seq;
  p.a.partition_size = partition_size;
  p.a.max_partitions = max_partitions;
  p.a.spb_shift = spb_shift_of(block_size);
  p.a.bs_shift = log2_or_neg(block_size);
  p.a.part_shift = log2_or_neg(p.a.partition_size);
  p.a.scale_log2 = scale * pkv::kLog2e;
  p.query_start = query_start;
  p.max_q = max_query_len;
  p.q_tiles = (int32_t)q_tiles;
  p.row_ctx = row_context_lens;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return head_dim == 64 ? launch_prefill<64, true>(p, grid, st)
                        : launch_prefill<128, true>(p, grid, st);
}

int kv_cache_append_q8(void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                       const void* k_new, const void* v_new, const int64_t* slot_mapping,
                       int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_dim, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0)
    return PKV_ERR_INVALID_ARG;
  if (!k_codes || !v_codes || !k_scales || !v_scales || !aligned(k_codes, 16) ||
      !aligned(v_codes, 16) || !aligned(k_scales, 16) || !aligned(v_scales, 16))
    return PKV_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim) || !block_size_ok(block_size)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(slot_mapping, 8))
    return PKV_ERR_INVALID_ARG;
  pkv::AppendQ8Params p;
  p.k_codes = static_cast<int8_t*>(k_codes);
  p.v_codes = static_cast<int8_t*>(v_codes);
  p.k_scales = k_scales;
  p.v_scales = v_scales;
  p.k_new = static_cast<const pkv::f16*>(k_new);
  p.v_new = static_cast<const pkv::f16*>(v_new);
  p.slot_mapping = slot_mapping;
  p.num_slots = (int64_t)num_blocks * block_size;
  p.num_tokens = num_tokens;
  p.Hkv = num_kv_heads;
  p.D = head_dim;
  p.block_size = block_size;
  const int64_t threads = (int64_t)num_tokens * num_kv_heads * (head_dim / 8);
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(pkv::append_q8_kernel, dim3((unsigned)grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_attention_decode_q8(void* out, const void* q, const void* k_codes, const void* v_codes,
                              const float* k_scales, const float* v_scales,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, float scale, void* stream) {
  pkv::Q8Params p;
  int rc = fill_q8(p, q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens, B,
                   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                   max_blocks_per_seq, scale);
  if (rc != PKV_OK) return rc;
  if (B == 0) return PKV_OK;
  if (!out || !aligned(out, 16)) return PKV_ERR_INVALID_ARG;
  const int64_t grid = (int64_t)B * num_kv_heads;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;
  p.a.out = static_cast<pkv::f16*>(out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return head_dim == 64 ? launch_q8<64, 0>(p, grid, st) : launch_q8<128, 0>(p, grid, st);
}

int paged_attention_decode_split_q8(float* partial_out, float* partial_lse, const void* q,
                                    const void* k_codes, const void* v_codes,
                                    const float* k_scales, const float* v_scales,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t max_blocks_per_seq, int32_t partition_size,
                                    int32_t max_partitions, float scale, void* stream) {
  pkv::Q8Params p;
  int rc = fill_q8(p, q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens, B,
                   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                   max_blocks_per_seq, scale);
  if (rc != PKV_OK) return rc;
  if (partition_size <= 0 || max_partitions <= 0 || partition_size % block_size != 0)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size < (int64_t)max_blocks_per_seq * block_size)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!partial_out || !partial_lse || !aligned(partial_out, 16) || !aligned(partial_lse, 4))
    return PKV_ERR_INVALID_ARG;
  const int64_t grid = (int64_t)B * num_kv_heads * max_partitions;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;
  p.a.partial_out = partial_out;
  p.a.partial_lse = partial_lse;
  p.a.partition_size = partition_size;
  p.a.part_shift = log2_or_neg(partition_size);
  p.a.max_partitions = max_partitions;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return head_dim == 64 ? launch_q8<64, 1>(p, grid, st) : launch_q8<128, 1>(p, grid, st);
}

int paged_decode_step_q8(void* out, float* lse_out, void* k_codes, void* v_codes,
                         float* k_scales, float* v_scales, const void* q, const void* k_new,
                         const void* v_new, const int64_t* slot_mapping,
                         const int32_t* block_tables, const int32_t* context_lens,
                         float* partial_out, float* partial_lse, int32_t* counters, int32_t B,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t partition_size, int32_t max_partitions, float scale,
                         void* stream) {
  pkv::Q8Params p;
  int rc = fill_q8(p, q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens, B,
                   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                   max_blocks_per_seq, scale);
  if (rc != PKV_OK) return rc;
  if (partition_size <= 0 || max_partitions <= 0 || partition_size % block_size != 0)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size < (int64_t)max_blocks_per_seq * block_size)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (!out || !partial_out || !partial_lse || !counters) return PKV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(partial_out, 16) || !aligned(partial_lse, 4) ||
      !aligned(counters, 8) || (lse_out && !aligned(lse_out, 4)))
    return PKV_ERR_INVALID_ARG;
  if (slot_mapping) {
    if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16) ||
        !aligned(slot_mapping, 8))
      return PKV_ERR_INVALID_ARG;
  }
  const int64_t grid = (int64_t)B * num_kv_heads * max_partitions;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;
  // as paged_decode_step: a pair's partials fit one buffer resource below the
  // merge's out-of-range offset (2^30)
  if ((int64_t)(num_q_heads / num_kv_heads) * max_partitions * head_dim * 4 >= (1 << 30))
    return PKV_ERR_UNSUPPORTED;
  p.a.out = static_cast<pkv::f16*>(out);
  p.a.lse_out = lse_out;
  p.a.partial_out = partial_out;
  p.a.partial_lse = partial_lse;
  p.a.counters = counters;
  p.a.B = B;
  p.a.partition_size = partition_size;
  p.a.part_shift = log2_or_neg(partition_size);
  p.a.max_partitions = max_partitions;
  p.a.k_new = static_cast<const pkv::f16*>(k_new);
  p.a.v_new = static_cast<const pkv::f16*>(v_new);
  p.a.slot_mapping = slot_mapping;
  p.k_codes_w = static_cast<int8_t*>(k_codes);
  p.v_codes_w = static_cast<int8_t*>(v_codes);
  p.k_scales_w = k_scales;
  p.v_scales_w = v_scales;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return head_dim == 64 ? launch_q8<64, 2>(p, grid, st) : launch_q8<128, 2>(p, grid, st);
}

// The row-batched merge walks a pair's partitions four at a time, one memory
// round trip per four; the per-pair kernel keeps 16 rows in flight.  So the
// row-batched form is taken only where it needs at most four round trips.
constexpr int64_t kRowsMergeAbove = 4096;
constexpr int32_t kRowsMergeMaxPartitions = 16;

int split_reduce(void* out, float* lse_out, const float* partial_out, const float* partial_lse,
                 const int32_t* context_lens, int32_t B, int32_t num_q_heads, int32_t head_dim,
                 int32_t partition_size, int32_t max_partitions, void* stream) {
  if (B < 0 || num_q_heads <= 0 || partition_size <= 0 || max_partitions <= 0)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_partitions * partition_size > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (!head_dim_ok(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (B == 0) return PKV_OK;
  if (!out || !partial_out || !partial_lse || !context_lens) return PKV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(partial_out, 16) || !aligned(partial_lse, 4) ||
      !aligned(context_lens, 4) || (lse_out && !aligned(lse_out, 4)))
    return PKV_ERR_INVALID_ARG;
  const int64_t grid = (int64_t)B * num_q_heads;
  if (grid > INT32_MAX) return PKV_ERR_INVALID_ARG;

  ReduceParams p;
  p.out = static_cast<pkv::f16*>(out);
  p.lse_out = lse_out;
  p.partial_out = partial_out;
  p.partial_lse = partial_lse;
  p.context_lens = context_lens;
  p.Hq = num_q_heads;
  p.partition_size = partition_size;
  p.max_partitions = max_partitions;
  p.B = B;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // Many (row, head) pairs with few partitions each (the rows of a split
  // prefill): a workgroup per 16 (D=64) or 8 (D=128) pairs instead of one per
  // pair, whose dispatches would dominate (7,168 for 8 x 64-row chunks).
  if (grid >= kRowsMergeAbove && max_partitions <= kRowsMergeMaxPartitions) {
    const int rpw = 256 / (head_dim / 4);
    const unsigned g = (unsigned)((grid + rpw - 1) / rpw);
    if (head_dim == 64)
      hipLaunchKernelGGL(pkv::split_reduce_rows_kernel<64>, dim3(g), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL(pkv::split_reduce_rows_kernel<128>, dim3(g), dim3(256), 0, st, p);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
  }
  if (head_dim == 64)
    hipLaunchKernelGGL(pkv::split_reduce_kernel<64>, dim3((unsigned)grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(pkv::split_reduce_kernel<128>, dim3((unsigned)grid), dim3(256), 0, st, p);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"
