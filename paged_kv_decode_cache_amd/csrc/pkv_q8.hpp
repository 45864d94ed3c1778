// 8-bit KV cache on gfx950: the quantising cache write and the decode passes
// (unsplit and split) over int8 codes with one fp32 scale per (token, KV
// head) row.
//
// Format (this library's; the pages only mention another system's q8 cache):
// codes [num_blocks, Hkv, block_size, D] int8, scales [num_blocks, Hkv,
// block_size] fp32: head-major within a block, so one head's rows of a block
// are contiguous (16 rows of 64 codes fill whole 128-byte lines; with the
// heads interleaved per token, as in the fp16 pools, a workgroup reading one
// head used half of every line it fetched), and a lane fetches its four
// tokens' scales with one 16-byte load.  A row's value is
// code * scale, quantised when written: amax = max |x|, inv = 127 / amax and
// code = rint(x * inv) in fp32 (IEEE division, nearest-even), scale =
// amax / 127; a zero row has codes 0 and scale 0.
//
// Decode over codes keeps the fp16 kernel's structure and arithmetic:
//   * K: a lane loads 16 contiguous codes of its token (one 16-byte load per
//     64 dims); the MFMA's k order is free, so q is loaded in the same
//     permuted order.  Codes become exact fp16 integers with one byte
//     permute per two values (0x64 high byte: the fp16 value 1024 + code +
//     128) and a packed-half subtract of 1152.  S = scale_k(t) * (q . code_t)
//     in fp32.
//   * V: codes become exact fp16 integers the same way and go through LDS
//     for the transposing read; the row scale folds into the softmax weight
//     (p * scale_v(t)) before its fp16 high/remainder split, so P.V keeps
//     fp32-level accuracy.  The weight sums (unscaled p) are taken on the
//     VALU per lane and reduced across the four quads once at the end.
#pragma once

#include "pkv_kernels.hpp"

namespace pkv {

typedef f16 f16x2 __attribute__((ext_vector_type(2)));

struct Q8Params {
  AttnParams a;            // k_pool / v_pool unused
  const int8_t* k_codes;   // [NB, Hkv, bs, D]
  const int8_t* v_codes;
  const float* k_scales;   // [NB, Hkv, bs]
  const float* v_scales;
  // fused decode step: the same arrays, written by the step's append
  int8_t* k_codes_w;
  int8_t* v_codes_w;
  float* k_scales_w;
  float* v_scales_w;
};

struct AppendQ8Params {
  int8_t* k_codes;
  int8_t* v_codes;
  float* k_scales;
  float* v_scales;
  const f16* k_new;        // [N, Hkv, D]
  const f16* v_new;
  const int64_t* slot_mapping;
  int64_t num_slots;
  int32_t num_tokens, Hkv, D, block_size;
};

// Quantising cache write: D/8 consecutive threads hold one (token, head) row,
// 8 values each; the row's amax is reduced across them with shuffles.
__global__ __launch_bounds__(256) void append_q8_kernel(const AppendQ8Params p) {
  const int D = p.D;
  const int per_row = D >> 3;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)p.num_tokens * p.Hkv;
  const int64_t row = gid / per_row;
  const int part = (int)(gid % per_row);
  const bool live = row < rows;
  const int64_t n = live ? row / p.Hkv : 0;
  const int h = live ? (int)(row % p.Hkv) : 0;
  const int64_t slot = live ? p.slot_mapping[n] : -1;
  f16x8 kx = zero8(), vx = zero8();
  if (live) {
    kx = *reinterpret_cast<const f16x8*>(p.k_new + (n * p.Hkv + h) * D + 8 * part);
    vx = *reinterpret_cast<const f16x8*>(p.v_new + (n * p.Hkv + h) * D + 8 * part);
  }
  float ka = 0.0f, va = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ka = fmaxf(ka, fabsf((float)kx[i]));
    va = fmaxf(va, fabsf((float)vx[i]));
  }
  // every lane takes part in the reductions (row groups are aligned in a wave)
  for (int off = 1; off < per_row; off <<= 1) {
    ka = fmaxf(ka, __shfl_xor(ka, off));
    va = fmaxf(va, __shfl_xor(va, off));
  }
  if (!live || slot < 0 || slot >= p.num_slots) return;
  const float kinv = ka > 0.0f ? 127.0f / ka : 0.0f;  // IEEE division
  const float vinv = va > 0.0f ? 127.0f / va : 0.0f;
  uint32_t kw[2] = {0, 0}, vw[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float kc = fminf(fmaxf(__builtin_rintf((float)kx[i] * kinv), -127.0f), 127.0f);
    const float vc = fminf(fmaxf(__builtin_rintf((float)vx[i] * vinv), -127.0f), 127.0f);
    kw[i >> 2] |= (uint32_t)((int)kc & 0xFF) << (8 * (i & 3));
    vw[i >> 2] |= (uint32_t)((int)vc & 0xFF) << (8 * (i & 3));
  }
  const int64_t blk = slot / p.block_size;
  const int off = (int)(slot - blk * p.block_size);
  const int64_t si = (blk * p.Hkv + h) * p.block_size + off;  // (block, head, offset)
  const int64_t base = si * D + 8 * part;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2*>(p.k_codes + base) = u32x2{kw[0], kw[1]};
  *reinterpret_cast<u32x2*>(p.v_codes + base) = u32x2{vw[0], vw[1]};
  if (part == 0) {
    p.k_scales[si] = ka / 127.0f;
    p.v_scales[si] = va / 127.0f;
  }
}

// Two int8 codes (bytes `sel` of w) as exact fp16 values.
__device__ __forceinline__ f16x2 codes_to_f16x2(uint32_t w_offset_binary, uint32_t sel) {
  const uint32_t r = __builtin_amdgcn_perm(0x64646464u, w_offset_binary, sel);
  f16x2 bias;
  bias[0] = (f16)1152.0f;
  bias[1] = (f16)1152.0f;
  return __builtin_bit_cast(f16x2, r) - bias;
}

// Eight codes (words 2h and 2h+1 of a 16-byte chunk) as fp16.
__device__ __forceinline__ f16x8 codes_to_f16x8(u32x4 w, int h) {
  const uint32_t a = w[2 * h] ^ 0x80808080u;
  const uint32_t b = w[2 * h + 1] ^ 0x80808080u;
  const f16x2 p0 = codes_to_f16x2(a, 0x04010400u);
  const f16x2 p1 = codes_to_f16x2(a, 0x04030402u);
  const f16x2 p2 = codes_to_f16x2(b, 0x04010400u);
  const f16x2 p3 = codes_to_f16x2(b, 0x04030402u);
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

template <int D, int NS>
struct KVTile8 {
  u32x4 k[NS][D / 64];  // 16 codes per 64 dims: token lane%16, dims 64c + 16*quad ..
  u32x4 v[NS][D / 64];
  f32x4 ks[NS];         // scales of tokens 4*quad .. 4*quad+3
  f32x4 vs[NS];
  int okmask;
  int s0;
  int new_phys;  // block id of subtile s_new when the tile holds it, else -1
  bool full;
};

// The fused step's new token row of one KV head (fp16, D values at `row`),
// quantised by the format's rule into a tile's lane layout: lane quad q holds
// the codes of dims 64c + 16q .. 64c + 16q + 15 (bytes in dim order), and
// every lane gets the row's scale.  The decisions are append_q8_kernel's
// (fp32 amax, IEEE division 127 / amax, nearest-even rint of x * inv, clip),
// so the codes and scale are bit-identical to the cache write's.  All 64
// lanes of the wave must run it (cross-quad maximum).
template <int D>
__device__ __forceinline__ void quantize_row_lanes(const f16* row, int quad,
                                                   u32x4 (&codes)[D / 64], float& scale) {
  f16x8 x[D / 64][2];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < D / 64; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      x[c][h] = *reinterpret_cast<const f16x8*>(row + 64 * c + 16 * quad + 8 * h);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf((float)x[c][h][i]));
    }
  amax = max_across_quads(amax);
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;  // IEEE division
#pragma unroll
  for (int c = 0; c < D / 64; ++c) {
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q =
            fminf(fmaxf(__builtin_rintf((float)x[c][h][i] * inv), -127.0f), 127.0f);
        w[2 * h + (i >> 2)] |= (uint32_t)((int)q & 0xFF) << (8 * (i & 3));
      }
    codes[c] = w;
  }
  scale = amax / 127.0f;
}

// Codes and scales are each read once per pass: non-temporal loads, as the
// fp16 kernels' K/V lines (bit-cast through a float vector, as load_b128).
__device__ __forceinline__ f32x4 load_b128_stream(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNonTemporal));
}

template <int D, int NS>
__device__ __forceinline__ void load_kv_tile8(KVTile8<D, NS>& T, const Q8Params& P, int ids,
                                              int s0, int sub_end, int t_end, int spb,
                                              int spb_shift, int kvh, int lane,
                                              int s_new = -1) {
  const AttnParams& a = P.a;
  const int quad = lane >> 4;
  T.s0 = s0;
  int okm = 0;
  int new_phys = -1;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int phys = __builtin_amdgcn_readlane(ids, j);
    new_phys = s0 + j == s_new ? phys : new_phys;
    const bool ok = s0 + j < sub_end && phys >= 0 && phys < a.num_blocks;
    okm |= (ok ? 1 : 0) << j;
    const int s = s0 + j;
    const int sib = spb_shift >= 0 ? (s & (spb - 1)) : (s % spb);
    const int64_t p0 = ok ? phys : 0;
    // the subtile's codes of head kvh (16 contiguous rows of D codes) and
    // its 16 scales, through empty resources when masked out
    const int64_t so = (p0 * a.Hkv + kvh) * a.block_size + sib * 16;
    const int64_t co = so * D;
    const int code_bytes = ok ? 16 * D : 0;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(P.k_codes + co, code_bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(P.v_codes + co, code_bytes);
    const int lo = (lane & 15) * D + 16 * quad;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      T.k[j][c] = __builtin_bit_cast(u32x4, load_b128_stream(kr, lo + 64 * c));
      T.v[j][c] = __builtin_bit_cast(u32x4, load_b128_stream(vr, lo + 64 * c));
    }
    const __amdgpu_buffer_rsrc_t ksr = buffer_rsrc(P.k_scales + so, ok ? 64 : 0);
    const __amdgpu_buffer_rsrc_t vsr = buffer_rsrc(P.v_scales + so, ok ? 64 : 0);
    T.ks[j] = load_b128_stream(ksr, 16 * quad);
    T.vs[j] = load_b128_stream(vsr, 16 * quad);
  }
  T.okmask = okm;
  T.new_phys = new_phys;
  T.full = okm == (1 << NS) - 1 && ((s0 + NS) << 4) <= t_end;
}

// QK^T, online-softmax update and PV for one tile of codes (see the header).
// SUB: position (s_new, tok_new) takes the codes and scales of the fused
// step's new token (kq/vq, ksc/vsc, quantised in registers and written to
// the cache by this launch) when `slot` is the position's slot in the table.
// lsum: this lane's running sum of its column's (unscaled) weights.
template <int D, int NS, bool DUAL, bool SUB>
__device__ __forceinline__ void consume_tile8(KVTile8<D, NS>& T, SoftmaxState<D>& st,
                                              float& lsum, const f16x8 (&qb)[D / 32],
                                              f16* stage, float c, int t_end, int lane,
                                              float rem_mul, int s_new, int tok_new,
                                              int64_t slot, int new_off, int block_size,
                                              const u32x4 (&kq)[D / 64],
                                              const u32x4 (&vq)[D / 64], float ksc,
                                              float vsc) {
  constexpr int KC = D / 32;
  constexpr int NDB = D / 16;
  constexpr int ROW = D + 4;
  const int g = lane & 15;
  const int quad = lane >> 4;
  if (SUB && T.new_phys >= 0 && (int64_t)T.new_phys * block_size + new_off == slot) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const bool here = T.s0 + j == s_new;
      const bool mine = here && (lane & 15) == tok_new;
#pragma unroll
      for (int cc = 0; cc < D / 64; ++cc) {
        T.k[j][cc] = mine ? kq[cc] : T.k[j][cc];
        T.v[j][cc] = mine ? vq[cc] : T.v[j][cc];
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const bool its = here && 4 * quad + v == tok_new;
        T.ks[j][v] = its ? ksc : T.ks[j][v];
        T.vs[j][v] = its ? vsc : T.vs[j][v];
      }
    }
  }

  f32x4 sc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    f32x4 acc = zero4f();
#pragma unroll
    for (int m = 0; m < KC; ++m)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes_to_f16x8(T.k[j][m >> 1], m & 1), qb[m],
                                                   acc, 0, 0, 0);
    sc[j] = acc * T.ks[j];
  }
  if (!T.full) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = ((T.s0 + j) << 4) + 4 * quad + v;
        const bool ok = ((T.okmask >> j) & 1) && tok < t_end;
        sc[j][v] = ok ? sc[j][v] : -INFINITY;
        T.vs[j][v] = ok ? T.vs[j][v] : 0.0f;  // an unwritten slot's scale may be NaN
      }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) tmax = fmaxf(tmax, sc[j][v]);
  tmax = max_across_quads(tmax);
  const float tmax_s = tmax * c;
  const bool grow = tmax_s > st.m + kRescaleLog2;
  if (__any(grow)) {
    const float m_new = grow ? tmax_s : st.m;
    const float alpha = grow ? fast_exp2(st.m - m_new) : 1.0f;
    st.m = m_new;
    lsum *= alpha;
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
      const float p = fast_exp2(fmaf(sc[j][v], c, neg_m));
      lsum += p;
      pv[v] = p * T.vs[j][v];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f16 h = (f16)pv[v];
      if (DUAL) {
        ph[j][v] = (f16)fmaf((float)h, rem_mul, pv[v]);
      } else {
        ph[j][v] = h;
        pl[j][v] = (f16)fmaf((float)h, rem_mul, pv[v]);
      }
    }
  }

  // V codes -> exact fp16 -> LDS row-major [token][dim]; masked rows as zeros
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    f16* row = stage + (j * 16 + (lane & 15)) * ROW + 16 * quad;
    const int tok = ((T.s0 + j) << 4) + (lane & 15);
    const bool keep = T.full || (((T.okmask >> j) & 1) && tok < t_end);
#pragma unroll
    for (int cc = 0; cc < D / 64; ++cc) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f16x8 v = keep ? codes_to_f16x8(T.v[j][cc], h) : zero8();
        *reinterpret_cast<f16x4*>(row + 64 * cc + 8 * h) = v.lo;
        *reinterpret_cast<f16x4*>(row + 64 * cc + 8 * h + 4) = v.hi;
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  const f16* tr = stage + (4 * quad + (g >> 2)) * ROW + 4 * (g & 3);
#pragma unroll
  for (int j = 0; j < NS; ++j) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(tr + j * 16 * ROW + 16 * db));
      const f16x4 va = __builtin_bit_cast(f16x4, raw);
      // without DUAL: both parts of P in one 16x16x32 MFMA (as in the fp16
      // kernel: the lane's high parts then remainders against V twice)
      if (DUAL)
        st.o[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, ph[j], st.o[db], 0, 0, 0);
      else
        st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_shufflevector(va, va, 0, 1, 2, 3, 0, 1, 2, 3),
            __builtin_shufflevector(ph[j], pl[j], 0, 1, 2, 3, 4, 5, 6, 7), st.o[db], 0, 0, 0);
    }
  }
  asm volatile("" ::: "memory");
}

// Decode over the 8-bit cache.  MODE 0: one workgroup per (sequence, KV
// head), fp16 out.  MODE 1: one per partition, fp32 partials + lse (merged by
// split_reduce).  MODE 2: the fused decode step -- MODE 1 plus, in the same
// launch, the quantising cache write of each sequence's new token and the
// merge of each (sequence, KV head) by the holder of its last ticket, with
// the fp16 step's hand-off (device-coherent partial rows polled until
// written; merge_step_partitions).  MODE 3: MODE 2 with the two-level merge
// of launches with more than kFlatMerge partitions per pair; MODE 4: MODE 2
// with the direct merge of launches with at most kDirectMergeItems.
template <int D, int NS, int NW, int DEPTH, int MODE, bool DUAL>
__global__ __launch_bounds__(NW * 64) void attn_q8_kernel(const Q8Params P) {
  constexpr int KC = D / 32;
  constexpr int NDB = D / 16;
  constexpr int DC = D / 64;  // 16-code chunks per lane and row
  constexpr bool SPLIT = MODE >= 1;
  constexpr bool STEP = MODE >= 2;
  constexpr bool TWO = MODE == 3;
  constexpr bool DIRECT = MODE == 4;
  using SM = AttnSmem<D, NS>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[NW * SM::kWaveBytes];
  const AttnParams& a = P.a;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15;
  const int quad = lane >> 4;
  const int head_col = DUAL ? (g & 7) : g;
  const int Hkv = a.Hkv;
  const int kvh = blockIdx.x % Hkv;
  const int rest = blockIdx.x / Hkv;
  int b, p = 0;
  if (SPLIT) {
    p = rest % a.max_partitions;
    b = rest / a.max_partitions;
  } else {
    b = rest;
  }
  const int spb = a.block_size >> 4;
  const int spb_shift = a.spb_shift;
  const int32_t* bt_row = a.block_tables + (size_t)b * a.max_blocks;
  const __amdgpu_buffer_rsrc_t bt_rs = buffer_rsrc(bt_row, a.max_blocks * 4);
  constexpr int TSTEP = NW * NS;
  const int t_begin = SPLIT ? p * a.partition_size : 0;
  const int s_first = (t_begin >> 4) + wave * NS;
  const int sub_cap = a.max_blocks * spb;
  int ids[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    ids[i] = load_block_ids<NS>(bt_rs, s_first + i * TSTEP, sub_cap, spb, spb_shift, lane);

  const int cap = a.max_blocks * a.block_size;
  int ctx = a.context_lens[b];
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
  const int n_parts = STEP ? (ctx + a.partition_size - 1) / a.partition_size : 1;

  // Fused step: the workgroup owning position ctx-1 (partition 0 if ctx = 0)
  // quantises the new token's K/V rows of its head in registers, attends
  // over them in place of the cache's position ctx-1 when the slot is that
  // position's slot in the block table, and writes codes and scales at the
  // end (the launch never reads its own write).
  const bool owns_new =
      STEP && a.slot_mapping != nullptr && p == (ctx > 0 ? (ctx - 1) / a.partition_size : 0);
  // The slot is needed only at the tile holding position ctx-1 and at the
  // end, so it is requested after the length (the slot pointer comes in a
  // later batch of argument loads than the length pointer).
  const int64_t slot = owns_new ? a.slot_mapping[b] : -1;
  int s_new = -1, tok_new = -1, new_off = 0;
  u32x4 kq[DC], vq[DC];
  float ksc = 0.0f, vsc = 0.0f;
  if (owns_new) {
    if (ctx > 0) {
      const int pos = ctx - 1;
      new_off = pos % a.block_size;
      s_new = pos >> 4;
      tok_new = pos & 15;
    }
    const size_t new_row = ((size_t)b * Hkv + kvh) * D;
    quantize_row_lanes<D>(a.k_new + new_row, quad, kq, ksc);
    quantize_row_lanes<D>(a.v_new + new_row, quad, vq, vsc);
  } else {
#pragma unroll
    for (int cc = 0; cc < DC; ++cc) {
      kq[cc] = u32x4{0u, 0u, 0u, 0u};
      vq[cc] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // q as the B operand in the codes' dim order: MFMA m takes dims
  // 64*(m/2) + 16*quad + 8*(m%2) .. +7
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
      qb[m] = load_q16(q_rs, (head_col * D + 16 * quad + 64 * (m >> 1) + 8 * (m & 1)) * 2, sign);
  }
  float rem_mul = DUAL ? (g >= 8 ? -1.0f : 0.0f) : -1.0f;  // as in the fp16 kernel
  asm volatile("" : "+v"(rem_mul));
  SoftmaxState<D> st;
#pragma unroll
  for (int i = 0; i < NDB; ++i) st.o[i] = zero4f();
  st.lsum = zero4f();
  st.m = -INFINITY;
  float lsum = 0.0f;
  f16* stage = reinterpret_cast<f16*>(smem + wave * SM::kWaveBytes);

  // The fp16 kernel's pipeline: the loop runs while a tile remains to be
  // requested, then the tiles in flight are consumed with no more requests.
  const int n_tiles = s_first < sub_end ? (sub_end - s_first + TSTEP - 1) / TSTEP : 0;
  KVTile8<D, NS> buf[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) {
    // past the wave's last tile: empty resources, no memory access
    load_kv_tile8<D, NS>(buf[i], P, ids[i], s_first + i * TSTEP, sub_end, t_end, spb, spb_shift,
                         kvh, lane, s_new);
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
      consume_tile8<D, NS, DUAL, STEP>(buf[i], st, lsum, qb, stage, c, t_end, lane, rem_mul,
                                       s_new, tok_new, slot, new_off, a.block_size, kq, vq,
                                       ksc, vsc);
      load_kv_tile8<D, NS>(buf[i], P, ids[i], s_first + (u + DEPTH) * TSTEP, sub_end, t_end,
                           spb, spb_shift, kvh, lane, s_new);
      ids[i] = load_block_ids<NS>(bt_rs, s_first + (u + 2 * DEPTH) * TSTEP, sub_end, spb,
                                  spb_shift, lane);
    }
  }
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    if (u0 + i < n_tiles)
      consume_tile8<D, NS, DUAL, STEP>(buf[i], st, lsum, qb, stage, c, t_end, lane, rem_mul,
                                       s_new, tok_new, slot, new_off, a.block_size, kq, vq,
                                       ksc, vsc);

  if (DUAL) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v) st.o[db][v] += __shfl_xor(st.o[db][v], 8);
  }
  // the column's weight sum: this lane's tokens plus the other three quads'
  float l_tot = lsum + __shfl_xor(lsum, 16);
  l_tot += __shfl_xor(l_tot, 32);

  // Fused step: whether and what this workgroup merges (its ticket closes
  // its group, or the pair).
  __shared__ int s_merge;
  __shared__ __attribute__((aligned(16))) float own[STEP ? 16 * D + 16 : 4];
  if (STEP && n_parts > 1 && threadIdx.x == 0)
    s_merge = step_merge_role<TWO>(a, b, kvh, n_parts, p, ticket);
  if (NW == 1 && STEP) __syncthreads();

  // Fused step: the new token's codes and scale of this head, at (block,
  // head, offset) of the head-major layout.
  if (owns_new && slot >= 0 && slot < (int64_t)a.num_blocks * a.block_size && wave == 0 &&
      g == 0) {
    const int64_t blk = slot / a.block_size;
    const int off = (int)(slot - blk * a.block_size);
    const int64_t si = (blk * Hkv + kvh) * a.block_size + off;
#pragma unroll
    for (int cc = 0; cc < DC; ++cc) {
      *reinterpret_cast<u32x4*>(P.k_codes_w + si * D + 64 * cc + 16 * quad) = kq[cc];
      *reinterpret_cast<u32x4*>(P.v_codes_w + si * D + 64 * cc + 16 * quad) = vq[cc];
    }
    if (quad == 0) {
      P.k_scales_w[si] = ksc;
      P.v_scales_w[si] = vsc;
    }
  }

  const bool emits = (DUAL ? g < 8 : true) && head_col < a.G;
  auto emit = [&](int db, f32x4 acc, float L, float M) {
    if (!emits) return;
    const int h = kvh * a.G + head_col;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
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
        *reinterpret_cast<f32x4*>(a.partial_out +
                                  (((size_t)b * a.Hq + h) * a.max_partitions + p) * D + d0) = r;
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

}  // namespace pkv
