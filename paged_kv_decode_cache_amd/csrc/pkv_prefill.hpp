// Chunked-prefill attention over the paged cache on gfx950.
//
// A chunk of n new tokens of one sequence (Inference Engineering, Day 12 post
// on chunked prefill: a long prompt is processed a chunk per pass, and each
// pass writes the chunk's K/V into the cache) attends causally: the chunk's
// row i sits at position p = ctx - n + i and sees positions 0..p, which are
// the cached prefix and the chunk's own earlier rows, all already in the pool.
//
// The decode kernel's structure carries over with a wider B operand.  A
// workgroup owns (sequence, KV head, query tile).  Its MFMA columns are
// (query row, head of the group) pairs, 16 per column tile, NCT tiles, so one
// read of each K/V row serves QT = 16*NCT/G query rows times the G heads.
// Each column has its own causal limit.  The waves split the context's
// 16-token subtiles round-robin, keep DEPTH of them in flight, and merge
// through LDS at the end, one column tile at a time.
#pragma once

#include "pkv_kernels.hpp"

namespace pkv {

struct PrefillParams {
  AttnParams a;                // q and out are [total_q, Hq, D]
  const int32_t* query_start;  // [B + 1]: sequence b's rows are query_start[b] .. [b+1]-1
  int32_t max_q;               // bound on every chunk length
  int32_t q_tiles;             // ceil(max_q / QT)
  int32_t* row_ctx;            // split pass: [total_q], each row's context_lens[b]
};

// Query rows per workgroup for a group of G heads over NCT column tiles.
__host__ __device__ constexpr int prefill_rows_per_tile(int nct, int G) { return 16 * nct / G; }

// SPLIT: the context is cut into partitions of a.partition_size positions,
// one workgroup per (sequence, KV head, query tile, partition); each writes
// fp32 partials and lse per (row, head) into a.partial_out / a.partial_lse
// ([total_q, Hq, max_partitions, ...]), merged by split_reduce over rows with
// pp.row_ctx as their lengths.  A row that sees none of a partition's
// positions gets lse = -inf and a zero row there.
template <int D, int NCT, int NW, int DEPTH, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(const PrefillParams pp) {
  constexpr int NS = 1;
  constexpr int KC = D / 32;
  constexpr int NDB = D / 16;
  constexpr int ROW = D + 4;
  using SM = AttnSmem<D, NS>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[NW * SM::kWaveBytes];
  const AttnParams& a = pp.a;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane & 15;
  const int quad = lane >> 4;
  const int Hkv = a.Hkv;
  const int G = a.G;
  const int QT = prefill_rows_per_tile(NCT, G);
  const int kvh = blockIdx.x % Hkv;
  int rest = blockIdx.x / Hkv;
  int p = 0;
  if (SPLIT) {
    p = rest % a.max_partitions;
    rest /= a.max_partitions;
  }
  const int qt = rest % pp.q_tiles;
  const int b = rest / pp.q_tiles;
  const int t_lo = SPLIT ? p * a.partition_size : 0;  // first position of the partition

  const int spb = a.block_size >> 4;
  const int spb_shift = a.spb_shift;
  const int64_t tok_stride = (int64_t)Hkv * D;
  const int lane_off_b = ((lane & 15) * Hkv * D + 8 * quad) * 2;
  const int32_t* bt_row = a.block_tables + (size_t)b * a.max_blocks;
  const __amdgpu_buffer_rsrc_t bt_rs = buffer_rsrc(bt_row, a.max_blocks * 4);
  constexpr int TSTEP = NW;
  const int s_first = (t_lo >> 4) + wave;
  const int sub_cap = a.max_blocks * spb;
  // first block ids together with the lengths (every table entry is readable)
  int ids[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i)
    ids[i] = load_block_ids<NS>(bt_rs, s_first + i * TSTEP, sub_cap, spb, spb_shift, lane);

  const int r0 = pp.query_start[b];
  int n = pp.query_start[b + 1] - r0;
  n = n < 0 ? 0 : (n > pp.max_q ? pp.max_q : n);
  const int q0 = qt * QT;
  if (q0 >= n) return;
  const int nq = min(QT, n - q0);
  const int cap = a.max_blocks * a.block_size;
  int ctx = a.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  const int pos_first = ctx - n + q0;          // position of the tile's first row
  const int t_end = max(0, pos_first + nq);    // positions any row of the tile sees
  // the partition's positions end at a subtile boundary (partition_size is a
  // multiple of the block size) or at t_end, so the masks below need no change
  const int sub_end = ((SPLIT ? min(t_end, t_lo + a.partition_size) : t_end) + 15) >> 4;
  if (SPLIT && p == 0 && kvh == 0 && (int)threadIdx.x < nq)
    pp.row_ctx[r0 + q0 + threadIdx.x] = ctx;

  // Columns: c = 16 t + g is (row q0 + c / G, head c % G); its causal limit
  // qpos[t] (-1: the column is padding or its row precedes position 0).
  const bool neg_scale = a.scale_log2 < 0.0f;
  const float c_scale = fmaxf(neg_scale ? -a.scale_log2 : a.scale_log2, 1.17549435e-38f);
  f16x8 qb[NCT][KC];
  int qpos[NCT];
  // the tile's nq rows of the group's G heads (row stride Hq * D); padding
  // columns read past the resource (zeros)
  const __amdgpu_buffer_rsrc_t q_rs =
      buffer_rsrc(a.q + ((size_t)(r0 + q0) * a.Hq + kvh * G) * D, ((nq - 1) * a.Hq + G) * D * 2);
  const unsigned sign = neg_scale ? 0x80008000u : 0u;
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
    const int col = 16 * t + g;
    const int i = col / G;
    const bool valid = col < QT * G && i < nq;
    qpos[t] = valid ? pos_first + i : -1;
    const int qoff = valid ? ((i * a.Hq + col % G) * D + 8 * quad) * 2 : kOutOfRange;
#pragma unroll
    for (int m = 0; m < KC; ++m) qb[t][m] = load_q16(q_rs, qoff + 64 * m, sign);
  }
  // positions every valid column sees: [0, pos_first]
  const int vis_all = pos_first;
  // the remainder P - fp16(P) as one mixed-precision FMA: the multiplier -1
  // is opaque to the compiler, which otherwise emits convert, subtract, convert
  float neg1 = -1.0f;
  asm volatile("" : "+v"(neg1));
  f16x4 ones;
#pragma unroll
  for (int i = 0; i < 4; ++i) ones[i] = (f16)(g == 0 ? 1.0f : 0.0f);

  SoftmaxState<D> st[NCT];
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
#pragma unroll
    for (int i = 0; i < NDB; ++i) st[t].o[i] = zero4f();
    st[t].lsum = zero4f();
    st[t].m = -INFINITY;
  }
  f16* stage = reinterpret_cast<f16*>(smem + wave * SM::kWaveBytes);

  const int n_tiles = s_first < sub_end ? (sub_end - s_first + TSTEP - 1) / TSTEP : 0;
  KVTile<D, NS> buf[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) {
    // past the wave's last tile: empty resources, no memory access
    load_kv_tile<D, NS>(buf[i], a, ids[i], s_first + i * TSTEP, sub_end, t_end, spb, spb_shift,
                        tok_stride, kvh, lane_off_b);
    ids[i] = load_block_ids<NS>(bt_rs, s_first + (i + DEPTH) * TSTEP, sub_end, spb, spb_shift,
                                lane);
  }
  for (int u0 = 0; u0 < n_tiles; u0 += DEPTH) {
#pragma unroll
    for (int di = 0; di < DEPTH; ++di) {
      const int u = u0 + di;
      if (u < n_tiles) {
        KVTile<D, NS>& T = buf[di];
        const int tok0 = T.s0 << 4;
        // logits S^T[token][column] per column tile
        f32x4 sc[NCT];
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
          f32x4 acc = zero4f();
#pragma unroll
          for (int m = 0; m < KC; ++m)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(T.k[0][m], qb[t][m], acc, 0, 0, 0);
          sc[t] = acc;
        }
        // tokens past some column's limit, or of an unread block, drop out
        if (!(T.full && tok0 + 15 <= vis_all)) {
#pragma unroll
          for (int t = 0; t < NCT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int tok = tok0 + 4 * quad + v;
              sc[t][v] = ((T.okmask & 1) && tok <= qpos[t]) ? sc[t][v] : -INFINITY;
            }
        }
        f16x4 ph[NCT], pl[NCT];
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
          float tmax = fmaxf(fmaxf(sc[t][0], sc[t][1]), fmaxf(sc[t][2], sc[t][3]));
          tmax = max_across_quads(tmax);
          const float tmax_s = tmax * c_scale;
          const bool grow = tmax_s > st[t].m + kRescaleLog2;
          if (__any(grow)) {
            // only growing columns rescale: a column still at -inf (every token
            // so far past its causal limit) must not form -inf - -inf
            const float m_new = grow ? tmax_s : st[t].m;
            const float alpha = grow ? fast_exp2(st[t].m - m_new) : 1.0f;
            st[t].m = m_new;
            st[t].lsum *= alpha;
#pragma unroll
            for (int i = 0; i < NDB; ++i) st[t].o[i] *= alpha;
          }
          const float neg_m = (st[t].m == -INFINITY) ? 0.0f : -st[t].m;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p = fast_exp2(fmaf(sc[t][v], c_scale, neg_m));
            const f16 h = (f16)p;
            ph[t][v] = h;
            pl[t][v] = (f16)fmaf((float)h, neg1, p);
          }
        }
        // V subtile -> LDS row-major (rows no column sees as zeros), then the
        // transposed A operand once for all column tiles
        {
          f16* row = stage + (lane & 15) * ROW + 8 * quad;
          const int tok = tok0 + (lane & 15);
          const bool keep = (T.okmask & 1) && tok < t_end;
#pragma unroll
          for (int m = 0; m < KC; ++m) {
            const f16x8 v = keep ? T.v[0][m] : zero8();
            *reinterpret_cast<f16x4*>(row + 32 * m) = v.lo;
            *reinterpret_cast<f16x4*>(row + 32 * m + 4) = v.hi;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        f16x4 va[NDB];
        {
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          const f16* tr = stage + (4 * quad + (g >> 2)) * ROW + 4 * (g & 3);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            va[db] = __builtin_bit_cast(
                f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (__attribute__((address_space(3))) s16x4*)(tr + 16 * db)));
        }
        // P.V with both parts of P in one 16x16x32 MFMA: in the k = 32 layout
        // this lane holds k = 8 quad .. 8 quad + 7, taken here as its own 4
        // tokens' high parts then their remainders (B operand), against the
        // same 4 tokens' V values twice (A operand).  The product is
        // V.P_high + V.P_remainder at half the MFMA issue of two 16x16x16.
        const f16x8 ones8 = __builtin_shufflevector(ones, ones, 0, 1, 2, 3, 4, 5, 6, 7);
        f16x8 va8[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          va8[db] = __builtin_shufflevector(va[db], va[db], 0, 1, 2, 3, 0, 1, 2, 3);
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
          const f16x8 pb = __builtin_shufflevector(ph[t], pl[t], 0, 1, 2, 3, 4, 5, 6, 7);
          st[t].lsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, pb, st[t].lsum, 0, 0, 0);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            st[t].o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va8[db], pb, st[t].o[db], 0, 0, 0);
        }
        asm volatile("" ::: "memory");  // the next subtile's LDS writes stay after these reads
      }
      load_kv_tile<D, NS>(buf[di], a, ids[di], s_first + (u + DEPTH) * TSTEP, sub_end, t_end, spb,
                          spb_shift, tok_stride, kvh, lane_off_b);
      ids[di] = load_block_ids<NS>(bt_rs, s_first + (u + 2 * DEPTH) * TSTEP, sub_end, spb,
                                   spb_shift, lane);
    }
  }

  // Merge the waves and write each valid column, one column tile at a time.
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
    const float l_tot = __shfl(st[t].lsum[0], g);
    const int col = 16 * t + g;
    const bool emits = qpos[t] >= 0 || (col < QT * G && col / G < nq);
    const int i = col / G;
    auto emit = [&](int db, f32x4 acc, float L, float M) {
      if (!emits) return;
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const size_t rh = (size_t)(r0 + q0 + i) * a.Hq + kvh * G + col % G;  // (row, head)
      if (SPLIT) {
        f32x4 r;
#pragma unroll
        for (int v = 0; v < 4; ++v) r[v] = acc[v] * inv;
        *reinterpret_cast<f32x4*>(a.partial_out + (rh * a.max_partitions + p) * D + 16 * db +
                                  4 * quad) = r;
        if (db == 0 && quad == 0)
          a.partial_lse[rh * a.max_partitions + p] =
              L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
      } else {
        f16x4 r;
#pragma unroll
        for (int v = 0; v < 4; ++v) r[v] = (f16)(acc[v] * inv);
        *reinterpret_cast<f16x4*>(a.out + rh * D + 16 * db + 4 * quad) = r;
      }
    };
    if (NW == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) emit(db, st[t].o[db], l_tot, st[t].m);
    } else {
      merge_waves_impl<D, NW>(st[t], l_tot, smem, SM::kWaveBytes, wave, lane, emit);
    }
  }
}

}  // namespace pkv
