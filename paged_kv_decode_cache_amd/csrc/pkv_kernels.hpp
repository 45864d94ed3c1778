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
//   sizes are multiples of 16); wave w takes tiles of NS subtiles round-robin.
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
//     zero weight), read back one 16-bit element per lane and k-slot.
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
constexpr float kLn2 = 0.69314718055994530942f;

struct AttnParams {
  const f16* q;
  const f16* k_pool;
  const f16* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  f16* out;             // unsplit: [B, Hq, D]
  float* partial_out;   // split:   [B, Hq, P_max, D]
  float* partial_lse;   // split:   [B, Hq, P_max]
  int32_t Hq, Hkv, G;
  int32_t block_size, num_blocks, max_blocks;
  int32_t partition_size, max_partitions;
  float scale_log2;     // softmax scale * log2(e)
};

struct ReduceParams {
  f16* out;
  float* lse_out;
  const float* partial_out;
  const float* partial_lse;
  const int32_t* context_lens;
  int32_t Hq, partition_size, max_partitions;
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

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
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

template <int D, int NS, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const AttnParams a) {
  constexpr int KC = D / 32;   // QK MFMAs (16x16x32) per subtile
  constexpr int NDB = D / 16;  // PV MFMA column blocks (16 dims each)
  using SM = AttnSmem<D, NS>;
  constexpr int ROW = SM::kRow;
  __shared__ __attribute__((aligned(16))) unsigned char smem[NW * SM::kWaveBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane & 15;     // MFMA column: query head within the group
  const int quad = lane >> 4;  // 0..3

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

  const int cap = a.max_blocks * a.block_size;
  int ctx = a.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  int t_begin = 0, t_end = ctx;
  if (SPLIT) {
    t_begin = p * a.partition_size;
    if (t_begin >= ctx) {
      if (threadIdx.x < a.G)
        a.partial_lse[((size_t)b * a.Hq + kvh * a.G + threadIdx.x) * a.max_partitions + p] =
            -INFINITY;
      return;
    }
    t_end = min(ctx, t_begin + a.partition_size);
  }

  // Query group as the B operand: lane l holds q[head l%16][8*(l/16) + 32m ..].
  f16x8 qb[KC];
  {
    const bool hv = g < a.G;
    const f16* qrow = a.q + ((size_t)b * a.Hq + kvh * a.G + (hv ? g : 0)) * D + 8 * quad;
#pragma unroll
    for (int m = 0; m < KC; ++m) {
      const f16x8 v = *reinterpret_cast<const f16x8*>(qrow + 32 * m);
      qb[m] = hv ? v : zero8();
    }
  }

  const int sub_begin = t_begin >> 4;
  const int sub_end = (t_end + 15) >> 4;
  const int spb = a.block_size >> 4;  // subtiles per block
  const int64_t tok_stride = (int64_t)Hkv * D;
  const int lane_off = (lane & 15) * Hkv * D + 8 * quad;
  const int32_t* bt_row = a.block_tables + (size_t)b * a.max_blocks;

  f32x4 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = zero4f();
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f16* stage = reinterpret_cast<f16*>(smem + wave * SM::kWaveBytes);

  for (int s0 = sub_begin + wave * NS; s0 < sub_end; s0 += NW * NS) {
    bool ok[NS];
    int64_t base[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int s = s0 + j;
      const int blk = s / spb;
      bool v = s < sub_end;
      const int phys = v ? bt_row[blk] : 0;
      v = v && phys >= 0 && phys < a.num_blocks;
      ok[j] = v;
      base[j] = ((int64_t)(v ? phys : 0) * a.block_size + (s - blk * spb) * 16) * tok_stride +
                (int64_t)kvh * D;
    }

    f16x8 kr[NS][KC], vr[NS][KC];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (ok[j]) {
        const f16* kp = a.k_pool + base[j] + lane_off;
        const f16* vp = a.v_pool + base[j] + lane_off;
#pragma unroll
        for (int m = 0; m < KC; ++m) {
          kr[j][m] = *reinterpret_cast<const f16x8*>(kp + 32 * m);
          vr[j][m] = *reinterpret_cast<const f16x8*>(vp + 32 * m);
        }
      } else {
#pragma unroll
        for (int m = 0; m < KC; ++m) {
          kr[j][m] = zero8();
          vr[j][m] = zero8();
        }
      }
    }

    // S^T[token][head] for each subtile.
    f32x4 sc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      f32x4 acc = zero4f();
#pragma unroll
      for (int m = 0; m < KC; ++m)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr[j][m], qb[m], acc, 0, 0, 0);
      sc[j] = acc;
    }

    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = ((s0 + j) << 4) + 4 * quad + v;
        float x = sc[j][v] * a.scale_log2;
        x = (ok[j] && tok < t_end) ? x : -INFINITY;
        sc[j][v] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] *= alpha;

    f16x4 ph[NS], pl[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float pv = fast_exp2(sc[j][v] - m_use);
        l_run += pv;
        const f16 hi = (f16)pv;
        ph[j][v] = hi;
        pl[j][v] = (f16)(pv - (float)hi);
      }
    }

    // V subtiles -> LDS, row-major [token][dim], masked rows as zeros.
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int tok = ((s0 + j) << 4) + (lane & 15);
      const bool keep = ok[j] && tok < t_end;
      f16* row = stage + (j * 16 + (lane & 15)) * ROW + 8 * quad;
#pragma unroll
      for (int m = 0; m < KC; ++m) {
        const f16x8 v = keep ? vr[j][m] : zero8();
        *reinterpret_cast<f16x4*>(row + 32 * m) = v.lo;
        *reinterpret_cast<f16x4*>(row + 32 * m + 4) = v.hi;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const f16* col = stage + (j * 16 + 4 * quad) * ROW + g;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f16x4 va;
        va[0] = col[16 * db];
        va[1] = col[16 * db + ROW];
        va[2] = col[16 * db + 2 * ROW];
        va[3] = col[16 * db + 3 * ROW];
        o[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, ph[j], o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pl[j], o[db], 0, 0, 0);
      }
    }
    asm volatile("" ::: "memory");
  }

  // Sum of the wave's weights per head: lanes of one head differ in quad.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);

  // Final value for column block db of this lane's head: o_sum / l_sum with
  // the running maximum m_max (log2 domain).
  auto emit = [&](int db, f32x4 acc, float L, float M) {
    if (g >= a.G) return;
    const int h = kvh * a.G + g;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int d0 = 16 * db + 4 * quad;
    if (SPLIT) {
      f32x4 r;
#pragma unroll
      for (int v = 0; v < 4; ++v) r[v] = acc[v] * inv;
      float* dst = a.partial_out + (((size_t)b * a.Hq + h) * a.max_partitions + p) * D + d0;
      *reinterpret_cast<f32x4*>(dst) = r;
      if (db == 0 && quad == 0)
        a.partial_lse[((size_t)b * a.Hq + h) * a.max_partitions + p] =
            L > 0.0f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    } else {
      f16x4 r;
#pragma unroll
      for (int v = 0; v < 4; ++v) r[v] = (f16)(acc[v] * inv);
      *reinterpret_cast<f16x4*>(a.out + ((size_t)b * a.Hq + h) * D + d0) = r;
    }
  };

  if (NW == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) emit(db, o[db], l_tot, m_run);
    return;
  }

  __syncthreads();  // every wave is done with its staging area
  float* mine = reinterpret_cast<float*>(smem + wave * SM::kWaveBytes);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int v = 0; v < 4; ++v) mine[(db * 4 + v) * 64 + lane] = o[db][v];
  if (quad == 0) {
    mine[NDB * 4 * 64 + g] = m_run;
    mine[NDB * 4 * 64 + 16 + g] = l_tot;
  }
  __syncthreads();

  for (int db = wave; db < NDB; db += NW) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* theirs = reinterpret_cast<const float*>(smem + w * SM::kWaveBytes);
      M = fmaxf(M, theirs[NDB * 4 * 64 + g]);
    }
    const float mu = (M == -INFINITY) ? 0.0f : M;
    float L = 0.0f;
    f32x4 acc = zero4f();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* theirs = reinterpret_cast<const float*>(smem + w * SM::kWaveBytes);
      const float e = fast_exp2(theirs[NDB * 4 * 64 + g] - mu);
      L += e * theirs[NDB * 4 * 64 + 16 + g];
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += e * theirs[(db * 4 + v) * 64 + lane];
    }
    emit(db, acc, L, M);
  }
}

// LSE-weighted merge of the valid partitions of one (sequence, query head);
// one wave per pair, lane = dim (D = 64) or dim pair (D = 128).
template <int D>
__global__ __launch_bounds__(64) void split_reduce_kernel(const ReduceParams a) {
  constexpr int PER = D / 64;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int lane = threadIdx.x;
  const int cap = a.max_partitions * a.partition_size;
  int ctx = a.context_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  const int np = (ctx + a.partition_size - 1) / a.partition_size;
  const float* lse = a.partial_lse + (size_t)bh * a.max_partitions;
  const float* po = a.partial_out + (size_t)bh * a.max_partitions * D;

  float M = -INFINITY;
  for (int i = lane; i < np; i += 64) M = fmaxf(M, lse[i]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, __shfl_xor(M, sh));

  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
  float L = 0.0f;
  if (M != -INFINITY) {
    const float M2 = M * kLog2e;
    for (int i = 0; i < np; ++i) {
      const float e = fast_exp2(fmaf(lse[i], kLog2e, -M2));
      L += e;
      const float* row = po + (size_t)i * D + PER * lane;
      if (PER == 1) {
        acc[0] = fmaf(e, row[0], acc[0]);
      } else {
        const float2 x = *reinterpret_cast<const float2*>(row);
        acc[0] = fmaf(e, x.x, acc[0]);
        acc[1] = fmaf(e, x.y, acc[1]);
      }
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  f16* dst = a.out + (size_t)bh * D + PER * lane;
#pragma unroll
  for (int k = 0; k < PER; ++k) dst[k] = (f16)(acc[k] * inv);
  if (a.lse_out != nullptr && lane == 0)
    a.lse_out[bh] = L > 0.0f ? M + logf(L) : -INFINITY;
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
  const int64_t slot = a.slot_mapping[n];
  if (slot < 0 || slot >= a.num_slots) return;
  const int64_t dst = (slot * a.Hkv + h) * a.D + 8 * c;
  const int64_t src = (n * a.Hkv + h) * a.D + 8 * c;
  *reinterpret_cast<uint4*>(a.k_pool + dst) = *reinterpret_cast<const uint4*>(a.k_new + src);
  *reinterpret_cast<uint4*>(a.v_pool + dst) = *reinterpret_cast<const uint4*>(a.v_new + src);
}

}  // namespace pkv
