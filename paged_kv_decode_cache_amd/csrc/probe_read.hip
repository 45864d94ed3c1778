// Read-bandwidth probes for the benchmark: kernels that only read memory and
// write nothing (unless an XOR of everything they read hits one fixed
// pattern), so their time measures what a launch reading that many bytes can
// achieve.  Measurement aids, not part of the decode path.
//
//   pkv_probe_stream_read   a contiguous buffer, grid-stride, U 16-byte
//                           non-temporal loads in flight per lane: the plain
//                           streaming-read ceiling for a byte count.
//   pkv_probe_paged_read    the decode's own K/V access pattern with no
//                           arithmetic: a workgroup per (sequence, KV head,
//                           partition) of 4 waves, each wave reading its
//                           16-token subtiles round-robin through the block
//                           table, two subtiles in flight, whole 128-byte
//                           head rows per 8 lanes, non-temporal.
//   pkv_probe_paged_read_q8 the same over the 8-bit cache: per subtile one
//                           head's 16 rows of 64 codes (1 KiB, one 16-byte
//                           load per lane) of K and of V, and their 16 scales
//                           (a 16-byte load per lane quad), as the 8-bit
//                           decode kernels read them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          int64_t n16, u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0x85EBCA6Bu &&
      acc[3] == 0xC2B2AE35u)
    sink[0] = acc;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// head_dim 64, block_size 16: a subtile is one block's 16 rows of one head
// (128 bytes each, rows Hkv * 128 bytes apart); lane l reads row 8m + l/8,
// chunk l%8 of load m (m = 0, 1), as the decode kernels do.
constexpr int kWaves = 4;

__global__ __launch_bounds__(kWaves * 64) void paged_read_kernel(
    const unsigned char* __restrict__ kp, const unsigned char* __restrict__ vp,
    const int* __restrict__ bt, int max_blocks, int num_blocks, int Hkv, int ctx,
    int partition_size, u32x4* sink) {
  const int kvh = blockIdx.x, p = blockIdx.y, b = blockIdx.z;
  // The wave index must be known to be wave-uniform: taken straight from
  // threadIdx it is a vector value, the bounds check below becomes per-lane,
  // and each load of the second subtile turns into a readfirstlane loop over
  // its buffer resource (measured 13.4 against 12.0 us at 32 x 4096).
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = p * partition_size;
  const int t1 = min(ctx, t0 + partition_size);
  const int s_begin = t0 >> 4, s_end = (t1 + 15) >> 4;
  const int row_bytes = Hkv * 128;
  const int loff = (lane >> 3) * row_bytes + kvh * 128 + (lane & 7) * 16;
  const int* row = bt + (size_t)b * max_blocks;
  // the wave's block ids in one vector load (lane i: its i-th subtile), as
  // the decode kernels request them ahead of the K/V
  const int mine = s_begin + wave + kWaves * lane;
  const int ids = mine < s_end ? row[mine] : 0;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int i0 = 0; s_begin + wave + kWaves * i0 < s_end; i0 += 2) {
    u32x4 x[2][4];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int s = s_begin + wave + kWaves * (i0 + d);
      const int blk = __builtin_amdgcn_readlane(ids, (i0 + d) & 63);
      const bool ok = s < s_end && blk >= 0 && blk < num_blocks;
      const auto kr = rsrc(kp + (size_t)(ok ? blk : 0) * 16 * row_bytes, ok ? 16 * row_bytes : 0);
      const auto vr = rsrc(vp + (size_t)(ok ? blk : 0) * 16 * row_bytes, ok ? 16 * row_bytes : 0);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        x[d][m] = __builtin_amdgcn_raw_buffer_load_b128(kr, loff + m * 8 * row_bytes, 0, 2);
        x[d][2 + m] = __builtin_amdgcn_raw_buffer_load_b128(vr, loff + m * 8 * row_bytes, 0, 2);
      }
    }
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc ^= x[d][m];
  }
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0x85EBCA6Bu &&
      acc[3] == 0xC2B2AE35u)
    sink[0] = acc;
}

// 8-bit cache, head_dim 64, block size 16: codes [num_blocks, Hkv, 16, 64]
// int8, scales [num_blocks, Hkv, 16] fp32.  A subtile is one block of one
// head: 1 KiB of codes (lane l reads bytes 16l..16l+15) and 64 bytes of
// scales (lane quad q reads tokens 4q..4q+3), for K and for V.
__global__ __launch_bounds__(kWaves * 64) void paged_read_q8_kernel(
    const unsigned char* __restrict__ kc, const unsigned char* __restrict__ vc,
    const unsigned char* __restrict__ ks, const unsigned char* __restrict__ vs,
    const int* __restrict__ bt, int max_blocks, int num_blocks, int Hkv, int ctx,
    int partition_size, u32x4* sink) {
  const int kvh = blockIdx.x, p = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = p * partition_size;
  const int t1 = min(ctx, t0 + partition_size);
  const int s_begin = t0 >> 4, s_end = (t1 + 15) >> 4;
  const int* row = bt + (size_t)b * max_blocks;
  const int mine = s_begin + wave + kWaves * lane;
  const int ids = mine < s_end ? row[mine] : 0;
  const int coff = lane * 16, soff = (lane >> 4) * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int i0 = 0; s_begin + wave + kWaves * i0 < s_end; i0 += 2) {
    u32x4 x[2][4];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int s = s_begin + wave + kWaves * (i0 + d);
      const int blk = __builtin_amdgcn_readlane(ids, (i0 + d) & 63);
      const bool ok = s < s_end && blk >= 0 && blk < num_blocks;
      const size_t unit = (size_t)(ok ? blk : 0) * Hkv + kvh;  // (block, head)
      const auto kr = rsrc(kc + unit * 1024, ok ? 1024 : 0);
      const auto vr = rsrc(vc + unit * 1024, ok ? 1024 : 0);
      const auto ksr = rsrc(ks + unit * 64, ok ? 64 : 0);
      const auto vsr = rsrc(vs + unit * 64, ok ? 64 : 0);
      x[d][0] = __builtin_amdgcn_raw_buffer_load_b128(kr, coff, 0, 2);
      x[d][1] = __builtin_amdgcn_raw_buffer_load_b128(vr, coff, 0, 2);
      x[d][2] = __builtin_amdgcn_raw_buffer_load_b128(ksr, soff, 0, 2);
      x[d][3] = __builtin_amdgcn_raw_buffer_load_b128(vsr, soff, 0, 2);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc ^= x[d][m];
  }
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0x85EBCA6Bu &&
      acc[3] == 0xC2B2AE35u)
    sink[0] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) of src: grid workgroups of 256 lanes,
// loads_in_flight (4, 8 or 16) loads per lane.
extern "C" int pkv_probe_stream_read(const void* src, int64_t bytes, void* sink, int grid,
                                     int loads_in_flight, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || grid <= 0) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* k = static_cast<u32x4*>(sink);
  switch (loads_in_flight) {
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(256), 0, st, s, bytes / 16, k); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(256), 0, st, s, bytes / 16, k); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, dim3(grid), dim3(256), 0, st, s, bytes / 16, k); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// The K/V read of a split pass over B sequences of ctx positions each (fp16
// pools [num_blocks, 16, Hkv, 64], tables [B, max_blocks]), no arithmetic.
extern "C" int pkv_probe_paged_read(const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, int B, int Hkv, int ctx,
                                    int num_blocks, int max_blocks, int partition_size,
                                    void* sink, void* stream) {
  if (!k_pool || !v_pool || !block_tables || !sink || B <= 0 || B > 65535 || Hkv <= 0 ||
      ctx <= 0 || num_blocks <= 0 || max_blocks <= 0 || ctx > max_blocks * 16 ||
      partition_size <= 0 || partition_size % 16 != 0 || partition_size > 16 * 64 * kWaves ||
      (int64_t)16 * Hkv * 128 > INT32_MAX)
    return -1;
  const int parts = (ctx + partition_size - 1) / partition_size;
  if (parts > 65535) return -1;
  hipLaunchKernelGGL(paged_read_kernel, dim3(Hkv, parts, B), dim3(kWaves * 64), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const unsigned char*>(k_pool),
                     static_cast<const unsigned char*>(v_pool), block_tables, max_blocks,
                     num_blocks, Hkv, ctx, partition_size, static_cast<u32x4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// The code and scale reads of an 8-bit split pass over B sequences of ctx
// positions each (head_dim 64, block size 16: codes [num_blocks, Hkv, 16, 64]
// int8, scales [num_blocks, Hkv, 16] fp32; tables [B, max_blocks]), no
// arithmetic.
extern "C" int pkv_probe_paged_read_q8(const void* k_codes, const void* v_codes,
                                       const void* k_scales, const void* v_scales,
                                       const int32_t* block_tables, int B, int Hkv, int ctx,
                                       int num_blocks, int max_blocks, int partition_size,
                                       void* sink, void* stream) {
  if (!k_codes || !v_codes || !k_scales || !v_scales || !block_tables || !sink || B <= 0 ||
      B > 65535 || Hkv <= 0 || ctx <= 0 || num_blocks <= 0 || max_blocks <= 0 ||
      ctx > max_blocks * 16 || partition_size <= 0 || partition_size % 16 != 0 ||
      partition_size > 16 * 64 * kWaves || (int64_t)num_blocks * Hkv * 1024 > ((int64_t)1 << 40))
    return -1;
  const int parts = (ctx + partition_size - 1) / partition_size;
  if (parts > 65535) return -1;
  hipLaunchKernelGGL(paged_read_q8_kernel, dim3(Hkv, parts, B), dim3(kWaves * 64), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const unsigned char*>(k_codes),
                     static_cast<const unsigned char*>(v_codes),
                     static_cast<const unsigned char*>(k_scales),
                     static_cast<const unsigned char*>(v_scales), block_tables, max_blocks,
                     num_blocks, Hkv, ctx, partition_size, static_cast<u32x4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
