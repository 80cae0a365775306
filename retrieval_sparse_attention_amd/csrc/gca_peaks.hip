// Microbenchmarks for the peaks measured on the GPU at hand (include/gca_peaks.h):
// a streaming read, a streaming copy, a gather of 16 KB tiles into LDS and a
// loop of independent 16x16x32 bf16 MFMAs.  Grids are fixed: 2048 workgroups
// of 256 threads for the streaming kernels (eight per CU on 256 CUs), 4096 for
// the gather (four resident per CU, as the attention kernels), 1024 for the
// MFMA loop (four waves per SIMD).  They share no arithmetic with the GCA
// kernels.

#include "gca_device.h"
#include "gca_launch.h"

namespace gca {

constexpr int kPeakMemBlocks = 2048;
constexpr int kPeakMfmaBlocks = 1024;
constexpr int kPeakGatherBlocks = 4096;

// Each workgroup streams one contiguous range (whole DRAM pages, one open
// stream per workgroup); every thread keeps kPeakU 16-byte loads in flight and
// folds all four words of each into one 32-bit value, stored at the end.  The
// read uses nontemporal loads (data read once need not stay in the caches):
// 6.6-6.7 TB/s against 5.9-6.2 with plain loads on one box.
constexpr int kPeakU = 8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_peak_read(const uint4* __restrict__ src, int64_t n,
                                                   uint32_t* __restrict__ out) {
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n ? beg + per : n;
  uint32_t acc = 0;
  int64_t i = beg + threadIdx.x;
  for (; i + (kPeakU - 1) * 256 < end; i += kPeakU * 256) {
    uint4 v[kPeakU];
#pragma unroll
    for (int u = 0; u < kPeakU; ++u) {
      const u32x4 t = __builtin_nontemporal_load((const u32x4*)(src + i + u * 256));
      v[u] = make_uint4(t[0], t[1], t[2], t[3]);
    }
#pragma unroll
    for (int u = 0; u < kPeakU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += 256) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void k_peak_copy(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, int64_t n) {
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n ? beg + per : n;
  int64_t i = beg + threadIdx.x;
  for (; i + (kPeakU - 1) * 256 < end; i += kPeakU * 256) {
    uint4 v[kPeakU];
#pragma unroll
    for (int u = 0; u < kPeakU; ++u) v[u] = src[i + u * 256];
#pragma unroll
    for (int u = 0; u < kPeakU; ++u) dst[i + u * 256] = v[u];
  }
  for (; i < end; i += 256) dst[i] = src[i];
}

// Each workgroup moves `iters` tiles of 16 KB (the K and V tiles of one 64 x 64
// bf16 chunk), picked by a per-workgroup linear congruential sequence among the
// n_tiles of the buffer, into LDS with 16-byte global_load_lds: every wave
// copies 4 KB of the tile, waits, and the workgroup meets at a barrier before
// the next tile (one tile in flight, as the attention kernels' slot loop).  36 KB
// of LDS per workgroup: four resident per CU.  Each workgroup writes one word
// of its last tile, so no copy can be dropped.
__global__ __launch_bounds__(256) void k_peak_gather(const char* __restrict__ src, int64_t n_tiles,
                                                     int iters, uint32_t* __restrict__ out) {
  __shared__ __align__(16) uint32_t buf[2][4096];
  __shared__ uint32_t pad[1024];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint32_t h = (uint32_t)blockIdx.x * 2654435761u + 12345u;
  for (int it = 0; it < iters; ++it) {
    h = h * 1664525u + 1013904223u;
    const char* tile = src + (int64_t)((h >> 8) % (uint64_t)n_tiles) * 16384;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = wave * 4 + p;  // 1 KB pieces, 16 per tile
      __builtin_amdgcn_global_load_lds((const void*)(tile + piece * 1024 + lane * 16),
                                       (lds_void*)(&buf[it & 1][piece * 256]), 16, 0, 0);
    }
    wait_vmem();
    __syncthreads();
  }
  if (tid == 0) pad[0] = buf[(iters - 1) & 1][h & 4095];
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = pad[0];
}

// Eight accumulators per wave, each updated once per round: consecutive MFMAs
// never depend on each other, so the matrix pipe issues back to back.
__global__ __launch_bounds__(256) void k_peak_mfma(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(0.001f * (float)(lane + e));
    b[e] = (bf16)(0.002f * (float)(lane - e));
  }
  f32x4 acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = zero4();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] = mfma16x16x32(a, b, acc[r]);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r) s += (acc[r][0] + acc[r][1]) + (acc[r][2] + acc[r][3]);
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_peak_read(const void* src, size_t bytes, void* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_peak_read, dim3(kPeakMemBlocks), dim3(256), 0, stream, (const uint4*)src,
                     (int64_t)(bytes / 16), (uint32_t*)out);
  return hipGetLastError();
}

hipError_t launch_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  hipLaunchKernelGGL(k_peak_copy, dim3(kPeakMemBlocks), dim3(256), 0, stream, (const uint4*)src,
                     (uint4*)dst, (int64_t)(bytes / 16));
  return hipGetLastError();
}

hipError_t launch_peak_gather(const void* src, size_t bytes, void* out, int iters,
                              hipStream_t stream) {
  hipLaunchKernelGGL(k_peak_gather, dim3(kPeakGatherBlocks), dim3(256), 0, stream,
                     (const char*)src, (int64_t)(bytes / 16384), iters, (uint32_t*)out);
  return hipGetLastError();
}

hipError_t launch_peak_mfma(void* out, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(k_peak_mfma, dim3(kPeakMfmaBlocks), dim3(256), 0, stream, (float*)out,
                     iters);
  return hipGetLastError();
}

}  // namespace gca
