// Packed gather of the retrieved K/V tiles, for K/V offloaded to host memory.
//
// Definition (paperlayer.ai summary, section 3.2: past chunk representations
// can live in CPU memory, and the transfers retrieval causes happen only when
// it runs; paperhub.cn review page, authors' reply "Q2": the offloaded GCA K/V
// is shared within a group and moves over a host link of more than 20 GB/s).
// Only the k retrieved tiles of each query chunk travel: slot (t, i) of a head
// becomes packed row t*k + i, so attention over the packed rows with packed
// indices t*k + i gives the same result as over the resident arrays.
//
// One workgroup of 256 threads per (head, query chunk, slot).  Each thread
// issues all of its loads (K and V) before its first store, so every read of
// the workgroup is in flight at once: over the host link a read takes
// microseconds, and thousands of independent tiles keep the link busy.  The
// source may be device memory or host memory mapped into the device's address
// space; loads are plain vector loads either way.

#include "gca_device.h"
#include "gca_launch.h"

namespace gca {

template <typename Word, int PER>
__global__ __launch_bounds__(256) void k_gather_kv(const char* __restrict__ k_src,
                                                   const char* __restrict__ v_src,
                                                   const int32_t* __restrict__ idx,
                                                   char* __restrict__ k_out,
                                                   char* __restrict__ v_out,
                                                   int32_t* __restrict__ idx_out,
                                                   int64_t n_query, int64_t n_key, int topk,
                                                   int64_t tile_bytes) {
  const int64_t slot = blockIdx.x;  // (head * n_query + t) * topk + i
  const int64_t per_head = n_query * topk;
  const int64_t head = slot / per_head;
  const int64_t row = slot % per_head;  // packed row t * topk + i
  const int c = idx[slot];
  const bool ok = c >= 0 && c < n_key;
  if (threadIdx.x == 0) idx_out[slot] = ok ? (int32_t)row : -1;
  const int64_t n_words = tile_bytes / (int64_t)sizeof(Word);
  const Word* ks = (const Word*)(k_src + (head * n_key + (ok ? c : 0)) * tile_bytes);
  const Word* vs = (const Word*)(v_src + (head * n_key + (ok ? c : 0)) * tile_bytes);
  Word* kd = (Word*)(k_out + slot * tile_bytes);
  Word* vd = (Word*)(v_out + slot * tile_bytes);
  for (int64_t w0 = 0; w0 < n_words; w0 += 256 * PER) {
    Word a[PER], b[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int64_t w = w0 + threadIdx.x + 256 * p;
      a[p] = Word{};
      b[p] = Word{};
      if (ok && w < n_words) {
        a[p] = ks[w];
        b[p] = vs[w];
      }
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int64_t w = w0 + threadIdx.x + 256 * p;
      if (w < n_words) {
        kd[w] = a[p];
        vd[w] = b[p];
      }
    }
  }
}

hipError_t launch_gather_kv(const LaunchGather& a) {
  const int64_t slots = a.heads * a.n_query * a.k;
  if (slots == 0) return hipSuccess;
  const bool wide = a.tile_bytes % 16 == 0 && ((uintptr_t)a.k_src | (uintptr_t)a.v_src |
                                               (uintptr_t)a.k_out | (uintptr_t)a.v_out) %
                                                      16 == 0;
  KernelTimer timer(kKernGather, a.stream);
  if (wide)
    hipLaunchKernelGGL((k_gather_kv<uint4, 2>), dim3((unsigned)slots), dim3(256), 0, a.stream,
                       (const char*)a.k_src, (const char*)a.v_src, a.idx, (char*)a.k_out,
                       (char*)a.v_out, a.idx_out, a.n_query, a.n_key, a.k, a.tile_bytes);
  else
    hipLaunchKernelGGL((k_gather_kv<uint16_t, 4>), dim3((unsigned)slots), dim3(256), 0,
                       a.stream, (const char*)a.k_src, (const char*)a.v_src, a.idx,
                       (char*)a.k_out, (char*)a.v_out, a.idx_out, a.n_query, a.n_key, a.k,
                       a.tile_bytes);
  return hipGetLastError();
}

}  // namespace gca
