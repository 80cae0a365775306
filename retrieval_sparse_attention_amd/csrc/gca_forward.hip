// GCA forward: Eq. 2 per-chunk attention and Eq. 3 weighted fusion.
//
// Definition (long-context-modeling README, "Model Architecture"; paperlayer.ai
// summary, section 3.1 and appendix B): every token x of query chunk t attends
// separately to the S tokens of each retrieved chunk c_i, giving O^i[x] and the
// log-sum-exp L_i[x]; the output is O[x] = sum_i w_i O^i[x].
//
// bf16 path (S = 64, D = 64 or 32).  One workgroup of four waves per query
// chunk; wave w owns query rows 16w .. 16w+15 and works on 16x16x32 MFMA
// tiles (D/32 contraction steps for the scores, D/16 column tiles of O).  Per
// retrieved chunk:
//   1. the K and V tiles (2D bytes per row) of the next retrieved chunk stream from
//      global memory straight into the other half of a double-buffered,
//      XOR-swizzled LDS area (global_load_lds, scalar tile base plus per-lane
//      offsets computed once) while the current chunk is computed; one barrier
//      per chunk, and the chunk loop is unrolled by two so that both buffers
//      are fixed LDS addresses;
//   2. S^T = K Q^T on MFMA (A = K rows from LDS, B = Q^T kept in registers), so a
//      lane holds 16 of the 64 logits of ONE query row and the lanes l ^ 16,
//      l ^ 32, l ^ 48 the others: the row max and row sum need two exchanges;
//   3. p = exp2((s - max) * attn_scale * log2 e), rounded to bf16 once;
//   4. V^T P^T (V^T from LDS through the gfx950 transpose read) and the row
//      sums l = 1^T P^T are both MFMA products of the same bf16 p, so the
//      softmax's sum costs no vector adds; L = attn_scale * max + ln l;
//   5. O^T += (w_i / l) V^T P^T: all k slots accumulate into ONE float32
//      accumulator.  Each chunk's softmax is complete inside one 64-key tile:
//      no running rescale is needed.
// O is rounded to bf16 once at the end.  The workgroup's only LDS is the two
// K/V tile buffers (32 KB at D = 64): every wave forms the slot table itself
// from one ballot (lane i holds slot i's chunk and weight, read back with
// readlane), the L rows stay in registers until the loop ends, and the V^T
// operands are read right before their products.  At 92 registers five
// workgroups then share a CU (20 waves against 16): on the 16K-token
// two-group step the forward went from 352-354 to 341 us.
//
// Generic path (other sizes, float32 or bf16 elements).  One thread per query
// row, float32 arithmetic, one rounding of the output (small workloads).

#include "gca_device.h"
#include "gca_fwd64.h"
#include "gca_launch.h"

namespace gca {

template <int D>
__global__ __launch_bounds__(256, 5) void k_fwd_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, bf16* __restrict__ o,
    float* __restrict__ lse, int64_t n_query, int64_t n_key, int topk, float attn_scale) {
  __shared__ __align__(16) bf16 k_lds[2][64 * D];
  __shared__ __align__(16) bf16 v_lds[2][64 * D];
  const int lane = threadIdx.x & 63;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);  // = head * n_query + t
  // every wave reads the slot table itself: lane i holds slot i
  const int i0 = lane < topk ? lane : 0;
  const int c_in = idx[tile * topk + i0];
  const float w_in = w[tile * topk + i0];
  const bool ok = lane < topk && c_in >= 0 && c_in < n_key;
  fwd_tile<D>(q, kk, v, o, lse, tile, n_query, n_key, topk, attn_scale, c_in, w_in, ok, k_lds,
              v_lds);
}

// Generic path (any S, D <= 64; float32 or bf16 elements): 64 threads per
// query chunk, thread x owns query row x (< S); float32 arithmetic, with the
// output row accumulated in registers and rounded to the element type once.
template <typename T>
__global__ __launch_bounds__(64) void k_fwd_gen(
    const T* __restrict__ q, const T* __restrict__ kk, const T* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, T* __restrict__ o,
    float* __restrict__ lse, int64_t n_query, int64_t n_key, int S, int D, int topk,
    float attn_scale) {
  __shared__ float kt[64 * 64];
  __shared__ float vt[64 * 64];
  __shared__ float pr[64 * 65];
  const int x = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int64_t head = tile / n_query;
  const int64_t tsz = (int64_t)S * D;
  const T* qrow = q + tile * tsz + (int64_t)x * D;
  float oa[64];
#pragma unroll
  for (int d = 0; d < 64; ++d) oa[d] = 0.0f;
  for (int i = 0; i < topk; ++i) {
    const int c = idx[tile * topk + i];
    const float wi = w[tile * topk + i];
    float* lse_row = lse ? lse + (tile * topk + i) * S : nullptr;
    if (c < 0 || c >= n_key) {
      if (lse_row && x < S) lse_row[x] = -__builtin_huge_valf();
      continue;
    }
    __syncthreads();
    const T* ks = kk + (head * n_key + c) * tsz;
    const T* vs = v + (head * n_key + c) * tsz;
    for (int e = x; e < S * D; e += 64) {
      kt[e] = load_f(ks + e);
      vt[e] = load_f(vs + e);
    }
    __syncthreads();
    if (x < S) {
      float* p = pr + x * 65;
      float m = -__builtin_huge_valf();
      for (int j = 0; j < S; ++j) {
        float acc = 0.0f;
        for (int d = 0; d < D; ++d) acc = fmaf(load_f(qrow + d), kt[j * D + d], acc);
        p[j] = acc * attn_scale;
        m = fmaxf(m, p[j]);
      }
      float l = 0.0f;
      for (int j = 0; j < S; ++j) {
        p[j] = expf(p[j] - m);
        l += p[j];
      }
      if (lse_row) lse_row[x] = m + logf(l);
      const float sc = wi / l;
#pragma unroll
      for (int d = 0; d < 64; ++d) {
        if (d < D) {
          float acc = 0.0f;
          for (int j = 0; j < S; ++j) acc = fmaf(p[j], vt[j * D + d], acc);
          oa[d] = fmaf(sc, acc, oa[d]);
        }
      }
    }
  }
  if (x < S) {
    T* orow = o + tile * tsz + (int64_t)x * D;
#pragma unroll
    for (int d = 0; d < 64; ++d)
      if (d < D) store_f(orow + d, oa[d]);
  }
}

hipError_t launch_forward(const LaunchForward& a) {
  const int64_t tiles = a.G * a.B * a.H * a.n_query;
  if (tiles == 0) return hipSuccess;
  KernelTimer timer(kKernForward, a.stream);
  if (a.dtype == 1 && a.S == 16 && (a.D == 64 || a.D == 32)) {
    return launch_forward_s16(a, tiles);
  } else if (a.dtype == 1 && a.S == 64 && (a.D == 64 || a.D == 32)) {
    auto kern = a.D == 64 ? k_fwd_bf16<64> : k_fwd_bf16<32>;
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(256), 0, a.stream, (const bf16*)a.q,
                       (const bf16*)a.kk, (const bf16*)a.v, a.idx, a.w, (bf16*)a.o, a.lse,
                       a.n_query, a.n_key, a.k, a.attn_scale);
  } else if (a.dtype == 1) {
    hipLaunchKernelGGL(k_fwd_gen<bf16>, dim3((unsigned)tiles), dim3(64), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, a.idx, a.w,
                       (bf16*)a.o, a.lse, a.n_query, a.n_key, a.S, a.D, a.k, a.attn_scale);
  } else {
    hipLaunchKernelGGL(k_fwd_gen<float>, dim3((unsigned)tiles), dim3(64), 0, a.stream,
                       (const float*)a.q, (const float*)a.kk, (const float*)a.v, a.idx, a.w,
                       (float*)a.o, a.lse, a.n_query, a.n_key, a.S, a.D, a.k, a.attn_scale);
  }
  return hipGetLastError();
}

}  // namespace gca
