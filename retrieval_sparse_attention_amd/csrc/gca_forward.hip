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
// O is rounded to bf16 once at the end.
//
// Generic path (other sizes, float32 or bf16 elements).  One thread per query
// row, float32 arithmetic, one rounding of the output (small workloads).

#include "gca_device.h"
#include "gca_launch.h"

namespace gca {

// Per-workgroup state of the bf16 forward shared by its chunk steps.
template <int D>
struct FwdCtx {
  const TileDma<4, D>* dma;
  const bf16* k_head;
  const bf16* v_head;
  const int* s_c;      // LDS: chunk of each valid slot
  const float* s_w;    // LDS: its fusion weight
  const int* s_slot;   // LDS: its slot number
  float* s_lse;        // LDS [16][64]: log-sum-exp rows, written out at the end
  int x;
  int n, lane, grp, col;
  float c2, attn_scale;
};

// DMA of the K and V tiles of valid slot u into kd / vd.
template <int D>
__device__ __forceinline__ void fwd_issue(const FwdCtx<D>& cx, int u, bf16* __restrict__ kd,
                                          bf16* __restrict__ vd) {
  const int64_t c = uniform(cx.s_c[u]);
  cx.dma->copy_async(kd, cx.k_head + c * (64 * D));
  cx.dma->copy_async(vd, cx.v_head + c * (64 * D));
}

// One retrieved chunk: kt/vt hold its tiles; the next chunk's tiles are sent
// to kn/vn.  The restrict qualifiers tell the compiler that the LDS reads of
// this chunk never touch the buffers being filled, so it does not wait for
// that copy before reading (it would otherwise drain the copy at once).
template <int D>
__device__ __forceinline__ void fwd_chunk(const FwdCtx<D>& cx, int u, const bf16x8 (&bq)[D / 32],
                                          f32x4 (&oacc)[D / 16], const bf16* __restrict__ kt,
                                          const bf16* __restrict__ vt, bf16* __restrict__ kn,
                                          bf16* __restrict__ vn) {
  const int lane = cx.lane, grp = cx.grp, col = cx.col;
  wait_vmem();
  __syncthreads();  // tiles of slot u are in LDS; slot u-1 is done with the other buffer
  if (u + 1 < cx.n) fwd_issue(cx, u + 1, kn, vn);
  // S^T = K Q^T: key tile mt (16 keys) x this wave's 16 queries; the lane
  // holds keys 16mt + 4*grp + r of its query column x.
  f32x4 sacc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    sacc[mt] = zero4();
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd)
      sacc[mt] = mfma16x16x32(lds_row8<D>(kt, 16 * mt + col, 4 * kd + grp), bq[kd], sacc[mt]);
  }
  // V^T operands of this slot, requested now so that the LDS latency overlaps
  // the softmax arithmetic below.
  bf16x8 va[2][D / 16];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      va[kb][dt] =
          lds_tr_operand16<D>(vt, 16 * dt, 32 * kb + 4 * grp, 32 * kb + 16 + 4 * grp, lane);
  float m = max_nc(max_nc(sacc[0][0], sacc[1][0]), max_nc(sacc[2][0], sacc[3][0]));
#pragma unroll
  for (int r = 1; r < 4; ++r)
    m = max_nc(m, max_nc(max_nc(sacc[0][r], sacc[1][r]), max_nc(sacc[2][r], sacc[3][r])));
  m = xor32_max(xor16_max(m));
  const float mb = m * cx.c2;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sacc[mt][r] = fast_exp2(fmaf(sacc[mt][r], cx.c2, -mb));
  // V^T P^T (d x x) of this chunk and its row sums 1^T P^T, both on MFMA from
  // the same bf16 probabilities; K-step kb covers keys 32kb + 4*grp + 0..3
  // (key tile 2kb) and 32kb + 16 + 4*grp + 0..3 (key tile 2kb+1): exactly what
  // this lane holds; V^T comes by transpose reads.
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;
  f32x4 pv[D / 16], lacc = zero4();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bf16x8 bp;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bp[e] = (bf16)sacc[2 * kb][e];
      bp[4 + e] = (bf16)sacc[2 * kb + 1][e];
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) pv[dt] = mfma16x16x32(va[kb][dt], bp, kb ? pv[dt] : zero4());
    lacc = mfma16x16x32(ones, bp, lacc);
  }
  const float l = lacc[0];
  if (grp == 0) cx.s_lse[uniform(cx.s_slot[u]) * 64 + cx.x] = cx.attn_scale * m + fast_ln(l);
  // O^T += (w_i / l) V^T P^T: the fusion weight and the normalisation in one factor
  const float ps = cx.s_w[u] * fast_rcp(l);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) oacc[dt][e] = fmaf(ps, pv[dt][e], oacc[dt][e]);
}

template <int D>
__global__ __launch_bounds__(256) void k_fwd_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, bf16* __restrict__ o,
    float* __restrict__ lse, int64_t n_query, int64_t n_key, int topk, float attn_scale) {
  __shared__ __align__(16) bf16 k_lds[2][64 * D];
  __shared__ __align__(16) bf16 v_lds[2][64 * D];
  __shared__ int s_c[16];
  __shared__ float s_w[16];
  __shared__ int s_slot[16];
  __shared__ int s_n;
  __shared__ int s_mask;
  // Log-sum-exp rows of the k slots, staged here and stored once at the end:
  // a store per chunk would be waited on by the next chunk's copy wait.
  __shared__ float s_lse[16 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);  // = head * n_query + t
  const int64_t head = tile / n_query;
  const int x = 16 * wave + col;  // query row owned by this lane
  for (int e = tid; e < topk * 64; e += 256) s_lse[e] = -__builtin_huge_valf();  // empty slots

  // compact list of the valid slots, built in one step from a wave ballot
  if (wave == 0) {
    const int i = lane < topk ? lane : 0;
    const int c = idx[tile * topk + i];
    const float wv = w[tile * topk + i];
    const bool ok = lane < topk && c >= 0 && c < n_key;
    const uint64_t mask = __ballot(ok);
    if (ok) {
      const int pos = __popcll(mask & ((1ull << lane) - 1));
      s_c[pos] = c;
      s_w[pos] = wv;
      s_slot[pos] = lane;
    }
    if (lane == 0) {
      s_n = __popcll(mask);
      s_mask = (int)mask;
    }
  }
  bf16x8 bq[D / 32];  // Q^T as the B operand: column x, dims 32*kd + 8*grp + 0..7
  {
    const bf16* row = q + tile * (64 * D) + x * D + 8 * grp;
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) bq[kd] = *(const bf16x8*)(row + 32 * kd);
  }
  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = zero4();
  const TileDma<4, D> dma(wave, lane);
  FwdCtx<D> cx;
  cx.dma = &dma;
  cx.k_head = kk + head * n_key * (64 * D);
  cx.v_head = v + head * n_key * (64 * D);
  cx.s_c = s_c;
  cx.s_w = s_w;
  cx.s_slot = s_slot;
  cx.s_lse = s_lse;
  cx.x = x;
  cx.lane = lane;
  cx.grp = grp;
  cx.col = col;
  cx.c2 = attn_scale * kLog2e;
  cx.attn_scale = attn_scale;
  __syncthreads();
  const int n = uniform(s_n);
  cx.n = n;
  if (n > 0) fwd_issue(cx, 0, k_lds[0], v_lds[0]);
  // unrolled by two: each step's buffers are fixed LDS addresses
  for (int u = 0; u < n; u += 2) {
    fwd_chunk(cx, u, bq, oacc, k_lds[0], v_lds[0], k_lds[1], v_lds[1]);
    if (u + 1 < n) fwd_chunk(cx, u + 1, bq, oacc, k_lds[1], v_lds[1], k_lds[0], v_lds[0]);
  }
  if (lse) {
    __syncthreads();
    for (int e = tid; e < topk * 64; e += 256) lse[tile * topk * 64 + e] = s_lse[e];
  }
  // O[x][d]: this lane holds d = 16dt + 4*grp + 0..3 for its row x.
  bf16* orow = o + tile * (64 * D) + x * D + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    bf16x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) val[e] = (bf16)oacc[dt][e];
    *(bf16x4*)(orow + 16 * dt) = val;
  }
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
