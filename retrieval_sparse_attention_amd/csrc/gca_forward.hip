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
#include "gca_launch.h"

namespace gca {

// Per-workgroup state of the bf16 forward shared by its chunk steps.
template <int D>
struct FwdCtx {
  const TileDma<4, D>* dma;
  const bf16* k_head;
  const bf16* v_head;
  int c_lane;     // lane i: chunk of slot i (valid slots only)
  float w_lane;   // lane i: fusion weight of slot i
  int x;
  int lane, grp, col;
  float c2, attn_scale;
};

// DMA of the K and V tiles of slot i into kd / vd.
template <int D>
__device__ __forceinline__ void fwd_issue(const FwdCtx<D>& cx, int i, bf16* __restrict__ kd,
                                          bf16* __restrict__ vd) {
  const int64_t c = __builtin_amdgcn_readlane(cx.c_lane, i);
  cx.dma->copy_async(kd, cx.k_head + c * (64 * D));
  cx.dma->copy_async(vd, cx.v_head + c * (64 * D));
}

// One retrieved chunk (slot i, the u-th valid one; next: the next valid slot
// or -1): kt/vt hold its tiles; the next chunk's tiles are sent to kn/vn.
// The restrict qualifiers tell the compiler that the LDS reads of this chunk
// never touch the buffers being filled, so it does not wait for that copy
// before reading (it would otherwise drain the copy at once).
template <int D>
__device__ __forceinline__ void fwd_chunk(const FwdCtx<D>& cx, int u, int i, int next,
                                          const bf16x8 (&bq)[D / 32], f32x4 (&oacc)[D / 16],
                                          float (&lsev)[4], const bf16* __restrict__ kt,
                                          const bf16* __restrict__ vt, bf16* __restrict__ kn,
                                          bf16* __restrict__ vn) {
  const int lane = cx.lane, grp = cx.grp, col = cx.col;
  wait_vmem();
  __syncthreads();  // tiles of slot i are in LDS; the previous slot is done with the other buffer
  if (next >= 0) fwd_issue(cx, next, kn, vn);
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
  // the same bf16 probabilities; K-step kb covers keys 32kb + 4*grp + 0..3 and
  // 32kb + 16 + 4*grp + 0..3, exactly what this lane holds; V^T comes by
  // transpose reads, each right before its product.
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
    for (int dt = 0; dt < D / 16; ++dt) {
      const bf16x8 va =
          lds_tr_operand16<D>(vt, 16 * dt, 32 * kb + 4 * grp, 32 * kb + 16 + 4 * grp, lane);
      pv[dt] = mfma16x16x32(va, bp, kb ? pv[dt] : zero4());
    }
    lacc = mfma16x16x32(ones, bp, lacc);
  }
  const float l = lacc[0];
  // this slot's L row, kept by the lanes with grp == u % 4 (every lane of the
  // column holds m and l) and stored after the loop
  const float lv = cx.attn_scale * m + fast_ln(l);
#pragma unroll
  for (int j = 0; j < 4; ++j) lsev[j] = (u == 4 * j + grp) ? lv : lsev[j];
  // O^T += (w_i / l) V^T P^T: the fusion weight and the normalisation in one factor
  const float ps = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cx.w_lane), i)) *
                   fast_rcp(l);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) oacc[dt][e] = fmaf(ps, pv[dt][e], oacc[dt][e]);
}

template <int D>
__global__ __launch_bounds__(256, 5) void k_fwd_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, bf16* __restrict__ o,
    float* __restrict__ lse, int64_t n_query, int64_t n_key, int topk, float attn_scale) {
  __shared__ __align__(16) bf16 k_lds[2][64 * D];
  __shared__ __align__(16) bf16 v_lds[2][64 * D];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);  // = head * n_query + t
  const int64_t head = tile / n_query;
  const int x = 16 * wave + col;  // query row owned by this lane

  // every wave reads the slot table itself: lane i holds slot i
  const int i0 = lane < topk ? lane : 0;
  const int c_in = idx[tile * topk + i0];
  const float w_in = w[tile * topk + i0];
  const bool ok = lane < topk && c_in >= 0 && c_in < n_key;
  const uint32_t mask = (uint32_t)__ballot(ok);  // topk <= 16
  const int n = __popc(mask);
  bf16x8 bq[D / 32];  // Q^T as the B operand: column x, dims 32*kd + 8*grp + 0..7
  {
    const bf16* row = q + tile * (64 * D) + x * D + 8 * grp;
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) bq[kd] = *(const bf16x8*)(row + 32 * kd);
  }
  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = zero4();
  float lsev[4];  // L rows of the valid slots with ordinal 4j + grp (topk <= 16)
#pragma unroll
  for (int j = 0; j < 4; ++j) lsev[j] = 0.0f;
  const TileDma<4, D> dma(wave, lane);
  FwdCtx<D> cx;
  cx.dma = &dma;
  cx.k_head = kk + head * n_key * (64 * D);
  cx.v_head = v + head * n_key * (64 * D);
  cx.c_lane = ok ? c_in : 0;
  cx.w_lane = w_in;
  cx.x = x;
  cx.lane = lane;
  cx.grp = grp;
  cx.col = col;
  cx.c2 = attn_scale * kLog2e;
  cx.attn_scale = attn_scale;
  int i = mask ? (int)__builtin_ctz(mask) : -1;
  if (i >= 0) fwd_issue(cx, i, k_lds[0], v_lds[0]);
  // unrolled by two: each step's buffers are fixed LDS addresses
  for (int u = 0; u < n; u += 2) {
    int nx = next_slot(mask, i);
    fwd_chunk(cx, u, i, nx, bq, oacc, lsev, k_lds[0], v_lds[0], k_lds[1], v_lds[1]);
    i = nx;
    if (u + 1 < n) {
      nx = next_slot(mask, i);
      fwd_chunk(cx, u + 1, i, nx, bq, oacc, lsev, k_lds[1], v_lds[1], k_lds[0], v_lds[0]);
      i = nx;
    }
  }
  if (lse) {
    float* lt = lse + tile * topk * 64;
    for (int e = lane; e < topk * 16; e += 64) {  // empty slots of this wave's 16 rows
      const int s = e >> 4;
      if (!((mask >> s) & 1)) lt[s * 64 + 16 * wave + (e & 15)] = -__builtin_huge_valf();
    }
    // valid slot with ordinal 4j + grp: its L row for this lane's query row
    int ord = 0;
    for (int s = 0; s < topk; ++s) {
      if (!((mask >> s) & 1)) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ord == 4 * j + grp) lt[s * 64 + x] = lsev[j];
      ++ord;
    }
  }
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
