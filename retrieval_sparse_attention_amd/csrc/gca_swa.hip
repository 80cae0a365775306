// Causal sliding-window self-attention: the other attention of a DRT layer.
//
// Definition (paperlayer.ai summary, section 1 and section 3.2: each layer
// pairs GCA over retrieved chunks with fixed-size sliding-window
// self-attention; section 4.1.2: a 512-token window).  Token x attends to the
// keys y with x - W < y <= x:
//   O[x] = sum_y P[x,y] V[y],  P[x,.] = softmax_y(scale <Q[x], K[y]>),
//   L[x] = log sum_y exp(scale <Q[x], K[y]>)
// and the backward, with D[x] = <dO[x], O[x]>:
//   dS = P (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
//
// bf16, D = 64, T a multiple of 64.  Q, K, V are cut into 64-token blocks
// (8 KB tiles, the same layout as the GCA chunks), so query block t needs
// key blocks max(0, floor((64t - W + 1) / 64)) .. t: 9 tiles at W = 512.  Only
// the diagonal tile and the tile where the window starts need masks.
//   k_swa_fwd_bf16    : one 4-wave workgroup per query block; each wave owns 16
//                       query rows; K/V tiles stream into double-buffered LDS
//                       (asynchronous copies) and an online softmax carries O
//                       across tiles (offset raised only when the row max grows
//                       by more than 2^8; the row sum formed on MFMA).
//   k_swa_bwd_q_bf16  : one workgroup per query block; D from dO and O, then
//                       dQ over the block's key tiles; writes D.
//   k_swa_bwd_kv_bf16 : one workgroup per key block; dK, dV over the query
//                       blocks that see it (reads D and L).
// No floating-point atomics: every output has one writer and a fixed order.

#include "gca_device.h"
#include "gca_launch.h"

namespace gca {

// Pair (key row y_local of key block j, query row x_local of query block t) is
// inside the window iff dy = 64 (j - t) + y_local - x_local is in (-W, 0].
__device__ __forceinline__ bool in_window(int dy, int window) { return dy <= 0 && dy > -window; }

// Whether the tile pair (key block j, query block t) has any pair outside the
// window (the diagonal block, or a key block that reaches below the window).
__device__ __forceinline__ bool edge_tile(int j, int t, int window) {
  return j == t || 64 * j + window <= 64 * t + 63;
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
struct SwaFwdCtx {
  const TileDma<4>* dma;
  const bf16* k_head;
  const bf16* v_head;
  int t, j_lo, n, window;
  int x, lane, grp, col;
  float c2;
};

__device__ __forceinline__ void swa_fwd_issue(const SwaFwdCtx& cx, int u, bf16* __restrict__ kd,
                                              bf16* __restrict__ vd) {
  const int64_t j = cx.j_lo + u;
  cx.dma->copy_async(kd, cx.k_head + j * 4096);
  cx.dma->copy_async(vd, cx.v_head + j * 4096);
}

// Offset growth (log2 units) tolerated before O and the row sum are rescaled:
// probabilities stay below 2^8 in the meantime, far inside float32 and bf16
// range, and O and the sum always share one offset, so the result is exact.
constexpr float kRescaleSlack = 8.0f;

// Key tile u of the block (buffers kt/vt); the next tile goes to kn/vn.  mb is
// the row's exponent offset in log2 units (starts at -1e30: no key yet), lacc
// the row sum of the bf16 probabilities, formed on MFMA with an all-ones
// operand so that it matches the probabilities that multiply V.
__device__ __forceinline__ void swa_fwd_tile(const SwaFwdCtx& cx, int u, const bf16x8 (&bq)[2],
                                             f32x4 (&oacc)[4], f32x4& lacc, float& mb,
                                             const bf16* __restrict__ kt,
                                             const bf16* __restrict__ vt, bf16* __restrict__ kn,
                                             bf16* __restrict__ vn) {
  const int lane = cx.lane, grp = cx.grp, col = cx.col;
  wait_vmem();
  __syncthreads();  // tiles of u are in LDS; tile u-1 is done with the other buffer
  if (u + 1 < cx.n) swa_fwd_issue(cx, u + 1, kn, vn);
  // S^T = K Q^T: the lane holds keys 16mt + 4grp + r of its query row x.
  f32x4 sacc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    sacc[mt] = zero4();
#pragma unroll
    for (int kd = 0; kd < 2; ++kd)
      sacc[mt] = mfma16x16x32(lds_row8(kt, 16 * mt + col, 4 * kd + grp), bq[kd], sacc[mt]);
  }
  bf16x8 va[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      va[kb][dt] = lds_tr_operand16(vt, 16 * dt, 32 * kb + 4 * grp, 32 * kb + 16 + 4 * grp, lane);
  const int j = cx.j_lo + u;
  if (edge_tile(j, cx.t, cx.window)) {
    const int base = 64 * (j - cx.t) - cx.x + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!in_window(base + 16 * mt + r, cx.window)) sacc[mt][r] = -__builtin_huge_valf();
  }
  float m = max_nc(max_nc(sacc[0][0], sacc[1][0]), max_nc(sacc[2][0], sacc[3][0]));
#pragma unroll
  for (int r = 1; r < 4; ++r)
    m = max_nc(m, max_nc(max_nc(sacc[0][r], sacc[1][r]), max_nc(sacc[2][r], sacc[3][r])));
  m = xor32_max(xor16_max(m));
  const float mt2 = m * cx.c2;  // -inf while the row has no key in the window
  if (__any(mt2 > mb + kRescaleSlack)) {
    const float mb_new = mt2 > mb + kRescaleSlack ? mt2 : mb;
    const float alpha = fast_exp2(mb - mb_new);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[dt][e] *= alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) lacc[e] *= alpha;
    mb = mb_new;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sacc[mt][r] = fast_exp2(fmaf(sacc[mt][r], cx.c2, -mb));
  // O^T (d x x) += V^T (d x j) P^T (j x x) and the row sum 1^T P^T, P unnormalised
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bf16x8 bp;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bp[e] = (bf16)sacc[2 * kb][e];
      bp[4 + e] = (bf16)sacc[2 * kb + 1][e];
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = mfma16x16x32(va[kb][dt], bp, oacc[dt]);
    lacc = mfma16x16x32(ones, bp, lacc);
  }
}

__global__ __launch_bounds__(256) void k_swa_fwd_bf16(const bf16* __restrict__ q,
                                                      const bf16* __restrict__ kk,
                                                      const bf16* __restrict__ v,
                                                      bf16* __restrict__ o,
                                                      float* __restrict__ lse, int64_t n_tok,
                                                      int window, float scale) {
  __shared__ __align__(16) bf16 k_lds[2][kTileElems];
  __shared__ __align__(16) bf16 v_lds[2][kTileElems];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int64_t nb = n_tok / 64;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);  // = head * nb + t
  const int64_t head = tile / nb;
  const int t = (int)(tile % nb);
  const int x = 16 * wave + col;  // query row of this lane in the block
  const int lo = 64 * t - window + 1;
  const int j_lo = lo <= 0 ? 0 : lo / 64;
  bf16x8 bq[2];
  {
    const bf16* row = q + tile * 4096 + x * 64 + 8 * grp;
#pragma unroll
    for (int kd = 0; kd < 2; ++kd) bq[kd] = *(const bf16x8*)(row + 32 * kd);
  }
  f32x4 oacc[4] = {zero4(), zero4(), zero4(), zero4()};
  f32x4 lacc = zero4();
  float mb = -1e30f;
  const TileDma<4> dma(wave, lane);
  SwaFwdCtx cx;
  cx.dma = &dma;
  cx.k_head = kk + head * n_tok * 64;
  cx.v_head = v + head * n_tok * 64;
  cx.t = t;
  cx.j_lo = j_lo;
  cx.n = t - j_lo + 1;
  cx.window = window;
  cx.x = x;
  cx.lane = lane;
  cx.grp = grp;
  cx.col = col;
  cx.c2 = scale * kLog2e;
  const int n = cx.n;
  swa_fwd_issue(cx, 0, k_lds[0], v_lds[0]);
  for (int u = 0; u < n; u += 2) {
    swa_fwd_tile(cx, u, bq, oacc, lacc, mb, k_lds[0], v_lds[0], k_lds[1], v_lds[1]);
    if (u + 1 < n)
      swa_fwd_tile(cx, u + 1, bq, oacc, lacc, mb, k_lds[1], v_lds[1], k_lds[0], v_lds[0]);
  }
  // every row sees at least its own key: l > 0
  const float l_run = lacc[0];
  const float inv_l = fast_rcp(l_run);
  bf16* orow = o + tile * 4096 + x * 64 + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    bf16x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) val[e] = (bf16)(oacc[dt][e] * inv_l);
    *(bf16x4*)(orow + 16 * dt) = val;
  }
  if (lse && grp == 0) lse[tile * 64 + x] = mb * 0.69314718055994531f + fast_ln(l_run);
}

// ---------------------------------------------------------------------------
// Query-side backward
// ---------------------------------------------------------------------------
struct SwaBwdQCtx {
  const TileDma<4>* dma;
  const bf16* k_head;
  const bf16* v_head;
  int t, j_lo, n, window;
  int x, lane, grp, col;
  float c2, l2, dsum;
};

__device__ __forceinline__ void swa_bwdq_tile(const SwaBwdQCtx& cx, int u, const bf16x8 (&bq)[2],
                                              const bf16x8 (&bdo)[2], f32x4 (&dqacc)[4],
                                              const bf16* __restrict__ kt,
                                              const bf16* __restrict__ vt, bf16* __restrict__ kn,
                                              bf16* __restrict__ vn) {
  const int lane = cx.lane, grp = cx.grp, col = cx.col;
  wait_vmem();
  __syncthreads();
  if (u + 1 < cx.n) {
    const int64_t jn = cx.j_lo + u + 1;
    cx.dma->copy_async(kn, cx.k_head + jn * 4096);
    cx.dma->copy_async(vn, cx.v_head + jn * 4096);
  }
  // S^T = K Q^T and dP^T = V dO^T; the lane holds keys 16mt + 4grp + r of row x
  f32x4 sacc[4], pacc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    sacc[mt] = zero4();
    pacc[mt] = zero4();
#pragma unroll
    for (int kd = 0; kd < 2; ++kd) {
      sacc[mt] = mfma16x16x32(lds_row8(kt, 16 * mt + col, 4 * kd + grp), bq[kd], sacc[mt]);
      pacc[mt] = mfma16x16x32(lds_row8(vt, 16 * mt + col, 4 * kd + grp), bdo[kd], pacc[mt]);
    }
  }
  const int j = cx.j_lo + u;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sacc[mt][r] = fast_exp2(fmaf(sacc[mt][r], cx.c2, -cx.l2));
  if (edge_tile(j, cx.t, cx.window)) {  // wave-uniform: only 2 of the block's tiles
    const int base = 64 * (j - cx.t) - cx.x + 4 * grp;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!in_window(base + 16 * mt + r, cx.window)) sacc[mt][r] = 0.0f;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sacc[mt][r] = sacc[mt][r] * (pacc[mt][r] - cx.dsum);  // dS
  // dQ^T (d x x) += K^T (d x j) dS^T (j x x)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bf16x8 bs;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bs[e] = (bf16)sacc[2 * kb][e];
      bs[4 + e] = (bf16)sacc[2 * kb + 1][e];
    }
    // K^T operands read right before their products (register budget of four
    // workgroups per CU)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      dqacc[dt] = mfma16x16x32(
          lds_tr_operand16(kt, 16 * dt, 32 * kb + 4 * grp, 32 * kb + 16 + 4 * grp, lane), bs,
          dqacc[dt]);
  }
}

__global__ __launch_bounds__(256, 4) void k_swa_bwd_q_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const bf16* __restrict__ o, const float* __restrict__ lse, const bf16* __restrict__ dout,
    bf16* __restrict__ dq, float* __restrict__ delta, int64_t n_tok, int window, float scale) {
  __shared__ __align__(16) bf16 k_lds[2][kTileElems];
  __shared__ __align__(16) bf16 v_lds[2][kTileElems];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int64_t nb = n_tok / 64;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t head = tile / nb;
  const int t = (int)(tile % nb);
  const int x = 16 * wave + col;
  const int lo = 64 * t - window + 1;
  const int j_lo = lo <= 0 ? 0 : lo / 64;
  const TileDma<4> dma(wave, lane);
  SwaBwdQCtx cx;
  cx.dma = &dma;
  cx.k_head = kk + head * n_tok * 64;
  cx.v_head = v + head * n_tok * 64;
  cx.t = t;
  cx.j_lo = j_lo;
  cx.n = t - j_lo + 1;
  cx.window = window;
  cx.x = x;
  cx.lane = lane;
  cx.grp = grp;
  cx.col = col;
  cx.c2 = scale * kLog2e;
  cx.dma->copy_async(k_lds[0], cx.k_head + (int64_t)j_lo * 4096);
  cx.dma->copy_async(v_lds[0], cx.v_head + (int64_t)j_lo * 4096);
  // Q^T, dO^T (B operands: column x, dims 32kd + 8grp + 0..7) and O for D
  bf16x8 bq[2], bdo[2], bo[2];
  {
    const int64_t off = tile * 4096 + x * 64 + 8 * grp;
#pragma unroll
    for (int kd = 0; kd < 2; ++kd) {
      bq[kd] = *(const bf16x8*)(q + off + 32 * kd);
      bdo[kd] = *(const bf16x8*)(dout + off + 32 * kd);
      bo[kd] = *(const bf16x8*)(o + off + 32 * kd);
    }
  }
  const float row_lse = lse[tile * 64 + x];
  float d = 0.0f;
#pragma unroll
  for (int kd = 0; kd < 2; ++kd)
#pragma unroll
    for (int e = 0; e < 8; ++e) d = fmaf((float)bdo[kd][e], (float)bo[kd][e], d);
  cx.dsum = xor32_sum(xor16_sum(d));
  cx.l2 = row_lse * kLog2e;
  f32x4 dqacc[4] = {zero4(), zero4(), zero4(), zero4()};
  const int n = cx.n;
  for (int u = 0; u < n; u += 2) {
    swa_bwdq_tile(cx, u, bq, bdo, dqacc, k_lds[0], v_lds[0], k_lds[1], v_lds[1]);
    if (u + 1 < n) swa_bwdq_tile(cx, u + 1, bq, bdo, dqacc, k_lds[1], v_lds[1], k_lds[0], v_lds[0]);
  }
  bf16* dqrow = dq + tile * 4096 + x * 64 + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    bf16x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) val[e] = (bf16)(scale * dqacc[dt][e]);
    *(bf16x4*)(dqrow + 16 * dt) = val;
  }
  if (grp == 0) delta[tile * 64 + x] = cx.dsum;
}

// ---------------------------------------------------------------------------
// Key-side backward
// ---------------------------------------------------------------------------
struct SwaBwdKVCtx {
  const TileDma<4>* dma;
  const bf16* q_head;
  const bf16* do_head;
  const float* lse_head;
  const float* d_head;
  int j, t_lo, n, window;
  int tid, lane, grp, col, jl;
  float c2;
};

// Query block t_lo + u: tiles of Q and dO to qd / dod, its L and D rows to `row`.
__device__ __forceinline__ void swa_bwdkv_fetch(const SwaBwdKVCtx& cx, int u, float& row,
                                                bf16* __restrict__ qd, bf16* __restrict__ dod) {
  const int64_t t = cx.t_lo + u;
  cx.dma->copy_async(qd, cx.q_head + t * 4096);
  cx.dma->copy_async(dod, cx.do_head + t * 4096);
  // both rows from wave-uniform bases (no per-lane 64-bit pointer kept live);
  // threads 0..63 keep L, 64..127 keep D
  const int tid = cx.tid;
  const float a = cx.lse_head[t * 64 + (tid & 63)];
  const float b = cx.d_head[t * 64 + (tid & 63)];
  row = tid < 64 ? a : b;
}

__device__ __forceinline__ void swa_bwdkv_block(const SwaBwdKVCtx& cx, int u, float& row,
                                                const bf16x8 (&bk)[2], const bf16x8 (&bv)[2],
                                                f32x4 (&dkacc)[4], f32x4 (&dvacc)[4],
                                                const bf16* __restrict__ qt,
                                                const bf16* __restrict__ dot,
                                                float* __restrict__ l2r, float* __restrict__ dr,
                                                bf16* __restrict__ qn, bf16* __restrict__ don) {
  const int lane = cx.lane, grp = cx.grp, col = cx.col, tid = cx.tid;
  wait_vmem();
  if (tid < 64)
    l2r[tid] = row * kLog2e;
  else if (tid < 128)
    dr[tid - 64] = row;
  __syncthreads();
  if (u + 1 < cx.n) swa_bwdkv_fetch(cx, u + 1, row, qn, don);
  const int t = cx.t_lo + u;
  const bool edge = edge_tile(cx.j, t, cx.window);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // S (x x j) = Q K^T and dP = dO V^T for query rows x = 32kb + 16h + 4grp + r
    f32x4 sacc[2], pacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int xr = 32 * kb + 16 * h + col;
      sacc[h] = zero4();
      pacc[h] = zero4();
#pragma unroll
      for (int kd = 0; kd < 2; ++kd) {
        sacc[h] = mfma16x16x32(lds_row8(qt, xr, 4 * kd + grp), bk[kd], sacc[h]);
        pacc[h] = mfma16x16x32(lds_row8(dot, xr, 4 * kd + grp), bv[kd], pacc[h]);
      }
      const int x0 = 32 * kb + 16 * h + 4 * grp;
      const f32x4 l4 = *(const f32x4*)(l2r + x0);
      const f32x4 d4 = *(const f32x4*)(dr + x0);
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[h][e] = fast_exp2(fmaf(sacc[h][e], cx.c2, -l4[e]));
      if (edge) {  // wave-uniform: only 2 of the key block's query blocks
        const int base = 64 * (cx.j - t) + cx.jl - x0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!in_window(base - e, cx.window)) sacc[h][e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pacc[h][e] = sacc[h][e] * (pacc[h][e] - d4[e]);
    }
    // dV^T (d x j) += dO^T (d x x) P (x x j);  dK^T (d x j) += Q^T (d x x) dS (x x j)
    bf16x8 bp, bs;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bp[e] = (bf16)sacc[0][e];
      bp[4 + e] = (bf16)sacc[1][e];
      bs[e] = (bf16)pacc[0][e];
      bs[4 + e] = (bf16)pacc[1][e];
    }
    // dO^T and Q^T operands read right before their products (register
    // budget of four workgroups per CU; the other waves cover the LDS latency)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x8 ado =
          lds_tr_operand16(dot, 16 * dt, 32 * kb + 4 * grp, 32 * kb + 16 + 4 * grp, lane);
      const bf16x8 aq =
          lds_tr_operand16(qt, 16 * dt, 32 * kb + 4 * grp, 32 * kb + 16 + 4 * grp, lane);
      dvacc[dt] = mfma16x16x32(ado, bp, dvacc[dt]);
      dkacc[dt] = mfma16x16x32(aq, bs, dkacc[dt]);
    }
  }
}

__global__ __launch_bounds__(256, 4) void k_swa_bwd_kv_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const float* __restrict__ lse, const bf16* __restrict__ dout,
    const float* __restrict__ delta, bf16* __restrict__ dk, bf16* __restrict__ dv,
    int64_t n_tok, int window, float scale) {
  __shared__ __align__(16) bf16 q_lds[2][kTileElems];
  __shared__ __align__(16) bf16 do_lds[2][kTileElems];
  __shared__ __align__(16) float l2_lds[2][64];
  __shared__ __align__(16) float d_lds[2][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int64_t nb = n_tok / 64;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);  // = head * nb + j
  const int64_t head = tile / nb;
  const int j = (int)(tile % nb);
  const int jl = 16 * wave + col;  // key row owned by this lane
  // query blocks that see key block j: x in [64j, 64j + 63 + W - 1]
  const int64_t hi = (64 * (int64_t)j + 62 + window) / 64;
  const int t_hi = (int)(hi < nb - 1 ? hi : nb - 1);
  bf16x8 bk[2], bv[2];
  {
    const int64_t off = tile * 4096 + jl * 64 + 8 * grp;
#pragma unroll
    for (int kd = 0; kd < 2; ++kd) {
      bk[kd] = *(const bf16x8*)(kk + off + 32 * kd);
      bv[kd] = *(const bf16x8*)(v + off + 32 * kd);
    }
  }
  f32x4 dkacc[4] = {zero4(), zero4(), zero4(), zero4()};
  f32x4 dvacc[4] = {zero4(), zero4(), zero4(), zero4()};
  const TileDma<4> dma(wave, lane);
  SwaBwdKVCtx cx;
  cx.dma = &dma;
  cx.q_head = q + head * n_tok * 64;
  cx.do_head = dout + head * n_tok * 64;
  cx.lse_head = lse + head * n_tok;
  cx.d_head = delta + head * n_tok;
  cx.j = j;
  cx.t_lo = j;
  cx.n = t_hi - j + 1;
  cx.window = window;
  cx.tid = tid;
  cx.lane = lane;
  cx.grp = grp;
  cx.col = col;
  cx.jl = jl;
  cx.c2 = scale * kLog2e;
  float row = 0.0f;
  swa_bwdkv_fetch(cx, 0, row, q_lds[0], do_lds[0]);
  const int n = cx.n;
  for (int u = 0; u < n; u += 2) {
    swa_bwdkv_block(cx, u, row, bk, bv, dkacc, dvacc, q_lds[0], do_lds[0], l2_lds[0], d_lds[0],
                    q_lds[1], do_lds[1]);
    if (u + 1 < n)
      swa_bwdkv_block(cx, u + 1, row, bk, bv, dkacc, dvacc, q_lds[1], do_lds[1], l2_lds[1],
                      d_lds[1], q_lds[0], do_lds[0]);
  }
  const int64_t off = tile * 4096 + jl * 64 + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    bf16x4 kv4, vv4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv4[e] = (bf16)(scale * dkacc[dt][e]);
      vv4[e] = (bf16)dvacc[dt][e];
    }
    *(bf16x4*)(dk + off + 16 * dt) = kv4;
    *(bf16x4*)(dv + off + 16 * dt) = vv4;
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
hipError_t launch_swa_forward(const LaunchSwa& a) {
  const int64_t blocks = a.heads * (a.n_tok / 64);
  if (blocks == 0) return hipSuccess;
  KernelTimer timer(kKernSwaForward, a.stream);
  hipLaunchKernelGGL(k_swa_fwd_bf16, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                     (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, (bf16*)a.o, a.lse,
                     a.n_tok, a.window, a.scale);
  return hipGetLastError();
}

hipError_t launch_swa_backward(const LaunchSwa& a) {
  const int64_t blocks = a.heads * (a.n_tok / 64);
  if (blocks == 0) return hipSuccess;
  {
    KernelTimer timer(kKernSwaBackwardQ, a.stream);
    hipLaunchKernelGGL(k_swa_bwd_q_bf16, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, (const bf16*)a.o,
                       (const float*)a.lse, (const bf16*)a.dout, (bf16*)a.dq, a.delta, a.n_tok,
                       a.window, a.scale);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KernelTimer timer(kKernSwaBackwardKV, a.stream);
  hipLaunchKernelGGL(k_swa_bwd_kv_bf16, dim3((unsigned)blocks), dim3(256), 0, a.stream,
                     (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, (const float*)a.lse,
                     (const bf16*)a.dout, (const float*)a.delta, (bf16*)a.dk, (bf16*)a.dv,
                     a.n_tok, a.window, a.scale);
  return hipGetLastError();
}

}  // namespace gca
