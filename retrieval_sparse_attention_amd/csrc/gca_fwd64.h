// 64-token bf16 forward (S = 64, D = 64 or 32): the per-query-chunk body shared
// by k_fwd_bf16 (slot table read from idx / w) and the fused top-k merge +
// forward of a sliced retrieval (slot table from the merge).  The kernel's
// description is in gca_forward.hip.
#pragma once

#include "gca_device.h"

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

// One query chunk's forward in a 256-thread workgroup: lane i of every wave
// holds slot i's chunk c_in and weight w_in, ok when the slot is valid (lanes
// >= topk pass ok = false).  k_lds / v_lds: the workgroup's two K and V tile
// buffers; no other LDS is used.
template <int D>
__device__ __forceinline__ void fwd_tile(const bf16* __restrict__ q, const bf16* __restrict__ kk,
                                         const bf16* __restrict__ v, bf16* __restrict__ o,
                                         float* __restrict__ lse, int64_t tile, int64_t n_query,
                                         int64_t n_key, int topk, float attn_scale, int c_in,
                                         float w_in, bool ok, bf16 (*k_lds)[64 * D],
                                         bf16 (*v_lds)[64 * D]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int64_t head = tile / n_query;
  const int x = 16 * wave + col;  // query row owned by this lane
  const uint32_t mask = (uint32_t)__ballot(ok);  // bit i: slot i valid (topk <= 16)
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

}  // namespace gca
