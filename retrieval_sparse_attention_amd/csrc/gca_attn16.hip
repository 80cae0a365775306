// GCA attention with 16-token chunks (S = 16, D = 64 or 32) on MFMA.
//
// The same definitions as the 64-token kernels (long-context-modeling README,
// "Model Architecture"; paperlayer.ai summary, section 3.1 and appendix B):
// every token x of query chunk t attends separately to the S tokens of each
// retrieved chunk, O = sum_i w_i O^i, and the backward returns the gradients
// of Q, K, V and the weights.
//
// A 16-token chunk is one 16-row MFMA tile, so one wave owns a whole query
// chunk (forward, query side) or a whole key chunk (key side): four
// independent waves per workgroup, each with its own double-buffered LDS
// tiles filled by its own asynchronous copies, and no workgroup barrier.
// The contractions over the 16 keys (P V, dS K) or the 16 query rows
// (P_w^T dO, dS^T Q) use the 16x16x16 MFMA, whose A operand is one transpose
// read and whose B operand is exactly the lane layout the 16x16x32 score
// products leave behind.
//
// Workgroups take their four chunks in XCD order (xcd_tile): a head's
// consecutive chunks go to one XCD, whose L2 then holds that head's gathered
// tiles; the key side also sends the early chunks of each XCD range's last
// heads first (kv_tile_order over blocks of four chunks), as the 64-token
// key-side kernel does.  Against round-robin block order this took the
// key-side kernel from 565-571 to 467 us (head_dim 64) and 323-328 to 242 us
// (head_dim 32) on the 16K-token two-group step.

#include "gca_device.h"
#include "gca_launch.h"

namespace gca {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// A operand of a 16x16x16 MFMA from a swizzled 16-row LDS tile: the lane owns
// tile column c_base + lane % 16 and its 4 contraction values are tile rows
// 4g .. 4g+3 (g = lane / 16).
template <int D>
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* tile, int c_base, int g, int lane) {
  const int s = lane & 15;
  return lds_read_tr(tile + swz<D>(4 * g + (s >> 2), c_base + 4 * (s & 3)));
}

// ---------------------------------------------------------------------------
// Forward.  Wave = one query chunk (16 rows).  Per valid slot: S^T = K Q^T
// (the lane holds keys 4g .. 4g+3 of query column x = lane % 16), the row max
// over the 16 keys through two lane exchanges, P = exp2((s - max) * scale *
// log2 e) rounded to bf16 once, l = 1^T P^T and O^T += (w / l) V^T P^T on
// MFMA; L = scale * max + ln l.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_fwd_bf16_s16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, bf16* __restrict__ o,
    float* __restrict__ lse, int64_t n_query, int64_t n_key, int topk, float attn_scale,
    int64_t tiles) {
  constexpr int TE = 16 * D;
  __shared__ __align__(16) bf16 tiles_lds[4][2][2][TE];  // [wave][buffer][K, V]
  __shared__ int s_c[4][16];
  __shared__ float s_w[4][16];
  __shared__ int s_slot[4][16];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), grp = lane >> 4,
            col = lane & 15;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x) * 4 + wave;  // = head * n_query + t
  if (tile >= tiles) return;  // waves never wait on each other
  const int64_t head = tile / n_query;

  const int i0 = lane < topk ? lane : 0;
  const int c_in = idx[tile * topk + i0];
  const float w_in = w[tile * topk + i0];
  const bool ok = lane < topk && c_in >= 0 && c_in < n_key;
  const uint64_t mask = __ballot(ok);
  if (ok) {
    const int pos = __popcll(mask & ((1ull << lane) - 1));
    s_c[wave][pos] = c_in;
    s_w[wave][pos] = w_in;
    s_slot[wave][pos] = lane;
  }
  __builtin_amdgcn_wave_barrier();
  const int n = __popcll(mask);
  float* lse_tile = lse ? lse + tile * topk * 16 : nullptr;
  if (lse_tile)  // empty slots; the valid ones are written below
    for (int e = lane; e < topk * 16; e += 64)
      if (!((mask >> (e >> 4)) & 1)) lse_tile[e] = -__builtin_huge_valf();

  bf16x8 bq[D / 32];  // Q^T as the B operand: column x, dims 32kd + 8g + 0..7
  {
    const bf16* row = q + tile * TE + col * D + 8 * grp;
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) bq[kd] = *(const bf16x8*)(row + 32 * kd);
  }
  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = zero4();
  bf16x4 ones;
#pragma unroll
  for (int e = 0; e < 4; ++e) ones[e] = (bf16)1.0f;
  const TileDma<1, D, 16> dma(0, lane);
  const bf16* k_head = kk + head * n_key * TE;
  const bf16* v_head = v + head * n_key * TE;
  const float c2 = attn_scale * kLog2e;
  float lsev[4];  // L rows of slots 4j + grp (topk <= 16)
#pragma unroll
  for (int j = 0; j < 4; ++j) lsev[j] = 0.0f;
  if (n > 0) {
    const int64_t c = uniform(s_c[wave][0]);
    dma.copy_async(tiles_lds[wave][0][0], k_head + c * TE);
    dma.copy_async(tiles_lds[wave][0][1], v_head + c * TE);
  }
  for (int u = 0; u < n; ++u) {
    const bf16* kt = tiles_lds[wave][u & 1][0];
    const bf16* vt = tiles_lds[wave][u & 1][1];
    wait_vmem();  // this slot's tiles are in LDS (this wave's own copies)
    if (u + 1 < n) {
      const int64_t c = uniform(s_c[wave][u + 1]);
      dma.copy_async(tiles_lds[wave][(u + 1) & 1][0], k_head + c * TE);
      dma.copy_async(tiles_lds[wave][(u + 1) & 1][1], v_head + c * TE);
    }
    f32x4 sacc = zero4();
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd)
      sacc = mfma16x16x32(lds_row8<D>(kt, col, 4 * kd + grp), bq[kd], sacc);
    bf16x4 va[D / 16];  // V^T operands, requested before the softmax arithmetic
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) va[dt] = lds_tr4<D>(vt, 16 * dt, grp, lane);
    float m = max_nc(max_nc(sacc[0], sacc[1]), max_nc(sacc[2], sacc[3]));
    m = xor32_max(xor16_max(m));
    const float mb = m * c2;
    bf16x4 bp;
#pragma unroll
    for (int r = 0; r < 4; ++r) bp[r] = (bf16)fast_exp2(fmaf(sacc[r], c2, -mb));
    const float l = mfma16x16x16(ones, bp, zero4())[0];
    const float ps = s_w[wave][u] * fast_rcp(l);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4 pv = mfma16x16x16(va[dt], bp, zero4());
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[dt][e] = fmaf(ps, pv[e], oacc[dt][e]);
    }
    // this slot's L row, kept by the lanes with grp == u % 4 (every lane of a
    // column holds m and l): a store here would be waited on by the next
    // slot's copy wait
    const float lv = attn_scale * m + fast_ln(l);
#pragma unroll
    for (int j = 0; j < 4; ++j) lsev[j] = (u == 4 * j + grp) ? lv : lsev[j];
  }
  if (lse_tile) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * j + grp < n) lse_tile[s_slot[wave][4 * j + grp] * 16 + col] = lsev[j];
  }
  // O[x][d]: this lane holds d = 16dt + 4g + 0..3 of row x = col
  bf16* orow = o + tile * TE + col * D + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    bf16x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) val[e] = (bf16)oacc[dt][e];
    *(bf16x4*)(orow + 16 * dt) = val;
  }
}

// ---------------------------------------------------------------------------
// Query-side backward.  Wave = one query chunk.  Per valid slot: P_w = w P
// from the saved L, dP~^T = V dO^T, D = rowsum(P dP~), dw_i = sum_x D,
// dS^T = P_w (dP~ - D), dQ^T += K^T dS^T; D rows go to the workspace for the
// key side.  Then dscore_i = w_i (dw_i - sum_l w_l dw_l) and dlq.
// ---------------------------------------------------------------------------
template <int D, bool ACC>
__global__ __launch_bounds__(256) void k_bwd_q_bf16_s16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, const float* __restrict__ lse,
    const bf16* __restrict__ dout, const bf16* __restrict__ lk, bf16* __restrict__ dq,
    float* __restrict__ dw_out, float* __restrict__ dscore_out, float* __restrict__ dlq,
    float* __restrict__ delta, float* __restrict__ ds_layer, int64_t n_query, int64_t n_key,
    int topk, int dl, float attn_scale, float score_scale, int64_t tiles) {
  constexpr int TE = 16 * D;
  __shared__ __align__(16) bf16 tiles_lds[4][2][2][TE];  // [wave][buffer][K, V]
  __shared__ int s_list[4][16];
  __shared__ float s_dw[4][16];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), grp = lane >> 4,
            col = lane & 15;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x) * 4 + wave;
  if (tile >= tiles) return;
  const int64_t head = tile / n_query;

  const int i0 = lane < topk ? lane : 0;
  const int c_in = idx[tile * topk + i0];
  const float w_lane = w[tile * topk + i0];  // this lane's slot weight (lane < topk)
  const bool ok = lane < topk && c_in >= 0 && c_in < n_key;
  const int c_lane = ok ? c_in : -1;
  const uint64_t mask = __ballot(ok);
  if (ok) s_list[wave][__popcll(mask & ((1ull << lane) - 1))] = lane;
  if (lane < 16) s_dw[wave][lane] = 0.0f;
  __builtin_amdgcn_wave_barrier();
  const int n = __popcll(mask);
  float* delta_tile = delta + tile * topk * 16;
  for (int e = lane; e < topk * 16; e += 64)  // empty slots; the valid ones are written below
    if (!((mask >> (e >> 4)) & 1)) delta_tile[e] = 0.0f;

  bf16x8 bq[D / 32], bdo[D / 32];  // Q^T, dO^T as B operands: column x, dims 32kd + 8g
  {
    const bf16* qr = q + tile * TE + col * D + 8 * grp;
    const bf16* dr = dout + tile * TE + col * D + 8 * grp;
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) {
      bq[kd] = *(const bf16x8*)(qr + 32 * kd);
      bdo[kd] = *(const bf16x8*)(dr + 32 * kd);
    }
  }
  f32x4 dqacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) dqacc[dt] = zero4();
  const TileDma<1, D, 16> dma(0, lane);
  const bf16* k_head = kk + head * n_key * TE;
  const bf16* v_head = v + head * n_key * TE;
  const float* lse_tile = lse + tile * topk * 16;
  const float c2 = attn_scale * kLog2e;
  float l_next = 0.0f;
  float dlt[4];  // D rows of valid slots 4j + grp (topk <= 16)
#pragma unroll
  for (int j = 0; j < 4; ++j) dlt[j] = 0.0f;
  if (n > 0) {
    const int i = uniform(s_list[wave][0]);
    const int64_t c = __builtin_amdgcn_readlane(c_lane, i);
    dma.copy_async(tiles_lds[wave][0][0], k_head + c * TE);
    dma.copy_async(tiles_lds[wave][0][1], v_head + c * TE);
    l_next = lse_tile[i * 16 + col];
  }
  for (int u = 0; u < n; ++u) {
    const bf16* kt = tiles_lds[wave][u & 1][0];
    const bf16* vt = tiles_lds[wave][u & 1][1];
    const int i = uniform(s_list[wave][u]);
    const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_lane), i));
    wait_vmem();
    // P_w = w P: log2 w joins the row offset (w = 0 gives P_w = 0)
    const float l2 = l_next * kLog2e - __builtin_amdgcn_logf(wi);
    if (u + 1 < n) {
      const int in = uniform(s_list[wave][u + 1]);
      const int64_t c = __builtin_amdgcn_readlane(c_lane, in);
      dma.copy_async(tiles_lds[wave][(u + 1) & 1][0], k_head + c * TE);
      dma.copy_async(tiles_lds[wave][(u + 1) & 1][1], v_head + c * TE);
      l_next = lse_tile[in * 16 + col];
    }
    f32x4 sacc = zero4(), pacc = zero4();
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) {
      sacc = mfma16x16x32(lds_row8<D>(kt, col, 4 * kd + grp), bq[kd], sacc);
      pacc = mfma16x16x32(lds_row8<D>(vt, col, 4 * kd + grp), bdo[kd], pacc);
    }
    bf16x4 ka[D / 16];  // K^T operands
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) ka[dt] = lds_tr4<D>(kt, 16 * dt, grp, lane);
    float p[4], dp = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(fmaf(sacc[r], c2, -l2));  // = w P
      dp = fmaf(p[r], pacc[r], dp);
    }
    // D = rowsum(P dP~) = rowsum(P_w dP~) / w  (0 when w = 0)
    const float dsw = xor32_sum(xor16_sum(dp));
    const float dsum = wi > 0.0f ? dsw * fast_rcp(wi) : 0.0f;
    // kept by the lanes with grp == u % 4 and stored after the loop (a store
    // here would be waited on by the next slot's copy wait)
#pragma unroll
    for (int j = 0; j < 4; ++j) dlt[j] = (u == 4 * j + grp) ? dsum : dlt[j];
    const float part = row16_sum(dsum);  // over the 16 query rows
    if (lane == 0) s_dw[wave][i] = part;
    bf16x4 bs;
#pragma unroll
    for (int r = 0; r < 4; ++r) bs[r] = (bf16)(p[r] * (pacc[r] - dsum));
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) dqacc[dt] = mfma16x16x16(ka[dt], bs, dqacc[dt]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (4 * j + grp < n) delta_tile[s_list[wave][4 * j + grp] * 16 + col] = dlt[j];
  bf16* dqrow = dq + tile * TE + col * D + 4 * grp;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    bf16x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) val[e] = (bf16)(attn_scale * dqacc[dt][e]);
    *(bf16x4*)(dqrow + 16 * dt) = val;
  }
  // dscore_i = w_i (dw_i - sum_l w_l dw_l) over the valid slots; lane i holds slot i
  __builtin_amdgcn_wave_barrier();
  const float ds_lane = slot_dscore<ACC>(lane, topk, ok, w_lane, s_dw[wave][lane < 16 ? lane : 0],
                                         dw_out + tile * topk, dscore_out + tile * topk,
                                         ACC ? ds_layer + tile * topk : nullptr);
  if (dlq) {
    const bf16* lk_head = lk ? lk + head * n_key * dl : nullptr;
    for (int d = lane; d < dl; d += 64) {
      float acc = 0.0f;
      if (lk_head) {
        for (int i = 0; i < topk; ++i) {
          const int c = __builtin_amdgcn_readlane(c_lane, i);
          const float dsi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ds_lane), i));
          // empty slots have dscore 0; chunk 0 stands in so every load is issued
          acc = fmaf(dsi, (float)lk_head[(int64_t)(c >= 0 ? c : 0) * dl + d], acc);
        }
      }
      if (lk_head || !ACC) put<ACC>(dlq + tile * dl + d, score_scale * acc);
    }
  }
}

// ---------------------------------------------------------------------------
// Key-side backward.  Wave = one key chunk c; it walks c's reverse list
// (entries t * k + i, ascending).  Per entry: S = Q_t K_c^T and dP~ = dO_t V_c^T
// with the lane holding query rows 4g .. 4g+3 of key column j = lane % 16,
// P_w from the saved L and w, dS = P_w (dP~ - D), then dV^T += dO^T P_w and
// dK^T += Q^T dS over the 16 query rows, and dlk += dscore lq_t.
// ---------------------------------------------------------------------------
template <int D, bool ACC>
__global__ __launch_bounds__(256) void k_bwd_kv_bf16_s16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const float* __restrict__ w, const float* __restrict__ lse, const bf16* __restrict__ dout,
    const float* __restrict__ delta, const int32_t* __restrict__ rev_off,
    const int32_t* __restrict__ rev_ent, const bf16* __restrict__ lq,
    const float* __restrict__ dscore, void* __restrict__ dk, void* __restrict__ dv,
    float* __restrict__ dlk, int64_t n_query, int64_t n_key, int topk, int dl,
    float attn_scale, float score_scale, int64_t tiles) {
  constexpr int TE = 16 * D;
  __shared__ __align__(16) bf16 tiles_lds[4][2][2][TE];  // [wave][buffer][Q, dO]
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6), grp = lane >> 4,
            col = lane & 15;
  // blocks in the key side's XCD order, early chunks of each range's last
  // heads first (kv_tile_order over blocks of four chunks)
  const int64_t blk = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t tile =
      (n_key % 4 == 0 ? kv_tile_order(blk, n_key / 4, gridDim.x) : blk) * 4 + wave;
  if (tile >= tiles) return;
  const int64_t head = tile / n_key;
  const int64_t c = tile % n_key;

  bf16x8 bk[D / 32], bv[D / 32];  // K_c^T, V_c^T as B operands: column j, dims 32kd + 8g
  {
    const bf16* kr = kk + tile * TE + col * D + 8 * grp;
    const bf16* vr = v + tile * TE + col * D + 8 * grp;
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) {
      bk[kd] = *(const bf16x8*)(kr + 32 * kd);
      bv[kd] = *(const bf16x8*)(vr + 32 * kd);
    }
  }
  f32x4 dkacc[D / 16], dvacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) dkacc[dt] = dvacc[dt] = zero4();
  float dlk_acc = 0.0f;
  const int beg = rev_off[head * (n_key + 1) + c];
  const int end = rev_off[head * (n_key + 1) + c + 1];
  const int32_t* ents = rev_ent + head * n_query * topk;
  const int64_t pair0 = head * n_query * topk;
  const bf16* q_head = q + head * n_query * TE;
  const bf16* do_head = dout + head * n_query * TE;
  const bf16* lq_head = lq ? lq + head * n_query * dl : nullptr;
  const float c2 = attn_scale * kLog2e;
  const TileDma<1, D, 16> dma(0, lane);

  for (int b0 = beg; b0 < end; b0 += 64) {
    const int nb = (end - b0) < 64 ? (end - b0) : 64;
    const int my_ent = ents[b0 + (lane < nb ? lane : 0)];  // the block's entries, one per lane
    // the first entry's tiles and rows
    f32x4 l4, d4;
    float wv, ds = 0.0f;
    bf16 lqv = (bf16)0.0f;
    {
      const int ent = __builtin_amdgcn_readlane(my_ent, 0);
      const int64_t t = ent / topk;
      dma.copy_async(tiles_lds[wave][0][0], q_head + t * TE);
      dma.copy_async(tiles_lds[wave][0][1], do_head + t * TE);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        l4[r] = lse[(pair0 + ent) * 16 + 4 * grp + r];
        d4[r] = delta[(pair0 + ent) * 16 + 4 * grp + r];
      }
      wv = w[pair0 + ent];
      if (lq_head) {
        ds = dscore[pair0 + ent];
        lqv = lq_head[t * dl + (lane < dl ? lane : 0)];
      }
    }
    for (int u = 0; u < nb; ++u) {
      const bf16* qt = tiles_lds[wave][u & 1][0];
      const bf16* dot = tiles_lds[wave][u & 1][1];
      wait_vmem();
      const f32x4 lc = l4, dc = d4;
      const float wc = wv, dsc = ds;
      const bf16 lqc = lqv;
      if (u + 1 < nb) {
        const int ent = __builtin_amdgcn_readlane(my_ent, u + 1);
        const int64_t t = ent / topk;
        dma.copy_async(tiles_lds[wave][(u + 1) & 1][0], q_head + t * TE);
        dma.copy_async(tiles_lds[wave][(u + 1) & 1][1], do_head + t * TE);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          l4[r] = lse[(pair0 + ent) * 16 + 4 * grp + r];
          d4[r] = delta[(pair0 + ent) * 16 + 4 * grp + r];
        }
        wv = w[pair0 + ent];
        if (lq_head) {
          ds = dscore[pair0 + ent];
          lqv = lq_head[t * dl + (lane < dl ? lane : 0)];
        }
      }
      if (lq_head && lane < dl) dlk_acc = fmaf(dsc, (float)lqc, dlk_acc);
      f32x4 sacc = zero4(), pacc = zero4();
#pragma unroll
      for (int kd = 0; kd < D / 32; ++kd) {
        sacc = mfma16x16x32(lds_row8<D>(qt, col, 4 * kd + grp), bk[kd], sacc);
        pacc = mfma16x16x32(lds_row8<D>(dot, col, 4 * kd + grp), bv[kd], pacc);
      }
      bf16x4 ado[D / 16], aq[D / 16];  // dO^T and Q^T operands
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        ado[dt] = lds_tr4<D>(dot, 16 * dt, grp, lane);
        aq[dt] = lds_tr4<D>(qt, 16 * dt, grp, lane);
      }
      const float lw = __builtin_amdgcn_logf(wc);
      bf16x4 bp, bs;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pw = fast_exp2(fmaf(sacc[r], c2, -(lc[r] * kLog2e - lw)));
        bp[r] = (bf16)pw;
        bs[r] = (bf16)(pw * (pacc[r] - dc[r]));
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        dvacc[dt] = mfma16x16x16(ado[dt], bp, dvacc[dt]);
        dkacc[dt] = mfma16x16x16(aq[dt], bs, dkacc[dt]);
      }
    }
  }
  // dK^T, dV^T (d x j): this lane holds d = 16dt + 4g + 0..3 of key row j = col
  const int64_t orow = tile * TE + col * D + 4 * grp;
  if (ACC) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4* dka = (f32x4*)((float*)dk + orow + 16 * dt);
      f32x4* dva = (f32x4*)((float*)dv + orow + 16 * dt);
      f32x4 ka = *dka, va = *dva;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ka[e] += attn_scale * dkacc[dt][e];
        va[e] += dvacc[dt][e];
      }
      *dka = ka;
      *dva = va;
    }
  } else {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      bf16x4 kv4, vv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv4[e] = (bf16)(attn_scale * dkacc[dt][e]);
        vv4[e] = (bf16)dvacc[dt][e];
      }
      *(bf16x4*)((bf16*)dk + orow + 16 * dt) = kv4;
      *(bf16x4*)((bf16*)dv + orow + 16 * dt) = vv4;
    }
  }
  if (dlk && lane < dl) put<ACC>(dlk + tile * dl + lane, score_scale * dlk_acc);
}

hipError_t launch_forward_s16(const LaunchForward& a, int64_t tiles) {
  const unsigned blocks = (unsigned)((tiles + 3) / 4);
  auto kern = a.D == 64 ? k_fwd_bf16_s16<64> : k_fwd_bf16_s16<32>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, a.stream, (const bf16*)a.q,
                     (const bf16*)a.kk, (const bf16*)a.v, a.idx, a.w, (bf16*)a.o, a.lse,
                     a.n_query, a.n_key, a.k, a.attn_scale, tiles);
  return hipGetLastError();
}

hipError_t launch_backward_s16(const LaunchBackward& a, int64_t qtiles, int64_t ktiles) {
  hipError_t err;
  if (qtiles > 0) {
    KernelTimer timer(kKernBackwardQ, a.stream);
    auto kern = a.D == 64
                    ? (a.accumulate ? k_bwd_q_bf16_s16<64, true> : k_bwd_q_bf16_s16<64, false>)
                    : (a.accumulate ? k_bwd_q_bf16_s16<32, true> : k_bwd_q_bf16_s16<32, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)((qtiles + 3) / 4)), dim3(256), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, a.idx, a.w, a.lse,
                       (const bf16*)a.dout, (const bf16*)a.lk, (bf16*)a.dq, a.dw, a.dscore,
                       a.dlq, a.delta, a.ds_layer, a.n_query, a.n_key, a.k, a.dl,
                       a.attn_scale, a.score_scale, qtiles);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ktiles > 0) {
    KernelTimer timer(kKernBackwardKV, a.stream);
    auto kern = a.D == 64
                    ? (a.accumulate ? k_bwd_kv_bf16_s16<64, true> : k_bwd_kv_bf16_s16<64, false>)
                    : (a.accumulate ? k_bwd_kv_bf16_s16<32, true> : k_bwd_kv_bf16_s16<32, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)((ktiles + 3) / 4)), dim3(256), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, a.w, a.lse,
                       (const bf16*)a.dout, a.delta, a.rev_off, a.rev_ent, (const bf16*)a.lq,
                       a.accumulate ? a.ds_layer : a.dscore, a.dk, a.dv, a.dlk, a.n_query,
                       a.n_key, a.k, a.dl, a.attn_scale, a.score_scale, ktiles);
  }
  return hipGetLastError();
}

}  // namespace gca
