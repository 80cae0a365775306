// GCA backward: gradients of Eq. 2 / Eq. 3 and, through the fusion weights, of
// the Eq. 1 relevance scores and the landmarks.
//
// Definition (paperlayer.ai summary, appendix B: the backward returns gradients
// for Q, K, V and the weights; long-context-modeling README, "Model
// Architecture": the loss reaches the retrieval scores through the weights).
// For pair (t, i) with chunk c = idx[t, i], P = softmax(attn_scale Q_t K_c^T):
//   dP~   = dO_t V_c^T,     D[x] = sum_j P dP~ = <dO_t[x], O^i[x]>
//   dw_i  = sum_x D[x]
//   dS    = w_i P (dP~ - D)
//   dQ_t += attn_scale dS K_c,  dK_c += attn_scale dS^T Q_t,  dV_c += w_i P^T dO_t
//   dscore_i = w_i (dw_i - sum_l w_l dw_l)
//   dlq_t += score_scale sum_i dscore_i lk_c,  dlk_c += score_scale dscore_i lq_t
//
// No floating-point atomics: three kernels run in stream order.
//   k_reverse_index : per head, the list of (t, i) pairs of every key chunk, in
//                     ascending (t, i) order (counting sort, deterministic).
//   k_bwd_q_*       : one workgroup per query chunk; recomputes P from the
//                     saved log-sum-exp, accumulates dQ over the k slots and
//                     writes dw, dscore, dlq and D (workspace "delta").
//   k_bwd_kv_*      : one workgroup per key chunk; walks its reverse list,
//                     recomputes P, reads D, and accumulates dK, dV and dlk.
// The extra recomputation (S and dP~ in both kernels: 7 instead of 5 tile
// products per pair) buys a fixed summation order for every output.

#include "gca_device.h"
#include "gca_launch.h"

namespace gca {

constexpr int kLdsStrideB = 72;  // bf16 per LDS tile row (64 + 8 pad)

template <int NTHREADS>
__device__ __forceinline__ void tile64_to_lds(bf16* dst, const bf16* __restrict__ src, int tid) {
#pragma unroll
  for (int r = 0; r < 512 / NTHREADS; ++r) {
    const int ch = tid + NTHREADS * r;
    const int row = ch >> 3, c8 = (ch & 7) * 8;
    *(bf16x8*)(dst + row * kLdsStrideB + c8) = *(const bf16x8*)(src + row * 64 + c8);
  }
}

// ---------------------------------------------------------------------------
// Reverse index.  One workgroup (256 threads, 4 waves) per head.
// rev_off[head][c] .. rev_off[head][c+1] delimit the entries (t*k + i) of key
// chunk c in rev_ent[head][...], in ascending entry order.  Out-of-range idx
// values are skipped.  Stable counting sort: the entries are cut into 4
// segments (one per wave); per pass over 512 key chunks, (segment, chunk)
// counts give every segment its own write cursor per chunk, and lane l of wave
// s appends, in entry order, the entries of segment s whose chunk is one of its
// 8 chunks.  Integer counts only, so the result does not depend on timing.
// ---------------------------------------------------------------------------
constexpr int kRevKeys = 512;  // key chunks per pass = 64 lanes x 8
constexpr int kRevSeg = 4;     // entry segments = waves

__global__ __launch_bounds__(256) void k_reverse_index(const int32_t* __restrict__ idx,
                                                       int64_t n_query, int64_t n_key, int topk,
                                                       int32_t* __restrict__ rev_off,
                                                       int32_t* __restrict__ rev_ent) {
  __shared__ int cnt[kRevSeg][kRevKeys];
  __shared__ int part[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t head = blockIdx.x;
  const int64_t n_ent = n_query * topk;
  const int64_t segsz = (n_ent + kRevSeg - 1) / kRevSeg;
  const int32_t* ih = idx + head * n_ent;
  int32_t* off = rev_off + head * (n_key + 1);
  int32_t* out = rev_ent + head * n_ent;
  int base = 0;
  for (int64_t c0 = 0; c0 < n_key; c0 += kRevKeys) {
    const int nc = (int)((n_key - c0) < kRevKeys ? (n_key - c0) : kRevKeys);
    for (int u = tid; u < kRevSeg * kRevKeys; u += 256) (&cnt[0][0])[u] = 0;
    __syncthreads();
    for (int64_t e = tid; e < n_ent; e += 256) {
      const int64_t c = ih[e];
      if (c >= c0 && c < c0 + nc) atomicAdd(&cnt[e / segsz][c - c0], 1);
    }
    __syncthreads();
    // thread owns chunks 2*tid, 2*tid+1: totals, then a block-wide exclusive scan
    int tot[2];
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int t = 0;
#pragma unroll
      for (int sg = 0; sg < kRevSeg; ++sg) t += cnt[sg][2 * tid + u];
      tot[u] = t;
      sum += t;
    }
    part[tid] = sum;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int add = tid >= o ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    const int total = part[255];
    int run = base + part[tid] - sum;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int key = 2 * tid + u;
      if (key < nc) off[c0 + key] = run;
      int cur = run;
#pragma unroll
      for (int sg = 0; sg < kRevSeg; ++sg) {
        const int cs = cnt[sg][key];
        cnt[sg][key] = cur;  // becomes the write cursor of (segment, chunk)
        cur += cs;
      }
      run += tot[u];
    }
    __syncthreads();
    int cur[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) cur[u] = cnt[wave][lane * 8 + u];
    const int64_t e_beg = wave * segsz;
    const int64_t e_end = (e_beg + segsz) < n_ent ? (e_beg + segsz) : n_ent;
    const int64_t my0 = c0 + lane * 8;
    for (int64_t e = e_beg; e < e_end; ++e) {
      const int64_t rel = (int64_t)ih[e] - my0;
      if (rel >= 0 && rel < 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (rel == u) out[cur[u]++] = (int)e;
      }
    }
    base += total;
    __syncthreads();
  }
  if (tid == 0) off[n_key] = base;
}

// Score / landmark epilogue of one query chunk, run by the whole workgroup.
// dw_slot[i] holds dw_i (only valid slots); writes dw, dscore and dlq.
template <typename LT>
__device__ void score_epilogue(int tid, int nthreads, int topk, const int* slot_c,
                               const float* wv, float* dw_slot, float* ds_slot,
                               float* __restrict__ dw_out, float* __restrict__ dscore_out,
                               const LT* __restrict__ lk_head, float* __restrict__ dlq_row,
                               int dl, float score_scale) {
  if (tid == 0) {
    float sw = 0.0f;
    for (int i = 0; i < topk; ++i)
      if (slot_c[i] >= 0) sw += wv[i] * dw_slot[i];
    for (int i = 0; i < topk; ++i) {
      const bool ok = slot_c[i] >= 0;
      ds_slot[i] = ok ? wv[i] * (dw_slot[i] - sw) : 0.0f;
      dw_out[i] = ok ? dw_slot[i] : 0.0f;
      dscore_out[i] = ds_slot[i];
    }
  }
  __syncthreads();
  if (dlq_row) {
    for (int d = tid; d < dl; d += nthreads) {
      float acc = 0.0f;
      for (int i = 0; i < topk; ++i)
        if (slot_c[i] >= 0) acc = fmaf(ds_slot[i], load_f(lk_head + (int64_t)slot_c[i] * dl + d), acc);
      dlq_row[d] = score_scale * acc;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 query-side backward (S = D = 64).  Two waves; wave w owns rows 32w..
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void k_bwd_q_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, const float* __restrict__ lse,
    const bf16* __restrict__ dout, const bf16* __restrict__ lk, bf16* __restrict__ dq,
    float* __restrict__ dw_out, float* __restrict__ dscore_out, float* __restrict__ dlq,
    float* __restrict__ delta, int64_t n_query, int64_t n_key, int topk, int dl,
    float attn_scale, float score_scale) {
  __shared__ bf16 k_lds[64 * kLdsStrideB];
  __shared__ bf16 v_lds[64 * kLdsStrideB];
  __shared__ float dw_part[2][16];
  __shared__ int slot_c[16];
  __shared__ float slot_w[16];
  __shared__ float dw_slot[16];
  __shared__ float ds_slot[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t head = tile / n_query;
  const int x = 32 * wave + col;

  if (tid < topk) {
    const int c = idx[tile * topk + tid];
    slot_c[tid] = (c >= 0 && c < n_key) ? c : -1;
    slot_w[tid] = w[tile * topk + tid];
  }
  bf16x8 bq[4], bdo[4];
  {
    const bf16* qr = q + tile * 4096 + x * 64 + 32 * half;
    const bf16* dr = dout + tile * 4096 + x * 64 + 32 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bq[ks] = *(const bf16x8*)(qr + 8 * ks);
      bdo[ks] = *(const bf16x8*)(dr + 8 * ks);
    }
  }
  f32x16 dqacc[2] = {zero16(), zero16()};
  const float c2 = attn_scale * kLog2e;
  __syncthreads();

  for (int i = 0; i < topk; ++i) {
    const int c = slot_c[i];
    float* drow = delta + (tile * topk + i) * 64;
    if (c < 0) {
      if (half == 0) drow[x] = 0.0f;
      if (lane == 0) dw_part[wave][i] = 0.0f;
      continue;
    }
    const float wi = slot_w[i];
    __syncthreads();
    tile64_to_lds<128>(k_lds, kk + (head * n_key + c) * 4096, tid);
    tile64_to_lds<128>(v_lds, v + (head * n_key + c) * 4096, tid);
    __syncthreads();
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = zero16();
      pacc[mt] = zero16();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = (32 * mt + col) * kLdsStrideB + 32 * half + 8 * ks;
        sacc[mt] = mfma32x32x16(*(const bf16x8*)(k_lds + off), bq[ks], sacc[mt]);
        pacc[mt] = mfma32x32x16(*(const bf16x8*)(v_lds + off), bdo[ks], pacc[mt]);
      }
    }
    const float l2 = lse[(tile * topk + i) * 64 + x] * kLog2e;
    float dsum = 0.0f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[mt][r], c2, -l2));
        sacc[mt][r] = p;
        dsum = fmaf(p, pacc[mt][r], dsum);
      }
    dsum += __shfl_xor(dsum, 32);
    if (half == 0) drow[x] = dsum;
    const float part = wave_sum(half == 0 ? dsum : 0.0f);
    if (lane == 0) dw_part[wave][i] = part;
    // dS^T = w P (dP~ - D), then dQ^T (d x x) += K^T (d x j) dS^T (j x x)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int mt = ks >> 1, g0 = 2 * (ks & 1);
      bf16x8 bs;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bs[e] = (bf16)(wi * sacc[mt][4 * g0 + e] * (pacc[mt][4 * g0 + e] - dsum));
        bs[4 + e] = (bf16)(wi * sacc[mt][4 * g0 + 4 + e] * (pacc[mt][4 * g0 + 4 + e] - dsum));
      }
      const int j0 = 16 * ks + 4 * half;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        bf16x8 ak;
        const bf16* kc = k_lds + 32 * dt + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ak[e] = kc[(j0 + e) * kLdsStrideB];
          ak[4 + e] = kc[(j0 + 8 + e) * kLdsStrideB];
        }
        dqacc[dt] = mfma32x32x16(ak, bs, dqacc[dt]);
      }
    }
  }
  bf16* dqrow = dq + tile * 4096 + x * 64;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = (bf16)(attn_scale * dqacc[dt][4 * g + e]);
      *(bf16x4*)(dqrow + 32 * dt + 8 * g + 4 * half) = val;
    }
  __syncthreads();
  if (tid < topk) dw_slot[tid] = dw_part[0][tid] + dw_part[1][tid];
  __syncthreads();
  score_epilogue<bf16>(tid, 128, topk, slot_c, slot_w, dw_slot, ds_slot, dw_out + tile * topk,
                       dscore_out + tile * topk, lk ? lk + head * n_key * dl : nullptr,
                       dlq ? dlq + tile * dl : nullptr, dl, score_scale);
}

// ---------------------------------------------------------------------------
// bf16 key-side backward (S = D = 64).  Two waves; wave w owns key rows 32w..
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void k_bwd_kv_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const float* __restrict__ w, const float* __restrict__ lse, const bf16* __restrict__ dout,
    const float* __restrict__ delta, const int32_t* __restrict__ rev_off,
    const int32_t* __restrict__ rev_ent, const bf16* __restrict__ lq,
    const float* __restrict__ dscore, bf16* __restrict__ dk, bf16* __restrict__ dv,
    float* __restrict__ dlk, int64_t n_query, int64_t n_key, int topk, int dl,
    float attn_scale, float score_scale) {
  __shared__ bf16 q_lds[64 * kLdsStrideB];
  __shared__ bf16 do_lds[64 * kLdsStrideB];
  __shared__ float l2_lds[64];
  __shared__ float d_lds[64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);  // = head * n_key + c
  const int64_t head = tile / n_key;
  const int64_t c = tile % n_key;
  const int j = 32 * wave + col;  // key row owned by this lane

  bf16x8 bk[4], bv[4];  // K_c^T and V_c^T as B operands: column j
  {
    const bf16* kr = kk + tile * 4096 + j * 64 + 32 * half;
    const bf16* vr = v + tile * 4096 + j * 64 + 32 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bk[ks] = *(const bf16x8*)(kr + 8 * ks);
      bv[ks] = *(const bf16x8*)(vr + 8 * ks);
    }
  }
  f32x16 dkacc[2] = {zero16(), zero16()};
  f32x16 dvacc[2] = {zero16(), zero16()};
  float dlk_acc = 0.0f;
  const float c2 = attn_scale * kLog2e;
  const int beg = rev_off[head * (n_key + 1) + c];
  const int end = rev_off[head * (n_key + 1) + c + 1];
  const int32_t* ents = rev_ent + head * n_query * topk;

  for (int e = beg; e < end; ++e) {
    const int ent = ents[e];
    const int64_t t = ent / topk;
    const int64_t pair = head * n_query * topk + ent;  // (head, t, i)
    const float wi = w[pair];
    __syncthreads();
    tile64_to_lds<128>(q_lds, q + (head * n_query + t) * 4096, tid);
    tile64_to_lds<128>(do_lds, dout + (head * n_query + t) * 4096, tid);
    if (tid < 64) {
      l2_lds[tid] = lse[pair * 64 + tid] * kLog2e;
      d_lds[tid] = delta[pair * 64 + tid];
    }
    if (lq && tid < dl)
      dlk_acc = fmaf(dscore[pair], (float)lq[(head * n_query + t) * dl + tid], dlk_acc);
    __syncthreads();
    // S (x x j) = Q K_c^T and dP~ (x x j) = dO V_c^T; lane holds column j.
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = zero16();
      pacc[mt] = zero16();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = (32 * mt + col) * kLdsStrideB + 32 * half + 8 * ks;
        sacc[mt] = mfma32x32x16(*(const bf16x8*)(q_lds + off), bk[ks], sacc[mt]);
        pacc[mt] = mfma32x32x16(*(const bf16x8*)(do_lds + off), bv[ks], pacc[mt]);
      }
    }
    // P_w = w P (kept in sacc) and dS = P_w (dP~ - D) (kept in pacc)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int xr = 32 * mt + c_row(r, half);
        const float pw = wi * fast_exp2(fmaf(sacc[mt][r], c2, -l2_lds[xr]));
        sacc[mt][r] = pw;
        pacc[mt][r] = pw * (pacc[mt][r] - d_lds[xr]);
      }
    // dV^T (d x j) += dO^T (d x x) P_w (x x j);  dK^T (d x j) += Q^T (d x x) dS (x x j)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int mt = ks >> 1, g0 = 2 * (ks & 1);
      bf16x8 bp, bs;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bp[e] = (bf16)sacc[mt][4 * g0 + e];
        bp[4 + e] = (bf16)sacc[mt][4 * g0 + 4 + e];
        bs[e] = (bf16)pacc[mt][4 * g0 + e];
        bs[4 + e] = (bf16)pacc[mt][4 * g0 + 4 + e];
      }
      const int x0 = 16 * ks + 4 * half;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        bf16x8 ado, aq;
        const bf16* dc = do_lds + 32 * dt + col;
        const bf16* qc = q_lds + 32 * dt + col;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ado[u] = dc[(x0 + u) * kLdsStrideB];
          ado[4 + u] = dc[(x0 + 8 + u) * kLdsStrideB];
          aq[u] = qc[(x0 + u) * kLdsStrideB];
          aq[4 + u] = qc[(x0 + 8 + u) * kLdsStrideB];
        }
        dvacc[dt] = mfma32x32x16(ado, bp, dvacc[dt]);
        dkacc[dt] = mfma32x32x16(aq, bs, dkacc[dt]);
      }
    }
  }
  bf16* dkrow = dk + tile * 4096 + j * 64;
  bf16* dvrow = dv + tile * 4096 + j * 64;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 kv4, vv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv4[e] = (bf16)(attn_scale * dkacc[dt][4 * g + e]);
        vv4[e] = (bf16)dvacc[dt][4 * g + e];
      }
      *(bf16x4*)(dkrow + 32 * dt + 8 * g + 4 * half) = kv4;
      *(bf16x4*)(dvrow + 32 * dt + 8 * g + 4 * half) = vv4;
    }
  if (dlk && tid < dl) dlk[tile * dl + tid] = score_scale * dlk_acc;
}

// ---------------------------------------------------------------------------
// float32 query-side backward: 64 threads per query chunk, thread x owns row x.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_bwd_q_f32(
    const float* __restrict__ q, const float* __restrict__ kk, const float* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, const float* __restrict__ lse,
    const float* __restrict__ dout, const float* __restrict__ lk, float* __restrict__ dq,
    float* __restrict__ dw_out, float* __restrict__ dscore_out, float* __restrict__ dlq,
    float* __restrict__ delta, int64_t n_query, int64_t n_key, int S, int D, int topk, int dl,
    float attn_scale, float score_scale) {
  __shared__ float kt[64 * 64];
  __shared__ float vt[64 * 64];
  __shared__ float pr[64 * 65];
  __shared__ float red[64];
  __shared__ int slot_c[16];
  __shared__ float slot_w[16];
  __shared__ float dw_slot[16];
  __shared__ float ds_slot[16];
  const int x = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int64_t head = tile / n_query;
  const int64_t tsz = (int64_t)S * D;
  const float* qrow = q + tile * tsz + (int64_t)x * D;
  const float* dorow = dout + tile * tsz + (int64_t)x * D;
  float* dqrow = dq + tile * tsz + (int64_t)x * D;
  if (x < topk) {
    const int c = idx[tile * topk + x];
    slot_c[x] = (c >= 0 && c < n_key) ? c : -1;
    slot_w[x] = w[tile * topk + x];
  }
  if (x < S)
    for (int d = 0; d < D; ++d) dqrow[d] = 0.0f;
  __syncthreads();
  for (int i = 0; i < topk; ++i) {
    const int c = slot_c[i];
    float* drow = delta + (tile * topk + i) * S;
    if (c < 0) {
      if (x < S) drow[x] = 0.0f;
      if (x == 0) dw_slot[i] = 0.0f;
      continue;
    }
    const float wi = slot_w[i];
    __syncthreads();
    const float* ks = kk + (head * n_key + c) * tsz;
    const float* vs = v + (head * n_key + c) * tsz;
    for (int e = x; e < S * D; e += 64) {
      kt[e] = ks[e];
      vt[e] = vs[e];
    }
    __syncthreads();
    float dsum = 0.0f;
    if (x < S) {
      float* p = pr + x * 65;
      const float lx = lse[(tile * topk + i) * S + x];
      for (int jj = 0; jj < S; ++jj) {
        float s = 0.0f, dp = 0.0f;
        for (int d = 0; d < D; ++d) {
          s = fmaf(qrow[d], kt[jj * D + d], s);
          dp = fmaf(dorow[d], vt[jj * D + d], dp);
        }
        const float pj = expf(s * attn_scale - lx);
        p[jj] = pj;
        dsum = fmaf(pj, dp, dsum);
      }
      drow[x] = dsum;
      for (int jj = 0; jj < S; ++jj) {
        float dp = 0.0f;
        for (int d = 0; d < D; ++d) dp = fmaf(dorow[d], vt[jj * D + d], dp);
        p[jj] = wi * p[jj] * (dp - dsum);
      }
      for (int d = 0; d < D; ++d) {
        float acc = 0.0f;
        for (int jj = 0; jj < S; ++jj) acc = fmaf(p[jj], kt[jj * D + d], acc);
        dqrow[d] += attn_scale * acc;
      }
    }
    red[x] = (x < S) ? dsum : 0.0f;
    __syncthreads();
    if (x == 0) {
      float t = 0.0f;
      for (int u = 0; u < S; ++u) t += red[u];
      dw_slot[i] = t;
    }
  }
  __syncthreads();
  score_epilogue<float>(x, 64, topk, slot_c, slot_w, dw_slot, ds_slot, dw_out + tile * topk,
                        dscore_out + tile * topk, lk ? lk + head * n_key * dl : nullptr,
                        dlq ? dlq + tile * dl : nullptr, dl, score_scale);
}

// ---------------------------------------------------------------------------
// float32 key-side backward: 64 threads per key chunk, thread j owns row j.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_bwd_kv_f32(
    const float* __restrict__ q, const float* __restrict__ kk, const float* __restrict__ v,
    const float* __restrict__ w, const float* __restrict__ lse, const float* __restrict__ dout,
    const float* __restrict__ delta, const int32_t* __restrict__ rev_off,
    const int32_t* __restrict__ rev_ent, const float* __restrict__ lq,
    const float* __restrict__ dscore, float* __restrict__ dk, float* __restrict__ dv,
    float* __restrict__ dlk, int64_t n_query, int64_t n_key, int S, int D, int topk, int dl,
    float attn_scale, float score_scale) {
  __shared__ float qt[64 * 64];
  __shared__ float dot[64 * 64];
  __shared__ float lx[64];
  __shared__ float dx[64];
  const int jj = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int64_t head = tile / n_key;
  const int64_t c = tile % n_key;
  const int64_t tsz = (int64_t)S * D;
  const float* krow = kk + tile * tsz + (int64_t)jj * D;
  const float* vrow = v + tile * tsz + (int64_t)jj * D;
  float* dkrow = dk + tile * tsz + (int64_t)jj * D;
  float* dvrow = dv + tile * tsz + (int64_t)jj * D;
  if (jj < S)
    for (int d = 0; d < D; ++d) {
      dkrow[d] = 0.0f;
      dvrow[d] = 0.0f;
    }
  float dlk_acc[2] = {0.0f, 0.0f};  // dl <= 128: thread covers d = jj and jj + 64
  const int beg = rev_off[head * (n_key + 1) + c];
  const int end = rev_off[head * (n_key + 1) + c + 1];
  const int32_t* ents = rev_ent + head * n_query * topk;
  for (int e = beg; e < end; ++e) {
    const int ent = ents[e];
    const int64_t t = ent / topk;
    const int64_t pair = head * n_query * topk + ent;
    const float wi = w[pair];
    __syncthreads();
    const float* qs = q + (head * n_query + t) * tsz;
    const float* ds = dout + (head * n_query + t) * tsz;
    for (int u = jj; u < S * D; u += 64) {
      qt[u] = qs[u];
      dot[u] = ds[u];
    }
    if (jj < S) {
      lx[jj] = lse[pair * S + jj];
      dx[jj] = delta[pair * S + jj];
    }
    if (lq) {
      const float dsc = dscore[pair];
      const float* lqr = lq + (head * n_query + t) * dl;
      if (jj < dl) dlk_acc[0] = fmaf(dsc, lqr[jj], dlk_acc[0]);
      if (jj + 64 < dl) dlk_acc[1] = fmaf(dsc, lqr[jj + 64], dlk_acc[1]);
    }
    __syncthreads();
    if (jj < S) {
      for (int xx = 0; xx < S; ++xx) {
        float s = 0.0f, dp = 0.0f;
        for (int d = 0; d < D; ++d) {
          s = fmaf(qt[xx * D + d], krow[d], s);
          dp = fmaf(dot[xx * D + d], vrow[d], dp);
        }
        const float pw = wi * expf(s * attn_scale - lx[xx]);
        const float dsv = pw * (dp - dx[xx]);
        for (int d = 0; d < D; ++d) {
          dvrow[d] = fmaf(pw, dot[xx * D + d], dvrow[d]);
          dkrow[d] = fmaf(attn_scale * dsv, qt[xx * D + d], dkrow[d]);
        }
      }
    }
  }
  if (dlk) {
    if (jj < dl) dlk[tile * dl + jj] = score_scale * dlk_acc[0];
    if (jj + 64 < dl) dlk[tile * dl + jj + 64] = score_scale * dlk_acc[1];
  }
}

hipError_t launch_backward(const LaunchBackward& a) {
  const int64_t heads = a.G * a.B * a.H;
  if (heads == 0) return hipSuccess;
  hipLaunchKernelGGL(k_reverse_index, dim3((unsigned)heads), dim3(256), 0, a.stream, a.idx,
                     a.n_query, a.n_key, a.k, a.rev_off, a.rev_ent);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t qtiles = heads * a.n_query, ktiles = heads * a.n_key;
  if (a.dtype == 1) {
    if (qtiles > 0)
      hipLaunchKernelGGL(k_bwd_q_bf16, dim3((unsigned)qtiles), dim3(128), 0, a.stream,
                         (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, a.idx, a.w,
                         a.lse, (const bf16*)a.dout, (const bf16*)a.lk, (bf16*)a.dq, a.dw,
                         a.dscore, a.dlq, a.delta, a.n_query, a.n_key, a.k, a.dl,
                         a.attn_scale, a.score_scale);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ktiles > 0)
      hipLaunchKernelGGL(k_bwd_kv_bf16, dim3((unsigned)ktiles), dim3(128), 0, a.stream,
                         (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, a.w, a.lse,
                         (const bf16*)a.dout, a.delta, a.rev_off, a.rev_ent, (const bf16*)a.lq,
                         a.dscore, (bf16*)a.dk, (bf16*)a.dv, a.dlk, a.n_query, a.n_key, a.k,
                         a.dl, a.attn_scale, a.score_scale);
  } else {
    if (qtiles > 0)
      hipLaunchKernelGGL(k_bwd_q_f32, dim3((unsigned)qtiles), dim3(64), 0, a.stream,
                         (const float*)a.q, (const float*)a.kk, (const float*)a.v, a.idx, a.w,
                         a.lse, (const float*)a.dout, (const float*)a.lk, (float*)a.dq, a.dw,
                         a.dscore, a.dlq, a.delta, a.n_query, a.n_key, a.S, a.D, a.k, a.dl,
                         a.attn_scale, a.score_scale);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ktiles > 0)
      hipLaunchKernelGGL(k_bwd_kv_f32, dim3((unsigned)ktiles), dim3(64), 0, a.stream,
                         (const float*)a.q, (const float*)a.kk, (const float*)a.v, a.w, a.lse,
                         (const float*)a.dout, a.delta, a.rev_off, a.rev_ent,
                         (const float*)a.lq, a.dscore, (float*)a.dk, (float*)a.dv, a.dlk,
                         a.n_query, a.n_key, a.S, a.D, a.k, a.dl, a.attn_scale, a.score_scale);
  }
  return hipGetLastError();
}

}  // namespace gca
