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

// ---------------------------------------------------------------------------
// Reverse index.  One workgroup (512 threads, 8 waves) per head.
// rev_off[head][c] .. rev_off[head][c+1] delimit the entries (t*k + i) of key
// chunk c in rev_ent[head][...], in ascending entry order.  Out-of-range idx
// values are skipped.  Stable counting sort with integer counts only:
//   1. the entries are cut into 8 segments, one per wave; per pass over 512
//      key chunks each wave counts the chunks of its segment (LDS atomics);
//   2. an exclusive scan over (chunk, segment) gives every segment its own
//      write cursor per chunk (a wave scan of the chunk totals, then the
//      8 wave sums through LDS);
//   3. each wave places its entries 64 at a time.  A lane's rank among the
//      earlier lanes with the same chunk comes from ten ballots, one per bit
//      of the chunk number within the pass (and one for "not in this pass"):
//      AND-ing each ballot or its complement, as the lane's own bit says,
//      leaves exactly the lanes whose chunk equals the lane's, and the
//      population count of that mask below the lane is the rank.  All lanes
//      write in parallel and the order inside each list is the entry order.
// RES: every segment has at most 512 entries, which stay in registers
// between the counting and the placing sweep (one read of idx).
// ---------------------------------------------------------------------------
constexpr int kRevWaves = 8;
constexpr int kRevKeys = 512;  // key chunks per pass = threads per workgroup
constexpr int kRevKeyBits = 10;  // bits of a chunk within a pass, plus "outside the pass"

template <bool RES>
__global__ __launch_bounds__(512) void k_reverse_index(const int32_t* __restrict__ idx,
                                                       int64_t n_query, int64_t n_key, int topk,
                                                       int32_t* __restrict__ rev_off,
                                                       int32_t* __restrict__ rev_ent) {
  static_assert((1 << (kRevKeyBits - 1)) == kRevKeys, "one bit above the chunk bits");
  __shared__ int cnt[kRevWaves][kRevKeys];
  __shared__ int wsum[kRevWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t head = blockIdx.x;
  const int n_ent = (int)(n_query * topk);  // < 2^31, checked on the host
  const int nk = (int)n_key;
  const int segsz = (n_ent + kRevWaves - 1) / kRevWaves;
  const int32_t* ih = idx + head * (int64_t)n_ent;
  int32_t* off = rev_off + head * (n_key + 1);
  int32_t* out = rev_ent + head * (int64_t)n_ent;
  const int e_beg = wave * segsz;
  const int e_end = min(e_beg + segsz, n_ent);
  int kres[8];  // RES: the segment (unconditional loads from clamped addresses)
  if (RES) {
#pragma unroll
    for (int r = 0; r < 8; ++r) kres[r] = ih[min(e_beg + 64 * r + lane, n_ent - 1)];
  }
  const uint64_t below = (1ull << lane) - 1;       // lanes before this one
  const uint64_t upto = (2ull << lane) - 1;        // ... and this one (all 64 for lane 63)
  int base = 0;
  for (int c0 = 0; c0 < nk; c0 += kRevKeys) {
    const int nc = min(kRevKeys, nk - c0);
#pragma unroll
    for (int w8 = 0; w8 < kRevWaves; ++w8) cnt[w8][tid] = 0;
    __syncthreads();
    for (int e0 = e_beg; e0 < e_end; e0 += 64 * 8) {
      int kv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) kv[r] = RES ? kres[r] : ih[min(e0 + 64 * r + lane, n_ent - 1)];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int rel = kv[r] - c0;
        if (e0 + 64 * r + lane < e_end && rel >= 0 && rel < nc) atomicAdd(&cnt[wave][rel], 1);
      }
    }
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w8 = 0; w8 < kRevWaves; ++w8) tot += cnt[w8][tid];
    int incl = tot;  // inclusive scan of the chunk totals across the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int pre = 0, total = 0;
#pragma unroll
    for (int w8 = 0; w8 < kRevWaves; ++w8) {
      const int ws = wsum[w8];
      pre += w8 < wave ? ws : 0;
      total += ws;
    }
    int cur = base + pre + incl - tot;
    if (tid < nc) off[c0 + tid] = cur;
#pragma unroll
    for (int w8 = 0; w8 < kRevWaves; ++w8) {
      const int cs = cnt[w8][tid];
      cnt[w8][tid] = cur;  // becomes the write cursor of (segment, chunk)
      cur += cs;
    }
    __syncthreads();
    for (int e0 = e_beg; e0 < e_end; e0 += 64 * 8) {
      int kv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) kv[r] = RES ? kres[r] : ih[min(e0 + 64 * r + lane, n_ent - 1)];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (e0 + 64 * r >= e_end) break;  // wave-uniform: all 64 lanes take part below
        const int e = e0 + 64 * r + lane;
        const int rel = kv[r] - c0;
        const bool inr = e < e_end && rel >= 0 && rel < nc;
        const unsigned key = inr ? (unsigned)rel : (unsigned)kRevKeys;
        uint64_t same = ~0ull;  // lanes whose key equals this lane's
#pragma unroll
        for (int bit = 0; bit < kRevKeyBits; ++bit) {
          const bool on = (key >> bit) & 1u;
          const uint64_t set = __ballot(on);
          same &= on ? set : ~set;
        }
        const int rank = __popcll(same & below);
        const bool later = (same & ~upto) != 0;
        if (inr) out[cnt[wave][rel] + rank] = e;
        if (inr && !later) cnt[wave][rel] += rank + 1;  // the last lane of the key advances
      }
    }
    base += total;
    __syncthreads();
  }
  if (tid == 0) off[n_key] = base;
}

// Score / landmark epilogue of one query chunk, run by a one-wave workgroup
// (lane = thread).  dw_slot[i] holds dw_i (only valid slots); writes dw,
// dscore and dlq (ACC: adds them to the float32 accumulators instead).  With
// no resident chunk (lk_head null) every slot is empty and dlq is 0.
template <typename LT, bool ACC>
__device__ void score_epilogue(int lane, int topk, const int* slot_c, const float* wv,
                               const float* dw_slot, float* ds_slot, float* __restrict__ dw_out,
                               float* __restrict__ dscore_out, float* __restrict__ ds_layer,
                               const LT* __restrict__ lk_head, float* __restrict__ dlq_row,
                               int dl, float score_scale) {
  const int i = lane < topk ? lane : 0;
  const bool ok = lane < topk && slot_c[i] >= 0;
  const float ds = slot_dscore<ACC>(lane, topk, ok, wv[i], dw_slot[i], dw_out, dscore_out,
                                    ds_layer);
  if (lane < topk) ds_slot[lane] = ds;
  __syncthreads();
  if (dlq_row && !lk_head) {
    if (!ACC)
      for (int d = lane; d < dl; d += 64) dlq_row[d] = 0.0f;
  } else if (dlq_row) {
    for (int d = lane; d < dl; d += 64) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i >= topk) break;
        // empty slots have ds_slot = 0; chunk 0 stands in so every load is issued
        const int c = slot_c[i] >= 0 ? slot_c[i] : 0;
        acc = fmaf(ds_slot[i], load_f(lk_head + (int64_t)c * dl + d), acc);
      }
      put<ACC>(dlq_row + d, score_scale * acc);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 query-side backward (S = 64, D = 64 or 32).  Four waves; wave w owns
// query rows 16w .. 16w+15 on 16x16x32 MFMA tiles.  The next valid slot's K and V tiles
// stream into the other half of a double-buffered swizzled LDS area while the
// current slot is computed (asynchronous copies the compiler does not wait
// on; the slot loop is unrolled by two so both buffers are fixed addresses).
// ---------------------------------------------------------------------------
template <int D>
struct BwdQCtx {
  const TileDma<4, D>* dma;
  const bf16* k_head;
  const bf16* v_head;
  const int* slot_c;   // LDS: chunk of each slot
  const float* slot_w; // LDS: its weight
  float (*dw_part)[16];  // LDS [4][16]
  const float* lse_row;  // lse + tile * topk * 64 + x
  float* s_delta;        // LDS [16][64]: D rows, written out at the end
  int x;
  int n, lane, wave, grp, col;
  float c2;
};

template <int D>
__device__ __forceinline__ void bwdq_issue(const BwdQCtx<D>& cx, int i, bf16* __restrict__ kd,
                                           bf16* __restrict__ vd) {
  const int64_t c = uniform(cx.slot_c[i]);
  cx.dma->copy_async(kd, cx.k_head + c * (64 * D));
  cx.dma->copy_async(vd, cx.v_head + c * (64 * D));
}

template <int D>
__device__ __forceinline__ void bwdq_slot(const BwdQCtx<D>& cx, int i, int nx, float& l2_next,
                                          const bf16x8 (&bq)[D / 32], const bf16x8 (&bdo)[D / 32],
                                          f32x4 (&dqacc)[D / 16], const bf16* __restrict__ kt,
                                          const bf16* __restrict__ vt, bf16* __restrict__ kn,
                                          bf16* __restrict__ vn) {
  const int lane = cx.lane, grp = cx.grp, col = cx.col;
  const float wi = cx.slot_w[i];
  wait_vmem();
  __syncthreads();
  // the next slot's log-sum-exp row is loaded raw and scaled only here, after
  // the wait: using it earlier would drain the tile copies issued with it
  // P_w = w P comes out of the exponential directly: log2 w joins the row's
  // offset (w = 0 gives P_w = 0 through exp2(-inf)).
  const float l2 = l2_next * kLog2e - __builtin_amdgcn_logf(wi);
  if (nx >= 0) {
    bwdq_issue(cx, nx, kn, vn);
    l2_next = cx.lse_row[nx * 64];
  }
  // S^T = K Q^T and dP~^T = V dO^T per key tile mt; lane holds keys 16mt + 4grp + r.
  f32x4 sacc[4], pacc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    sacc[mt] = zero4();
    pacc[mt] = zero4();
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) {
      sacc[mt] = mfma16x16x32(lds_row8<D>(kt, 16 * mt + col, 4 * kd + grp), bq[kd], sacc[mt]);
      pacc[mt] = mfma16x16x32(lds_row8<D>(vt, 16 * mt + col, 4 * kd + grp), bdo[kd], pacc[mt]);
    }
  }
  // K^T operands of this slot, requested now so that the LDS latency overlaps
  // the elementwise arithmetic below.
  bf16x8 ka[2][D / 16];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      ka[kb][dt] =
          lds_tr_operand16<D>(kt, 16 * dt, 32 * kb + 4 * grp, 32 * kb + 16 + 4 * grp, lane);
  float dp[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    dp[mt] = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = fast_exp2(fmaf(sacc[mt][r], cx.c2, -l2));  // = w P
      sacc[mt][r] = p;
      dp[mt] = fmaf(p, pacc[mt][r], dp[mt]);
    }
  }
  // D = rowsum(P dP~) = rowsum(P_w dP~) / w  (0 when w = 0: P_w is 0 there)
  const float dsw = xor32_sum(xor16_sum((dp[0] + dp[1]) + (dp[2] + dp[3])));
  const float dsum = wi > 0.0f ? dsw * fast_rcp(wi) : 0.0f;
  if (grp == 0) cx.s_delta[i * 64 + cx.x] = dsum;
  const float part = row16_sum(dsum);  // the 16 query rows of this wave
  if (lane == 0) cx.dw_part[cx.wave][i] = part;
  // dS^T = w P (dP~ - D); dQ^T (d x x) += K^T (d x j) dS^T (j x x)
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bf16x8 bs;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bs[e] = (bf16)(sacc[2 * kb][e] * (pacc[2 * kb][e] - dsum));
      bs[4 + e] = (bf16)(sacc[2 * kb + 1][e] * (pacc[2 * kb + 1][e] - dsum));
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) dqacc[dt] = mfma16x16x32(ka[kb][dt], bs, dqacc[dt]);
  }
}

template <int D, bool ACC>
__global__ __launch_bounds__(256, 4) void k_bwd_q_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, const float* __restrict__ lse,
    const bf16* __restrict__ dout, const bf16* __restrict__ lk, bf16* __restrict__ dq,
    float* __restrict__ dw_out, float* __restrict__ dscore_out, float* __restrict__ dlq,
    float* __restrict__ delta, float* __restrict__ ds_layer, int64_t n_query, int64_t n_key,
    int topk, int dl, float attn_scale, float score_scale) {
  __shared__ __align__(16) bf16 k_lds[2][64 * D];
  __shared__ __align__(16) bf16 v_lds[2][64 * D];
  __shared__ float dw_part[4][16];
  __shared__ int slot_c[16];
  __shared__ float slot_w[16];
  __shared__ float ds_slot[16];
  __shared__ int s_n;
  __shared__ int s_mask;
  // D rows of the k slots, staged here and stored once at the end: a store per
  // slot would be waited on by the next slot's copy wait.
  __shared__ float s_delta[16 * 64];
  // landmark rows lk[c_i] of the k slots for dlq, copied in with slot 0's tiles
  __shared__ __align__(16) bf16 lk_lds[16 * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t head = tile / n_query;
  const int x = 16 * wave + col;
  for (int e = tid; e < topk * 64; e += 256) s_delta[e] = 0.0f;  // empty slots

  if (wave == 0) {  // slot table and the ballot of the valid slots, in one step
    const int i = lane < topk ? lane : 0;
    const int c = idx[tile * topk + i];
    const float wv = w[tile * topk + i];
    const bool ok = lane < topk && c >= 0 && c < n_key;
    const uint64_t mask = __ballot(ok);
    if (lane < topk) {
      slot_c[lane] = ok ? c : -1;
      slot_w[lane] = wv;
    }
    if (lane == 0) {
      s_n = __popcll(mask);
      s_mask = (int)mask;
    }
  }
  if (tid < 64) dw_part[tid >> 4][tid & 15] = 0.0f;
  bf16x8 bq[D / 32], bdo[D / 32];  // Q^T and dO^T as B operands: column x, dims 32kd + 8grp + 0..7
  {
    const bf16* qr = q + tile * (64 * D) + x * D + 8 * grp;
    const bf16* dr = dout + tile * (64 * D) + x * D + 8 * grp;
#pragma unroll
    for (int kd = 0; kd < D / 32; ++kd) {
      bq[kd] = *(const bf16x8*)(qr + 32 * kd);
      bdo[kd] = *(const bf16x8*)(dr + 32 * kd);
    }
  }
  f32x4 dqacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) dqacc[dt] = zero4();
  const TileDma<4, D> dma(wave, lane);
  BwdQCtx<D> cx;
  cx.dma = &dma;
  cx.k_head = kk + head * n_key * (64 * D);
  cx.v_head = v + head * n_key * (64 * D);
  cx.slot_c = slot_c;
  cx.slot_w = slot_w;
  cx.dw_part = dw_part;
  cx.lse_row = lse + tile * topk * 64 + x;
  cx.s_delta = s_delta;
  cx.x = x;
  cx.lane = lane;
  cx.wave = wave;
  cx.grp = grp;
  cx.col = col;
  cx.c2 = attn_scale * kLog2e;
  __syncthreads();
  const int n = uniform(s_n);
  const uint32_t vmask = (uint32_t)uniform(s_mask);  // bit i: slot i valid
  cx.n = n;
  float l2_next = 0.0f;
  int i = vmask ? (int)__builtin_ctz(vmask) : -1;  // slot of the u-th valid one
  if (n > 0) {
    bwdq_issue(cx, i, k_lds[0], v_lds[0]);
    if (dlq && lk && wave < dl / 32) {
      // 16-byte piece e of the 16 x dl row block: row e / (dl / 8); rows of empty
      // slots and past topk take chunk 0 (their dscore is 0 or they are not read)
      const int e = wave * 64 + lane, r = e / (dl / 8);
      const int c = r < topk && slot_c[r] >= 0 ? slot_c[r] : 0;
      copy16_async(lk_lds + wave * 512, lk + (head * n_key + c) * dl + (e % (dl / 8)) * 8);
    }
    l2_next = cx.lse_row[i * 64];
  }
  for (int u = 0; u < n; u += 2) {
    int nx = next_slot(vmask, i);
    bwdq_slot(cx, i, nx, l2_next, bq, bdo, dqacc, k_lds[0], v_lds[0], k_lds[1], v_lds[1]);
    i = nx;
    if (u + 1 < n) {
      nx = next_slot(vmask, i);
      bwdq_slot(cx, i, nx, l2_next, bq, bdo, dqacc, k_lds[1], v_lds[1], k_lds[0], v_lds[0]);
      i = nx;
    }
  }
  // the row offset is formed again here from an opaque copy of the thread
  // index, so the compiler does not keep it live across the slot loop
  int t2 = tid;
  asm volatile("" : "+v"(t2));
  bf16* dqrow = dq + tile * (64 * D) + (16 * (t2 >> 6) + (t2 & 15)) * D + 4 * ((t2 & 63) >> 4);
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    bf16x4 val;
#pragma unroll
    for (int e = 0; e < 4; ++e) val[e] = (bf16)(attn_scale * dqacc[dt][e]);
    *(bf16x4*)(dqrow + 16 * dt) = val;
  }
  __syncthreads();
  for (int e = tid; e < topk * 64; e += 256) delta[tile * topk * 64 + e] = s_delta[e];
  if (wave == 0) {  // lane i: slot i
    const int i = lane < topk ? lane : 0;
    const float dwi = (dw_part[0][i] + dw_part[1][i]) + (dw_part[2][i] + dw_part[3][i]);
    const float ds = slot_dscore<ACC>(lane, topk, lane < topk && slot_c[i] >= 0, slot_w[i], dwi,
                                      dw_out + tile * topk, dscore_out + tile * topk,
                                      ACC ? ds_layer + tile * topk : nullptr);
    if (lane < topk) ds_slot[lane] = ds;
  }
  __syncthreads();
  // dlq = score_scale sum_i dscore_i lk[c_i] from the staged rows (0 with no
  // valid slot; ACC then adds nothing where lk is absent)
  if (dlq && tid < dl) {
    float acc = 0.0f;
    if (lk && s_n > 0)
      for (int i = 0; i < topk; ++i) acc = fmaf(ds_slot[i], (float)lk_lds[i * dl + tid], acc);
    if (lk || !ACC) put<ACC>(dlq + tile * dl + tid, score_scale * acc);
  }
}

// ---------------------------------------------------------------------------
// bf16 key-side backward (S = 64, D = 64 or 32).  Four waves; wave w owns key rows
// 16w .. 16w+15 on 16x16x32 MFMA tiles.  The reverse-list entries are staged
// in LDS 256 at a time; the next entry's Q and dO tiles stream into the other
// half of a double-buffered swizzled LDS area (asynchronous copies) and its
// log-sum-exp / D rows and scalars into registers while the current entry is
// computed.  The 64 query rows of a pair are processed as two 32-row
// contraction steps; the entry loop is unrolled by two so both buffers are
// fixed LDS addresses.
// ---------------------------------------------------------------------------
template <int D>
struct BwdKVCtx {
  const TileDma<4, D>* dma;
  const bf16* q_head;     // q + head * n_query * 64 * D
  const bf16* do_head;    // dout + head * n_query * 64 * D
  const float* lse_head;  // lse + pair0 * 64
  const float* d_head;    // delta + pair0 * 64
  const float* w_head;    // w + pair0
  const float* ds_head;   // dscore + pair0
  const bf16* lq_head;    // lq + head * n_query * dl, or NULL
  const int* s_ent;       // LDS
  int topk, dl, tid, lane, grp, col;
  float c2;
};

// Registers that carry one entry's scalars from its fetch to its use, raw as
// loaded: converting them at fetch time would make the compiler wait for the
// loads there, and with them for the tile copies issued just before.
struct KVNext {
  float row, w, ds;
  bf16 lq;
};

template <int D>
__device__ __forceinline__ void bwdkv_fetch(const BwdKVCtx<D>& cx, int u, KVNext& nx,
                                            bf16* __restrict__ qd, bf16* __restrict__ dod) {
  const int ent = uniform(cx.s_ent[u]);
  const int t = ent / cx.topk;
  cx.dma->copy_async(qd, cx.q_head + (int64_t)t * (64 * D));
  cx.dma->copy_async(dod, cx.do_head + (int64_t)t * (64 * D));
  const int tid = cx.tid;
  if (tid < 128)
    nx.row = tid < 64 ? cx.lse_head[(int64_t)ent * 64 + tid]
                      : cx.d_head[(int64_t)ent * 64 + (tid - 64)];
  nx.w = cx.w_head[ent];
  if (cx.lq_head && tid < 64) {  // wave 0 carries dlk (dl <= 64)
    nx.ds = cx.ds_head[ent];
    nx.lq = cx.lq_head[(int64_t)t * cx.dl + (tid < cx.dl ? tid : 0)];
  }
}

template <int D>
__device__ __forceinline__ void bwdkv_entry(const BwdKVCtx<D>& cx, int u, int nb, KVNext& nx,
                                            float& dlk_acc, const bf16x8 (&bk)[D / 32],
                                            const bf16x8 (&bv)[D / 32], f32x4 (&dkacc)[D / 16],
                                            f32x4 (&dvacc)[D / 16], const bf16* __restrict__ qt,
                                            const bf16* __restrict__ dot, float* __restrict__ l2r,
                                            float* __restrict__ dr, bf16* __restrict__ qn,
                                            bf16* __restrict__ don) {
  const int lane = cx.lane, grp = cx.grp, col = cx.col, tid = cx.tid;
  wait_vmem();
  // P_w = w P comes out of the exponential directly: log2 w joins the row
  // offset (w = 0 gives P_w = 0 through exp2(-inf)).
  if (tid < 64)
    l2r[tid] = nx.row * kLog2e - __builtin_amdgcn_logf(nx.w);
  else if (tid < 128)
    dr[tid - 64] = nx.row;
  if (cx.lq_head && tid < cx.dl) dlk_acc = fmaf(nx.ds, (float)nx.lq, dlk_acc);
  __syncthreads();
  if (u + 1 < nb) bwdkv_fetch(cx, u + 1, nx, qn, don);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // S (x x j) = Q K_c^T and dP~ = dO V_c^T for query tiles 2kb, 2kb+1;
    // the lane holds rows x = 32kb + 16h + 4grp + r of its key column j.
    f32x4 sacc[2], pacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int xr = 32 * kb + 16 * h + col;
      sacc[h] = zero4();
      pacc[h] = zero4();
#pragma unroll
      for (int kd = 0; kd < D / 32; ++kd) {
        sacc[h] = mfma16x16x32(lds_row8<D>(qt, xr, 4 * kd + grp), bk[kd], sacc[h]);
        pacc[h] = mfma16x16x32(lds_row8<D>(dot, xr, 4 * kd + grp), bv[kd], pacc[h]);
      }
      // P_w = w P (kept in sacc) and dS = P_w (dP~ - D) (kept in pacc)
      const int x0 = 32 * kb + 16 * h + 4 * grp;
      const f32x4 l4 = *(const f32x4*)(l2r + x0);
      const f32x4 d4 = *(const f32x4*)(dr + x0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pw = fast_exp2(fmaf(sacc[h][e], cx.c2, -l4[e]));
        sacc[h][e] = pw;
        pacc[h][e] = pw * (pacc[h][e] - d4[e]);
      }
    }
    // dV^T (d x j) += dO^T (d x x) P_w (x x j);  dK^T (d x j) += Q^T (d x x) dS (x x j)
    bf16x8 bp, bs;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bp[e] = (bf16)sacc[0][e];
      bp[4 + e] = (bf16)sacc[1][e];
      bs[e] = (bf16)pacc[0][e];
      bs[4 + e] = (bf16)pacc[1][e];
    }
    // dO^T and Q^T operands, read right before their products: holding all
    // eight across the arithmetic above would need 32 more registers, and at
    // 128 registers four workgroups share a CU, whose other waves cover the
    // LDS latency.
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const bf16x8 ado =
          lds_tr_operand16<D>(dot, 16 * dt, 32 * kb + 4 * grp, 32 * kb + 16 + 4 * grp, lane);
      const bf16x8 aq =
          lds_tr_operand16<D>(qt, 16 * dt, 32 * kb + 4 * grp, 32 * kb + 16 + 4 * grp, lane);
      dvacc[dt] = mfma16x16x32(ado, bp, dvacc[dt]);
      dkacc[dt] = mfma16x16x32(aq, bs, dkacc[dt]);
    }
  }
}


// ACC: dk and dv are float32 accumulators that this layer's gradients are
// added to (in place of bf16 outputs), dlk likewise.
template <int D, bool ACC>
__global__ __launch_bounds__(256, 4) void k_bwd_kv_bf16(
    const bf16* __restrict__ q, const bf16* __restrict__ kk, const bf16* __restrict__ v,
    const float* __restrict__ w, const float* __restrict__ lse, const bf16* __restrict__ dout,
    const float* __restrict__ delta, const int32_t* __restrict__ rev_off,
    const int32_t* __restrict__ rev_ent, const bf16* __restrict__ lq,
    const float* __restrict__ dscore, void* __restrict__ dk, void* __restrict__ dv,
    float* __restrict__ dlk, int64_t n_query, int64_t n_key, int topk, int dl,
    float attn_scale, float score_scale) {
  __shared__ __align__(16) bf16 q_lds[2][64 * D];
  __shared__ __align__(16) bf16 do_lds[2][64 * D];
  __shared__ __align__(16) float l2_lds[2][64];
  __shared__ __align__(16) float d_lds[2][64];
  __shared__ int s_ent[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  // = head * n_key + c
  const int64_t tile = kv_tile_order(xcd_tile(blockIdx.x, gridDim.x), n_key, gridDim.x);
  const int64_t head = tile / n_key;
  const int64_t c = tile % n_key;
  const int j = 16 * wave + col;  // key row owned by this lane

  bf16x8 bk[D / 32], bv[D / 32];  // K_c^T and V_c^T as B operands: column j, dims 32kd + 8grp + 0..7
  {
    const bf16* kr = kk + tile * (64 * D) + j * D + 8 * grp;
    const bf16* vr = v + tile * (64 * D) + j * D + 8 * grp;
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
  const TileDma<4, D> dma(wave, lane);
  BwdKVCtx<D> cx;
  cx.dma = &dma;
  cx.q_head = q + head * n_query * (64 * D);
  cx.do_head = dout + head * n_query * (64 * D);
  cx.lse_head = lse + pair0 * 64;
  cx.d_head = delta + pair0 * 64;
  cx.w_head = w + pair0;
  cx.ds_head = dscore + pair0;
  cx.lq_head = lq ? lq + head * n_query * dl : nullptr;
  cx.s_ent = s_ent;
  cx.topk = topk;
  cx.dl = dl;
  cx.tid = tid;
  cx.lane = lane;
  cx.grp = grp;
  cx.col = col;
  cx.c2 = attn_scale * kLog2e;

  for (int b0 = beg; b0 < end; b0 += 256) {
    const int nb = (end - b0) < 256 ? (end - b0) : 256;
    __syncthreads();  // every wave is done with the previous block
    if (tid < nb) s_ent[tid] = ents[b0 + tid];
    __syncthreads();
    KVNext nx{0.0f, 0.0f, 0.0f, (bf16)0.0f};
    bwdkv_fetch(cx, 0, nx, q_lds[0], do_lds[0]);
    for (int u = 0; u < nb; u += 2) {
      bwdkv_entry(cx, u, nb, nx, dlk_acc, bk, bv, dkacc, dvacc, q_lds[0], do_lds[0], l2_lds[0],
                  d_lds[0], q_lds[1], do_lds[1]);
      if (u + 1 < nb)
        bwdkv_entry(cx, u + 1, nb, nx, dlk_acc, bk, bv, dkacc, dvacc, q_lds[1], do_lds[1],
                    l2_lds[1], d_lds[1], q_lds[0], do_lds[0]);
    }
  }
  const int64_t orow = tile * (64 * D) + j * D + 4 * grp;
  if (ACC) {
    f32x4* dka = (f32x4*)((float*)dk + orow);
    f32x4* dva = (f32x4*)((float*)dv + orow);
    f32x4 ka[D / 16], va[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      ka[dt] = dka[4 * dt];
      va[dt] = dva[4 * dt];
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ka[dt][e] += attn_scale * dkacc[dt][e];
        va[dt][e] += dvacc[dt][e];
      }
      dka[4 * dt] = ka[dt];
      dva[4 * dt] = va[dt];
    }
  } else {
    bf16* dkrow = (bf16*)dk + orow;
    bf16* dvrow = (bf16*)dv + orow;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      bf16x4 kv4, vv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv4[e] = (bf16)(attn_scale * dkacc[dt][e]);
        vv4[e] = (bf16)dvacc[dt][e];
      }
      *(bf16x4*)(dkrow + 16 * dt) = kv4;
      *(bf16x4*)(dvrow + 16 * dt) = vv4;
    }
  }
  if (dlk && tid < dl) put<ACC>(dlk + tile * dl + tid, score_scale * dlk_acc);
}

// ---------------------------------------------------------------------------
// Generic query-side backward (any S, D <= 64; float32 or bf16 elements): 64
// threads per query chunk, thread x owns row x; float32 arithmetic, dQ
// accumulated in registers and rounded to the element type once.
// ---------------------------------------------------------------------------
template <typename T, bool ACC>
__global__ __launch_bounds__(64) void k_bwd_q_gen(
    const T* __restrict__ q, const T* __restrict__ kk, const T* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ w, const float* __restrict__ lse,
    const T* __restrict__ dout, const T* __restrict__ lk, T* __restrict__ dq,
    float* __restrict__ dw_out, float* __restrict__ dscore_out, float* __restrict__ dlq,
    float* __restrict__ delta, float* __restrict__ ds_layer, int64_t n_query, int64_t n_key,
    int S, int D, int topk, int dl, float attn_scale, float score_scale) {
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
  const T* qrow = q + tile * tsz + (int64_t)x * D;
  const T* dorow = dout + tile * tsz + (int64_t)x * D;
  if (x < topk) {
    const int c = idx[tile * topk + x];
    slot_c[x] = (c >= 0 && c < n_key) ? c : -1;
    slot_w[x] = w[tile * topk + x];
  }
  float dqa[64];
#pragma unroll
  for (int d = 0; d < 64; ++d) dqa[d] = 0.0f;
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
    const T* ks = kk + (head * n_key + c) * tsz;
    const T* vs = v + (head * n_key + c) * tsz;
    for (int e = x; e < S * D; e += 64) {
      kt[e] = load_f(ks + e);
      vt[e] = load_f(vs + e);
    }
    __syncthreads();
    float dsum = 0.0f;
    if (x < S) {
      float* p = pr + x * 65;
      const float lx = lse[(tile * topk + i) * S + x];
      for (int jj = 0; jj < S; ++jj) {
        float sv = 0.0f, dp = 0.0f;
        for (int d = 0; d < D; ++d) {
          sv = fmaf(load_f(qrow + d), kt[jj * D + d], sv);
          dp = fmaf(load_f(dorow + d), vt[jj * D + d], dp);
        }
        const float pj = expf(sv * attn_scale - lx);
        p[jj] = pj;
        dsum = fmaf(pj, dp, dsum);
      }
      drow[x] = dsum;
      for (int jj = 0; jj < S; ++jj) {
        float dp = 0.0f;
        for (int d = 0; d < D; ++d) dp = fmaf(load_f(dorow + d), vt[jj * D + d], dp);
        p[jj] = wi * p[jj] * (dp - dsum);
      }
#pragma unroll
      for (int d = 0; d < 64; ++d) {
        if (d < D) {
          float acc = 0.0f;
          for (int jj = 0; jj < S; ++jj) acc = fmaf(p[jj], kt[jj * D + d], acc);
          dqa[d] = fmaf(attn_scale, acc, dqa[d]);
        }
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
  if (x < S) {
    T* dqrow = dq + tile * tsz + (int64_t)x * D;
#pragma unroll
    for (int d = 0; d < 64; ++d)
      if (d < D) store_f(dqrow + d, dqa[d]);
  }
  __syncthreads();
  score_epilogue<T, ACC>(x, topk, slot_c, slot_w, dw_slot, ds_slot, dw_out + tile * topk,
                         dscore_out + tile * topk, ACC ? ds_layer + tile * topk : nullptr,
                         lk ? lk + head * n_key * dl : nullptr, dlq ? dlq + tile * dl : nullptr,
                         dl, score_scale);
}

// ---------------------------------------------------------------------------
// Generic key-side backward (any S, D <= 64; float32 or bf16 elements): 64
// threads per key chunk, thread j owns row j; dK and dV accumulated in
// registers (ACC: on top of the float32 accumulators) and stored once.
// ---------------------------------------------------------------------------
template <typename T, bool ACC>
__global__ __launch_bounds__(64) void k_bwd_kv_gen(
    const T* __restrict__ q, const T* __restrict__ kk, const T* __restrict__ v,
    const float* __restrict__ w, const float* __restrict__ lse, const T* __restrict__ dout,
    const float* __restrict__ delta, const int32_t* __restrict__ rev_off,
    const int32_t* __restrict__ rev_ent, const T* __restrict__ lq,
    const float* __restrict__ dscore, void* __restrict__ dk, void* __restrict__ dv,
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
  const T* krow = kk + tile * tsz + (int64_t)jj * D;
  const T* vrow = v + tile * tsz + (int64_t)jj * D;
  // ACC: dk, dv are float32 accumulators; else element-type outputs
  float* dka_out = ACC ? (float*)dk + tile * tsz + (int64_t)jj * D : nullptr;
  float* dva_out = ACC ? (float*)dv + tile * tsz + (int64_t)jj * D : nullptr;
  float dka[64], dva[64];
#pragma unroll
  for (int d = 0; d < 64; ++d) {
    dka[d] = (ACC && jj < S && d < D) ? dka_out[d] : 0.0f;
    dva[d] = (ACC && jj < S && d < D) ? dva_out[d] : 0.0f;
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
    const T* qs = q + (head * n_query + t) * tsz;
    const T* ds = dout + (head * n_query + t) * tsz;
    for (int u = jj; u < S * D; u += 64) {
      qt[u] = load_f(qs + u);
      dot[u] = load_f(ds + u);
    }
    if (jj < S) {
      lx[jj] = lse[pair * S + jj];
      dx[jj] = delta[pair * S + jj];
    }
    if (lq) {
      const float dsc = dscore[pair];
      const T* lqr = lq + (head * n_query + t) * dl;
      if (jj < dl) dlk_acc[0] = fmaf(dsc, load_f(lqr + jj), dlk_acc[0]);
      if (jj + 64 < dl) dlk_acc[1] = fmaf(dsc, load_f(lqr + jj + 64), dlk_acc[1]);
    }
    __syncthreads();
    if (jj < S) {
      for (int xx = 0; xx < S; ++xx) {
        float sv = 0.0f, dp = 0.0f;
        for (int d = 0; d < D; ++d) {
          sv = fmaf(qt[xx * D + d], load_f(krow + d), sv);
          dp = fmaf(dot[xx * D + d], load_f(vrow + d), dp);
        }
        const float pw = wi * expf(sv * attn_scale - lx[xx]);
        const float dsv = pw * (dp - dx[xx]);
#pragma unroll
        for (int d = 0; d < 64; ++d) {
          if (d < D) {
            dva[d] = fmaf(pw, dot[xx * D + d], dva[d]);
            dka[d] = fmaf(attn_scale * dsv, qt[xx * D + d], dka[d]);
          }
        }
      }
    }
  }
  if (jj < S) {
    if (ACC) {
#pragma unroll
      for (int d = 0; d < 64; ++d) {
        if (d < D) {
          dka_out[d] = dka[d];
          dva_out[d] = dva[d];
        }
      }
    } else {
      T* dkrow = (T*)dk + tile * tsz + (int64_t)jj * D;
      T* dvrow = (T*)dv + tile * tsz + (int64_t)jj * D;
#pragma unroll
      for (int d = 0; d < 64; ++d) {
        if (d < D) {
          store_f(dkrow + d, dka[d]);
          store_f(dvrow + d, dva[d]);
        }
      }
    }
  }
  if (dlk) {
    if (jj < dl) put<ACC>(dlk + tile * dl + jj, score_scale * dlk_acc[0]);
    if (jj + 64 < dl) put<ACC>(dlk + tile * dl + jj + 64, score_scale * dlk_acc[1]);
  }
}

template <typename T>
static hipError_t launch_backward_gen(const LaunchBackward& a, int64_t qtiles, int64_t ktiles) {
  hipError_t err;
  if (qtiles > 0) {
    KernelTimer timer(kKernBackwardQ, a.stream);
    auto kern = a.accumulate ? k_bwd_q_gen<T, true> : k_bwd_q_gen<T, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)qtiles), dim3(64), 0, a.stream, (const T*)a.q,
                       (const T*)a.kk, (const T*)a.v, a.idx, a.w, a.lse, (const T*)a.dout,
                       (const T*)a.lk, (T*)a.dq, a.dw, a.dscore, a.dlq, a.delta, a.ds_layer,
                       a.n_query, a.n_key, a.S, a.D, a.k, a.dl, a.attn_scale, a.score_scale);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ktiles > 0) {
    KernelTimer timer(kKernBackwardKV, a.stream);
    auto kern = a.accumulate ? k_bwd_kv_gen<T, true> : k_bwd_kv_gen<T, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)ktiles), dim3(64), 0, a.stream, (const T*)a.q,
                       (const T*)a.kk, (const T*)a.v, a.w, a.lse, (const T*)a.dout, a.delta,
                       a.rev_off, a.rev_ent, (const T*)a.lq, a.accumulate ? a.ds_layer : a.dscore,
                       a.dk, a.dv, a.dlk, a.n_query, a.n_key, a.S, a.D, a.k, a.dl, a.attn_scale,
                       a.score_scale);
  }
  return hipGetLastError();
}

hipError_t launch_backward(const LaunchBackward& a) {
  const int64_t heads = a.G * a.B * a.H;
  if (heads == 0) return hipSuccess;
  // The reverse index first (it needs only idx), then the query-side and the
  // key-side kernel, all in the caller's stream order.
  hipError_t err;
  {
    KernelTimer timer(kKernReverseIndex, a.stream);
    const bool res = (a.n_query * a.k + kRevWaves - 1) / kRevWaves <= 512;
    auto kern = res ? k_reverse_index<true> : k_reverse_index<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)heads), dim3(512), 0, a.stream, a.idx, a.n_query,
                       a.n_key, a.k, a.rev_off, a.rev_ent);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t qtiles = heads * a.n_query, ktiles = heads * a.n_key;
  if (a.dtype == 1 && a.S == 16 && (a.D == 64 || a.D == 32)) {
    err = launch_backward_s16(a, qtiles, ktiles);
    if (err != hipSuccess) return err;
  } else if (a.dtype == 1 && a.S == 64 && (a.D == 64 || a.D == 32)) {
    if (qtiles > 0) {
      KernelTimer timer(kKernBackwardQ, a.stream);
      auto kern = a.D == 64 ? (a.accumulate ? k_bwd_q_bf16<64, true> : k_bwd_q_bf16<64, false>)
                            : (a.accumulate ? k_bwd_q_bf16<32, true> : k_bwd_q_bf16<32, false>);
      hipLaunchKernelGGL(kern, dim3((unsigned)qtiles), dim3(256), 0, a.stream,
                         (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, a.idx, a.w,
                         a.lse, (const bf16*)a.dout, (const bf16*)a.lk, (bf16*)a.dq, a.dw,
                         a.dscore, a.dlq, a.delta, a.ds_layer, a.n_query, a.n_key, a.k, a.dl,
                         a.attn_scale, a.score_scale);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ktiles > 0) {
      KernelTimer timer(kKernBackwardKV, a.stream);
      auto kern = a.D == 64 ? (a.accumulate ? k_bwd_kv_bf16<64, true> : k_bwd_kv_bf16<64, false>)
                            : (a.accumulate ? k_bwd_kv_bf16<32, true> : k_bwd_kv_bf16<32, false>);
      hipLaunchKernelGGL(kern, dim3((unsigned)ktiles), dim3(256), 0, a.stream,
                         (const bf16*)a.q, (const bf16*)a.kk, (const bf16*)a.v, a.w, a.lse,
                         (const bf16*)a.dout, a.delta, a.rev_off, a.rev_ent, (const bf16*)a.lq,
                         a.accumulate ? a.ds_layer : a.dscore, a.dk, a.dv, a.dlk, a.n_query,
                         a.n_key, a.k,
                         a.dl, a.attn_scale, a.score_scale);
    }
  } else if (a.dtype == 1) {
    err = launch_backward_gen<bf16>(a, qtiles, ktiles);
    if (err != hipSuccess) return err;
  } else {
    err = launch_backward_gen<float>(a, qtiles, ktiles);
    if (err != hipSuccess) return err;
  }
  return hipGetLastError();
}

}  // namespace gca
