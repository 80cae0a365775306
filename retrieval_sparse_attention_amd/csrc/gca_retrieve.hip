// GCA retrieval: Eq. 1 relevance scores, top-k selection and Eq. 3 fusion weights.
//
// Definition (paperhub.cn review page, authors' reply "Cmt 1"; long-context-
// modeling README, "Model Architecture"): query chunk t scores every eligible
// past chunk j < q_pos[t] - 1 with r_j = score_scale * <lq_t, lk_j>, keeps the k
// best and weights them with softmax(r) (or softmax off-by-one, paperhub.cn
// authors' reply "Q4").
//
// bf16 path.  The scan is a dense contraction of 32 query landmarks with a
// stream of candidate landmarks, so it runs on MFMA and is bound by the single
// pass over lk in HBM.  S^T = LK_block (32 x Dl) * LQ^T (Dl x 32) puts, in each
// lane, 16 dot products of ONE query.  Selection is by threshold: only
// candidates at or above a running lower bound of the k-th best score are
// appended to a per-query LDS bucket, and the bucket is reduced to its exact
// top k now and then (see k_scan_topk_bf16).  Large candidate sets are cut
// into slices whose partial top-k lists a second kernel merges.
//
// f32 path.  One thread per query computes float32 dot products and keeps a
// sorted register list; it serves the small float32 workloads.
//
// Gumbel top-k (paperlayer.ai summary, section 3.2: during training, Gumbel
// noise is added to the relevance scores before the top-k selection).  Every
// kernel here has a NOISE variant: candidate j of query q in linear head h is
// ranked by r_j + G_j, with G_j = -ln(-ln U) and U = (m + 1/2) 2^-23 from the top
// 23 bits m of word (j mod 4) of Philox4x32-10 (Salmon et al., SC 2011) at
// counter (j / 4, q, h, 0) under the 64-bit seed.  The noise decides the
// selection only: the reported scores and the fusion weights are computed from
// the clean r of the selected chunks.

#include "gca_device.h"
#include "gca_fwd64.h"
#include "gca_launch.h"

namespace gca {

// Fills the k output slots of one query from its sorted (by `better`) list:
// indices ascending, scores, and the fusion weights.
template <int KMAX>
__device__ void finalize_query(const float (&s_in)[KMAX], const int (&i_in)[KMAX], int k,
                               int softmax_one, int32_t* idx_out, float* score_out,
                               float* w_out) {
  float s[KMAX];
  int id[KMAX];
  int m = 0;
#pragma unroll
  for (int p = 0; p < KMAX; ++p) {
    const bool keep = (p < k) && (i_in[p] != kIdxNone);
    s[p] = keep ? s_in[p] : 0.0f;
    id[p] = keep ? i_in[p] : kIdxNone;
    m += keep ? 1 : 0;
  }
  // ascending chunk index (odd-even transposition sort; unused slots sort last)
#pragma unroll
  for (int pass = 0; pass < KMAX; ++pass) {
#pragma unroll
    for (int p = (pass & 1); p + 1 < KMAX; p += 2) {
      const bool sw = id[p] > id[p + 1];
      const int ia = id[p], ib = id[p + 1];
      const float sa = s[p], sb = s[p + 1];
      id[p] = sw ? ib : ia;
      id[p + 1] = sw ? ia : ib;
      s[p] = sw ? sb : sa;
      s[p + 1] = sw ? sa : sb;
    }
  }
  float mx = -__builtin_huge_valf();
#pragma unroll
  for (int p = 0; p < KMAX; ++p)
    if (p < m) mx = fmaxf(mx, s[p]);
  const float shift = softmax_one ? fmaxf(mx, 0.0f) : mx;
  // exponentials by the hardware exp2 (a few ulps), one reciprocal of z
  float e[KMAX];
  float z = softmax_one ? fast_exp2(-shift * kLog2e) : 0.0f;
#pragma unroll
  for (int p = 0; p < KMAX; ++p) {
    e[p] = (p < m) ? fast_exp2((s[p] - shift) * kLog2e) : 0.0f;
    z += e[p];
  }
  const float rz = 1.0f / z;  // z >= 1 when m > 0 (the largest term is 1)
#pragma unroll
  for (int p = 0; p < KMAX; ++p) {
    if (p < k) {
      const bool ok = p < m;
      idx_out[p] = ok ? id[p] : -1;
      score_out[p] = ok ? s[p] : 0.0f;
      w_out[p] = ok ? e[p] * rz : 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// Candidate keys.  A candidate (score x, chunk j) is packed into one 64-bit key
// whose unsigned order is the selection order: the high word maps the float
// bits of x to an order-preserving unsigned value, the low word is ~j, so that
// among equal scores the lower chunk index is the larger key.  Key 0 is below
// every real key and marks an empty entry.  Keys of one query are distinct
// because chunk indices are.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ord_score(float x) {
  const uint32_t u = __float_as_uint(x);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t h = (uint32_t)(key >> 32);
  return __uint_as_float((h & 0x80000000u) ? (h ^ 0x80000000u) : ~h);
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ uint64_t make_key(float x, int j) {
  return ((uint64_t)ord_score(x) << 32) | (uint32_t)~(uint32_t)j;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011): ten rounds, each
// multiplying words 0 and 2 by the two round constants and recombining the
// halves of the 64-bit products with words 1 and 3 and the key; the key steps
// by the two Weyl increments between rounds.  The key is wave-uniform.
struct Words4 {
  uint32_t w[4];
};
__device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // one 32 x 32 -> 64-bit product each (a single v_mad_u64_u32)
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u, p1 = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return Words4{{c0, c1, c2, c3}};
}

// Standard Gumbel variate from one 32-bit word: U = (m + 1/2) 2^-23 (exact in
// float32, strictly inside (0, 1)), E = -ln U, G = -ln E, with the hardware
// base-2 logarithm and no library calls.  Above U = 15/16, E comes from
// t = 1 - U (exact) by the series t + t^2/2 + ... + t^6/6, whose first left-out
// term is below t^7/7 <= 2^-24 t / 7 (t <= 1/16), so E keeps full relative
// accuracy near U = 1; below, E = -log2(U) ln 2, where |log2 U| >= 0.09.  Over
// all 2^23 words, E is within 1.3e-7 relative and G within 1.1e-6 absolute of
// the exact values if log2 were correctly rounded; v_log_f32 is not (about one
// ulp), which leaves G within a few 1e-6.
__device__ __forceinline__ float gumbel_from_word(uint32_t word) {
  constexpr float kLn2 = 0.69314718f;
  const float u = (float)(word >> 9) * 0x1p-23f + 0x1p-24f;
  const float t = 1.0f - u;
  float s = fmaf(t, 1.0f / 6.0f, 0.2f);
  s = fmaf(t, s, 0.25f);
  s = fmaf(t, s, 1.0f / 3.0f);
  s = fmaf(t, s, 0.5f);
  s = fmaf(t, s, 1.0f);
  const float e = u > 0.9375f ? t * s : -__builtin_amdgcn_logf(u) * kLn2;
  return -__builtin_amdgcn_logf(e) * kLn2;
}

// Word e (0..3, any lane-varying value) without indexing a register array.
__device__ __forceinline__ uint32_t word_at(const Words4& n, int e) {
  return e == 0 ? n.w[0] : (e == 1 ? n.w[1] : (e == 2 ? n.w[2] : n.w[3]));
}

// Noise of candidates 4c .. 4c+3 of query q in linear head h.
__device__ __forceinline__ Words4 gumbel_words(uint64_t seed, int64_t c, int64_t q, int64_t h) {
  return philox4x32_10((uint32_t)c, (uint32_t)q, (uint32_t)h, 0u, (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}

// float32 dot product of two bf16 landmark rows (16-byte aligned, DL % 8 == 0),
// in dimension order: the clean score of a selected candidate.
__device__ __forceinline__ float dot_bf16_rows(const bf16* a, const bf16* b, int dl) {
  float acc = 0.0f;
  for (int d0 = 0; d0 < dl; d0 += 8) {
    const bf16x8 x = *(const bf16x8*)(a + d0);
    const bf16x8 y = *(const bf16x8*)(b + d0);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
  }
  return acc;
}

// Lower bound, in unscaled dot-product units, of every dot product a whose
// score fl(a * scale) reaches t (inv_scale = 1 / scale, rounded): the relative
// margin 2^-20 covers the three roundings involved and the absolute 1e-30
// covers scores that underflow to zero.  -inf stays -inf.
__device__ __forceinline__ float raw_bound(float t, float inv_scale) {
  const float r = t * inv_scale;
  return (r >= 0.0f ? r * (1.0f - 0x1p-20f) : r * (1.0f + 0x1p-20f)) - 1e-30f;
}

// Sorted (descending) key list -> the (score, index) list finalize_query takes.
template <int KMAX>
__device__ __forceinline__ void keys_to_list(const uint64_t* keys, int m, float (&s)[KMAX],
                                             int (&id)[KMAX]) {
#pragma unroll
  for (int p = 0; p < KMAX; ++p) {
    const uint64_t key = keys[p];
    s[p] = p < m ? key_score(key) : -__builtin_huge_valf();
    id[p] = p < m ? key_index(key) : kIdxNone;
  }
}

// ---------------------------------------------------------------------------
// bf16 scan.  Grid: heads * nsplit * n_qtiles workgroups of 256 threads.
//
// Each workgroup owns 32 queries and one slice of candidates, visited in
// rounds of 128 (one 32-candidate block per wave).  Per query it keeps a
// threshold tau (in unscaled dot-product units, see raw_bound), a sorted list
// of the best keys found so far and an LDS bucket.  A candidate whose dot
// product reaches tau is appended to its query's bucket; candidates below tau
// cannot be in the top k.  Whenever a bucket could overflow in the next round,
// and after the last round, the workgroup reduces list + bucket to the exact
// top k and raises tau to the k-th best.  In the first round, where no tau
// exists yet, each of the 8 groups of 16 candidates a query gets (4 waves x 2
// lane halves) offers its c-th best (c = 1 for k <= 8, else 2) and the
// smallest offer serves as tau: 8c >= k candidates reach it.  For k <= 8 the
// same bound is refreshed every round from the 8 lanes' running maxima.
// Exactness never depends on tau's quality, only the amount of work does.
// ---------------------------------------------------------------------------
// Rows of the 32-row block at blk that lie below lim, for the lane half whose
// rows start 4*half in, clamped to [0, 32].  Formed in 64 bits: blk passes
// n_key by up to a round in the last blocks, so lim - blk can fall below
// -2^31 when n_key is close to 2^31.
__device__ __forceinline__ int eligible_rows(int64_t lim, int64_t blk, int half) {
  const int64_t r = lim - blk - 4 * half;
  return r <= 0 ? 0 : (r >= 32 ? 32 : (int)r);
}

constexpr int kScanCap = 160;  // bucket entries per query (>= 128 + 16)
// Row stride in 8-byte entries: room past kScanCap for the packed kept keys
// and 2 spare slots, and odd, so the 32 rows a wave appends to at the same
// position fall in 32 different bank pairs.
constexpr int kScanStride = kScanCap + 25;
// Landmark blocks in flight per wave.  One suffices: the next block's load
// overlaps the current round's selection, and a second one costs registers
// and loop unrolling (16M scan: 84 us with one, 90 us with two).
#ifndef GCA_SCAN_PREFETCH
#define GCA_SCAN_PREFETCH 1
#endif
constexpr int kScanPrefetch = GCA_SCAN_PREFETCH;

// Bucket entries hold the raw dot product (with noise: the perturbed score
// itself) and the chunk index of a candidate; the selection key is formed only
// here.
struct ScanEntry {
  float raw;
  int j;
};

template <bool NOISE>
__device__ __forceinline__ uint64_t entry_key(ScanEntry e, float score_scale) {
  if (NOISE) return make_key(e.raw + 0.0f, e.j);
  return make_key(e.raw * score_scale + 0.0f, e.j);  // +0.0f: -0 scores compare as +0
}

// The threshold in the units the scan compares: raw dot products without
// noise (a bound through raw_bound), the perturbed score itself with noise.
template <bool NOISE>
__device__ __forceinline__ float tau_from_score(float t, float inv_scale) {
  return NOISE ? t : raw_bound(t, inv_scale);
}

// Completes this wave's LDS accesses before any later one issues; the compiler
// moves no memory access across it.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Exact top k of every query's kept list plus its bucket (256 threads: 8 per
// query, all in one wave).  Everything of query q (bucket row, kept list,
// counts, tau) is touched only by its 8 threads, so the steps order within
// the wave; one workgroup barrier at the end publishes the result.
// Afterwards kept[q] holds the sorted top-k keys, the bucket is empty and
// tau_raw[q] bounds the k-th best from below.
//  1. Thread `sub` of query q takes bucket entries sub, sub+8, ... and kept
//     entries sub, sub+8, and finds its c-th best key (c = 1 for k <= 8, else
//     2); the minimum over the 8 threads bounds the k-th best key from below
//     (8c >= k distinct entries reach it).
//  2. Keys at or above that bound are packed to the front of the bucket.
//  3. Each packed key's rank is the number of packed keys above it; ranks
//     below k give the sorted top k.
// Inlined: as a call it waits for every landmark load in flight on entry (the
// calling convention), saves registers to scratch and reaches LDS through
// generic pointers; inlined it takes about a quarter less time.
template <int KMAX, bool NOISE>
__device__ __forceinline__ void scan_compact(ScanEntry* bucket, uint64_t (*kept)[KMAX], int* cnt,
                                             int* nkept, int* ncnt, float* tau_raw, int k,
                                             float score_scale, float inv_scale) {
  constexpr int E = kScanCap / 8;
  constexpr int EK = (KMAX + 7) / 8;
  const int tid = threadIdx.x;
  const int q = tid >> 3, sub = tid & 7;
  ScanEntry* b = bucket + q * kScanStride;
  const int n = cnt[q], nk = nkept[q];
  // entries per thread this wave needs (its 8 queries' largest bucket); the
  // xor 8/16/32 maximum covers all 8 queries of the wave, so it is uniform and
  // the loops below branch on a scalar
  int nw = n;
  nw = max(nw, __shfl_xor(nw, 8));
  nw = max(nw, __shfl_xor(nw, 16));
  nw = max(nw, __shfl_xor(nw, 32));
  const int per = __builtin_amdgcn_readfirstlane((nw + 7) >> 3);
  uint64_t e[E + EK];
#pragma unroll
  for (int p = 0; p < E; ++p) {
    e[p] = 0;
    if (p < per) {
      const int i = sub + 8 * p;
      const ScanEntry v = b[i];
      e[p] = i < n ? entry_key<NOISE>(v, score_scale) : 0;
    }
  }
#pragma unroll
  for (int p = 0; p < EK; ++p) {
    const int i = sub + 8 * p;
    const uint64_t v = kept[q][i < KMAX ? i : 0];
    e[E + p] = i < nk ? v : 0;
  }
  uint64_t m1 = 0, m2 = 0;
#pragma unroll
  for (int p = 0; p < E + EK; ++p) {
    if (KMAX > 8) m2 = umax64(m2, umin64(m1, e[p]));
    m1 = umax64(m1, e[p]);
  }
  uint64_t thr = (KMAX > 8 && k > 8) ? m2 : m1;
  thr = umin64(thr, shfl_xor64(thr, 1));
  thr = umin64(thr, shfl_xor64(thr, 2));
  thr = umin64(thr, shfl_xor64(thr, 4));
  if (sub == 0) ncnt[q] = 0;
  wave_lds_sync();
  // The pack has no branches: a key below thr (or empty) goes to the row's
  // last slot, which no rank read reaches (n2 + 3 < kScanStride - 1).
  uint64_t* pk = (uint64_t*)b;  // packed keys reuse the bucket row
  int np = 0;
#pragma unroll
  for (int p = 0; p < E + EK; ++p) np += (e[p] != 0 && e[p] >= thr) ? 1 : 0;
  int o = np ? atomicAdd(&ncnt[q], np) : 0;
  wait_lds();
#pragma unroll
  for (int p = 0; p < E + EK; ++p) {
    if (p < E && p >= per) continue;  // uniform: entries this wave never loaded
    const bool keep = e[p] != 0 && e[p] >= thr;
    pk[keep ? o : kScanStride - 1] = e[p];
    o += keep ? 1 : 0;
  }
  wave_lds_sync();
  const int n2 = ncnt[q];
  for (int u0 = 0; u0 < n2; u0 += 32) {
    uint64_t mine[4];
    int rank[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = u0 + sub + 8 * u;
      mine[u] = i < n2 ? pk[i] : 0;
      rank[u] = 0;
    }
    // f + 3 < n2 + 3 <= kScanCap + KMAX + 3 < kScanStride: reads stay in the row
    for (int f = 0; f < n2; f += 4) {
      uint64_t F[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) F[t] = f + t < n2 ? pk[f + t] : 0;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) rank[u] += F[t] > mine[u] ? 1 : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (mine[u] != 0 && rank[u] < k) kept[q][rank[u]] = mine[u];
  }
  wave_lds_sync();
  const int m = n2 < k ? n2 : k;
  if (sub == 0) {
    cnt[q] = 0;
    nkept[q] = m;
    tau_raw[q] = m == k ? tau_from_score<NOISE>(key_score(kept[q][k - 1]), inv_scale)
                        : -__builtin_huge_valf();
  }
  __syncthreads();
}

template <int DL, int KMAX, bool NOISE>
__global__ __launch_bounds__(256, 3) void k_scan_topk_bf16(
    const bf16* __restrict__ lq, const bf16* __restrict__ lk, const int32_t* __restrict__ q_pos,
    int64_t n_query, int64_t n_key, int n_qtiles, int nsplit, int64_t split_len,
    float score_scale, int k, int softmax_one, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, float* __restrict__ w_out, uint64_t* __restrict__ part,
    uint64_t seed) {
  constexpr int NKS = DL / 16;  // MFMA K-steps over the landmark dimension
  constexpr int HALF = DL / 2;  // landmark dims supplied by each lane half
  constexpr int PF = kScanPrefetch;
  __shared__ ScanEntry bucket[32 * kScanStride];
  __shared__ uint64_t kept[32][KMAX];  // sorted top keys of the compacted candidates
  __shared__ int cnt[32], nkept[32], ncnt[32];
  __shared__ float tau_raw[32];  // raw dot-product bound of the k-th best score
  __shared__ uint32_t first_bound[32];  // min over groups of the ordered c-th best dot product
  // running maximum of each of the 8 lanes (4 waves x 2 halves) that hold a
  // query's candidates: [query][2 wave + half]
  __shared__ __align__(16) float run_max[32][8];
  __shared__ int full[3];  // per round (mod 3): some bucket may overflow next round

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  const int64_t bid = blockIdx.x;
  const int qt = (int)(bid % n_qtiles);
  const int64_t rest = bid / n_qtiles;
  const int sp = (int)(rest % nsplit);
  const int64_t head = rest / nsplit;

  const int64_t q = (int64_t)qt * 32 + col;
  const bool q_ok = q < n_query;
  int64_t n_cand = 0;
  if (q_ok) {
    const int64_t pos = q_pos[q];
    n_cand = pos - 1 < n_key ? pos - 1 : n_key;
    if (n_cand < 0) n_cand = 0;
  }
  // largest candidate count of the tile (every wave sees the same 32 queries)
  int tile_max = (int)n_cand;  // n_key < 2^31 is checked on the host
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tile_max = max(tile_max, __shfl_xor(tile_max, o));
  tile_max = __builtin_amdgcn_readfirstlane(tile_max);  // uniform: keeps the loops scalar
  const int64_t c_begin = (int64_t)sp * split_len;
  int64_t c_end = c_begin + split_len;
  if (c_end > tile_max) c_end = tile_max;
  const int64_t lim = n_cand < c_end ? n_cand : c_end;  // this lane's query: j < lim
  const int c_first = (KMAX > 8 && k > 8) ? 2 : 1;

  if (tid < 32) {
    cnt[tid] = 0;
    nkept[tid] = 0;
    tau_raw[tid] = -__builtin_huge_valf();
    first_bound[tid] = 0xFFFFFFFFu;
  }
  if (tid < 3) full[tid] = 0;

  // Query landmarks as the MFMA B operand.  Lanes past the last query read
  // query 0's row and select nothing (their candidate count is 0).  The loads
  // are unconditional: loads under a lane mask leave the compiler unsure how
  // many loads are in flight, and it then drains every landmark block at the
  // top of each round instead of keeping the next ones in flight.
  bf16x8 bq[NKS];
  {
    const bf16* row = lq + (head * n_query + (q_ok ? q : 0)) * DL + HALF * half;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) bq[ks] = *(const bf16x8*)(row + 8 * ks);
  }
  const float inv_scale = 1.0f / score_scale;

  // Landmark rows: this lane reads row (block + col), half `half`, clamped to
  // the last row: rows past the slice are read (in bounds) but never selected.
  // Every round issues its loads unconditionally, so the compiler's wait
  // counts let PF blocks per wave stay in flight.
  const bf16* lk_head = lk + head * n_key * DL + HALF * half;
  auto load_block = [&](int64_t blk, bf16x8 (&a)[NKS]) {
    const int64_t r = blk + col;
    const bf16* p = lk_head + (r < n_key ? r : n_key - 1) * DL;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) a[ks] = *(const bf16x8*)(p + 8 * ks);
  };
  const int n_rounds = c_end > c_begin ? (int)((c_end - c_begin + 127) >> 7) : 0;
  bf16x8 ring[PF][NKS];  // slot s holds rounds s, s + PF, s + 2 PF, ...
  if (n_rounds > 0) {
#pragma unroll
    for (int s = 0; s < PF; ++s) load_block(c_begin + 128 * s + 32 * wave, ring[s]);
  }
  __syncthreads();

  // The overflow decision after round R reads full[R % 3], which only round R
  // sets; it is cleared during round R + 2, after every wave has read it (two
  // barriers later) and before round R + 3 can set it again.  Rounds past the
  // slice (up to PF - 1 at the end) select nothing.
  // this lane's query threshold, kept in a register: tau_raw changes only in
  // round 0 and in a compaction, and both refresh it.  It never drops below
  // -FLT_MAX (a bound every finite score meets), so -inf marks ineligible rows.
  float tl = -__FLT_MAX__;
  // Running bound (k <= 8): the 8 lanes of a query see disjoint candidates, so
  // the smallest of their running maxima is reached by 8 distinct candidates
  // and bounds the k-th best from below.  It rises every round, between the
  // compactions that set tau exactly; the maxima of round R are read in round
  // R + 1, after the barrier that ends round R.
  constexpr bool run_bound = KMAX <= 8;  // k <= KMAX
  float rmax = -__builtin_huge_valf();
  for (int round0 = 0; round0 < n_rounds; round0 += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int round = round0 + s;
      const int64_t blk = c_begin + 128 * round + 32 * wave;
      if (tid == 0) full[(round + 1) % 3] = 0;
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc = mfma32x32x16(ring[s][ks], bq[ks], acc);
      load_block(blk + 128 * PF, ring[s]);
      if (NOISE) {
        // perturbed scores fl(r * scale + G): rows 8g + 4 half + e (e = 0..3)
        // are four consecutive candidates, one Philox call
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const Words4 nz = gumbel_words(seed, (blk + 4 * half + 8 * g4) >> 2, q, head);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[4 * g4 + e] = fmaf(acc[4 * g4 + e], score_scale, gumbel_from_word(nz.w[e]));
        }
      }
      // candidate blk + c_row(r, half) is eligible iff c_row(r, half) - 4*half < rem.
      // Ineligible rows become -inf, below every threshold (tl >= -FLT_MAX),
      // so the tests below need no eligibility mask; only the blocks where a
      // query's candidates end take this branch.
      const int rem = eligible_rows(lim, blk, half);
      if (!__all(rem >= 28)) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[r] = (8 * (r >> 2) + (r & 3)) < rem ? acc[r] : -__builtin_huge_valf();
      }
      if (round == 0) {
        float m1 = -__builtin_huge_valf(), m2 = -__builtin_huge_valf();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (KMAX > 8) m2 = fmaxf(m2, fminf(m1, acc[r]));
          m1 = fmaxf(m1, acc[r]);
        }
        atomicMin(&first_bound[col], ord_score(c_first == 2 ? m2 : m1));
        __syncthreads();
        const uint32_t fb = first_bound[col];
        const float b_raw = (fb & 0x80000000u) ? __uint_as_float(fb ^ 0x80000000u)
                                               : __uint_as_float(~fb);
        // the scores of the offered candidates reach fl(b_raw * scale) (with
        // noise: b_raw is the perturbed score); the bound stays valid for
        // every later round
        tl = fmaxf(tl, NOISE ? b_raw : raw_bound(b_raw * score_scale + 0.0f, inv_scale));
        if (tid < 32) tau_raw[tid] = tl;  // lane tid < 32 holds query col = tid
      }
      // Fast test: once tau has risen, most blocks hold no candidate at or
      // above it; the lane's best value decides with one compare.
      float best = acc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) best = fmaxf(best, acc[r]);
      if (run_bound) {
        if (round > 0) {
          const f32x4 rm_lo = *(const f32x4*)&run_max[col][0];
          const f32x4 rm_hi = *(const f32x4*)&run_max[col][4];
          const float rb = fminf(fminf(fminf(rm_lo[0], rm_lo[1]), fminf(rm_lo[2], rm_lo[3])),
                                 fminf(fminf(rm_hi[0], rm_hi[1]), fminf(rm_hi[2], rm_hi[3])));
          tl = fmaxf(tl, NOISE ? rb : raw_bound(rb * score_scale + 0.0f, inv_scale));
        }
        rmax = fmaxf(rmax, best);
        run_max[col][2 * wave + half] = rmax;
      }
      if (__any(best >= tl)) {
        int nh = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) nh += acc[r] >= tl ? 1 : 0;
        // One LDS atomic per lane reserves its entries; the writes then go out
        // without waiting on each other: a lane without a hit at r writes to
        // its spare slot past kScanCap, so branches stay uniform.
        int o = nh ? atomicAdd(&cnt[col], nh) : 0;
        wait_lds();
        ScanEntry* bb = bucket + col * kScanStride;
        const int spare = kScanCap + half;
        const int j0 = (int)(blk + 4 * half);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool hit = acc[r] >= tl;
          if (__any(hit)) {
            ScanEntry* d = bb + (hit ? o : spare);
            d->raw = acc[r];
            d->j = j0 + 8 * (r >> 2) + (r & 3);
            o += hit ? 1 : 0;
          }
        }
        // the last lane to append to a query sees its final count
        if (nh && o > kScanCap - 128) full[round % 3] = 1;
      }
      __syncthreads();
      if (round + 1 < n_rounds && full[round % 3]) {
        scan_compact<KMAX, NOISE>(bucket, kept, cnt, nkept, ncnt, tau_raw, k, score_scale,
                                  inv_scale);
        tl = fmaxf(tl, tau_raw[col]);  // raised by the compaction
      }
    }
  }
  scan_compact<KMAX, NOISE>(bucket, kept, cnt, nkept, ncnt, tau_raw, k, score_scale, inv_scale);

  const int qs = tid >> 3, sub = tid & 7;
  const int64_t qq = (int64_t)qt * 32 + qs;
  if (qq >= n_query) return;
  const int m = nkept[qs];
  const int64_t qrow = head * n_query + qq;
  if (nsplit == 1) {
    float clean[KMAX];
    if (NOISE) {
      // clean scores of the selected candidates: thread sub computes entries
      // sub and sub + 8, then the 8 threads of the query share them
      const bf16* lq_row = lq + qrow * DL;
      const bf16* lk_h = lk + head * n_key * DL;
      float c0 = 0.0f, c1 = 0.0f;
      if (sub < m)
        c0 = dot_bf16_rows(lq_row, lk_h + (int64_t)key_index(kept[qs][sub]) * DL, DL) *
             score_scale;
      if (KMAX > 8 && sub + 8 < m)
        c1 = dot_bf16_rows(lq_row, lk_h + (int64_t)key_index(kept[qs][sub + 8]) * DL, DL) *
             score_scale;
      const int base = lane & ~7;
#pragma unroll
      for (int p = 0; p < KMAX; ++p) clean[p] = __shfl(p < 8 ? c0 : c1, base + (p & 7));
    }
    if (sub == 0) {
      float s[KMAX];
      int id[KMAX];
      keys_to_list<KMAX>(kept[qs], m, s, id);
      if (NOISE) {
#pragma unroll
        for (int p = 0; p < KMAX; ++p) s[p] = p < m ? clean[p] : -__builtin_huge_valf();
      }
      finalize_query<KMAX>(s, id, k, softmax_one, idx_out + qrow * k, score_out + qrow * k,
                           w_out + qrow * k);
    }
  } else {
    uint64_t* dst = part + (qrow * nsplit + sp) * KMAX;
    for (int p = sub; p < KMAX; p += 8) dst[p] = p < m ? kept[qs][p] : 0;
  }
}

// ---------------------------------------------------------------------------
// bf16 scan for a few queries per head (a decoding step scores one new chunk's
// landmark against the whole context).  In k_scan_topk_bf16 such a query
// would fill one column of a 32-query MFMA tile, and the tile's fixed costs
// (bucket set-up, compactions over 32 queries) would set the step's latency.
// Here one workgroup takes one (head, query) row and 256 consecutive
// candidates, one landmark row per DL / 8 lanes (16 bytes each, so every wave
// load covers whole rows), and writes the slice's KMAX best keys to the list
// the merge kernel reads.  Grid: heads * n_query * nsplit, slice sp of row
// (head, q) at block (head * n_query + q) * nsplit + sp.
//   1. all of the slice's landmark loads are issued at once; each lane forms
//      the float32 dot product of its 8 dimensions, and DPP moves sum the
//      row's lanes (quad swaps, then the 8-lane mirror for DL = 64);
//   2. key = (ordered score bits, ~j) as in the other scans, 0 for j past the
//      query's candidates (j >= q_pos - 1 or >= n_key);
//   3. each wave ranks its 64 keys among themselves in LDS; a key beaten by
//      KMAX keys of its own wave cannot be among the slice's KMAX best, so at
//      most 4 * KMAX survivors are ranked against each other, and rank r < KMAX
//      goes to list entry r (entries past the slice's valid keys are 0).
// ---------------------------------------------------------------------------
template <int DL, int KMAX>
__global__ __launch_bounds__(256) void k_scan_few_bf16(
    const bf16* __restrict__ lq, const bf16* __restrict__ lk, const int32_t* __restrict__ q_pos,
    int64_t n_query, int64_t n_key, int nsplit, float score_scale, uint64_t* __restrict__ part) {
  constexpr int LPR = DL / 8;     // lanes per landmark row
  constexpr int RPP = 256 / LPR;  // rows per pass of the workgroup
  constexpr int NP = LPR;         // passes over the slice's 256 rows
  static_assert(DL == 64 || DL == 32, "landmark rows of 64 or 32 bf16 values");
  __shared__ __align__(16) uint64_t keys[256];
  __shared__ __align__(16) uint64_t surv[4 * KMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sp = (int)(blockIdx.x % nsplit);
  const int64_t qrow = blockIdx.x / nsplit;  // = head * n_query + q
  const int64_t head = qrow / n_query;
  const int64_t pos = q_pos[qrow - head * n_query];
  int64_t n_cand = pos - 1 < n_key ? pos - 1 : n_key;
  if (n_cand < 0) n_cand = 0;
  const int64_t c0 = (int64_t)sp * 256;
  const int p = tid % LPR, r0 = tid / LPR;  // dims 8p .. 8p+7 of row r0 of each pass
  const bf16x8 qv = *(const bf16x8*)(lq + qrow * DL + 8 * p);
  const bf16* lk_head = lk + head * n_key * DL;
  bf16x8 kv[NP];
#pragma unroll
  for (int s = 0; s < NP; ++s) {
    const int64_t j = c0 + s * RPP + r0;
    kv[s] = *(const bf16x8*)(lk_head + (j < n_key ? j : n_key - 1) * DL + 8 * p);
  }
  if (tid < 4 * KMAX) surv[tid] = 0;
  float qf[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qf[e] = (float)qv[e];
#pragma unroll
  for (int s = 0; s < NP; ++s) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(qf[e], (float)kv[s][e], acc);
    acc += dpp_f<0xB1>(acc);                 // quad_perm [1,0,3,2]
    acc += dpp_f<0x4E>(acc);                 // quad_perm [2,3,0,1]
    if (LPR == 8) acc += dpp_f<0x141>(acc);  // row_half_mirror: the other 4 lanes
    const int rl = s * RPP + r0;
    const int64_t j = c0 + rl;
    if (p == 0) keys[rl] = j < n_cand ? make_key(acc * score_scale + 0.0f, (int)j) : 0;
  }
  __syncthreads();
  const uint64_t mine = keys[tid];
  int rw = 0;  // keys of this wave above mine
#pragma unroll 8
  for (int u = 0; u < 64; u += 2) {
    const ulonglong2 o = *(const ulonglong2*)&keys[64 * wave + u];
    rw += (o.x > mine ? 1 : 0) + (o.y > mine ? 1 : 0);
  }
  const bool keep = mine != 0 && rw < KMAX;
  const uint64_t mask = __ballot(keep);
  if (keep)
    surv[KMAX * wave + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0))] =
        mine;
  const int nv = __syncthreads_count(keep);
  uint64_t* dst = part + (qrow * nsplit + sp) * KMAX;
  if (tid < 4 * KMAX) {
    const uint64_t me = surv[tid];
    int r = 0;
#pragma unroll
    for (int u = 0; u < 4 * KMAX; ++u) r += surv[u] > me ? 1 : 0;
    if (me != 0 && r < KMAX) dst[r] = me;
  }
  if (tid >= nv && tid < KMAX) dst[tid] = 0;
}

// ---------------------------------------------------------------------------
// Merge of the per-slice lists: one wave per (head, query) row, n = nsplit *
// KMAX keys (0 = empty).  The k-th largest of the 64 lane maxima bounds the
// k-th best key from below; entries at or above it are packed into LDS and
// ranked exactly.  With MW > 0 (n <= 64 MW) every key of the row is loaded
// into registers at once, so the row costs one round trip to memory; with
// MW = 0 the keys are streamed twice, 256 at a time.
// ---------------------------------------------------------------------------
constexpr int kMergeMax = 4096;  // nsplit * KMAX limit (LDS list size)

// Barrier of the merge: the workgroup's when the workgroup is the merging wave
// alone, else this wave's LDS order (the fused kernel merges in one wave).
template <bool WG>
__device__ __forceinline__ void merge_sync() {
  if (WG)
    __syncthreads();
  else
    wave_lds_sync();
}

// The merge of row qrow by one wave (lane = 0..63).  lst, out, lane_max and
// clean are LDS areas of 64 MW (or kMergeMax), KMAX, 64 and KMAX entries;
// the row's k slots go to idx_out / score_out / w_out + qrow * k.
template <int KMAX, bool NOISE, int MW, bool WG>
__device__ __forceinline__ void merge_row(
    int lane, int64_t qrow, const uint64_t* __restrict__ part, int n, int k, int softmax_one,
    int32_t* idx_out, float* score_out, float* w_out, const bf16* __restrict__ lq,
    const bf16* __restrict__ lk, int64_t n_query, int64_t n_key, int dl, float score_scale,
    uint64_t* lst, uint64_t* out, uint64_t* lane_max, float* clean) {
  const uint64_t* src = part + qrow * n;

  uint64_t mx = 0;
  uint64_t reg[MW > 0 ? MW : 1];  // MW > 0: key lane + 64 u of the row
  if (MW > 0) {
#pragma unroll
    for (int u = 0; u < MW; ++u) {
      const int e = lane + 64 * u;
      reg[u] = src[e < n ? e : n - 1];
    }
#pragma unroll
    for (int u = 0; u < MW; ++u) {
      reg[u] = lane + 64 * u < n ? reg[u] : 0;
      mx = umax64(mx, reg[u]);
    }
  } else {
    for (int e0 = 0; e0 < n; e0 += 256) {
      uint64_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + lane + 64 * u;
        v[u] = src[e < n ? e : n - 1];
        v[u] = e < n ? v[u] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) mx = umax64(mx, v[u]);
    }
  }
  // rank of this lane's maximum among the 64 (ties between empty lanes broken
  // by lane number), then the maximum of rank k-1; the 64 maxima go through
  // LDS once and come back as broadcast reads, all issued together
  lane_max[lane] = mx;
  merge_sync<WG>();
  int rank = 0;
#pragma unroll
  for (int l = 0; l < 64; l += 2) {
    const ulonglong2 o = *(const ulonglong2*)&lane_max[l];
    rank += (o.x > mx || (o.x == mx && l < lane)) ? 1 : 0;
    rank += (o.y > mx || (o.y == mx && l + 1 < lane)) ? 1 : 0;
  }
  const uint64_t sel = __ballot(rank == k - 1);
  const int src_lane = __builtin_ctzll(sel);  // k <= 16 < 64: exactly one lane
  const uint32_t thr_hi = __builtin_amdgcn_readlane((uint32_t)(mx >> 32), src_lane);
  const uint32_t thr_lo = __builtin_amdgcn_readlane((uint32_t)mx, src_lane);
  const uint64_t thr = ((uint64_t)thr_hi << 32) | thr_lo;

  int n2 = 0;
  auto pack = [&](uint64_t key) {
    const bool pass = key != 0 && key >= thr;
    const uint64_t mask = __ballot(pass);
    const int pos = n2 + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
    if (pass) lst[pos] = key;
    n2 += __builtin_popcountll(mask);
  };
  if (MW > 0) {
#pragma unroll
    for (int u = 0; u < MW; ++u) pack(reg[u]);
  } else {
    for (int e0 = 0; e0 < n; e0 += 256) {
      uint64_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + lane + 64 * u;
        v[u] = src[e < n ? e : n - 1];
        v[u] = e < n ? v[u] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) pack(v[u]);
    }
  }
  merge_sync<WG>();
  for (int i = lane; i < n2; i += 64) {
    const uint64_t me = lst[i];
    int r = 0;
    for (int f = 0; f < n2; ++f) r += lst[f] > me ? 1 : 0;
    if (r < k) out[r] = me;
  }
  merge_sync<WG>();
  const int m = n2 < k ? n2 : k;
  if (NOISE) {
    if (lane < m) {
      const int64_t head = qrow / n_query;
      clean[lane] = dot_bf16_rows(lq + qrow * dl,
                                  lk + (head * n_key + key_index(out[lane])) * dl, dl) *
                    score_scale;
    }
    merge_sync<WG>();
  }
  if (lane == 0) {
    float s[KMAX];
    int id[KMAX];
    keys_to_list<KMAX>(out, m, s, id);
    if (NOISE) {
#pragma unroll
      for (int p = 0; p < KMAX; ++p) s[p] = p < m ? clean[p] : -__builtin_huge_valf();
    }
    finalize_query<KMAX>(s, id, k, softmax_one, idx_out + qrow * k, score_out + qrow * k,
                         w_out + qrow * k);
  }
}

template <int KMAX, bool NOISE, int MW>
__global__ __launch_bounds__(64) void k_topk_merge(const uint64_t* __restrict__ part, int n,
                                                   int k, int softmax_one,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ score_out,
                                                   float* __restrict__ w_out,
                                                   const bf16* __restrict__ lq,
                                                   const bf16* __restrict__ lk, int64_t n_query,
                                                   int64_t n_key, int dl, float score_scale) {
  __shared__ uint64_t lst[MW > 0 ? 64 * MW : kMergeMax];  // packed keys: at most n
  __shared__ uint64_t out[KMAX];
  __shared__ __align__(16) uint64_t lane_max[64];
  __shared__ float clean[KMAX];  // with noise: clean scores of the selected
  merge_row<KMAX, NOISE, MW, true>(threadIdx.x, blockIdx.x, part, n, k, softmax_one, idx_out,
                                   score_out, w_out, lq, lk, n_query, n_key, dl, score_scale, lst,
                                   out, lane_max, clean);
}

// ---------------------------------------------------------------------------
// A sliced plain retrieval's merge fused with the 64-token forward (the
// retrieval-plus-forward call): one 256-thread workgroup per query chunk, in
// the forward's order.  Wave 0 merges the chunk's slice lists (n <= 64 MW
// keys, held in registers) into the exact top k, which go to idx / score / w
// and, through LDS, straight into the forward's slot table; the merge's key
// list borrows the K tile buffers, which the forward fills only afterwards.
// One launch and one round trip to memory fewer than the merge followed by
// the forward, with the same results bit for bit.
// ---------------------------------------------------------------------------
template <int D, int KMAX, int MW>
__global__ __launch_bounds__(256) void k_merge_fwd_bf16(
    const uint64_t* __restrict__ part, int n, int k, int softmax_one, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, float* __restrict__ w_out, const bf16* __restrict__ q,
    const bf16* __restrict__ kk, const bf16* __restrict__ v, bf16* __restrict__ o,
    float* __restrict__ lse, int64_t n_query, int64_t n_key, float attn_scale) {
  static_assert(64 * MW * 8 <= 2 * 64 * D * 2, "the merge list fits the K tile buffers");
  __shared__ __align__(16) bf16 k_lds[2][64 * D];
  __shared__ __align__(16) bf16 v_lds[2][64 * D];
  __shared__ uint64_t m_out[KMAX];
  __shared__ __align__(16) uint64_t m_lane_max[64];
  __shared__ int s_idx[16];
  __shared__ float s_score[16], s_w[16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);  // = head * n_query + t
  if (tid < 64)
    merge_row<KMAX, false, MW, false>(lane, 0, part + tile * n, n, k, softmax_one, s_idx, s_score,
                                      s_w, nullptr, nullptr, n_query, n_key, 0, 0.0f,
                                      (uint64_t*)&k_lds[0][0], m_out, m_lane_max, nullptr);
  __syncthreads();
  if (tid < k) {
    idx_out[tile * k + tid] = s_idx[tid];
    score_out[tile * k + tid] = s_score[tid];
    w_out[tile * k + tid] = s_w[tid];
  }
  const int i0 = lane < k ? lane : 0;
  const int c_in = s_idx[i0];
  const float w_in = s_w[i0];
  const bool ok = lane < k && c_in >= 0 && c_in < n_key;
  fwd_tile<D>(q, kk, v, o, lse, tile, n_query, n_key, k, attn_scale, c_in, w_in, ok, k_lds,
              v_lds);
}

// ---------------------------------------------------------------------------
// float32 scan: one thread per (head, query).
// ---------------------------------------------------------------------------
template <int KMAX, bool NOISE>
__global__ __launch_bounds__(64) void k_scan_topk_f32(
    const float* __restrict__ lq, const float* __restrict__ lk, const int32_t* __restrict__ q_pos,
    int64_t n_heads, int64_t n_query, int64_t n_key, int dl, float score_scale, int k,
    int softmax_one, int32_t* __restrict__ idx_out, float* __restrict__ score_out,
    float* __restrict__ w_out, uint64_t seed) {
  const int64_t qrow = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (qrow >= n_heads * n_query) return;
  const int64_t head = qrow / n_query, q = qrow % n_query;
  int64_t n_cand = (int64_t)q_pos[q] - 1;
  if (n_cand > n_key) n_cand = n_key;
  if (n_cand < 0) n_cand = 0;
  const float* lqr = lq + qrow * dl;
  const float* lkh = lk + head * n_key * dl;
  float s[KMAX];
  int id[KMAX];
  list_clear(s, id);
  for (int64_t j = 0; j < n_cand; ++j) {
    float acc = 0.0f;
    for (int d = 0; d < dl; ++d) acc = fmaf(lqr[d], lkh[j * dl + d], acc);
    float x = acc * score_scale;
    if (NOISE) {
      const Words4 nz = gumbel_words(seed, j >> 2, q, head);
      x = fmaf(acc, score_scale, gumbel_from_word(word_at(nz, (int)(j & 3))));
    }
    if (better(x, (int)j, s[KMAX - 1], id[KMAX - 1])) list_insert(s, id, x, (int)j);
  }
  if (NOISE) {
    // clean scores of the selected: the same dot products, recomputed in the
    // same order
#pragma unroll
    for (int p = 0; p < KMAX; ++p) {
      if (id[p] == kIdxNone) continue;
      float acc = 0.0f;
      for (int d = 0; d < dl; ++d) acc = fmaf(lqr[d], lkh[(int64_t)id[p] * dl + d], acc);
      s[p] = acc * score_scale;
    }
  }
  finalize_query<KMAX>(s, id, k, softmax_one, idx_out + qrow * k, score_out + qrow * k,
                       w_out + qrow * k);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <int KMAX, bool NOISE>
static hipError_t launch_scan_k(const ScanPlan& pl, const LaunchRetrieve& a) {
  const int64_t heads = a.G * a.B * a.H;
  if (a.dtype == 1) {
    const int64_t nblk = heads * pl.nsplit * pl.n_qtiles;
    {
    KernelTimer timer(kKernScan, a.stream);
    if (pl.few && !NOISE) {
      const unsigned fblk = (unsigned)(heads * a.n_query * pl.nsplit);
      if (a.dl == 64)
        hipLaunchKernelGGL((k_scan_few_bf16<64, KMAX>), dim3(fblk), dim3(256), 0, a.stream,
                           (const bf16*)a.lq, (const bf16*)a.lk, a.q_pos, a.n_query, a.n_key,
                           pl.nsplit, a.score_scale, a.part);
      else
        hipLaunchKernelGGL((k_scan_few_bf16<32, KMAX>), dim3(fblk), dim3(256), 0, a.stream,
                           (const bf16*)a.lq, (const bf16*)a.lk, a.q_pos, a.n_query, a.n_key,
                           pl.nsplit, a.score_scale, a.part);
    } else if (a.dl == 64)
      hipLaunchKernelGGL((k_scan_topk_bf16<64, KMAX, NOISE>), dim3((unsigned)nblk), dim3(256), 0,
                         a.stream, (const bf16*)a.lq, (const bf16*)a.lk, a.q_pos, a.n_query,
                         a.n_key, pl.n_qtiles, pl.nsplit, pl.split_len, a.score_scale, a.k,
                         a.softmax_one, a.idx, a.score, a.w, a.part, a.seed);
    else
      hipLaunchKernelGGL((k_scan_topk_bf16<32, KMAX, NOISE>), dim3((unsigned)nblk), dim3(256), 0,
                         a.stream, (const bf16*)a.lq, (const bf16*)a.lk, a.q_pos, a.n_query,
                         a.n_key, pl.n_qtiles, pl.nsplit, pl.split_len, a.score_scale, a.k,
                         a.softmax_one, a.idx, a.score, a.w, a.part, a.seed);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.nsplit == 1) return e;
    const int64_t rows = heads * a.n_query;
    const int n = pl.nsplit * KMAX;
    const LaunchForward* f = a.fuse;
    if (f && !NOISE && n <= 1024 && f->dtype == 1 && f->S == 64 && (f->D == 64 || f->D == 32)) {
      KernelTimer timer(kKernMergeForward, a.stream);
      auto fused = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3((unsigned)rows), dim3(256), 0, a.stream, a.part, n, a.k,
                           a.softmax_one, a.idx, a.score, a.w, (const bf16*)f->q,
                           (const bf16*)f->kk, (const bf16*)f->v, (bf16*)f->o, f->lse,
                           a.n_query, a.n_key, f->attn_scale);
      };
      if (f->D == 64)
        n <= 512 ? fused(k_merge_fwd_bf16<64, KMAX, 8>) : fused(k_merge_fwd_bf16<64, KMAX, 16>);
      else
        n <= 512 ? fused(k_merge_fwd_bf16<32, KMAX, 8>) : fused(k_merge_fwd_bf16<32, KMAX, 16>);
      if (a.fused) *a.fused = 1;
      return hipGetLastError();
    }
    KernelTimer timer(kKernMerge, a.stream);
    auto merge = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)rows), dim3(64), 0, a.stream, a.part, n, a.k,
                         a.softmax_one, a.idx, a.score, a.w, (const bf16*)a.lq,
                         (const bf16*)a.lk, a.n_query, a.n_key, a.dl, a.score_scale);
    };
    if (n <= 512)
      merge(k_topk_merge<KMAX, NOISE, 8>);
    else if (n <= 1024)
      merge(k_topk_merge<KMAX, NOISE, 16>);
    else
      merge(k_topk_merge<KMAX, NOISE, 0>);
    return hipGetLastError();
  }
  const int64_t rows = heads * a.n_query;
  KernelTimer timer(kKernScan, a.stream);
  hipLaunchKernelGGL((k_scan_topk_f32<KMAX, NOISE>), dim3((unsigned)((rows + 63) / 64)), dim3(64),
                     0, a.stream, (const float*)a.lq, (const float*)a.lk, a.q_pos, heads,
                     a.n_query, a.n_key, a.dl, a.score_scale, a.k, a.softmax_one, a.idx,
                     a.score, a.w, a.seed);
  return hipGetLastError();
}

template <int KMAX>
static hipError_t launch_scan_n(const ScanPlan& pl, const LaunchRetrieve& a) {
  return a.noise ? launch_scan_k<KMAX, true>(pl, a) : launch_scan_k<KMAX, false>(pl, a);
}

hipError_t launch_retrieve(const ScanPlan& pl, const LaunchRetrieve& a) {
  if (pl.kmax == 4) return launch_scan_n<4>(pl, a);
  if (pl.kmax == 8) return launch_scan_n<8>(pl, a);
  return launch_scan_n<16>(pl, a);
}

}  // namespace gca
