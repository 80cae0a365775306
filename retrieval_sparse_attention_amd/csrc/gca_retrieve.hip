// GCA retrieval: Eq. 1 relevance scores, top-k selection and Eq. 3 fusion weights.
//
// Definition (paperhub.cn review page, authors' reply "Cmt 1"; long-context-
// modeling README, "Model Architecture"): query chunk t scores every eligible
// past chunk j < q_pos[t] - 1 with r_j = score_scale * <lq_t, lk_j>, keeps the k
// best and weights them with softmax(r) (or softmax off-by-one, paperhub.cn
// authors' reply "Q4").
//
// bf16 path.  The scan is a dense contraction of 32 query landmarks with a
// stream of candidate landmarks, so it runs on MFMA and stays bound by the
// single pass over lk in HBM.  S^T = LK_block (32 x Dl) * LQ^T (Dl x 32) puts, in
// each lane, 16 scores of ONE query; the lane keeps its own sorted top-KMAX list
// in registers and only a score that beats the lane's current k-th best pays
// for an insertion.  Each workgroup (4 waves) covers one 32-query tile and one
// slice of candidates; its 8 lists per query are merged with a 3-level LDS
// tree.  Large candidate sets are cut into slices that a second kernel merges.
//
// f32 path.  One thread per query computes float32 dot products and the same
// sorted list; it serves the small float32 workloads.

#include "gca_device.h"
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
  float e[KMAX];
  float z = softmax_one ? expf(-shift) : 0.0f;
#pragma unroll
  for (int p = 0; p < KMAX; ++p) {
    e[p] = (p < m) ? expf(s[p] - shift) : 0.0f;
    z += e[p];
  }
  for (int p = 0; p < k; ++p) {
    float sv = 0.0f, wv = 0.0f;
    int iv = -1;
#pragma unroll
    for (int u = 0; u < KMAX; ++u)
      if (u == p && p < m) {
        sv = s[u];
        wv = e[u] / z;
        iv = id[u];
      }
    idx_out[p] = iv;
    score_out[p] = sv;
    w_out[p] = wv;
  }
}

// Merges two sorted lists held in LDS into the top KMAX of their union.
template <int KMAX>
__device__ __forceinline__ void merge_lists(const float* as, const int* ai, const float* bs,
                                            const int* bi, float (&os)[KMAX], int (&oi)[KMAX]) {
  int pa = 0, pb = 0;
#pragma unroll
  for (int p = 0; p < KMAX; ++p) {
    const float xa = as[pa], xb = bs[pb];
    const int ja = ai[pa], jb = bi[pb];
    const bool ta = better(xa, ja, xb, jb);
    os[p] = ta ? xa : xb;
    oi[p] = ta ? ja : jb;
    pa += ta ? 1 : 0;
    pb += ta ? 0 : 1;
  }
}

// ---------------------------------------------------------------------------
// bf16 scan.  Grid: heads * nsplit * n_qtiles workgroups of 256 threads.
// ---------------------------------------------------------------------------
template <int DL, int KMAX>
__global__ __launch_bounds__(256) void k_scan_topk_bf16(
    const bf16* __restrict__ lq, const bf16* __restrict__ lk, const int32_t* __restrict__ q_pos,
    int64_t n_query, int64_t n_key, int n_qtiles, int nsplit, int64_t split_len,
    float score_scale, int k, int softmax_one, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, float* __restrict__ w_out, float* __restrict__ part_s,
    int32_t* __restrict__ part_i) {
  constexpr int NKS = DL / 16;  // MFMA K-steps over the landmark dimension
  constexpr int HALF = DL / 2;  // landmark dims supplied by each lane half
  __shared__ float ls[8][32][KMAX];
  __shared__ int li[8][32][KMAX];

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
  // largest candidate count of the tile (all waves see the same 32 queries)
  int tile_max = (int)n_cand;  // n_key < 2^31 is checked on the host
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tile_max = max(tile_max, __shfl_xor(tile_max, o));
  const int64_t c_begin = (int64_t)sp * split_len;
  int64_t c_end = c_begin + split_len;
  if (c_end > tile_max) c_end = tile_max;

  bf16x8 bq[NKS];
  {
    const bf16* row = lq + (head * n_query + (q_ok ? q : 0)) * DL + HALF * half;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      bq[ks] = q_ok ? *(const bf16x8*)(row + 8 * ks) : zero_bf16x8();
  }

  float s[KMAX];
  int id[KMAX];
  list_clear(s, id);

  // Each wave walks blocks of 32 candidates (stride 128); the next block's
  // landmarks are loaded while the current block is scored.  Rows past n_key
  // are read from the last row (in bounds) and masked out by j < n_cand.
  const bf16* lk_head = lk + head * n_key * DL + HALF * half;
  auto load_block = [&](int64_t blk, bf16x8 (&a)[NKS]) {
    int64_t row = blk + col;
    row = row < n_key ? row : n_key - 1;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) a[ks] = *(const bf16x8*)(lk_head + row * DL + 8 * ks);
  };
  bf16x8 a[NKS];
  int64_t blk = c_begin + 32 * wave;
  if (blk < c_end) load_block(blk, a);
  for (; blk < c_end; blk += 128) {
    bf16x8 an[NKS];
    const bool more = blk + 128 < c_end;
    if (more) load_block(blk + 128, an);
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) acc = mfma32x32x16(a[ks], bq[ks], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t j = blk + c_row(r, half);
      const float x = acc[r] * score_scale;
      const bool hit = (j < c_end) && (j < n_cand) && better(x, (int)j, s[KMAX - 1], id[KMAX - 1]);
      if (hit) list_insert(s, id, x, (int)j);
    }
    if (more) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) a[ks] = an[ks];
    }
  }

  // 8 lists per query: g = 2 * wave + half.  Tree merge through LDS.
  const int g = 2 * wave + half;
#pragma unroll
  for (int p = 0; p < KMAX; ++p) {
    ls[g][col][p] = s[p];
    li[g][col][p] = id[p];
  }
  __syncthreads();
#pragma unroll
  for (int step = 1; step < 8; step <<= 1) {
    if ((g % (2 * step)) == 0) {
      merge_lists<KMAX>(ls[g][col], li[g][col], ls[g + step][col], li[g + step][col], s, id);
#pragma unroll
      for (int p = 0; p < KMAX; ++p) {
        ls[g][col][p] = s[p];
        li[g][col][p] = id[p];
      }
    }
    __syncthreads();
  }
  if (g == 0 && q_ok) {
    const int64_t qrow = head * n_query + q;
    if (nsplit == 1) {
      finalize_query<KMAX>(s, id, k, softmax_one, idx_out + qrow * k, score_out + qrow * k,
                           w_out + qrow * k);
    } else {
      float* ps = part_s + (qrow * nsplit + sp) * KMAX;
      int32_t* pi = part_i + (qrow * nsplit + sp) * KMAX;
#pragma unroll
      for (int p = 0; p < KMAX; ++p) {
        ps[p] = s[p];
        pi[p] = id[p];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of the per-slice lists.  One wave per (head, query), 4 per workgroup.
// ---------------------------------------------------------------------------
template <int KMAX>
__global__ __launch_bounds__(256) void k_topk_merge(
    const float* __restrict__ part_s, const int32_t* __restrict__ part_i, int64_t n_rows,
    int nsplit, int k, int softmax_one, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, float* __restrict__ w_out) {
  __shared__ float ls[4][64][KMAX];
  __shared__ int li[4][64][KMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t qrow = (int64_t)blockIdx.x * 4 + wave;
  const bool ok = qrow < n_rows;
  float s[KMAX];
  int id[KMAX];
  list_clear(s, id);
  if (ok) {
    const int64_t n = (int64_t)nsplit * KMAX;
    const float* ps = part_s + qrow * n;
    const int32_t* pi = part_i + qrow * n;
    for (int64_t e = lane; e < n; e += 64) {
      const float x = ps[e];
      const int j = pi[e];
      if (j != kIdxNone && better(x, j, s[KMAX - 1], id[KMAX - 1])) list_insert(s, id, x, j);
    }
  }
#pragma unroll
  for (int p = 0; p < KMAX; ++p) {
    ls[wave][lane][p] = s[p];
    li[wave][lane][p] = id[p];
  }
  __syncthreads();
#pragma unroll
  for (int step = 1; step < 64; step <<= 1) {
    if ((lane % (2 * step)) == 0) {
      merge_lists<KMAX>(ls[wave][lane], li[wave][lane], ls[wave][lane + step],
                        li[wave][lane + step], s, id);
#pragma unroll
      for (int p = 0; p < KMAX; ++p) {
        ls[wave][lane][p] = s[p];
        li[wave][lane][p] = id[p];
      }
    }
    __syncthreads();
  }
  if (ok && lane == 0)
    finalize_query<KMAX>(s, id, k, softmax_one, idx_out + qrow * k, score_out + qrow * k,
                         w_out + qrow * k);
}

// ---------------------------------------------------------------------------
// float32 scan: one thread per (head, query).
// ---------------------------------------------------------------------------
template <int KMAX>
__global__ __launch_bounds__(64) void k_scan_topk_f32(
    const float* __restrict__ lq, const float* __restrict__ lk, const int32_t* __restrict__ q_pos,
    int64_t n_heads, int64_t n_query, int64_t n_key, int dl, float score_scale, int k,
    int softmax_one, int32_t* __restrict__ idx_out, float* __restrict__ score_out,
    float* __restrict__ w_out) {
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
    const float x = acc * score_scale;
    if (better(x, (int)j, s[KMAX - 1], id[KMAX - 1])) list_insert(s, id, x, (int)j);
  }
  finalize_query<KMAX>(s, id, k, softmax_one, idx_out + qrow * k, score_out + qrow * k,
                       w_out + qrow * k);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <int KMAX>
static hipError_t launch_scan_k(const ScanPlan& pl, const LaunchRetrieve& a) {
  const int64_t heads = a.G * a.B * a.H;
  if (a.dtype == 1) {
    const int64_t nblk = heads * pl.nsplit * pl.n_qtiles;
    {
    KernelTimer timer(kKernScan, a.stream);
    if (a.dl == 64)
      hipLaunchKernelGGL((k_scan_topk_bf16<64, KMAX>), dim3((unsigned)nblk), dim3(256), 0,
                         a.stream, (const bf16*)a.lq, (const bf16*)a.lk, a.q_pos, a.n_query,
                         a.n_key, pl.n_qtiles, pl.nsplit, pl.split_len, a.score_scale, a.k,
                         a.softmax_one, a.idx, a.score, a.w, a.part_s, a.part_i);
    else
      hipLaunchKernelGGL((k_scan_topk_bf16<32, KMAX>), dim3((unsigned)nblk), dim3(256), 0,
                         a.stream, (const bf16*)a.lq, (const bf16*)a.lk, a.q_pos, a.n_query,
                         a.n_key, pl.n_qtiles, pl.nsplit, pl.split_len, a.score_scale, a.k,
                         a.softmax_one, a.idx, a.score, a.w, a.part_s, a.part_i);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.nsplit == 1) return e;
    const int64_t rows = heads * a.n_query;
    KernelTimer timer(kKernMerge, a.stream);
    hipLaunchKernelGGL((k_topk_merge<KMAX>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                       a.stream, a.part_s, a.part_i, rows, pl.nsplit, a.k, a.softmax_one, a.idx,
                       a.score, a.w);
    return hipGetLastError();
  }
  const int64_t rows = heads * a.n_query;
  KernelTimer timer(kKernScan, a.stream);
  hipLaunchKernelGGL((k_scan_topk_f32<KMAX>), dim3((unsigned)((rows + 63) / 64)), dim3(64), 0,
                     a.stream, (const float*)a.lq, (const float*)a.lk, a.q_pos, heads,
                     a.n_query, a.n_key, a.dl, a.score_scale, a.k, a.softmax_one, a.idx,
                     a.score, a.w);
  return hipGetLastError();
}

hipError_t launch_retrieve(const ScanPlan& pl, const LaunchRetrieve& a) {
  if (pl.kmax == 4) return launch_scan_k<4>(pl, a);
  if (pl.kmax == 8) return launch_scan_k<8>(pl, a);
  return launch_scan_k<16>(pl, a);
}

}  // namespace gca
