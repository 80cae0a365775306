/*
 * gca.h -- C ABI of the Grouped Cross Attention (GCA) hot path for AMD Instinct
 * MI355X (gfx950).
 *
 * GCA is the retrieval attention of the Differentiable Retrieval-based
 * Transformer ("Efficient Length-Generalizable Attention via Causal Retrieval
 * for Long-Context Language Modeling", Hu et al., ICML 2025).  The sequence is
 * cut into chunks of S tokens; each query chunk uses a landmark vector to score
 * past chunks, keeps the top-k, attends to each retrieved chunk separately and
 * fuses the k results with softmax-normalised relevance weights.
 *
 * Three calls cover the path, in the order a training step makes them:
 *   gca_retrieve  -- relevance scores, top-k selection, fusion weights
 *   gca_forward   -- per-chunk attention of every token + weighted fusion
 *   gca_backward  -- gradients of Q, K, V, the weights, the scores and the
 *                    landmarks
 * and the calls around them:
 *   gca_retrieve_gumbel -- gca_retrieve with Gumbel-noised selection (training)
 *   gca_gather_kv       -- packs the retrieved K/V tiles, e.g. out of pinned
 *                          host memory, for K/V offloaded from the GPU
 *   gca_swa_forward / gca_swa_backward -- the layer's causal sliding-window
 *                          self-attention
 * An upper layer group reuses one gca_retrieve (and one K/V) for all of its
 * layers: each layer calls gca_forward, then gca_backward_accumulate, with the
 * same idx, w, K and V; the library adds every layer's gradients of the shared
 * tensors into float32 accumulators.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *   never allocates or frees device memory.  Its only state is a thread-local
 *   error string, while enabled the event timing records below, and the
 *   fixed device array of gca_retrieve_noalloc.
 * - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream) and
 *   return without synchronising.
 * - All arrays are dense, contiguous, row-major, with the layouts given below.
 *   G (retrieval groups) is an independent leading axis: every (g, b, h) slice
 *   is a separate problem.  Tensors named "big" below must be 16-byte aligned,
 *   the others 4-byte aligned.
 * - Outputs are fully overwritten.  Empty slots (fewer candidates than k, or an
 *   index outside [0, n_key) passed to forward/backward) read as idx = -1,
 *   score = w = dw = dscore = 0 and lse = -inf; chunks nobody retrieved get
 *   dk = dv = dlk = 0.
 * - Every argument is checked before anything is launched.  On failure the call
 *   returns GCA_ERR_INVALID_ARGUMENT / GCA_ERR_UNSUPPORTED / GCA_ERR_WORKSPACE,
 *   touches no output and sets gca_last_error().  A failed launch returns
 *   GCA_ERR_DEVICE with the HIP error text in gca_last_error().
 * - NaN: in gca_forward and gca_backward a NaN in Q, K, V or dO reaches
 *   every output element that depends on it, in the pattern exact arithmetic
 *   gives (e.g. a NaN in K of chunk c makes every O and L row of the slots
 *   that retrieved c NaN; one in V makes one column of those O tiles NaN),
 *   so a diverging step is not masked.  Retrieval orders finite scores only:
 *   which chunks a NaN score selects is unspecified.
 * - Setting the environment variable GCA_DEBUG_SYNC=1 makes every call
 *   synchronise its stream and check for device errors before returning.
 *
 * Supported sizes (anything else returns GCA_ERR_UNSUPPORTED):
 *   dtype GCA_BF16 : chunk_size 1..64, head_dim 1..64, landmark_dim 32 or 64
 *                    (gca_forward / gca_backward run MFMA kernels at
 *                    chunk_size 64, the pages' chunk size, and 16, each with
 *                    head_dim 64 or 32; other sizes take a float32 VALU path
 *                    with bf16 loads and one rounding of each output, correct
 *                    but about two orders of magnitude slower)
 *   dtype GCA_F32  : chunk_size 1..64, head_dim 1..64, landmark_dim 1..128
 *   top_k 1..16; n_key < 2^31 - 1; at most 2^31 - 1 query or key chunk tiles
 *   (G*B*H*n_query, G*B*H*n_key); gca_backward needs n_query * top_k < 2^31.
 */
#ifndef GCA_H
#define GCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GCA_ABI_VERSION 2

typedef int gca_status;
enum {
  GCA_OK = 0,
  GCA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size or flag */
  GCA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (see sizes above) */
  GCA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
  GCA_ERR_DEVICE = 4            /* a HIP launch or device error */
};

typedef int gca_dtype;
enum {
  GCA_F32 = 0, /* float32 q, k, v, o, dout, dq, dk, dv, lq, lk */
  GCA_BF16 = 1 /* bfloat16 for the same tensors; accumulation is float32 */
};

/* Problem description shared by the three calls. */
typedef struct {
  int64_t G;            /* retrieval groups (independent problems)          */
  int64_t B;            /* batch                                            */
  int64_t H;            /* heads; retrieval is per (g, b, h)                */
  int64_t n_query;      /* Nq: query chunks                                 */
  int64_t n_key;        /* Nk: resident (candidate) chunks                  */
  int32_t chunk_size;   /* S: tokens per chunk (query and key chunks)       */
  int32_t head_dim;     /* D                                                */
  int32_t landmark_dim; /* Dl: length of one landmark vector per head       */
  int32_t top_k;        /* k: chunks retrieved per query chunk              */
  int32_t dtype;        /* gca_dtype of the "big" tensors                   */
  int32_t softmax_one;  /* 0: softmax fusion weights; 1: softmax off-by-one */
  float attn_scale;     /* token logit scale, usually 1/sqrt(D)             */
  float score_scale;    /* relevance score scale, usually 1/sqrt(Dl)        */
} gca_shape;

/* Returns GCA_ABI_VERSION of the loaded library. */
int gca_abi_version(void);

/* Static text for a status code (never NULL). */
const char* gca_status_string(gca_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* gca_last_error(void);

/* Device workspace needed by an operation: op 0 = gca_retrieve,
 * 1 = gca_forward (always 0), 2 = gca_backward.  *bytes receives the size;
 * a workspace of at least that many bytes, 256-byte aligned, must be passed. */
gca_status gca_workspace_size(const gca_shape* shape, int op, size_t* bytes);

/*
 * gca_retrieve -- Eq. 1 relevance scores, top-k and Eq. 3 fusion weights.
 *
 * Definition: paperhub.cn review page, authors' reply "Cmt 1" (score of past
 * chunk j for query chunk t is <lq_t, lk_j> / sqrt(d)); long-context-modeling
 * README, "Model Architecture" (a chunk retrieves the top-k past chunks with the
 * landmark of the chunk before it; their softmax-normalised scores are the
 * fusion weights); paperhub.cn, authors' reply "Q4" (softmax off-by-one).
 *
 * For every (g, b, h, t):  candidates j = 0 .. min(q_pos[t] - 1, n_key) - 1,
 *   r_j = score_scale * <lq[g,b,h,t,:], lk[g,b,h,j,:]>   (float32 accumulate)
 *   the min(k, #candidates) best by (r descending, j ascending) are written to
 *   idx[.., 0:m] in ascending j, with score = r and
 *   w = e^r / sum e^r               (softmax_one = 0)
 *   w = e^r / (1 + sum e^r)         (softmax_one = 1), sums over the m kept.
 *
 *   lq    [G, B, H, Nq, Dl]   dtype, big        query landmarks
 *   lk    [G, B, H, Nk, Dl]   dtype, big        candidate landmarks
 *   q_pos [Nq]                int32             chunk position of each query
 *                                               chunk (training: q_pos[t] = t)
 *   idx   [G, B, H, Nq, k]    int32   output
 *   score [G, B, H, Nq, k]    float32 output
 *   w     [G, B, H, Nq, k]    float32 output
 *   ws / ws_bytes             workspace (gca_workspace_size op 0)
 *
 * With dtype GCA_BF16, score_scale must be > 0 (else GCA_ERR_UNSUPPORTED): the
 * scan prunes candidates on unscaled dot products, whose order is the order of
 * r only for a positive scale.  GCA_F32 takes any finite scale.
 */
gca_status gca_retrieve(const gca_shape* shape, const void* lq, const void* lk,
                        const int32_t* q_pos, int32_t* idx, float* score, float* w,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * gca_retrieve_noalloc -- gca_retrieve for callers that cannot allocate.
 *
 * For callers that may not call hipMalloc or take a workspace from an
 * allocator: code under HIP graph capture, tight serving loops (one retrieval
 * per 64-token chunk step), harnesses that forbid allocation.  Same arguments,
 * layouts, results and errors as gca_retrieve, without ws / ws_bytes: the
 * partial top-k lists of a sliced scan go to a scratch array the library owns,
 * 4 MiB per device (a file-scope device array each GPU holds until the process
 * ends; its address is looked up once per device).  The call allocates
 * nothing.  A shape whose gca_workspace_size (op 0) exceeds 4 MiB is refused
 * with GCA_ERR_UNSUPPORTED before anything is launched (every shape whose
 * scan is not sliced needs none).  All calls on one GPU share that GPU's
 * array: two calls that overlap in time on one device (on different streams,
 * or from different threads) race on it and give undefined results; calls
 * ordered on one stream do not.
 */
gca_status gca_retrieve_noalloc(const gca_shape* shape, const void* lq, const void* lk,
                                const int32_t* q_pos, int32_t* idx, float* score, float* w,
                                void* stream);

/*
 * gca_retrieve_gumbel -- gca_retrieve with Gumbel top-k selection (training).
 *
 * Definition: paperlayer.ai summary, section 3.2 (Training & Inference): while
 * training, Gumbel noise is added to the relevance scores before the top-k
 * selection, so that lower-scoring chunks keep a chance of being retrieved;
 * section 5 credits Gumbel top-k sampling for pre-training up to 64K tokens.
 *
 * Same arguments, layouts, workspace (gca_workspace_size op 0) and errors as
 * gca_retrieve, plus `seed`.  For every (g, b, h, t) and candidate j:
 *   G_j = -ln(-ln U_j),  U_j = (m + 1/2) / 2^23,  m = top 23 bits of word
 *   (j mod 4) of Philox4x32-10 (Salmon et al., SC 2011) with counter
 *   (j / 4, t, (g*B + b)*H + h, 0) and key (seed mod 2^32, seed / 2^32);
 *   the min(k, #candidates) best by (r_j + G_j descending, j ascending) are
 *   selected (r_j + G_j formed as fma(dot, score_scale, G_j) in float32, with
 *   G_j computed in float32 to within a few 1e-6 of its exact value: the
 *   hardware base-2 logarithm is not correctly rounded);
 *   idx holds them in ascending j; score = the clean r_j of each selected
 *   chunk (float32 dot product times score_scale) and w = Eq. 3 over those
 *   clean scores, exactly as in gca_retrieve.  So gradients of w reach r, and
 *   the noise only decides which chunks are kept.
 * The same seed gives the same result on every call and for every workspace
 * plan; the noise of a candidate does not depend on n_key or on other queries.
 */
gca_status gca_retrieve_gumbel(const gca_shape* shape, uint64_t seed, const void* lq,
                               const void* lk, const int32_t* q_pos, int32_t* idx,
                               float* score, float* w, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * gca_gather_kv -- packs the retrieved K/V tiles, for K/V kept in host memory.
 *
 * Definition: paperlayer.ai summary, section 3.2 (past chunk representations
 * may be offloaded to CPU memory; the transfers retrieval needs happen only
 * when it runs); paperhub.cn review page, authors' reply "Q2" (the offloaded
 * GCA K/V is shared within a group; a host link above 20 GB/s suffices).
 *
 * For every (g, b, h, t) and slot i with c = idx[g,b,h,t,i]:
 *   c in [0, n_key):  k_packed[g,b,h, t*k + i] = k[g,b,h,c] (one S x D tile),
 *                     v_packed likewise, idx_packed[g,b,h,t,i] = t*k + i
 *   otherwise:        zero tiles and idx_packed = -1.
 * gca_forward over (k_packed, v_packed, idx_packed) with a shape whose n_key
 * is n_query * top_k gives the same O and lse, bit for bit, as over (k, v, idx):
 * only k tiles per query chunk cross the host link instead of the whole K/V.
 * (gca_backward over packed arrays returns dK/dV per packed row, i.e. per
 * retrieved slot; summing the rows that hold chunk c gives dK/dV of chunk c.)
 *
 *   shape           G, B, H, n_query, n_key, chunk_size, head_dim, top_k, dtype
 *                   (the same limits as gca_forward)
 *   idx        [G, B, H, Nq, k]          int32, device memory
 *   k, v       [G, B, H, Nk, S, D]       dtype, big; device memory OR pinned host
 *                                        memory (hipHostMalloc); other host memory
 *                                        is refused with GCA_ERR_INVALID_ARGUMENT
 *   k_packed, v_packed [G, B, H, Nq*k, S, D]  dtype, big, device, output
 *   idx_packed [G, B, H, Nq, k]          int32, device, output
 * The whole [G, B, H, Nk, S, D] range of k and v must lie in one allocation.
 */
gca_status gca_gather_kv(const gca_shape* shape, const int32_t* idx, const void* k,
                         const void* v, void* k_packed, void* v_packed, int32_t* idx_packed,
                         void* stream);

/*
 * Sliding-window self-attention -- the other attention of a DRT layer.
 *
 * Definition: paperlayer.ai summary, section 1 and section 3.2 (every layer
 * pairs GCA with fixed-size sliding-window self-attention, keeping the cost
 * linear in the sequence) and section 4.1.2 (a 512-token window).  Token x of
 * a (b, h) sequence attends to the keys y with x - window < y <= x:
 *   O[x] = sum_y P[x,y] V[y],  P[x,.] = softmax_y(scale <Q[x], K[y]>),
 *   lse[x] = log sum_y exp(scale <Q[x], K[y]>)                (float32)
 * Backward, with D[x] = <dO[x], O[x]> (O as written by the forward):
 *   dS = P (dO V^T - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
 *
 *   q, k, v, o, dout, dq, dk, dv   [B, H, T, head_dim]   bf16, big
 *   lse                            [B, H, T]             float32
 * Supported: dtype GCA_BF16, head_dim 64, T a multiple of 64 (whole 64-token
 * chunks) below 2^30, window >= 1 (any value; windows >= T give causal
 * attention), B*H*T/64 < 2^31.  Same conventions, checks and errors as the GCA calls.
 * gca_swa_forward needs scale >= 0, as gca_forward does for bf16 (else
 * GCA_ERR_UNSUPPORTED).
 * gca_swa_backward needs a workspace of gca_swa_workspace_size bytes (D rows).
 */
typedef struct {
  int64_t B, H, T;  /* batch, heads, tokens per sequence */
  int32_t head_dim; /* D */
  int32_t window;   /* W */
  gca_dtype dtype;
  float scale;      /* usually 1/sqrt(head_dim) */
} gca_swa_shape;

gca_status gca_swa_workspace_size(const gca_swa_shape* shape, size_t* bytes);

gca_status gca_swa_forward(const gca_swa_shape* shape, const void* q, const void* k,
                           const void* v, void* o, float* lse /* or NULL */, void* stream);

gca_status gca_swa_backward(const gca_swa_shape* shape, const void* q, const void* k,
                            const void* v, const void* o, const float* lse, const void* dout,
                            void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * gca_forward -- Eq. 2 per-chunk attention and Eq. 3 weighted fusion.
 *
 * Definition: long-context-modeling README, "Model Architecture" (first stage:
 * each token attends to the tokens of each retrieved chunk separately, giving
 * O^i; second stage: weighted sum of the O^i); paperlayer.ai summary,
 * appendix B (the kernel returns O and the log-sum-exp L).
 *
 * For every (g, b, h, t), token x < S and slot i with c = idx[.., t, i] in
 * [0, n_key):
 *   s_j   = attn_scale * <q[.., t, x, :], k[.., c, j, :]>,  j < S (no mask)
 *   lse   = log sum_j exp(s_j)            -> lse[.., t, i, x]
 *   O^i   = sum_j exp(s_j - lse) v[.., c, j, :]
 *   o[.., t, x, :] = sum_i w[.., t, i] * O^i   (float32, rounded once)
 *
 *   q     [G, B, H, Nq, S, D]  dtype, big
 *   k, v  [G, B, H, Nk, S, D]  dtype, big
 *   idx   [G, B, H, Nq, k]     int32      (from gca_retrieve, any order)
 *   w     [G, B, H, Nq, k]     float32
 *   o     [G, B, H, Nq, S, D]  dtype, big, output
 *   lse   [G, B, H, Nq, k, S]  float32 output, may be NULL (then not written;
 *                              gca_backward needs it)
 *
 * With dtype GCA_BF16, chunk_size 64 or 16 and head_dim 64 or 32, attn_scale must be >= 0
 * (else GCA_ERR_UNSUPPORTED): those kernels subtract each row's largest unscaled
 * product before exponentiating, which bounds the exponents only for a
 * non-negative scale.
 */
gca_status gca_forward(const gca_shape* shape, const void* q, const void* k,
                       const void* v, const int32_t* idx, const float* w, void* o,
                       float* lse, void* stream);

/*
 * gca_retrieve_forward -- gca_retrieve followed by gca_forward in one call.
 *
 * Definition: as gca_retrieve and gca_forward (long-context-modeling README,
 * "Model Architecture": a chunk retrieves its top-k past chunks, then attends
 * to each and fuses the results), with the retrieval's idx and w feeding the
 * forward.  The outputs are those of the two calls made in turn, bit for bit:
 * idx, score, w as gca_retrieve writes them, o and lse as gca_forward writes
 * them from that idx and w.
 *
 *   lq, lk, q_pos, idx, score, w  as for gca_retrieve (idx, score, w outputs)
 *   q, k, v, o, lse               as for gca_forward
 *   ws / ws_bytes                 workspace of the retrieval (gca_workspace_size
 *                                 op 0); the forward needs none
 *
 * When the retrieval is cut into slices (long candidate lists) and the chunks
 * are bf16 with chunk_size 64 and head_dim 64 or 32, the merge of the slices'
 * lists runs inside the forward's kernel, which saves a launch and a round
 * trip to memory on latency-bound steps (decoding, long-context retrieval).
 * Every argument of both parts is checked before anything is launched; the
 * conditions and error codes are those of gca_retrieve and gca_forward.
 */
gca_status gca_retrieve_forward(const gca_shape* shape, const void* lq, const void* lk,
                                const int32_t* q_pos, const void* q, const void* k,
                                const void* v, int32_t* idx, float* score, float* w, void* o,
                                float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * gca_backward -- gradients of the forward and of the fusion weights/scores.
 *
 * Definition: paperlayer.ai summary, appendix B (the backward returns gradients
 * for Q, K, V and the weights); long-context-modeling README, "Model
 * Architecture" (back-propagation reaches the retrieval scores through the
 * weights); Eq. 1 as for gca_retrieve.  With dO = dL/do:
 *   dw_i   = sum_x <dO[x], O^i[x]>
 *   dS     = w_i P (dO v_c^T - rowsum(dO * O^i))        per (t, i) pair
 *   dq_t  += attn_scale dS k_c,   dk_c += attn_scale dS^T q_t,
 *   dv_c  += w_i P^T dO
 *   dscore_i = w_i (dw_i - sum_l w_l dw_l)   (valid for both weight forms,
 *                                            w must come from gca_retrieve)
 *   dlq_t += score_scale sum_i dscore_i lk_c,   dlk_c += score_scale dscore_i lq_t
 * Top-k selection is treated as fixed.  Sums over (t, i) run in a fixed order,
 * so results are bitwise reproducible.  The bf16 path forms w_i P directly
 * (log2 w_i joins the exponent); a slot whose weight is below about 1e-35
 * (far below any contribution to dq, dk, dv or dscore) reports dw_i = 0.
 *
 *   q, dout        [G, B, H, Nq, S, D]  dtype, big
 *   k, v           [G, B, H, Nk, S, D]  dtype, big
 *   idx, w         [G, B, H, Nq, k]     int32 / float32 (as passed to forward)
 *   lse            [G, B, H, Nq, k, S]  float32 from gca_forward
 *   lq, lk         landmarks as in gca_retrieve; may be NULL only if dlq/dlk
 *                  (respectively dlk/dlq) are NULL; lk is never read when
 *                  n_key = 0 (every slot is then empty and dlq = 0)
 *   dq             [G, B, H, Nq, S, D]  dtype output
 *   dk, dv         [G, B, H, Nk, S, D]  dtype output
 *   dw, dscore     [G, B, H, Nq, k]     float32 output
 *   dlq            [G, B, H, Nq, Dl]    float32 output or NULL
 *   dlk            [G, B, H, Nk, Dl]    float32 output or NULL
 *   ws / ws_bytes  workspace (gca_workspace_size op 2)
 * dlq needs lk (unless n_key = 0); dlk needs lq.
 *
 * Streams: three kernels (the reverse index of the retrieved chunks, the
 * query side, the key side) run in order on `stream`; the call keeps no
 * stream or event of its own, so it can be captured into a HIP graph.
 */
gca_status gca_backward(const gca_shape* shape, const void* q, const void* k,
                        const void* v, const int32_t* idx, const float* w,
                        const float* lse, const void* dout, const void* lq,
                        const void* lk, void* dq, void* dk, void* dv, float* dw,
                        float* dscore, float* dlq, float* dlk, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * gca_backward_accumulate -- gca_backward for the upper layers of a group that
 * share one retrieval and one K/V, summing the shared gradients in the library.
 *
 * Definition: paperlayer.ai summary, section 3.1 (the retrieved chunks'
 * representations, and the key/value transformations, are shared across the
 * upper layers of a group); paperhub.cn review page, authors' reply "Q2" (the
 * GCA K/V is shared within a group).  Each upper layer l brings its own
 * queries q_l and upstream gradient dO_l and attends with the same idx, w, K,
 * V; the loss is a sum over layers, so the gradients of the shared tensors
 * are the sums over layers of gca_backward's per-layer values.
 *
 * Same arguments, checks, workspace (gca_workspace_size op 2) and errors as
 * gca_backward, with these outputs:
 *   dq          [G, B, H, Nq, S, D]  dtype, big: this layer's dQ (overwritten)
 *   dk_acc, dv_acc [G, B, H, Nk, S, D] float32, big: dK, dV of this layer
 *               are ADDED (float32, before any rounding)
 *   dw_acc, dscore_acc [G, B, H, Nq, k] float32: dw, dscore ADDED
 *   dlq_acc [G, B, H, Nq, Dl], dlk_acc [G, B, H, Nk, Dl] float32 or NULL: ADDED
 * The caller zeroes the accumulators before the first layer and calls once per
 * layer on one stream; each element's sum then runs over the layers in call
 * order, and each layer's own terms in gca_backward's fixed order, so results
 * are bitwise reproducible.  Rounding the float32 sums (e.g. to bf16) is the
 * caller's.
 */
gca_status gca_backward_accumulate(const gca_shape* shape, const void* q, const void* k,
                                   const void* v, const int32_t* idx, const float* w,
                                   const float* lse, const void* dout, const void* lq,
                                   const void* lk, void* dq, float* dk_acc, float* dv_acc,
                                   float* dw_acc, float* dscore_acc, float* dlq_acc,
                                   float* dlk_acc, void* ws, size_t ws_bytes, void* stream);

/*
 * Per-kernel timing with HIP events (benchmarks, profiling).
 *
 * gca_timing_enable(1) makes every later call record a HIP event before and
 * after each kernel it launches, on that call's stream (a small cost per
 * launch); gca_timing_enable(0) stops recording.  gca_timing_collect() waits
 * for the recorded events, then writes per-kernel sums since the previous
 * collect into total_ms[i] (milliseconds) and launches[i] (count) for
 * i < gca_num_kernels(), and resets the sums.  Either array may be NULL.
 * Returns GCA_ERR_DEVICE if an event could not be read.  Thread-safe.
 * gca_kernel_name(i) names kernel i ("" outside the range).
 */
int gca_num_kernels(void);
const char* gca_kernel_name(int kernel_id);
gca_status gca_timing_enable(int on);
gca_status gca_timing_collect(double* total_ms, int64_t* launches);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* GCA_H */
