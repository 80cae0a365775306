// C ABI of the GCA hot path: argument checks, workspace sizing and launches.
// Everything here runs on the host; the checks finish before any HIP call, so
// a rejected call has touched neither the device nor any output.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gca.h"
#include "gca_peaks.h"
#include "gca_launch.h"

namespace {

thread_local char g_err[512] = "";

gca_status fail(gca_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("GCA_DEBUG_SYNC");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

gca_status device_status(hipError_t e, hipStream_t stream, const char* what) {
  if (e == hipSuccess && debug_sync()) {
    e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess)
    return fail(GCA_ERR_DEVICE, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
  g_err[0] = '\0';
  return GCA_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

enum Op { kRetrieve = 0, kForward = 1, kBackward = 2 };

struct Sizes {
  int64_t heads;    // G * B * H
  int64_t q_rows;   // heads * n_query
  int64_t k_rows;   // heads * n_key
  int64_t q_elems;  // q_rows * S * D
  int64_t k_elems;  // k_rows * S * D
  int64_t slots;    // q_rows * top_k
};

gca_status check_shape(const gca_shape* s, int op, Sizes* z) {
  if (s == nullptr) return fail(GCA_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->G < 1 || s->B < 1 || s->H < 1)
    return fail(GCA_ERR_INVALID_ARGUMENT, "G, B, H must be >= 1 (got %lld, %lld, %lld)",
                (long long)s->G, (long long)s->B, (long long)s->H);
  if (s->n_query < 0 || s->n_key < 0)
    return fail(GCA_ERR_INVALID_ARGUMENT, "n_query and n_key must be >= 0");
  if (s->n_key > 0x7ffffffeLL)
    return fail(GCA_ERR_INVALID_ARGUMENT, "n_key must be below 2^31 - 1");
  if (s->chunk_size < 1 || s->head_dim < 1 || s->landmark_dim < 1)
    return fail(GCA_ERR_INVALID_ARGUMENT, "chunk_size, head_dim, landmark_dim must be >= 1");
  if (s->top_k < 1) return fail(GCA_ERR_INVALID_ARGUMENT, "top_k must be >= 1");
  if (s->top_k > 16) return fail(GCA_ERR_UNSUPPORTED, "top_k > 16 is not supported");
  if (s->dtype != GCA_F32 && s->dtype != GCA_BF16)
    return fail(GCA_ERR_INVALID_ARGUMENT, "dtype must be GCA_F32 or GCA_BF16");
  if (s->softmax_one != 0 && s->softmax_one != 1)
    return fail(GCA_ERR_INVALID_ARGUMENT, "softmax_one must be 0 or 1");
  if (!std::isfinite(s->attn_scale) || !std::isfinite(s->score_scale))
    return fail(GCA_ERR_INVALID_ARGUMENT, "attn_scale and score_scale must be finite");
  if (s->dtype == GCA_BF16) {
    if (op != kRetrieve && (s->chunk_size > 64 || s->head_dim > 64))
      return fail(GCA_ERR_UNSUPPORTED, "bf16 attention needs chunk_size, head_dim <= 64");
    if (op != kForward && s->landmark_dim != 32 && s->landmark_dim != 64)
      return fail(GCA_ERR_UNSUPPORTED, "bf16 landmarks need landmark_dim 32 or 64");
  } else {
    if (s->chunk_size > 64 || s->head_dim > 64)
      return fail(GCA_ERR_UNSUPPORTED, "f32 attention needs chunk_size, head_dim <= 64");
    if (s->landmark_dim > 128)
      return fail(GCA_ERR_UNSUPPORTED, "f32 landmarks need landmark_dim <= 128");
  }
  Sizes t{};
  int64_t gb, td;
  if (!mul_ok(s->G, s->B, &gb) || !mul_ok(gb, s->H, &t.heads) ||
      !mul_ok(t.heads, s->n_query, &t.q_rows) || !mul_ok(t.heads, s->n_key, &t.k_rows) ||
      !mul_ok((int64_t)s->chunk_size, s->head_dim, &td) || !mul_ok(t.q_rows, td, &t.q_elems) ||
      !mul_ok(t.k_rows, td, &t.k_elems) || !mul_ok(t.q_rows, s->top_k, &t.slots) ||
      t.q_elems > (int64_t(1) << 50) || t.k_elems > (int64_t(1) << 50))
    return fail(GCA_ERR_INVALID_ARGUMENT, "tensor sizes overflow");
  if (t.q_rows > 0x7fffffffLL || t.k_rows > 0x7fffffffLL)
    return fail(GCA_ERR_UNSUPPORTED, "more than 2^31 - 1 query or key chunk tiles");
  if (op == kBackward && s->n_query * (int64_t)s->top_k > 0x7fffffffLL)
    return fail(GCA_ERR_UNSUPPORTED, "n_query * top_k must be below 2^31");
  if (z) *z = t;
  return GCA_OK;
}

#ifndef GCA_SCAN_TARGET_WGS
#define GCA_SCAN_TARGET_WGS 768
#endif
constexpr int64_t kScanTargetWgs = GCA_SCAN_TARGET_WGS;
constexpr int64_t kMergeMax = 4096;  // partial keys per query the merge kernel holds in LDS
constexpr int64_t kFewQueries = 4;   // query chunks per head up to which k_scan_few_bf16 runs
constexpr int64_t kFewSlice = 256;   // its candidates per workgroup

gca::ScanPlan plan_scan(const gca_shape* s, const Sizes& z) {
  gca::ScanPlan p{};
  p.kmax = s->top_k <= 4 ? 4 : (s->top_k <= 8 ? 8 : 16);
  p.n_qtiles = (int)((s->n_query + 31) / 32);
  p.nsplit = 1;
  p.split_len = 128;
  if (s->dtype != GCA_BF16 || s->n_key <= 1024) {
    p.split_len = ((s->n_key + 127) / 128) * 128;
    if (p.split_len == 0) p.split_len = 128;
    return p;
  }
  // Slice the candidates so that the grid has about kScanTargetWgs workgroups,
  // with slices of whole 128-candidate rounds and at most kMergeMax partial
  // entries per query for the merge.
  const int64_t base = z.heads * (p.n_qtiles > 0 ? p.n_qtiles : 1);
  const int64_t max_split = (s->n_key + 127) / 128;
  int64_t want = (kScanTargetWgs + base - 1) / base;
  if (want > max_split) want = max_split;
  if (want > kMergeMax / p.kmax) want = kMergeMax / p.kmax;
  if (want < 1) want = 1;
  int64_t len = (s->n_key + want - 1) / want;
  len = ((len + 127) / 128) * 128;
  p.split_len = len;
  p.nsplit = (int)((s->n_key + len - 1) / len);
  // A few queries per head (decoding steps): slices of 256 candidates, one
  // workgroup per (head, query, slice), while the merge can hold the lists.
  const int64_t few_split = (s->n_key + kFewSlice - 1) / kFewSlice;
  if (s->n_query <= kFewQueries && few_split * p.kmax <= kMergeMax) {
    p.few = 1;
    p.split_len = kFewSlice;
    p.nsplit = (int)few_split;
  }
  return p;
}

struct RetrieveWs {
  size_t part, total;
};

RetrieveWs retrieve_ws(const gca_shape* s, const Sizes& z, const gca::ScanPlan& p) {
  RetrieveWs w{0, 0};
  if (p.nsplit <= 1) return w;
  const size_t n = (size_t)z.q_rows * (size_t)p.nsplit * (size_t)p.kmax;
  w.part = 0;
  w.total = align_up(n * sizeof(uint64_t));
  (void)s;
  return w;
}

struct BackwardWs {
  size_t delta, rev_off, rev_ent, ds_layer, total;
};

BackwardWs backward_ws(const gca_shape* s, const Sizes& z) {
  BackwardWs w{};
  w.delta = 0;
  w.rev_off = align_up((size_t)z.slots * (size_t)s->chunk_size * sizeof(float));
  w.rev_ent = w.rev_off + align_up((size_t)z.heads * (size_t)(s->n_key + 1) * sizeof(int32_t));
  w.ds_layer = w.rev_ent + align_up((size_t)z.slots * sizeof(int32_t));
  w.total = w.ds_layer + align_up((size_t)z.slots * sizeof(float));
  return w;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

gca_status need(const void* p, const char* name, size_t align) {
  if (p == nullptr) return fail(GCA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(p, align))
    return fail(GCA_ERR_INVALID_ARGUMENT, "%s is not %zu-byte aligned", name, align);
  return GCA_OK;
}

gca_status opt(const void* p, const char* name, size_t align) {
  if (p != nullptr && !aligned(p, align))
    return fail(GCA_ERR_INVALID_ARGUMENT, "%s is not %zu-byte aligned", name, align);
  return GCA_OK;
}

// Device-side address of a buffer the GPU may read: device or managed memory
// as is; pinned host memory through the address its mapping has on the
// device.  Unregistered host memory is refused: a kernel reading it would
// fault.
gca_status readable_on_device(const void* p, const char* name, const void** dev) {
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess || at.type == hipMemoryTypeUnregistered) {
    (void)hipGetLastError();  // clear the sticky error of the query
    return fail(GCA_ERR_INVALID_ARGUMENT,
                "%s is neither device memory nor pinned (hipHostMalloc) host memory", name);
  }
  if (at.type == hipMemoryTypeHost) {
    if (at.devicePointer == nullptr)
      return fail(GCA_ERR_INVALID_ARGUMENT, "%s: host memory without a device mapping", name);
    const char* base = at.hostPointer ? (const char*)at.hostPointer : (const char*)p;
    *dev = (const char*)at.devicePointer + ((const char*)p - base);
  } else {
    *dev = p;
  }
  return GCA_OK;
}

#define GCA_TRY(expr)                 \
  do {                                \
    gca_status st_ = (expr);          \
    if (st_ != GCA_OK) return st_;    \
  } while (0)

}  // namespace

extern "C" {

int gca_abi_version(void) { return GCA_ABI_VERSION; }

const char* gca_status_string(gca_status status) {
  switch (status) {
    case GCA_OK: return "GCA_OK";
    case GCA_ERR_INVALID_ARGUMENT: return "GCA_ERR_INVALID_ARGUMENT";
    case GCA_ERR_UNSUPPORTED: return "GCA_ERR_UNSUPPORTED";
    case GCA_ERR_WORKSPACE: return "GCA_ERR_WORKSPACE";
    case GCA_ERR_DEVICE: return "GCA_ERR_DEVICE";
    default: return "GCA_UNKNOWN_STATUS";
  }
}

const char* gca_last_error(void) { return g_err; }

gca_status gca_workspace_size(const gca_shape* shape, int op, size_t* bytes) {
  if (bytes == nullptr) return fail(GCA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (op < 0 || op > 2) return fail(GCA_ERR_INVALID_ARGUMENT, "op must be 0, 1 or 2");
  Sizes z;
  GCA_TRY(check_shape(shape, op, &z));
  if (op == kRetrieve)
    *bytes = retrieve_ws(shape, z, plan_scan(shape, z)).total;
  else if (op == kForward)
    *bytes = 0;
  else
    *bytes = backward_ws(shape, z).total;
  g_err[0] = '\0';
  return GCA_OK;
}

static gca_status retrieve_impl(const char* fn, const gca_shape* shape, int noise, uint64_t seed,
                                const void* lq, const void* lk, const int32_t* q_pos,
                                int32_t* idx, float* score, float* w, void* ws, size_t ws_bytes,
                                void* stream, const gca::LaunchForward* fuse = nullptr,
                                int* fused = nullptr) {
  Sizes z;
  GCA_TRY(check_shape(shape, kRetrieve, &z));
  // the bf16 scan prunes on unscaled dot products (ordered like r only for a
  // positive scale); the noisy scan prunes on the perturbed scores themselves
  if (shape->dtype == GCA_BF16 && noise == 0 && !(shape->score_scale > 0.0f))
    return fail(GCA_ERR_UNSUPPORTED, "%s: bf16 retrieval needs score_scale > 0", fn);
  if (z.q_rows == 0) {
    g_err[0] = '\0';
    return GCA_OK;
  }
  GCA_TRY(need(lq, "lq", 16));
  if (shape->n_key > 0) GCA_TRY(need(lk, "lk", 16));
  GCA_TRY(need(q_pos, "q_pos", 4));
  GCA_TRY(need(idx, "idx", 4));
  GCA_TRY(need(score, "score", 4));
  GCA_TRY(need(w, "w", 4));
  const gca::ScanPlan plan = plan_scan(shape, z);
  const RetrieveWs wl = retrieve_ws(shape, z, plan);
  if (wl.total > 0) {
    if (ws == nullptr || ws_bytes < wl.total)
      return fail(GCA_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", fn, wl.total,
                  ws == nullptr ? (size_t)0 : ws_bytes);
    if (!aligned(ws, kAlign)) return fail(GCA_ERR_INVALID_ARGUMENT, "ws is not 256-byte aligned");
  }
  const int64_t nblk = shape->dtype == GCA_BF16
                           ? z.heads * plan.nsplit *
                                 (plan.few ? shape->n_query : (int64_t)plan.n_qtiles)
                           : (z.q_rows + 63) / 64;
  if (nblk > 0x7fffffffLL) return fail(GCA_ERR_UNSUPPORTED, "retrieval grid too large");
  gca::LaunchRetrieve a{};
  a.G = shape->G;
  a.B = shape->B;
  a.H = shape->H;
  a.n_query = shape->n_query;
  a.n_key = shape->n_key;
  a.dl = shape->landmark_dim;
  a.k = shape->top_k;
  a.dtype = shape->dtype;
  a.softmax_one = shape->softmax_one;
  a.score_scale = shape->score_scale;
  a.lq = lq;
  a.lk = lk;
  a.q_pos = q_pos;
  a.idx = idx;
  a.score = score;
  a.w = w;
  a.part = wl.total ? (uint64_t*)((char*)ws + wl.part) : nullptr;
  a.noise = noise;
  a.seed = seed;
  a.stream = (hipStream_t)stream;
  a.fuse = fuse;
  a.fused = fused;
  return device_status(gca::launch_retrieve(plan, a), a.stream, fn);
}

gca_status gca_retrieve(const gca_shape* shape, const void* lq, const void* lk,
                        const int32_t* q_pos, int32_t* idx, float* score, float* w, void* ws,
                        size_t ws_bytes, void* stream) {
  return retrieve_impl("gca_retrieve", shape, 0, 0, lq, lk, q_pos, idx, score, w, ws, ws_bytes,
                       stream);
}

gca_status gca_retrieve_noalloc(const gca_shape* shape, const void* lq, const void* lk,
                                const int32_t* q_pos, int32_t* idx, float* score, float* w,
                                void* stream) {
  Sizes z;
  GCA_TRY(check_shape(shape, kRetrieve, &z));
  const size_t need_bytes = retrieve_ws(shape, z, plan_scan(shape, z)).total;
  if (need_bytes > gca::kScratchBytes)
    return fail(GCA_ERR_UNSUPPORTED,
                "gca_retrieve_noalloc: this shape needs %zu scratch bytes, more than the "
                "library's %zu; call gca_retrieve with a workspace",
                need_bytes, gca::kScratchBytes);
  void* ws = nullptr;
  if (need_bytes > 0) {
    const hipError_t e = gca::scratch_address(&ws);
    if (e != hipSuccess)
      return fail(GCA_ERR_DEVICE, "gca_retrieve_noalloc: scratch address: %s (%s)",
                  hipGetErrorName(e), hipGetErrorString(e));
  }
  return retrieve_impl("gca_retrieve_noalloc", shape, 0, 0, lq, lk, q_pos, idx, score, w, ws,
                       need_bytes > 0 ? gca::kScratchBytes : 0, stream);
}

gca_status gca_retrieve_gumbel(const gca_shape* shape, uint64_t seed, const void* lq,
                               const void* lk, const int32_t* q_pos, int32_t* idx, float* score,
                               float* w, void* ws, size_t ws_bytes, void* stream) {
  return retrieve_impl("gca_retrieve_gumbel", shape, 1, seed, lq, lk, q_pos, idx, score, w, ws,
                       ws_bytes, stream);
}

gca_status gca_gather_kv(const gca_shape* shape, const int32_t* idx, const void* k,
                         const void* v, void* k_packed, void* v_packed, int32_t* idx_packed,
                         void* stream) {
  Sizes z;
  GCA_TRY(check_shape(shape, kForward, &z));
  if (z.slots == 0) {
    g_err[0] = '\0';
    return GCA_OK;
  }
  if (z.slots > 0x7fffffffLL)
    return fail(GCA_ERR_UNSUPPORTED, "G*B*H*n_query*top_k must be below 2^31");
  GCA_TRY(need(idx, "idx", 4));
  GCA_TRY(need(k_packed, "k_packed", 16));
  GCA_TRY(need(v_packed, "v_packed", 16));
  GCA_TRY(need(idx_packed, "idx_packed", 4));
  gca::LaunchGather a{};
  if (shape->n_key > 0) {
    GCA_TRY(need(k, "k", 16));
    GCA_TRY(need(v, "v", 16));
    GCA_TRY(readable_on_device(k, "k", &a.k_src));
    GCA_TRY(readable_on_device(v, "v", &a.v_src));
  }
  a.heads = z.heads;
  a.n_query = shape->n_query;
  a.n_key = shape->n_key;
  a.k = shape->top_k;
  a.tile_bytes = (int64_t)shape->chunk_size * shape->head_dim *
                 (shape->dtype == GCA_BF16 ? 2 : 4);
  a.idx = idx;
  a.k_out = k_packed;
  a.v_out = v_packed;
  a.idx_out = idx_packed;
  a.stream = (hipStream_t)stream;
  return device_status(gca::launch_gather_kv(a), a.stream, "gca_gather_kv");
}

static gca_status check_swa(const gca_swa_shape* s, int64_t* heads) {
  if (s == nullptr) return fail(GCA_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->B < 1 || s->H < 1 || s->T < 0)
    return fail(GCA_ERR_INVALID_ARGUMENT, "B, H must be >= 1 and T >= 0");
  if (s->window < 1) return fail(GCA_ERR_INVALID_ARGUMENT, "window must be >= 1");
  if (s->dtype != GCA_F32 && s->dtype != GCA_BF16)
    return fail(GCA_ERR_INVALID_ARGUMENT, "dtype must be GCA_F32 or GCA_BF16");
  if (!std::isfinite(s->scale)) return fail(GCA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (s->dtype != GCA_BF16 || s->head_dim != 64)
    return fail(GCA_ERR_UNSUPPORTED, "sliding-window attention needs bf16 and head_dim 64");
  if (s->T % 64 != 0) return fail(GCA_ERR_UNSUPPORTED, "T must be a multiple of 64");
  if (s->T >= (int64_t(1) << 30)) return fail(GCA_ERR_UNSUPPORTED, "T must be below 2^30");
  int64_t h, rows;
  if (!mul_ok(s->B, s->H, &h) || !mul_ok(h, s->T, &rows) || rows > (int64_t(1) << 40))
    return fail(GCA_ERR_INVALID_ARGUMENT, "tensor sizes overflow");
  if (rows / 64 > 0x7fffffffLL) return fail(GCA_ERR_UNSUPPORTED, "more than 2^31 - 1 blocks");
  *heads = h;
  return GCA_OK;
}

gca_status gca_swa_workspace_size(const gca_swa_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return fail(GCA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  int64_t heads;
  GCA_TRY(check_swa(shape, &heads));
  *bytes = align_up((size_t)heads * (size_t)shape->T * sizeof(float));
  g_err[0] = '\0';
  return GCA_OK;
}

gca_status gca_swa_forward(const gca_swa_shape* shape, const void* q, const void* k,
                           const void* v, void* o, float* lse, void* stream) {
  int64_t heads;
  GCA_TRY(check_swa(shape, &heads));
  if (shape->scale < 0.0f)  // the row shift is the largest unscaled product, as in gca_forward
    return fail(GCA_ERR_UNSUPPORTED, "gca_swa_forward: needs scale >= 0");
  if (shape->T == 0) {
    g_err[0] = '\0';
    return GCA_OK;
  }
  GCA_TRY(need(q, "q", 16));
  GCA_TRY(need(k, "k", 16));
  GCA_TRY(need(v, "v", 16));
  GCA_TRY(need(o, "o", 16));
  GCA_TRY(opt(lse, "lse", 4));
  gca::LaunchSwa a{};
  a.heads = heads;
  a.n_tok = shape->T;
  // a window past the sequence start is the same as one of T tokens; the
  // kernels' block arithmetic then stays far inside 32-bit range
  a.window = shape->window < shape->T ? shape->window : (int)shape->T;
  a.scale = shape->scale;
  a.q = q;
  a.kk = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.stream = (hipStream_t)stream;
  return device_status(gca::launch_swa_forward(a), a.stream, "gca_swa_forward");
}

gca_status gca_swa_backward(const gca_swa_shape* shape, const void* q, const void* k,
                            const void* v, const void* o, const float* lse, const void* dout,
                            void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                            void* stream) {
  int64_t heads;
  GCA_TRY(check_swa(shape, &heads));
  if (shape->T == 0) {
    g_err[0] = '\0';
    return GCA_OK;
  }
  GCA_TRY(need(q, "q", 16));
  GCA_TRY(need(k, "k", 16));
  GCA_TRY(need(v, "v", 16));
  GCA_TRY(need(o, "o", 16));
  GCA_TRY(need(lse, "lse", 4));
  GCA_TRY(need(dout, "dout", 16));
  GCA_TRY(need(dq, "dq", 16));
  GCA_TRY(need(dk, "dk", 16));
  GCA_TRY(need(dv, "dv", 16));
  const size_t wsz = align_up((size_t)heads * (size_t)shape->T * sizeof(float));
  if (ws == nullptr || ws_bytes < wsz)
    return fail(GCA_ERR_WORKSPACE, "gca_swa_backward needs %zu workspace bytes, got %zu", wsz,
                ws == nullptr ? (size_t)0 : ws_bytes);
  if (!aligned(ws, kAlign)) return fail(GCA_ERR_INVALID_ARGUMENT, "ws is not 256-byte aligned");
  gca::LaunchSwa a{};
  a.heads = heads;
  a.n_tok = shape->T;
  // a window past the sequence start is the same as one of T tokens; the
  // kernels' block arithmetic then stays far inside 32-bit range
  a.window = shape->window < shape->T ? shape->window : (int)shape->T;
  a.scale = shape->scale;
  a.q = q;
  a.kk = k;
  a.v = v;
  a.o = o;
  a.lse = (float*)lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = (float*)ws;
  a.stream = (hipStream_t)stream;
  return device_status(gca::launch_swa_backward(a), a.stream, "gca_swa_backward");
}

// Checks of the forward's arguments and its launch description; *empty: no
// query row (nothing to launch).  idx and w are checked only when check_slots
// is set (the retrieval-plus-forward call writes them itself).
static gca_status forward_args(const char* fn, const gca_shape* shape, const void* q,
                               const void* k, const void* v, const int32_t* idx, const float* w,
                               void* o, float* lse, void* stream, bool check_slots,
                               gca::LaunchForward* a, bool* empty) {
  Sizes z;
  GCA_TRY(check_shape(shape, kForward, &z));
  // the bf16 MFMA kernels (chunk_size 64 or 16, head_dim 64 or 32) shift by the
  // largest unscaled product: a bound on the exponents only for a
  // non-negative scale
  if (shape->dtype == GCA_BF16 && (shape->chunk_size == 64 || shape->chunk_size == 16) &&
      (shape->head_dim == 64 || shape->head_dim == 32) && shape->attn_scale < 0.0f)
    return fail(GCA_ERR_UNSUPPORTED, "%s: bf16 attention on MFMA tiles needs attn_scale >= 0",
                fn);
  *empty = z.q_rows == 0;
  if (*empty) return GCA_OK;
  GCA_TRY(need(q, "q", 16));
  if (shape->n_key > 0) {
    GCA_TRY(need(k, "k", 16));
    GCA_TRY(need(v, "v", 16));
  }
  if (check_slots) {
    GCA_TRY(need(idx, "idx", 4));
    GCA_TRY(need(w, "w", 4));
  }
  GCA_TRY(need(o, "o", 16));
  GCA_TRY(opt(lse, "lse", 4));
  *a = gca::LaunchForward{};
  a->G = shape->G;
  a->B = shape->B;
  a->H = shape->H;
  a->n_query = shape->n_query;
  a->n_key = shape->n_key;
  a->S = shape->chunk_size;
  a->D = shape->head_dim;
  a->k = shape->top_k;
  a->dtype = shape->dtype;
  a->attn_scale = shape->attn_scale;
  a->q = q;
  a->kk = k;
  a->v = v;
  a->idx = idx;
  a->w = w;
  a->o = o;
  a->lse = lse;
  a->stream = (hipStream_t)stream;
  return GCA_OK;
}

gca_status gca_forward(const gca_shape* shape, const void* q, const void* k, const void* v,
                       const int32_t* idx, const float* w, void* o, float* lse, void* stream) {
  gca::LaunchForward a;
  bool empty = false;
  GCA_TRY(forward_args("gca_forward", shape, q, k, v, idx, w, o, lse, stream, true, &a, &empty));
  if (empty) {
    g_err[0] = '\0';
    return GCA_OK;
  }
  return device_status(gca::launch_forward(a), a.stream, "gca_forward");
}

gca_status gca_retrieve_forward(const gca_shape* shape, const void* lq, const void* lk,
                                const int32_t* q_pos, const void* q, const void* k,
                                const void* v, int32_t* idx, float* score, float* w, void* o,
                                float* lse, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "gca_retrieve_forward";
  gca::LaunchForward f;
  bool empty = false;
  GCA_TRY(forward_args(fn, shape, q, k, v, idx, w, o, lse, stream, false, &f, &empty));
  f.idx = idx;
  f.w = w;
  int fused = 0;
  GCA_TRY(retrieve_impl(fn, shape, 0, 0, lq, lk, q_pos, idx, score, w, ws, ws_bytes, stream,
                        &f, &fused));
  if (empty || fused) return GCA_OK;
  return device_status(gca::launch_forward(f), f.stream, fn);
}

static gca_status backward_impl(const char* fn, int accumulate, const gca_shape* shape,
                                const void* q, const void* k, const void* v, const int32_t* idx,
                                const float* w, const float* lse, const void* dout,
                                const void* lq, const void* lk, void* dq, void* dk, void* dv,
                                float* dw, float* dscore, float* dlq, float* dlk, void* ws,
                                size_t ws_bytes, void* stream) {
  Sizes z;
  GCA_TRY(check_shape(shape, kBackward, &z));
  if (z.q_rows == 0 && z.k_rows == 0) {
    g_err[0] = '\0';
    return GCA_OK;
  }
  if (z.q_rows > 0) {
    GCA_TRY(need(q, "q", 16));
    GCA_TRY(need(dout, "dout", 16));
    GCA_TRY(need(idx, "idx", 4));
    GCA_TRY(need(w, "w", 4));
    GCA_TRY(need(lse, "lse", 4));
    GCA_TRY(need(dq, "dq", 16));
    GCA_TRY(need(dw, accumulate ? "dw_acc" : "dw", 4));
    GCA_TRY(need(dscore, accumulate ? "dscore_acc" : "dscore", 4));
  }
  if (z.k_rows > 0) {
    GCA_TRY(need(k, "k", 16));
    GCA_TRY(need(v, "v", 16));
    GCA_TRY(need(dk, accumulate ? "dk_acc" : "dk", 16));
    GCA_TRY(need(dv, accumulate ? "dv_acc" : "dv", 16));
  }
  GCA_TRY(opt(dlq, accumulate ? "dlq_acc" : "dlq", 4));
  GCA_TRY(opt(dlk, accumulate ? "dlk_acc" : "dlk", 4));
  // dlq sums over retrieved chunks' landmarks: with no resident chunk it is 0
  if (dlq != nullptr && z.q_rows > 0 && shape->n_key > 0)
    GCA_TRY(need(lk, "lk (needed for dlq)", 16));
  if (dlk != nullptr && z.k_rows > 0) GCA_TRY(need(lq, "lq (needed for dlk)", 16));
  GCA_TRY(opt(lq, "lq", 16));
  GCA_TRY(opt(lk, "lk", 16));
  const BackwardWs wl = backward_ws(shape, z);
  if (ws == nullptr || ws_bytes < wl.total)
    return fail(GCA_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", fn, wl.total,
                ws == nullptr ? (size_t)0 : ws_bytes);
  if (!aligned(ws, kAlign)) return fail(GCA_ERR_INVALID_ARGUMENT, "ws is not 256-byte aligned");
  gca::LaunchBackward a{};
  a.G = shape->G;
  a.B = shape->B;
  a.H = shape->H;
  a.n_query = shape->n_query;
  a.n_key = shape->n_key;
  a.S = shape->chunk_size;
  a.D = shape->head_dim;
  a.dl = shape->landmark_dim;
  a.k = shape->top_k;
  a.dtype = shape->dtype;
  a.attn_scale = shape->attn_scale;
  a.score_scale = shape->score_scale;
  a.q = q;
  a.kk = k;
  a.v = v;
  a.idx = idx;
  a.w = w;
  a.lse = lse;
  a.dout = dout;
  a.lq = dlk ? lq : nullptr;
  a.lk = (dlq && shape->n_key > 0) ? lk : nullptr;  // no resident chunk: dlq = 0, lk unread
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dw = dw;
  a.dscore = dscore;
  a.dlq = dlq;
  a.dlk = dlk;
  a.accumulate = accumulate;
  a.delta = (float*)((char*)ws + wl.delta);
  a.rev_off = (int32_t*)((char*)ws + wl.rev_off);
  a.rev_ent = (int32_t*)((char*)ws + wl.rev_ent);
  a.ds_layer = (float*)((char*)ws + wl.ds_layer);
  a.stream = (hipStream_t)stream;
  return device_status(gca::launch_backward(a), a.stream, fn);
}

gca_status gca_backward(const gca_shape* shape, const void* q, const void* k, const void* v,
                        const int32_t* idx, const float* w, const float* lse, const void* dout,
                        const void* lq, const void* lk, void* dq, void* dk, void* dv, float* dw,
                        float* dscore, float* dlq, float* dlk, void* ws, size_t ws_bytes,
                        void* stream) {
  return backward_impl("gca_backward", 0, shape, q, k, v, idx, w, lse, dout, lq, lk, dq, dk, dv,
                       dw, dscore, dlq, dlk, ws, ws_bytes, stream);
}

gca_status gca_backward_accumulate(const gca_shape* shape, const void* q, const void* k,
                                   const void* v, const int32_t* idx, const float* w,
                                   const float* lse, const void* dout, const void* lq,
                                   const void* lk, void* dq, float* dk_acc, float* dv_acc,
                                   float* dw_acc, float* dscore_acc, float* dlq_acc,
                                   float* dlk_acc, void* ws, size_t ws_bytes, void* stream) {
  return backward_impl("gca_backward_accumulate", 1, shape, q, k, v, idx, w, lse, dout, lq, lk,
                       dq, dk_acc, dv_acc, dw_acc, dscore_acc, dlq_acc, dlk_acc, ws, ws_bytes,
                       stream);
}

}  // extern "C"

// Microbenchmarks for the measured peaks (gca_peaks.h).
extern "C" {

gca_status gca_peak_read(const void* src, size_t bytes, void* out, void* stream) {
  GCA_TRY(need(src, "src", 16));
  GCA_TRY(need(out, "out", 4));
  if (bytes == 0 || bytes % 16 != 0)
    return fail(GCA_ERR_INVALID_ARGUMENT, "gca_peak_read: bytes must be a positive multiple of 16");
  hipStream_t st = (hipStream_t)stream;
  return device_status(gca::launch_peak_read(src, bytes, out, st), st, "gca_peak_read");
}

gca_status gca_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  GCA_TRY(need(src, "src", 16));
  GCA_TRY(need(dst, "dst", 16));
  if (bytes == 0 || bytes % 16 != 0)
    return fail(GCA_ERR_INVALID_ARGUMENT, "gca_peak_copy: bytes must be a positive multiple of 16");
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes)
    return fail(GCA_ERR_INVALID_ARGUMENT, "gca_peak_copy: src and dst overlap");
  hipStream_t st = (hipStream_t)stream;
  return device_status(gca::launch_peak_copy(src, dst, bytes, st), st, "gca_peak_copy");
}

gca_status gca_peak_gather(const void* src, size_t bytes, void* out, int iters, double* gathered,
                           void* stream) {
  GCA_TRY(need(src, "src", 16));
  GCA_TRY(need(out, "out", 4));
  if (bytes < 16384 || bytes % 16384 != 0)
    return fail(GCA_ERR_INVALID_ARGUMENT,
                "gca_peak_gather: bytes must be a positive multiple of 16384");
  if (iters < 1 || iters > 4096)
    return fail(GCA_ERR_INVALID_ARGUMENT, "gca_peak_gather: iters must be in 1 .. 4096");
  if (gathered) *gathered = 4096.0 * (double)iters * 16384.0;
  hipStream_t st = (hipStream_t)stream;
  return device_status(gca::launch_peak_gather(src, bytes, out, iters, st), st, "gca_peak_gather");
}

gca_status gca_peak_mfma(void* out, int iters, double* flops, void* stream) {
  GCA_TRY(need(out, "out", 4));
  if (iters < 1 || iters > (1 << 20))
    return fail(GCA_ERR_INVALID_ARGUMENT, "gca_peak_mfma: iters must be in 1 .. 2^20");
  if (flops) *flops = 1024.0 * 4.0 * (double)iters * 8.0 * (16.0 * 16.0 * 32.0 * 2.0);
  hipStream_t st = (hipStream_t)stream;
  return device_status(gca::launch_peak_mfma(out, iters, st), st, "gca_peak_mfma");
}

}  // extern "C"
