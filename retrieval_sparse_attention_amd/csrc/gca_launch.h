// Internal launch interface between the C ABI (gca_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gca {

// How the retrieval scan is cut into workgroups (chosen on the host, shared by
// gca_workspace_size and gca_retrieve so both agree).
struct ScanPlan {
  int kmax;          // register list length: 4, 8 or 16 (>= k)
  int n_qtiles;      // ceil(n_query / 32)
  int nsplit;        // candidate slices per (head, query tile)
  int64_t split_len; // candidates per slice (multiple of 128)
  int few;           // 1: one workgroup per (head, query, 256-candidate slice) in the
                     // plain bf16 scan (k_scan_few_bf16); split_len is then 256
};

struct LaunchForward {
  int64_t G, B, H, n_query, n_key;
  int S, D, k, dtype;
  float attn_scale;
  const void* q;
  const void* kk;
  const void* v;
  const int32_t* idx;
  const float* w;
  void* o;
  float* lse;
  hipStream_t stream;
};

struct LaunchRetrieve {
  int64_t G, B, H, n_query, n_key;
  int dl, k, dtype, softmax_one;
  float score_scale;
  const void* lq;
  const void* lk;
  const int32_t* q_pos;
  int32_t* idx;
  float* score;
  float* w;
  uint64_t* part;   // [heads * n_query * nsplit * kmax] candidate keys when nsplit > 1
  int noise;        // 1: Gumbel top-k (selection on r + G), 0: plain top-k
  uint64_t seed;    // Philox key of the Gumbel noise
  hipStream_t stream;
  // Retrieval followed by the forward in one call: when set, a sliced plain
  // retrieval at the 64-token tile sizes merges its slice lists inside the
  // forward's kernel and sets *fused to 1; otherwise *fused stays 0 and the
  // caller launches the forward.
  const LaunchForward* fuse = nullptr;
  int* fused = nullptr;
};


struct LaunchBackward {
  int64_t G, B, H, n_query, n_key;
  int S, D, dl, k, dtype;
  float attn_scale, score_scale;
  const void* q;
  const void* kk;
  const void* v;
  const int32_t* idx;
  const float* w;
  const float* lse;
  const void* dout;
  const void* lq;
  const void* lk;
  void* dq;
  void* dk;
  void* dv;
  float* dw;
  float* dscore;
  float* dlq;
  float* dlk;
  int accumulate;    // 1: dk, dv (float32), dw, dscore, dlq, dlk are accumulators added to
  float* delta;      // workspace [heads * n_query * k * S]: rowsum(P * dP) per pair
  float* ds_layer;   // workspace [heads * n_query * k]: this call's dscore (accumulate mode)
  int32_t* rev_off;  // workspace [heads * (n_key + 1)]
  int32_t* rev_ent;  // workspace [heads * n_query * k]: q * k + slot, grouped by chunk
  hipStream_t stream;
};

struct LaunchGather {
  int64_t heads, n_query, n_key;
  int k;
  int64_t tile_bytes;    // S * D * element size
  const void* k_src;     // device address of k (device memory or mapped host memory)
  const void* v_src;
  const int32_t* idx;
  void* k_out;           // [heads, n_query * k, S, D]
  void* v_out;
  int32_t* idx_out;      // [heads, n_query, k]
  hipStream_t stream;
};

struct LaunchSwa {
  int64_t heads, n_tok;  // B * H, T (a multiple of 64)
  int window;
  float scale;
  const void* q;
  const void* kk;
  const void* v;
  const void* o;         // backward: the forward's output
  float* lse;            // [heads, T]; written by the forward (may be NULL), read by the backward
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;          // workspace [heads, T]: <dO[x], O[x]>
  hipStream_t stream;
};

// Kernels the library launches, for the event timing facility.
enum KernelId {
  kKernScan = 0,
  kKernMerge = 1,
  kKernForward = 2,
  kKernReverseIndex = 3,
  kKernBackwardQ = 4,
  kKernBackwardKV = 5,
  kKernGather = 6,
  kKernSwaForward = 7,
  kKernSwaBackwardQ = 8,
  kKernSwaBackwardKV = 9,
  kKernMergeForward = 10,
  kNumKernels = 11
};

// Records a HIP event pair around one kernel launch on `stream` when timing is
// enabled (gca_timing_enable); otherwise does nothing.
class KernelTimer {
 public:
  KernelTimer(int kernel_id, hipStream_t stream);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  int kid_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

// Size of the library-owned scratch array gca_retrieve_noalloc uses in place
// of a workspace (one per device), and its device address on the current
// device (looked up once per device and kept).
constexpr size_t kScratchBytes = size_t(4) << 20;
hipError_t scratch_address(void** ptr);

hipError_t launch_retrieve(const ScanPlan& plan, const LaunchRetrieve& a);
hipError_t launch_forward(const LaunchForward& a);
hipError_t launch_backward(const LaunchBackward& a);
// bf16 attention with 16-token chunks (gca_attn16.hip): one wave per chunk
hipError_t launch_forward_s16(const LaunchForward& a, int64_t tiles);
hipError_t launch_peak_read(const void* src, size_t bytes, void* out, hipStream_t stream);
hipError_t launch_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_peak_gather(const void* src, size_t bytes, void* out, int iters,
                              hipStream_t stream);
hipError_t launch_peak_mfma(void* out, int iters, hipStream_t stream);
hipError_t launch_backward_s16(const LaunchBackward& a, int64_t qtiles, int64_t ktiles);
hipError_t launch_gather_kv(const LaunchGather& a);
hipError_t launch_swa_forward(const LaunchSwa& a);
hipError_t launch_swa_backward(const LaunchSwa& a);

}  // namespace gca
