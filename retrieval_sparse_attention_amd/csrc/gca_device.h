// Device-side helpers shared by the GCA kernels (gfx950 / CDNA4).
//
// MFMA conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand (32 x 16, M x K): lane l supplies row (l % 32), 8 K-values
//   B operand (16 x 32, K x N): lane l supplies column (l % 32), 8 K-values
//   C/D (32 x 32):              lane l, register r holds
//                               C[8*(r/4) + 4*(l/32) + (r%4)][l % 32]
// Lanes l and l+32 supply the two 8-wide halves of the 16-long contraction.  The
// assignment of contraction indices to (half, element) is the same for A and B,
// so any relabelling of the contraction index that both operands share leaves
// the product unchanged; the kernels use that freedom to read memory in
// contiguous 16-byte pieces.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gca {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kIdxNone = 0x7fffffff;  // sorts after every real chunk index

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row of C held by register r of a lane in half h (see the table above).
__device__ __forceinline__ int c_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Workgroups are handed to the 8 XCDs round-robin (block b -> XCD b % 8).  This
// returns the logical tile of block `bid` so that each XCD works through one
// contiguous range of tiles: neighbouring tiles (same head) then share that
// XCD's L2.  Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t nblk) {
  if (nblk % 8 != 0) return bid;
  return (bid % 8) * (nblk / 8) + bid / 8;
}

// Candidate order used by the top-k: higher score first, then lower chunk index.
__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// Sorted (by `better`) fixed-size list insertion with compile-time size: every
// position is updated with selects only, so the list stays in registers.
template <int KMAX>
__device__ __forceinline__ void list_insert(float (&s)[KMAX], int (&id)[KMAX], float x, int j) {
#pragma unroll
  for (int p = KMAX - 1; p >= 0; --p) {
    const float sp = s[p];
    const int ip = id[p];
    const bool place = better(x, j, sp, ip);
    if (p > 0) {
      const float sq = s[p - 1];
      const int iq = id[p - 1];
      const bool shift = better(x, j, sq, iq);
      s[p] = shift ? sq : (place ? x : sp);
      id[p] = shift ? iq : (place ? j : ip);
    } else {
      s[0] = place ? x : sp;
      id[0] = place ? j : ip;
    }
  }
}

template <int KMAX>
__device__ __forceinline__ void list_clear(float (&s)[KMAX], int (&id)[KMAX]) {
#pragma unroll
  for (int p = 0; p < KMAX; ++p) {
    s[p] = -__builtin_huge_valf();
    id[p] = kIdxNone;
  }
}

// Deterministic butterfly sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ float load_f(const float* p) { return *p; }
__device__ __forceinline__ float load_f(const bf16* p) { return (float)(*p); }

}  // namespace gca
