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

// v_mfma_f32_16x16x32_bf16 (wave64):
//   A (16 x 32): lane l supplies row (l % 16), 8 K-values
//   B (32 x 16): lane l supplies column (l % 16), 8 K-values
//   C/D (16 x 16): lane l, register r holds C[4*(l/16) + r][l % 16]
// The four 16-lane groups supply the four 8-wide quarters of the contraction.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = 0.0f;
  return z;
}

// Larger of two values (the library is built without NaN semantics, so this is
// a plain v_max_f32 / v_max3_f32).
__device__ __forceinline__ float max_nc(float a, float b) { return fmaxf(a, b); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
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

// Order in which key chunks go out.  Each XCD works through one contiguous
// range of tiles (xcd_tile), head after head, so that the Q/dO tiles in use
// are those of about one head, which its L2 can nearly hold.  A chunk's work
// grows with its reverse list, and in causal training the early chunks
// collect the longest lists (about k ln(n/c) entries for chunk c): in plain
// head order the range's last heads would start theirs near the end of the
// grid and run alone.  So the first 32 chunks of the range's last head and
// the first 8 of the head before it go out first; the rest keep head order.
__device__ __forceinline__ int64_t kv_tile_order(int64_t i, int64_t n_key, int64_t nblk) {
  if (nblk % 8 != 0) return i;  // xcd_tile is the identity then
  const int64_t R = nblk / 8;
  const int64_t s0 = (i / R) * R, li = i - s0;  // this XCD's range [s0, s0 + R)
  const int64_t hl = (s0 + R - 1) / n_key;      // its last head
  const int64_t b1 = hl * n_key, b2 = (hl - 1) * n_key;
  int64_t f1 = n_key < 32 ? n_key : 32, f2 = n_key < 8 ? n_key : 8;
  if (b1 < s0 || b1 + f1 > s0 + R) f1 = 0;  // hoisted blocks lie inside the range
  if (hl < 1 || b2 < s0) f2 = 0;
  if (li < f1) return b1 + li;
  if (li < f1 + f2) return b2 + (li - f1);
  int64_t t = s0 + (li - f1 - f2);  // the rest in order, skipping both blocks
  if (f2 && t >= b2) t += f2;
  if (f1 && t >= b1) t += f1;
  return t;
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

// Cross-lane all-reduce steps on VALU lane swaps (gfx950), no LDS round trip.
// permlane16_swap(x, x) returns, for every 16-lane row pair (0,1) and (2,3),
// the first row's and the second row's values; permlane32_swap(x, x) returns
// the two 32-lane halves.  op(r[0], r[1]) is therefore op(x[l], x[l ^ 16]) (or
// l ^ 32), identical on both partners, for any commutative op.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over each 16-lane row, left in every lane of the row (DPP row rotates).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0x128>(v);  // row_ror:8
  v += dpp_f<0x124>(v);  // row_ror:4
  v += dpp_f<0x122>(v);  // row_ror:2
  v += dpp_f<0x121>(v);  // row_ror:1
  return v;
}

// Deterministic butterfly sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// LDS tiles: 64 rows x D bf16 (D = 64: 128-byte rows; D = 32: 64-byte rows),
// XOR-swizzled at 16-byte granularity: chunk c (columns 8c .. 8c+7) of row r
// sits at chunk position c ^ (r mod D/8).  Consecutive rows reading the same
// logical chunk, and the 4-row x 16-column blocks of the transpose read, then
// hit distinct banks.
constexpr int kTileElems = 64 * 64;

template <int D = 64>
__device__ __forceinline__ int swz(int row, int col) {
  static_assert(D == 32 || D == 64, "tile rows of 32 or 64 elements");
  return row * D + ((((col >> 3) ^ (row & (D / 8 - 1)))) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous copy of one 64 x 64 bf16 tile (row-major, 128 B rows) from
// global memory straight into a swizzled LDS tile with gfx950's 16-byte
// global_load_lds: NW waves each move 8/NW pieces of 1 KB (8 rows).  The data
// is in LDS once the issuing wave's vector-memory counter drains
// (wait_vmem()) and a barrier has passed.
template <int NW>
__device__ __forceinline__ void tile_dma(bf16* lds_tile, const bf16* __restrict__ src, int wave,
                                         int lane) {
#pragma unroll
  for (int r = 0; r < 8 / NW; ++r) {
    const int piece = wave * (8 / NW) + r;
    const int row = piece * 8 + (lane >> 3), pc = lane & 7;
    __builtin_amdgcn_global_load_lds((const void*)(src + row * 64 + ((pc ^ (row & 7)) << 3)),
                                     (lds_void*)(lds_tile + piece * 512), 16, 0, 0);
  }
}

// The same copy with the per-lane part of the addresses computed once: `off`
// holds, for each of the wave's pieces (1 KB each: ROWS x D tiles have
// ROWS * D / 512 of them, shared by NW waves), this lane's byte offset inside
// the source tile, so
// a copy costs no vector arithmetic when the tile base is wave-uniform (it is
// then used as the scalar base of global_load_lds).
template <int NW, int D = 64, int ROWS = 64>
struct TileDma {
  static constexpr int kPieces = ROWS * D / 512 / NW;  // per wave
  static constexpr int kRows = 512 / D;       // tile rows per piece
  static constexpr int kChunks = D / 8;       // 16-byte chunks per row
  uint32_t off[kPieces];
  int first_piece;
  __device__ __forceinline__ TileDma(int wave, int lane) : first_piece(wave * kPieces) {
#pragma unroll
    for (int r = 0; r < kPieces; ++r) {
      const int row = (first_piece + r) * kRows + lane / kChunks, pc = lane % kChunks;
      off[r] = (uint32_t)(row * D + ((pc ^ (row & (kChunks - 1))) << 3)) * 2u;
    }
  }
  __device__ __forceinline__ void copy(bf16* lds_tile, const bf16* src) const {
    const char* base = (const char*)src;
#pragma unroll
    for (int r = 0; r < kPieces; ++r)
      __builtin_amdgcn_global_load_lds((const void*)(base + off[r]),
                                       (lds_void*)(lds_tile + (first_piece + r) * 512), 16, 0, 0);
  }
  // Same copy issued as plain instructions the compiler does not interpret:
  // it then never waits for the copy before unrelated LDS reads (it cannot
  // tell the destination apart from the tile being read and would otherwise
  // drain the copy right away).  The caller owns the wait: wait_vmem() and a
  // barrier before the tile is read.  `src` must be wave-uniform; M0 is
  // restored afterwards.
  __device__ __forceinline__ void copy_async(bf16* lds_tile, const bf16* src) const {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)lds_tile;
#pragma unroll
    for (int r = 0; r < kPieces; ++r) {
      const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(lds0 + (uint32_t)(first_piece + r) * 1024u));
      uint32_t saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %2, %3\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(dst), "v"(off[r]), "s"(src)
          : "memory");
    }
  }
};

// Asynchronous copy of 16 bytes per lane from a per-lane global address `src`
// to LDS at lds_block + 16 * lane (the wave's 1 KB block; lds_block must be
// wave-uniform), issued like TileDma::copy_async: the compiler does not track
// it and the caller owns the wait (wait_vmem() and a barrier) before reading.
__device__ __forceinline__ void copy16_async(void* lds_block, const void* src) {
  const uint32_t dst =
      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void*)lds_block);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(dst), "v"(src)
      : "memory");
}

// Valid-slot iteration over a wave's ballot of valid slots (bit i: slot i):
// the lowest set bit above bit i, or -1.
__device__ __forceinline__ int next_slot(uint32_t m, int i) {
  const uint32_t rest = i >= 31 ? 0u : (m & ~((2u << i) - 1u));
  return rest ? (int)__builtin_ctz(rest) : -1;
}

// Wave-uniform copy of an int read from LDS (lets the compiler keep it scalar).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Approximate reciprocal (v_rcp_f32, about 1 ulp) and natural log through the
// hardware log2 (v_log_f32, about 1 ulp); both are far inside the bf16
// accuracy of the attention path.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_ln(float x) {
  return __builtin_amdgcn_logf(x) * 0.69314718055994531f;
}

// s_waitcnt vmcnt(0): every vector memory access of this wave has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt lgkmcnt(0): every LDS (and scalar memory) access of this wave has
// completed.  Placed after a divergent LDS atomic, it settles the returned
// value on every path, so later uses need no waits of their own.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// 16-byte read of row `row`, logical chunk `chunk` of a swizzled tile.
template <int D = 64>
__device__ __forceinline__ bf16x8 lds_row8(const bf16* tile, int row, int chunk) {
  return *(const bf16x8*)(tile + swz<D>(row, 8 * chunk));
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, if lane s points at row r0 + s/4, columns c0 + 4*(s%4) .. +3 of a
// 16-bit tile, lane i receives column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// MFMA operand whose lane owns column (c_base + lane % 32) of a swizzled LDS
// tile and whose 8 contraction values are the tile rows r_a .. r_a+3 and
// r_b .. r_b+3 (the caller picks r_a, r_b per lane half).  Two transpose
// reads replace eight 2-byte reads.
__device__ __forceinline__ bf16x8 lds_tr_operand(const bf16* tile, int c_base, int r_a, int r_b,
                                                 int lane) {
  const int s = lane & 15;
  const int col = c_base + 16 * ((lane >> 4) & 1) + 4 * (s & 3);
  const bf16x4 a = lds_read_tr(tile + swz(r_a + (s >> 2), col));
  const bf16x4 b = lds_read_tr(tile + swz(r_b + (s >> 2), col));
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Operand for a 16x16x32 MFMA whose lane owns column (c_base + lane % 16) of a
// swizzled LDS tile and whose 8 contraction values are the tile rows
// r_a .. r_a+3 and r_b .. r_b+3 (picked per 16-lane group by the caller).
template <int D = 64>
__device__ __forceinline__ bf16x8 lds_tr_operand16(const bf16* tile, int c_base, int r_a, int r_b,
                                                   int lane) {
  const int s = lane & 15;
  const int col = c_base + 4 * (s & 3);
  const bf16x4 a = lds_read_tr(tile + swz<D>(r_a + (s >> 2), col));
  const bf16x4 b = lds_read_tr(tile + swz<D>(r_b + (s >> 2), col));
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}


// Output write: stored, or (ACC) added to a float32 accumulator.
template <bool ACC>
__device__ __forceinline__ void put(float* p, float v) {
  if (ACC)
    *p += v;
  else
    *p = v;
}

// Fusion-weight softmax backward for one query chunk, run by one whole wave
// with lane i holding slot i (lanes >= topk pass ok = false): dscore_i =
// w_i (dw_i - sum_l w_l dw_l) over the valid slots, 0 on empty ones.  Lanes
// < topk write dw_i and dscore_i (ACC: add them) and, in ACC mode, this
// layer's dscore_i to ds_layer for the key side.  Returns dscore_i.
template <bool ACC>
__device__ __forceinline__ float slot_dscore(int lane, int topk, bool ok, float w_lane,
                                             float dw_lane, float* __restrict__ dw_out,
                                             float* __restrict__ dscore_out,
                                             float* __restrict__ ds_layer) {
  const float dwv = ok ? dw_lane : 0.0f;
  const float sw = wave_sum(ok ? w_lane * dwv : 0.0f);
  const float ds = ok ? w_lane * (dwv - sw) : 0.0f;
  if (lane < topk) {
    put<ACC>(dw_out + lane, dwv);
    put<ACC>(dscore_out + lane, ds);
    if (ACC) ds_layer[lane] = ds;
  }
  return ds;
}

__device__ __forceinline__ float load_f(const float* p) { return *p; }
__device__ __forceinline__ float load_f(const bf16* p) { return (float)(*p); }
// One rounding of a float32 result to the element type (round to nearest even).
__device__ __forceinline__ void store_f(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_f(bf16* p, float v) { *p = (bf16)v; }

}  // namespace gca
