/*
 * gca_peaks.h: microbenchmarks for measuring, on the GPU at hand, the peaks
 * that the GCA kernels' roofline fractions are also quoted against, beside
 * the published MI355X figures (8 TB/s HBM, 2.5 PFLOP/s dense bf16 MFMA):
 *   - a streaming read of device memory (the landmark scan's access kind);
 *   - a streaming device-to-device copy (read + write);
 *   - a gather of randomly chosen 16 KB tiles into LDS (the attention kernels'
 *     K/V and Q/dO tile copies), whose rate depends on the cache level that
 *     holds the buffer: a buffer of a few MB stays in every XCD's L2;
 *   - a loop of independent 16x16x32 bf16 MFMAs (the attention kernels' tile
 *     instruction), eight accumulators per wave, four waves per SIMD.
 * They compute nothing the GCA path uses.  Same status codes, error string and
 * stream conventions as gca.h (gca_last_error() holds the detail of a failure).
 */
#ifndef GCA_PEAKS_H
#define GCA_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#include "gca.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the per-thread result buffer that gca_peak_read writes (one
 * 32-bit value per thread of its fixed grid), so that no load is dropped. */
#define GCA_PEAK_OUT_BYTES ((size_t)(2048 * 256 * 4))

/* Reads `bytes` of device memory at `src` once, with 16-byte loads spread over a
 * fixed grid of 2048 workgroups.  src: device pointer, 16-byte aligned; bytes:
 * a positive multiple of 16.  out: device buffer of GCA_PEAK_OUT_BYTES, 4-byte
 * aligned, overwritten with per-thread XOR folds of the data read.
 * GCA_ERR_INVALID_ARGUMENT for NULL, misaligned or badly sized arguments. */
gca_status gca_peak_read(const void* src, size_t bytes, void* out, void* stream);

/* Copies `bytes` from src to dst (device pointers, 16-byte aligned, not
 * overlapping; bytes a positive multiple of 16) with 16-byte loads and stores
 * over a fixed grid of 2048 workgroups. */
gca_status gca_peak_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Bytes of the per-workgroup result buffer that gca_peak_gather writes. */
#define GCA_PEAK_GATHER_OUT_BYTES ((size_t)(4096 * 4))

/* Copies `iters` tiles of 16 KB, each chosen pseudo-randomly among the bytes /
 * 16384 tiles at `src`, into LDS in every one of 4096 workgroups of 256 threads
 * (16-byte global_load_lds; one tile in flight per workgroup, four workgroups
 * resident per CU).  src: device pointer, 16-byte aligned; bytes: a positive
 * multiple of 16384.  out: device buffer of GCA_PEAK_GATHER_OUT_BYTES, 4-byte
 * aligned (one word of each workgroup's last tile).  *gathered (host pointer,
 * may be NULL) receives the bytes moved: 4096 * iters * 16384.  iters: 1 .. 4096.
 * GCA_ERR_INVALID_ARGUMENT for NULL, misaligned or badly sized arguments. */
gca_status gca_peak_gather(const void* src, size_t bytes, void* out, int iters, double* gathered,
                           void* stream);

/* Runs `iters` rounds of eight independent 16x16x32 bf16 MFMAs in every wave
 * of 1024 workgroups of four waves (4 waves per SIMD on 256 CUs) and writes one
 * float per thread to out (device buffer of 1024 * 256 floats, 4-byte aligned).
 * *flops (host pointer, may be NULL) receives the dense flop count the launch
 * performs: 1024 * 4 * iters * 8 * 16 * 16 * 32 * 2.  iters: 1 .. 1 << 20. */
gca_status gca_peak_mfma(void* out, int iters, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GCA_PEAKS_H */
