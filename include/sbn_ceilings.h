/*
 * sbn_ceilings.h - measured ceilings of the GPU the library runs on, for reporting the kernels'
 * rates against what the chip delivers beside its published peaks. Not part of the BitLinear path.
 *
 * The pages measure nothing on this hardware ("From 2:4 to 8:16 sparsity patterns in LLMs for
 * Outliers and Weights with Variance Correction", summary: the 8:16 speedups are projected rather
 * than measured), so every rate this library reports is measured here, against three probes:
 *   - a streaming read of a large buffer (the HBM rate a plain read kernel reaches),
 *   - a loop of dense INT8 MFMA instructions with no memory traffic (the matrix-core rate),
 *   - an empty kernel (the fixed cost of one launch).
 * Conventions as in sbn.h: device pointers, `stream` a hipStream_t passed as void*, validation
 * before any HIP call, negative sbn_status on failure with sbn_last_error() set. Every call only
 * enqueues one kernel.
 */
#ifndef SBN_CEILINGS_H
#define SBN_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#include "sbn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes at `buf` (16-byte aligned, bytes a multiple of 16) once, 16 bytes per lane
 * load, four loads in flight per lane, and XORs them together; a lane whose XOR equals `sentinel`
 * writes it to sink[0] (so the reads cannot be dropped; with a zero-filled buffer and a non-zero
 * sentinel nothing is written). Requires 16 <= bytes <= 2^40.
 */
sbn_status sbn_ceiling_stream_read(const void* buf, size_t bytes, uint32_t sentinel,
                                   uint32_t* sink, void* stream);

/*
 * Runs `iters` rounds of eight independent v_mfma_i32_16x16x64_i8 per wave on `waves` waves
 * (workgroups of four waves), no memory traffic except one guarded store to sink[0]. The work is
 * waves * iters * 8 * 32768 integer operations (2 * 16 * 16 * 64 per instruction); *ops (host)
 * receives that count. Requires 1 <= iters <= 2^24, 4 <= waves <= 2^20, waves % 4 == 0.
 */
sbn_status sbn_ceiling_mfma_i8(int64_t iters, int64_t waves, uint32_t* sink, double* ops /* host */,
                               void* stream);

/*
 * The same loop on the structured-sparse v_smfmac_i32_16x16x128_i8 (the instruction of the 2:4
 * GEMM): eight independent chains per wave, each instruction counted as its dense-equivalent
 * 2 * 16 * 16 * 128 = 65536 integer operations (it multiplies the 64 kept weights of each 128-K
 * row slice); *ops (host) receives waves * iters * 8 * 65536. Same argument limits.
 */
sbn_status sbn_ceiling_smfmac_i8(int64_t iters, int64_t waves, uint32_t* sink,
                                 double* ops /* host */, void* stream);

/* Enqueues one launch of an empty kernel (one workgroup of one wave). */
sbn_status sbn_ceiling_empty(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SBN_CEILINGS_H */
