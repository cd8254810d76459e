/*
 * lcsi_ceiling.h -- measurement helpers of the benchmark, in their own
 * library (libceiling.so), not steps of the method: the practical
 * matrix-core ceiling of the indexer score kernel on this GPU, the
 * practical rate of a plain streaming read from HBM, and that of a gather
 * of whole rows into LDS (the sparse attention's memory pattern).
 *
 * lcsi_ceiling_mfma launches n_wg workgroups of 8 waves (two per SIMD, as
 * the score kernel) that each issue `blocks` times the score kernel's block
 * of 16 v_mfma_f32_32x32x16_bf16 (two 32-row tiles x 8 k-steps of 16 dims,
 * two accumulator chains) and nothing else: no epilogue, no stores but one
 * float per wave, no key traffic from memory.
 *   data   device bf16, lcsi_ceiling_data_elems() values (the query rows, then
 *          256 key rows of 128 dims); the caller fills it with the value
 *          distribution under test (the benchmark: N(0,1)/8, the indexer's).
 *   out    device fp32, n_wg * 8 values (one per wave), written.
 *   mode   0: B operands in registers, changing block by block (4 sets);
 *          1: B operands read from two key tiles staged once in LDS, with
 *          the score kernel's LDS reads.
 *   blocks a multiple of 4, at least 4.
 * Work per launch: n_wg * 8 * blocks * 16 * 32768 flop.  Asynchronous on
 * `stream` (a hipStream_t as void*).  Returns 0, -1 for a bad argument, -5
 * for a misaligned pointer (data 16 bytes, out 4), -6 if the launch failed.
 */
#ifndef LCSI_CEILING_H
#define LCSI_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

size_t lcsi_ceiling_data_elems(void);
int lcsi_ceiling_mfma(const uint16_t *data, float *out, int n_wg, int blocks, int mode, void *stream);

/* lcsi_ceiling_read reads every 16-byte unit of `data` (device, `bytes` a
 * multiple of 16, 16-byte aligned) once: n_wg workgroups of 256 threads
 * stride over it with eight non-temporal 16-byte loads in flight per thread
 * and XOR each thread's words into out[thread] (device uint32, n_wg * 256
 * values, written).  Asynchronous on `stream`.  Returns 0, -1 for a bad
 * argument, -5 for a misaligned pointer, -6 if the launch failed. */
int lcsi_ceiling_read(const void *data, size_t bytes, uint32_t *out, int n_wg, void *stream);

/* lcsi_ceiling_gather copies whole rows into LDS the way the sparse
 * attention kernel gathers its KV rows, without the attention's arithmetic:
 * n_wg workgroups of 256 threads; workgroup w takes `tiles` (1..64) lists of
 * 32 row numbers, idx[(w * tiles + t) * 32 + r] (device int32, clamped to
 * [0, n_rows)), and copies each list's 32 rows of `row_bytes` bytes (16..1152,
 * a multiple of 16) from rows + number * row_bytes (device, 16-byte aligned)
 * into LDS with direct 16-byte loads, one list in flight while the previous
 * one is read back.  Thread i of workgroup w XORs the four words of LDS
 * 16-byte unit i of every list (chunk i % (row_bytes/16) of row
 * i / (row_bytes/16)) into out[w * 256 + i] (device uint32, written).
 * Asynchronous on `stream`.  Returns 0, -1 for a bad argument, -5 for a
 * misaligned pointer, -6 if the launch failed. */
int lcsi_ceiling_gather(const void *rows, int64_t n_rows, uint32_t row_bytes, const int32_t *idx, int n_wg,
                        int tiles, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LCSI_CEILING_H */
