/*
 * fp8probe.h -- measurement kernels of libfp8probe.so (MI355X, gfx950).
 *
 * Not part of the FP8 linear path: two microkernels that measure the
 * ceilings the path's kernels are judged against on the machine at hand.
 * The published peaks (dense FP8 MFMA 5.0 PFLOP/s, HBM3E 8 TB/s) assume a
 * clock and a memory system the chip does not hold under every load:
 *
 *   fp8probe_mfma    the rate of the FP8 matrix cores with nothing else in
 *                    the way: each of 8 waves per block (two per SIMD, as
 *                    the GEMM kernels run) issues `iters` rounds of four
 *                    independent v_mfma_f32_32x32x64_f8f6f4 accumulations
 *                    on register operands, one block per CU.  The operand
 *                    values matter: the chip lowers its clock under the
 *                    switching of random data.
 *   fp8probe_stream  the rate of a plain HBM stream: 16-byte lanes,
 *                    grid-stride, copy, read-only or write-only.
 *
 * All pointers are device pointers; work is enqueued on `stream` and timed
 * by the caller (events).  Status: 0 = ok, 2 = invalid size or mode,
 * 1 = a required pointer is NULL, 5 = launch failure.
 */
#ifndef FP8PROBE_H
#define FP8PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * MFMA-only kernel on `blocks` CUs (1..65535; one 512-thread block per CU
 * while blocks <= the CU count).  codes: device, 512 * 64 uint32 words of
 * e4m3 codes (lane t of a block takes words 64 t .. 64 t + 63 as its A and
 * B operands, the same in every block).  out: device float[blocks * 8], one
 * sum of accumulators per wave (keeps every MFMA live).  FLOPs performed:
 * blocks * 8 * iters * 4 * 2 * 32 * 32 * 64.
 */
int fp8probe_mfma(int32_t blocks, int32_t iters, const uint32_t* codes, float* out,
                  hipStream_t stream);

/*
 * Streaming kernel over `bytes` (a multiple of 16): mode 0 copies src to
 * dst, mode 1 reads src (XOR-folded into sink[0..3] only under a condition
 * that keeps the loads live), mode 2 writes dst.  blocks_per_cu: 256-thread
 * blocks launched per CU (1..32).
 */
int fp8probe_stream(const void* src, void* dst, int64_t bytes, int32_t mode, int32_t blocks_per_cu,
                    uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8PROBE_H */
