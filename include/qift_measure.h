/*
 * qift_measure.h -- measurement calls of libqift.so. They are no step of the
 * rotated W2A4/KV4 method: they measure, on the GPU the library runs on, the
 * streaming HBM rate and the int8 matrix-core rate against which the
 * method's kernels are reported, and the shader clock under matrix-core load.
 *
 * Conventions are those of qift.h: device pointers owned by the caller,
 * asynchronous on `stream`, arguments validated before anything is launched,
 * a non-zero qift_status (and qift_last_error()) on a rejected call.
 */
#ifndef QIFT_MEASURE_H
#define QIFT_MEASURE_H

#include "qift.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Entries of `sink`, a device buffer both calls take: it is written only if a
 * folded value equals a pattern that does not occur, which keeps the loads
 * and the matrix-core results live. */
#define QIFT_MEASURE_SINK_WORDS 8192

/* Streams `bytes` bytes (a positive multiple of 16, at most 2^40) of src
 * through the vector memory path: workgroup b of 256 threads owns the 64 KB
 * at b * 65536, four non-temporal 16-byte loads in flight per thread.
 * mode 0: read only (the HBM read rate: bytes / duration); mode 1: copy to
 * dst with non-temporal stores (2 * bytes / duration; dst must not overlap
 * src). src and dst 16-byte aligned; dst may be NULL in mode 0. sink:
 * QIFT_MEASURE_SINK_WORDS uint32. */
qift_status qift_measure_stream(const void* src, void* dst, int64_t bytes, int32_t mode,
                                uint32_t* sink, qift_stream stream);

/* `workgroups` workgroups of four waves each run `iters` rounds of eight
 * independent v_mfma_i32_16x16x64_i8 on register operands: 2 * 16*16*64 int8
 * operations per instruction, so 32 * 32768 * iters * workgroups operations
 * in all. clk (4 uint64, 16-byte aligned): the shader clock counter and the
 * constant 100 MHz counter read by the first wave of workgroup 0 at its start
 * (clk[0], clk[1]) and end (clk[2], clk[3]); the shader clock under this load
 * is 100 MHz * (clk[2] - clk[0]) / (clk[3] - clk[1]). 1 <= workgroups <= 2^20,
 * 1 <= iters <= 2^24. sink: QIFT_MEASURE_SINK_WORDS uint32. */
qift_status qift_measure_mfma_i8(int64_t iters, int64_t workgroups, uint32_t* sink,
                                 uint64_t* clk, qift_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* QIFT_MEASURE_H */
