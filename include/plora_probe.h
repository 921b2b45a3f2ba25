/*
 * plora_probe.h -- micro-benchmarks of the ceilings the packed multi-LoRA
 * operator's kernels are measured against on MI355X (gfx950).
 *
 * The pages report only how far a single-adapter job stays below the GPU's
 * capacity (its SM occupancy and memory utilisation) and the speed-up of the
 * packed operators [PLoRA technical summary (gist.science, arXiv
 * 2508.02932), 问题陈述 and 结果]; they give no absolute throughput.  The
 * operator's roofline fractions are therefore stated against the vendor
 * peaks (bf16 dense matrix cores 2.5 PFLOP/s, HBM 8 TB/s) and against what
 * these probes reach on the same GPU:
 *
 *   plora_probe_mfma   sustained bf16 matrix-core throughput: every wave
 *                      issues matrix-core instructions back to back on random
 *                      operands held in registers (operands changing every
 *                      instruction, no memory traffic in the loop)
 *                      (shape 2: the operands read from LDS at every step,
 *                      as the GEMM's inner loop reads them)
 *   plora_probe_copy   HBM bandwidth of a plain device copy (16-byte accesses)
 *   plora_probe_read   HBM bandwidth of a plain read
 *   plora_probe_lds_dma  rate of the L2 -> LDS path the pipelined kernels
 *                      stage their tiles through (16-byte buffer loads that
 *                      write LDS directly)
 *
 * Each call enqueues one kernel on `stream` and returns; the caller times it
 * (HIP events on the same stream).  Return values and errors as in plora.h
 * (PLORA_OK or a negative plora_status; plora_last_error() for the message).
 * All device pointers 16-byte aligned.  Nothing is allocated.
 */
#ifndef PLORA_PROBE_H
#define PLORA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the operand buffer plora_probe_mfma reads: 1024 wave slices of
 * 16 fragments x 64 lanes x 16 bytes (bf16 values; fill it with random
 * values for a figure under load). */
size_t plora_probe_mfma_operand_bytes(void);

/* One launch of `workgroups` workgroups of 4 waves; each wave loads its 16
 * fragments from `operands` (slice (4 * workgroup + wave) mod 1024) and runs
 * `iters` iterations of 128 x 128 x 32 multiply-adds on a 128 x 128 block of
 * fp32 accumulators held in registers:
 *   shape 0  32 v_mfma_f32_32x32x16_bf16 per iteration (4 x 4 accumulators, in
 *            serpentine order: consecutive instructions share one operand),
 *   shape 1  64 v_mfma_f32_16x16x32_bf16 per iteration (8 x 8, row by row),
 *   shape 2  as shape 0, each wave first copying its 16 fragments into LDS
 *            and then reading the 8 fragments of every half-iteration back
 *            from LDS before its 16 instructions (512 bytes of LDS reads per
 *            instruction, as in the operator's GEMM).
 * One workgroup per compute unit puts one wave on every SIMD.
 *   out    device fp32, workgroups * 256 values (each lane's accumulator sum)
 *   flops  host: receives the launch's floating-point operation count
 *          (workgroups * 4 * iters * 2 * 128 * 128 * 32) */
int plora_probe_mfma(const void* operands, int32_t shape, int32_t workgroups, int32_t iters, float* out,
                     double* flops, void* stream);

/* dst[0..bytes) = src[0..bytes) with `workgroups` workgroups of 256 threads,
 * grid-stride; bytes a multiple of 16; the buffers must not overlap.  Moves
 * 2 * bytes through HBM. */
int plora_probe_copy(const void* src, void* dst, size_t bytes, int32_t workgroups, void* stream);

/* Reads src[0..bytes) (bytes a multiple of 16) with `workgroups` workgroups
 * of 256 threads; out (device, workgroups * 256 uint32) receives each thread's
 * XOR of what it read. */
int plora_probe_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* out, void* stream);

/* `workgroups` workgroups of 4 waves each stream src[0..span_bytes) into LDS
 * `iters` times (wave w takes the 1 KiB pieces w, w + 4, ... of every 4 KiB;
 * up to 6 loads of 16 bytes per lane in flight per wave, into a ring of 8
 * LDS slots of 1 KiB per wave).  A span of a few MiB stays in L2 after the
 * first pass, so the launch measures the L2 -> LDS rate.  span_bytes a
 * positive multiple of 4096, at most 1 GiB.
 *   out    device, workgroups * 256 uint32 (a word each thread finds in LDS)
 *   bytes  host: receives workgroups * iters * span_bytes */
int plora_probe_lds_dma(const void* src, size_t span_bytes, int32_t workgroups, int32_t iters, uint32_t* out,
                        double* bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PLORA_PROBE_H */
