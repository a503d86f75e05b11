/*
 * libmla measurement aids: two kernels that give the chip's sustained ceilings
 * on the box at hand, so that the method's kernels can be read against what
 * the hardware delivers as well as against its published peaks (MI355X: HBM3E
 * 8 TB/s, dense 16-bit MFMA 2.5 PFLOP/s). They are not steps of the method.
 *
 * Conventions as in mla.h: device pointers are owned by the caller, calls are
 * asynchronous on `stream`, the return value reports argument validation and
 * launch errors only.
 */
#ifndef MLA_CEILING_H
#define MLA_CEILING_H

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of operand data mla_ceiling_mfma reads (48 fragments of 64 lanes x 8 fp16). */
#define MLA_CEILING_MFMA_OPERAND_BYTES 49152

/*
 * Streaming read of `bytes` bytes at `buf` (device, 16-byte aligned, `bytes` a
 * positive multiple of 16): every byte is loaded once with 16-byte
 * nontemporal loads, 8 in flight per thread over a grid of 16384 workgroups
 * of 512 threads (the fastest of a sweep over grid, block and unroll sizes
 * and cache policies on MI355X). Nothing is
 * written except, with negligible probability, one word of `sink` (device,
 * 4 bytes), which keeps the loads from being optimised away. Algorithmic bytes
 * per launch: `bytes`. A buffer well above the 256 MB last-level cache
 * measures HBM.
 * Errors: MLA_ERR_NULL (null buf or sink), MLA_ERR_SHAPE (size or alignment).
 */
mla_status mla_ceiling_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * Dense fp16 MFMA loop (v_mfma_f32_32x32x16_f16, fp32 accumulation) on 512
 * workgroups of 8 waves (two per compute unit), `iters` iterations, with the
 * operands taken from `operands` (device, MLA_CEILING_MFMA_OPERAND_BYTES bytes
 * of fp16 supplied by the caller: random values make the matrix cores draw
 * the power real data does; zeros do not).
 *   lds_operands = 0: A and B stay in registers, 4 independent accumulation
 *                     chains of 12 products per wave and iteration;
 *   lds_operands = 1: every A operand is a 16-byte LDS read, 2 chains of 12
 *                     products per wave and iteration (the operand traffic
 *                     of an attention kernel that keeps the query in
 *                     registers and streams keys and values through LDS).
 * `flops` (host, nullable) receives the launch's flop count (2*32*32*16 per
 * product). `sink` (device, 4 bytes) as above.
 * Errors: MLA_ERR_NULL (null operands or sink), MLA_ERR_SHAPE (iters < 1 or
 * lds_operands not 0/1).
 */
mla_status mla_ceiling_mfma(const uint16_t* operands, int32_t iters, int32_t lds_operands, float* sink,
                            double* flops, hipStream_t stream);

/*
 * The device's compute-unit count and peak shader and memory clocks (kHz), as
 * the HIP runtime reports them, for reading the published peaks against the
 * chip at hand (dense 16-bit MFMA: 4096 flop per clock per compute unit).
 * All outputs are host pointers. Errors: MLA_ERR_NULL, MLA_ERR_HIP (an
 * invalid device or a runtime failure).
 */
mla_status mla_device_info(int32_t device, int32_t* compute_units, int32_t* peak_sclk_khz, int32_t* peak_mclk_khz);

#ifdef __cplusplus
}
#endif

#endif /* MLA_CEILING_H */
