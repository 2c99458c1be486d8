/*
 * fluxmi_probe.h -- measurement entry point of libfluxmi (not part of the
 * fused operators): the matrix-core ceiling that the GEMM kernels are read
 * against.
 */
#ifndef FLUXMI_PROBE_H
#define FLUXMI_PROBE_H

#include "fluxmi.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fm_probe_mfma -- a register-only MFMA loop on every compute unit, with no
 * memory traffic inside the loop: one workgroup per CU of 4 * waves_per_simd
 * waves, each issuing iters x 8 MFMAs on eight different operand register
 * sets in turn (so the operand bits change from one instruction to the next,
 * as in a GEMM), into independent fp32 accumulator chains.  This is the rate
 * the dense peak (256 CUs x 2.4 GHz x 4096 flop/clk for fp16/bf16) assumes,
 * measured at the clock the chip actually holds under its power limit with
 * such operands.
 *   dt              FM_F16 or FM_BF16 operands.
 *   mfma16          0: v_mfma_f32_32x32x16 (32768 flop each, the form the
 *                   GEMMs use); 1: v_mfma_f32_16x16x32 (16384 flop each).
 *   waves_per_simd  1 or 2.
 *   iters           1 .. 2^30 loop iterations per wave.
 *   zero_operands   0: approximately N(0,1) operands (an Irwin-Hall sum of
 *                   four uniforms per value); 1: all-zero operands.
 *   out, out_words  device uint64 buffer of out_words words, 8-byte aligned,
 *                   at least 4 x the CU count (written): per workgroup, the
 *                   shader-clock cycles and the 100 MHz constant-rate ticks
 *                   across its loop, and a word derived from the
 *                   accumulators.
 * Flops of one launch = CUs x 4 x waves_per_simd x iters x 8 x flop per MFMA;
 * the caller times the launch with events.  FM_ERR_INVALID_ARG for values
 * outside these ranges.
 */
fm_status_t fm_probe_mfma(fm_dtype_t dt, int32_t mfma16, int32_t waves_per_simd, int64_t iters,
                          int32_t zero_operands, uint64_t* out, int64_t out_words,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FLUXMI_PROBE_H */
