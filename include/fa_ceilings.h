/*
 * fa_ceilings.h -- same-machine ceilings that the attention kernels' rooflines
 * are read against (libfa_ceilings.so).  The datasheet peaks are what a
 * kernel is finally measured against; these loops measure what this GPU
 * sustains at its running clock, one resource at a time, following the
 * order of "从 Volta/Turing、Ampere、Ada 到 Hopper：硬件、PTX 与 Kernel 编程范式
 * 演进", section "到不了理论性能：硬件限制还是优化问题", step 2: a
 * bandwidth ceiling first, then instruction ceilings.
 *
 * Every call is synchronous (it times its own launches with HIP events on
 * the null stream and waits for them), allocates and frees its own small
 * output buffers, and returns 0 on success or 1 with a message for
 * fa_ceil_last_error().  Buffers passed in are device memory owned by the
 * caller.
 */
#ifndef FA_CEILINGS_H_
#define FA_CEILINGS_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (a multiple of 16 KiB is used; 16-byte aligned
 * device buffer, much larger than the caches) `reps` times: GB/s. */
int fa_ceil_hbm_read(const void *buf, size_t bytes, int reps, double *gbps);

/* One wave per SIMD issuing independent v_mfma_f32_32x32x16_bf16 (fp8 = 0)
 * or v_mfma_f32_32x32x64_f8f6f4 (fp8 = 1) on four accumulators, `iters`
 * trips of 8: TFLOP/s, and the shader clock the loop ran at (MHz, from the
 * waves' cycle counters against the constant-rate real-time counter). */
int fa_ceil_mfma(int fp8, int iters, double *tflops, double *clock_mhz);

/* Cycles per MFMA when k_valu (0, 2, 4, 5, 6 or 8) independent v_fma_f32, or
 * -k_valu (1, 2 or 4) independent v_exp_f32, sit between consecutive MFMAs
 * of one wave, one wave per SIMD. */
int fa_ceil_coissue(int k_valu, int iters, double *cycles_per_mfma);

/* Conflict-free LDS read stream, 8 waves per CU: ds_read_b128
 * (transposing = 0) or ds_read_b64_tr_b16 (1): bytes per clock per CU. */
int fa_ceil_lds(int transposing, int iters, double *bytes_per_clk_cu);

/* Independent v_fma_f32 (exp = 0) or v_exp_f32 (1) stream, one wave per
 * SIMD: cycles per wave-wide instruction. */
int fa_ceil_valu(int exp, int iters, double *cycles_per_instr);

const char *fa_ceil_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_CEILINGS_H_ */
