/*
 * qk4v8_peaks.h - microbenchmarks that measure the MI355X (gfx950) peaks the
 * QK4V8 kernels are priced against: HBM streaming read bandwidth, the block-
 * scaled FP4 and FP8 matrix-core rates, and the exp2 rate of the vector ALU.
 *
 * The page "MpFA免训练量化：QK4V8混合精度在Blackwell上的推理加速实践" (§5.1) tunes
 * the kernel by comparing its compute and bandwidth utilisation with what the
 * hardware delivers; these calls measure that delivery on the machine at hand,
 * next to the vendor's nominal figures.  They compute nothing of the method.
 *
 * Conventions: device pointers, asynchronous on `stream` (time them with
 * events on that stream), host-side validation, status codes as in qk4v8.h
 * (0 ok, 1 null pointer, 2 bad size, 6 HIP error).  `sink` receives values
 * the loops depend on, so that no work is optimised away; its contents are
 * meaningless.  Separate library: libqk4v8_peaks.so.
 */
#ifndef QK4V8_PEAKS_H
#define QK4V8_PEAKS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read of `bytes` (a multiple of 16, at least 16) from the device
 * buffer `buf` (16-byte aligned) with non-temporal 16-byte loads, every byte
 * read once; one grid over all CUs.  sink: device uint32 [4096].
 */
int qk4v8_peak_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * Back-to-back matrix instructions on four independent accumulators per
 * wave, 8 waves per CU on every CU, `iters` rounds of four.
 *   fmt  : 4 = v_mfma_scale_f32_32x32x64_f8f6f4 FP4 (E2M1) x FP4,
 *          0 = the same instruction FP8 (E4M3) x FP8,
 *          16 = v_mfma_f32_32x32x16_bf16.
 *   iters: 1 .. 1<<24.
 *   flops: out (host), the dense flops the launch executes
 *          (2 * 32 * 32 * 64, or 2 * 32 * 32 * 16 for bf16, per instruction).
 * sink: device float [CUs * 512].
 */
int qk4v8_peak_mfma(int fmt, int iters, float* sink, double* flops, hipStream_t stream);

/*
 * v_exp_f32 on eight independent registers per lane, 8 waves per CU on every
 * CU, `iters` rounds (1 .. 1<<24).  exps: out (host), the lane-exponentials
 * the launch executes.  sink: device float [CUs * 512].
 */
int qk4v8_peak_exp2(int iters, float* sink, double* exps, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QK4V8_PEAKS_H */
