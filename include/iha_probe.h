/*
 * iha_probe.h - measurement probe used by the benchmark (libiha_probe.so).  Not part of
 * the IHA forward pass: it measures the chip the forward runs on.
 */
#ifndef IHA_PROBE_H
#define IHA_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Dense fp16 matrix-core rate under a pure-product load on the current device: every CU
 * runs two waves per SIMD issuing independent 32x32x16 fp16 products for about
 * `milliseconds` (after a sizing run and a full-length warm-up run).
 *   *tflops     achieved TFLOP/s (2 flops per multiply-add), from HIP events
 *   *clock_mhz  shader clock during the timed run: the shader-clock counter (s_memtime)
 *               against the constant 100 MHz counter (s_memrealtime), read by one wave
 *   *kernel_ms  duration of the timed run
 * Returns 0 on success, 1 for a bad argument, 2 if device memory or events could not be
 * created, 3 if the run failed.  Allocates (and frees) a small device buffer. */
int ihp_mfma_rate(int milliseconds, double* tflops, double* clock_mhz, double* kernel_ms);

#ifdef __cplusplus
}
#endif
#endif /* IHA_PROBE_H */
