/*
 * Measurement probe built beside the encoder library (libwenc_probe.so), used by the benchmark
 * only: the dense 16-bit (and MXFP8) MFMA rate the GPU sustains, to report each kernel's rate
 * against the measured peak as well as the rated one.  Not part of the encoder's C ABI.
 */
#ifndef WENC_PROBE_H
#define WENC_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

#define WENC_PROBE_F16 2
#define WENC_PROBE_BF16 1
#define WENC_PROBE_MXFP8 8

/*
 * Enqueue `blocks` workgroups of 256 threads on `stream`; each wavefront issues iters x 4
 * independent v_mfma_f32_32x32x16 of `dtype` (or, for WENC_PROBE_MXFP8,
 * v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 operands with unit scales) on register operands.
 * clocks: device, 2 values: shader-clock cycles and 100 MHz reference ticks across wavefront 0 of workgroup 0's loop
 * (their ratio x 100 MHz is the shader clock).  sink: device float[blocks * 256], never written
 * (keeps the work live).  Returns 0, 1 for a bad argument, 4 for a launch error.
 */
int wenc_probe_mfma(int dtype, int blocks, int iters, unsigned long long* clocks, float* sink,
                    void* stream);

/* Floating-point operations of one wenc_probe_mfma call of `dtype`. */
long long wenc_probe_mfma_flops(int dtype, int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif
