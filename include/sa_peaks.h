/*
 * sa_peaks.h -- C ABI of libsa_peaks.so, two micro-benchmarks that measure
 * the denominators of the roofline on the machine at hand: the bf16
 * matrix-core rate a kernel can sustain, and the HBM copy bandwidth.  They
 * are measurement aids beside the published peaks, not operations of the
 * attention path, and nothing in libsa uses them.
 */
#ifndef SA_PEAKS_H
#define SA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Sustained v_mfma_f32_32x32x16_bf16 rate in TFLOP/s (2*32*32*16 flops per
 * instruction): `blocks` workgroups of four waves, each wave issuing `iters`
 * rounds of eight independent products, timed with HIP events on `stream`
 * (a hipStream_t, NULL for the default stream): the best of three launches
 * after one untimed launch.
 * Blocks until done.  Returns a negative value if a HIP call fails.
 */
double sap_mfma_bf16_tflops(int blocks, int iters, void* stream);

/*
 * Device-to-device copy bandwidth in GB/s (bytes read + bytes written per
 * second): `reps` launches of a copy of `bytes` bytes from src to dst
 * (non-temporal 16-byte loads and stores; device pointers, 16-byte aligned,
 * bytes a multiple of 16, owned by the caller), timed with HIP events on
 * `stream` after one untimed launch.  Blocks until done.  Returns a negative value on a bad
 * argument or a failed HIP call.
 */
double sap_copy_gbs(void* dst, const void* src, size_t bytes, int reps, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_PEAKS_H */
