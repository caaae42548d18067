/*
 * ar_peaks -- measured peaks of the MI355X (gfx950) the library runs on: the
 * denominators, beside AMD's published figures (HBM3E 8 TB/s, dense bf16
 * MFMA 2.5 PFLOP/s), of the roofline fractions the benchmark reports for the
 * tuning kernels.  A measurement aid, not part of the tuning path.
 *
 * Every call runs on the current device, allocate what they need with
 * hipMalloc and free it before returning, time with HIP events on a stream
 * of their own and synchronize.  They return 0 on success or the
 * hipError_t of the failing HIP call; a result pointer that is NULL, a size
 * that is not a positive multiple of 4096 bytes or a count < 1 returns
 * hipErrorInvalidValue (1) before any HIP call.
 */
#ifndef AR_PEAKS_H
#define AR_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define ARP_API __attribute__((visibility("default")))
#else
#define ARP_API
#endif

/* Device-to-device copy of `bytes` bytes between two fresh buffers, 16-byte
 * nontemporal vector loads and stores, eight in flight per thread, over a
 * grid of 16 workgroups per compute unit,
 * repeated `reps` times after one untimed pass.  *gbs = 2 * bytes * reps /
 * elapsed (bytes read plus bytes written) in GB/s; with bytes well above the
 * 256 MB last-level cache this is the HBM bandwidth a streaming kernel sees. */
ARP_API int ar_peak_copy_gbs(int64_t bytes, int32_t reps, double* gbs);

/* Read-only stream of `bytes` bytes (a positive multiple of 65536; else
 * hipErrorInvalidValue) from a fresh buffer, loaded the way the GEMM main
 * loops load their operands: global_load_lds_dwordx4 straight into LDS, one
 * 512-thread workgroup per compute unit, each streaming its own run of 64 KB
 * pieces, two in flight per workgroup; nothing is written.  Repeated `reps` times after one
 * untimed pass.  *gbs = bytes * reps / elapsed in GB/s: the HBM read rate of
 * a kernel that only streams in. */
ARP_API int ar_peak_read_gbs(int64_t bytes, int32_t reps, double* gbs);

/* Back-to-back v_mfma_f32_32x32x16_bf16 (32*32*16*2 flops each) on operands
 * held in registers: four independent accumulators per wavefront, two
 * wavefronts per SIMD on every compute unit, `iters` rounds of four.
 * *tflops = flops / elapsed in TFLOP/s: the dense bf16 matrix rate reachable
 * with no memory traffic at all. */
ARP_API int ar_peak_mfma_tflops(int32_t iters, double* tflops);

#ifdef __cplusplus
}
#endif
#endif /* AR_PEAKS_H */
