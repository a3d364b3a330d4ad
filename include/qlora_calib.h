/*
 * qlora_calib.h - calibration kernels of the MI355X QLoRA library.
 *
 * They measure what the device delivers (HBM streaming bandwidth, dense bf16
 * MFMA rate) so that the layer kernels' roofline fractions can be read
 * against the achievable peaks as well as the published ones.  They are not
 * part of the QLoRA path.  Pointers are caller-owned device memory; work is
 * enqueued on `stream` (a hipStream_t, NULL = default) and the call returns
 * before it completes.
 */
#ifndef QLORA_MI355X_CALIB_H
#define QLORA_MI355X_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_CALIB_ERR 1

/*
 * qlora_calib_copy - dst[0:bytes) = src[0:bytes) with 128-bit nontemporal
 *   loads and stores, one contiguous 16 KB span per workgroup (each thread
 *   keeps four 16-byte loads in flight).  0 < bytes <= 2^44, a multiple of 16;
 *   src and dst 16-byte aligned and not overlapping.
 *   Returns 0, or QLORA_CALIB_ERR for bad arguments or a refused launch.
 */
int qlora_calib_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * qlora_calib_mfma - `workgroups` workgroups of four waves (one per SIMD of a
 *   CU), each wave running 16 independent chains of v_mfma_f32_32x32x16_bf16
 *   for `iters` rounds on operands read from seed[0:128) (32-bit words);
 *   out[workgroups * 256] receives one sum per thread.
 *   Returns 0, or QLORA_CALIB_ERR.
 */
int qlora_calib_mfma(const uint32_t* seed, float* out, int workgroups, int iters, void* stream);

/* qlora_calib_mfma_flops - the flops one qlora_calib_mfma call performs. */
double qlora_calib_mfma_flops(int workgroups, int iters);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_MI355X_CALIB_H */
