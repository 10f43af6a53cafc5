/*
 * ttt_peak.h -- C ABI of libttt_peak.so, the calibration kernels the
 * measurements put beside the published MI355X peaks: the HBM bandwidth a plain
 * copy kernel reaches, the dense bf16 matrix-core rate an MFMA loop reaches, and
 * the device's compute-unit count and clock. None of this is part of the layer's
 * computation; libttt.so does not depend on it.
 *
 * Conventions: device pointers are caller-owned; calls are asynchronous on
 * `hip_stream` (a hipStream_t, NULL = the null stream); argument errors are
 * reported before any HIP call. Return values are the TTT_* status codes of
 * ttt.h: 0 success, 1 invalid argument, 4 HIP error.
 */
#ifndef TTT_PEAK_H
#define TTT_PEAK_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Device `device`: number of compute units, shader clock in kHz, wavefront
 * width. Synchronous; any pointer may be NULL. */
int ttt_peak_device_info(int device, int* compute_units, int* clock_khz, int* wavefront_size);

/* dst[0 .. bytes) = src[0 .. bytes): a grid-stride copy with 16-byte accesses.
 * bytes must be a positive multiple of 16, both pointers 16-byte aligned, and
 * the ranges must not overlap. It moves 2 * bytes through HBM. */
int ttt_peak_copy(const void* src, void* dst, size_t bytes, void* hip_stream);

/* `blocks` workgroups of four waves; every wave runs `iters` iterations of four
 * independent v_mfma_f32_32x32x16_bf16 accumulation chains and writes one float
 * per lane to out[0 .. blocks * 256) (a checksum that keeps the work alive).
 * blocks >= 1, iters >= 1. */
int ttt_peak_mfma(float* out, int blocks, int iters, void* hip_stream);

/* Dense flops one ttt_peak_mfma call performs (2 * 32 * 32 * 16 per MFMA). */
double ttt_peak_mfma_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* TTT_PEAK_H */
