/*
 * qr_peaks.h - measurement probes of libqr: what this GPU attains for a
 * streaming copy and for back-to-back dense MFMAs.  The benchmark puts every
 * hot-path kernel against these measured ceilings beside the datasheet peaks
 * (HBM 8 TB/s, int8 MFMA 5.0 POP/s, fp16 MFMA 2.5 PFLOP/s).  They compute
 * nothing of the method.  Pointers are device pointers; calls are
 * asynchronous on `stream` and validate their arguments on the host first.
 */
#ifndef QR_PEAKS_H
#define QR_PEAKS_H

#include <stdint.h>

#include "qr.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` (a multiple of 16) from src to dst, both 16-byte aligned and
 * not overlapping: 16-byte nontemporal loads and stores, eight loads in
 * flight per lane, one 1024-thread block per CU.  HBM traffic = 2 * bytes.
 */
qr_status qr_peak_copy(const void *src, void *dst, int64_t bytes, void *stream);

/*
 * Number of waves qr_peak_mfma launches on the current device (8 per CU);
 * `out` must hold 64 int32 per wave.
 */
int64_t qr_peak_mfma_waves(void);

/*
 * Every wave issues `iters` (1 .. 2^24) rounds of four independent MFMAs with
 * no memory traffic: kind 0 = v_mfma_i32_32x32x32_i8 (65536 int8 ops each),
 * kind 1 = v_mfma_f32_16x16x32_f16 (16384 fp16 flops each), kind 2 =
 * v_mfma_f32_32x32x16_f16 (32768 fp16 flops each), kind 3 =
 * v_mfma_i32_16x16x64_i8 (32768 int8 ops each); any other kind is
 * QR_EINVAL.  Work per call =
 * waves * iters * 4 * (ops per MFMA).  `out` receives one checksum per lane
 * (so the loop cannot be removed), int32 [waves * 64], 4-byte aligned.
 */
qr_status qr_peak_mfma(int64_t kind, int64_t iters, int32_t *out, void *stream);

/*
 * The int8 MFMA loop of kind 0 on operands taken from packed int4 codes (two
 * per byte, as qr_rotate_quant writes them), widened once to the int8 form
 * the int4 GEMM multiplies (16 q): wave v, lane l loads the 16-byte pieces
 * ((64 v + l) * 8 + f) mod (bytes / 16), f < 8, of `a` (A operands) and of
 * `w` (W operands), then issues `iters` (1 .. 2^24) rounds of 32
 * v_mfma_i32_32x32x32_i8 over four accumulators.  On dense MFMA work this
 * part lowers its clock as more operand bits toggle, so with a workload's
 * own codes this is the int8 rate attainable on that data.  a_bytes and
 * w_bytes: multiples of 16, at least 16 (else QR_ESHAPE); a, w 16-byte
 * aligned, out 4-byte aligned (QR_EALIGN); null pointers QR_EINVAL.  Work per
 * call = waves * iters * 32 * 65536 int8 ops (waves = qr_peak_mfma_waves()).
 * `out` receives, per lane, the int32 sum of its 64 accumulator values.
 */
qr_status qr_peak_mfma_codes(const uint8_t *a, int64_t a_bytes, const uint8_t *w, int64_t w_bytes, int64_t iters,
                             int32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QR_PEAKS_H */
