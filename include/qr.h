/*
 * qr.h - C ABI of the QuaRot 4-bit linear-layer inference hot path on AMD
 * MI355X (gfx950).
 *
 * The method (QuaRot; abstract of the ISTA Research Explorer record and the
 * "Summary" / "Key points" of the Elamur Research summary): rotate the input
 * of a linear layer Y = X W by an orthogonal matrix R online, quantize the
 * rotated activations to 4 bits with round-to-nearest, multiply them in
 * integers against weights that were rotated by R^T and quantized offline,
 * and dequantize the output; the KV cache is stored in 4 bits after a
 * head-wise Hadamard rotation.  The identity that makes this exact before
 * quantization is Y = XW = (XR)(R^T W) (DuQuant page, Knowl 1).
 *
 * Conventions for every call:
 *  - Pointers marked "device" are HIP device (or managed) pointers; every
 *    call is asynchronous on `stream` (a hipStream_t passed as void*, NULL =
 *    the null stream) and never synchronises.
 *  - The caller owns every buffer.  The library keeps no pointer after
 *    return, allocates nothing, holds no mutable global state and may be
 *    called concurrently from several host threads.
 *  - Arguments are validated on the host before anything is launched.  On a
 *    bad argument the call returns a non-zero qr_status, launches nothing and
 *    writes nothing.  QR_EDEVICE reports a failed launch; faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Inputs must be finite; non-finite input gives unspecified codes.
 *  - fp16 data is IEEE binary16 stored as 16-bit words.
 *  - Packed 4-bit codes: two per byte, the element with the even index in
 *    the low nibble.  Symmetric codes are two's complement in [-8, 7];
 *    KV codes are unsigned in [0, 15].
 */
#ifndef QR_H
#define QR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QR_OK = 0,
  QR_EINVAL = 1,   /* null pointer, bad enum value, negative size        */
  QR_ESHAPE = 2,   /* sizes the operation does not support               */
  QR_EALIGN = 3,   /* pointer or leading dimension not aligned as needed */
  QR_EDEVICE = 4,  /* the HIP runtime reported an error at launch        */
  QR_ESCRATCH = 5  /* more scratch than qr_kv_attn_decode_noalloc holds  */
} qr_status;

/*
 * An orthogonal rotation R of row width n, applied as y = x R.
 *
 *   dense_m == 1:  R = D . H_n / sqrt(n)                   (had_n == n)
 *   dense_m  > 1:  R = D . ((H_p / sqrt(p)) kron O)         (p = had_n)
 *
 * H_p is the Sylvester Hadamard matrix in natural order (H_1 = [1],
 * H_2k = [[H_k, H_k], [H_k, -H_k]]), normalised by 1/sqrt(p) as the DuQuant
 * page (Knowl 12) states for its fixed Hadamard rotations.  D = diag(signs)
 * is the random +-1 diagonal of the randomized Hadamard transform (QuaRot
 * press article; QuaRot summary, "Summary"), applied to the input before the
 * transform.  O is a dense dense_m x dense_m orthogonal factor (random
 * orthogonal multiplication: QuIP summary, abstract; two-factor Kronecker
 * construction: the QuIP# quote on the same page) used where n is not a
 * power of two, e.g. n = 11008 = 64 * 172.  In the Kronecker product the
 * dense index is the fastest: element k = i * dense_m + a.
 *
 * Fields: n = had_n * dense_m, n even, 2 <= n <= 32768, had_n a power of two
 * in [1, 32768], dense_m in [1, 256], and dense_m <= 16 when n > 16384 (for
 * example n = 28672 = 4096 * 7).  `dense` (device, fp32, row-major
 * [dense_m][dense_m]) must be NULL iff dense_m == 1; the library does not
 * check that it is orthogonal.  `signs` (device, int8 [n], each +1 or -1,
 * 4-byte aligned) may be NULL for D = I.
 */
typedef struct {
  int64_t n;
  int64_t had_n;
  int64_t dense_m;
  const float *dense;
  const int8_t *signs;
} qr_rotation;

/*
 * Online rotation + symmetric 4-bit round-to-nearest quantization + packing
 * of `rows` activation rows (QuaRot summary, "Key points": activations
 * quantized on the fly with RTN; group size 128 as the group-wise option).
 *
 *   y     = x[r, :] R                      (fp32 arithmetic on fp16 input)
 *   s     = max |y| / 7 over the row (group == 0) or over each contiguous
 *           block of `group` elements of y
 *   q     = clamp(rint(y / s), -8, 7)      (round half to even)
 *   s = 0 and q = 0 for an all-zero row or group.
 *
 * x_f16   device, fp16, row r at x_f16 + r * ld_x (elements); ld_x >= n,
 *         ld_x a multiple of 8, x_f16 16-byte aligned.
 * rows    >= 0 (0 is a no-op).
 * group   0 (per row) or a power of two >= 32 that divides n.
 * codes   device, [rows][n/2] bytes, 16-byte aligned.
 * scales  device, fp32 [rows] (group 0) or [rows][n/group].
 *
 * The same call prepares weights offline: since (R^T W)^T = W^T R, rotating
 * and quantizing the rows of W^T ([N][K]) gives per-output-channel (or
 * group-wise along K) weight codes and scales in the layout qr_int4_gemm
 * takes.
 */
qr_status qr_rotate_quant(const void *x_f16, int64_t rows, int64_t ld_x,
                          const qr_rotation *rot, int64_t group,
                          uint8_t *codes, float *scales, void *stream);

/*
 * 4-bit integer GEMM with a dequantizing fp16 epilogue (QuaRot abstract: all
 * matrix multiplications performed in 4 bits).
 *
 *   acc[t, n]  = sum_k qa[t, k] * qw[n, k]            exact integer sum
 *   group 0:   y[t, n] = fp16(acc[t, n] * a_scales[t] * w_scales[n])
 *   group g:   y[t, n] = fp16(sum_j acc_j[t, n] * a_scales[t, j] * w_scales[n, j])
 *              acc_j summing k in [j g, (j+1) g)
 * The scale products and the sum over groups are formed in fp32; the
 * conversion to fp16 rounds to nearest even.
 *
 * a_codes   device, [M][K/2] packed two's-complement codes (16-byte aligned)
 * a_scales  device, fp32 [M] or [M][K/group]
 * w_codes   device, [N][K/2] packed codes, one row per output channel
 * w_scales  device, fp32 [N] or [N][K/group]
 * M, N >= 0; K > 0, a multiple of 128 and below 2^17, i.e. at most 130944
 * (every product is at most 2^14 in magnitude, so the int32 sums stay
 * exact; K >= 2^17 returns QR_ESHAPE); group 0 or a multiple of 128 that
 * divides K.
 * y_f16     device, fp16 [M][ld_y], ld_y >= N, 2-byte aligned.
 *
 * M <= 64 runs the memory-bound decode kernel (weights streamed once); larger
 * M runs the MFMA-bound prefill kernel.  Both give identical integer sums.
 */
qr_status qr_int4_gemm(const uint8_t *a_codes, const float *a_scales,
                       const uint8_t *w_codes, const float *w_scales,
                       int64_t M, int64_t N, int64_t K, int64_t group,
                       void *y_f16, int64_t ld_y, void *stream);

/*
 * qr_rotate_quant of the feed-forward activation that feeds down_proj,
 * formed on the fly (QuaRot abstract: the activations of the feed-forward
 * components are rotated too): row r is
 *   x = fp16(silu(gate[r, :]) * up[r, :]),   silu(g) = g / (1 + e^-g)
 * in fp32 with one fp16 rounding, then rotated, quantized and packed as by
 * qr_rotate_quant.  x itself is never written.
 * gate_f16, up_f16  device fp16, row r at ptr + r * ld (elements), 16-byte
 *                   aligned; ld >= n, a multiple of 8 (e.g. the two halves of
 *                   a fused gate/up projection output [rows][2n], ld = 2n).
 * All other arguments as for qr_rotate_quant.  n = 4096 * m (2 <= m <= 8, no
 * signs, per row; 28672 for LLaMA-2-70B) runs the MFMA kernel; other
 * rotations run the reference-shape kernel.
 */
qr_status qr_swiglu_rotate_quant(const void *gate_f16, const void *up_f16, int64_t rows, int64_t ld,
                                 const qr_rotation *rot, int64_t group, uint8_t *codes,
                                 float *scales, void *stream);

/*
 * 6- and 8-bit variants (QuaRot abstract: plain round-to-nearest gives
 * lossless 6- and 8-bit models).  The same rotation and symmetric RTN with
 * qmax = 2^(bits-1) - 1 (31 or 127) in place of 7:
 *   s = max |y| / qmax,  q = clamp(rint(y / s), -qmax-1, qmax)
 * codes are int8, one per byte, [rows][n] (16-byte aligned), not packed.
 * bits is 6 or 8 (anything else: QR_EINVAL); all other arguments as for
 * qr_rotate_quant.  Widths 4096 and 8192 without a dense factor (group 0 or
 * 128) run the MFMA kernel; other rotations run the reference-shape kernel.
 */
qr_status qr_rotate_quant_i8(const void *x_f16, int64_t rows, int64_t ld_x,
                             const qr_rotation *rot, int64_t group, int64_t bits,
                             int8_t *codes, float *scales, void *stream);

/*
 * The GEMM of qr_int4_gemm on int8 codes (the 6- and 8-bit variants): the
 * codes go into the int8 matrix cores as they are.  a_codes [M][K] and
 * w_codes [N][K] int8 (16-byte aligned); every other argument and the
 * epilogue as for qr_int4_gemm.  K < 2^17 (at most 130944) keeps the int32
 * sums exact.
 */
qr_status qr_int8_gemm(const int8_t *a_codes, const float *a_scales,
                       const int8_t *w_codes, const float *w_scales,
                       int64_t M, int64_t N, int64_t K, int64_t group,
                       void *y_f16, int64_t ld_y, void *stream);

/*
 * Head-wise rotated asymmetric 4-bit KV-cache quantization (QuaRot abstract:
 * the KV cache in 4 bits; DuQuant page, Knowl 12: fixed Hadamard rotation
 * +-1/sqrt(2^n) with per-token / per-head asymmetric quantization and the
 * step (gamma max - beta min)/(2^b - 1), here gamma = beta = 1, b = 4).
 *
 * For every token t and head h, with v = kv[t, h, :]:
 *   y    = (v * signs) H_D / sqrt(D)        (signs optional; D = head_dim)
 *   lo   = min(min y, 0),  hi = max(max y, 0),  step = (hi - lo) / 15
 *   z    = rint(-lo / step)
 *   q    = clamp(rint(y / step) + z, 0, 15)
 *   step = 0, z = 0, q = 0 when hi == lo.
 * Dequantization is (q - z) * step in the rotated domain.
 *
 * kv_f16  device fp16; element (t, h, d) at kv_f16 + t * ld_kv + h * head_dim + d.
 *         ld_kv >= H * head_dim, multiple of 8; 16-byte aligned.  This lets
 *         the K or V slice of a fused QKV output be quantized in place.
 * T, H    >= 0; head_dim == 128.
 * signs   device int8 [head_dim] of +-1 (4-byte aligned), or NULL.
 * codes   device [T][H][head_dim/2] unsigned packed codes (16-byte aligned)
 * scales  device fp32 [T][H] (the step)
 * zeros   device uint8 [T][H] (the zero point z)
 */
qr_status qr_kv_quant(const void *kv_f16, int64_t T, int64_t H, int64_t head_dim,
                      int64_t ld_kv, const int8_t *signs,
                      uint8_t *codes, float *scales, uint8_t *zeros, void *stream);

/*
 * One decode step of attention over the rotated 4-bit KV cache (QuaRot
 * abstract: computational invariance of the attention mechanism and the KV
 * cache under the rotation, the cache held in 4 bits; DuQuant page, Knowl 12:
 * Query x Key and attention output x Value pass through fixed head-wise
 * Hadamard rotations, the softmax output stays unquantized).
 *
 * For sequence b and query head h (KV head g = h / (Hq / Hkv)), over the
 * tokens t < lens[b] of the cache written by qr_kv_quant with the same signs:
 *   K_t = ((c_t - z_t) step_t) R^T,   V_t likewise,   R = diag(signs) H_128 / sqrt(128)
 *   out = sum_t softmax_t(sm_scale q . K_t) V_t            (fp32 inside)
 * computed as ((q R) against the stored rotated cache) R^T.  An empty
 * sequence (lens[b] == 0 or T == 0) gives zeros.
 *
 * q_f16     device fp16 [B][Hq][128] (2-byte aligned)
 * k_codes   device [B][T][Hkv][64] packed unsigned codes, as qr_kv_quant
 *           writes them for B*T tokens (16-byte aligned); v_codes likewise.
 * k_scales  device fp32 [B][T][Hkv] steps; k_zeros device uint8 [B][T][Hkv]
 *           zero points; v_* likewise.
 * lens      device int32 [B], tokens per sequence (clamped to [0, T]), or NULL
 *           for T everywhere.
 * signs     device int8 [128] of +-1 the cache was quantized with, or NULL.
 * sm_scale  softmax scale, typically 1/sqrt(128); finite.
 * workspace device scratch of at least qr_kv_attn_decode_workspace(...) bytes
 *           (16-byte aligned) when that size is non-zero: a sequence is then
 *           split into chunks of tokens whose partial results are merged by a
 *           second kernel.  NULL with workspace_bytes == 0 runs one chunk per
 *           sequence instead (no workspace; fewer blocks for small batches).
 *           A non-NULL workspace smaller than required gives QR_EINVAL.
 * out_f16   device fp16 [B][Hq][128] (2-byte aligned).
 * Hq % Hkv == 0; head_dim == 128; T * Hkv * 64 < 2^31 (one sequence's
 * codes).  The caller owns every buffer; concurrent calls must not share a
 * workspace.
 */
qr_status qr_kv_attn_decode(const void *q_f16, int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                            int64_t head_dim, const uint8_t *k_codes, const float *k_scales,
                            const uint8_t *k_zeros, const uint8_t *v_codes, const float *v_scales,
                            const uint8_t *v_zeros, const int32_t *lens, const int8_t *signs,
                            float sm_scale, void *workspace, int64_t workspace_bytes, void *out_f16,
                            void *stream);

/*
 * qr_kv_attn_decode for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * plan, kernels and results as qr_kv_attn_decode with a workspace of
 * qr_kv_attn_decode_workspace(...) bytes, with the split partials kept in a
 * static device array of the library instead (16 MiB per GPU, part of the
 * library's code object, held until the process ends).  Nothing is
 * allocated and no library routine that allocates is called.
 * Arguments as for qr_kv_attn_decode without the workspace.  A shape whose
 * workspace would exceed 16 MiB (16777216 bytes) returns QR_ESCRATCH and
 * launches nothing.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams, other host threads) race and give
 * undefined results; calls ordered on one stream are safe.  The first call on
 * a device looks up the array's device address (hipGetSymbolAddress) with
 * that device current.
 */
qr_status qr_kv_attn_decode_noalloc(const void *q_f16, int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                                    int64_t head_dim, const uint8_t *k_codes, const float *k_scales,
                                    const uint8_t *k_zeros, const uint8_t *v_codes, const float *v_scales,
                                    const uint8_t *v_zeros, const int32_t *lens, const int8_t *signs,
                                    float sm_scale, void *out_f16, void *stream);

/*
 * Workspace bytes qr_kv_attn_decode needs for this shape (0: none).  Depends
 * on the shape only, not on the device.  Host-only; launches nothing.
 */
qr_status qr_kv_attn_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t head_dim,
                                      int64_t *bytes);

/*
 * Test and diagnostic export: the exact integer sums of qr_int4_gemm without
 * the epilogue, from the same kernels.  acc is int32 [M][N] (group 0) or
 * [K/group][M][N] (one slice per group), contiguous.  Same argument rules as
 * qr_int4_gemm.
 */
qr_status qr_int4_gemm_i32(const uint8_t *a_codes, const uint8_t *w_codes,
                           int64_t M, int64_t N, int64_t K, int64_t group,
                           int32_t *acc, void *stream);

/* The same test export for qr_int8_gemm (int8 codes [M][K], [N][K]). */
qr_status qr_int8_gemm_i32(const int8_t *a_codes, const int8_t *w_codes,
                           int64_t M, int64_t N, int64_t K, int64_t group,
                           int32_t *acc, void *stream);

/* Static English text for a status code (never NULL). */
const char *qr_status_str(qr_status s);

/* Library version as 10000 * major + 100 * minor + patch. */
int qr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QR_H */
