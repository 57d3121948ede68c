// Internal launch interface between the C ABI (abi.hip) and the kernels.
// Arguments have been validated by the caller; these only pick a grid and
// launch on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace qr {

// Compute units of the current device.  Queried once per device and kept:
// the launch code sits on the host path of latency-bound calls.
inline int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

struct RotArgs {
  int n;          // row width
  int had_n;      // power-of-two Hadamard size
  int dense_m;    // 1 or the dense factor size
  const float *dense;
  const int8_t *signs;
};

// Rotate + quantize, any validated shape (LDS-resident row, one block per row).
hipError_t launch_rq_generic(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group,
                             uint8_t *codes, float *scales, hipStream_t stream);
// bits 4 (packed) or 6, 8 (int8 codes, one per byte)
hipError_t launch_rq_generic_bits(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group, int bits,
                                  uint8_t *codes, float *scales, hipStream_t stream);
// ... with x = fp16(silu(x) * up) formed on the fly when up != nullptr
hipError_t launch_rq_generic_full(const void *x, const void *up, int64_t rows, int64_t ld_x, const RotArgs &r,
                                  int group, int bits, uint8_t *codes, float *scales, hipStream_t stream);

// Rotate + quantize for n in {4096, 8192}, no dense factor, group 0 or 128
// (first Hadamard factor on fp16 MFMA, the rest in registers, one wave per row).
bool rq_pow2_supported(const RotArgs &r, int group);
hipError_t launch_rq_pow2(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group,
                          uint8_t *codes, float *scales, hipStream_t stream);
hipError_t launch_rq_pow2_bits(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group, int bits,
                               uint8_t *codes, float *scales, hipStream_t stream);

// Rotate + quantize for n = 64 * m with a dense m x m factor (m <= 176),
// dense factor on fp16 MFMA (hi/lo split), 64-point Hadamard in registers.
bool rq_kron_supported(const RotArgs &r, int group);
hipError_t launch_rq_kron(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group,
                          uint8_t *codes, float *scales, hipStream_t stream);

// Rotate + quantize for n = 4096 * m with a dense m x m factor (2 <= m <= 8),
// H_8 kron O on fp16 MFMA (hi/lo split), 512-point Hadamard in registers.
bool rq_kron4096_supported(const RotArgs &r, int group);
hipError_t launch_rq_kron4096(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, uint8_t *codes,
                              float *scales, hipStream_t stream);
// the same with the row formed as fp16(silu(gate) * up)
hipError_t launch_swiglu_rq_kron4096(const void *gate, const void *up, int64_t rows, int64_t ld, const RotArgs &r,
                                     uint8_t *codes, float *scales, hipStream_t stream);

// Integer GEMM.  out_i32 == false: fp16 output with ld_y; true: int32 sums.
hipError_t launch_gemm_prefill(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw,
                               int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                               bool out_i32, hipStream_t stream);
hipError_t launch_gemm_decode(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw,
                              int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                              bool out_i32, hipStream_t stream);
// The same GEMMs on int8 codes [rows][K] (the 6- and 8-bit variants).
hipError_t launch_gemm_prefill_i8(const int8_t *a, const float *sa, const int8_t *w, const float *sw,
                                  int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                                  bool out_i32, hipStream_t stream);
hipError_t launch_gemm_decode_i8(const int8_t *a, const float *sa, const int8_t *w, const float *sw,
                                 int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                                 bool out_i32, hipStream_t stream);

// Decode attention over the rotated 4-bit KV cache, head_dim 128.  The plan
// (tokens per chunk, chunks per sequence, workspace size) depends on the
// shape only.
struct AttnPlan {
  int64_t chunk;            // tokens per chunk
  int64_t splits;           // chunks per sequence
  int64_t nhg;              // groups of up to eight KV heads
  int64_t tiles;            // B * nhg * splits
  int64_t blocks;           // grid size
  int64_t workspace_bytes;
  bool gqa;                 // 4..16 query heads per KV head: one block serves them all (MFMA kernel)
};
AttnPlan attn_decode_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t T);
hipError_t launch_attn_decode(const void *q, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const uint8_t *kc,
                              const float *ks, const uint8_t *kz, const uint8_t *vc, const float *vs,
                              const uint8_t *vz, const int *lens, const int8_t *signs, float sm_scale,
                              const AttnPlan &plan, float *ws, void *out, hipStream_t stream);

// KV-cache quantizer, head_dim 128.
hipError_t launch_kv_quant(const void *kv, int64_t T, int64_t H, int64_t ld_kv, const int8_t *signs,
                           uint8_t *codes, float *scales, uint8_t *zeros, hipStream_t stream);

}  // namespace qr
