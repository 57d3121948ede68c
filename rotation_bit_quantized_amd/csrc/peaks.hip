// Measured-peak probes (include/qr_peaks.h): the attainable HBM copy rate and
// the attainable dense MFMA rate of this part, the second denominators next to
// the datasheet peaks when the hot-path kernels are put against a roofline.
#include "../../include/qr_peaks.h"
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

// Streaming copy: each lane moves 16-byte pieces with eight loads in flight
// before its stores, nontemporal both ways, grid-strided over a persistent
// grid of one 1024-thread block per CU (the fastest of the block shapes and
// depths tried: 256 to 1024 threads, one to four blocks per CU, four or
// eight loads in flight).
__global__ __launch_bounds__(1024) void peak_copy_kernel(const v4u *__restrict__ src, v4u *__restrict__ dst,
                                                          int64_t pieces) {
  constexpr int kDepth = 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (kDepth - 1) * stride < pieces; i += kDepth * stride) {
    v4u v[kDepth];
#pragma unroll
    for (int j = 0; j < kDepth; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < kDepth; ++j) __builtin_nontemporal_store(v[j], dst + i + j * stride);
  }
  for (; i < pieces; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Back-to-back MFMAs on four independent accumulators per wave (no memory
// traffic in the loop); the sums are stored so that nothing is eliminated.
// KIND 0: v_mfma_i32_32x32x32_i8 (65536 ops each); KIND 1:
// v_mfma_f32_16x16x32_f16 (16384 flops each); KIND 2: v_mfma_f32_32x32x16_f16
// (32768 flops each); KIND 3: v_mfma_i32_16x16x64_i8 (32768 ops each).  The
// 16x16 shapes and the 32x32 ones bound the kernels built on them.
template <int KIND>
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, int *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if constexpr (KIND == 0) {
    const v4i a = {lane, lane + 1, lane + 2, lane + 3};
    const v4i b = {iters, lane, 3, 5};
    v16i c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[wave * 64 + lane] = s;
  } else if constexpr (KIND == 1) {
    v8h a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = (_Float16)(0.001f * (lane + j));
      b[j] = (_Float16)(0.002f * (iters - j));
    }
    v4f c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[wave * 64 + lane] = (int)f2u(s);
  } else if constexpr (KIND == 3) {
    const v4i a = {lane, lane + 1, lane + 2, lane + 3};
    const v4i b = {iters, lane, 3, 5};
    v4i c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[wave * 64 + lane] = s;
  } else {
    v8h a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = (_Float16)(0.001f * (lane + j));
      b[j] = (_Float16)(0.002f * (iters - j));
    }
    v16f c0{}, c1{}, c2{}, c3{};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[wave * 64 + lane] = (int)f2u(s);
  }
}

// Back-to-back v_mfma_i32_32x32x32_i8 on operands taken from the caller's
// packed int4 codes, widened once to the GEMM's high-nibble int8 form
// (16 q): each lane loads eight 16-byte A pieces and eight W pieces (piece
// (64 wave + lane) * 8 + f, wrapping over each buffer), then every round
// issues 32 MFMAs over four accumulator chains in the GEMM's order
// (consecutive MFMAs share the A operand and change the W one).  The chip's
// clock under dense MFMA work depends on how many operand bits toggle, so on
// the codes of a real workload this loop gives the rate the matrix cores
// attain for that data, below the constant-operand loop above.
__global__ __launch_bounds__(256) void peak_mfma_codes_kernel(const v4u *__restrict__ a, int64_t a_pieces,
                                                               const v4u *__restrict__ w, int64_t w_pieces,
                                                               int iters, int *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  v4i opa[8][2], opw[8][2];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int64_t piece = (wave * 64 + lane) * 8 + f;
    widen_hi_nibble(a[piece % a_pieces], opa[f][0], opa[f][1]);
    widen_hi_nibble(w[piece % w_pieces], opw[f][0], opw[f][1]);
  }
  v16i c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          c[2 * ks + j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(opa[f][ks], opw[(f + 4 * j) & 7][ks], c[2 * ks + j],
                                                                0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[q][r];
  out[wave * 64 + lane] = s;
}

}  // namespace
}  // namespace qr

extern "C" {

qr_status qr_peak_copy(const void *src, void *dst, int64_t bytes, void *stream) {
  if (bytes < 0) return QR_EINVAL;
  if (bytes % 16 != 0) return QR_ESHAPE;
  if (bytes == 0) return QR_OK;
  if (src == nullptr || dst == nullptr) return QR_EINVAL;
  if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return QR_EALIGN;
  const int64_t pieces = bytes / 16;
  const int64_t want = (int64_t)qr::device_cu_count();
  const int64_t need = (pieces + 1023) / 1024;
  const int64_t grid = need < want ? need : want;
  qr::peak_copy_kernel<<<dim3((unsigned)grid), dim3(1024), 0, (hipStream_t)stream>>>((const qr::v4u *)src,
                                                                                       (qr::v4u *)dst, pieces);
  return hipGetLastError() == hipSuccess ? QR_OK : QR_EDEVICE;
}

int64_t qr_peak_mfma_waves(void) { return (int64_t)qr::device_cu_count() * 8; }

qr_status qr_peak_mfma(int64_t kind, int64_t iters, int32_t *out, void *stream) {
  if (kind < 0 || kind > 3) return QR_EINVAL;
  if (iters <= 0 || iters > ((int64_t)1 << 24)) return QR_ESHAPE;
  if (out == nullptr) return QR_EINVAL;
  if ((uintptr_t)out & 3) return QR_EALIGN;
  const int64_t blocks = (int64_t)qr::device_cu_count() * 2;   // 8 waves per CU, two per SIMD
  if (kind == 0)
    qr::peak_mfma_kernel<0><<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>((int)iters, out);
  else if (kind == 1)
    qr::peak_mfma_kernel<1><<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>((int)iters, out);
  else if (kind == 2)
    qr::peak_mfma_kernel<2><<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>((int)iters, out);
  else
    qr::peak_mfma_kernel<3><<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>((int)iters, out);
  return hipGetLastError() == hipSuccess ? QR_OK : QR_EDEVICE;
}

qr_status qr_peak_mfma_codes(const uint8_t *a, int64_t a_bytes, const uint8_t *w, int64_t w_bytes, int64_t iters,
                             int32_t *out, void *stream) {
  if (a == nullptr || w == nullptr || out == nullptr) return QR_EINVAL;
  if (a_bytes < 16 || w_bytes < 16 || a_bytes % 16 != 0 || w_bytes % 16 != 0) return QR_ESHAPE;
  if (iters <= 0 || iters > ((int64_t)1 << 24)) return QR_ESHAPE;
  if (((uintptr_t)a & 15) || ((uintptr_t)w & 15) || ((uintptr_t)out & 3)) return QR_EALIGN;
  const int64_t blocks = (int64_t)qr::device_cu_count() * 2;   // 8 waves per CU, two per SIMD
  qr::peak_mfma_codes_kernel<<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>(
      (const qr::v4u *)a, a_bytes / 16, (const qr::v4u *)w, w_bytes / 16, (int)iters, out);
  return hipGetLastError() == hipSuccess ? QR_OK : QR_EDEVICE;
}

}  // extern "C"
