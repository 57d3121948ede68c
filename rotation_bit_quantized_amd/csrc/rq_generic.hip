// Rotate + symmetric 4-bit RTN + pack, for any row width the ABI accepts.
//
// One workgroup owns one token row at a time (grid-stride over rows).  The
// row is staged in LDS as fp32:
//   0. (fused call) x = fp16(silu(gate) * up): the feed-forward activation
//      before down_proj, formed here instead of being read
//   1. x * signs                       (the random diagonal D, input side)
//   2. dense factor: t[i*m + b] = sum_a x[i*m + a] O[a][b]   (if m > 1)
//   3. Walsh-Hadamard butterflies over the Hadamard index i, in place
//   4. max |.| per row or per group, s = max / (qmax sqrt(p)), codes
//      rint(v * qmax / max): qmax = 7 packed two per byte, or the 6- and
//      8-bit variants qmax = 31, 127 as one int8 per byte (QuaRot abstract:
//      lossless 6- and 8-bit RTN).
// This is the reference-shape path of the library: small or unusual widths
// (n = 2 .. 32768, any power-of-two Hadamard size, dense factors up to 256;
// a factor of size m <= 16 is applied in place, one i-group per thread in
// registers, so that rows up to 32768 fit in LDS as one fp32 copy).
// The wide power-of-two and the 64 x m Kronecker shapes have MFMA kernels.
//
// Method: QuaRot summary (Elamur Research), "Key points" (RTN on the fly,
// group 128); Hadamard normalisation +-1/sqrt(2^n): DuQuant page, Knowl 12;
// Kronecker construction: QuIP summary, QuIP# quote.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kBlock = 256;
constexpr int kInPlaceM = 16;   // dense factors up to this size are applied in place

__global__ __launch_bounds__(kBlock) void rq_generic_kernel(
    const unsigned short *__restrict__ x, const unsigned short *__restrict__ up, int64_t rows, int64_t ld_x, int n,
    int had_n, int dense_m,
    const float *__restrict__ dense, const int8_t *__restrict__ signs, int group, int qmax,
    uint8_t *__restrict__ codes, float *__restrict__ scales, float scale_mul) {
  extern __shared__ float smem[];
  float *buf = smem;
  const bool in_place = dense_m <= kInPlaceM;
  float *tmp = smem + n;   // (second row copy: large dense factors only)
  const int g = group ? group : n;
  const int ngroups = n / g;
  float *red = smem + (dense_m > 1 && !in_place ? 2 * n : n);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int kWaves = kBlock / 64;

  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const unsigned short *xr = x + row * ld_x;
    const unsigned short *ur = up != nullptr ? up + row * ld_x : nullptr;
    for (int k = tid; k < n; k += kBlock) {
      float v = half_bits_to_float(xr[k]);
      if (ur != nullptr) {   // x = fp16(silu(gate) * up)
        const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * v);
        v = (float)(_Float16)(v * __builtin_amdgcn_rcpf(1.0f + e) * half_bits_to_float(ur[k]));
      }
      if (signs != nullptr && signs[k] < 0) v = -v;
      buf[k] = v;
    }
    __syncthreads();

    float *cur = buf;
    if (dense_m > 1 && in_place) {
      // one i-group (dense_m consecutive values) per thread, in registers
      for (int i = tid; i < n / dense_m; i += kBlock) {
        float xi[kInPlaceM], yi[kInPlaceM];
#pragma unroll
        for (int a = 0; a < kInPlaceM; ++a) xi[a] = a < dense_m ? buf[i * dense_m + a] : 0.f;
#pragma unroll
        for (int b = 0; b < kInPlaceM; ++b) {
          float acc = 0.f;
#pragma unroll
          for (int a = 0; a < kInPlaceM; ++a)
            if (a < dense_m && b < dense_m) acc = __builtin_fmaf(xi[a], dense[a * dense_m + b], acc);
          yi[b] = acc;
        }
#pragma unroll
        for (int b = 0; b < kInPlaceM; ++b)
          if (b < dense_m) buf[i * dense_m + b] = yi[b];
      }
      __syncthreads();
    } else if (dense_m > 1) {
      for (int idx = tid; idx < n; idx += kBlock) {
        const int i = idx / dense_m;
        const int b = idx - i * dense_m;
        const float *xi = buf + i * dense_m;
        float acc = 0.f;
        for (int a = 0; a < dense_m; ++a) acc = __builtin_fmaf(xi[a], dense[a * dense_m + b], acc);
        tmp[idx] = acc;
      }
      __syncthreads();
      cur = tmp;
    }

    // Butterflies over the Hadamard index i (stride dense_m in memory).
    for (int h = 1; h < had_n; h <<= 1) {
      for (int q = tid; q < n / 2; q += kBlock) {
        const int j = q / dense_m;
        const int b = q - j * dense_m;
        const int i = (j / h) * 2 * h + (j % h);
        float *p0 = cur + i * dense_m + b;
        float *p1 = p0 + h * dense_m;
        const float u = *p0, v = *p1;
        *p0 = u + v;
        *p1 = u - v;
      }
      __syncthreads();
    }

    // Max |y| of every group (or of the row): one wave per group.
    for (int s = wave; s < ngroups; s += kWaves) {
      float m = 0.f;
      for (int k = lane; k < g; k += 64) m = fmaxf(m, fabsf(cur[s * g + k]));
      m = wave_max(m);
      if (lane == 0) red[s] = m;
    }
    __syncthreads();

    if (qmax > 7) {
      int8_t *cr8 = (int8_t *)codes + row * (int64_t)n;
      const float qm = (float)qmax;
      for (int k = tid; k < n; k += kBlock) {
        const float m = red[k / g];
        const int q = (int)rintf(cur[k] * (m > 0.f ? qm / m : 0.f));
        cr8[k] = (int8_t)min(qmax, max(-qmax - 1, q));
      }
    }
    uint8_t *cr = codes + row * (int64_t)(n / 2);
    for (int c = tid; c < (qmax > 7 ? 0 : n / 2); c += kBlock) {
      const int k = 2 * c;
      const float m0 = red[k / g];
      const float m1 = red[(k + 1) / g];
      const float i0 = m0 > 0.f ? 7.0f / m0 : 0.f;
      const float i1 = m1 > 0.f ? 7.0f / m1 : 0.f;
      int q0 = (int)rintf(cur[k] * i0);
      int q1 = (int)rintf(cur[k + 1] * i1);
      q0 = min(7, max(-8, q0));
      q1 = min(7, max(-8, q1));
      cr[c] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
    }
    for (int s = tid; s < ngroups; s += kBlock) scales[row * ngroups + s] = red[s] * scale_mul;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_rq_generic(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group,
                             uint8_t *codes, float *scales, hipStream_t stream) {
  return launch_rq_generic_bits(x, rows, ld_x, r, group, 4, codes, scales, stream);
}

hipError_t launch_rq_generic_bits(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group, int bits,
                                  uint8_t *codes, float *scales, hipStream_t stream) {
  return launch_rq_generic_full(x, nullptr, rows, ld_x, r, group, bits, codes, scales, stream);
}

hipError_t launch_rq_generic_full(const void *x, const void *up, int64_t rows, int64_t ld_x, const RotArgs &r,
                                  int group, int bits, uint8_t *codes, float *scales, hipStream_t stream) {
  const int qmax = (1 << (bits - 1)) - 1;
  const int g = group ? group : r.n;
  const bool two_copies = r.dense_m > kInPlaceM;
  const size_t lds = sizeof(float) * ((two_copies ? 2 * (size_t)r.n : (size_t)r.n) + (size_t)(r.n / g));
  if (lds > 64 * 1024) {
    // the kernel's dynamic LDS limit, raised once per device to the largest
    // size asked for so far (not on every launch)
    constexpr int kMaxDevices = 64;
    static std::atomic<int> raised[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices || raised[dev].load(std::memory_order_relaxed) < (int)lds) {
      e = hipFuncSetAttribute((const void *)rq_generic_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      if (dev >= 0 && dev < kMaxDevices) {
        int cur = raised[dev].load(std::memory_order_relaxed);
        while (cur < (int)lds && !raised[dev].compare_exchange_weak(cur, (int)lds)) {
        }
      }
    }
  }
  const int64_t grid = rows < 4096 ? rows : 4096;
  const float scale_mul = (float)(1.0 / ((double)qmax * __builtin_sqrt((double)r.had_n)));
  rq_generic_kernel<<<dim3((unsigned)grid), dim3(kBlock), lds, stream>>>(
      (const unsigned short *)x, (const unsigned short *)up, rows, ld_x, r.n, r.had_n, r.dense_m, r.dense, r.signs,
      group, qmax, codes,
      scales, scale_mul);
  return hipGetLastError();
}

}  // namespace qr
