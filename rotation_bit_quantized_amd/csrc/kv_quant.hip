// Head-wise rotated asymmetric 4-bit KV-cache quantization, head_dim 128.
//
// Method: QuaRot abstract (the KV cache in 4 bits, with the rotation applied
// to it); DuQuant page, Knowl 12 (fixed Hadamard rotation +-1/sqrt(2^n),
// per-token / per-head asymmetric quantization; step
// (gamma max - beta min)/(2^b - 1) with gamma = beta = 1, b = 4).
//
// Per (token, head) vector v of 128 fp16:
//   u = (v * signs) H_128            (unnormalised; y = u / sqrt(128))
//   lo = min(min u, 0), hi = max(max u, 0)
//   step = (hi - lo) / (15 sqrt(128)), z = rint(-lo * 15/(hi - lo)),
//   q = clamp(rint(u * 15/(hi - lo)) + z, 0, 15)
//
// The 128-point transform splits as H_128 = H_4 kron H_32 over the element
// index k = 32 s + r and the output index jj = 32 q + p (Sylvester order:
// H[k][jj] = H_4[s][q] H_32[r][p]).  For each 32-element slice s, one pass of
// v_mfma_f32_16x16x32_f16 per 16 outputs computes Y_s = H_32^T X_s (A = H_32
// with its columns permuted, +-1 in fp16, exact; B = 16 vectors of the tile
// as columns, one 16-byte load per lane; sums in fp32), and two butterfly
// stages over s in registers give the four q blocks.  8 MFMAs per 16 vectors,
// and the A operand is 8 registers, so several waves per SIMD stream tiles.
// With the permutation p = 8 (row >> 2) + 4 mt + (row & 3), lane (c16, g)
// ends with outputs 32 q + 8 g + 0..7 of vector c16; a 4 x 4 transpose of
// (lane bits 4, 5) x q with permlane swaps gives it codes 32 g .. 32 g + 31,
// one 16-byte store.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kWavesPerBlock = 4;

// max / min over the four lanes c16 + 16 g (lane bits 4 and 5)
__device__ __forceinline__ float max_g(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  v = fmaxf(u2f(a[0]), u2f(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  return fmaxf(u2f(b[0]), u2f(b[1]));
}
__device__ __forceinline__ float min_g(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  v = fminf(u2f(a[0]), u2f(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  return fminf(u2f(b[0]), u2f(b[1]));
}

// SIGNS: a sign vector is applied (its XOR masks take 16 registers, which
// the unsigned variant spends on occupancy instead).
template <bool SIGNS>
__global__ __launch_bounds__(64 * kWavesPerBlock) void kv_quant_kernel(
    const unsigned short *__restrict__ kv, int64_t T, int H, int64_t ld_kv, const int8_t *__restrict__ signs,
    uint8_t *__restrict__ codes, float *__restrict__ scales, uint8_t *__restrict__ zeros, float step_mul) {
  const int lane = threadIdx.x & 63;
  const int c16 = lane & 15;
  const int g = lane >> 4;

  // A[mt]: lane (c16, g) holds H_32[8 g + j][p] for j < 8 with
  // p = 8 (c16 >> 2) + 4 mt + (c16 & 3): +-1 as fp16, two per word.
  v8h hop[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int pcol = 8 * (c16 >> 2) + 4 * mt + (c16 & 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) hop[mt][j] = (__builtin_popcount((8 * g + j) & pcol) & 1) ? (_Float16)-1.0f : (_Float16)1.0f;
  }
  // sign masks for this lane's k-range 32 s + 8 g + 0..7 (two aligned words)
  unsigned smask[4][4];
  if constexpr (SIGNS) {
    unsigned sw[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int d = 0; d < 2; ++d) sw[s][d] = *(const unsigned *)(signs + 32 * s + 8 * g + 4 * d);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int d = 0; d < 2; ++d) sign_masks4(sw[s][d], smask[s][2 * d], smask[s][2 * d + 1]);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int d = 0; d < 4; ++d) smask[s][d] = 0u;
  }

  const int64_t nvec = T * (int64_t)H;
  const int64_t ntiles = (nvec + 15) / 16;
  const int64_t wave_id = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t wave_stride = (int64_t)gridDim.x * kWavesPerBlock;
  const unsigned magic = f2u(kRoundMagic);

  // B: this lane loads vector c16 of a tile, elements 32 s + 8 g .. + 7.
  // The loads of the wave's next two tiles are in flight while a tile is
  // computed.
  auto load_tile = [&](int64_t tile, v4u (&raw)[4]) {
    const int64_t v = tile * 16 + c16;
    const bool valid = v < nvec;
    const int64_t vt = valid ? v / H : 0;
    const int vh = valid ? (int)(v - vt * H) : 0;
    const unsigned short *src = kv + vt * ld_kv + vh * 128 + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      raw[s] = valid ? __builtin_nontemporal_load((const v4u *)(src + 32 * s)) : v4u{0u, 0u, 0u, 0u};
  };
  v4u raw[4], nxt[4];
  if (wave_id < ntiles) load_tile(wave_id, raw);
  if (wave_id + wave_stride < ntiles) load_tile(wave_id + wave_stride, nxt);

  int it = 0;
  for (int64_t tile = wave_id; tile < ntiles; tile += wave_stride, ++it) {
    set_prio_by_progress(it);   // the waves sharing a SIMD keep pace
    v4u nxt2[4];
    if (tile + 2 * wave_stride < ntiles) load_tile(tile + 2 * wave_stride, nxt2);

    // Y_s for the two 16-output halves mt of p, then H_4 over s:
    // c[q][mt][r] = output 32 q + 8 g + 4 mt + r of vector c16
    v4f c[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4u w = raw[s];
      if constexpr (SIGNS) {
        w[0] ^= smask[s][0];
        w[1] ^= smask[s][1];
        w[2] ^= smask[s][2];
        w[3] ^= smask[s][3];
      }
      const v8h b = __builtin_bit_cast(v8h, w);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        c[s][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hop[mt], b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
#pragma unroll
    for (int sb = 1; sb <= 2; sb <<= 1)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s & sb) continue;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float u = c[s][mt][r], v = c[s | sb][mt][r];
            c[s][mt][r] = u + v;
            c[s | sb][mt][r] = u - v;
          }
      }

    // Range widened to include 0, over the lane's 32 outputs, then over the
    // four lanes g of the vector.
    float mn = 0.f, mx = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mn = fminf(mn, c[q][mt][r]);
          mx = fmaxf(mx, c[q][mt][r]);
        }
    mn = min_g(mn);
    mx = max_g(mx);
    const float rng = mx - mn;
    const float inv = rng > 0.f ? 15.0f / rng : 0.f;
    const int z = rng > 0.f ? (int)rintf(-mn * inv) : 0;
    const unsigned bias = magic - (unsigned)z;  // bits(fma) - bias = rint(u*inv) + z
    // word[q]: codes of outputs 32 q + 8 g + 0..7 (element 0 in the low nibble)
    unsigned word[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unsigned acc = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        int qq = (int)(round_bits(c[q][t >> 2][t & 3], inv) - bias);
        qq = min(15, max(0, qq));
        acc |= (unsigned)qq << (4 * t);
      }
      word[q] = acc;
    }
    // 4 x 4 transpose of (lane bits 4, 5) x q: afterwards word[i] of lane g
    // holds the codes of outputs 32 g + 8 i + 0..7
    swap16u(word[0], word[1]);
    swap16u(word[2], word[3]);
    swap32u(word[0], word[2]);
    swap32u(word[1], word[3]);
    const int64_t vo = tile * 16 + c16;
    if (vo < nvec) {
      __builtin_nontemporal_store(v4u{word[0], word[1], word[2], word[3]}, (v4u *)(codes + vo * 64 + 16 * g));
      if (g == 0) {
        scales[vo] = rng * step_mul;
        zeros[vo] = (uint8_t)z;
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      raw[s] = nxt[s];
      nxt[s] = nxt2[s];
    }
  }
}

}  // namespace

namespace {
template <bool SIGNS>
hipError_t launch_kv(const void *kv, int64_t T, int64_t H, int64_t ld_kv, const int8_t *signs, uint8_t *codes,
                     float *scales, uint8_t *zeros, hipStream_t stream) {
  const int cus = device_cu_count();
  // persistent grid: as many blocks as are resident at once, each wave
  // walking its tiles with the next two in flight
  // resident blocks per CU: a constant of the kernel, queried once (a
  // function-local static is initialised exactly once, thread-safely)
  static const int per_cu = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kv_quant_kernel<SIGNS>, 64 * kWavesPerBlock, 0) != hipSuccess ||
        b < 1)
      b = 1;
    return b;
  }();
  const int64_t tiles = (T * H + 15) / 16;
  const int64_t blocks = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = (int64_t)cus * per_cu;
  const int64_t grid = blocks < cap ? blocks : cap;
  const float step_mul = (float)(1.0 / (15.0 * __builtin_sqrt(128.0)));
  kv_quant_kernel<SIGNS><<<dim3((unsigned)grid), dim3(64 * kWavesPerBlock), 0, stream>>>(
      (const unsigned short *)kv, T, (int)H, ld_kv, signs, codes, scales, zeros, step_mul);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_kv_quant(const void *kv, int64_t T, int64_t H, int64_t ld_kv, const int8_t *signs,
                           uint8_t *codes, float *scales, uint8_t *zeros, hipStream_t stream) {
  return signs != nullptr ? launch_kv<true>(kv, T, H, ld_kv, signs, codes, scales, zeros, stream)
                          : launch_kv<false>(kv, T, H, ld_kv, signs, codes, scales, zeros, stream);
}

}  // namespace qr
