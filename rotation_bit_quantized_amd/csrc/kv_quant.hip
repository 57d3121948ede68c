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
// The whole 128-point transform is one pass of v_mfma_f32_16x16x32_f16
// (input fp16 is exact, H entries +-1 are exact, sums in fp32), computed
// transposed: A = H_128 with its rows (the output index) permuted, held in
// registers; B = 16 vectors of the tile as columns (one 16-byte load per lane
// per k-step); C[output][vector].  With the permutation, lane (c16, g) holds
// outputs 32 g .. 32 g + 31 of vector c16: the range reduction needs two
// cross-lane steps, and the 32 codes leave as one 16-byte store.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kWavesPerBlock = 4;

// The A operands (permuted H_128) of every lane, computed at compile time:
// entry [mt][s][lane] is the v8h of M-tile mt, k-step s for lane (c16, g):
// slot j holds H[32 s + 8 g + j][32 (c16 >> 2) + 4 mt + (c16 & 3)] as fp16
// +-1 (0x3C00 / 0xBC00), two per 32-bit word.  Loading it (32 KB, coalesced,
// cache resident after the first waves) replaces ~1500 VALU ops per wave of
// operand construction, which matter when a wave has only a few tiles.
struct HopTable {
  unsigned w[8][4][64][4];
};
constexpr HopTable make_hop_table() {
  HopTable t{};
  for (int mt = 0; mt < 8; ++mt)
    for (int s = 0; s < 4; ++s)
      for (int lane = 0; lane < 64; ++lane) {
        const int c16 = lane & 15, g = lane >> 4;
        const int jj = 32 * (c16 >> 2) + 4 * mt + (c16 & 3);
        for (int d = 0; d < 4; ++d) {
          unsigned word = 0;
          for (int half = 0; half < 2; ++half) {
            const int k = 32 * s + 8 * g + 2 * d + half;
            int bits = k & jj, par = 0;
            while (bits) {
              par ^= bits & 1;
              bits >>= 1;
            }
            word |= (par ? 0xBC00u : 0x3C00u) << (16 * half);
          }
          t.w[mt][s][lane][d] = word;
        }
      }
  return t;
}
__device__ constexpr HopTable kHop = make_hop_table();

__global__ __launch_bounds__(64 * kWavesPerBlock) void kv_quant_kernel(
    const unsigned short *__restrict__ kv, int64_t T, int H, int64_t ld_kv, const int8_t *__restrict__ signs,
    uint8_t *__restrict__ codes, float *__restrict__ scales, uint8_t *__restrict__ zeros, float step_mul) {
  const int lane = threadIdx.x & 63;
  const int c16 = lane & 15;
  const int g = lane >> 4;

  // A[mt][s]: this lane's row c16 of M-tile mt is output
  // jj = 32 (c16 >> 2) + 4 mt + (c16 & 3); slot j holds H[k][jj] for
  // k = 32 s + 8 g + j.  (C row 4 g' + r of M-tile mt is then output
  // 32 g' + 4 mt + r.)
  v8h hop[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s) hop[mt][s] = __builtin_bit_cast(v8h, *(const v4u *)kHop.w[mt][s][lane]);
  // sign masks for this lane's k-range 32 s + 8 g + 0..7 (two aligned words)
  unsigned smask[4][4];
  if (signs != nullptr) {
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
  // The next tile's loads are issued before this tile is computed, so a
  // wave always has a tile in flight.
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
  v4u raw[4];
  if (wave_id < ntiles) load_tile(wave_id, raw);

  for (int64_t tile = wave_id; tile < ntiles; tile += wave_stride) {
    v4u nxt[4];
    if (tile + wave_stride < ntiles) load_tile(tile + wave_stride, nxt);

    v4f c[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) c[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4u w = raw[s];
      w[0] ^= smask[s][0];
      w[1] ^= smask[s][1];
      w[2] ^= smask[s][2];
      w[3] ^= smask[s][3];
      const v8h b = __builtin_bit_cast(v8h, w);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) c[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hop[mt][s], b, c[mt], 0, 0, 0);
    }

    // c[mt][r] = output 32 g + 4 mt + r of vector c16.  Range widened to
    // include 0, over the lane's 32 outputs, then over the 4 lanes g.
    float mn = 0.f, mx = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mn = fminf(mn, c[mt][r]);
        mx = fmaxf(mx, c[mt][r]);
      }
    mn = fminf(mn, __shfl_xor(mn, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mn = fminf(mn, __shfl_xor(mn, 32, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float rng = mx - mn;
    const float inv = rng > 0.f ? 15.0f / rng : 0.f;
    const int z = rng > 0.f ? (int)rintf(-mn * inv) : 0;
    const unsigned bias = magic - (unsigned)z;  // bits(fma) - bias = rint(u*inv) + z
    unsigned word[4];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      unsigned acc = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {   // output 32 g + 8 wd + t = mt 2 wd + t/4, r t%4
        int q = (int)(round_bits(c[2 * wd + (t >> 2)][t & 3], inv) - bias);
        q = min(15, max(0, q));
        acc |= (unsigned)q << (4 * t);
      }
      word[wd] = acc;
    }
    const int64_t vo = tile * 16 + c16;
    if (vo < nvec) {
      *(v4u *)(codes + vo * 64 + 16 * g) = v4u{word[0], word[1], word[2], word[3]};
      if (g == 0) {
        scales[vo] = rng * step_mul;
        zeros[vo] = (uint8_t)z;
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) raw[s] = nxt[s];
  }
}

}  // namespace

hipError_t launch_kv_quant(const void *kv, int64_t T, int64_t H, int64_t ld_kv, const int8_t *signs,
                           uint8_t *codes, float *scales, uint8_t *zeros, hipStream_t stream) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  int cus = 256;
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  // persistent grid: as many blocks as are resident at once, each wave
  // walking its tiles with the next one always in flight
  static int per_cu = 0;
  if (per_cu == 0) {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kv_quant_kernel, 64 * kWavesPerBlock, 0) != hipSuccess ||
        b < 1)
      b = 1;
    per_cu = b;
  }
  const int64_t tiles = (T * H + 15) / 16;
  const int64_t blocks = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = (int64_t)cus * per_cu;
  const int64_t grid = blocks < cap ? blocks : cap;
  const float step_mul = (float)(1.0 / (15.0 * __builtin_sqrt(128.0)));
  kv_quant_kernel<<<dim3((unsigned)grid), dim3(64 * kWavesPerBlock), 0, stream>>>(
      (const unsigned short *)kv, T, (int)H, ld_kv, signs, codes, scales, zeros, step_mul);
  return hipGetLastError();
}

}  // namespace qr
