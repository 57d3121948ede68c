// Rotate + symmetric 4-bit RTN + pack for Kronecker rotations
//   R = (H_64 / 8) kron O,  n = 64 m,  m <= 176, m % 4 == 0, no signs,
// e.g. the 11008-wide down_proj input of LLaMA-2-7B (m = 172).
//
// Method: y = x R per token row, s = max|y| / 7, q = rint(y / s) packed two
// per byte (QuaRot summary, "Key points": RTN on the fly).  A random
// orthogonal factor for widths that are not a power of two: QuIP summary,
// abstract (random orthogonal multiplication) and the QuIP# quote on the
// same page (two-factor Kronecker construction).
//
// With x viewed as X[i][a] (i < 64 rows, a < m fastest), y viewed as Y[j][b]
// is Y = H_64^T X O / 8: a dense m x m product per token, then a 64-point
// Walsh-Hadamard transform over the row index.
//
// Design (one wave per token row, four waves per block, persistent grid):
//  * The dense product runs on v_mfma_f32_32x32x16_f16 with A = X (the fp16
//    input, exact) and B = O split into an fp16 high part and an fp16 low
//    part (O - hi); both products accumulate into the same fp32
//    accumulators, which keeps the error near 2^-22 relative (one fp16 pass
//    alone would round O to 2^-11 and move codes that sit near a rounding
//    boundary).  K (a) is padded to 16 k-steps of 16, N (b) to 6 N-tiles
//    of 32 with the column map b = 6 * lane + nt, so each lane ends up with
//    six consecutive outputs of every row j.
//  * O's hi/lo B-fragments are laid out once per block in LDS (KS x 6 x 2
//    KB, 132 KB for m = 172) straight from the fp32 factor.
//  * The 64-point transform over i: the accumulator rows carry i bits
//    {0,1,3,4} in the register index and i5 in the M-tile, i2 in lane bit 5;
//    butterflies in registers, then one v_permlane32_swap brings i2 into a
//    register bit for the last stage.
//  * Codes: each lane writes three bytes (six codes) per output row j.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxKS = 11;      // k-steps of 16: m <= 176
constexpr int kNT = 6;          // N-tiles of 32 columns: b < 192

__device__ __forceinline__ void swap32(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane32_swap(f2u(a), f2u(b), false, false);
  a = u2f(r[0]);
  b = u2f(r[1]);
}

__global__ __launch_bounds__(64 * kWaves, 1) void rq_kron_kernel(
    const unsigned short *__restrict__ x, int64_t rows, int64_t ld_x, int m, const float *__restrict__ dense,
    uint8_t *__restrict__ codes, float *__restrict__ scales, float scale_mul) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // [ks][nt][hi/lo][64 lanes][16 B]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int KS = (m + 15) / 16;
  const int n = 64 * m;

  // ---- B-fragments of O (hi and lo fp16 parts), once per block
  for (int f = tid; f < KS * kNT * 64; f += 64 * kWaves) {
    const int ks = f / (kNT * 64);
    const int nt = (f / 64) % kNT;
    const int l = f % 64;
    const int b = 6 * (l & 31) + nt;
    v8h hi, lo;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int a = 16 * ks + 8 * (l >> 5) + s;
      const float o = (a < m && b < m) ? dense[a * m + b] : 0.f;
      const _Float16 h = (_Float16)o;
      hi[s] = h;
      lo[s] = (_Float16)(o - (float)h);
    }
    *(v8h *)(smem + (((ks * kNT + nt) * 2 + 0) * 64 + l) * 16) = hi;
    *(v8h *)(smem + (((ks * kNT + nt) * 2 + 1) * 64 + l) * 16) = lo;
  }
  __syncthreads();

  const int64_t wave_id = (int64_t)blockIdx.x * kWaves + (tid >> 6);
  const int64_t wave_stride = (int64_t)gridDim.x * kWaves;
  const int ri = lane & 31;          // row of A (i within an M-tile), column of C
  const int h = lane >> 5;           // k-half

  for (int64_t row = wave_id; row < rows; row += wave_stride) {
    const unsigned short *xr = x + row * ld_x;
    v16f c[2][kNT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) c[mt][nt] = v16f{};

    // ---- dense factor on MFMA: C[i][b] += X[i][a] (O_hi + O_lo)[a][b]
    v2u nxt[2][2];
    auto load_a = [&](int ks, v2u (&dst)[2][2]) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const unsigned short *p = xr + (32 * mt + ri) * m + 16 * ks + 8 * h;
        const int a0 = 16 * ks + 8 * h;
        dst[mt][0] = a0 < m ? *(const v2u *)p : v2u{0u, 0u};
        dst[mt][1] = a0 + 4 < m ? *(const v2u *)(p + 4) : v2u{0u, 0u};
      }
    };
    load_a(0, nxt);
    for (int ks = 0; ks < KS; ++ks) {
      v8h a[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        v4u w = {nxt[mt][0][0], nxt[mt][0][1], nxt[mt][1][0], nxt[mt][1][1]};
        a[mt] = __builtin_bit_cast(v8h, w);
      }
      if (ks + 1 < KS) load_a(ks + 1, nxt);
      const uint8_t *fb = smem + (ks * kNT * 2 * 64 + lane) * 16;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const v8h bhi = *(const v8h *)(fb + (nt * 2 + 0) * 64 * 16);
        const v8h blo = *(const v8h *)(fb + (nt * 2 + 1) * 64 * 16);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) c[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mt], bhi, c[mt][nt], 0, 0, 0);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) c[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mt], blo, c[mt][nt], 0, 0, 0);
      }
    }

    // ---- 64-point Walsh-Hadamard over i.  c[mt][nt][r] holds row
    // i = 32 mt + 8 (r >> 2) + 4 h + (r & 3): register bits r0, r1, r2, r3
    // carry i0, i1, i3, i4; mt carries i5; lane bit 5 carries i2.
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (r & (1 << rb)) continue;
            const float u = c[mt][nt][r], v = c[mt][nt][r | (1 << rb)];
            c[mt][nt][r] = u + v;
            c[mt][nt][r | (1 << rb)] = u - v;
          }
#pragma unroll
      for (int r = 0; r < 16; ++r) {   // i5
        const float u = c[0][nt][r], v = c[1][nt][r];
        c[0][nt][r] = u + v;
        c[1][nt][r] = u - v;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {   // i2: lane bit 5 <-> the M-tile bit, then butterfly
        float u = c[0][nt][r], v = c[1][nt][r];
        swap32(u, v);
        c[0][nt][r] = u + v;
        c[1][nt][r] = u - v;
      }
    }
    // Now c[q][nt][r] is output row j = (r & 3) | q << 2 | (r >> 2) << 3 | h << 5,
    // column b = 6 ri + nt (zero for b >= m: padded O columns are zero).

    float mx = 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(c[q][nt][r]));
    mx = wave_max(mx);
    if (lane == 0) scales[row] = mx * scale_mul;
    const float inv = mx > 0.f ? 7.0f / mx : 0.f;

    uint8_t *cr = codes + row * (int64_t)(n / 2);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = (r & 3) | (q << 2) | ((r >> 2) << 3) | (h << 5);
        uint8_t *dst = cr + (j * m + 6 * ri) / 2;
#pragma unroll
        for (int pr = 0; pr < 3; ++pr) {
          if (6 * ri + 2 * pr < m) {
            const unsigned b0 = round_bits(c[q][2 * pr][r], inv);
            const unsigned b1 = round_bits(c[q][2 * pr + 1][r], inv);
            dst[pr] = (uint8_t)((b0 & 0xFu) | ((b1 & 0xFu) << 4));
          }
        }
      }
  }
}

}  // namespace

bool rq_kron_supported(const RotArgs &r, int group) {
  return r.dense_m > 1 && r.had_n == 64 && r.dense_m <= 16 * kMaxKS && r.dense_m % 4 == 0 &&
         r.signs == nullptr && group == 0;
}

hipError_t launch_rq_kron(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group,
                          uint8_t *codes, float *scales, hipStream_t stream) {
  (void)group;
  const int KS = (r.dense_m + 15) / 16;
  const size_t lds = (size_t)KS * kNT * 2 * 64 * 16;
  hipError_t e = hipFuncSetAttribute((const void *)rq_kron_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t blocks = (rows + kWaves - 1) / kWaves;
  const int64_t grid = blocks < cus ? blocks : cus;
  const float scale_mul = (float)(1.0 / (7.0 * 8.0));   // 1/(7 sqrt(64))
  rq_kron_kernel<<<dim3((unsigned)grid), dim3(64 * kWaves), lds, stream>>>(
      (const unsigned short *)x, rows, ld_x, r.dense_m, r.dense, codes, scales, scale_mul);
  return hipGetLastError();
}

}  // namespace qr
