// 4-bit integer GEMM for decode shapes (M <= 64 tokens): memory-bound, the
// weight codes are streamed from HBM exactly once.
//
// Method: as the prefill kernel (QuaRot abstract: all matrix
// multiplications in 4 bits; dequantizing epilogue per output channel or
// per K-group of 128).  Decoding is the memory-bound phase where the 4-bit
// weights cut the bytes moved (QuaRot summary, "Key points": decode peak
// memory; QuaRot press article: decoding is usually memory-bound).
//
// One workgroup (16 waves) owns 16 output channels and all M <= 64 tokens.
// Wave w handles the K-units w, w + 16, ... (a unit is one 64-byte piece of
// each row per-channel, or one K-group); it loads up to four pieces at once
// (16 weight rows and 64 token rows, 16 bytes per lane each) straight into
// registers, so that one memory latency covers them, widens them to 16*q
// int8 (see gemm_prefill.hip) and issues v_mfma_i32_16x16x64_i8 with
// A = weight rows, B = token rows, giving C[channel][token].  The 16 per-wave partials are reduced through LDS in
// int32 (per-channel, exact) or fp32 (group-wise, after scaling).
//
// 8-bit codes (CB = 8; the 6- and 8-bit RTN variants, QuaRot abstract): a
// lane's 16 codes of a 64-code step are 16 bytes, used as the MFMA operand
// as they are (no widening, no 1/256).
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kWaves = 16;
constexpr int kNT = 16;  // output channels per workgroup

template <bool GROUPED, bool OUT_I32, int CB = 4>
__global__ __launch_bounds__(64 * kWaves) void gemm_decode_kernel(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ W,
    const float *__restrict__ sw, int M, int N, int K, int group, void *__restrict__ out, int64_t ld_y) {
  // partial sums: [wave][frag 0..3][lane][4], int32 or fp32 bits
  __shared__ int red[kWaves][4][64][4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * kNT;
  static_assert(CB == 4 || CB == 8, "code width");
  constexpr int SHIFT = CB == 4 ? 8 : 0;           // widened 4-bit products carry 16 * 16
  constexpr float UNSCALE = CB == 4 ? 1.0f / 256.0f : 1.0f;
  // A piece is 64 bytes of a row: 128 4-bit or 64 8-bit codes, one 16-byte
  // load per lane (lane >> 4 picks the quarter) and KS MFMA k-steps of 64.
  constexpr int PIECE_CODES = 64 * 8 / CB;
  constexpr int KS = CB == 4 ? 2 : 1;
  constexpr int BATCH = GROUPED ? 2 : 4;            // pieces loaded together per wave (128 registers at most)
  const int64_t kbytes = (int64_t)K * CB / 8;
  const int ppu = GROUPED ? group / PIECE_CODES : 1;   // pieces per unit (a unit: one K-group, or one piece)
  const int units = K / PIECE_CODES / ppu;
  const int G = GROUPED ? K / group : 1;

  const int wrow = n0 + (lane & 15);                 // weight row (output channel) of this lane
  const int kofs = (lane >> 4) * 16;                 // byte offset of this lane's quarter of a piece
  const bool wvalid = wrow < N;
  const uint8_t *wp = W + (int64_t)(wvalid ? wrow : 0) * kbytes + kofs;
  const uint8_t *ap[4];
  bool avalid[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int t = f * 16 + (lane & 15);
    avalid[f] = t < M;
    ap[f] = A + (int64_t)(avalid[f] ? t : 0) * kbytes + kofs;
  }

  v4i acc[4] = {v4i{}, v4i{}, v4i{}, v4i{}};
  v4f facc[4] = {v4f{}, v4f{}, v4f{}, v4f{}};
  v4i uacc[4] = {v4i{}, v4i{}, v4i{}, v4i{}};

  // This wave's pieces: units u = wave, wave + kWaves, ...; piece j of unit
  // u is global piece u * ppu + j; flat index i = (unit ordinal) * ppu + j.
  const int my_units = units > wave ? (units - wave + kWaves - 1) / kWaves : 0;
  const int my_pieces = my_units * ppu;
  for (int i0 = 0; i0 < my_pieces; i0 += BATCH) {
    v4u wv[BATCH], av[BATCH][4];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {   // all loads of the batch first: one memory latency
      const int i = i0 + b;
      const bool ok = i < my_pieces;
      const int64_t off = ok ? ((int64_t)(wave + kWaves * (i / ppu)) * ppu + i % ppu) * 64 : 0;
      wv[b] = ok && wvalid ? __builtin_nontemporal_load((const v4u *)(wp + off)) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
      for (int f = 0; f < 4; ++f) av[b][f] = ok && avalid[f] ? *(const v4u *)(ap[f] + off) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = i0 + b;
      if (i >= my_pieces) break;
      v4i wop[KS], aop[4][KS];
      if constexpr (CB == 4) {
        widen_hi_nibble(wv[b], wop[0], wop[1]);
#pragma unroll
        for (int f = 0; f < 4; ++f) widen_hi_nibble(av[b][f], aop[f][0], aop[f][1]);
      } else {
        wop[0] = __builtin_bit_cast(v4i, wv[b]);
#pragma unroll
        for (int f = 0; f < 4; ++f) aop[f][0] = __builtin_bit_cast(v4i, av[b][f]);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if (GROUPED)
            uacc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop[ks], aop[f][ks], uacc[f], 0, 0, 0);
          else
            acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop[ks], aop[f][ks], acc[f], 0, 0, 0);
        }
      if constexpr (GROUPED) {
        if (i % ppu == ppu - 1) {   // unit (K-group) u complete
          const int u = wave + kWaves * (i / ppu);
          // this lane holds C[channel 4*(lane/16)+r][token f*16 + lane%16]
          if constexpr (OUT_I32) {
            int32_t *o = (int32_t *)out + (int64_t)u * M * N;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
              const int t = f * 16 + (lane & 15);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int ch = n0 + 4 * (lane >> 4) + r;
                if (t < M && ch < N) o[(int64_t)t * N + ch] = uacc[f][r] >> SHIFT;
              }
            }
          } else {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
              const int t = f * 16 + (lane & 15);
              const float sav = t < M ? sa[(int64_t)t * G + u] * UNSCALE : 0.f;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int ch = n0 + 4 * (lane >> 4) + r;
                const float swv = ch < N ? sw[(int64_t)ch * G + u] : 0.f;
                facc[f][r] = __builtin_fmaf((float)uacc[f][r], sav * swv, facc[f][r]);
              }
            }
          }
#pragma unroll
          for (int f = 0; f < 4; ++f) uacc[f] = v4i{};
        }
      }
    }
  }

  if constexpr (GROUPED && OUT_I32) return;

#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][f][lane][r] = GROUPED ? (int)f2u(facc[f][r]) : acc[f][r];
  __syncthreads();

  // 1024 outputs (4 frags x 64 lanes x 4 regs), one per thread.
  const int f = tid >> 8;
  const int l = (tid >> 2) & 63;
  const int r = tid & 3;
  const int t = f * 16 + (l & 15);
  const int ch = n0 + 4 * (l >> 4) + r;
  if (t >= M || ch >= N) return;
  if constexpr (GROUPED) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += u2f((unsigned)red[w][f][l][r]);
    ((unsigned short *)out)[(int64_t)t * ld_y + ch] = float_to_half_bits(sum);
  } else {
    int sum = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[w][f][l][r];
    if constexpr (OUT_I32) {
      ((int32_t *)out)[(int64_t)t * N + ch] = sum >> SHIFT;
    } else {
      const float val = (float)sum * (sa[t] * sw[ch] * UNSCALE);
      ((unsigned short *)out)[(int64_t)t * ld_y + ch] = float_to_half_bits(val);
    }
  }
}

template <int CB>
hipError_t launch_decode(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw, int64_t M, int64_t N,
                         int64_t K, int group, void *y, int64_t ld_y, bool out_i32, hipStream_t stream) {
  dim3 grid((unsigned)((N + kNT - 1) / kNT)), block(64 * kWaves);
  if (group == 0) {
    if (out_i32)
      gemm_decode_kernel<false, true, CB><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N, (int)K, 0, y, ld_y);
    else
      gemm_decode_kernel<false, false, CB><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N, (int)K, 0, y, ld_y);
  } else {
    if (out_i32)
      gemm_decode_kernel<true, true, CB><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N, (int)K, group, y, ld_y);
    else
      gemm_decode_kernel<true, false, CB><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N, (int)K, group, y,
                                                                      ld_y);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_decode(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw,
                              int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                              bool out_i32, hipStream_t stream) {
  return launch_decode<4>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
}

hipError_t launch_gemm_decode_i8(const int8_t *a, const float *sa, const int8_t *w, const float *sw,
                                 int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                                 bool out_i32, hipStream_t stream) {
  return launch_decode<8>((const uint8_t *)a, sa, (const uint8_t *)w, sw, M, N, K, group, y, ld_y, out_i32,
                          stream);
}

}  // namespace qr
