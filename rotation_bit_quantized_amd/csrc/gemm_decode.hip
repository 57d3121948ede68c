// Integer GEMM for decode shapes (M <= 64 tokens): memory-bound, the weight
// codes are streamed from HBM exactly once.
//
// Method: as the prefill kernel (QuaRot abstract: all matrix
// multiplications in 4 bits; dequantizing epilogue per output channel or
// per K-group of 128).  Decoding is the memory-bound phase where the 4-bit
// weights cut the bytes moved (QuaRot summary, "Key points": decode peak
// memory; QuaRot press article: decoding is usually memory-bound).
//
// One workgroup (16 waves) owns 16 output channels and all M <= 64 tokens;
// v_mfma_i32_16x16x64_i8 runs with A = weight rows, B = token rows, giving
// C[channel][token], on codes widened to 16 q int8 (see gemm_prefill.hip) or
// 8-bit codes used as they are (CB = 8, the 6- and 8-bit RTN variants of
// the QuaRot abstract).
//
// Per-channel scales (gemm_decode_lds_kernel): the rows travel in chunks of
// 1 KB per row (the 64 token rows and the block's 16 weight rows) by
// global_load_lds into two LDS buffers; every wave issues its share of the
// first two chunks at once, so that the whole weight slice of a block is in
// flight from the start for K <= 4096.  Chunk c is multiplied as soon as it
// has landed, while chunk c + 1 is still arriving; wave w takes the four
// 16-byte pieces 4w .. 4w + 3 of every row of the chunk.  The DMA lanes
// fetch XOR-swizzled pieces (slot = piece ^ (row & 15)) so that the
// fragment reads, 16 rows at one piece, hit distinct banks.  The 16 wave
// partials are reduced through LDS in int32 (exact), laid out
// [wave][token][channel] so that both the writes and the sums are
// conflict-free, and the output scales are loaded before the first DMA.
//
// Group-wise scales (gemm_decode_grouped_kernel): wave w handles the K-groups w,
// w + 16, ...; it loads up to two 64-byte pieces of each row at once straight
// into registers, folds every finished group into fp32 with its scales, and
// the fp32 partials are reduced through LDS.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kWaves = 16;
constexpr int kNT = 16;  // output channels per workgroup

template <bool OUT_I32, int CB>
__global__ __launch_bounds__(64 * kWaves) void gemm_decode_grouped_kernel(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ W,
    const float *__restrict__ sw, int M, int N, int K, int group, void *__restrict__ out, int64_t ld_y) {
  // fp32 partial sums (as bits): [wave][frag 0..3][lane][4]
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
  constexpr int BATCH = 2;                          // pieces loaded together per wave (128 registers at most)
  const int64_t kbytes = (int64_t)K * CB / 8;
  const int ppu = group / PIECE_CODES;              // pieces per unit (a unit: one K-group)
  const int units = K / group;
  const int G = units;

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
        for (int f = 0; f < 4; ++f)
          uacc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop[ks], aop[f][ks], uacc[f], 0, 0, 0);
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

  if constexpr (OUT_I32) return;   // every group's sums are stored

#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][f][lane][r] = (int)f2u(facc[f][r]);
  __syncthreads();

  // 1024 outputs (4 frags x 64 lanes x 4 regs), one per thread.
  const int f = tid >> 8;
  const int l = (tid >> 2) & 63;
  const int r = tid & 3;
  const int t = f * 16 + (l & 15);
  const int ch = n0 + 4 * (l >> 4) + r;
  if (t >= M || ch >= N) return;
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += u2f((unsigned)red[w][f][l][r]);
  ((unsigned short *)out)[(int64_t)t * ld_y + ch] = float_to_half_bits(sum);
}

constexpr int kDChunk = 1024;             // bytes per row per chunk
constexpr int kDRows = 64 + kNT;           // token rows, then the block's weight rows
constexpr int kDBuf = kDRows * kDChunk;    // one LDS buffer: 80 KB
constexpr int kDDma = kDRows / kWaves;     // DMA wave-instructions per wave and chunk (5)

template <bool OUT_I32, int CB>
__global__ __launch_bounds__(64 * kWaves) void gemm_decode_lds_kernel(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ W,
    const float *__restrict__ sw, int M, int N, int K, void *__restrict__ out, int64_t ld_y) {
  static_assert(CB == 4 || CB == 8, "code width");
  static_assert(kDRows % kWaves == 0 && kDDma == 5, "rows per wave");
  constexpr int SHIFT = CB == 4 ? 8 : 0;            // widened 4-bit products carry 16 * 16
  constexpr float UNSCALE = CB == 4 ? 1.0f / 256.0f : 1.0f;
  constexpr int KS = CB == 4 ? 2 : 1;               // MFMA k-steps per 16-byte piece
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kDBuf];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index in an SGPR: the DMA addresses and row choices stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kNT;
  const int kbytes = K * CB / 8;                    // a multiple of 64 (K % 128 == 0)
  const int nchunks = (kbytes + kDChunk - 1) / kDChunk;

  // the output element of this thread after the reduction, and its scale,
  // loaded first (clamped indices, always valid) so that it has long landed
  const int t = tid >> 4, ch = tid & 15;
  float sav = 0.f, swv = 0.f;
  if constexpr (!OUT_I32) {
    sav = sa[min(t, M - 1)];
    swv = sw[min(n0 + ch, N - 1)];
  }

  // DMA: this wave fills rows 16 q + wave of each chunk (q = 0..3 the token
  // rows, q = 4 the weight row n0 + wave); rows past M or N re-read the last
  // row, whose results are never stored.  Lane l fetches piece l ^ wave, so
  // LDS slot s of row r holds piece s ^ (r & 15).
  const uint8_t *rowp[kDDma];
#pragma unroll
  for (int q = 0; q < 4; ++q) rowp[q] = A + (int64_t)min(16 * q + wave, M - 1) * kbytes;
  rowp[4] = W + (int64_t)min(n0 + wave, N - 1) * kbytes;
  const unsigned lds0 = lds_addr(smem);
  auto issue = [&](int c, int b) __attribute__((always_inline)) {
    const int rem = kbytes - c * kDChunk;
    const int np = (rem < kDChunk ? rem : kDChunk) >> 4;   // pieces in this chunk (a multiple of 4)
    const int p = min(lane ^ wave, np - 1);
    const int off = c * kDChunk + 16 * p;
    // the weight row first: it comes from HBM, the token rows from L2
    dma16_to_lds(rowp[4] + off, lds0 + (unsigned)(b * kDBuf + (64 + wave) * kDChunk));
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16_to_lds(rowp[q] + off, lds0 + (unsigned)(b * kDBuf + (16 * q + wave) * kDChunk));
  };

  v4i acc[4] = {v4i{}, v4i{}, v4i{}, v4i{}};
  issue(0, 0);
  if (nchunks > 1) issue(1, 1);
  for (int c = 0; c < nchunks; ++c) {
    // chunk c has landed (this wave's part); the next one may stay in flight
    if (c + 1 < nchunks) wait_vm<kDDma>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();   // every wave's part of chunk c is in
    const int rem = kbytes - c * kDChunk;
    const int np = (rem < kDChunk ? rem : kDChunk) >> 4;
    if (4 * wave < np) {
      const uint8_t *buf = smem + (c & 1) * kDBuf;
      const int slot = ((4 * wave + g) ^ i16) * 16;
      const v4u wv = *(const v4u *)(buf + (64 + i16) * kDChunk + slot);
      v4u av[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) av[f] = *(const v4u *)(buf + (16 * f + i16) * kDChunk + slot);
      v4i wop[KS], aop[4][KS];
      if constexpr (CB == 4) {
        widen_hi_nibble(wv, wop[0], wop[1]);
#pragma unroll
        for (int f = 0; f < 4; ++f) widen_hi_nibble(av[f], aop[f][0], aop[f][1]);
      } else {
        wop[0] = __builtin_bit_cast(v4i, wv);
#pragma unroll
        for (int f = 0; f < 4; ++f) aop[f][0] = __builtin_bit_cast(v4i, av[f]);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wop[ks], aop[f][ks], acc[f], 0, 0, 0);
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();   // every wave is done with buffer c & 1
    if (c + 2 < nchunks) issue(c + 2, c & 1);
  }

  // reduction over the 16 waves: red[wave][token][channel]; lane (i16, g)
  // holds channels 4g .. 4g + 3 of token 16 f + i16 in acc[f]
  int *red = (int *)smem;
#pragma unroll
  for (int f = 0; f < 4; ++f) *(v4i *)(red + (wave * 64 + 16 * f + i16) * kNT + 4 * g) = acc[f];
  __syncthreads();
  int sum = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += red[(w * 64 + t) * kNT + ch];
  const int col = n0 + ch;
  if (t >= M || col >= N) return;
  if constexpr (OUT_I32) {
    ((int32_t *)out)[(int64_t)t * N + col] = sum >> SHIFT;
  } else {
    const float val = (float)sum * (sav * swv * UNSCALE);
    ((unsigned short *)out)[(int64_t)t * ld_y + col] = float_to_half_bits(val);
  }
}

template <int CB>
hipError_t launch_decode(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw, int64_t M, int64_t N,
                         int64_t K, int group, void *y, int64_t ld_y, bool out_i32, hipStream_t stream) {
  dim3 grid((unsigned)((N + kNT - 1) / kNT)), block(64 * kWaves);
  if (group == 0) {
    if (out_i32)
      gemm_decode_lds_kernel<true, CB><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N, (int)K, y, ld_y);
    else
      gemm_decode_lds_kernel<false, CB><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N, (int)K, y, ld_y);
  } else {
    if (out_i32)
      gemm_decode_grouped_kernel<true, CB><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N, (int)K, group, y,
                                                                       ld_y);
    else
      gemm_decode_grouped_kernel<false, CB><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N, (int)K, group, y,
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
