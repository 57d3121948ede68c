// Online randomized Hadamard rotation + symmetric 4-bit RTN + nibble packing
// for n = 2^L, L in {12, 13} (LLaMA hidden sizes 4096 and 8192), no dense
// factor, per-row or group-128 scales.
//
// Method: y = (x * d) H_n / sqrt(n) (QuaRot summary, "Summary"; randomized
// Hadamard: QuaRot press article), s = max|y|/7, q = rint(y/s) packed two per
// byte (QuaRot summary, "Key points": RTN on the fly; group size 128).
//
// Design (one wave per token row, rows grid-strided over a persistent grid):
//  * Data path: each wave owns two one-row LDS buffers.  Rows are brought in
//    by global_load_lds_dwordx4 (no VGPR staging); as soon as pass 1 has
//    read a buffer, the DMA of the wave's row after next is issued into it,
//    so two rows stream from HBM while the wave works on a third.
//  * Element index bits e0..e(L-1).  Since H_n[e][f] = (-1)^popcount(e & f),
//    the transform factors over any split of the bits into two sets; here
//      i_b = {e0, e1, e6, e7, e8, e9}   (64-point factor, on MFMA)
//      i_a = {e2..e5, e10..e(L-1)}       (the rest, in registers)
//  * Pass 1: v_mfma_f32_16x16x32_f16 with A = the fp16 input (exact, sign-
//    flipped by XOR) and B = the +-1 64-point factor.  Each lane reads 8-byte
//    pieces: lane bits 0..3 select e2..e5 (rows of A), lane bits 4..5 select
//    e6, e7 (k-groups), the two 8-byte halves select e8, the k-step e9 and the
//    M-tile e10.. - so every LDS read instruction covers 512 contiguous bytes.
//  * B's columns are permuted so that the MFMA output puts e0, e1 in the
//    N-tile index and e6..e9 in lane bits 0..3; the output rows carry e2, e3
//    in the register index and e4, e5 in lane bits 4, 5.
//  * Pass 2: butterflies on e2, e3, e10.. in registers; e4 and e5 are first
//    swapped into registers with v_permlane16_swap / v_permlane32_swap (each
//    a 2x2 transpose of a lane bit and a register bit), then butterflied.
//  * After pass 2 each lane holds 64 consecutive outputs (two runs for
//    n = 8192) and lane l owns outputs [64 l, 64 l + 64): absmax, rounding
//    and packing stay in the lane and the codes go out as 16-byte stores.
// The 1/sqrt(n) is folded into the stored scale (codes do not depend on it).
// BITS = 6 or 8 (QuaRot abstract: lossless 6- and 8-bit RTN): s = max|y|/qmax
// with qmax = 2^(BITS-1) - 1, one int8 code per byte, four 16-byte stores
// per lane and run.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

// n = 4096: four waves per block, each with two row buffers (two of its
// rows stream in while it works on a third): 64 KB per block, two blocks per
// CU.  n = 8192: eight waves per block, each with one row buffer refilled as
// soon as pass 1 has read it (the row streams in while the wave transforms,
// quantizes and stores the previous one), and the per-lane sign masks in
// LDS rather than in 64 registers: 128 KB + 16 KB per block, one block per
// CU, two waves per SIMD (the 1-wave-per-SIMD form left the SIMD idle on
// its own latencies).
template <int L>
constexpr int waves_of() {
  return L == 13 ? 8 : 4;
}
template <int L>
constexpr int bufs_of() {
  return L == 13 ? 1 : 2;
}
template <int L>
constexpr bool lds_signs() {
  return L == 13;
}
template <int L>
constexpr int sign_lds_bytes() {
  return lds_signs<L>() ? 64 * (8 << (L - 10)) * 4 : 0;   // [words / 4][lane][4] of unsigned
}
template <int L>
constexpr int lds_bytes() {
  return waves_of<L>() * bufs_of<L>() * (2 << L) + sign_lds_bytes<L>();
}

// The B operands (the +-1 64-point factor, columns permuted) of every lane,
// computed at compile time: entry [s][nt][lane] is the v8h for k-step s and
// N-tile nt; slot j holds (-1)^parity with parity = popcount((j & 3) & nt) +
// popcount(g & (c16 & 3)) + ((j >> 2) & (c16 >> 2) & 1) + (s & (c16 >> 3)).
struct BopTable {
  unsigned w[2][4][64][4];
};
constexpr BopTable make_bop_table() {
  BopTable t{};
  for (int s = 0; s < 2; ++s)
    for (int nt = 0; nt < 4; ++nt)
      for (int lane = 0; lane < 64; ++lane) {
        const int c16 = lane & 15, g = lane >> 4;
        for (int d = 0; d < 4; ++d) {
          unsigned word = 0;
          for (int half = 0; half < 2; ++half) {
            const int j = 2 * d + half;
            int par = ((j & 3) & nt) ^ (g & (c16 & 3));
            par = (par & 1) ^ ((par >> 1) & 1);
            par ^= ((j >> 2) & (c16 >> 2) & 1) ^ (s & (c16 >> 3));
            word |= (par ? 0xBC00u : 0x3C00u) << (16 * half);
          }
          t.w[s][nt][lane][d] = word;
        }
      }
  return t;
}
__device__ constexpr BopTable kBop = make_bop_table();

// Register index of a value: bits 0-1 = r (MFMA output row within the 4-row
// group), bits 2-3 = N-tile, bits 4.. = M-tile.
template <int L, int GROUP, int BITS = 4>
__global__ __launch_bounds__(64 * waves_of<L>()) void rq_pow2_kernel(
    const unsigned short *__restrict__ x, int64_t rows, int64_t ld_x, const int8_t *__restrict__ signs,
    uint8_t *__restrict__ codes, float *__restrict__ scales, float scale_mul) {
  constexpr int n = 1 << L;
  constexpr int ROWB = 2 * n;         // bytes per input row
  constexpr int DMA = ROWB / 1024;    // 1 KB DMA wave-instructions per row
  constexpr int MT = 1 << (L - 10);   // M-tiles of 16 rows of the 64-column view
  constexpr int NV = MT * 16;         // values per lane
  constexpr int RUNS = NV / 64;
  static_assert(BITS == 4 || BITS == 6 || BITS == 8, "code width");
  constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);
  constexpr int CODE_BYTES = BITS == 4 ? n / 2 : n;   // per row
  constexpr int CODE_STORES = BITS == 4 ? 2 : 4;      // 16-byte stores per lane and run
  // vector-memory instructions per row after its compute: the code stores
  // of every run, then the scale stores (one per run for groups)
  constexpr int STORES = CODE_STORES * RUNS + (GROUP == 0 ? 1 : RUNS);
  static_assert(L == 12 || L == 13, "pass-2 layout written for n = 4096, 8192");
  static_assert(2 * STORES + DMA < 64, "vmcnt range");
  constexpr int kWaves = waves_of<L>();
  constexpr int kBufs = bufs_of<L>();
  constexpr bool SIGNS_LDS = lds_signs<L>();

  __shared__ __attribute__((aligned(1024))) uint8_t smem[lds_bytes<L>()];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t *const bufs = smem + wave * kBufs * ROWB;
  unsigned *const sign_lds = (unsigned *)(smem + kWaves * kBufs * ROWB);

  const int c16 = lane & 15;
  const int g = lane >> 4;

  // B operands: b[s][nt][j] = H(k, col), k bits from (slot j, k-group g, step
  // s), column bits from (N-tile nt, lane column c16).
  v8h bop[2][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bop[s][nt] = __builtin_bit_cast(v8h, *(const v4u *)kBop.w[s][nt][lane]);

  const int64_t wave_id = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t wave_stride = (int64_t)gridDim.x * kWaves;

  // Sign masks for the pieces this lane reads: piece (m, s, h) covers
  // elements base + 0..3 with base = 4 c16 + 64 g + 256 h + 512 s + 1024 m;
  // their four int8 signs are one aligned 32-bit word, two mask words each.
  // With SIGNS_LDS the 8 MT words of a lane live in LDS as [w / 4][lane][4]
  // (16-byte reads of consecutive lanes: no bank conflicts), written once
  // by wave 0 before any wave may leave.
  constexpr int NMASK = SIGNS_LDS ? 1 : MT;
  unsigned smask[NMASK][2][2][2];
  const bool have_signs = signs != nullptr;
  if constexpr (SIGNS_LDS) {
    if (have_signs && wave == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            unsigned m0, m1;
            sign_masks4(*(const unsigned *)(signs + 4 * c16 + 64 * g + 256 * h + 512 * s + 1024 * m), m0, m1);
            const int w = ((m * 2 + s) * 2 + h) * 2;   // words w, w + 1
            sign_lds[((w >> 2) * 64 + lane) * 4 + (w & 3)] = m0;
            sign_lds[(((w + 1) >> 2) * 64 + lane) * 4 + ((w + 1) & 3)] = m1;
          }
    }
    __syncthreads();
  }
  if (wave_id >= rows) return;

  // DMA of row r (< rows) into buffer b.
  auto issue_row = [&](int64_t r, int b) {
    const uint8_t *src = (const uint8_t *)(x + r * ld_x);
#pragma unroll
    for (int i = 0; i < DMA; ++i)
      __builtin_amdgcn_global_load_lds((const void *)(src + 1024 * i + 16 * lane),
                                       (lds_void *)(bufs + b * ROWB + 1024 * i), 16, 0, 0);
  };

  // Register sign masks: the sign words are loaded as one batch, and the
  // first rows' DMA goes out before the masks wait for them.
  unsigned sword[SIGNS_LDS ? 1 : MT][2][2];
  if constexpr (!SIGNS_LDS) {
    if (have_signs) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            sword[m][s][h] = *(const unsigned *)(signs + 4 * c16 + 64 * g + 256 * h + 512 * s + 1024 * m);
    }
  }

  issue_row(wave_id, 0);
  if constexpr (kBufs == 2) {
    if (wave_id + wave_stride < rows) issue_row(wave_id + wave_stride, 1);
  }

  if constexpr (!SIGNS_LDS) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          smask[m][s][h][0] = smask[m][s][h][1] = 0u;
          if (have_signs) sign_masks4(sword[m][s][h], smask[m][s][h][0], smask[m][s][h][1]);
        }
  }

  int it = 0;
  for (int64_t row = wave_id; row < rows; row += wave_stride, ++it) {
    set_prio_by_progress(it);   // the waves sharing a SIMD keep pace
    const uint8_t *buf = bufs + (kBufs == 2 ? (it & 1) * ROWB : 0);
    // Wait for this row's DMA.  Two buffers: issued after it are the DMA of
    // the wave's following row (when that row exists; DMAs of rows past the
    // end are not issued), the stores of the previous row (it >= 1) and of
    // the one before (it >= 2).  One buffer: only the previous row's stores
    // (it >= 1).  The sign words, where loaded, went out before the first
    // row's DMA.  The branches are wave-uniform.
    if constexpr (kBufs == 2) {
      const bool follower = row + wave_stride < rows;
      if (it == 0) {
        if (follower) wait_vm<DMA>();
        else wait_vm<0>();
      } else if (it == 1) {
        if (follower) wait_vm<DMA + STORES>();
        else wait_vm<STORES>();
      } else {
        if (follower) wait_vm<DMA + 2 * STORES>();
        else wait_vm<2 * STORES>();
      }
    } else {
      if (it > 0) wait_vm<STORES>();
      else wait_vm<0>();
    }

    // ---- pass 1: 64-point factor on MFMA, A read from the LDS row buffer
    v2u pc[MT][2][2];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          pc[m][s][h] = *(const v2u *)(buf + 2 * (4 * c16 + 64 * g + 256 * h + 512 * s + 1024 * m));
    if constexpr (SIGNS_LDS) {
      if (have_signs) {
#pragma unroll
        for (int q = 0; q < 2 * MT; ++q) {   // 4 words per read: pieces (m, s) = q, h = 0, 1
          const v4u mw = *(const v4u *)(sign_lds + (q * 64 + lane) * 4);
          const int m = q >> 1, s = q & 1;
          pc[m][s][0][0] ^= mw[0];
          pc[m][s][0][1] ^= mw[1];
          pc[m][s][1][0] ^= mw[2];
          pc[m][s][1][1] ^= mw[3];
        }
      }
    }
    // every read has returned: the buffer takes its next row (none past the
    // end: the waits above count only the DMAs of rows that exist)
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    if constexpr (kBufs == 2) {
      if (row + 2 * wave_stride < rows) issue_row(row + 2 * wave_stride, it & 1);
    } else if (row + wave_stride < rows) {
      issue_row(row + wave_stride, 0);
    }

    float v[NV];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      v8h a[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v4u w;
        if constexpr (SIGNS_LDS) {
          w[0] = pc[m][s][0][0];
          w[1] = pc[m][s][0][1];
          w[2] = pc[m][s][1][0];
          w[3] = pc[m][s][1][1];
        } else {
          w[0] = pc[m][s][0][0] ^ smask[m][s][0][0];
          w[1] = pc[m][s][0][1] ^ smask[m][s][0][1];
          w[2] = pc[m][s][1][0] ^ smask[m][s][1][0];
          w[3] = pc[m][s][1][1] ^ smask[m][s][1][1];
        }
        a[s] = __builtin_bit_cast(v8h, w);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        v4f c = {0.f, 0.f, 0.f, 0.f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], bop[0][nt], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], bop[1][nt], c, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[(m << 4) | (nt << 2) | r] = c[r];
      }
    }

    // ---- pass 2: butterflies over i_a
    // register bits 0, 1 (e2, e3) and the M-tile bits (e10..)
#pragma unroll
    for (int bit = 0; bit < L - 8; ++bit) {
      const int rb = bit < 2 ? bit : bit + 2;  // skip the N-tile bits 2, 3
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (i & (1 << rb)) continue;
        const float a = v[i], b = v[i | (1 << rb)];
        v[i] = a + b;
        v[i | (1 << rb)] = a - b;
      }
    }
    // lane bit 4 (e4) <-> register bit 4 (M-tile bit 0, already transformed)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i & 16) continue;
      swap16(v[i], v[i | 16]);
      const float a = v[i], b = v[i | 16];
      v[i] = a + b;
      v[i | 16] = a - b;
    }
    // lane bit 5 (e5) <-> register bit 5 (M-tile bit 1)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i & 32) continue;
      swap32(v[i], v[i | 32]);
      const float a = v[i], b = v[i | 32];
      v[i] = a + b;
      v[i | 32] = a - b;
    }

    // Lane now owns outputs e = 64*lane + f(i) (+ 4096 * bit6 of i for L=13)
    // with f(i) = ((i>>2)&3) | (i&3)<<2 | ((i>>4)&3)<<4.
    float amax[RUNS];
#pragma unroll
    for (int run = 0; run < RUNS; ++run) {
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < 64; ++i) mx = fmaxf(mx, fabsf(v[run * 64 + i]));
      amax[run] = mx;
    }
    if (GROUP == 0) {
      float mx = amax[0];
#pragma unroll
      for (int run = 1; run < RUNS; ++run) mx = fmaxf(mx, amax[run]);
      mx = wave_max(mx);
#pragma unroll
      for (int run = 0; run < RUNS; ++run) amax[run] = mx;
    } else {
      // a group of 128 spans lanes 2q, 2q+1 of one run
#pragma unroll
      for (int run = 0; run < RUNS; ++run) amax[run] = fmaxf(amax[run], __shfl_xor(amax[run], 1, 64));
    }

    uint8_t *cr = codes + row * (int64_t)CODE_BYTES;
#pragma unroll
    for (int run = 0; run < RUNS; ++run) {
      const float inv = amax[run] > 0.f ? QMAX / amax[run] : 0.f;
      if constexpr (BITS != 4) {
        // 64 int8 codes of this lane, in output order, as 16 words
        unsigned words[16];
#pragma unroll
        for (int w = 0; w < 16; ++w) {
          unsigned wd = 0u;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int e = 4 * w + t;  // position within the 64-run
            const int i = ((e >> 2) & 3) | ((e & 3) << 2) | (((e >> 4) & 3) << 4);
            wd |= (round_bits(v[run * 64 + i], inv) & 0xFFu) << (8 * t);
          }
          words[w] = wd;
        }
        v4u *dst = (v4u *)(cr + run * 4096 + 64 * lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = v4u{words[4 * q], words[4 * q + 1], words[4 * q + 2], words[4 * q + 3]};
        continue;
      }
      unsigned words[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        unsigned bits[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int e = 8 * w + t;  // position within the 64-run
          const int i = ((e >> 2) & 3) | ((e & 3) << 2) | (((e >> 4) & 3) << 4);
          bits[t] = round_bits(v[run * 64 + i], inv);
        }
        words[w] = pack8_nibbles(bits[0], bits[1], bits[2], bits[3], bits[4], bits[5], bits[6], bits[7]);
      }
      v4u *dst = (v4u *)(cr + run * (n / 4) + 32 * lane);
      dst[0] = v4u{words[0], words[1], words[2], words[3]};
      dst[1] = v4u{words[4], words[5], words[6], words[7]};
    }
    if (GROUP == 0) {
      if (lane == 0) scales[row] = amax[0] * scale_mul;
    } else {
#pragma unroll
      for (int run = 0; run < RUNS; ++run)
        if ((lane & 1) == 0) scales[row * (n / 128) + run * 32 + (lane >> 1)] = amax[run] * scale_mul;
    }
  }
  wait_vm<0>();   // no DMA may still be writing this block's LDS when it exits
}

template <int L, int GROUP, int BITS = 4>
hipError_t launch_one(const void *x, int64_t rows, int64_t ld_x, const int8_t *signs, uint8_t *codes,
                      float *scales, hipStream_t stream) {
  const int cus = device_cu_count();
  // persistent grid: as many blocks as are resident at once
  // resident blocks per CU: a constant of the kernel, queried once (a
  // function-local static is initialised exactly once, thread-safely)
  static const int per_cu = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, rq_pow2_kernel<L, GROUP, BITS>, 64 * waves_of<L>(), 0) != hipSuccess ||
        b < 1)
      b = 1;
    return b;
  }();
  constexpr int kWaves = waves_of<L>();
  const int64_t blocks_needed = (rows + kWaves - 1) / kWaves;
  const int64_t cap = (int64_t)cus * per_cu;
  const int64_t grid = blocks_needed < cap ? blocks_needed : cap;
  const double qmax = (double)((1 << (BITS - 1)) - 1);
  const float scale_mul = (float)(1.0 / (qmax * __builtin_sqrt((double)(1 << L))));
  rq_pow2_kernel<L, GROUP, BITS><<<dim3((unsigned)grid), dim3(64 * kWaves), 0, stream>>>(
      (const unsigned short *)x, rows, ld_x, signs, codes, scales, scale_mul);
  return hipGetLastError();
}

}  // namespace

bool rq_pow2_supported(const RotArgs &r, int group) {
  return r.dense_m == 1 && (r.n == 4096 || r.n == 8192) && (group == 0 || group == 128);
}

hipError_t launch_rq_pow2(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group,
                          uint8_t *codes, float *scales, hipStream_t stream) {
  return launch_rq_pow2_bits(x, rows, ld_x, r, group, 4, codes, scales, stream);
}

hipError_t launch_rq_pow2_bits(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group, int bits,
                               uint8_t *codes, float *scales, hipStream_t stream) {
#define QR_POW2(L, B)                                                                          \
  return group ? launch_one<L, 128, B>(x, rows, ld_x, r.signs, codes, scales, stream)          \
               : launch_one<L, 0, B>(x, rows, ld_x, r.signs, codes, scales, stream)
  if (r.n == 4096) {
    if (bits == 8) QR_POW2(12, 8);
    if (bits == 6) QR_POW2(12, 6);
    QR_POW2(12, 4);
  }
  if (bits == 8) QR_POW2(13, 8);
  if (bits == 6) QR_POW2(13, 6);
  QR_POW2(13, 4);
#undef QR_POW2
}

}  // namespace qr
