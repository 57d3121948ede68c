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
// Design (one token row at a time per block of four waves, persistent grid,
// one block per CU):
//  * The dense product runs on v_mfma_f32_16x16x32_f16 with A = X (the fp16
//    input, exact) and B = O
//    split into an fp16 high part and an fp16 low part (O - hi); both
//    products accumulate into the same fp32 accumulators (error near 2^-22
//    relative; one fp16 pass alone would round O to 2^-11 and move codes that
//    sit near a rounding boundary).  K (a) and N (b) are padded to 192.
//  * O's B-fragments stay in AGPRs for the whole kernel, split over the
//    waves: wave w owns N-tiles 3w .. 3w+2 (144 registers of hi/lo parts).
//  * The X row travels by coalesced global_load_lds DMA (1 KB per wave
//    instruction, one per k-step) into one of three LDS buffers shared by
//    the four waves, two rows ahead (HBM latency stays hidden although the
//    DMA is spread over a whole row step).  M-tile mt holds the rows
//    i = 32 (mt >> 1) + 2 c + (mt & 1), c < 16: with the 344-byte row pitch
//    of m = 172, sixteen such rows start in sixteen distinct bank groups.
//  * Software pipeline over rows with two accumulator sets in VGPRs: while
//    the MFMAs of row r run, the same wave finishes row r - 1 (64-point
//    transform, absmax, quantization, code staging) and stores the codes of
//    row r - 2, interleaved with those MFMAs.
//  * The 64-point transform over i is in registers: i0, i5 are M-tile bits,
//    i1, i2 register bits, i3, i4 lane bits 4, 5 brought into register bits
//    with v_permlane16_swap / v_permlane32_swap.
//  * The absmax is reduced with DPP and lane swaps, then across the four
//    waves through LDS.  Codes are packed eight to a word in registers, a
//    4 x 4 nibble transpose within lane quads (DPP, v_perm, v_alignbit) makes
//    each 16-bit half four consecutive codes of one output row, and the
//    block stores the row from LDS as 16-byte chunks.
#include "qr_common.h"
#include "qr_launch.h"

#include <type_traits>

namespace qr {
namespace {

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
template <int V>
using IC = std::integral_constant<int, V>;

constexpr int kWaves = 4;
constexpr int kMT = 4;          // M-tiles of 16 rows i
constexpr int kKS = 6;          // k-steps of 32: a < 192
constexpr int kNTW = 3;         // N-tiles of 16 per wave: b < 192
constexpr int kRowBuf = 23552;  // one X row (<= 22528 bytes) plus the A-read overrun past it
constexpr int kGroupPitch = 1408;                // LDS bytes per 16 output rows j of codes (16 * 176 / 2)
constexpr int kRowBufs = 3;                      // X rows r_k, r_{k+1} resident, r_{k+2} landing
// The codes, a sink and the maxima live in an LDS array of their own: the
// compiler can then tell that their reads do not alias the X rows' DMA
// (otherwise it waits for that DMA before each such read).
constexpr int kCodeOff = 0;                          // codes of one row, four groups of 16 rows j
constexpr int kSinkOff = kCodeOff + 4 * kGroupPitch;   // masked-off code writes land here
constexpr int kMaxOff = kSinkOff + 4 * kGroupPitch;    // the four waves' maxima
constexpr int kAux = kMaxOff + 16;

__global__ __launch_bounds__(64 * kWaves, 1) void rq_kron_kernel(
    const unsigned short *__restrict__ x, int64_t rows, int64_t ld_x, int m, const float *__restrict__ dense,
    uint8_t *__restrict__ codes, float *__restrict__ scales, float scale_mul) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRowBufs * kRowBuf];   // X rows
  __shared__ __attribute__((aligned(16))) uint8_t aux[kAux];
  float *const wmax = (float *)(aux + kMaxOff);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int g = lane >> 4;
  const int rowb = 128 * m;                 // bytes of one X row (64 m fp16)
  const int nchunks = rowb / 1024 + (rowb % 1024 != 0);   // <= 22 = 4 waves x 6 k-steps - 2
  const int code_bytes = 32 * m;            // n / 2
  const int half_m = m >> 1;

  // ---- this wave's B-fragments of O, fp16 hi and lo parts: lane (c16, g)
  // holds O[32 ks + 8 g + j][b], j < 8, b = 16 (3 wave + t) + c16; zero
  // past m.
  v8h ob[kNTW][kKS][2];
  auto o_at = [&](int a, int b) __attribute__((always_inline)) {
    const bool in = a < m && b < m;
    const float o = dense[in ? a * m + b : 0];   // clamped load, then select
    return in ? o : 0.f;
  };
#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
    const int b = 16 * (kNTW * wave + t) + c16;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float o = o_at(32 * ks + 8 * g + j, b);
        const _Float16 h = (_Float16)o;
        ob[t][ks][0][j] = h;
        ob[t][ks][1][j] = (_Float16)(o - (float)h);
      }
  }

  // O lives in AGPRs (MFMA reads its B operand from there); the VGPRs hold
  // the two accumulator sets, which the VALU transform works on in place.
  // (This file is built with MFMA results in VGPRs.)
#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) asm volatile("" : "+a"(ob[t][ks][hl]));
  }
  // A reads that run past a row's DMA'd bytes (small m) must see finite
  // values (they meet zero columns of O): clear each buffer's tail once.
  for (int off = rowb + 16 * tid; off + 16 <= kRowBuf; off += 16 * 64 * kWaves) {
#pragma unroll
    for (int b = 0; b < kRowBufs; ++b) *(v4u *)(smem + b * kRowBuf + off) = v4u{0u, 0u, 0u, 0u};
  }

  // ---- per-lane constants
  // A: M-tile mt, lane (c16, g) reads row i = 32 (mt >> 1) + 2 c16 + (mt & 1):
  // with the 344-byte row pitch of m = 172 the sixteen rows of a read start
  // in sixteen distinct bank groups.
  int a_off[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) a_off[mt] = (32 * (mt >> 1) + 2 * c16 + (mt & 1)) * 2 * m;
  // code writes: after the nibble transpose, half h of word (t, R) holds the
  // codes of row j = g | (c16 & 3) << 2 | h << 4 | R << 5, columns
  // col .. col + 3 with col = 16 (3 wave + t) + 4 (c16 >> 2); LDS keeps 16
  // rows j per group of kGroupPitch bytes, group 2 R + h.
  int cw_off[kNTW];
#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
    const int col = 16 * (kNTW * wave + t) + 4 * (c16 >> 2);
    // (columns past m: a sink address of the lane's own, so such writes
    // do not pile up on one LDS address)
    cw_off[t] = col < m ? kCodeOff + (g | ((c16 & 3) << 2)) * half_m + (col >> 1) : kSinkOff + 2 * lane;
  }
  // code stores: 16-byte chunks ch = tid, tid + 256 of the row; a lane past
  // the row's end stores chunk ch mod nst again (the same bytes, at
  // distinct addresses: no branch, no pile-up on one address); a chunk never
  // straddles a group (8 m bytes).
  int cs_lds[2], cs_glb[2];
  {
    const int nst = code_bytes / 16;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      int ch = tid + 64 * kWaves * pp;
      ch = ch < nst ? ch : ch % nst;
      const int grp = ch / (half_m), within = ch - grp * half_m;
      cs_lds[pp] = kCodeOff + grp * kGroupPitch + 16 * within;
      cs_glb[pp] = 16 * ch;
    }
  }
  // nibble transpose within lane quads
  const unsigned perm_sel = (lane & 2) ? 0x03070105u : 0x06020400u;
  const unsigned rot_sh = (lane & 1) ? 4u : 28u;
  const unsigned keep = (lane & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;

  // DMA of X row r into LDS buffer bsel, one wave-instruction per k-step
  // region: instruction q of this wave covers bytes 1024 (4 q + wave) ..
  // +1023 of the row (a coalesced 1 KB).  Lanes past the row's end re-read its
  // last 16 bytes; instructions past the last chunk repeat it (small m only).
  int dma_src[kKS], dma_dst[kKS];
#pragma unroll
  for (int q = 0; q < kKS; ++q) {
    int chunk = q * kWaves + wave;
    chunk = chunk < nchunks ? chunk : nchunks - 1;
    dma_dst[q] = 1024 * chunk;
    const int off = 1024 * chunk + 16 * lane;
    dma_src[q] = off < rowb - 16 ? off : rowb - 16;
  }
  const unsigned smem_lds = lds_addr(smem);
  auto issue_dma = [&](const uint8_t *src, int bsel, int q) __attribute__((always_inline)) {
    dma16_to_lds(src + dma_src[q], smem_lds + (unsigned)(bsel * kRowBuf + dma_dst[q]));
  };

  v4f S[2][kMT][kNTW];   // two rows: one in the MFMA phase, one being finished
  v8h apre[kMT];         // the next row's k-step 0 A-fragments, read a region ahead

  // One row step k, all compile-time flags: the MFMAs of row r_k (in LDS
  // buffer k % 3) into register set MS (MS < 0: none), and the transform,
  // maximum, quantization, code staging and stores of row prow in register
  // set PS (PS < 0: none).  Six k-step regions; the MFMAs of each are
  // interleaved with one part of the other row's work:
  //   0-2: transform of N-tile t = ks   3: absmax, then barrier
  //   4: quantize, transpose, stage codes; DMA wait for r_{k+1}; barrier
  //   5: store prow's codes; read r_{k+1}'s k-step 0 A-fragments
  auto step = [&](auto ms_tag, auto ps_tag, int xbuf, int nbuf, int dbuf, uint8_t *cr, float *sp,
                  const uint8_t *next_src)
                  __attribute__((always_inline)) {
    constexpr int MS = decltype(ms_tag)::value;
    constexpr int PS = decltype(ps_tag)::value;
    // r_k is in buffer k % 3; r_{k+2} goes to (k + 2) % 3, which r_{k-1}
    // left at the previous step's k-step 4 barrier
    const uint8_t *xb = smem + xbuf * kRowBuf;
    v8h acur[kMT], anxt[kMT];
    unsigned w[kNTW][2];
    float mx = 0.f, inv = 0.f;
    if constexpr (MS >= 0) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) acur[mt] = apre[mt];
    }
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if constexpr (MS >= 0) {
        issue_dma(next_src, dbuf, ks);
        if (ks + 1 < kKS) {
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt)
            anxt[mt] = __builtin_bit_cast(v8h, *(const v4u *)(xb + a_off[mt] + 16 * g + 64 * (ks + 1)));
        }
        // the twelve hi products, then the twelve lo ones: an accumulator's
        // two updates are twelve MFMAs apart
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
          for (int t = 0; t < kNTW; ++t)
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
              if (ks == 0 && hl == 0)   // the row's first product: C = 0
                S[MS][mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(acur[mt], ob[t][ks][hl], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
              else
                S[MS][mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(acur[mt], ob[t][ks][hl], S[MS][mt][t], 0, 0, 0);
            }
        if (ks + 1 < kKS) {
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt) acur[mt] = anxt[mt];
        }
        if (ks == kKS - 1) {
          // r_{k+1} is in every wave's part of buffer nbuf since the k-step 4 barrier
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt)
            apre[mt] = __builtin_bit_cast(v8h, *(const v4u *)(smem + nbuf * kRowBuf + a_off[mt] + 16 * g));
        }
      }
      if constexpr (PS >= 0) {
        if (ks <= 2) {
          // 64-point Walsh-Hadamard over i for N-tile t = ks.  Element r of
          // S[PS][mt][t] is row i = 32 (mt >> 1) + 8 g + 2 r + (mt & 1):
          // i0 = mt bit 0, i1 = r bit 0, i2 = r bit 1, i3 = lane bit 4,
          // i4 = lane bit 5, i5 = mt bit 1.
          const int t = ks;
#pragma unroll
          for (int mb = 1; mb <= 2; mb <<= 1)
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
              if (mt & mb) continue;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float u = S[PS][mt][t][r], v = S[PS][mt | mb][t][r];
                S[PS][mt][t][r] = u + v;
                S[PS][mt | mb][t][r] = u - v;
              }
            }
#pragma unroll
          for (int rb = 1; rb <= 2; rb <<= 1)
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                if (r & rb) continue;
                const float u = S[PS][mt][t][r], v = S[PS][mt][t][r | rb];
                S[PS][mt][t][r] = u + v;
                S[PS][mt][t][r | rb] = u - v;
              }
          // i3: lane bit 4 <-> M-tile bit 0 (done), then butterfly over M-tile bit 0
#pragma unroll
          for (int mt = 0; mt < kMT; mt += 2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float u = S[PS][mt][t][r], v = S[PS][mt + 1][t][r];
              swap16(u, v);
              S[PS][mt][t][r] = u + v;
              S[PS][mt + 1][t][r] = u - v;
            }
          // i4: lane bit 5 <-> register bit 0 (done), then butterfly over register bit 0
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              float u = S[PS][mt][t][r], v = S[PS][mt][t][r + 1];
              swap32(u, v);
              S[PS][mt][t][r] = u + v;
              S[PS][mt][t][r + 1] = u - v;
            }
          // Element r of S[PS][mt][t] is now output row
          //   j = g | (r >> 1) << 2 | (mt & 1) << 3 | (r & 1) << 4 | (mt >> 1) << 5,
          // column b = 16 (3 wave + t) + c16 (zero for b >= m: O's padding is zero).
        }
        if (ks == 3) {
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int t = 0; t < kNTW; ++t)
#pragma unroll
              for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(S[PS][mt][t][r]));
          mx = wave_max_dpp(mx);
          if (lane == 0) wmax[wave] = mx;
        }
        if (ks == 4) {
          mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
          inv = mx > 0.f ? 7.0f / mx : 0.f;
          // four-bit two's complement codes; nibble 4 k + 16 h of w[t][R]
          // is the code of element r of S[PS][mt][t] with
          // k = (r >> 1) | (mt & 1) << 1, h = r & 1, R = mt >> 1.  Each
          // alignbit shifts the word right by four and inserts the next code
          // at the top, so codes enter in nibble order.
#pragma unroll
          for (int t = 0; t < kNTW; ++t)
#pragma unroll
            for (int R = 0; R < 2; ++R) {
              unsigned acc = 0u;
#pragma unroll
              for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                  const int mt = 2 * R + (kk >> 1), r = (kk & 1) * 2 + h;
                  acc = __builtin_amdgcn_alignbit(round_bits(S[PS][mt][t][r], inv), acc, 4);
                }
              w[t][R] = acc;
            }
          // 4 x 4 nibble transposes within each lane quad, exchanging the
          // quad lane index (the column's low two bits) with k
#pragma unroll
          for (int t = 0; t < kNTW; ++t)
#pragma unroll
            for (int R = 0; R < 2; ++R) {
              unsigned v = w[t][R];
              v = __builtin_amdgcn_perm(dpp<kQuadXor2>(v), v, perm_sel);   // lane bit 1 <-> k bit 1
              const unsigned o = dpp<kQuadXor1>(v);                         // lane bit 0 <-> k bit 0
              const unsigned sh = __builtin_amdgcn_alignbit(o, o, rot_sh);
              v = (keep & v) | (~keep & sh);
#pragma unroll
              for (int h = 0; h < 2; ++h)
                *(unsigned short *)(aux + cw_off[t] + (2 * R + h) * kGroupPitch) = (unsigned short)(v >> (16 * h));
            }
        }
        if (ks == 5) {
          // the block stores the row's codes as 16-byte chunks, one lane the scale
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const v4u v = *(const v4u *)(aux + cs_lds[pp]);
            *(v4u *)(cr + cs_glb[pp]) = v;
          }
          if (tid == 0) *sp = mx * scale_mul;
        }
      }
      // block-wide hand-offs: the four partial maxima (k-step 3); the staged
      // codes and r_{k+1}'s row (k-step 4).  r_{k+1}'s DMA was issued during
      // the previous step; this step has issued five DMA instructions since
      // (and the previous step's stores went out before them): with
      // in-order completion, at most five outstanding operations means
      // r_{k+1} is in.
      if (ks == 3 && PS >= 0) {
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
      }
      if (ks == 4 && (MS >= 0 || PS >= 0)) {
        if (MS >= 0) wait_vm<kKS - 1>();
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
      }
      // region fence: the A reads a region issues for the next one stay a
      // whole region of MFMAs ahead of their first use
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Rows r_k = block + k * grid: X of row r_{k+2} is in flight while row r_k
  // is multiplied, and row r_{k-1} is finished and stored during those
  // MFMAs.
  // Per-step bookkeeping is scalar and cheap: rotating buffer indices and
  // running row pointers.
  const int stride = (int)gridDim.x;
  const int64_t row0 = blockIdx.x;   // the grid is no larger than rows
  // rows of this block, wave-uniform in an SGPR
  const int nblk = __builtin_amdgcn_readfirstlane((int)((rows - row0 + stride - 1) / stride));
  const int64_t x_step = (int64_t)stride * ld_x * 2;   // bytes between a block's rows
  const uint8_t *const x0 = (const uint8_t *)(x + row0 * ld_x);
  const uint8_t *const x_last = x0 + (int64_t)(nblk - 1) * x_step;
  // (past the block's last row: that row again, into a free buffer)
  auto clamp_src = [&](int kk, const uint8_t *p) { return kk < nblk ? p : x_last; };
  auto rot = [](int b) { return b == kRowBufs - 1 ? 0 : b + 1; };
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint8_t *src = clamp_src(b, x0 + b * x_step);
#pragma unroll
    for (int q = 0; q < kKS; ++q) issue_dma(src, b, q);
  }
  wait_vm<kKS>();   // r_0 is in (r_1's six instructions may be outstanding)
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) apre[mt] = __builtin_bit_cast(v8h, *(const v4u *)(smem + a_off[mt] + 16 * g));
  const uint8_t *src2 = x0 + 2 * x_step;               // row r_{k+2}
  uint8_t *crow = codes + row0 * (int64_t)code_bytes;  // codes of row r_{k-1}
  float *srow = scales + row0;
  const int64_t c_step = (int64_t)stride * code_bytes;
  step(IC<0>{}, IC<-1>{}, 0, 1, 2, crow, srow, clamp_src(2, src2));
  src2 += x_step;
  int k = 1, xb = 1, nb = 2, db = 0;
  auto advance = [&]() __attribute__((always_inline)) {
    src2 += x_step;
    crow += c_step;
    srow += stride;
    xb = rot(xb);
    nb = rot(nb);
    db = rot(db);
  };
  for (; k + 1 < nblk; k += 2) {
    step(IC<1>{}, IC<0>{}, xb, nb, db, crow, srow, clamp_src(k + 2, src2));
    advance();
    step(IC<0>{}, IC<1>{}, xb, nb, db, crow, srow, clamp_src(k + 3, src2));
    advance();
  }
  if (k < nblk) {
    step(IC<1>{}, IC<0>{}, xb, nb, db, crow, srow, clamp_src(k + 2, src2));
    advance();
    ++k;
  }
  // the last row r_{n-1} is in register set (n - 1) & 1
  if ((nblk - 1) & 1)
    step(IC<-1>{}, IC<1>{}, 0, 0, 0, crow, srow, nullptr);
  else
    step(IC<-1>{}, IC<0>{}, 0, 0, 0, crow, srow, nullptr);
  wait_vm<0>();   // no DMA may still be writing this block's LDS when it exits
}

}  // namespace

bool rq_kron_supported(const RotArgs &r, int group) {
  return r.dense_m > 1 && r.had_n == 64 && r.dense_m <= 176 && r.dense_m % 4 == 0 && r.signs == nullptr &&
         group == 0;
}

hipError_t launch_rq_kron(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, int group,
                          uint8_t *codes, float *scales, hipStream_t stream) {
  (void)group;
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t grid = rows < cus ? rows : cus;
  const float scale_mul = (float)(1.0 / (7.0 * 8.0));   // 1/(7 sqrt(64))
  rq_kron_kernel<<<dim3((unsigned)grid), dim3(64 * kWaves), 0, stream>>>(
      (const unsigned short *)x, rows, ld_x, r.dense_m, r.dense, codes, scales, scale_mul);
  return hipGetLastError();
}

}  // namespace qr
