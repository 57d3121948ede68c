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
// two blocks per CU):
//  * The dense product runs on v_mfma_f32_16x16x32_f16 with A = X (the fp16
//    input, exact) and B = O split into an fp16 high part and an fp16 low
//    part (O - hi); both products accumulate into the same fp32 accumulators
//    (error near 2^-22 relative; one fp16 pass alone would round O to 2^-11
//    and move codes that sit near a rounding boundary).  K (a) and N (b) are
//    padded to 192.
//  * O's B-fragments stay in AGPRs for the whole kernel, split over the
//    waves: wave w owns N-tiles 3w .. 3w+2 (144 registers of hi/lo parts).
//    With one accumulator set and the A-fragments of two M-tiles at a time,
//    a wave fits in 256 registers, so each SIMD holds a wave of each of two
//    blocks: a wave does not overlap its own VALU work with its own MFMAs,
//    but one block's transform runs beside the other block's products.
//  * The X row travels by coalesced global_load_lds DMA (1 KB per wave
//    instruction, one per k-step) into one of three LDS buffers shared by
//    the four waves: the DMA of row r_{k+2} is issued during row r_k.  M-tile
//    mt holds the rows i = 32 (mt >> 1) + 2 c + (mt & 1), c < 16: with the
//    344-byte row pitch of m = 172, sixteen such rows start in sixteen
//    distinct bank groups.  With a pitch of 8 mod 16 bytes every odd row
//    starts half-way into a 16-byte unit, so each A-fragment is read as two
//    8-byte halves: a 16-byte LDS read from such an address stalls the wave
//    (at 131072 x 11008 the single-read form took about 1.4 ms, the split
//    form about 1.3 ms).
//  * The 64-point transform over i is in registers: i0, i5 are M-tile bits,
//    i1, i2 register bits, i3, i4 lane bits 4, 5 brought into register bits
//    with v_permlane16_swap / v_permlane32_swap.
//  * The absmax is reduced with DPP and lane swaps, then across the four
//    waves through LDS.  Codes are packed eight to a word in registers, a
//    4 x 4 nibble transpose within lane quads (DPP, v_perm, v_alignbit) makes
//    each 16-bit half four consecutive codes of one output row, and the
//    block stores the row from LDS as 16-byte chunks after the next row's
//    first barrier (two barriers per row).
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kWaves = 4;
constexpr int kMT = 4;          // M-tiles of 16 rows i
constexpr int kKS = 6;          // k-steps of 32: a < 192
constexpr int kNTW = 3;         // N-tiles of 16 per wave: b < 192
constexpr int kRowBuf = 23552;  // one X row (<= 22528 bytes) plus the A-read overrun past it
constexpr int kGroupPitch = 1408;                // LDS bytes per 16 output rows j of codes (16 * 176 / 2)
constexpr int kRowBufs = 3;                      // X rows r_k, r_{k+1} resident, r_{k+2} landing
// The code staging lives in an LDS array of its own (the compiler can then
// tell that its reads do not alias the X rows' DMA, and does not wait for
// that DMA before them): the codes (four groups of 16 rows j), the four
// waves' maxima, then a sink for the writes of columns past m (a lane's own
// 2 bytes plus the group offsets of its four writes).
constexpr int kMaxOff = 4 * kGroupPitch;
constexpr int kSinkOff = kMaxOff + 16;
constexpr int kAux = kSinkOff + 128 + 3 * kGroupPitch;

// MC: the dense factor's order when fixed at compile time (the 11008-wide
// input, m = 172: row offsets, code offsets and divisions by m / 2 become
// immediates), 0 to take it from m_arg.
template <int MC>
__global__ __launch_bounds__(64 * kWaves, 2) void rq_kron_kernel(
    const unsigned short *__restrict__ x, int64_t rows, int64_t ld_x, int m_arg, const float *__restrict__ dense,
    uint8_t *__restrict__ codes, float *__restrict__ scales, float scale_mul) {
  const int m = MC > 0 ? MC : m_arg;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRowBufs * kRowBuf];   // X rows
  __shared__ __attribute__((aligned(16))) uint8_t aux[kAux];
  float *const wmax = (float *)(aux + kMaxOff);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int g = lane >> 4;
  const int rowb = 128 * m;
  const int nchunks = rowb / 1024 + (rowb % 1024 != 0);
  const int code_bytes = 32 * m;
  const int half_m = m >> 1;

  // O's B-fragments (hi, lo) for N-tiles 3 wave .. 3 wave + 2, as in the
  // one-block kernel, pinned in AGPRs
  v8h ob[kNTW][kKS][2];
#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
    const int b = 16 * (kNTW * wave + t) + c16;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int a = 32 * ks + 8 * g + j;
        const bool in = a < m && b < m;
        const float o0 = dense[in ? a * m + b : 0];
        const float o = in ? o0 : 0.f;
        const _Float16 h = (_Float16)o;
        ob[t][ks][0][j] = h;
        ob[t][ks][1][j] = (_Float16)(o - (float)h);
      }
    // into AGPRs one N-tile at a time (loading all of O at once would need
    // more registers than the loop does)
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl) asm volatile("" : "+a"(ob[t][ks][hl]));
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int off = rowb + 16 * tid; off + 16 <= kRowBuf; off += 16 * 64 * kWaves) {
#pragma unroll
    for (int b = 0; b < kRowBufs; ++b) *(v4u *)(smem + b * kRowBuf + off) = v4u{0u, 0u, 0u, 0u};
  }

  int a_off[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) a_off[mt] = (32 * (mt >> 1) + 2 * c16 + (mt & 1)) * 2 * m;
  // Per-lane offsets of the code writes and stores are recomputed where
  // they are used (a few VALU ops per row): registers are the limit here.
  auto cw_off = [&](int t) __attribute__((always_inline)) {
    const int col = 16 * (kNTW * wave + t) + 4 * (c16 >> 2);
    return col < m ? (g | ((c16 & 3) << 2)) * half_m + (col >> 1) : kSinkOff + 2 * lane;
  };
  auto cs_chunk = [&](int pp) __attribute__((always_inline)) {
    const int nst = code_bytes / 16;
    const int ch = tid + 64 * kWaves * pp;
    return ch < nst ? ch : ch % nst;
  };

  // DMA of a row: wave-instruction q covers bytes 1024 (4 q + wave) .. +1023
  // (lanes past the end re-read the row's last 16 bytes, instructions past
  // the last chunk repeat it)
  const unsigned smem_lds = lds_addr(smem);
  auto issue_dma = [&](const uint8_t *src, int bsel, int q) __attribute__((always_inline)) {
    int chunk = q * kWaves + wave;
    chunk = chunk < nchunks ? chunk : nchunks - 1;
    const int off = 1024 * chunk + 16 * lane;
    dma16_to_lds(src + (off < rowb - 16 ? off : rowb - 16), smem_lds + (unsigned)(bsel * kRowBuf + 1024 * chunk));
  };

  const int stride = (int)gridDim.x;
  const int64_t row0 = blockIdx.x;   // the grid is no larger than rows
  const int nblk = __builtin_amdgcn_readfirstlane((int)((rows - row0 + stride - 1) / stride));
  const int64_t x_step = (int64_t)stride * ld_x * 2;
  const uint8_t *const x0 = (const uint8_t *)(x + row0 * ld_x);
  const uint8_t *const x_last = x0 + (int64_t)(nblk - 1) * x_step;
  auto row_src = [&](int kk) { return kk < nblk ? x0 + kk * x_step : x_last; };

#pragma unroll
  for (int q = 0; q < kKS; ++q) issue_dma(row_src(0), 0, q);
#pragma unroll
  for (int q = 0; q < kKS; ++q) issue_dma(row_src(1), 1, q);

  uint8_t *crow = codes + row0 * (int64_t)code_bytes;
  float *srow = scales + row0;
  const int64_t c_step = (int64_t)stride * code_bytes;
  // The codes of row r_{k-1}, staged in LDS at the end of step k - 1, are
  // stored after step k's first barrier (which every wave passes after
  // staging them): one barrier per row fewer.  Step k's own codes are staged
  // only after its absmax barrier, which every wave passes after reading
  // r_{k-1}'s from LDS.
  auto store_codes = [&](uint8_t *cr, float *sr, float smax) __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int ch = cs_chunk(pp);
      const int grp = ch / half_m, within = ch - grp * half_m;
      const v4u v = *(const v4u *)(aux + grp * kGroupPitch + 16 * within);
      *(v4u *)(cr + 16 * ch) = v;
    }
    if (tid == 0) *sr = smax * scale_mul;
  };
  float prev_mx = 0.f;
  int xb = 0, db = 2;
  for (int k = 0; k < nblk; ++k) {
    // the two blocks of a CU keep pace (two blocks per CU: the older one
    // otherwise finished ~19% of the launch ahead, the younger then alone)
    set_prio_by_progress(k);
    // Row r_k has landed.  Issued after its DMA (in step k - 2): the DMA of
    // r_{k+1} (kKS operations, in step k - 1) and, for k >= 2, the two code
    // stores of r_{k-2} per wave before it (the scale store of wave 0 only
    // adds).
    if (k < 2) wait_vm<kKS>();
    else wait_vm<kKS + 2>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();   // every wave's part of r_k is in; r_{k-1}'s buffer and codes are ready
    if (k > 0) store_codes(crow - c_step, srow - stride, prev_mx);
    const uint8_t *xbuf = smem + xb * kRowBuf;
    const uint8_t *nsrc = row_src(k + 2);

    // per k-step and pair of M-tiles: their A-fragments (8 registers), then
    // the six hi products and the six lo ones (an accumulator's two updates
    // are six MFMAs apart)
    v4f S[kMT][kNTW];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      issue_dma(nsrc, db, ks);
#pragma unroll
      for (int mp = 0; mp < kMT; mp += 2) {
        v8h acur[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint8_t *pa = xbuf + a_off[mp + u] + 16 * g + 64 * ks;
          const v2u lo = *(const v2u *)pa;
          const v2u hi = *(const v2u *)(pa + 8);
          acur[u] = __builtin_bit_cast(v8h, v4u{lo[0], lo[1], hi[0], hi[1]});
        }
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
          for (int t = 0; t < kNTW; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int mt = mp + u;
              if (ks == 0 && hl == 0)
                S[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(acur[u], ob[t][ks][hl], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
              else
                S[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(acur[u], ob[t][ks][hl], S[mt][t], 0, 0, 0);
            }
      }
    }

    // 64-point Walsh-Hadamard over i, absmax (register layout as in the
    // one-block kernel)
    float mx = 0.f;
#pragma unroll
    for (int t = 0; t < kNTW; ++t) {
#pragma unroll
      for (int mb = 1; mb <= 2; mb <<= 1)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          if (mt & mb) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float u = S[mt][t][r], v = S[mt | mb][t][r];
            S[mt][t][r] = u + v;
            S[mt | mb][t][r] = u - v;
          }
        }
#pragma unroll
      for (int rb = 1; rb <= 2; rb <<= 1)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (r & rb) continue;
            const float u = S[mt][t][r], v = S[mt][t][r | rb];
            S[mt][t][r] = u + v;
            S[mt][t][r | rb] = u - v;
          }
#pragma unroll
      for (int mt = 0; mt < kMT; mt += 2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float u = S[mt][t][r], v = S[mt + 1][t][r];
          swap16(u, v);
          S[mt][t][r] = u + v;
          S[mt + 1][t][r] = u - v;
        }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          float u = S[mt][t][r], v = S[mt][t][r + 1];
          swap32(u, v);
          S[mt][t][r] = u + v;
          S[mt][t][r + 1] = u - v;
        }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(S[mt][t][r]));
    }
    mx = wave_max_dpp(mx);
    if (lane == 0) wmax[wave] = mx;
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float inv = mx > 0.f ? 7.0f / mx : 0.f;

    // codes: eight per word, 4 x 4 nibble transpose in lane quads, staged
    // in LDS in output order
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
            acc = __builtin_amdgcn_alignbit(round_bits(S[mt][t][r], inv), acc, 4);
          }
        const unsigned perm_sel = (lane & 2) ? 0x03070105u : 0x06020400u;
        const unsigned rot_sh = (lane & 1) ? 4u : 28u;
        const unsigned keep = (lane & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
        unsigned v = acc;
        v = __builtin_amdgcn_perm(dpp<kQuadXor2>(v), v, perm_sel);
        const unsigned o = dpp<kQuadXor1>(v);
        const unsigned sh = __builtin_amdgcn_alignbit(o, o, rot_sh);
        v = (keep & v) | (~keep & sh);
        const int cw = cw_off(t);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *(unsigned short *)(aux + cw + (2 * R + h) * kGroupPitch) = (unsigned short)(v >> (16 * h));
      }
    // every wave has read the maxima before the next row's first barrier,
    // and writes the next maxima only after it
    prev_mx = mx;
    crow += c_step;
    srow += stride;
    xb = xb == kRowBufs - 1 ? 0 : xb + 1;
    db = db == kRowBufs - 1 ? 0 : db + 1;
  }
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();   // the last row's codes are staged
  store_codes(crow - c_step, srow - stride, prev_mx);
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
  const int cus = device_cu_count();
  const float scale_mul = (float)(1.0 / (7.0 * 8.0));   // 1/(7 sqrt(64))
  const int64_t grid = rows < 2 * cus ? rows : 2 * cus;   // two blocks per CU
  if (r.dense_m == 172)
    rq_kron_kernel<172><<<dim3((unsigned)grid), dim3(64 * kWaves), 0, stream>>>(
        (const unsigned short *)x, rows, ld_x, r.dense_m, r.dense, codes, scales, scale_mul);
  else
    rq_kron_kernel<0><<<dim3((unsigned)grid), dim3(64 * kWaves), 0, stream>>>(
        (const unsigned short *)x, rows, ld_x, r.dense_m, r.dense, codes, scales, scale_mul);
  return hipGetLastError();
}

}  // namespace qr
