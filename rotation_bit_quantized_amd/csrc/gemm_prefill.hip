// 4-bit (and 8-bit) integer GEMM for prefill shapes (M > 64):
// y = dequant(qa . qw^T).
//
// Method: QuaRot abstract (all matrix multiplications in 4 bits);
// dequantizing epilogue y = acc * s_x * s_w per output channel, or the sum
// over K-groups of acc_g * s_x[g] * s_w[g] (QuaRot summary, "Key points":
// group size 128).
//
// CDNA4 has no 4-bit integer MFMA, so codes are widened to int8 in
// registers right after they are read from LDS, in "high-nibble" form:
//   lo = (w << 4) & 0xF0F0F0F0,  hi = w & 0xF0F0F0F0
// turns 8 packed codes into 8 int8 values 16*q (exact for q in [-8, 7]) in
// three VALU ops.  A and W are widened identically, so the product sums
// 256 * q_a * q_w; the k order inside a dword is permuted the same way on
// both sides and cancels.  |acc| <= 64 * 256 * K < 2^31 for K < 2^17 (the
// host rejects larger K).
// The 1/256 is an exact power of two folded into the epilogue (or a shift
// for the int32 output).
//
// Data movement: block tile BM x BN, K-tile 256 codes = 128 bytes per row,
// i.e. one whole 128-byte cache line per row and K-tile (half-line rows
// halve the L2 -> LDS fill rate of a CU).  K-tiles travel from global memory
// straight into LDS with global_load_lds_dwordx4 (no VGPR staging) through
// STAGES LDS buffers.  A DMA wave instruction fills 1 KB of LDS contiguously
// (lane i -> bytes 16i..16i+15), i.e. 8 rows x eight 16-byte pieces; each
// lane fetches the global piece swz(row, slot), so that the fragment reads
// (16 consecutive rows at one piece) hit 16 distinct bank groups.
//
// The K loop is software-pipelined over 64-code chunks (one 16-byte LDS read
// per fragment row and lane, two MFMA k-steps after widening): the read of
// chunk c+1 is in flight while chunk c is multiplied.  Once per K-tile, a
// wave waits (vmcnt, its own DMA pieces only) for the next tile and meets
// the other waves at one s_barrier, which makes that tile visible and
// certifies that every wave holds the current tile's last chunk in
// registers, so the current buffer is refilled at once.  When K is an odd
// multiple of 128 the last K-tile carries 128 codes (two chunks); its DMA
// lanes for the missing half re-read the present half.
//
// Compute: each wave owns a WM x WN sub-tile of 32x32 fragments of
// v_mfma_i32_32x32x32_i8, so each widened operand feeds FN (or FM) MFMAs.
// The host picks the block shape whose tile count fills the CU slots best.
//
// Tiles: the 256 x 192 shape with per-channel scales runs persistent blocks
// (one per CU, each looping over every gridDim-th tile); the next tile's
// output scales and first two K-tiles are fetched while the current tile's
// epilogue runs.  The other shapes run one block per tile.
//
// 8-bit codes (the 6- and 8-bit RTN variants; QuaRot abstract: lossless 6-
// and 8-bit RTN): the same kernel with CB = 8.  A K-tile is still 128 bytes
// per row, now 128 codes; a 16-byte fragment read is one MFMA k-step used as
// is (no widening, no 1/256).
#include "qr_common.h"
#include "qr_launch.h"

#include <type_traits>

namespace qr {
namespace {

constexpr int kRowBytes = 128;   // bytes per row per K-tile (256 4-bit or 128 8-bit codes)

// LDS slot of 16-byte piece p (0..7) of tile row r (an involution in p).
// Rows are 128 bytes, so rows 2t and 2t+1 share a 256-byte bank window;
// xoring with t spreads 16 consecutive rows over all 16 slots of the window.
__device__ __forceinline__ int swz(int r, int p) { return p ^ ((r >> 1) & 7); }

// A compile-time range [LO, HI) of DMA wave-instructions.
template <int LO, int HI>
struct DmaRange {
  static constexpr int lo = LO, hi = HI;
};
using NoDma = DmaRange<0, 0>;

// Map the linear block id to a (tile_m, tile_n): consecutive hardware block
// ids go to different XCDs (round robin over 8), so first regroup them so
// that each XCD receives a contiguous range of logical tiles, then walk
// the logical range in column-major bands of kGroupM row-tiles so that the
// tiles running together on one XCD share A rows and W rows in its L2.
__device__ __forceinline__ void tile_of(int bid, int tm_count, int tn_count, int &tm, int &tn) {
  constexpr int kXcd = 8;
  constexpr int kGroupM = 8;
  const int total = tm_count * tn_count;
  const int full = total / kXcd * kXcd;
  int id = bid;
  if (bid < full) id = (bid % kXcd) * (full / kXcd) + bid / kXcd;
  const int band = kGroupM * tn_count;
  const int first_m = (id / band) * kGroupM;
  const int gm = min(tm_count - first_m, kGroupM);
  const int in_band = id % band;
  tm = first_m + in_band % gm;
  tn = in_band / gm;
}

constexpr bool persistent_shape(int bm, bool grouped) { return bm == 256 && !grouped; }

// OCC waves per SIMD: blocks of 4 waves run OCC to a CU, blocks of 8 waves
// OCC/2.  At OCC 1 a wave has the whole register file (AGPR accumulators).
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool GROUPED, bool OUT_I32, bool SHORT_TAIL,
          int OCC = 2, int CB = 4>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, OCC * 4 / (WAVES_M * WAVES_N)) void gemm_prefill_kernel(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ W,
    const float *__restrict__ sw, int M, int N, int K, int group, void *__restrict__ out, int64_t ld_y) {
  static_assert(CB == 4 || CB == 8, "code width");
  constexpr int kBK = CB == 4 ? 256 : 128;        // codes per K-tile
  constexpr int kHalfCodes = kBK / 2;             // a group spans whole halves of a K-tile
  constexpr int KS = CB == 4 ? 2 : 1;             // MFMA k-steps per 16-byte fragment read
  constexpr int SHIFT = CB == 4 ? 8 : 0;          // widened 4-bit products carry 16 * 16
  constexpr float UNSCALE = CB == 4 ? 1.0f / 256.0f : 1.0f;
  static_assert(CB == 4 || !SHORT_TAIL, "8-bit K-tiles are whole");
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int ROWS = BM + BN;
  constexpr bool SCALES = GROUPED && !OUT_I32;   // group scales travel with the K-tiles
  // one scale set (s_x of the BM rows, then s_w of the BN columns) per K-tile half
  constexpr int SCALE_BYTES = SCALES ? 2 * ROWS * 4 : 0;
  constexpr int SCALE_INST = SCALES ? 2 * ROWS / 64 : 0;   // 4-byte DMA wave-instructions per stage
  constexpr int STAGE_BYTES = ROWS * kRowBytes;
  // the scales live in a ring of three slots after the stages (K-tile kt in
  // slot kt % 3): the refill of tile kt+2 then never touches the scales of
  // tiles kt and kt+1, which group epilogues may still read
  constexpr int SCALE_SLOTS = SCALES ? 3 : 0;
  static_assert(!SCALES || (ROWS % 32 == 0 && SCALE_INST % NW == 0), "scale DMA split");
  constexpr int SCALE_LOADS = SCALE_INST / NW;
  constexpr int TI = ROWS / 8;                    // DMA wave-instructions per stage (8 rows each)
  constexpr int LOADS = TI / NW;                  // per wave
  static_assert(TI % NW == 0, "tile rows must split evenly over the waves' DMA instructions");
  static_assert(NW % 2 == 0, "the upper-piece rule below assumes an even wave count");
  constexpr int WAVE_LOADS = LOADS + SCALE_LOADS;  // vmem ops per wave per stage
  static_assert(STAGES >= 2 && STAGES <= 3, "pipeline depth");
  static_assert(WAVE_LOADS * (STAGES - 1) < 64, "vmcnt range");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");

  // Per-channel fp16 output: the tile's output scales (s_x of the BM rows,
  // then s_w of the BN columns) travel by DMA into LDS at the start, so that
  // the epilogue does not wait a memory round trip for them; only where the
  // 4 bytes per row still let the CU hold as many blocks.
  constexpr int BLOCKS_PER_CU = OCC * 4 / NW;
  // Persistent blocks for the 256-row shape with per-channel scales; the
  // others keep one block per tile (a loop over tiles would push them past
  // the register file).
  constexpr bool PERSIST = persistent_shape(BM, GROUPED);
  // Two slots, so that the next tile's scales can arrive during this
  // tile's epilogue.
  constexpr bool OSC = !GROUPED && !OUT_I32 &&
                       (STAGES * STAGE_BYTES + 2 * ROWS * 4) * BLOCKS_PER_CU <= 160 * 1024;
  constexpr int OSC_INST = OSC ? ROWS / 64 : 0;   // 4-byte DMA wave-instructions
  static_assert(!OSC || (ROWS % 64 == 0 && OSC_INST <= NW), "output scale DMA split");
  __shared__ __attribute__((aligned(1024))) uint8_t
      smem[STAGES * STAGE_BYTES + SCALE_SLOTS * SCALE_BYTES + (OSC ? 2 * ROWS * 4 : 0)];
  uint8_t *const scale_ring = smem + STAGES * STAGE_BYTES;
  float *const osc_base = (float *)(smem + STAGES * STAGE_BYTES + SCALE_SLOTS * SCALE_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index in an SGPR: everything derived from it (DMA counts, the
  // vmcnt thresholds) is then provably wave-uniform and stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int tm_count = (M + BM - 1) / BM;
  const int tn_count = (N + BN - 1) / BN;
  const int tiles = tm_count * tn_count;
  const int64_t kbytes = (int64_t)K * CB / 8;
  const int KT = (K + kBK - 1) / kBK;
  // SHORT_TAIL: K is an odd multiple of 128, the last K-tile holds 128 codes
  const int halves_per_group = GROUPED ? group / kHalfCodes : 1;

  // DMA sources: wave-instruction q of this wave fills tile rows
  // 8 (NW q + wave) .. +7 (A rows first, then W rows); lane l writes LDS
  // slot l % 8 of row l / 8 with global piece swz(row, l % 8).  Rows past
  // the matrix edge re-read the last row; their results are never stored.
  // Whether an instruction reads A or W is uniform; the per-lane part is a
  // 32-bit offset from the block's first row.
  // The DMA state describes the tile whose K-tiles the DMA instructions
  // fetch: the current one during its K loop, the next one from the end of
  // the K loop on (its first two K-tiles and output scales arrive during the
  // current tile's epilogue).  m0, n0 stay the current tile's.
  int dm0, dn0;
  const uint8_t *a_base, *w_base;
  uint32_t src_off[LOADS];
  auto set_dma_tile = [&](int bid) __attribute__((always_inline)) {
    int tm, tn;
    tile_of(bid, tm_count, tn_count, tm, tn);
    dm0 = tm * BM;
    dn0 = tn * BN;
    a_base = A + (int64_t)dm0 * kbytes;
    w_base = W + (int64_t)dn0 * kbytes;
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      const int trow = 8 * (NW * q + wave) + (lane >> 3);   // 0 .. ROWS-1
      const int piece = swz(trow, lane & 7);
      const int rel = trow < BM ? min(trow, M - 1 - dm0) : min(trow - BM, N - 1 - dn0);
      src_off[q] = (uint32_t)rel * (uint32_t)kbytes + (uint32_t)(piece * 16);
    }
  };
  int bid = blockIdx.x;
  set_dma_tile(bid);
  int m0 = dm0, n0 = dn0;
  // Whether this lane's global piece lies in the upper half of the row
  // (piece >= 4): with trow = 8 X + (lane >> 3), (trow >> 1) & 7 equals
  // 4 (X & 1) + (lane >> 4), and X = NW q + wave has the parity of wave, so
  // bit 2 of the piece is bit 2 of lane xor bit 0 of wave, for every q.
  const int upper_piece = ((lane >> 2) ^ wave) & 1;
  const uint32_t tail_back = upper_piece ? 64u : 0u;   // a short last tile re-reads the lower half

  // DMA wave-instruction q of K-tile kt into `stage` (the group scales go
  // with the last one).
  auto issue_q = [&](int kt, int stage, int q) __attribute__((always_inline)) {
    const bool short_tile = SHORT_TAIL && kt == KT - 1;
    const bool in_a = 8 * (NW * q + wave) < BM;
    const uint8_t *base = (in_a ? a_base : w_base) + kt * kRowBytes;
    const uint32_t o = short_tile ? src_off[q] - tail_back : src_off[q];
    __builtin_amdgcn_global_load_lds((const void *)(base + o),
                                     (lds_void *)(smem + stage * STAGE_BYTES + (NW * q + wave) * 1024), 16, 0, 0);
    if constexpr (SCALES) {
      if (q == LOADS - 1) {
        const int G = K / group;
#pragma unroll
        for (int qs = 0; qs < SCALE_LOADS; ++qs) {
          const int e = 64 * (NW * qs + wave) + lane;   // 0 .. 2 ROWS - 1
          const int h = e >= ROWS;
          const int ee = e - h * ROWS;
          const int gidx = min((kt * kBK + h * kHalfCodes) / group, G - 1);
          const float *p = ee < BM ? sa + (int64_t)min(dm0 + ee, M - 1) * G + gidx
                                   : sw + (int64_t)min(dn0 + ee - BM, N - 1) * G + gidx;
          __builtin_amdgcn_global_load_lds((const void *)p,
                                           (lds_void *)(scale_ring + (kt % 3) * SCALE_BYTES +
                                                        256 * (NW * qs + wave)),
                                           4, 0, 0);
        }
      }
    }
  };
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) issue_q(kt, stage, q);
  };
  // the DMA tile's output scales into slot `slot` (before its K-tiles, so
  // that the wait for its first K-tile covers them)
  auto issue_osc = [&](int slot) __attribute__((always_inline)) {
    if constexpr (OSC) {
      if (wave < OSC_INST) {
        const int e = 64 * wave + lane;
        const float *p = e < BM ? sa + min(dm0 + e, M - 1) : sw + min(dn0 + e - BM, N - 1);
        __builtin_amdgcn_global_load_lds((const void *)p, (lds_void *)(osc_base + slot * ROWS + 64 * wave), 4, 0,
                                         0);
      }
    }
  };

  v16i acc[FM][FN];
  v16f facc[GROUPED ? FM : 1][GROUPED ? FN : 1];

  // Lane-dependent offsets, set again at the start of every tile from an
  // opaque copy of the lane index: otherwise the compiler hoists everything
  // derived from them (every LDS and output address of the epilogue) out of
  // the tile loop and keeps it live through the K loop, which spills.
  int lrow, lcol, ra, rb, half;
  auto set_lane_offsets = [&]() __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    lrow = 4 * (l >> 5);            // output row offset within a fragment: + 8*(r/4) + r%4
    lcol = l & 31;
    ra = wm * WM + (l & 31);        // tile row of this lane in A fragment 0
    rb = BM + wn * WN + (l & 31);   // tile row of this lane in W fragment 0
    half = l >> 5;                  // which 16-byte piece of a 32-byte chunk
  };

  // Chunk pipeline registers: the raw codes of two chunks (LDS -> VGPR, one
  // read in flight while the other is widened) and the widened operands of
  // two chunks (the one being multiplied, the next one being widened).
  v4u rawA[2][FM], rawB[2][FN];        // [buffer][fragment]
  v4i opA[2][FM][2], opB[2][FN][2];   // [buffer][fragment][k-step]

  // Raw fragment reads of chunk `kk` (codes 64 kk .. 64 kk + 63) of the
  // K-tile in `st` into raw buffer `rb_`.
  auto read_raw = [&](const uint8_t *st, int kk, int rbuf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = ra + 32 * i;
      rawA[rbuf][i] = *(const v4u *)(st + r * kRowBytes + swz(r, 2 * kk + half) * 16);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = rb + 32 * j;
      rawB[rbuf][j] = *(const v4u *)(st + r * kRowBytes + swz(r, 2 * kk + half) * 16);
    }
  };
  auto widen_into = [&](int rbuf, int obuf) __attribute__((always_inline)) {
    if constexpr (CB == 4) {
#pragma unroll
      for (int i = 0; i < FM; ++i) widen_hi_nibble(rawA[rbuf][i], opA[obuf][i][0], opA[obuf][i][1]);
#pragma unroll
      for (int j = 0; j < FN; ++j) widen_hi_nibble(rawB[rbuf][j], opB[obuf][j][0], opB[obuf][j][1]);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) opA[obuf][i][0] = __builtin_bit_cast(v4i, rawA[rbuf][i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) opB[obuf][j][0] = __builtin_bit_cast(v4i, rawB[rbuf][j]);
    }
  };
  // The MFMAs of the chunk in operand buffer `obuf` (two k-steps); with
  // ZERO the first k-step starts from zero (a new K-group).  DMA
  // instructions [Q_LO, Q_HI) of K-tile dkt (into dstage) are issued one
  // after each MFMA: issued as a burst, they would hold up the wave at the
  // memory pipeline while the matrix core idles.
  auto mma_chunk = [&](int obuf, auto zero_c, auto dma_c, int dkt, int dstage) __attribute__((always_inline)) {
    constexpr bool ZERO = decltype(zero_c)::value;
    constexpr int Q_LO = decltype(dma_c)::lo, Q_HI = decltype(dma_c)::hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (ZERO && ks == 0)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(opA[obuf][i][ks], opB[obuf][j][ks], v16i{}, 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(opA[obuf][i][ks], opB[obuf][j][ks], acc[i][j], 0, 0, 0);
          // DMA instructions spaced evenly over the chunk's MFMAs: after
          // MFMA idx when idx is a multiple of the spacing
          constexpr int NMF = KS * FM * FN, ND = Q_HI - Q_LO;
          constexpr int SP = ND > 0 && NMF / (ND > 0 ? ND : 1) > 0 ? NMF / (ND > 0 ? ND : 1) : 1;
          const int idx = (ks * FM + i) * FN + j;
          if (idx % SP == 0 && idx / SP < ND) issue_q(dkt, dstage, Q_LO + idx / SP);
        }
  };
  // Multiply operand buffer `obuf` and, interleaved with it, widen raw
  // buffer `rbuf` into the other operand buffer (when `do_widen`) and issue
  // the DMA instructions of dma_c.
  auto compute = [&](int obuf, int rbuf, bool zero, auto widen_c, auto dma_c, int dkt,
                     int dstage) __attribute__((always_inline)) {
    constexpr bool DO_WIDEN = decltype(widen_c)::value;
    constexpr int ND = decltype(dma_c)::hi - decltype(dma_c)::lo;
    constexpr int NMFMA = KS * FM * FN;
    constexpr int NVALU = DO_WIDEN && CB == 4 ? 12 * (FM + FN) : 0;
    constexpr int VPM = (NVALU + NMFMA - 1) / NMFMA;
    if (GROUPED && zero) {
      mma_chunk(obuf, std::true_type{}, dma_c, dkt, dstage);
    } else {
      mma_chunk(obuf, std::false_type{}, dma_c, dkt, dstage);
    }
    if constexpr (DO_WIDEN) widen_into(rbuf, 1 - obuf);
    // order: MFMAs with the DMA instructions spread evenly between them and
    // the widening VALU work shared out
    constexpr int SP = ND > 0 && NMFMA / (ND > 0 ? ND : 1) > 0 ? NMFMA / (ND > 0 ? ND : 1) : 1;
#pragma unroll
    for (int k = 0; k < NMFMA; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (k % SP == 0 && k / SP < ND) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      if (VPM > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    }
  };
  // Wait until this wave's DMA pieces of a tile have landed; `issued_after`
  // tiles issued later may stay in flight (scalar branches: uniform).
  auto wait_tile = [&](int issued_after) __attribute__((always_inline)) {
    if (issued_after >= 2) wait_vm<2 * WAVE_LOADS>();
    else if (issued_after == 1) wait_vm<WAVE_LOADS>();
    else wait_vm<0>();
  };

  // Group scales of K-tile half h, from the stage at `st`, into registers
  // (s_w pre-multiplied by the 1/256 of the widening).
  v4f gsa[SCALES ? FM : 1][4];
  float gsw[SCALES ? FN : 1];
  auto read_scales = [&](int kt, int h) __attribute__((always_inline)) {
    const float *sc = (const float *)(scale_ring + (kt % 3) * SCALE_BYTES) + h * ROWS;
#pragma unroll
    for (int j = 0; j < FN; ++j) gsw[j] = sc[BM + wn * WN + j * 32 + lcol] * UNSCALE;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) gsa[i][r4] = *(const v4f *)(sc + wm * WM + i * 32 + 8 * r4 + lrow);
  };
  // A K-group ends with half h of K-tile kt: fold or store its partial sums.
  auto group_end = [&](int kt, int h) __attribute__((always_inline)) {
    if constexpr (OUT_I32) {
      const int gidx = (kt * kBK + h * kHalfCodes) / group;
      int32_t *o = (int32_t *)out + (int64_t)gidx * M * N;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WN + j * 32 + lcol;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + lrow + (r & 3);
            if (row < M && col < N) o[(int64_t)row * N + col] = acc[i][j][r] >> SHIFT;
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              facc[i][j][4 * r4 + r] =
                  __builtin_fmaf((float)acc[i][j][4 * r4 + r], gsa[i][r4][r] * gsw[j], facc[i][j][4 * r4 + r]);
    }
  };
  // Chunk boundary: the raw read issued a chunk ago must have landed (the
  // wait is fenced so that nothing is scheduled across it).
  auto chunk_fence = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();
    __builtin_amdgcn_sched_barrier(0);
  };

  // One K-tile.  On entry chunk 0 is widened in operand buffer 0 and the
  // raw read of chunk 1 (raw buffer 1) is in flight.  Each chunk: wait for
  // the raw read issued a chunk ago, issue the raw read of the chunk after
  // next into the free raw buffer, then multiply while widening the next
  // chunk into the other operand buffer.  Reads are pinned in place (the
  // scheduler would otherwise sink them next to their use).  At chunk 2 the
  // waves meet at the tile barrier: every wave then holds this tile's last
  // raw chunk, so its LDS buffer is refilled at once, and the next tile
  // (waited for just before) becomes readable.  Mode kNext: a tile followed
  // by another; kLastFull: the last tile, 256 codes; kLastShort: the last
  // tile, 128 codes.
  // The DMA of K-tile kt+2 goes into this tile's buffer, free after the
  // chunk-2 barrier: about a third of it interleaved with the MFMAs of chunk
  // 2, the rest with those of chunk 3; it is waited for at chunk 2 of tile
  // kt+1.  Chunk 2 follows the barrier, where the waves of a SIMD are closest
  // together and compete hardest for issue slots: with half of the DMA there
  // the launch took 1-3% longer.
  // Wave priority falls chunk by chunk from the barrier on (3 for chunk 2,
  // then 2, 1, 0): the two waves of a SIMD share its issue slots, and the
  // older one wins every tie, so without this it finished each barrier
  // interval well ahead and idled at the barrier while the younger ran
  // alone (~1650 against ~300 cycles of wait per K-tile at 256 x 192).  A
  // wave that is a chunk ahead now yields to the one behind it.
  constexpr int kNext = 0, kNextNoDma = 1, kLastFull = 2, kLastShort = 3;
  constexpr int Q1 = LOADS / 3 > LOADS - KS * FM * FN ? LOADS / 3 : LOADS - KS * FM * FN;
  static_assert(STAGES == 2, "the refill schedule assumes two stages");
  static_assert(Q1 <= KS * FM * FN && LOADS - Q1 <= KS * FM * FN, "one DMA instruction per MFMA at most");
  auto tile = [&](int kt, auto mode_c) __attribute__((always_inline)) {
    constexpr int mode = decltype(mode_c)::value;
    constexpr bool NEXT = mode == kNext || mode == kNextNoDma;
    const uint8_t *st = smem + (kt % STAGES) * STAGE_BYTES;
    const uint8_t *nst = smem + ((kt + 1) % STAGES) * STAGE_BYTES;
    // groups are whole halves: one can start with half 0 or half 1 and end with either
    const bool start0 = GROUPED && ((2 * kt) % halves_per_group == 0);
    const bool start1 = GROUPED && ((2 * kt + 1) % halves_per_group == 0);
    const bool end1 = GROUPED && ((2 * kt + 2) % halves_per_group == 0);
    const int dkt = kt + STAGES, dstage = kt % STAGES;   // the tile refilled into this tile's buffer

    if constexpr (mode == kLastShort) {
      chunk_fence();
      compute(0, 1, start0, std::true_type{}, NoDma{}, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      compute(1, 0, false, std::false_type{}, NoDma{}, 0, 0);
      if constexpr (GROUPED) {   // the last half ends the last group
        if constexpr (SCALES) read_scales(kt, 0);
        group_end(kt, 0);
      }
      return;
    } else {
      // chunk 0
      chunk_fence();
      __builtin_amdgcn_s_setprio(1);
      read_raw(st, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      compute(0, 1, start0, std::true_type{}, NoDma{}, 0, 0);
      // chunk 1
      chunk_fence();
      __builtin_amdgcn_s_setprio(0);
      read_raw(st, 3, 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(1, 0, false, std::true_type{}, NoDma{}, 0, 0);
      if constexpr (GROUPED) {
        if (start1) {   // half 0 closes a group
          if constexpr (SCALES) read_scales(kt, 0);
          group_end(kt, 0);
        }
      }
      // chunk 2
      chunk_fence();
      if constexpr (NEXT) {
        wait_vm<0>();   // tile kt+1 has landed
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        read_raw(nst, 0, 0);
      }
      __builtin_amdgcn_s_setprio(3);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (mode == kNext)
        compute(0, 1, start1, std::true_type{}, DmaRange<0, Q1>{}, dkt, dstage);
      else
        compute(0, 1, start1, std::true_type{}, NoDma{}, 0, 0);
      // chunk 3
      if constexpr (NEXT) {
        chunk_fence();
        __builtin_amdgcn_s_setprio(2);
        read_raw(nst, 1, 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (mode == kNext)
          compute(1, 0, false, std::true_type{}, DmaRange<Q1, LOADS>{}, dkt, dstage);
        else
          compute(1, 0, false, std::true_type{}, NoDma{}, 0, 0);
      } else {
        __builtin_amdgcn_sched_barrier(0);
        compute(1, 0, false, std::false_type{}, NoDma{}, 0, 0);
      }
      if constexpr (GROUPED) {
        if (end1) {
          if constexpr (SCALES) read_scales(kt, 1);
          group_end(kt, 1);
        }
      }
    }
  };

  // Persistent blocks (PERSIST): block b takes the tiles b, b + gridDim.x,
  // ... (the grid is a multiple of 8, so every tile keeps the XCD that
  // tile_of gave it).  The first tile's scales and K-tiles 0, 1 go out here;
  // each later tile's during its predecessor's epilogue.  Otherwise one
  // block per tile.
  issue_osc(0);
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < KT) issue(s, s);

  for (int iter = 0;; ++iter) {
    const int nbid = bid + (int)gridDim.x;
    const bool has_next = PERSIST && nbid < tiles;   // uniform over the block
    set_lane_offsets();

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v16i{};
    if constexpr (GROUPED) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) facc[i][j] = v16f{};
    }

    // K-tile 0 has landed (for a later tile: issued after it are K-tile 1
    // and the previous tile's output stores, so waiting until at most one
    // stage's DMA count is outstanding implies it, loads returning in order)
    wait_tile(min(STAGES - 1, KT - 1));
    __builtin_amdgcn_s_barrier();
    read_raw(smem, 0, 0);
    wait_lgkm0();
    widen_into(0, 0);
    read_raw(smem, 1, 1);
    __builtin_amdgcn_sched_barrier(0);

    // Tiles followed by another (refilling their buffer while one remains),
    // then the last tile, peeled.
    int kt = 0;
    for (; kt + STAGES < KT; ++kt) tile(kt, std::integral_constant<int, kNext>{});
    for (; kt + 1 < KT; ++kt) tile(kt, std::integral_constant<int, kNextNoDma>{});
    if constexpr (SHORT_TAIL)
      tile(KT - 1, std::integral_constant<int, kLastShort>{});
    else
      tile(KT - 1, std::integral_constant<int, kLastFull>{});
    __builtin_amdgcn_sched_barrier(0);   // keep the epilogue out of the last MFMAs

    // every wave is done with the stage buffers and the scale ring
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    // ---- epilogue, with the next tile's first K-tiles on their way
    if constexpr (OUT_I32) {
      if (has_next) {
        set_dma_tile(nbid);
#pragma unroll
        for (int s = 0; s < STAGES; ++s)
          if (s < KT) issue(s, s);
      }
      if constexpr (!GROUPED) {
        int32_t *o = (int32_t *)out;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WN + j * 32 + lcol;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + lrow + (r & 3);
              if (row < M && col < N) o[(int64_t)row * N + col] = acc[i][j][r] >> SHIFT;
            }
          }
      }
    } else {
      // fp16 output, staged through LDS: each wave writes 32 rows of its
      // WM x WN tile at a time row-major into a private region of stage
      // buffer 1, reads them back and stores whole 16-byte row pieces
      // (2-byte stores straight from the fragment layout, one column per
      // lane, would take 8x the store instructions).  The next tile's K-tile
      // 0 goes into buffer 0 at once, its K-tile 1 into buffer 1 after the
      // staging.
      constexpr int PITCH = WN * 2 + 16;   // bytes per LDS row; the pad spreads the two half-waves' banks
      constexpr int HROWS = 32;            // rows staged at a time: one fragment row
      static_assert(NW * HROWS * PITCH <= STAGE_BYTES, "epilogue staging must fit in one stage buffer");
      static_assert((HROWS * (WN / 8)) % 64 == 0, "whole wave passes over the output pieces");
      static_assert(STAGES == 2, "staging in buffer 1 while buffer 0 takes the next tile");
      unsigned short *y = (unsigned short *)out;
      // Output scales: from LDS (OSC), or every load issued at once from
      // clamped (always valid) indices so that one memory latency covers
      // them; rows or columns past the edge are never stored.
      float swv[FN], sav[GROUPED ? 1 : FM][16];
      if constexpr (OSC) {
        const float *osc = osc_base + (iter & 1) * ROWS;
#pragma unroll
        for (int j = 0; j < FN; ++j) swv[j] = osc[BM + wn * WN + j * 32 + lcol] * UNSCALE;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const v4f v = *(const v4f *)(osc + wm * WM + i * 32 + 8 * r4 + lrow);
#pragma unroll
            for (int r = 0; r < 4; ++r) sav[i][4 * r4 + r] = v[r];
          }
      } else if constexpr (!GROUPED) {
#pragma unroll
        for (int j = 0; j < FN; ++j) swv[j] = sw[min(n0 + wn * WN + j * 32 + lcol, N - 1)] * UNSCALE;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sav[i][r] = sa[min(m0 + wm * WM + i * 32 + 8 * (r >> 2) + lrow + (r & 3), M - 1)];
      }
      if (has_next) {
        set_dma_tile(nbid);
        issue_osc((iter + 1) & 1);
        issue(0, 0);
      }
      uint8_t *ot = smem + STAGE_BYTES + wave * HROWS * PITCH;
      constexpr int PIECES = WN / 8;   // 16-byte pieces per row
      constexpr int PASSES = HROWS * PIECES / 64;
      const bool vec_ok = ((uintptr_t)y % 16 == 0) && (ld_y % 8 == 0);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int trow = 8 * (r >> 2) + lrow + (r & 3);   // row within the 32 staged rows
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            float val;
            if constexpr (GROUPED)
              val = facc[i][j][r];
            else
              val = (float)acc[i][j][r] * (sav[i][r] * swv[j]);
            *(unsigned short *)(ot + trow * PITCH + (j * 32 + lcol) * 2) = float_to_half_bits(val);
          }
        }
        // the wave reads back only what it wrote itself (LDS operations of
        // one wave complete in order), before it overwrites the region
        v4u pv[PASSES];   // all reads first, then the (edge-guarded) stores
#pragma unroll
        for (int it = 0; it < PASSES; ++it) {
          const int p = it * 64 + lane;
          pv[it] = *(const v4u *)(ot + (p / PIECES) * PITCH + (p % PIECES) * 16);
        }
#pragma unroll
        for (int it = 0; it < PASSES; ++it) {
          const int p = it * 64 + lane;
          const int trow = p / PIECES, cp = p % PIECES;
          const int row = m0 + wm * WM + i * HROWS + trow;
          const int col = n0 + wn * WN + cp * 8;
          const v4u v = pv[it];
          if (row < M) {
            unsigned short *dst = y + (int64_t)row * ld_y + col;
            if (vec_ok && col + 8 <= N) {
              *(v4u *)dst = v;
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (col + e < N) dst[e] = (unsigned short)(v[e >> 1] >> (16 * (e & 1)));
            }
          }
        }
      }
      // K-tile 1 of the next tile: once every wave has read its staged rows
      // back (its loads then follow this tile's stores, which the next
      // tile's first wait does not need to cover)
      if (has_next && KT > 1) {
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        issue(1, 1);
      }
    }
    if (!has_next) break;
    bid = nbid;
    m0 = dm0;
    n0 = dn0;
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool GROUPED, int CB, int OCC = 2>
hipError_t launch_cfg(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw, int64_t M,
                      int64_t N, int64_t K, int group, void *y, int64_t ld_y, bool out_i32,
                      hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  // persistent shapes: as many blocks as are resident at once (a multiple
  // of 8, the XCD count); otherwise one per tile
  const int64_t resident = (int64_t)device_cu_count() * (OCC * 4 / (WAVES_M * WAVES_N)) / 8 * 8;
  const int64_t nblocks = persistent_shape(BM, GROUPED) && resident >= 8 && tiles > resident ? resident : tiles;
  dim3 grid((unsigned)nblocks), block(64 * WAVES_M * WAVES_N);
#define QR_GEMM_LAUNCH(I32, TAIL)                                                                \
  gemm_prefill_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, GROUPED, I32, TAIL, OCC, CB><<<grid, block, 0, stream>>>( \
      a, sa, w, sw, (int)M, (int)N, (int)K, group, y, ld_y)
  if constexpr (CB == 4) {
    const bool short_tail = K % 256 != 0;
    if (out_i32) {
      if (short_tail) QR_GEMM_LAUNCH(true, true);
      else QR_GEMM_LAUNCH(true, false);
    } else {
      if (short_tail) QR_GEMM_LAUNCH(false, true);
      else QR_GEMM_LAUNCH(false, false);
    }
  } else {   // K % 128 == 0: whole 128-code tiles
    if (out_i32) QR_GEMM_LAUNCH(true, false);
    else QR_GEMM_LAUNCH(false, false);
  }
#undef QR_GEMM_LAUNCH
  return hipGetLastError();
}

template <int CB>
hipError_t launch_prefill(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw, int64_t M,
                          int64_t N, int64_t K, int group, void *y, int64_t ld_y, bool out_i32,
                          hipStream_t stream) {
  if (group != 0)
    return launch_cfg<128, 128, 2, 2, 2, true, CB>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
  const int cus = device_cu_count();
  // fraction of the busy slot-rounds doing useful work, times the fraction of
  // the tile area inside the matrix, times a mild preference for bigger tiles
  auto score = [&](int64_t bm, int64_t bn, int64_t per_cu, double size_pref) __attribute__((always_inline)) {
    const int64_t slots = per_cu * cus;
    const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
    const int64_t tiles = tm * tn;
    const int64_t rounds = (tiles + slots - 1) / slots;
    return (double)tiles / (double)(rounds * slots) * (double)(M * N) / (double)(tm * bm * tn * bn) * size_pref;
  };
  // 256 x 192 blocks of 8 waves run one to a CU and move the fewest bytes
  // per multiply-add; the 4-wave shapes (two to a CU) fill small grids better.
  const double s_256x192 = score(256, 192, 1, 1.0), s_128x192 = score(128, 192, 2, 0.95),
               s_128x128 = score(128, 128, 2, 0.93);
  if (s_256x192 >= s_128x192 && s_256x192 >= s_128x128)
    return launch_cfg<256, 192, 4, 2, 2, false, CB>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
  if (s_128x192 >= s_128x128)
    return launch_cfg<128, 192, 2, 2, 2, false, CB>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
  return launch_cfg<128, 128, 2, 2, 2, false, CB>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
}

}  // namespace

hipError_t launch_gemm_prefill(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw,
                               int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                               bool out_i32, hipStream_t stream) {
  return launch_prefill<4>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
}

hipError_t launch_gemm_prefill_i8(const int8_t *a, const float *sa, const int8_t *w, const float *sw,
                                  int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                                  bool out_i32, hipStream_t stream) {
  return launch_prefill<8>((const uint8_t *)a, sa, (const uint8_t *)w, sw, M, N, K, group, y, ld_y, out_i32,
                           stream);
}

}  // namespace qr
