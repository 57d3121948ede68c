// 4-bit integer GEMM for prefill shapes (M > 64): y = dequant(qa . qw^T).
//
// Method: QuaRot abstract (all matrix multiplications in 4 bits);
// dequantizing epilogue y = acc * s_x * s_w per output channel, or the sum
// over K-groups of 128 of acc_g * s_x[g] * s_w[g] (QuaRot summary, "Key
// points": group size 128).
//
// CDNA4 has no 4-bit integer MFMA, so codes are widened to int8 in
// registers right after they are read from LDS, in "high-nibble" form:
//   lo = (w << 4) & 0xF0F0F0F0,  hi = w & 0xF0F0F0F0
// turns 8 packed codes into 8 int8 values 16*q (exact for q in [-8, 7]) in
// three VALU ops.  A and W are widened identically, so the product sums
// 256 * q_a * q_w; the k order inside a dword is permuted the same way on
// both sides and cancels.  |acc| <= 64 * 256 * K < 2^31 for K <= 131072.
// The 1/256 is an exact power of two folded into the epilogue (or a shift
// for the int32 output).
//
// Data movement: 256 threads (2 x 2 waves), two blocks per CU, block tile
// BM x BN, K-tile 128 codes = 64 bytes per row.  K-tiles travel from global
// memory straight into LDS with global_load_lds_dwordx4 (no VGPR staging),
// through STAGES LDS buffers: while the waves multiply K-tile kt, the loads
// of K-tiles kt+1 .. kt+STAGES-1 are in flight.  A wave waits (vmcnt) only
// for its own pieces of tile kt, then one s_barrier makes everyone's pieces
// visible and also certifies that the buffer about to be refilled has been
// consumed.  A DMA wave instruction fills 1 KB of LDS contiguously (lane i
// -> bytes 16i..16i+15), i.e. 16 rows x four 16-byte pieces; each lane
// fetches the global piece (slot ^ swz(row)) so that the fragment reads -
// 16 consecutive rows at one piece - hit 16 distinct bank groups.
//
// Compute: each wave owns a (BM/2) x (BN/2) sub-tile of 32x32 fragments (up
// to 128 x 128 = 256 accumulators), so each widened operand feeds FN (or FM)
// MFMAs; one 16-byte LDS read per fragment row feeds two
// v_mfma_i32_32x32x32_i8 k-steps, and the second read of a K-tile is issued
// before the first is widened.  The host picks BN so that the tile count
// fills the CU slots evenly (128 x 192 tiles for 2048 x 12288).
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kBK = 128;        // codes per K-tile
constexpr int kRowBytes = 64;   // bytes per row per K-tile

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void widen(const v4u &w, v4i &op0, v4i &op1) {
  op0[0] = (int)((w[0] << 4) & 0xF0F0F0F0u);
  op0[1] = (int)(w[0] & 0xF0F0F0F0u);
  op0[2] = (int)((w[1] << 4) & 0xF0F0F0F0u);
  op0[3] = (int)(w[1] & 0xF0F0F0F0u);
  op1[0] = (int)((w[2] << 4) & 0xF0F0F0F0u);
  op1[1] = (int)(w[2] & 0xF0F0F0F0u);
  op1[2] = (int)((w[3] << 4) & 0xF0F0F0F0u);
  op1[3] = (int)(w[3] & 0xF0F0F0F0u);
}

// LDS slot of 16-byte piece p (0..3) of tile row r (an involution in p).
__device__ __forceinline__ int swz(int r, int p) { return p ^ ((r >> 2) & 3); }

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

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

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool GROUPED, bool OUT_I32>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 8 / (WAVES_M * WAVES_N) > 0 ? 2 : 1) void gemm_prefill_kernel(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ W,
    const float *__restrict__ sw, int M, int N, int K, int group, void *__restrict__ out, int64_t ld_y) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr bool SCALES = GROUPED && !OUT_I32;   // group scales travel with the K-tiles
  constexpr int SCALE_BYTES = SCALES ? (BM + BN) * 4 : 0;
  constexpr int SCALE_INST = SCALES ? (BM + BN) / 64 : 0;   // 4-byte DMA wave-instructions per stage
  constexpr int STAGE_BYTES = (BM + BN) * kRowBytes + SCALE_BYTES;
  static_assert(!SCALES || ((BM + BN) % 64 == 0 && SCALE_INST % NW == 0), "scale DMA split");
  constexpr int SCALE_LOADS = SCALE_INST / NW;
  constexpr int TI = (BM + BN) / 16;              // DMA wave-instructions per stage (16 rows each)
  constexpr int LOADS = TI / NW;                  // per wave
  static_assert(TI % NW == 0, "tile rows must split evenly over the waves' DMA instructions");
  constexpr int WAVE_LOADS = LOADS + SCALE_LOADS;  // vmem ops per wave per stage
  static_assert(WAVE_LOADS * (STAGES - 2) < 64, "vmcnt range");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(STAGES >= 2 && STAGES <= 4, "pipeline depth");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index in an SGPR: everything derived from it (DMA counts, the
  // vmcnt thresholds) is then provably wave-uniform and stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int tm_count = (M + BM - 1) / BM;
  const int tn_count = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tm_count, tn_count, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t kbytes = K / 2;
  const int KT = K / kBK;
  const int tiles_per_group = GROUPED ? group / kBK : 1;

  // DMA sources: wave-instruction q of this wave fills tile rows
  // 16 (NW q + wave) .. +15 (A rows first, then W rows); lane l writes LDS
  // slot l % 4 of row l / 4 with global piece swz(row, slot).  Rows past the
  // matrix edge re-read the last row; their results are never stored.
  const uint8_t *src[LOADS];
#pragma unroll
  for (int q = 0; q < LOADS; ++q) {
    const int trow = 16 * (NW * q + wave) + (lane >> 2);   // 0 .. BM+BN-1
    const int piece = swz(trow, lane & 3);
    if (trow < BM) {
      const int gr = min(m0 + trow, M - 1);
      src[q] = A + (int64_t)gr * kbytes + piece * 16;
    } else {
      const int gr = min(n0 + trow - BM, N - 1);
      src[q] = W + (int64_t)gr * kbytes + piece * 16;
    }
  }
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q)
      __builtin_amdgcn_global_load_lds((const void *)(src[q] + kt * kRowBytes),
                                       (lds_void *)(smem + stage * STAGE_BYTES + (NW * q + wave) * 1024), 16,
                                       0, 0);
    if constexpr (SCALES) {
      // the group's scales: s_x of the BM tile rows, then s_w of the BN tile columns
      const int G = K / group;
      const int gidx = kt * kBK / group;
#pragma unroll
      for (int q = 0; q < SCALE_LOADS; ++q) {
        const int e = 64 * (NW * q + wave) + lane;
        const float *p = e < BM ? sa + (int64_t)min(m0 + e, M - 1) * G + gidx
                                : sw + (int64_t)min(n0 + e - BM, N - 1) * G + gidx;
        __builtin_amdgcn_global_load_lds((const void *)p,
                                         (lds_void *)(smem + stage * STAGE_BYTES + (BM + BN) * kRowBytes +
                                                      256 * (NW * q + wave)),
                                         4, 0, 0);
      }
    }
  };

  v16i acc[FM][FN];
  v16f facc[GROUPED ? FM : 1][GROUPED ? FN : 1];
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

  const int lrow = 4 * (lane >> 5);   // output row offset within a fragment: + 8*(r/4) + r%4
  const int lcol = lane & 31;
  const int ra = wm * WM + (lane & 31);            // tile row of this lane in A fragment 0
  const int rb = BM + wn * WN + (lane & 31);       // tile row of this lane in W fragment 0
  const int half = lane >> 5;                      // which 16-byte half of a 32-byte chunk

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s, s);

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt % STAGES;
    // wait for this wave's pieces of tile kt; later tiles may stay in flight
    // (kt is uniform, so these are scalar branches)
    const int ahead = min(STAGES - 2, KT - 1 - kt);
    if (ahead >= 2) wait_vm<2 * WAVE_LOADS>();
    else if (ahead == 1) wait_vm<WAVE_LOADS>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);

    const uint8_t *st = smem + cur * STAGE_BYTES;
    const bool fresh = GROUPED && (kt % tiles_per_group == 0);
    v4u araw[2][FM], braw[2][FN];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = ra + 32 * i;
        araw[kk][i] = *(const v4u *)(st + r * kRowBytes + swz(r, 2 * kk + half) * 16);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = rb + 32 * j;
        braw[kk][j] = *(const v4u *)(st + r * kRowBytes + swz(r, 2 * kk + half) * 16);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v4i aop[FM][2], bop[FN][2];
#pragma unroll
      for (int i = 0; i < FM; ++i) widen(araw[kk][i], aop[i][0], aop[i][1]);
#pragma unroll
      for (int j = 0; j < FN; ++j) widen(braw[kk][j], bop[j][0], bop[j][1]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            if (GROUPED && fresh && kk == 0 && ks == 0)
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[i][ks], bop[j][ks], v16i{}, 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[i][ks], bop[j][ks], acc[i][j], 0, 0, 0);
          }
    }

    if constexpr (GROUPED) {
      if ((kt + 1) % tiles_per_group == 0) {
        const int gidx = kt / tiles_per_group;
        const int G = K / group;
        if constexpr (OUT_I32) {
          int32_t *o = (int32_t *)out + (int64_t)gidx * M * N;
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              const int col = n0 + wn * WN + j * 32 + lcol;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + lrow + (r & 3);
                if (row < M && col < N) o[(int64_t)row * N + col] = acc[i][j][r] >> 8;
              }
            }
        } else {
          const float *sc = (const float *)(st + (BM + BN) * kRowBytes);
          float gsw[FN];
#pragma unroll
          for (int j = 0; j < FN; ++j) gsw[j] = sc[BM + wn * WN + j * 32 + lcol] * (1.0f / 256.0f);
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const v4f s4 = *(const v4f *)(sc + wm * WM + i * 32 + 8 * r4 + lrow);
#pragma unroll
              for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                  facc[i][j][4 * r4 + r] =
                      __builtin_fmaf((float)acc[i][j][4 * r4 + r], s4[r] * gsw[j], facc[i][j][4 * r4 + r]);
            }
        }
      }
    }
  }

  // ---- epilogue
  if constexpr (OUT_I32 && !GROUPED) {
    int32_t *o = (int32_t *)out;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WN + j * 32 + lcol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + lrow + (r & 3);
          if (row < M && col < N) o[(int64_t)row * N + col] = acc[i][j][r] >> 8;
        }
      }
  } else if constexpr (!OUT_I32) {
    unsigned short *y = (unsigned short *)out;
    float swv[FN];
    if constexpr (!GROUPED) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WN + j * 32 + lcol;
        swv[j] = col < N ? sw[col] * (1.0f / 256.0f) : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + lrow + (r & 3);
        if (row >= M) continue;
        const float sav = GROUPED ? 0.f : sa[row];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WN + j * 32 + lcol;
          if (col >= N) continue;
          float val;
          if constexpr (GROUPED)
            val = facc[i][j][r];
          else
            val = (float)acc[i][j][r] * (sav * swv[j]);
          y[(int64_t)row * ld_y + col] = float_to_half_bits(val);
        }
      }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, bool GROUPED>
hipError_t launch_cfg(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw, int64_t M,
                      int64_t N, int64_t K, int group, void *y, int64_t ld_y, bool out_i32,
                      hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid((unsigned)tiles), block(64 * WAVES_M * WAVES_N);
  if (out_i32)
    gemm_prefill_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, GROUPED, true><<<grid, block, 0, stream>>>(
        a, sa, w, sw, (int)M, (int)N, (int)K, group, y, ld_y);
  else
    gemm_prefill_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, GROUPED, false><<<grid, block, 0, stream>>>(
        a, sa, w, sw, (int)M, (int)N, (int)K, group, y, ld_y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_prefill(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw,
                               int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                               bool out_i32, hipStream_t stream) {
  // 4-wave blocks sized so that two fit on a CU (LDS and registers): the two
  // waves sharing a SIMD then come from independent blocks whose barriers
  // drift out of phase, and one multiplies while the other waits.
  if (group != 0)
    return launch_cfg<128, 128, 2, 2, 3, true>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t slots = 2 * (int64_t)cus;
  // fraction of the busy slot-rounds doing useful work, times the fraction of
  // the tile area inside the matrix, times a mild preference for bigger tiles
  auto score = [&](int64_t bm, int64_t bn, double size_pref) {
    const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
    const int64_t tiles = tm * tn;
    const int64_t rounds = (tiles + slots - 1) / slots;
    return (double)tiles / (double)(rounds * slots) * (double)(M * N) / (double)(tm * bm * tn * bn) * size_pref;
  };
  const double s_256x128 = score(256, 128, 1.0), s_128x192 = score(128, 192, 0.99), s_128x128 = score(128, 128, 0.9);
  if (s_256x128 >= s_128x192 && s_256x128 >= s_128x128)
    return launch_cfg<256, 128, 2, 2, 3, false>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
  if (s_128x192 >= s_128x128)
    return launch_cfg<128, 192, 2, 2, 3, false>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
  return launch_cfg<128, 128, 2, 2, 3, false>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
}

}  // namespace qr
