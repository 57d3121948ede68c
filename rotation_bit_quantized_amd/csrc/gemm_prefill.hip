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
// Tiling: 256 threads (2 x 2 waves), block tile BM x BN, K-tile 128 codes
// (64 bytes per row), LDS double buffer with an 80-byte row pitch (16-byte
// pieces of 8 consecutive rows land in distinct banks).  Each wave owns a
// (BM/2) x (BN/2) sub-tile of 32x32 MFMA fragments; one 16-byte LDS read
// per fragment row feeds two v_mfma_i32_32x32x32_i8 k-steps.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kBK = 128;        // codes per K-tile
constexpr int kRowBytes = 64;   // bytes per row per K-tile
constexpr int kPitch = 80;      // LDS row pitch in bytes

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

template <int BM, int BN, bool GROUPED, bool OUT_I32>
__global__ __launch_bounds__(256, GROUPED ? 1 : 2) void gemm_prefill_kernel(
    const uint8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ W,
    const float *__restrict__ sw, int M, int N, int K, int group, void *__restrict__ out, int64_t ld_y) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_LOADS = BM * 4 / 256;  // 16-byte pieces per thread
  constexpr int B_LOADS = BN * 4 / 256;
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small for 256 threads");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * kPitch];
  auto sA = [&](int buf) { return smem + buf * (BM + BN) * kPitch; };
  auto sB = [&](int buf) { return smem + buf * (BM + BN) * kPitch + BM * kPitch; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tm_count = (M + BM - 1) / BM;
  const int tn_count = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, tm_count, tn_count, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t kbytes = K / 2;
  const int KT = K / kBK;
  const int tiles_per_group = GROUPED ? group / kBK : 0;

  // global -> register staging
  v4u ra[A_LOADS], rb[B_LOADS];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 2, part = c & 3;
      const int gr = m0 + r;
      if (gr < M)
        ra[i] = *(const v4u *)(A + (int64_t)gr * kbytes + kt * kRowBytes + part * 16);
      else
        ra[i] = v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 2, part = c & 3;
      const int gr = n0 + r;
      if (gr < N)
        rb[i] = *(const v4u *)(W + (int64_t)gr * kbytes + kt * kRowBytes + part * 16);
      else
        rb[i] = v4u{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int c = tid + 256 * i;
      *(v4u *)(sA(buf) + (c >> 2) * kPitch + (c & 3) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int c = tid + 256 * i;
      *(v4u *)(sB(buf) + (c >> 2) * kPitch + (c & 3) * 16) = rb[i];
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

  // per-lane output coordinates
  const int lrow = 4 * (lane >> 5);   // + 8*(r/4) + r%4
  const int lcol = lane & 31;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_tile(kt + 1);
    const bool fresh = GROUPED && (kt % tiles_per_group == 0);

#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v4i aop[FM][2], bop[FN][2];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const v4u w = *(const v4u *)(sA(cur) + (wm * WM + i * 32 + (lane & 31)) * kPitch + kk * 32 +
                                     (lane >> 5) * 16);
        widen(w, aop[i][0], aop[i][1]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v4u w = *(const v4u *)(sB(cur) + (wn * WN + j * 32 + (lane & 31)) * kPitch + kk * 32 +
                                     (lane >> 5) * 16);
        widen(w, bop[j][0], bop[j][1]);
      }
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
          float swv[FN];
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WN + j * 32 + lcol;
            swv[j] = col < N ? sw[(int64_t)col * G + gidx] * (1.0f / 256.0f) : 0.f;
          }
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + lrow + (r & 3);
              const float sav = row < M ? sa[(int64_t)row * G + gidx] : 0.f;
#pragma unroll
              for (int j = 0; j < FN; ++j)
                facc[i][j][r] = __builtin_fmaf((float)acc[i][j][r], sav * swv[j], facc[i][j][r]);
            }
        }
      }
    }

    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
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

template <int BM, int BN, bool GROUPED>
hipError_t launch_cfg(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw, int64_t M,
                      int64_t N, int64_t K, int group, void *y, int64_t ld_y, bool out_i32,
                      hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid((unsigned)tiles), block(256);
  if (out_i32)
    gemm_prefill_kernel<BM, BN, GROUPED, true><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N,
                                                                          (int)K, group, y, ld_y);
  else
    gemm_prefill_kernel<BM, BN, GROUPED, false><<<grid, block, 0, stream>>>(a, sa, w, sw, (int)M, (int)N,
                                                                           (int)K, group, y, ld_y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_prefill(const uint8_t *a, const float *sa, const uint8_t *w, const float *sw,
                               int64_t M, int64_t N, int64_t K, int group, void *y, int64_t ld_y,
                               bool out_i32, hipStream_t stream) {
  if (group != 0) return launch_cfg<128, 128, true>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
  return launch_cfg<256, 128, false>(a, sa, w, sw, M, N, K, group, y, ld_y, out_i32, stream);
}

}  // namespace qr
