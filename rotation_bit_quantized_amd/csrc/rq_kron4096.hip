// Rotate + symmetric 4-bit RTN + pack for Kronecker rotations with a
// 4096-point Hadamard and a small dense factor:
//   R = (H_4096 / 64) kron O,  n = 4096 M,  2 <= M <= 8, no signs,
// e.g. the 28672-wide down_proj input of LLaMA-2-70B (M = 7).
//
// Method: y = x R per token row, s = max|y| / 7, q = rint(y / s) packed two
// per byte (QuaRot summary, "Key points": RTN on the fly).  Random orthogonal
// factor for widths that are not a power of two: QuIP summary, abstract, and
// the QuIP# quote on the same page (two-factor Kronecker construction).
//
// Index algebra.  Element k = i M + a (a fastest); split i = 8 t + i' and the
// output j = 8 u + j'.  Sylvester H_4096[i][j] = H_512[t][u] H_8[i'][j'], so
// with the row viewed as 512 blocks X[t] of 8 M contiguous elements,
//   Z[t] = X[t] B,   B[M i' + a][M j' + b] = H_8[i'][j'] O[a][b]   (8M x 8M)
//   Y[u] = sum_t H_512[t][u] Z[t] / 64,   y[8 M u + n] = Y[u][n].
//
// Design (one token row at a time per block of four waves, persistent grid,
// two blocks per CU so that one block's transform overlaps the other's
// MFMAs):
//  * Z = X B on v_mfma_f32_16x16x32_f16: A = X (the fp16 input, exact; M-tile
//    mt holds blocks t = 16 mt + c, k-steps of 32 over the padded width 64),
//    B = the fp16 high and low parts of H_8 kron O (both products accumulate
//    in fp32, error near 2^-22 relative).  Wave w owns output columns
//    n = 16 w .. 16 w + 15 (N padded to 64) for all 512 blocks: 32 M-tiles,
//    128 MFMAs per row and wave.
//  * The row arrives by coalesced DMA (1 KB per wave-instruction) into one
//    LDS buffer; the next row's DMA is issued as soon as every wave has read
//    its A-fragments, and lands while the transform runs.
//  * The 512-point transform over t is in registers: t0, t1 are register
//    bits of a C tile, t4..t8 the M-tile index, t2, t3 lane bits 4, 5 brought
//    into register bits with v_permlane16_swap / v_permlane32_swap.
//  * Absmax: DPP and lane swaps, then the four waves through LDS.  Codes are
//    packed eight to a word; a 4 x 4 nibble transpose within lane quads
//    turns each 16-bit half into four consecutive codes of one output block,
//    staged in LDS in the output layout and stored as 16-byte chunks.
//
// FUSED: the row is the feed-forward activation x = fp16(silu(gate) * up)
// of the block before down_proj (QuaRot abstract: the feed-forward
// activations are rotated too).  The gate row arrives by DMA as x would;
// right after it lands, every thread loads its pieces of the up row from
// global memory (coalesced, 16 bytes each) and rewrites the row in LDS as
// x (fp32 arithmetic, one fp16 rounding), so the fused call reads gate and
// up once and never writes x.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kWaves = 4;
constexpr int kMT = 32;       // M-tiles of 16 blocks: t < 512
constexpr int kKS = 2;        // k-steps of 32: block width 8 M <= 64
constexpr int kGrp = 4;       // M-tiles per A-read group

// silu(g) u in fp32 for the two fp16 halves of a word, rounded to fp16.
__device__ __forceinline__ unsigned swiglu2(unsigned gw, unsigned uw) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 g = __builtin_bit_cast(h2, gw), u = __builtin_bit_cast(h2, uw);
  h2 r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float gf = (float)g[k];
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * gf);   // e^-g
    r[k] = (_Float16)(gf * __builtin_amdgcn_rcpf(1.0f + e) * (float)u[k]);
  }
  return __builtin_bit_cast(unsigned, r);
}

// Two blocks per CU, except at M = 8, whose wave needs more than the 256
// registers that two waves per SIMD leave it (one block per CU; the launch
// sizes its grid from the occupancy query).
template <int M, bool FUSED>
__global__ __launch_bounds__(64 * kWaves, M == 8 ? 1 : 2) void rq_kron4096_kernel(
    const unsigned short *__restrict__ x, const unsigned short *__restrict__ up, int64_t rows, int64_t ld_x,
    const float *__restrict__ dense, uint8_t *__restrict__ codes, float *__restrict__ scales, float scale_mul) {
  static_assert(M >= 2 && M <= 8, "dense factor size");
  constexpr int kRowBytes = 8192 * M;        // 4096 M fp16
  constexpr int kBlkBytes = 16 * M;          // one block t: 8 M fp16
  constexpr int kCodeBytes = 2048 * M;       // n / 2
  constexpr int kW = 8 * M;                  // block width = output columns per block
  constexpr int kNst = kCodeBytes / 16;      // 16-byte code chunks per row
  constexpr int kPerThread = (kNst + 64 * kWaves - 1) / (64 * kWaves);
  constexpr int kDmaPerWave = kRowBytes / 1024 / kWaves;
  static_assert(kRowBytes % (1024 * kWaves) == 0, "row DMA split");

  // X row + 128 zero bytes: A-fragments span 64 fp16 from a block's start,
  // past the row's end for the last blocks when 8 M < 64
  __shared__ __attribute__((aligned(1024))) uint8_t xrow[kRowBytes + 128];
  __shared__ __attribute__((aligned(16))) uint8_t cbuf[kCodeBytes];   // codes, output layout
  __shared__ float wmax[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15;
  const int g = lane >> 4;

  // ---- B-fragments of H_8 kron O: lane (c16, g) holds B[32 ks + 8 g + j][16 wave + c16],
  // fp16 hi and lo parts, zero outside the 8M x 8M matrix
  v8h bf[kKS][2];
  {
    const int n = 16 * wave + c16;
    const int jp = n / M, b = n - (n / M) * M;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = 32 * ks + 8 * g + j;
        const int ip = k / M, a = k - (k / M) * M;
        const bool in = k < kW && n < kW;
        float v = dense[in ? a * M + b : 0];   // clamped load, then select
        v = (__builtin_popcount(ip & jp) & 1) ? -v : v;
        v = in ? v : 0.f;
        const _Float16 h = (_Float16)v;
        bf[ks][0][j] = h;
        bf[ks][1][j] = (_Float16)(v - (float)h);
      }
  }
  if (tid < 32) *(unsigned *)(xrow + kRowBytes + 4 * tid) = 0u;

  // per-lane constants: A-read offset (block c16 of an M-tile, k-piece g),
  // code-write offset (see below), DMA chunk
  const int a_off = c16 * kBlkBytes + 16 * g;
  const int n0 = 16 * wave + 4 * (c16 >> 2);          // first of the lane's four columns after the transpose
  const bool col_ok = n0 < kW;                         // (kW % 4 == 0: four valid columns or none)
  const int cw_off = 4 * M * (g | ((c16 & 3) << 2)) + (n0 >> 1);
  const unsigned perm_sel = (lane & 2) ? 0x03070105u : 0x06020400u;
  const unsigned rot_sh = (lane & 1) ? 4u : 28u;
  const unsigned keep = (lane & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
  const unsigned xrow_lds = lds_addr(xrow);
  int cs_off[kPerThread];
#pragma unroll
  for (int p = 0; p < kPerThread; ++p) {
    const int ch = tid + 64 * kWaves * p;
    cs_off[p] = 16 * (ch < kNst ? ch : ch % kNst);   // surplus lanes rewrite an existing chunk
  }

  auto issue_row = [&](int64_t r) __attribute__((always_inline)) {
    const uint8_t *src = (const uint8_t *)(x + r * ld_x);
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {
      const int chunk = q * kWaves + wave;
      dma16_to_lds(src + 1024 * chunk + 16 * lane, xrow_lds + 1024 * chunk);
    }
  };

  const int64_t stride = gridDim.x;
  int64_t row = blockIdx.x;   // the grid is no larger than rows
  issue_row(row);
  bool first = true;
  constexpr int kPieces = FUSED ? kRowBytes / 16 / (64 * kWaves) : 1;   // 16-byte pieces of up per thread
  for (int k = 0; row < rows; row += stride, ++k) {
    set_prio_by_progress(k);   // the two blocks of a CU keep pace
    // FUSED: this row's up pieces, loaded while the gate row's DMA finishes
    v4u uv[kPieces];
    if constexpr (FUSED) {
      const uint8_t *ur = (const uint8_t *)(up + row * ld_x);
#pragma unroll
      for (int p = 0; p < kPieces; ++p) uv[p] = *(const v4u *)(ur + 16 * (tid + 64 * kWaves * p));
    }
    // this row's DMA; issued after it (except for the first row): the
    // previous row's kPerThread chunk stores (and one scale store), then
    // the up pieces
    if (first) wait_vm<0>();
    else wait_vm<kPerThread + (FUSED ? kPieces : 0)>();
    first = false;
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    if constexpr (FUSED) {
      // the gate row is in xrow: rewrite it as x = silu(gate) up
#pragma unroll
      for (int p = 0; p < kPieces; ++p) {
        v4u *px = (v4u *)(xrow + 16 * (tid + 64 * kWaves * p));
        const v4u gv = *px;
        *px = v4u{swiglu2(gv[0], uv[p][0]), swiglu2(gv[1], uv[p][1]), swiglu2(gv[2], uv[p][2]),
                  swiglu2(gv[3], uv[p][3])};
      }
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
    }

    // ---- Z = X B for this wave's 16 columns, all 512 blocks
    v4f c[kMT];
    v4u abuf[2][kGrp][kKS];
    auto read_grp = [&](int grp, v4u (&dst)[kGrp][kKS]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < kGrp; ++i)
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
          dst[i][ks] = *(const v4u *)(xrow + (kGrp * grp + i) * 16 * kBlkBytes + a_off + 64 * ks);
    };
    read_grp(0, abuf[0]);
#pragma unroll
    for (int grp = 0; grp < kMT / kGrp; ++grp) {
      if (grp + 1 < kMT / kGrp) read_grp(grp + 1, abuf[(grp + 1) & 1]);
      // an accumulator's four updates are kGrp MFMAs apart
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
          for (int i = 0; i < kGrp; ++i) {
            const int mt = kGrp * grp + i;
            const v8h av = __builtin_bit_cast(v8h, abuf[grp & 1][i][ks]);
            if (ks == 0 && hl == 0)
              c[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bf[ks][hl], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            else
              c[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bf[ks][hl], c[mt], 0, 0, 0);
          }
      __builtin_amdgcn_sched_barrier(0);
    }
    // every wave has read its A-fragments: the buffer takes the next row
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    const uint8_t *nsrc = (const uint8_t *)(x + (row + stride < rows ? row + stride : row) * ld_x);

    // ---- 512-point Walsh-Hadamard over t.  Element r of c[mt] is block
    // t = 16 mt + 4 g + r: t0, t1 = r bits, t2, t3 = lane bits 4, 5,
    // t4..t8 = mt bits.  First the four bits inside each tile, with the next
    // row's DMA spread over them (a burst of DMA instructions would stall
    // the wave on the full memory-instruction queue), then the tile bits.
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      float e0 = c[mt][0], e1 = c[mt][1], e2 = c[mt][2], e3 = c[mt][3];
      // t0, t1: register bits 0, 1 -> u0, u1
      float a0 = e0 + e1, a1 = e0 - e1, a2 = e2 + e3, a3 = e2 - e3;
      e0 = a0 + a2; e1 = a1 + a3; e2 = a0 - a2; e3 = a1 - a3;
      // t2: lane bit 4 <-> register bit 0 (holding u0), then butterfly over
      // register bit 0; t3 likewise with lane bit 5 and register bit 1
      swap16(e0, e1);
      swap16(e2, e3);
      float f0 = e0 + e1, f1 = e0 - e1, f2 = e2 + e3, f3 = e2 - e3;
      swap32(f0, f2);
      swap32(f1, f3);
      c[mt] = v4f{f0 + f2, f1 + f3, f0 - f2, f1 - f3};
      if ((mt & 1) && (mt >> 1) < kDmaPerWave) {
        const int chunk = (mt >> 1) * kWaves + wave;
        dma16_to_lds(nsrc + 1024 * chunk + 16 * lane, xrow_lds + 1024 * chunk);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    static_assert(kDmaPerWave <= kMT / 2, "DMA slots in the tile loop");
#pragma unroll
    for (int mb = 1; mb < kMT; mb <<= 1)
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if (mt & mb) continue;
        const v4f u = c[mt], w = c[mt | mb];
        c[mt] = u + w;
        c[mt | mb] = u - w;
      }
    // Element r of c[mt] is now Y[u][16 wave + c16] with
    //   u = g | (r & 1) << 2 | (r >> 1) << 3 | mt << 4
    // (columns n >= 8 M hold zero: B's padding is zero).

    float mx = 0.f;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(c[mt][0]), fabsf(c[mt][1])), fmaxf(fabsf(c[mt][2]), fabsf(c[mt][3]))));
    mx = wave_max_dpp(mx);
    if (lane == 0) wmax[wave] = mx;
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    mx = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float inv = mx > 0.f ? 7.0f / mx : 0.f;

    // codes: bits 4 r + 16 h of word w2 hold the code of element r of
    // c[2 w2 + h] (alignbit shifts right by four and inserts at the top);
    // a 4 x 4 transpose within lane quads exchanges the quad lane index (the
    // column's low bits) with r: half h of w2 then holds the codes of columns
    // n0 .. n0 + 3 of block u = g | (c16 & 3) << 2 | (2 w2 + h) << 4, at
    // output byte (8 M u + n0) / 2.
    if (col_ok) {
#pragma unroll
      for (int w2 = 0; w2 < kMT / 2; ++w2) {
        unsigned acc = 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_alignbit(round_bits(c[2 * w2 + h][r], inv), acc, 4);
        unsigned v = __builtin_amdgcn_perm(dpp<kQuadXor2>(acc), acc, perm_sel);   // lane bit 1 <-> r bit 1
        const unsigned o = dpp<kQuadXor1>(v);                                      // lane bit 0 <-> r bit 0
        v = (keep & v) | (~keep & __builtin_amdgcn_alignbit(o, o, rot_sh));
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *(unsigned short *)(cbuf + cw_off + 64 * M * (2 * w2 + h)) = (unsigned short)(v >> (16 * h));
      }
    } else {
      // (no codes: the DPP partners of the transpose are in this lane's quad,
      // which is masked off as a whole)
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    uint8_t *cr = codes + row * (int64_t)kCodeBytes;
#pragma unroll
    for (int p = 0; p < kPerThread; ++p)
      __builtin_nontemporal_store(*(const v4u *)(cbuf + cs_off[p]), (v4u *)(cr + cs_off[p]));
    if (tid == 0) scales[row] = mx * scale_mul;
  }
  wait_vm<0>();   // no DMA may still be writing this block's LDS when it exits
}

template <int M, bool FUSED>
hipError_t launch_m(const void *x, const void *up, int64_t rows, int64_t ld_x, const float *dense, uint8_t *codes,
                    float *scales, hipStream_t stream) {
  const int cus = device_cu_count();
  // resident blocks per CU: a constant of the kernel, queried once (a
  // function-local static is initialised exactly once, thread-safely)
  static const int per_cu = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, rq_kron4096_kernel<M, FUSED>, 64 * kWaves, 0) != hipSuccess ||
        b < 1)
      b = 1;
    return b;
  }();
  const int64_t cap = (int64_t)cus * per_cu;
  const int64_t grid = rows < cap ? rows : cap;
  const float scale_mul = (float)(1.0 / (7.0 * 64.0));   // 1/(7 sqrt(4096))
  rq_kron4096_kernel<M, FUSED><<<dim3((unsigned)grid), dim3(64 * kWaves), 0, stream>>>(
      (const unsigned short *)x, (const unsigned short *)up, rows, ld_x, dense, codes, scales, scale_mul);
  return hipGetLastError();
}

}  // namespace

bool rq_kron4096_supported(const RotArgs &r, int group) {
  return r.had_n == 4096 && r.dense_m >= 2 && r.dense_m <= 8 && r.signs == nullptr && group == 0;
}

template <bool FUSED>
hipError_t launch_fused_or_not(const void *x, const void *up, int64_t rows, int64_t ld_x, const RotArgs &r,
                               uint8_t *codes, float *scales, hipStream_t stream) {
  switch (r.dense_m) {
    case 2: return launch_m<2, FUSED>(x, up, rows, ld_x, r.dense, codes, scales, stream);
    case 3: return launch_m<3, FUSED>(x, up, rows, ld_x, r.dense, codes, scales, stream);
    case 4: return launch_m<4, FUSED>(x, up, rows, ld_x, r.dense, codes, scales, stream);
    case 5: return launch_m<5, FUSED>(x, up, rows, ld_x, r.dense, codes, scales, stream);
    case 6: return launch_m<6, FUSED>(x, up, rows, ld_x, r.dense, codes, scales, stream);
    case 7: return launch_m<7, FUSED>(x, up, rows, ld_x, r.dense, codes, scales, stream);
    default: return launch_m<8, FUSED>(x, up, rows, ld_x, r.dense, codes, scales, stream);
  }
}

hipError_t launch_rq_kron4096(const void *x, int64_t rows, int64_t ld_x, const RotArgs &r, uint8_t *codes,
                              float *scales, hipStream_t stream) {
  return launch_fused_or_not<false>(x, nullptr, rows, ld_x, r, codes, scales, stream);
}

hipError_t launch_swiglu_rq_kron4096(const void *gate, const void *up, int64_t rows, int64_t ld, const RotArgs &r,
                                     uint8_t *codes, float *scales, hipStream_t stream) {
  return launch_fused_or_not<true>(gate, up, rows, ld, r, codes, scales, stream);
}

}  // namespace qr
