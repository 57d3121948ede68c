// One decode step of attention over the rotated 4-bit KV cache written by the
// KV quantizer (QuaRot abstract: the KV cache held in 4 bits, with the
// attention mechanism kept computationally invariant under the rotation;
// DuQuant, Knowl 12: Query x Key and attention output x Value pass through a
// fixed head-wise Hadamard rotation, the softmax output stays unquantized).
//
// The cache holds, per token t and KV head, codes c (128 unsigned nibbles),
// a step D and a zero point z with the rotated key / value k_rot = (c - z) D,
// k_rot = k R for R = diag(signs) H_128 / sqrt(128).  R is orthogonal, so
//   q . k = (q R) . k_rot,   sum_t p_t v_t = (sum_t p_t v_rot,t) R^T :
// the query is rotated once, the cache is used as stored, and the output is
// rotated back once.  Per token:
//   score = D (q' . c - z sum(q')),   q' = q R * sm_scale * log2(e)
// with q' . c on v_dot4_i32_i8 against q' split into three int8 parts (as
// exact as fp32), and the value side accumulates sum_t w_t c_t - sum_t w_t z_t
// with w_t = p_t D_t in fp32 (v_fma_mix on the codes read as fp16).
//
// Layout of the work: one block of four waves per (sequence, group of up to
// eight KV heads, chunk of tokens, query head within a KV head's group).  A
// 16-row step covers tps = 16 / hpg tokens of the group's hpg heads, whose
// code rows are contiguous in the cache: lane (tau, qd) = (lane >> 2,
// lane & 3) holds dims 32 qd .. 32 qd + 31 of head tau % hpg of token
// tau / hpg, its 16-byte quarter of a 64-byte code row.  Every lane keeps its
// own online-softmax state over its tokens (the four lanes of a row share
// it); the lanes and waves are merged through LDS at the end.  A sequence
// split into several chunks leaves one partial (max, sum, 128 accumulators)
// per chunk and query head in the caller's workspace; a second kernel merges
// them.  The query heads that share a KV head are placed on one XCD, one
// after the other, so that they read the group's cache rows through the
// same L2.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kStep = 16;          // tokens per wave step
constexpr int kGroup = 2;          // steps per online-softmax group
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const unsigned short *q;         // [B][Hq][128] fp16
  const uint8_t *kc, *vc;          // [B][T][Hkv][64]
  const float *ks, *vs;            // [B][T][Hkv]
  const uint8_t *kz, *vz;          // [B][T][Hkv]
  const int *lens;                 // [B] or null
  const int8_t *signs;             // [128] or null
  float qmul;                      // sm_scale * log2(e) / sqrt(128)
  int T, Hq, Hkv, G, nhg, chunk, splits;
  int64_t U;                       // tiles: B * nhg * splits
  float *ws;                       // [B][Hq][splits][kPart] when splits > 1
  unsigned short *out;             // [B][Hq][128] fp16
};

constexpr int kPart = 132;         // m, l, 2 pad, o[128]

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_to_float(unsigned short h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ unsigned short float_to_half(float f) {
  return __builtin_bit_cast(unsigned short, (_Float16)f);
}

// In-place unnormalised 128-point Walsh-Hadamard transform of buf[0..127]
// by threads 0..63 of the block (one butterfly pair each per level); every
// thread of the block must call it.
// In-place unnormalised 128-point Walsh-Hadamard transform of rows
// 0..nh-1 of buf (stride 128) by the whole block; every thread must call it.
__device__ __forceinline__ void wht128_rows(float *buf, int nh) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 1; h < kD; h <<= 1) {
    __syncthreads();
    for (int p = tid; p < nh * (kD / 2); p += blockDim.x) {
      const int row = p >> 6, j = p & 63;
      float *r = buf + row * kD + (j / h) * 2 * h + (j % h);
      const float x0 = r[0], x1 = r[h];
      r[0] = x0 + x1;
      r[h] = x0 - x1;
    }
  }
  __syncthreads();
}

constexpr int kHG = 8;             // KV heads per block
constexpr int kStage = 34;         // floats per lane in the merge stage: acc[32], m, l

__global__ __launch_bounds__(64 * kWaves) void attn_decode_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float qbuf[kHG * kD];
  __shared__ __attribute__((aligned(16))) float stage[kWaves * 64 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qd = lane & 3, tau = lane >> 2;

  // block -> (tile u, query variant gi): the G variants of a tile are
  // consecutive blocks of one XCD (blocks are dealt to the 8 XCDs in turn)
  const int L = blockIdx.x;
  const int k8 = L >> 3;
  const int gi = k8 % a.G;
  const int64_t u = (int64_t)(k8 / a.G) * 8 + (L & 7);
  if (u >= a.U) return;
  const int s = (int)(u % a.splits);
  const int64_t bh = u / a.splits;
  const int hg = (int)(bh % a.nhg);
  const int b = (int)(bh / a.nhg);
  const int h0 = hg * kHG;
  const int hpg = a.Hkv - h0 < kHG ? a.Hkv - h0 : kHG;      // heads in this group, 1..8
  const int tps = 16 / hpg;                                   // tokens per 16-row step
  const int hh = tau % hpg;                                   // this lane's head in the group
  const int toff = tau / hpg;                                 // and token within a step
  const bool lane_ok = toff < tps;

  int len = a.lens != nullptr ? a.lens[b] : a.T;
  len = len < 0 ? 0 : (len > a.T ? a.T : len);
  const int t0 = s * a.chunk;
  const int t1 = t0 + a.chunk < len ? t0 + a.chunk : len;

  unsigned qe[3][4], qo[3][4];   // the query in int8 parts, filled below
  float qscale[3];
  float qsum = 0.f;

  float m = -__builtin_inff();
  float l = 0.f, zacc = 0.f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;

  const int64_t head_row = h0 + hh;                            // + (b T + t) Hkv
  const int nsteps = t1 > t0 ? (t1 - t0 + tps - 1) / tps : 0;

  // one online-softmax group: kGroup steps of this wave, loaded one group
  // ahead of the arithmetic
  struct Grp {
    v4u kw[kGroup], vw[kGroup];
    float kd[kGroup], vd[kGroup], kzf[kGroup], vzf[kGroup];
    bool ok[kGroup];
  };
  auto load = [&](int j0, Grp &G) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int t = t0 + (j0 + g * kWaves) * tps + toff;
      G.ok[g] = lane_ok && t < t1;
      const int tc = G.ok[g] ? t : t0;                         // an in-range row for masked lanes
      const int64_t row = ((int64_t)b * a.T + tc) * a.Hkv + head_row;
      G.kw[g] = *(const v4u *)(a.kc + row * 64 + 16 * qd);
      G.vw[g] = *(const v4u *)(a.vc + row * 64 + 16 * qd);
      G.kd[g] = a.ks[row];
      G.vd[g] = a.vs[row];
      G.kzf[g] = (float)a.kz[row];
      G.vzf[g] = (float)a.vz[row];
    }
  };
  auto compute = [&](const Grp &G) __attribute__((always_inline)) {
    float sc[kGroup];
    float gmax = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      // q' . c on the int8 dot product: codes are bytes 0..15 after masking
      int d0 = 0, d1 = 0, d2 = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        unsigned lo = G.kw[g][w] & 0x0F0F0F0Fu, hi = (G.kw[g][w] >> 4) & 0x0F0F0F0Fu;
        d0 = __builtin_amdgcn_sdot4((int)lo, (int)qe[0][w], d0, false);
        d0 = __builtin_amdgcn_sdot4((int)hi, (int)qo[0][w], d0, false);
        d1 = __builtin_amdgcn_sdot4((int)lo, (int)qe[1][w], d1, false);
        d1 = __builtin_amdgcn_sdot4((int)hi, (int)qo[1][w], d1, false);
        d2 = __builtin_amdgcn_sdot4((int)lo, (int)qe[2][w], d2, false);
        d2 = __builtin_amdgcn_sdot4((int)hi, (int)qo[2][w], d2, false);
      }
      float dot = __builtin_fmaf(qscale[0], (float)d0, __builtin_fmaf(qscale[1], (float)d1, qscale[2] * (float)d2));
      dot += dpp<kQuadXor1>(dot);
      dot += dpp<kQuadXor2>(dot);
      sc[g] = G.ok[g] ? G.kd[g] * (dot - G.kzf[g] * qsum) : -__builtin_inff();
      gmax = fmaxf(gmax, sc[g]);
    }
    const float m_new = fmaxf(m, gmax);
    const float m_ref = m_new == -__builtin_inff() ? 0.f : m_new;
    if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {          // rescale only when a max moved
      const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
      l *= alpha;
      zacc *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] *= alpha;
    }
    m = m_new;
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const float p = __builtin_amdgcn_exp2f(sc[g] - m_ref);
      l += p;
      const float w8 = p * G.vd[g];
      zacc = __builtin_fmaf(w8, G.vzf[g], zacc);
      // A masked nibble n read as an fp16 is the subnormal n 2^-24, exact in
      // v_fma_mix's conversion; the weight carries the 2^24.
      const float w24 = w8 * 16777216.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const unsigned v = G.vw[g][w];
        h2 e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) e[k] = __builtin_bit_cast(h2, (v >> (4 * k)) & 0x000F000Fu);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[8 * w + k] = __builtin_fmaf(w24, (float)e[k][0], acc[8 * w + k]);
          acc[8 * w + 4 + k] = __builtin_fmaf(w24, (float)e[k][1], acc[8 * w + 4 + k]);
        }
      }
    }
  };

  constexpr int kAdv = kWaves * kGroup;                          // steps between a wave's groups
  Grp ga, gb;
  int j = wave;
  if (j < nsteps) load(j, ga);     // in flight while the query is prepared

  // ---- q' = (q * signs) H_128 * qmul for the group's query heads
  for (int p = tid; p < hpg * kD; p += 64 * kWaves) {
    const int r = p >> 7, d = p & 127;
    const int hq = (h0 + r) * a.G + gi;
    float v = half_to_float(a.q[((int64_t)b * a.Hq + hq) * kD + d]);
    if (a.signs != nullptr && a.signs[d] < 0) v = -v;
    qbuf[p] = v;
  }
  wht128_rows(qbuf, hpg);
  // The lane's 32 query values as three int8 parts, q' ~ s1 p1 + s2 p2 + s3 p3
  // with |p| <= 127 and s_{k+1} = s_k / 254 (each remainder is at most half a
  // step, so the next part fits; the last remainder is below 2^-23 of the
  // lane's max |q'|).  Part bytes are laid out as the code bytes: word w of
  // qe holds dims 8w, 8w+2, 8w+4, 8w+6 (the low nibbles of a code word),
  // qo dims 8w+1, ..., 8w+7 (the high nibbles).
  {
    float qv[32];
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      qv[i] = qbuf[hh * kD + 32 * qd + i] * a.qmul;
      qsum += qv[i];
      mx = fmaxf(mx, fabsf(qv[i]));
    }
    float sc = mx > 0.f ? mx / 127.0f : 1.0f;
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      const float inv = 1.0f / sc;
      qscale[part] = sc;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        unsigned e = 0u, o = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float ve = __builtin_rintf(qv[8 * w + 2 * k] * inv);
          const float vo = __builtin_rintf(qv[8 * w + 2 * k + 1] * inv);
          qv[8 * w + 2 * k] = __builtin_fmaf(-ve, sc, qv[8 * w + 2 * k]);
          qv[8 * w + 2 * k + 1] = __builtin_fmaf(-vo, sc, qv[8 * w + 2 * k + 1]);
          e |= ((unsigned)(int)ve & 0xFFu) << (8 * k);
          o |= ((unsigned)(int)vo & 0xFFu) << (8 * k);
        }
        qe[part][w] = e;
        qo[part][w] = o;
      }
      sc *= 1.0f / 254.0f;
    }
  }
  qsum += dpp<kQuadXor1>(qsum);
  qsum += dpp<kQuadXor2>(qsum);

  while (j < nsteps) {
    const int jb = j + kAdv;
    if (jb < nsteps) load(jb, gb);
    compute(ga);
    if (jb >= nsteps) break;
    const int jc = jb + kAdv;
    if (jc < nsteps) load(jc, ga);
    compute(gb);
    j = jc;
  }

  // ---- stage every lane's state: acc - zacc (the zero-point term), m, l
  float *st = stage + (wave * 64 + lane) * kStage;
#pragma unroll
  for (int i = 0; i < 32; i += 2) *(v2f *)(st + i) = v2f{acc[i] - zacc, acc[i + 1] - zacc};
  *(v2f *)(st + 32) = v2f{m, l};
  __syncthreads();

  // ---- merge per (head, dim) over the waves and the tokens of a step
  for (int p = tid; p < hpg * kD; p += 64 * kWaves) {
    const int r = p >> 7, d = p & 127;
    const int dq = d >> 5, di = d & 31;
    float mb = -__builtin_inff();
    for (int w = 0; w < kWaves; ++w)
      for (int to = 0; to < tps; ++to) mb = fmaxf(mb, stage[(w * 64 + 4 * (to * hpg + r) + dq) * kStage + 32]);
    const float mref = mb == -__builtin_inff() ? 0.f : mb;
    float lb = 0.f, ob = 0.f;
    for (int w = 0; w < kWaves; ++w)
      for (int to = 0; to < tps; ++to) {
        const float *e = stage + (w * 64 + 4 * (to * hpg + r) + dq) * kStage;
        const float f = __builtin_amdgcn_exp2f(e[32] - mref);
        lb += f * e[33];
        ob += f * e[di];
      }
    const int hq = (h0 + r) * a.G + gi;
    if (a.splits == 1) {
      qbuf[p] = lb > 0.f ? ob / lb : 0.f;
    } else {
      float *part = a.ws + (((int64_t)b * a.Hq + hq) * a.splits + s) * kPart;
      part[4 + d] = ob;
      if (d == 0) {
        part[0] = mb;
        part[1] = lb;
      }
    }
  }
  if (a.splits == 1) {
    // out = o R^T: transform, then signs and 1/sqrt(128)
    wht128_rows(qbuf, hpg);
    for (int p = tid; p < hpg * kD; p += 64 * kWaves) {
      const int r = p >> 7, d = p & 127;
      const int hq = (h0 + r) * a.G + gi;
      float v = qbuf[p] * 0.08838834764831845f;
      if (a.signs != nullptr && a.signs[d] < 0) v = -v;
      a.out[((int64_t)b * a.Hq + hq) * kD + d] = float_to_half(v);
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped query heads (Hq / Hkv = G in 4..16, e.g. LLaMA-2-70B's 64 / 8): one
// block per (sequence, KV head, chunk) serves all G query heads on the matrix
// cores, so every cache row is read and unpacked once.  Per 16-token step of
// a wave (lane c16 = token for the A operands):
//  * scores S^T[token][head] = K Q'^T on v_mfma_f32_16x16x32_f16: A = the key
//    codes (a lane's 16 contiguous code bytes of its token; k-step s takes
//    word s), B = q' (fp16 high and low parts) in the same dim order: k =
//    8 kg + j <-> dim 32 kg + 8 s + perm[j], perm = 0 4 1 5 2 6 3 7.  A code
//    nibble enters as the fp16 bit pattern it forms in place, masked: the
//    subnormal n 2^-24 (perm slots 0, 1, 4, 5) or 16 n 2^-24 (slots 2, 3,
//    6, 7, whose B entries carry 1/16), all exact, one AND per two codes.
//    The output holds four consecutive tokens of one head per lane, in units
//    of 2^-24.
//  * the value tile turned into dims x tokens by an MFMA against selection
//    matrices (A = the value codes as above, B = 1 or 1/16; the output n
//    2^-24 is exact in fp16 as well; 16 dims per tile), which also leaves
//    four consecutive tokens per lane;
//  * O^T += V^T P'^T on v_mfma_f32_16x16x16_f16 (P' = p D for the value
//    steps, fp16 high and low parts; O^T in units of 2^-24): both operand
//    layouts (four consecutive k per lane) are exactly the two outputs above.
// Online softmax per head (lane column), merged over lanes and waves as in
// the per-head kernel; partials and outputs in the same formats.
constexpr int kGqaMaxG = 16;
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// The eight nibbles of a code word as fp16 subnormals, in perm order:
// slots (0, 1) = nibbles (0, 4) as n 2^-24, (2, 3) = nibbles (1, 5) as
// 16 n 2^-24, (4, 5) = nibbles (2, 6), (6, 7) = nibbles (3, 7) likewise.
__device__ __forceinline__ v8h codes_sub(unsigned w) {
  const unsigned w8 = w >> 8;
  return __builtin_bit_cast(v8h, v4u{w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u});
}
// scale of perm slot j in codes_sub, inverted
__device__ __forceinline__ constexpr float slot_unscale(int j) { return (j & 2) ? 0.0625f : 1.0f; }

__global__ __launch_bounds__(64 * kWaves, 3) void attn_decode_gqa_kernel(AttnArgs a) {
  __shared__ float qbuf[kGqaMaxG * kD];
  __shared__ float ostage[kWaves][kD][kGqaMaxG + 1];
  __shared__ float wml[kWaves][2][kGqaMaxG];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int G = a.G;

  const int64_t u = blockIdx.x;
  const int s = (int)(u % a.splits);
  const int64_t bh = u / a.splits;
  const int hk = (int)(bh % a.Hkv);
  const int b = (int)(bh / a.Hkv);

  int len = a.lens != nullptr ? a.lens[b] : a.T;
  len = len < 0 ? 0 : (len > a.T ? a.T : len);
  const int t0 = s * a.chunk;
  const int t1 = t0 + a.chunk < len ? t0 + a.chunk : len;
  const int nsteps = t1 > t0 ? (t1 - t0 + 15) / 16 : 0;

  // ---- loads of one 16-token step (issued one step ahead).  The sequence's
  // rows of this KV head start at uniform base pointers; a lane addresses
  // its rows with 32-bit offsets (the host checks T * Hkv * 64 < 2^31).
  const int64_t seq_row = (int64_t)b * a.T * a.Hkv + hk;
  const uint8_t *const kc_b = a.kc + seq_row * 64;
  const uint8_t *const vc_b = a.vc + seq_row * 64;
  const float *const ks_b = a.ks + seq_row;
  const float *const vs_b = a.vs + seq_row;
  const uint8_t *const kz_b = a.kz + seq_row;
  const uint8_t *const vz_b = a.vz + seq_row;
  const unsigned hkv = (unsigned)a.Hkv;
  // A step's per-token scales and zero points: lane l loads one value, of
  // token c16 (= l mod 16) from array g4 (k step, k zero, v step, v zero);
  // the lanes that need it fetch it with ds_bpermute when the step runs.
  // Small step buffers let three of them (two steps in flight) fit.
  struct Step {
    v4u kc, vc;   // this lane's token (c16): code words 4 g4 .. 4 g4 + 3
    float meta;
  };
  auto load = [&](int j, Step &st) __attribute__((always_inline)) {
    const int base = t0 + 16 * j;
    const int ta = base + c16;
    const unsigned ra = (unsigned)(ta < t1 ? ta : t0) * hkv;
    st.kc = *(const v4u *)(kc_b + (ra * 64u + 16u * (unsigned)g4));
    st.vc = *(const v4u *)(vc_b + (ra * 64u + 16u * (unsigned)g4));
    if (g4 & 1) st.meta = (float)((g4 & 2) ? vz_b : kz_b)[ra];
    else st.meta = *(const float *)((const uint8_t *)((g4 & 2) ? vs_b : ks_b) + ra * 4u);
  };
  Step sa, sb, sc;
  int j = wave;
  if (j < nsteps) load(j, sa);   // in flight while the queries are prepared
  if (j + kWaves < nsteps) load(j + kWaves, sb);

  // ---- q' for the G query heads of this KV head, as fp16 high / low B operands
  for (int p = tid; p < G * kD; p += 64 * kWaves) {
    const int r = p >> 7, d = p & 127;
    float v = half_to_float(a.q[((int64_t)b * a.Hq + (int64_t)hk * G + r) * kD + d]);
    if (a.signs != nullptr && a.signs[d] < 0) v = -v;
    qbuf[p] = v;
  }
  wht128_rows(qbuf, G);
  constexpr int kPerm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
  v8h qb[4][2];
  float qsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int d = 32 * g4 + 8 * ks + kPerm[jj];
      const float v = c16 < G ? qbuf[c16 * kD + d] * a.qmul : 0.f;
      const float vs = v * slot_unscale(jj);   // exact: a power of two
      const _Float16 hi = (_Float16)vs;
      qb[ks][0][jj] = hi;
      qb[ks][1][jj] = (_Float16)(vs - (float)hi);
      qsum += v;
    }
  qsum += __shfl_xor(qsum, 16);
  qsum += __shfl_xor(qsum, 32);   // sum of q' over all 128 dims of head c16
  const float qsum24 = qsum * 0x1p-24f;   // in the scores' units
  // selection B operands: output column n <- k = 8 (n >> 3) + (n & 7) of
  // the lower (kg < 2) or upper (kg >= 2) half of the k-step, weighted by the
  // slot's unscale so that every output is n 2^-24
  v8h selA, selB;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const _Float16 one = (_Float16)slot_unscale(jj);
    selA[jj] = (g4 < 2 && c16 == 8 * g4 + jj) ? one : (_Float16)0.0f;
    selB[jj] = (g4 >= 2 && c16 == 8 * (g4 - 2) + jj) ? one : (_Float16)0.0f;
  }

  float m = -__builtin_inff(), l = 0.f, zacc = 0.f;
  v4f o[8];   // O^T tiles (k-step s, half h) -> o[2 s + h]: dims x heads
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = v4f{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const Step &cur, int jj) __attribute__((always_inline)) {
    // this lane's four tokens 4 g4 + r: in range, and their scales and zero points
    bool ok[4];
    float kd[4], kz[4], vd[4], vz[4];
    const int mi = __builtin_bit_cast(int, cur.meta);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ok[r] = t0 + 16 * jj + 4 * g4 + r < t1;
      const int src = 4 * (4 * g4 + r);   // byte address of lane 4 g4 + r in the array-0 group
      kd[r] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, mi));
      kz[r] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src + 64, mi));
      vd[r] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src + 128, mi));
      vz[r] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src + 192, mi));
    }
    // scores
    v4f sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const v8h ak = codes_sub(cur.kc[ks]);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qb[ks][0], sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qb[ks][1], sc, 0, 0, 0);
    }
    float smax = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = ok[r] ? kd[r] * (sc[r] - kz[r] * qsum24) : -__builtin_inff();   // score 2^-24
      smax = fmaxf(smax, sc[r]);
    }
    {
      float x0 = smax, x1 = smax;
      swap16(x0, x1);
      smax = fmaxf(x0, x1);
      x0 = smax;
      x1 = smax;
      swap32(x0, x1);
      smax = fmaxf(x0, x1) * 0x1p24f;   // over the four lane groups: the head's step max
    }
    const float m_new = fmaxf(m, smax);
    const float m_ref = m_new == -__builtin_inff() ? 0.f : m_new;
    if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
      l *= alpha;
      zacc *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
    }
    m = m_new;
    v4h phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], 0x1p24f, -m_ref));
      l += p;
      const float pv = p * vd[r];
      zacc = __builtin_fmaf(pv, vz[r], zacc);
      phi[r] = (_Float16)pv;
      plo[r] = (_Float16)(pv - (float)phi[r]);
    }
    // values: dims x tokens tiles, then O^T += V^T P'^T
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const v8h av = codes_sub(cur.vc[ks]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4f t = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, h ? selB : selA, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        v4h vt;
#pragma unroll
        for (int r = 0; r < 4; ++r) vt[r] = (_Float16)t[r];   // exact: n 2^-24
        o[2 * ks + h] = __builtin_amdgcn_mfma_f32_16x16x16f16(vt, phi, o[2 * ks + h], 0, 0, 0);
        o[2 * ks + h] = __builtin_amdgcn_mfma_f32_16x16x16f16(vt, plo, o[2 * ks + h], 0, 0, 0);
      }
    }
  };
  // a ring of three step buffers, each loaded two steps ahead
  while (j < nsteps) {
    if (j + 2 * kWaves < nsteps) load(j + 2 * kWaves, sc);
    step(sa, j);
    j += kWaves;
    if (j >= nsteps) break;
    if (j + 2 * kWaves < nsteps) load(j + 2 * kWaves, sa);
    step(sb, j);
    j += kWaves;
    if (j >= nsteps) break;
    if (j + 2 * kWaves < nsteps) load(j + 2 * kWaves, sb);
    step(sc, j);
    j += kWaves;
  }

  // ---- per wave: l and the zero-point sum over the lane groups, stage O^T
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  zacc += __shfl_xor(zacc, 16);
  zacc += __shfl_xor(zacc, 32);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mrow = 4 * g4 + r;   // output column of the selection = row of O^T
        const int d = 32 * ((mrow >> 3) + 2 * h) + 8 * ks + kPerm[mrow & 7];
        ostage[wave][d][c16] = __builtin_fmaf(o[2 * ks + h][r], 0x1p24f, -zacc);
      }
  if (g4 == 0) {
    wml[wave][0][c16] = m;
    wml[wave][1][c16] = l;
  }
  __syncthreads();

  // ---- merge the waves per (head, dim)
  for (int p = tid; p < G * kD; p += 64 * kWaves) {
    const int hh = p >> 7, d = p & 127;
    float mb = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mb = fmaxf(mb, wml[w][0][hh]);
    const float mref = mb == -__builtin_inff() ? 0.f : mb;
    float lb = 0.f, ob = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(wml[w][0][hh] - mref);
      lb += f * wml[w][1][hh];
      ob += f * ostage[w][d][hh];
    }
    const int hq = hk * G + hh;
    if (a.splits == 1) {
      qbuf[p] = lb > 0.f ? ob / lb : 0.f;
    } else {
      float *part = a.ws + (((int64_t)b * a.Hq + hq) * a.splits + s) * kPart;
      part[4 + d] = ob;
      if (d == 0) {
        part[0] = mb;
        part[1] = lb;
      }
    }
  }
  if (a.splits == 1) {
    wht128_rows(qbuf, G);
    for (int p = tid; p < G * kD; p += 64 * kWaves) {
      const int hh = p >> 7, d = p & 127;
      float v = qbuf[p] * 0.08838834764831845f;
      if (a.signs != nullptr && a.signs[d] < 0) v = -v;
      a.out[((int64_t)b * a.Hq + (int64_t)hk * G + hh) * kD + d] = float_to_half(v);
    }
  }
}

constexpr int kMaxSplits = 2048;   // the plan never splits a sequence further

// Merge the chunks of one (sequence, query head): block-wide max of the
// chunk maxima, their weights in LDS, then each half of the block sums every
// other chunk's accumulators (independent loads, many in flight), output.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  __shared__ float fs[kMaxSplits];
  __shared__ float red[2][4];
  __shared__ float half_o[kD];
  __shared__ float buf[kD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hq = blockIdx.x, b = blockIdx.y;
  const int S = a.splits;
  const float *part = a.ws + ((int64_t)b * a.Hq + hq) * S * kPart;

  float mloc = -__builtin_inff();
  for (int s = tid; s < S; s += 256) mloc = fmaxf(mloc, part[s * kPart]);
  mloc = wave_max_dpp(mloc);
  if (lane == 0) red[0][wave] = mloc;
  __syncthreads();
  const float mb = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  const float mref = mb == -__builtin_inff() ? 0.f : mb;
  float lloc = 0.f;
  for (int s = tid; s < S; s += 256) {
    const float f = __builtin_amdgcn_exp2f(part[s * kPart] - mref);
    fs[s] = f;
    lloc += f * part[s * kPart + 1];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lloc += __shfl_xor(lloc, o);
  if (lane == 0) red[1][wave] = lloc;
  __syncthreads();
  const float lb = red[1][0] + red[1][1] + red[1][2] + red[1][3];

  const int d = tid & (kD - 1), h = tid >> 7;
  float o0 = 0.f, o1 = 0.f;
  int s = h;
#pragma unroll 4
  for (; s + 2 < S; s += 4) {
    o0 += fs[s] * part[s * kPart + 4 + d];
    o1 += fs[s + 2] * part[(s + 2) * kPart + 4 + d];
  }
  if (s < S) o0 += fs[s] * part[s * kPart + 4 + d];
  if (h == 1) half_o[d] = o0 + o1;
  __syncthreads();
  if (h == 0) buf[d] = lb > 0.f ? (o0 + o1 + half_o[d]) / lb : 0.f;
  wht128_rows(buf, 1);
  if (h == 0) {
    float v = buf[d] * 0.08838834764831845f;
    if (a.signs != nullptr && a.signs[d] < 0) v = -v;
    a.out[((int64_t)b * a.Hq + hq) * kD + d] = float_to_half(v);
  }
}

// Few chunks (at most kFewSplits; the loops over them are unrolled by four so
// that their loads overlap): one wave per (sequence, query head), four
// to a block.  A lane merges dims lane and lane + 64 over the chunks, and the
// inverse 128-point transform runs in the wave's registers: the butterfly
// over index bit 6 inside the lane, bits 0-5 by lane exchanges.  No LDS, no
// barrier; the block-wide kernel above serves long split lists.
constexpr int kFewSplits = 8;

__global__ __launch_bounds__(256) void attn_combine_few_kernel(AttnArgs a, int64_t nheads) {
  const int lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // b * Hq + hq
  if (u >= nheads) return;
  const int S = a.splits;
  const float *part = a.ws + u * S * kPart;
  float mb = -__builtin_inff();
#pragma unroll 4
  for (int s = 0; s < S; ++s) mb = fmaxf(mb, part[s * kPart]);
  const float mref = mb == -__builtin_inff() ? 0.f : mb;
  float lb = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float *e = part + s * kPart;
    const float f = __builtin_amdgcn_exp2f(e[0] - mref);
    lb += f * e[1];
    o0 += f * e[4 + lane];
    o1 += f * e[4 + 64 + lane];
  }
  float v0 = lb > 0.f ? o0 / lb : 0.f;
  float v1 = lb > 0.f ? o1 / lb : 0.f;
  // out = o R^T: H_128 (Sylvester) over d = 64 h + lane
  {
    const float t0 = v0 + v1, t1 = v0 - v1;
    v0 = t0;
    v1 = t1;
  }
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) {
    const float p0 = __shfl_xor(v0, k), p1 = __shfl_xor(v1, k);
    const bool hi = (lane & k) != 0;
    v0 = hi ? p0 - v0 : v0 + p0;
    v1 = hi ? p1 - v1 : v1 + p1;
  }
  unsigned short *out = a.out + u * kD;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int d = 64 * h + lane;
    float v = (h ? v1 : v0) * 0.08838834764831845f;
    if (a.signs != nullptr && a.signs[d] < 0) v = -v;
    out[d] = float_to_half(v);
  }
}

}  // namespace

AttnPlan attn_decode_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t T) {
  AttnPlan p{};
  const int64_t nhg = Hkv > 0 ? (Hkv + kHG - 1) / kHG : 0;
  const int64_t G = Hkv > 0 ? Hq / Hkv : 0;
  p.gqa = G >= 4 && G <= kGqaMaxG;                               // all query heads of a KV head per block
  const int64_t base = p.gqa ? B * Hkv : B * nhg * G;            // blocks without splitting
  int64_t splits = 1;
  if (T > 64 && base > 0) {
    // Both kernels run 4-wave blocks at 3 waves per SIMD: 768 resident blocks
    // on 256 CUs.  A launch takes ceil(blocks / 768) rounds, each as long as
    // one block: its chunk plus a fixed cost (query setup and merge, about
    // 80 tokens' worth).  Take the split count with the least estimate,
    // chunks of at least 64 tokens, at most kMaxSplits.
    constexpr int64_t kResident = 768, kFixed = 80;
    int64_t most = (T + 63) / 64;
    most = most < kMaxSplits ? most : kMaxSplits;
    int64_t best = -1;
    for (int64_t sp = 1; sp <= most; ++sp) {
      const int64_t ck = ((T + sp - 1) / sp + 15) / 16 * 16;
      const int64_t est = ((base * sp + kResident - 1) / kResident) * (ck + kFixed);
      if (best < 0 || est < best) {
        best = est;
        splits = sp;
      }
    }
  }
  int64_t chunk = (T + splits - 1) / splits;
  chunk = (chunk + 15) / 16 * 16;
  if (chunk < 16) chunk = 16;
  p.chunk = chunk;
  p.splits = (T + chunk - 1) / chunk;
  if (p.splits < 1) p.splits = 1;
  p.nhg = nhg;
  p.tiles = p.gqa ? B * Hkv * p.splits : B * nhg * p.splits;
  p.blocks = p.gqa ? p.tiles : (p.tiles + 7) / 8 * 8 * G;
  p.workspace_bytes = p.splits > 1 ? B * Hq * p.splits * kPart * (int64_t)sizeof(float) : 0;
  return p;
}

hipError_t launch_attn_decode(const void *q, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, const uint8_t *kc,
                              const float *ks, const uint8_t *kz, const uint8_t *vc, const float *vs,
                              const uint8_t *vz, const int *lens, const int8_t *signs, float sm_scale,
                              const AttnPlan &plan, float *ws, void *out, hipStream_t stream) {
  AttnArgs a{};
  a.q = (const unsigned short *)q;
  a.kc = kc;
  a.vc = vc;
  a.ks = ks;
  a.vs = vs;
  a.kz = kz;
  a.vz = vz;
  a.lens = lens;
  a.signs = signs;
  a.qmul = sm_scale * kLog2e * 0.08838834764831845f;   // and the 1/sqrt(128) of R
  a.T = (int)T;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.G = (int)(Hq / Hkv);
  a.nhg = (int)plan.nhg;
  a.U = plan.tiles;
  a.chunk = (int)plan.chunk;
  a.splits = (int)plan.splits;
  a.ws = ws;
  a.out = (unsigned short *)out;
  if (plan.gqa)
    attn_decode_gqa_kernel<<<dim3((unsigned)plan.blocks), dim3(64 * kWaves), 0, stream>>>(a);
  else
    attn_decode_kernel<<<dim3((unsigned)plan.blocks), dim3(64 * kWaves), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  if (plan.splits <= kFewSplits) {
    const int64_t nheads = B * Hq;
    attn_combine_few_kernel<<<dim3((unsigned)((nheads + 3) / 4)), dim3(256), 0, stream>>>(a, nheads);
  } else {
    attn_combine_kernel<<<dim3((unsigned)Hq, (unsigned)B), dim3(256), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace qr
