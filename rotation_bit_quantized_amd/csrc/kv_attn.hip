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
// and the value side accumulates sum_t w_t c_t - sum_t w_t z_t with
// w_t = p_t D_t, all in fp32.
//
// Layout of the work: one block of four waves per (sequence, query head,
// chunk of tokens).  Lane (tau, qd) = (lane >> 2, lane & 3) holds dims
// 32 qd .. 32 qd + 31 of token tau of a 16-token step: its 16-byte quarter of
// the token's 64-byte code row, so one load instruction reads 16 whole code
// rows.  Online softmax per group of four steps (64 tokens per wave).  A
// sequence split into several chunks leaves one partial (max, sum, 128
// accumulators) per chunk in the caller's workspace; a second kernel merges
// them.
#include "qr_common.h"
#include "qr_launch.h"

namespace qr {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kStep = 16;          // tokens per wave step
constexpr int kGroup = 4;          // steps per online-softmax group
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
  const unsigned short *q;         // [B][Hq][128] fp16
  const uint8_t *kc, *vc;          // [B][T][Hkv][64]
  const float *ks, *vs;            // [B][T][Hkv]
  const uint8_t *kz, *vz;          // [B][T][Hkv]
  const int *lens;                 // [B] or null
  const int8_t *signs;             // [128] or null
  float qmul;                      // sm_scale * log2(e) / sqrt(128)
  int T, Hq, Hkv, group, chunk, splits;
  float *ws;                       // [B][Hq][splits][kPart] when splits > 1
  unsigned short *out;             // [B][Hq][128] fp16
};

constexpr int kPart = 132;         // m, l, 2 pad, o[128]

// Hides a value's known bits from the optimiser, so that byte k of a masked
// word converts with one v_cvt_f32_ubyte<k> instead of a bit-field extract
// followed by a conversion.
__device__ __forceinline__ void opaque(unsigned &v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float half_to_float(unsigned short h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ unsigned short float_to_half(float f) {
  return __builtin_bit_cast(unsigned short, (_Float16)f);
}

// In-place unnormalised 128-point Walsh-Hadamard transform of buf[0..127]
// by threads 0..63 of the block (one butterfly pair each per level); every
// thread of the block must call it.
__device__ __forceinline__ void wht128_lds(float *buf) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 1; h < kD; h <<= 1) {
    __syncthreads();
    if (tid < kD / 2) {
      const int i = (tid / h) * 2 * h + (tid % h);
      const float a = buf[i], b = buf[i + h];
      buf[i] = a + b;
      buf[i + h] = a - b;
    }
  }
  __syncthreads();
}

// out = (o / l) R^T = WHT(o / l) * signs / sqrt(128), fp16; zeros when l == 0.
// buf holds o on entry (threads 0..127 wrote it); every thread calls this.
__device__ __forceinline__ void finish_output(float *buf, float l, const int8_t *signs, unsigned short *out) {
  const int tid = threadIdx.x;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  __syncthreads();
  if (tid < kD) buf[tid] *= inv;
  wht128_lds(buf);
  if (tid < kD) {
    float v = buf[tid] * 0.08838834764831845f;   // 1/sqrt(128)
    if (signs != nullptr && signs[tid] < 0) v = -v;
    out[tid] = float_to_half(v);
  }
}

__global__ __launch_bounds__(64 * kWaves) void attn_decode_kernel(AttnArgs a) {
  __shared__ float qbuf[kD];
  __shared__ float wpart[kWaves][kD];
  __shared__ float wml[kWaves][2];
  __shared__ float qsum_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int s = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int hk = hq / a.group;
  const int qd = lane & 3, tau = lane >> 2;

  int len = a.lens != nullptr ? a.lens[b] : a.T;
  len = len < 0 ? 0 : (len > a.T ? a.T : len);
  const int t0 = s * a.chunk;
  const int t1 = t0 + a.chunk < len ? t0 + a.chunk : len;

  // ---- q' = (q * signs) H_128 * qmul, and its sum
  if (tid < kD) {
    float v = half_to_float(a.q[((int64_t)b * a.Hq + hq) * kD + tid]);
    if (a.signs != nullptr && a.signs[tid] < 0) v = -v;
    qbuf[tid] = v;
  }
  wht128_lds(qbuf);
  if (tid < 64) {
    float v = (qbuf[2 * tid] + qbuf[2 * tid + 1]) * a.qmul;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    if (tid == 0) qsum_s = v;
  }
  __syncthreads();
  float qv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) qv[i] = qbuf[32 * qd + i] * a.qmul;
  const float qsum = qsum_s;

  // ---- this wave's tokens: steps j with token base t0 + (j * kWaves + wave) * kStep
  const int64_t tok_stride = (int64_t)a.Hkv;                  // rows of 64 bytes between tokens
  const int64_t seq_row0 = (int64_t)b * a.T * a.Hkv + hk;      // row index of token 0
  float m = -__builtin_inff();
  float l = 0.f, zacc = 0.f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;

  const int nsteps = (t1 - t0 + kStep - 1) / kStep;            // over the block; t1 <= t0 gives <= 0
  for (int j0 = wave; j0 < nsteps; j0 += kWaves * kGroup) {
    v4u kw[kGroup], vw[kGroup];
    float kd[kGroup], vd[kGroup], kzf[kGroup], vzf[kGroup];
    bool ok[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int t = t0 + (j0 + g * kWaves) * kStep + tau;
      ok[g] = t < t1;
      const int tc = ok[g] ? t : t1 - 1;                       // in-range row for masked lanes
      const int64_t row = seq_row0 + (int64_t)tc * tok_stride;
      kw[g] = *(const v4u *)(a.kc + row * 64 + 16 * qd);
      vw[g] = *(const v4u *)(a.vc + row * 64 + 16 * qd);
      kd[g] = a.ks[row];
      vd[g] = a.vs[row];
      kzf[g] = (float)a.kz[row];
      vzf[g] = (float)a.vz[row];
    }
    float sc[kGroup];
    float gmax = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      float dot = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        unsigned lo = kw[g][w] & 0x0F0F0F0Fu, hi = (kw[g][w] >> 4) & 0x0F0F0F0Fu;
        opaque(lo);
        opaque(hi);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          dot = __builtin_fmaf(qv[8 * w + 2 * k], (float)((lo >> (8 * k)) & 0xFFu), dot);
          dot = __builtin_fmaf(qv[8 * w + 2 * k + 1], (float)((hi >> (8 * k)) & 0xFFu), dot);
        }
      }
      dot += dpp<kQuadXor1>(dot);
      dot += dpp<kQuadXor2>(dot);
      sc[g] = ok[g] ? kd[g] * (dot - kzf[g] * qsum) : -__builtin_inff();
      gmax = fmaxf(gmax, sc[g]);
    }
    gmax = wave_max_dpp(gmax);
    const float m_new = fmaxf(m, gmax);
    const float m_ref = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
    m = m_new;
    l *= alpha;
    zacc *= alpha;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] *= alpha;
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const float p = __builtin_amdgcn_exp2f(sc[g] - m_ref);
      l += p;
      const float w8 = p * vd[g];
      zacc = __builtin_fmaf(w8, vzf[g], zacc);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        unsigned lo = vw[g][w] & 0x0F0F0F0Fu, hi = (vw[g][w] >> 4) & 0x0F0F0F0Fu;
        opaque(lo);
        opaque(hi);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[8 * w + 2 * k] = __builtin_fmaf(w8, (float)((lo >> (8 * k)) & 0xFFu), acc[8 * w + 2 * k]);
          acc[8 * w + 2 * k + 1] = __builtin_fmaf(w8, (float)((hi >> (8 * k)) & 0xFFu), acc[8 * w + 2 * k + 1]);
        }
      }
    }
  }

  // ---- per wave: subtract the zero-point term, sum over the 16 tokens of a step
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float v = acc[i] - zacc;
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    acc[i] = v;
  }
  // l is the same in the four lanes of a token: sum one lane per token
  float lw = qd == 0 ? l : 0.f;
#pragma unroll
  for (int o = 4; o <= 32; o <<= 1) lw += __shfl_xor(lw, o);
  if (tau == 0) {
#pragma unroll
    for (int i = 0; i < 32; ++i) wpart[wave][32 * qd + i] = acc[i];
  }
  if (lane == 0) {
    wml[wave][0] = m;
    wml[wave][1] = lw;
  }
  __syncthreads();

  // ---- merge the four waves
  float mb = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mb = fmaxf(mb, wml[w][0]);
  const float mref = mb == -__builtin_inff() ? 0.f : mb;
  float lb = 0.f, ob = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float f = __builtin_amdgcn_exp2f(wml[w][0] - mref);
    lb += f * wml[w][1];
    if (tid < kD) ob += f * wpart[w][tid];
  }
  if (a.splits == 1) {
    if (tid < kD) qbuf[tid] = ob;
    finish_output(qbuf, lb, a.signs, a.out + ((int64_t)b * a.Hq + hq) * kD);
  } else {
    float *part = a.ws + (((int64_t)b * a.Hq + hq) * a.splits + s) * kPart;
    if (tid < kD) part[4 + tid] = ob;
    if (tid == 0) {
      part[0] = mb;
      part[1] = lb;
    }
  }
}

// Merge the chunks of one (sequence, query head): max, rescaled sums, output.
__global__ __launch_bounds__(kD) void attn_combine_kernel(AttnArgs a) {
  __shared__ float buf[kD];
  const int tid = threadIdx.x;
  const int hq = blockIdx.x, b = blockIdx.y;
  const float *part = a.ws + ((int64_t)b * a.Hq + hq) * a.splits * kPart;
  float mb = -__builtin_inff();
  for (int s = 0; s < a.splits; ++s) mb = fmaxf(mb, part[s * kPart]);
  const float mref = mb == -__builtin_inff() ? 0.f : mb;
  float lb = 0.f, ob = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float f = __builtin_amdgcn_exp2f(part[s * kPart] - mref);
    lb += f * part[s * kPart + 1];
    ob += f * part[s * kPart + 4 + tid];
  }
  buf[tid] = ob;
  finish_output(buf, lb, a.signs, a.out + ((int64_t)b * a.Hq + hq) * kD);
}

}  // namespace

AttnPlan attn_decode_plan(int64_t B, int64_t Hq, int64_t T) {
  const int64_t cus = 256;   // the split depends on the shape only, not on the device
  AttnPlan p{};
  const int64_t pairs = B * Hq;
  int64_t splits = 1;
  if (T > 256 && pairs > 0) {
    const int64_t want = (8LL * cus + pairs - 1) / pairs;          // about eight blocks per CU
    const int64_t most = (T + 255) / 256;                            // chunks of at least 256 tokens
    splits = want < most ? want : most;
    if (splits < 1) splits = 1;
  }
  int64_t chunk = (T + splits - 1) / splits;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk < 64) chunk = 64;
  p.chunk = chunk;
  p.splits = (T + chunk - 1) / chunk;
  if (p.splits < 1) p.splits = 1;
  p.workspace_bytes = p.splits > 1 ? pairs * p.splits * kPart * (int64_t)sizeof(float) : 0;
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
  a.group = (int)(Hq / Hkv);
  a.chunk = (int)plan.chunk;
  a.splits = (int)plan.splits;
  a.ws = ws;
  a.out = (unsigned short *)out;
  attn_decode_kernel<<<dim3((unsigned)plan.splits, (unsigned)Hq, (unsigned)B), dim3(64 * kWaves), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  attn_combine_kernel<<<dim3((unsigned)Hq, (unsigned)B), dim3(kD), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qr
