// Shared device helpers for the gfx950 kernels of the QuaRot hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qr {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// 1.5 * 2^23: adding it to |v| < 2^22 leaves rint(v) (half to even, the
// hardware default) in the low mantissa bits, two's complement.
constexpr float kRoundMagic = 12582912.0f;

__device__ __forceinline__ unsigned f2u(float f) { return __builtin_bit_cast(unsigned, f); }
__device__ __forceinline__ float u2f(unsigned u) { return __builtin_bit_cast(float, u); }

// rint(v * inv) as the low bits of the returned word, in one fused op.
__device__ __forceinline__ unsigned round_bits(float v, float inv) {
  return f2u(__builtin_fmaf(v, inv, kRoundMagic));
}

// Pack the low nibbles of eight words, element 0 in the lowest nibble.
__device__ __forceinline__ unsigned pack8_nibbles(unsigned b0, unsigned b1, unsigned b2, unsigned b3,
                                                  unsigned b4, unsigned b5, unsigned b6, unsigned b7) {
  unsigned lo01 = (b0 & 0xFu) | ((b1 & 0xFu) << 4);
  unsigned lo23 = (b2 & 0xFu) | ((b3 & 0xFu) << 4);
  unsigned lo45 = (b4 & 0xFu) | ((b5 & 0xFu) << 4);
  unsigned lo67 = (b6 & 0xFu) | ((b7 & 0xFu) << 4);
  return lo01 | (lo23 << 8) | (lo45 << 16) | (lo67 << 24);
}

__device__ __forceinline__ float half_bits_to_float(unsigned short h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ unsigned short float_to_half_bits(float f) {
  return __builtin_bit_cast(unsigned short, (_Float16)f);
}

// XOR masks that flip the fp16 sign of elements whose int8 sign is negative,
// for four consecutive int8 signs packed in one word: elements 0, 1 go to
// (bit 15, bit 31) of m01, elements 2, 3 to those of m23.
__device__ __forceinline__ void sign_masks4(unsigned w, unsigned &m01, unsigned &m23) {
  m01 = ((w & 0x80u) << 8) | ((w & 0x8000u) << 16);
  m23 = ((w & 0x800000u) >> 8) | (w & 0x80000000u);
}

// Wave-wide (64 lanes) reductions.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}


// ---- synchronisation, lane exchange and LDS-DMA helpers

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0), vmcnt and expcnt left alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wave priority 3, 2, 1, 0 for iterations k = 0, 1, 2, 3 (mod 4) of a
// persistent loop over rows or tiles (k wave-uniform).  Where waves of equal
// work share a SIMD, the hardware gives every issue tie to the older wave,
// so it finishes its share well ahead and the younger one then runs its last
// iterations alone; with the priority falling as a wave advances, the one
// that is ahead yields to the one behind and both finish together.
__device__ __forceinline__ void set_prio_by_progress(int k) {
  switch (k & 3) {
    case 0: __builtin_amdgcn_s_setprio(3); break;
    case 1: __builtin_amdgcn_s_setprio(2); break;
    case 2: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// 2 x 2 transposes of (register, lane bit 4) and (register, lane bit 5).
__device__ __forceinline__ void swap16(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane16_swap(f2u(a), f2u(b), false, false);
  a = u2f(r[0]);
  b = u2f(r[1]);
}
__device__ __forceinline__ void swap32(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane32_swap(f2u(a), f2u(b), false, false);
  a = u2f(r[0]);
  b = u2f(r[1]);
}
__device__ __forceinline__ void swap16u(unsigned &a, unsigned &b) {
  auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap32u(unsigned &a, unsigned &b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// 32 packed 4-bit codes (16 bytes) -> two int8 MFMA operands of 16 values
// 16 q each, in "high-nibble" form: lo = (w << 4) & 0xF0F0F0F0 and
// hi = w & 0xF0F0F0F0 (exact for q in [-8, 7], three VALU ops per 8 codes).
// The k order inside a dword is permuted; widening both GEMM operands the
// same way makes the permutation cancel, and the sum carries 256 q_a q_w.
__device__ __forceinline__ void widen_hi_nibble(const v4u &w, v4i &op0, v4i &op1) {
  op0[0] = (int)((w[0] << 4) & 0xF0F0F0F0u);
  op0[1] = (int)(w[0] & 0xF0F0F0F0u);
  op0[2] = (int)((w[1] << 4) & 0xF0F0F0F0u);
  op0[3] = (int)(w[1] & 0xF0F0F0F0u);
  op1[0] = (int)((w[2] << 4) & 0xF0F0F0F0u);
  op1[1] = (int)(w[2] & 0xF0F0F0F0u);
  op1[2] = (int)((w[3] << 4) & 0xF0F0F0F0u);
  op1[3] = (int)(w[3] & 0xF0F0F0F0u);
}

template <int CTRL>
__device__ __forceinline__ unsigned dpp(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return u2f(dpp<CTRL>(f2u(v)));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Max over the 64 lanes without LDS: DPP within rows of 16, then the
// row-pair swaps.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));   // lanes i and 7 - i of each half row
  v = fmaxf(v, dpp<kRowMirror>(v));       // lanes i and 15 - i of each row
  auto a = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  v = fmaxf(u2f(a[0]), u2f(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  return fmaxf(u2f(b[0]), u2f(b[1]));
}

// LDS address (byte offset in the workgroup's LDS) of a __shared__ pointer.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// One wave-instruction of global -> LDS DMA: lane l's 16 bytes at src land at
// LDS byte dst + 16 l (dst wave-uniform).  Issued from inline assembly: the
// compiler then does not see an LDS write it would wait for before every
// later LDS read it cannot prove disjoint (a full memory round trip); the
// caller orders uses with explicit vmcnt waits.  No register is written (the
// scratch SGPR keeps m0, which is reserved to the compiler).
__device__ __forceinline__ void dma16_to_lds(const void *src, unsigned dst) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(dst))
      : "memory");
}

}  // namespace qr
