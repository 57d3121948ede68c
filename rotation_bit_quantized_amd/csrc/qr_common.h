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

}  // namespace qr
