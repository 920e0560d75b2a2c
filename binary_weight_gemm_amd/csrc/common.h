// Shared device helpers for the gfx950 kernels of libbrq.
//
// Operand scheme used by every binary product in this library
// ------------------------------------------------------------
// A binary weight only chooses between +x and -x ("LLM binarization,
// Episode 01: DBF", section 1). The products here run on the fp16 matrix
// cores: the weight operand of an MFMA is built in registers as the fp16 value
// +-c, where c is the group scale (group-128 format), a per-k diagonal entry
// (the DBF input diagonal) or 1.0. A scale is never negative, so the operand
// is the sign bit OR-ed onto c: one shift and one and-or per pair of weights;
// a diagonal entry is real-valued and may be negative, so there the weight's
// sign bit is XOR-ed onto c's (one shift, one and, one xor). Both
// operands are exact in fp16 and every product is exact in the fp32
// accumulator.
//
// The shift trick needs the two weights of an fp16 pair to sit 16 bits apart
// in a 32-bit sign word. Inside every run of 32 consecutive k the operands are
// therefore taken in the order
//      slot 2*b + h  <->  k = 16*h + b      (b = 0..15, h = 0..1)
// for both the weight and the activation operand. A matrix-core product sums
// over all k of its operands, so any order shared by both operands gives the
// same sum; activations are written in this order ("permuted") before they are
// fed to the matrix cores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace brq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// fp16 weight pair for bits (b, b+16) of sign word `dw`: the two sign bits are
// moved to bit 15 and bit 31 and OR-ed onto the (non-negative) magnitude pair.
template <int B>
__device__ __forceinline__ uint32_t sign_pair(uint32_t dw, uint32_t mag2) {
  return ((dw << (15 - B)) & 0x80008000u) | mag2;
}

// Four consecutive pairs b = 4*Q .. 4*Q+3 (one MFMA operand's worth for a lane).
template <int Q>
__device__ __forceinline__ u32x4 sign_quad(uint32_t dw, uint32_t mag2) {
  u32x4 r;
  r[0] = sign_pair<4 * Q + 0>(dw, mag2);
  r[1] = sign_pair<4 * Q + 1>(dw, mag2);
  r[2] = sign_pair<4 * Q + 2>(dw, mag2);
  r[3] = sign_pair<4 * Q + 3>(dw, mag2);
  return r;
}

template <int Q>
__device__ __forceinline__ u32x4 sign_quad4(uint32_t dw, u32x4 mag2) {
  u32x4 r;
  r[0] = sign_pair<4 * Q + 0>(dw, mag2[0]);
  r[1] = sign_pair<4 * Q + 1>(dw, mag2[1]);
  r[2] = sign_pair<4 * Q + 2>(dw, mag2[2]);
  r[3] = sign_pair<4 * Q + 3>(dw, mag2[3]);
  return r;
}

// Position of element k (0..31 within a run of 32) in the permuted order.
__host__ __device__ __forceinline__ int perm32(int k) { return 2 * (k & 15) + (k >> 4); }

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest, ties to even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN): gfx950's
// hardware conversion.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  const __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// fp32 value as an fp16 hi/lo pair: hi = fp16(v), lo = fp16(v - hi).
__device__ __forceinline__ void split_f16(float v, uint16_t& hi, uint16_t& lo) {
  _Float16 h = (_Float16)v;
  float r = v - (float)h;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, (_Float16)r);
}

// Largest value of the wave, returned to every lane (uniform): quad swaps,
// half-row and row mirrors, then the row broadcasts carry it to lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ void store_out(void* y, size_t idx, float v, int out_bf16) {
  if (out_bf16)
    reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(y)[idx] = v;
}

}  // namespace brq
