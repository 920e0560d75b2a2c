// Fixed-point digit operands of the fp8 x fp4 matrix cores, shared by the
// kernels that multiply bf16 activation rows by +-1 weights that way (see
// the single-row product in dec.hip for the full statement of the scheme):
// per wave slice of a row, 2^e the largest power of two (biased exponent
// ebs), every |x| becomes the 24-bit integer X = trunc(|x| * 2^(150 - ebs));
// its six 4-bit digits (most significant first) are sign-magnitude e4m3 codes
// (code c <= 15 is c * 2^-9) with block exponent ebs - 2 - 4p for digit p
// (the zero row takes exponent 0: ebs - 26 would reach the E8M0 NaN code),
// against weights +-6 in fp4: every product and partial sum is an integer
// times one power of two, exact in fp32. The single-row kernel in dec.hip
// keeps its own inline form of these steps: built on these helpers it
// compiled to the same instructions in another order and measured about 1 %
// slower on one of the decode launch shapes.
#pragma once

#include "common.h"

namespace brq {

typedef int f4_i32x8 __attribute__((ext_vector_type(8)));

// (group, word) transpose across the four 16-lane rows: on entry register w
// of row g holds word w of group g; on exit register i of row b holds word b
// of group i
__device__ __forceinline__ void f4_transpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = d[0];
  r3 = d[1];
}

// biased exponent of the largest |x| of a wave's slice (at least 24, so that
// zeros and bf16 subnormals fall out of the 24-bit field) and 2^(150 - ebs)
template <int C>
__device__ __forceinline__ uint32_t f4_slice_exponent(const uint4 (&v)[C], float& S) {
  uint32_t mx = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const uint32_t w4[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) mx = max(mx, max(w4[h] & 0x7fffu, (w4[h] >> 16) & 0x7fffu));
  }
  mx = wave_max_u32(mx);
  const uint32_t ebs = max(mx >> 7, 24u);
  S = __uint_as_float((277u - ebs) << 23);
  return ebs;
}

// the six digit rows of lane L's 8 values (k = 8L .. 8L+7 of a 512-wide
// chunk: group L/16, word (L%16)/4) into LDS rows row0 .. row0 + 5 of the
// lane's group; base = the region + (L/16) * group stride + 32 ((L%16)/4) +
// 2 (L%4). Value e lands at in-word position 8 (e%4) + 2 (L%4) + e/4.
__device__ __forceinline__ void f4_digits(const uint4 v, float S, uint8_t* base, int row0) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
  uint32_t lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t wp = (e & 1) ? (w4[e >> 1] & 0xffff0000u) : (w4[e >> 1] << 16);
    const uint32_t X = (uint32_t)(fabsf(__uint_as_float(wp)) * S);
    const uint32_t sr = (wp >> 31) * 0x808080u;
    lo[e] = (X & 0x0f0f0fu) | sr;
    hi[e] = ((X >> 4) & 0x0f0f0fu) | sr;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t l02 = __builtin_amdgcn_perm(lo[t + 4], lo[t], 0x05010400u);
    const uint32_t l4 = __builtin_amdgcn_perm(lo[t + 4], lo[t], 0x0c0c0602u);
    const uint32_t h13 = __builtin_amdgcn_perm(hi[t + 4], hi[t], 0x05010400u);
    const uint32_t h5 = __builtin_amdgcn_perm(hi[t + 4], hi[t], 0x0c0c0602u);
    auto put = [&](int nib, uint32_t v16) {
      *reinterpret_cast<uint16_t*>(base + (row0 + 5 - nib) * 128 + 8 * t) = (uint16_t)v16;
    };
    put(0, l02);
    put(2, l02 >> 16);
    put(4, l4);
    put(1, h13);
    put(3, h13 >> 16);
    put(5, h5);
  }
}

// biased exponent of the largest |v| of a wave's slice of fp32 values (8 per
// lane per chunk), at least 24, and 2^(150 - ebs)
template <int C>
__device__ __forceinline__ uint32_t f4_slice_exponent_f32(const f32x4 (&v)[C][2], float& S) {
  uint32_t mx = 0;
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = max(mx, __float_as_uint(v[c][h][i]) & 0x7fffffffu);
  mx = wave_max_u32(mx);
  const uint32_t ebs = max(mx >> 23, 24u);
  S = __uint_as_float((277u - ebs) << 23);
  return ebs;
}

// as f4_digits for 8 fp32 values (v[0] holds values 0..3, v[1] 4..7): each
// |v| becomes trunc(|v| * 2^(150 - ebs)), the bits below 2^-23 of the slice
// maximum dropped
__device__ __forceinline__ void f4_digits_f32(const f32x4 (&v)[2], float S, uint8_t* base, int row0) {
  uint32_t lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = v[e >> 2][e & 3];
    const uint32_t X = (uint32_t)(fabsf(f) * S);
    const uint32_t sr = (__float_as_uint(f) >> 31) * 0x808080u;
    lo[e] = (X & 0x0f0f0fu) | sr;
    hi[e] = ((X >> 4) & 0x0f0f0fu) | sr;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t l02 = __builtin_amdgcn_perm(lo[t + 4], lo[t], 0x05010400u);
    const uint32_t l4 = __builtin_amdgcn_perm(lo[t + 4], lo[t], 0x0c0c0602u);
    const uint32_t h13 = __builtin_amdgcn_perm(hi[t + 4], hi[t], 0x05010400u);
    const uint32_t h5 = __builtin_amdgcn_perm(hi[t + 4], hi[t], 0x0c0c0602u);
    auto put = [&](int nib, uint32_t v16) {
      *reinterpret_cast<uint16_t*>(base + (row0 + 5 - nib) * 128 + 8 * t) = (uint16_t)v16;
    };
    put(0, l02);
    put(2, l02 >> 16);
    put(4, l4);
    put(1, h13);
    put(3, h13 >> 16);
    put(5, h5);
  }
}

// one scale group of 16 columns: A from LDS (32 bytes per lane at ab, digit
// row of the lane), B the +-6 operands of sign word w, block exponent sa
__device__ __forceinline__ f32x4 f4_group_mfma(const uint8_t* ab, uint32_t w, int sa) {
  const u32x4 a0 = *reinterpret_cast<const u32x4*>(ab);
  const u32x4 a1 = *reinterpret_cast<const u32x4*>(ab + 64);
  f4_i32x8 A, B;
  A[0] = a0[0]; A[1] = a0[1]; A[2] = a0[2]; A[3] = a0[3];
  A[4] = a1[0]; A[5] = a1[1]; A[6] = a1[2]; A[7] = a1[3];
  B[0] = (int)((w << 3) | 0x77777777u);
  B[1] = (int)((w << 2) | 0x77777777u);
  B[2] = (int)((w << 1) | 0x77777777u);
  B[3] = (int)(w | 0x77777777u);
  B[4] = 0; B[5] = 0; B[6] = 0; B[7] = 0;
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0, sa, 0, 135);
}

}  // namespace brq
