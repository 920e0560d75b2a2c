// Quantiser: fp32 weights -> SIGN1 sign plane (+ one fp16 scale per group of 128).
//
// Format of "Behaviour-Relearned Quantization" (item 02: sign bits with one scale
// per 128 of them) and "Banyan ..." (Abstract, 1.125 bits per weight); sign convention
// and 64-sign words of "LLM binarization, Episode 01: DBF" (sections 1, 3).
//
// Mapping: a row-major [rows][cols] matrix with cols % 128 == 0 is a flat run of
// rows*cols/128 groups, group G at w + 128*G, its sign words at 2*G and 2*G+1,
// its scale at G. One wave packs 64 consecutive groups: for each group the 64
// lanes read 2 x 256 contiguous bytes, two wave ballots of the IEEE sign bits
// give the two 64-bit words directly (lane l <-> bit l), and sum|w| is added
// in fp64 (each lane's two values, then the 64 lane partials in lane order).
// Lane i keeps group i's results so the stores are coalesced.
#include "common.h"
#include "kernels.h"

namespace brq {

// fp64 -> fp16 bits, one rounding to nearest, ties to even, straight from fp64
// (no detour through fp32, which could round twice).
__device__ uint16_t f64_to_f16_rne(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int ex = (int)((b >> 52) & 0x7ff);
  const uint64_t mant = b & ((1ull << 52) - 1);
  if (ex == 0x7ff) return sign | 0x7c00u | (mant ? 0x200u : 0u);
  if (ex == 0) return sign;  // fp64 subnormal: far below fp16's range
  int e = ex - 1023;
  if (e > 15) return sign | 0x7c00u;
  if (e < -25) return sign;
  const uint64_t sig = mant | (1ull << 52);
  const int shift = (e >= -14) ? 42 : 42 + (-14 - e);  // bits dropped
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (e >= -14) {
    if (q == 2048) { q = 1024; ++e; }
    if (e > 15) return sign | 0x7c00u;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q & 0x3ffu);
  }
  return sign | (uint16_t)q;  // subnormal (q == 1024 encodes the smallest normal)
}

__global__ __launch_bounds__(256) void k_pack_g128(const float* __restrict__ w, int64_t ngroups,
                                                   uint64_t* __restrict__ signs,
                                                   uint16_t* __restrict__ scales) {
  // per wave: |w| partials of 16 groups x 64 lanes, summed by the 16 lanes
  // that keep those groups (a transposed reduction instead of one butterfly
  // per group)
  __shared__ double part[4][16][65];  // rows padded: the 16 summing lanes hit different banks
  const int lane = threadIdx.x & 63, wl = threadIdx.x >> 6;
  const int64_t wv = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t t0 = wv * 64; t0 < ngroups; t0 += nw * 64) {
    const int cnt = (int)((ngroups - t0) < 64 ? (ngroups - t0) : 64);
    uint64_t my0 = 0, my1 = 0;
    double mysum = 0.0;
    // sixteen groups per round: all their loads first (groups past cnt
    // re-read the last one and are dropped), then the ballots, then the sums
    for (int i0 = 0; i0 < cnt; i0 += 16) {
      float a[16], c[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = i0 + q < cnt ? i0 + q : cnt - 1;
        const float* src = w + (t0 + i) * 128;
        a[q] = src[lane];
        c[q] = src[64 + lane];
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint64_t b0 = __ballot(__float_as_uint(a[q]) >> 31);
        const uint64_t b1 = __ballot(__float_as_uint(c[q]) >> 31);
        if (lane == i0 + q) { my0 = b0; my1 = b1; }
        part[wl][q][lane] = (double)fabsf(a[q]) + (double)fabsf(c[q]);
      }
      // lane i0 + q adds group i0 + q's 64 partials in lane order (the LDS
      // operations of one wave complete in order, so no barrier is needed)
      const int q = lane - i0;
      if (q >= 0 && q < 16) {
        double sum = 0.0;
        for (int j = 0; j < 64; ++j) sum += part[wl][q][j];
        mysum = sum;
      }
    }
    if (lane < cnt) {
      signs[2 * (t0 + lane)] = my0;
      signs[2 * (t0 + lane) + 1] = my1;
      scales[t0 + lane] = f64_to_f16_rne(mysum * 0.0078125);  // exact division by 128
    }
  }
}

__global__ __launch_bounds__(256) void k_pack_sign1(const float* __restrict__ w, int64_t nwords,
                                                    uint64_t* __restrict__ signs) {
  const int lane = threadIdx.x & 63;
  const int64_t wv = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t t0 = wv * 64; t0 < nwords; t0 += nw * 64) {
    const int cnt = (int)((nwords - t0) < 64 ? (nwords - t0) : 64);
    uint64_t my = 0;
    for (int i0 = 0; i0 < cnt; i0 += 8) {  // eight words per round, loads first
      float a[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) a[q] = w[(t0 + (i0 + q < cnt ? i0 + q : cnt - 1)) * 64 + lane];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint64_t b = __ballot(__float_as_uint(a[q]) >> 31);
        if (lane == i0 + q) my = b;
      }
    }
    if (lane < cnt) signs[t0 + lane] = my;
  }
}

static int pack_grid(int64_t units) {
  int64_t waves = (units + 63) / 64;
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

hipError_t launch_pack(const float* w, int64_t rows, int64_t cols, uint64_t* signs,
                       uint16_t* scales, hipStream_t st) {
  if (scales) {
    const int64_t ng = rows * (cols / 128);
    hipLaunchKernelGGL(k_pack_g128, dim3(pack_grid(ng)), dim3(256), 0, st, w, ng, signs, scales);
  } else {
    const int64_t nwd = rows * (cols / 64);
    hipLaunchKernelGGL(k_pack_sign1, dim3(pack_grid(nwd)), dim3(256), 0, st, w, nwd, signs);
  }
  return hipGetLastError();
}

}  // namespace brq
