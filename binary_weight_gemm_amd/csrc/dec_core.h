// Few-row binary product core (the decode regime: a matrix applied to one or a
// few vectors, "LLM binarization, Episode 01: DBF", section 4).
//
// Work split: a workgroup owns 16 output columns (16 weight rows n0..n0+15);
// its waves split the reduction axis K in chunks of 512 (4 groups of 128).
// Inside a wave, lane l = 16*kb + j reads group (4*chunk + kb) of weight row
// n0 + j with one 16-byte load of sign bits; those 128 signs become 16 MFMA
// weight operands (v_mfma_f32_16x16x32_f16, B operand: 8 fp16 per lane), each
// built with one shift and one and-or per pair of weights. The activation
// operand (A: up to 16 rows, one per token or per fp16 piece) is read from the
// permuted fp16 staging buffer, 16 bytes per lane per MFMA. Partial sums of the
// waves meet in LDS and are added in wave order (deterministic).
//
// Layout facts of the 16x16x32 MFMA used here: A lane l supplies row l%16 and
// 8 consecutive k of block l/16; B lane l supplies column l%16 and the same k
// block; D lane l holds rows 4*(l/16)+i (i = 0..3) of column l%16.
#pragma once

#include "common.h"

namespace brq {

// BMODE: how the magnitude of a weight operand is formed
enum { BM_GROUP = 0,  // group-128 fp16 scale of (row, group)
       BM_PERK = 1,   // per-k fp16 value shared by all rows (DBF input diagonal)
       BM_ONE = 2 };  // +-1

template <int BMODE, int NB, int TT>
__device__ __forceinline__ void dec_core(const uint4* const (&wsig)[NB],      // row start, uint4 per group
                                         const uint16_t* const (&wsc)[NB],    // row scales (BM_GROUP)
                                         const u32x4* __restrict__ kp,        // BM_PERK magnitudes
                                         const u32x4* const (&arow)[TT],      // A row starts (NULL: zero row)
                                         int G, int c0, int cstep, f32x4 (&acc)[NB][TT]) {
  const int kb = (threadIdx.x & 63) >> 4;
  for (int c = c0; 4 * c < G; c += cstep) {
    const int g = 4 * c + kb;
    const bool ok = g < G;
    uint4 d[NB];
    uint32_t S[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      d[nb] = make_uint4(0, 0, 0, 0);
      S[nb] = (BMODE == BM_ONE) ? 0x3c003c00u : 0u;
      if (ok && wsig[nb]) {
        d[nb] = wsig[nb][g];
        if (BMODE == BM_GROUP) {
          const uint32_t s = wsc[nb][g];
          S[nb] = s | (s << 16);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      u32x4 a[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        a[tt] = u32x4{0, 0, 0, 0};
        if (ok && arow[tt]) a[tt] = arow[tt][g * 16 + i];
      }
      u32x4 mk = u32x4{0, 0, 0, 0};
      if (BMODE == BM_PERK && ok) mk = kp[g * 16 + i];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t dw = (i < 4) ? d[nb].x : (i < 8) ? d[nb].y : (i < 12) ? d[nb].z : d[nb].w;
        u32x4 b;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int bit = 4 * (i & 3) + t;
          const uint32_t mag = (BMODE == BM_PERK) ? mk[t] : S[nb];
          b[t] = ((dw << (15 - bit)) & 0x80008000u) | mag;
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[nb][tt] = mfma16(a[tt], b, acc[nb][tt]);
      }
    }
  }
}

// Sum the per-wave partial tiles into wave 0 (wave order, deterministic).
// `red` must hold (waves-1)*NB*TT*64 f32x4 of shared memory.
template <int NB, int TT>
__device__ __forceinline__ void reduce_waves(f32x4 (&acc)[NB][TT], f32x4* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (nw == 1) return;
  if (wave > 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) red[(((wave - 1) * NB + nb) * TT + tt) * 64 + lane] = acc[nb][tt];
  }
  __syncthreads();
  if (wave == 0) {
    for (int w = 1; w < nw; ++w)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[nb][tt] += red[(((w - 1) * NB + nb) * TT + tt) * 64 + lane];
  }
}

// waves per workgroup for a reduction length of G groups: one to two chunks of
// 512 per wave, at most 16 waves
static inline int dec_waves(int G) {
  const int chunks = (G + 3) / 4;
  int w = chunks;
  if (w > 16) w = (chunks + 1) / 2;
  if (w > 16) w = 16;
  return w < 1 ? 1 : w;
}

// position of column index n inside a permuted row
__device__ __forceinline__ int perm_pos(int n) { return (n & ~31) + perm32(n & 31); }

}  // namespace brq
