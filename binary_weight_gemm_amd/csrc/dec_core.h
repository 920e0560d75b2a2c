// Few-row binary product core (the decode regime: a matrix applied to one or a
// few vectors, "LLM binarization, Episode 01: DBF", section 4).
//
// Work split: a workgroup owns 16 output columns (16 weight rows n0..n0+15);
// its waves split the reduction axis K in chunks of 512 (4 groups of 128),
// CPW chunks per wave. Inside a wave, lane l = 16*kb + j reads group
// (4*chunk + kb) of weight row n0 + j with one 16-byte load of sign bits; those
// 128 signs become 16 MFMA weight operands (v_mfma_f32_16x16x32_f16, B operand:
// 8 fp16 per lane), each built with one shift and one and-or per pair of
// weights. The activation operand (A: up to 16 rows, one per token or per fp16
// piece) comes from the permuted fp16 staging, 16 bytes per lane per MFMA.
//
// Latency: every wave issues the loads of its activation slice and of the
// sign/scale words of all its chunks before it waits for any of them; the
// slice is converted to the permuted fp16 order in a wave-private LDS region
// (stage_wave), so no wave waits on another wave's loads.
// Partial sums of the waves meet in LDS and are added in wave order
// (deterministic).
//
// Layout facts of the 16x16x32 MFMA used here: A lane l supplies row l%16 and
// 8 consecutive k of block l/16; B lane l supplies column l%16 and the same k
// block; D lane l holds rows 4*(l/16)+i (i = 0..3) of column l%16.
#pragma once

#include "common.h"
#include "gsync.h"

namespace brq {

// BMODE: how the magnitude of a weight operand is formed
enum { BM_GROUP = 0,  // group-128 fp16 scale of (row, group)
       BM_PERK = 1,   // per-k fp16 value shared by all rows (DBF input diagonal)
       BM_ONE = 2 };  // +-1

// Activation staging modes: ST_BF16 converts bf16 rows and permutes them,
// ST_F16 permutes fp16 rows, ST_COPY copies rows that are already permuted fp16.
enum { ST_BF16 = 0, ST_F16 = 1, ST_COPY = 2 };

template <int NB, int CPW>
struct BPre {
  uint4 d[NB][CPW];
  uint32_t s[NB][CPW];    // raw fp16 scale bits (BM_GROUP)
  bool ok[NB][CPW];       // group inside the matrix and row inside N
};

// Issue the sign (and scale) loads of chunks c0, c0+cstep, ... (CPW of them).
// Loads are unconditional (indices clamped to valid memory) and nothing is
// derived from the loaded values here, so no load waits for another; the
// validity masks are applied where the values are used.
template <int BMODE, int NB, int CPW>
__device__ __forceinline__ void b_prefetch(const uint4* const (&wsig)[NB], const uint16_t* const (&wsc)[NB],
                                           const bool (&row_ok)[NB], int G, int c0, int cstep, BPre<NB, CPW>& bp) {
  const int kb = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int g = 4 * (c0 + c * cstep) + kb;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bool ok = row_ok[nb] && g < G;
      const int gi = ok ? g : 0;
      bp.ok[nb][c] = ok;
      bp.d[nb][c] = wsig[nb][gi];
      if (BMODE == BM_GROUP) bp.s[nb][c] = wsc[nb][gi];
    }
  }
}

// MFMAs of the prefetched chunks. `aop(tt, g, i)` returns the A operand of row
// tile tt for MFMA i of group g; it is called for every lane with g clamped to
// G-1, so it must read valid, finite data for any row (rows past the end are
// never stored, and a zero weight operand cancels a clamped group).
// Two accumulators per tile alternate to halve the MFMA dependency chain.
// ALL: run every one of the CPW chunks (chunks past G contribute zero through
// the validity masks) so that the body has no branch; a branch here lets the
// compiler sink the prefetched loads into it, behind the first wait.
template <int BMODE, int NB, int TT, int CPW, bool ALL = false, class AOP>
__device__ __forceinline__ void b_compute(const BPre<NB, CPW>& bp, const u32x4* __restrict__ kp, int G, int c0,
                                          int cstep, AOP&& aop, f32x4 (&acc)[NB][TT]) {
  const int kb = (threadIdx.x & 63) >> 4;
  f32x4 acc2[NB][TT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc2[nb][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int chunk = c0 + c * cstep;
    if (!ALL && 4 * chunk >= G) break;  // uniform across the wave
    const int g = 4 * chunk + kb;
    const bool ok = g < G;
    const int ga = ok ? g : G - 1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      u32x4 a[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) a[tt] = aop(tt, ga, i);
      u32x4 mk = u32x4{0, 0, 0, 0};
      if (BMODE == BM_PERK) mk = kp[ga * 16 + i];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 d = bp.d[nb][c];
        const uint32_t dw = (i < 4) ? d.x : (i < 8) ? d.y : (i < 12) ? d.z : d.w;
        // magnitude pair; 0 for an out-of-range group or row (the operand is then +-0)
        uint32_t S = 0u;
        if (BMODE == BM_GROUP) S = bp.ok[nb][c] ? (bp.s[nb][c] | (bp.s[nb][c] << 16)) : 0u;
        if (BMODE == BM_ONE) S = bp.ok[nb][c] ? 0x3c003c00u : 0u;
        u32x4 b;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int bit = 4 * (i & 3) + t;
          const uint32_t mag = (BMODE == BM_PERK) ? (bp.ok[nb][c] ? mk[t] : 0u) : S;
          // a scale is never negative: the weight's sign bit is OR-ed on; a
          // per-k diagonal value may be, so its sign bit is flipped instead
          const uint32_t sw = (dw << (15 - bit)) & 0x80008000u;
          b[t] = (BMODE == BM_PERK) ? (sw ^ mag) : (sw | mag);
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          if (i & 1)
            acc2[nb][tt] = mfma16(a[tt], b, acc2[nb][tt]);
          else
            acc[nb][tt] = mfma16(a[tt], b, acc[nb][tt]);
        }
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[nb][tt] += acc2[nb][tt];
}

// Per-wave staging: the activation rows' values of chunks c0 .. c0+CPW-1 (a
// contiguous slice of K) go to the wave's LDS region xs, chunk c, row m at
// xs + (c*MAXR + m)*64 (uint4 units), in the permuted fp16 order. All MAXR x
// CPW slots are written (rows past `rows` repeat the last row, chunks past K
// repeat chunk 0): unconditional stores keep the compiler from sinking a
// load into a branch next to its store, which would make the first wait
// cover every load of the wave. Lane l
// handles pairs b = 4*(l%4) .. +3 of run l/4 of every (chunk, row): two 8-byte
// loads (k = b.. and k = 16+b..) and one 16-byte LDS store. The loads
// (WaveStage::load) are split from the conversion and store (WaveStage::store)
// so that a kernel can issue its weight loads in between. MODE as for
// stage_rows.
template <int MODE, int CPW, int MAXR>
struct WaveStage {
  uint2 lo[CPW][MAXR], hi[CPW][MAXR];
  // ST_BF16: each row of the wave's slice is staged as fp16(x * 2^s): s = 0
  // when the row's largest |x| lies in [2^-8, 2^15) (every bf16 value of at
  // least 2^-17 is exact in fp16 there, smaller ones move by at most 2^-25),
  // else the power of two that puts it in [2^14, 2^15) (no overflow at
  // 65504 whatever the magnitude, the same relative grid for tiny rows).
  // When every row is in that range (one wave maximum over the slice and one
  // ballot per row say so) no per-row maximum is taken. us[i] = -s of the row
  // whose MFMA output this lane holds in element i (rows 4kb .. 4kb+3 for lane
  // l = 16kb + j), undone exactly by unscale(). Other modes stage unscaled.
  int us[4];

  template <class ROWPTR>
  __device__ __forceinline__ void load(int rows, int K, int c0, ROWPTR&& rowptr) {
    const int lane = threadIdx.x & 63;
    const int run = lane >> 2, b0 = (lane & 3) * 4;
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int m = 0; m < MAXR; ++m) {
        // clamped, unconditional loads; out-of-range (chunk, row) slots are never stored
        const int kr = (c0 + c) * 512 + 32 * run;
        const int kc = kr < K ? kr : 0;
        const uint16_t* src = rowptr(m < rows ? m : rows - 1) + kc;
        if (MODE == ST_COPY) {
          lo[c][m] = *reinterpret_cast<const uint2*>(src + 2 * b0);
          hi[c][m] = *reinterpret_cast<const uint2*>(src + 2 * b0 + 4);
        } else {
          lo[c][m] = *reinterpret_cast<const uint2*>(src + b0);
          hi[c][m] = *reinterpret_cast<const uint2*>(src + 16 + b0);
        }
      }
  }

  __device__ __forceinline__ void store(uint4* xs) {
    const int lane = threadIdx.x & 63;
    const int run = lane >> 2, kb = lane >> 4;
    int sm[MAXR];
#pragma unroll
    for (int i = 0; i < 4; ++i) us[i] = 0;
#pragma unroll
    for (int m = 0; m < MAXR; ++m) sm[m] = 0;
    if (MODE == ST_BF16) {
      uint32_t lm[MAXR];  // this lane's largest |x| bits of each row
      uint32_t tm = 0;
#pragma unroll
      for (int m = 0; m < MAXR; ++m) {
        uint32_t mx = 0;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
          const uint32_t w4[4] = {lo[c][m].x, lo[c][m].y, hi[c][m].x, hi[c][m].y};
#pragma unroll
          for (int h = 0; h < 4; ++h) mx = max(mx, max(w4[h] & 0x7fffu, (w4[h] >> 16) & 0x7fffu));
        }
        lm[m] = mx;
        tm = max(tm, mx);
      }
      // every row in range: the slice's largest below 2^15 and a value of at
      // least 2^-8 in each row (bf16 exponent field 119 .. 141)
      bool all_in = wave_max_u32(tm) < (142u << 7);
#pragma unroll
      for (int m = 0; m < MAXR; ++m) all_in = all_in && __ballot(lm[m] >= (119u << 7)) != 0;
      if (!all_in) {  // uniform across the wave
#pragma unroll
        for (int m = 0; m < MAXR; ++m) {
          const int e = (int)(wave_max_u32(lm[m]) >> 7);  // biased exponent of the row's largest |x|
          sm[m] = (e >= 142 || e < 119) ? 141 - e : 0;   // an all-zero row gets 141: harmless
          // selected from scalars, not from an indexed array (which would go to scratch)
#pragma unroll
          for (int i = 0; i < 4; ++i) us[i] = (4 * kb + i == m) ? -sm[m] : us[i];
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int m = 0; m < MAXR; ++m) {
        uint32_t o[4];
        if (MODE == ST_COPY) {
          o[0] = lo[c][m].x; o[1] = lo[c][m].y; o[2] = hi[c][m].x; o[3] = hi[c][m].y;
        } else {
          const uint32_t l2[2] = {lo[c][m].x, lo[c][m].y}, h2[2] = {hi[c][m].x, hi[c][m].y};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (MODE == ST_BF16) {
              const uint32_t a = (t & 1) ? (l2[t >> 1] & 0xffff0000u) : (l2[t >> 1] << 16);
              const uint32_t b = (t & 1) ? (h2[t >> 1] & 0xffff0000u) : (h2[t >> 1] << 16);
              o[t] = (uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(__uint_as_float(a), sm[m])) |
                     ((uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(__uint_as_float(b), sm[m])) << 16);
            } else {
              const uint32_t a = (t & 1) ? (l2[t >> 1] >> 16) : (l2[t >> 1] & 0xffffu);
              const uint32_t b = (t & 1) ? (h2[t >> 1] >> 16) : (h2[t >> 1] & 0xffffu);
              o[t] = a | (b << 16);
            }
          }
        }
        xs[(c * MAXR + m) * 64 + run * 4 + (lane & 3)] = make_uint4(o[0], o[1], o[2], o[3]);
      }
  }

  // exponent that scales this lane's MFMA output element i back
  __device__ __forceinline__ int unscale(int i) const { return us[i]; }
};

// Per-wave staging of fp32 rows (intermediate vectors of a chain) as scaled
// fp16 pieces. Row m of the wave's slice becomes LDS rows 2m (hi) and 2m+1
// (lo) of u = v * 2^s[m]: hi = fp16(u), lo = fp16(u - hi). s[m] (uniform over
// the wave) puts the largest magnitude of the slice in [2^14, 2^15), so every
// value down to 2^-18 of that maximum keeps about 22 significant bits and the
// pieces never overflow, whatever the row's magnitude (an unscaled fp16 pair
// keeps fewer bits for every |v| < 2^-3, where lo is subnormal). A product of
// the two rows, added and scaled by 2^-s[m] (exact), is the product of the
// fp32 row to that precision. Slot (chunk c, piece row p) is xs + (c*2*MAXR +
// p)*64 (uint4 units) in the permuted order; loads are clamped as in
// WaveStage, so clamped chunks only enter the maximum with values of the row.
template <int CPW, int MAXR>
struct WaveStageF32 {
  f32x4 a[CPW][MAXR], b[CPW][MAXR];  // ext vectors: HIP float4 copies defeat SROA
  int us[2];  // -s of the rows 2kb and 2kb+1 (lane l = 16kb + j), the MFMA
              // output rows 4kb .. 4kb+3 of this lane being their pieces

  // COH: the rows were written by other workgroups of the same launch before a
  // grid-wide wait (gsync.h), so they are read at the device's coherence point
  template <bool COH = false, class ROWPTR>
  __device__ __forceinline__ void load(int rows, int K, int c0, ROWPTR&& rowptr) {
    const int lane = threadIdx.x & 63;
    const int run = lane >> 2, b0 = (lane & 3) * 4;
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int m = 0; m < MAXR; ++m) {
        const int kr = (c0 + c) * 512 + 32 * run;
        const int kc = kr < K ? kr : 0;
        const float* src = rowptr(m < rows ? m : rows - 1) + kc;
        if (COH) {
          const float4 u = coh_load4(src + b0), v = coh_load4(src + 16 + b0);
          a[c][m] = f32x4{u.x, u.y, u.z, u.w};
          b[c][m] = f32x4{v.x, v.y, v.z, v.w};
        } else {
          a[c][m] = *reinterpret_cast<const f32x4*>(src + b0);
          b[c][m] = *reinterpret_cast<const f32x4*>(src + 16 + b0);
        }
      }
  }

  __device__ __forceinline__ void store(uint4* xs) {
    const int lane = threadIdx.x & 63;
    const int run = lane >> 2, kb = lane >> 4;
    us[0] = us[1] = 0;
#pragma unroll
    for (int m = 0; m < MAXR; ++m) {
      uint32_t mx = 0;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        #pragma unroll
        for (int t = 0; t < 4; ++t)
          mx = max(mx, max(__float_as_uint(a[c][m][t]) & 0x7fffffffu, __float_as_uint(b[c][m][t]) & 0x7fffffffu));
      }
      mx = wave_max_u32(mx);
      const int sm = 14 - ((int)(mx >> 23) - 127);  // 0 -> s = 141, harmless: every value is 0
      // selected from scalars, not from an indexed array (which would go to scratch)
      us[0] = (2 * kb == m) ? -sm : us[0];
      us[1] = (2 * kb + 1 == m) ? -sm : us[1];
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        uint32_t oh[4], ol[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          uint16_t ha, la, hb, lb;
          split_f16(__builtin_amdgcn_ldexpf(a[c][m][t], sm), ha, la);
          split_f16(__builtin_amdgcn_ldexpf(b[c][m][t], sm), hb, lb);
          oh[t] = (uint32_t)ha | ((uint32_t)hb << 16);
          ol[t] = (uint32_t)la | ((uint32_t)lb << 16);
        }
        uint4* d = xs + (size_t)(c * 2 * MAXR + 2 * m) * 64 + run * 4 + (lane & 3);
        d[0] = make_uint4(oh[0], oh[1], oh[2], oh[3]);
        d[64] = make_uint4(ol[0], ol[1], ol[2], ol[3]);
      }
    }
  }

  // exponent that scales this lane's MFMA output row 4kb + i back
  __device__ __forceinline__ int unscale(int i) const { return us[i >> 1]; }
};

// Stage `rows` activation rows of K values in LDS as permuted fp16, row r at
// xs + r * (K/8) (uint4 units). MODE as below. rowptr(r) returns the global
// start of source row r.

template <int MODE, class ROWPTR>
__device__ __forceinline__ void stage_rows(uint4* xs, int rows, int K, ROWPTR&& rowptr) {
  const int rq = K >> 5;  // runs of 32 per row
  const int runs = rows * rq;
  for (int t = threadIdx.x; t < runs; t += blockDim.x) {
    const int r = t / rq, q = t - r * rq;
    const uint4* s = reinterpret_cast<const uint4*>(rowptr(r) + 32 * q);
    uint4* d = xs + (size_t)r * (K >> 3) + 4 * q;
    if (MODE == ST_COPY) {
      d[0] = s[0]; d[1] = s[1]; d[2] = s[2]; d[3] = s[3];
      continue;
    }
    const uint4 q0 = s[0], q1 = s[1], q2 = s[2], q3 = s[3];
    const uint32_t v[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                            q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
    uint32_t o[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      // element b lives in word b/2 (half b%2); element 16+b in word 8+b/2
      if (MODE == ST_BF16) {
        const uint32_t lo = (b & 1) ? (v[b >> 1] & 0xffff0000u) : (v[b >> 1] << 16);
        const uint32_t hi = (b & 1) ? (v[8 + (b >> 1)] & 0xffff0000u) : (v[8 + (b >> 1)] << 16);
        o[b] = (uint32_t)f32_to_f16_bits(__uint_as_float(lo)) |
               ((uint32_t)f32_to_f16_bits(__uint_as_float(hi)) << 16);
      } else {
        const uint32_t lo = (b & 1) ? (v[b >> 1] >> 16) : (v[b >> 1] & 0xffffu);
        const uint32_t hi = (b & 1) ? (v[8 + (b >> 1)] >> 16) : (v[8 + (b >> 1)] & 0xffffu);
        o[b] = lo | (hi << 16);
      }
    }
    d[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d[1] = make_uint4(o[4], o[5], o[6], o[7]);
    d[2] = make_uint4(o[8], o[9], o[10], o[11]);
    d[3] = make_uint4(o[12], o[13], o[14], o[15]);
  }
}

// Sum the per-wave partial tiles into wave 0 (wave order, deterministic).
// `red` must hold (waves-1)*NB*TT*64 f32x4 of shared memory. The caller must
// have synchronised if `red` aliases memory other waves may still read.
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

// Split of a reduction of G groups over the waves of a workgroup: `waves`
// waves with `cpw` chunks of 512 each (waves <= max_waves, cpw <= 8; beyond that the
// kernels loop over rounds of waves*cpw chunks).
struct DecSplit {
  int waves, cpw;
};
static inline DecSplit dec_split(int G, int max_waves = 16) {
  const int chunks = (G + 3) / 4;
  int w = chunks < max_waves ? chunks : max_waves;
  if (w < 1) w = 1;
  int cpw = (chunks + w - 1) / w;
  if (cpw > 8) {
    cpw = 8;
    w = (chunks + 7) / 8;
    if (w > 16) w = 16;
  }
  w = (chunks + cpw - 1) / cpw;  // no idle waves
  if (w > 16) w = 16;
  return {w, cpw};
}

// position of column index n inside a permuted row
__device__ __forceinline__ int perm_pos(int n) { return (n & ~31) + perm32(n & 31); }

// Dispatch a runtime chunks-per-wave value to a compile-time one.
#define BRQ_CPW_SWITCH(cpw, ...)                             \
  switch (cpw) {                                             \
    case 1: { constexpr int CPW = 1; __VA_ARGS__; } break;   \
    case 2: { constexpr int CPW = 2; __VA_ARGS__; } break;   \
    case 3: { constexpr int CPW = 3; __VA_ARGS__; } break;   \
    case 4: { constexpr int CPW = 4; __VA_ARGS__; } break;   \
    case 5: { constexpr int CPW = 5; __VA_ARGS__; } break;   \
    case 6: { constexpr int CPW = 6; __VA_ARGS__; } break;   \
    case 7: { constexpr int CPW = 7; __VA_ARGS__; } break;   \
    default: { constexpr int CPW = 8; __VA_ARGS__; } break;  \
  }

}  // namespace brq
