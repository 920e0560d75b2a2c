// Many-row binary product on the matrix cores (the prefill regime: one matrix
// applied to many vectors, so the weight unpack is amortised over a tile of
// rows; "LLM binarization, Episode 01: DBF", section 4).
//
// Block tile BM x BN x 64 on 4 waves (2 x 2), each wave (BM/2) x (BN/2) of
// v_mfma_f32_32x32x16_f16 tiles. Per k-step of 64:
//   A: activations, fp16 already in the permuted order (staged by
//      k_prep_rows, each row scaled by a power of two, or the DBF
//      intermediate's pieces), copied to LDS.
//   B: one 64-bit sign word per column; each pair of signs becomes an fp16
//      pair +-c (c = group scale, per-k value or 1) with one shift and one
//      and-or, written to LDS.
// Two LDS stages: the global loads of step k+1 are issued before the matrix
// products of step k, and land in the other stage afterwards.
//
// Layout facts of the 32x32x16 MFMA used here: A lane l supplies row l%32 and
// 8 consecutive k of block l/32; B lane l supplies column l%32 and the same k
// block; D lane l holds, in item r, row 8*(r/4) + 4*(l/32) + r%4 of column l%32.
//
// Epilogues: EPI_Y writes y (fp32 or bf16); EPI_HS32 undoes the rows' staging
// scale (2^-rexp[row]), multiplies by a per-column fp16 diagonal and writes
// fp32 rows (the DBF intermediate h_s); EPI_PAIRSUM
// adds the two piece rows of every token, applies the token's power of two
// (2^rexp, exact) and multiplies by a per-column diagonal (the DBF output).
#include "common.h"
#include "dec_core.h"
#include "kernels.h"
#include "tile.h"

namespace brq {

template <int BM, int BN, int AMODE, int BMODE, int EPI>
__global__ __launch_bounds__(256) void k_tile(TileArgs p) {
  constexpr int BK = 64, LDK = BK + 8;  // +16 bytes per LDS row against bank conflicts
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int A_UNITS = BM * 4 / 256;  // per thread: 16 activations (8 pairs)
  constexpr int B_UNITS = BN * 4 / 256;  // per thread: 8 pairs of one column
  static_assert(A_UNITS >= 1 && B_UNITS >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // tile id -> (tm, tn); contiguous ranges of tile ids per XCD so the
  // workgroups sharing an activation row-block share one L2
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  const int tm = bid / tiles_n, tn = bid % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  // K-slice blockIdx.y of p.ksplit: k-steps kt0 .. kt0 + nk - 1
  const int nk = p.K / BK / p.ksplit;
  const int kt0 = (int)blockIdx.y * nk;

  // ---- global -> register staging --------------------------------------
  uint4 ra[A_UNITS][2];
  uint2 rb[B_UNITS];   // .x = sign dword, .y = magnitude pair (BM_GROUP / BM_ONE)
  u32x4 rk[B_UNITS][2];  // BM_PERK magnitudes: 8 pairs

  auto load_stage = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int u = 0; u < A_UNITS; ++u) {
      const int unit = tid + 256 * u;
      const int row = unit >> 2, q = (unit >> 1) & 1, b0 = (unit & 1) * 8;
      const int gm = m0 + row;
      if (gm < p.M) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(p.a) + (size_t)gm * p.K + k0 + 32 * q + 2 * b0;
        ra[u][0] = *reinterpret_cast<const uint4*>(src);
        ra[u][1] = *reinterpret_cast<const uint4*>(src + 8);
      } else {
        ra[u][0] = make_uint4(0, 0, 0, 0);
        ra[u][1] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < B_UNITS; ++u) {
      const int unit = tid + 256 * u;
      const int col = unit >> 2, q = (unit >> 1) & 1, b0 = (unit & 1) * 8;
      const int gn = n0 + col;
      const int kw = p.K >> 5;  // 32-bit sign dwords per row
      uint32_t dw = 0, mag = (BMODE == BM_ONE) ? 0x3c003c00u : 0u;
      if (gn < p.N) {
        dw = reinterpret_cast<const uint32_t*>(p.signs)[(size_t)gn * kw + (k0 >> 5) + q];
        if (BMODE == BM_GROUP) {
          const uint32_t s = p.scales[(size_t)gn * (p.K >> 7) + (k0 >> 7)];
          mag = s | (s << 16);
        }
      }
      rb[u] = make_uint2(dw, mag);
      if (BMODE == BM_PERK) {
        // natural-order magnitudes of this unit's pairs (k, k + 16), k = run + b0 .. b0 + 7
        const uint16_t* kr = p.kmag + k0 + 32 * q + b0;
        rk[u][0] = *reinterpret_cast<const u32x4*>(kr);
        rk[u][1] = *reinterpret_cast<const u32x4*>(kr + 16);
      }
    }
  };

  // ---- register -> LDS (convert / unpack) ---------------------------------
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < A_UNITS; ++u) {
      const int unit = tid + 256 * u;
      const int row = unit >> 2, q = (unit >> 1) & 1, b0 = (unit & 1) * 8;
      uint32_t o[8];
      o[0] = ra[u][0].x; o[1] = ra[u][0].y; o[2] = ra[u][0].z; o[3] = ra[u][0].w;
      o[4] = ra[u][1].x; o[5] = ra[u][1].y; o[6] = ra[u][1].z; o[7] = ra[u][1].w;
      uint4* dst = reinterpret_cast<uint4*>(&As[buf][row * LDK + 32 * q + 2 * b0]);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
#pragma unroll
    for (int u = 0; u < B_UNITS; ++u) {
      const int unit = tid + 256 * u;
      const int col = unit >> 2, q = (unit >> 1) & 1, b0 = (unit & 1) * 8;
      const uint32_t dw = rb[u].x;
      uint32_t o[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int bit = b0 + t;
        uint32_t mag = rb[u].y;
        if (BMODE == BM_PERK) {
          const uint32_t lw = rk[u][0][t >> 1], hw = rk[u][1][t >> 1];
          mag = (t & 1) ? ((lw >> 16) | (hw & 0xffff0000u)) : ((lw & 0xffffu) | (hw << 16));
        }
        // a per-k diagonal value may be negative: flip its sign bit (a scale is OR-ed)
        const uint32_t sw = (dw << (15 - bit)) & 0x80008000u;
        o[t] = (BMODE == BM_PERK) ? (sw ^ mag) : (sw | mag);
      }
      uint4* dst = reinterpret_cast<uint4*>(&Bs[buf][col * LDK + 32 * q + 2 * b0]);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load_stage(kt0);
  store_stage(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage(kt0 + kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 af[TM], bfr[TN];
      const int kofs = 16 * ks + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(&As[cur][(wr * WM + 32 * i + (lane & 31)) * LDK + kofs]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(&Bs[cur][(wc * WN + 32 * j + (lane & 31)) * LDK + kofs]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wc * WN + 32 * j + (lane & 31);
      if (col >= p.N) continue;
      const int rbase = m0 + wr * WM + 32 * i + 4 * (lane >> 5);
      if (EPI == EPI_Y) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + 8 * (r >> 2) + (r & 3);
          if (row < p.M) store_out(p.out, (size_t)row * p.N + col, acc[i][j][r], p.out_bf16);
        }
      } else if (EPI == EPI_HS32) {
        const float dm = f16_bits_to_f32(p.diag[col]);
        float* hs = reinterpret_cast<float*>(p.out) + (size_t)blockIdx.y * p.M * p.N;  // this K-slice's partial
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + 8 * (r >> 2) + (r & 3);
          if (row < p.M) hs[(size_t)row * p.N + col] = __builtin_amdgcn_ldexpf(acc[i][j][r], -p.rexp[row]) * dm;
        }
      } else {  // EPI_PAIRSUM: rows 2t, 2t+1 are the two pieces of token t
        const float dg = f16_bits_to_f32(p.diag[col]);
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int row = rbase + 8 * (r >> 2) + (r & 3);
          if (row < p.M)
            store_out(p.out, (size_t)(row >> 1) * p.N + col,
                      __builtin_amdgcn_ldexpf(acc[i][j][r] + acc[i][j][r + 1], p.rexp[row >> 1]) * dg, p.out_bf16);
        }
      }
    }
}

template <int BM, int BN, int AMODE, int BMODE, int EPI>
static hipError_t run_tile(const TileArgs& a, hipStream_t st) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((k_tile<BM, BN, AMODE, BMODE, EPI>), dim3(tiles, a.ksplit), dim3(256), 0, st, a);
  return hipGetLastError();
}

// DBF stage 1 tiling: 128 x 128 tiles, the reduction axis split into
// ksplit slices (a power of two, at most 8, whole 64-wide k-steps) until
// tiles x slices gives two workgroups per compute unit (the second hides the
// first's loads); each slice writes its own fp32 partial h_s and k_dbf_split
// adds them in slice order
int dbf1_ksplit(int M, int r, int n) {
  const long tiles = (long)((M + 127) / 128) * ((r + 127) / 128);
  int s = 1;
  while (s < 8 && tiles * s < 512 && (n / 64) % (2 * s) == 0) s *= 2;
  return s;
}

hipError_t launch_tile_dbf1(const TileArgs& a, hipStream_t st) {
  return run_tile<128, 128, 1, BM_PERK, EPI_HS32>(a, st);
}

// DBF stage 2: 64 x 128 tiles (two or more workgroups per compute unit, so
// one workgroup's loads hide behind another's products) while they number at
// least two per compute unit, 64 x 64 below
hipError_t launch_tile_dbf2(const TileArgs& a, hipStream_t st) {
  const long mid = (long)((a.M + 63) / 64) * ((a.N + 127) / 128);
  if (mid >= 512) return run_tile<64, 128, 1, BM_ONE, EPI_PAIRSUM>(a, st);
  return run_tile<64, 64, 1, BM_ONE, EPI_PAIRSUM>(a, st);
}

}  // namespace brq
