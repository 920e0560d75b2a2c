// Double Binary Factorization chain y = D_out U D_mid V D_in x
// ("LLM binarization, Episode 01: DBF": section 1, the representation with
// V in {-1,+1}^(r x n), U in {-1,+1}^(m x r) and three diagonals; section 4,
// the deployed order x_s = D_in x, h = V x_s, h_s = D_mid h, y_core = U h_s,
// y = D_out y_core).
//
// Stage 1 folds D_in into the weight operand: V[j][k] * d_in[k] is the exact
// fp16 value +-d_in[k], so the first product reads x unscaled. Its epilogue
// applies D_mid in fp32 and stores h_s as an fp16 hi/lo pair (22 significant
// bits) in the permuted operand order. Stage 2 multiplies U (+-1 operands) by
// both pieces (two activation rows per token), adds the pieces and applies
// D_out in fp32.
#include "dec_core.h"
#include "kernels.h"
#include "tile.h"

namespace brq {

template <int TT>
__global__ __launch_bounds__(1024) void k_dbf1_dec(const uint16_t* __restrict__ xp, int M, int r, int n,
                                                   const uint4* __restrict__ v, const u32x4* __restrict__ dinp,
                                                   const uint16_t* __restrict__ d_mid, uint16_t* __restrict__ hp) {
  __shared__ f32x4 red[15 * TT * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15;
  const int col = blockIdx.x * 16 + j;  // row of V = output column of stage 1
  const int G = n >> 7;
  const uint4* wsig[1] = {col < r ? v + (size_t)col * G : nullptr};
  const uint16_t* wsc[1] = {nullptr};
  const u32x4* arow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int m = 16 * tt + j;
    arow[tt] = m < M ? reinterpret_cast<const u32x4*>(xp + (size_t)m * n) : nullptr;
  }
  f32x4 acc[1][TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[0][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  dec_core<BM_PERK, 1, TT>(wsig, wsc, dinp, arow, G, wave, nw, acc);
  reduce_waves<1, TT>(acc, red);
  if (wave != 0 || col >= r) return;
  const float dm = f16_bits_to_f32(d_mid[col]);
  const int pc = perm_pos(col);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * tt + 4 * (lane >> 4) + i;
      if (m < M) {
        uint16_t hi, lo;
        split_f16(acc[0][tt][i] * dm, hi, lo);
        hp[(size_t)(2 * m) * r + pc] = hi;
        hp[(size_t)(2 * m + 1) * r + pc] = lo;
      }
    }
}

template <int TT>
__global__ __launch_bounds__(1024) void k_dbf2_dec(const uint16_t* __restrict__ hp, int M, int m, int r,
                                                   const uint4* __restrict__ u, const uint16_t* __restrict__ d_out,
                                                   void* __restrict__ y, int y_bf16) {
  __shared__ f32x4 red[15 * TT * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15;
  const int col = blockIdx.x * 16 + j;  // row of U = output column
  const int G = r >> 7;
  const uint4* wsig[1] = {col < m ? u + (size_t)col * G : nullptr};
  const uint16_t* wsc[1] = {nullptr};
  const u32x4* arow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int pr = 16 * tt + j;  // piece row: token pr/2, piece pr%2
    arow[tt] = pr < 2 * M ? reinterpret_cast<const u32x4*>(hp + (size_t)pr * r) : nullptr;
  }
  f32x4 acc[1][TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[0][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  dec_core<BM_ONE, 1, TT>(wsig, wsc, nullptr, arow, G, wave, nw, acc);
  reduce_waves<1, TT>(acc, red);
  if (wave != 0 || col >= m) return;
  const float dg = f16_bits_to_f32(d_out[col]);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 * tt + 2 * (lane >> 4) + h;
      if (t < M) store_out(y, (size_t)t * m + col, (acc[0][tt][2 * h] + acc[0][tt][2 * h + 1]) * dg, y_bf16);
    }
}

size_t dbf_ws_bytes(int64_t M, int64_t m, int64_t n, int64_t r) {
  (void)m;
  return align256((size_t)M * n * 2) + align256((size_t)n * 2) + align256((size_t)2 * M * r * 2);
}

hipError_t launch_dbf(const uint16_t* x, int M, int m, int n, int r, const uint16_t* d_in,
                      const uint64_t* v, const uint16_t* d_mid, const uint64_t* u,
                      const uint16_t* d_out, void* y, int y_bf16, void* ws, hipStream_t st) {
  char* base = reinterpret_cast<char*>(ws);
  uint16_t* xp = reinterpret_cast<uint16_t*>(base);
  uint16_t* dinp = reinterpret_cast<uint16_t*>(base + align256((size_t)M * n * 2));
  uint16_t* hp = reinterpret_cast<uint16_t*>(base + align256((size_t)M * n * 2) + align256((size_t)n * 2));
  hipError_t e = launch_prep_f16(d_in, n, dinp, st);
  if (e != hipSuccess) return e;
  if (2 * M <= 64) {
    e = launch_prep_bf16(x, M, n, xp, st);
    if (e != hipSuccess) return e;
    const int TT1 = (M + 15) / 16;
    const dim3 g1((r + 15) / 16), b1(64 * dec_waves(n / 128));
    const uint4* v4 = reinterpret_cast<const uint4*>(v);
    const u32x4* dp = reinterpret_cast<const u32x4*>(dinp);
    if (TT1 == 1)
      hipLaunchKernelGGL(k_dbf1_dec<1>, g1, b1, 0, st, xp, M, r, n, v4, dp, d_mid, hp);
    else
      hipLaunchKernelGGL(k_dbf1_dec<2>, g1, b1, 0, st, xp, M, r, n, v4, dp, d_mid, hp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int TT2 = (2 * M + 15) / 16;
    const dim3 g2((m + 15) / 16), b2(64 * dec_waves(r / 128));
    const uint4* u4 = reinterpret_cast<const uint4*>(u);
    switch (TT2) {
      case 1: hipLaunchKernelGGL(k_dbf2_dec<1>, g2, b2, 0, st, hp, M, m, r, u4, d_out, y, y_bf16); break;
      case 2: hipLaunchKernelGGL(k_dbf2_dec<2>, g2, b2, 0, st, hp, M, m, r, u4, d_out, y, y_bf16); break;
      case 3: hipLaunchKernelGGL(k_dbf2_dec<3>, g2, b2, 0, st, hp, M, m, r, u4, d_out, y, y_bf16); break;
      default: hipLaunchKernelGGL(k_dbf2_dec<4>, g2, b2, 0, st, hp, M, m, r, u4, d_out, y, y_bf16); break;
    }
    return hipGetLastError();
  }
  TileArgs a1{};
  a1.a = x; a1.M = M; a1.N = r; a1.K = n; a1.signs = v; a1.kperm = dinp; a1.diag = d_mid; a1.out = hp;
  e = launch_tile_dbf1(a1, st);
  if (e != hipSuccess) return e;
  TileArgs a2{};
  a2.a = hp; a2.M = 2 * M; a2.N = m; a2.K = r; a2.signs = u; a2.diag = d_out; a2.out = y; a2.out_bf16 = y_bf16;
  return launch_tile_dbf2(a2, st);
}

}  // namespace brq
