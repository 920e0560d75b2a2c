// Binary product plus a rank-r weight correction: y = x . (Wq + U V)^T
// = x . Wq^T + (x . V^T) . U^T (BWLA commentary, section 4: the residual of
// the binarised weights approximated by a truncated SVD and added back as a
// correction term; V fp16 [r][K], U fp16 [N][r], r <= 64).
//
// Launches:
//  1. k_lr_prep: V padded to 64 rows (zeros past r); for M > 64 also U
//     padded to [N][64] fp16.
//  2. k_prep_rows: the rows' staging exponents s (and, for M > 64, the
//     staged rows of the prefill product).
//     k_lr_t: t = (x 2^s) . V^T on the fp16 matrix cores (x scaled and
//     converted to fp16 in registers, natural order; the eight waves of a
//     workgroup split K), fp32 accumulate; for M <= 64 scaled back by 2^-s.
//     M > 64: stored as the fp16 hi/lo pair [M][128] that the prefill kernel
//     takes as one extra k-step inside its epilogue; M <= 64: stored fp32.
//  3. M > 64: the prefill product with the fused correction step (pf.hip).
//     M <= 64: the product into an fp32 workspace (brq_gemm's own paths),
//     then k_lr_apply adds t . U^T per output and writes y once.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace brq {

namespace {

constexpr int LR_MAX = 64;  // rank capacity (padded)

struct LrWs {
  uint16_t* vb;     // [64][K] fp16: V with zero rows past r
  uint16_t* u_pad;  // [N][64] fp16 (M > 64 only)
  uint16_t* t16;    // [M][128] fp16 hi/lo of x V^T (M > 64)
  float* t32;       // [M][64] fp32 x V^T (M <= 64)
  float* y32;       // [M][N] fp32 product (M <= 64)
  int* rexp;        // [M] staging exponents of the rows
  void* gemm_ws;    // workspace of the product itself
};

// Carve (or size, with base == nullptr) the workspace of brq_gemm_lr.
size_t lr_carve(char* base, int64_t M, int64_t N, int64_t K, LrWs* w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = base ? base + off : nullptr;
    off += align256(bytes);
    return q;
  };
  LrWs l{};
  l.vb = reinterpret_cast<uint16_t*>(take((size_t)LR_MAX * K * 2));
  l.rexp = reinterpret_cast<int*>(take((size_t)M * 4));
  if (M > 64) {
    l.u_pad = reinterpret_cast<uint16_t*>(take((size_t)N * LR_MAX * 2));
    l.t16 = reinterpret_cast<uint16_t*>(take((size_t)M * 2 * LR_MAX * 2));
    l.gemm_ws = take((size_t)M * K * 2);  // the prefill's staged activations
  } else {
    l.t32 = reinterpret_cast<float*>(take((size_t)M * LR_MAX * 4));
    l.y32 = reinterpret_cast<float*>(take((size_t)M * N * 4));
    l.gemm_ws = take(gemm_dec_ws_bytes(M, N, K));
  }
  if (w) *w = l;
  return off;
}

}  // namespace

// V -> [64][K] fp16 with zero rows past r (entries e < 64*K); U -> [N][64]
// fp16 padded (entries 64*K <= e < 64*K + 64*N when pad_u).
__global__ __launch_bounds__(256) void k_lr_prep(const uint16_t* __restrict__ v, const uint16_t* __restrict__ u,
                                                 int N, int K, int r, int pad_u, uint16_t* __restrict__ vp,
                                                 uint16_t* __restrict__ u_pad) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nv = (int64_t)LR_MAX * K;
  if (e < nv) {
    const int i = (int)(e / K);
    vp[e] = i < r ? v[e] : (uint16_t)0;  // row i of V starts at i*K either way
    return;
  }
  const int64_t q = e - nv;
  if (!pad_u || q >= (int64_t)N * LR_MAX) return;
  const int n = (int)(q / LR_MAX), i = (int)(q - (int64_t)n * LR_MAX);
  u_pad[q] = i < r ? u[(size_t)n * r + i] : (uint16_t)0;
}

// t = x . V^T for 16 TT rows (TT 16-row tiles) per workgroup on the fp16
// matrix cores: x converted to fp16 in registers (the same conversion the
// product's own activation staging applies), V as given (fp16, padded to 64
// rows). The waves take interleaved 64-k blocks (wave w of eight: blocks w,
// w+8, ...) and all NC factor tiles of 16, BPR blocks per
// round with every load of the round issued first; the waves' partial sums
// meet in LDS in wave order.
// Lane (kb, j): A = row m0+16t+j, k 8kb.. of each 32-k half-block; B = factor
// 16c+j, same k. Factor tiles c >= NC (past the rank) are written as zeros.
// HILO: store fp16 hi/lo pairs [M][128] (hi at i, lo at 64+i), else fp32 [M][64].
template <bool HILO, int NC, int TT>
__global__ __launch_bounds__(512) void k_lr_t(const uint16_t* __restrict__ x, int M, int K,
                                              const uint16_t* __restrict__ vp, const int* __restrict__ rexp,
                                              uint16_t* __restrict__ t16, float* __restrict__ t32) {
  constexpr int BPR = NC <= 2 ? 4 : 2;  // blocks per round: the round's loads stay in registers
  constexpr int NW = 8;                 // waves: interleaved 64-k blocks
  __shared__ f32x4 red[NW - 1][TT][NC][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int m0 = blockIdx.x * 16 * TT;
  const int nblk = K >> 6;
  const uint16_t* xa[TT];
  int xs[TT];  // staging exponent of the lane's A row in each row tile
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int row = m0 + 16 * t + j < M ? m0 + 16 * t + j : M - 1;
    xa[t] = x + (size_t)row * K + 8 * kb;
    xs[t] = rexp[row];
  }
  const uint16_t* vr = vp + (size_t)j * K + 8 * kb;  // factor 16c + j at + 16c*K
  f32x4 acc[TT][NC];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int b0 = wave; b0 < nblk; b0 += NW * BPR) {
    u32x4 a[BPR][TT][2], v[BPR][NC][2];
    bool use[BPR];
#pragma unroll
    for (int q = 0; q < BPR; ++q) {
      const int blk = b0 + NW * q;
      use[q] = blk < nblk;
      const int k = 64 * (use[q] ? blk : b0);  // past K: repeat the round's first block
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int t = 0; t < TT; ++t) a[q][t][hh] = *reinterpret_cast<const u32x4*>(xa[t] + k + 32 * hh);
#pragma unroll
        for (int c = 0; c < NC; ++c) v[q][c][hh] = *reinterpret_cast<const u32x4*>(vr + (size_t)16 * c * K + k + 32 * hh);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the round issues before the products
    // straight-line products (a branch lets the compiler sink each block's
    // loads next to its products); blocks past K multiply zeros
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < BPR; ++q)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          u32x4 af;  // bf16 pairs -> fp16 pairs, round to nearest even
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t w = a[q][t][hh][d];
            af[d] = (uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(__uint_as_float(w << 16), xs[t])) |
                    ((uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(__uint_as_float(w & 0xffff0000u), xs[t]))
                     << 16);
          }
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[t][c] = mfma16(af, use[q] ? v[q][c][hh] : z, acc[t][c]);
        }
  }
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int c = 0; c < NC; ++c) red[wave - 1][t][c][lane] = acc[t][c];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) acc[t][c] += red[w][t][c][lane];
  // lane (kb, j) holds rows m0 + 16t + 4kb + i of factor 16c + j
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * t + 4 * kb + i;
      if (m >= M) continue;
      const int un = HILO ? 0 : -rexp[m];  // fp32 output: back to the unscaled row
#pragma unroll
      for (int c = 0; c < LR_MAX / 16; ++c) {
        const int f = 16 * c + j;
        const float val = c < NC ? __builtin_amdgcn_ldexpf(acc[t][c < NC ? c : 0][i], un) : 0.f;
        if (HILO) {
          uint16_t hi, lo;
          split_f16(val, hi, lo);
          t16[(size_t)m * 2 * LR_MAX + f] = hi;
          t16[(size_t)m * 2 * LR_MAX + LR_MAX + f] = lo;
        } else {
          t32[(size_t)m * LR_MAX + f] = val;
        }
      }
    }
}

// y[m][n] = y32[m][n] + sum_i t32[m][i] * U[n][i], in i order, written once.
__global__ __launch_bounds__(256) void k_lr_apply(const float* __restrict__ y32, const float* __restrict__ t32,
                                                  const uint16_t* __restrict__ u, int M, int N, int r,
                                                  void* __restrict__ y, int y_bf16) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)M * N) return;
  const int m = (int)(e / N), n = (int)(e - (int64_t)m * N);
  float v = y32[e];
  const float* tm = t32 + (size_t)m * LR_MAX;
  const uint16_t* un = u + (size_t)n * r;
  for (int i = 0; i < r; ++i) v = fmaf(tm[i], f16_bits_to_f32(un[i]), v);
  store_out(y, (size_t)e, v, y_bf16);
}

size_t lr_ws_bytes(int64_t M, int64_t N, int64_t K) { return lr_carve(nullptr, M, N, K, nullptr); }

hipError_t launch_gemm_lr(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                          const uint16_t* v, const uint16_t* u, int r, void* y, int y_bf16, void* ws,
                          hipStream_t st) {
  LrWs w;
  lr_carve(reinterpret_cast<char*>(ws), M, N, K, &w);
  const bool many = M > 64;
  const int64_t prep = (int64_t)LR_MAX * K + (many ? (int64_t)N * LR_MAX : 0);
  hipLaunchKernelGGL(k_lr_prep, dim3((unsigned)((prep + 255) / 256)), dim3(256), 0, st, v, u, N, K, r, many ? 1 : 0,
                     w.vb, w.u_pad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // two row tiles per workgroup once that still gives one workgroup per
  // compute unit, one below (M = 4096: 256 workgroups of 16 rows)
  const bool two = (M + 31) / 32 >= 256;
  const dim3 tg((unsigned)(two ? (M + 31) / 32 : (M + 15) / 16));
  const int nc = (r + 15) / 16;  // factor tiles of 16 that the rank needs
  auto lr_t = [&](auto hilo) {
    constexpr bool H = decltype(hilo)::value;
#define BRQ_LRT(NC)                                                                                   \
  if (two) hipLaunchKernelGGL((k_lr_t<H, NC, 2>), tg, dim3(512), 0, st, x, M, K, w.vb, w.rexp, w.t16, w.t32); \
  else hipLaunchKernelGGL((k_lr_t<H, NC, 1>), tg, dim3(512), 0, st, x, M, K, w.vb, w.rexp, w.t16, w.t32)
    switch (nc) {
      case 1: BRQ_LRT(1); break;
      case 2: BRQ_LRT(2); break;
      case 3: BRQ_LRT(3); break;
      default: BRQ_LRT(4); break;
    }
#undef BRQ_LRT
    return hipGetLastError();
  };
  // the rows' staging exponents (M > 64: with the staged rows themselves)
  uint16_t* xp = many ? reinterpret_cast<uint16_t*>(w.gemm_ws) : nullptr;
  e = launch_prep_rows(x, M, K, xp, w.rexp, 1, st);
  if (e != hipSuccess) return e;
  if (many) {
    e = lr_t(std::true_type{});
    if (e != hipSuccess) return e;
    return launch_gemm_pf_lr(xp, w.rexp, M, N, K, signs, scales, w.t16, w.u_pad, y, y_bf16, st);
  }
  e = lr_t(std::false_type{});
  if (e != hipSuccess) return e;
  e = launch_gemm_dec(x, M, N, K, signs, scales, w.y32, 0, w.gemm_ws, st);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)M * N;
  hipLaunchKernelGGL(k_lr_apply, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, w.y32, w.t32, u, M, N, r, y,
                     y_bf16);
  return hipGetLastError();
}

}  // namespace brq
