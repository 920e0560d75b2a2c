// Activation staging and the few-row (decode) group-128 product.
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} (+-x[m][k]): the activation x
// binary-weight product of "Banyan ..." (Abstract) on the group-128 format of
// "Behaviour-Relearned Quantization" (item 02), for M <= 64 activation rows.
#include "dec_core.h"
#include "kernels.h"

namespace brq {

// One thread per run of 32: load 32 values, write them in the permuted order
// slot 2b+h <- k = 16h+b, as fp16.
template <bool FROM_BF16>
__global__ __launch_bounds__(256) void k_prep(const uint16_t* __restrict__ src, int64_t runs,
                                              uint16_t* __restrict__ dst) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= runs) return;
  const uint4* s = reinterpret_cast<const uint4*>(src + t * 32);
  uint32_t v[16];
  const uint4 q0 = s[0], q1 = s[1], q2 = s[2], q3 = s[3];
  v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
  v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
  v[8] = q2.x; v[9] = q2.y; v[10] = q2.z; v[11] = q2.w;
  v[12] = q3.x; v[13] = q3.y; v[14] = q3.z; v[15] = q3.w;
  uint32_t o[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    // element b lives in word b/2 (half b%2); element 16+b in word 8+b/2
    const uint32_t lo16 = (b & 1) ? (v[b >> 1] >> 16) : (v[b >> 1] & 0xffffu);
    const uint32_t hi16 = (b & 1) ? (v[8 + (b >> 1)] >> 16) : (v[8 + (b >> 1)] & 0xffffu);
    uint32_t a, c;
    if (FROM_BF16) {
      a = f32_to_f16_bits(bf16_to_f32(lo16));
      c = f32_to_f16_bits(bf16_to_f32(hi16));
    } else {
      a = lo16;
      c = hi16;
    }
    o[b] = a | (c << 16);
  }
  uint4* d = reinterpret_cast<uint4*>(dst + t * 32);
  d[0] = make_uint4(o[0], o[1], o[2], o[3]);
  d[1] = make_uint4(o[4], o[5], o[6], o[7]);
  d[2] = make_uint4(o[8], o[9], o[10], o[11]);
  d[3] = make_uint4(o[12], o[13], o[14], o[15]);
}

hipError_t launch_prep_bf16(const uint16_t* x, int64_t rows, int64_t K, uint16_t* xp, hipStream_t st) {
  const int64_t runs = rows * (K / 32);
  hipLaunchKernelGGL(k_prep<true>, dim3((unsigned)((runs + 255) / 256)), dim3(256), 0, st, x, runs, xp);
  return hipGetLastError();
}

hipError_t launch_prep_f16(const uint16_t* v, int64_t K, uint16_t* vp, hipStream_t st) {
  const int64_t runs = K / 32;
  hipLaunchKernelGGL(k_prep<false>, dim3((unsigned)((runs + 255) / 256)), dim3(256), 0, st, v, runs, vp);
  return hipGetLastError();
}

template <int TT>
__global__ __launch_bounds__(1024) void k_gemm_dec(const uint16_t* __restrict__ xp, int M, int N, int K,
                                                   const uint4* __restrict__ signs,
                                                   const uint16_t* __restrict__ scales, void* __restrict__ y,
                                                   int y_bf16) {
  __shared__ f32x4 red[15 * TT * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int n = n0 + j;
  const int G = K >> 7;
  const uint4* wsig[1] = {n < N ? signs + (size_t)n * G : nullptr};
  const uint16_t* wsc[1] = {n < N ? scales + (size_t)n * G : nullptr};
  const u32x4* arow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int m = 16 * tt + j;
    arow[tt] = m < M ? reinterpret_cast<const u32x4*>(xp + (size_t)m * K) : nullptr;
  }
  f32x4 acc[1][TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[0][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  dec_core<BM_GROUP, 1, TT>(wsig, wsc, nullptr, arow, G, wave, nw, acc);
  reduce_waves<1, TT>(acc, red);
  if (wave != 0 || n >= N) return;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * tt + 4 * (lane >> 4) + i;
      if (m < M) store_out(y, (size_t)m * N + n, acc[0][tt][i], y_bf16);
    }
}

hipError_t launch_gemm_dec(const uint16_t* xp, int M, int N, int K, const uint64_t* signs,
                           const uint16_t* scales, void* y, int y_bf16, hipStream_t st) {
  const int G = K / 128;
  const int waves = dec_waves(G);
  const dim3 grid((N + 15) / 16), block(64 * waves);
  const uint4* s4 = reinterpret_cast<const uint4*>(signs);
  const int TT = (M + 15) / 16;
  switch (TT) {
    case 1: hipLaunchKernelGGL(k_gemm_dec<1>, grid, block, 0, st, xp, M, N, K, s4, scales, y, y_bf16); break;
    case 2: hipLaunchKernelGGL(k_gemm_dec<2>, grid, block, 0, st, xp, M, N, K, s4, scales, y, y_bf16); break;
    case 3: hipLaunchKernelGGL(k_gemm_dec<3>, grid, block, 0, st, xp, M, N, K, s4, scales, y, y_bf16); break;
    default: hipLaunchKernelGGL(k_gemm_dec<4>, grid, block, 0, st, xp, M, N, K, s4, scales, y, y_bf16); break;
  }
  return hipGetLastError();
}

}  // namespace brq
