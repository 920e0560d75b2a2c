// Kronecker-factored orthogonal activation rotation x' = (H (x) R) x, computed
// per token as X' = H X R^T with X the token reshaped row-major to [64][64]
// (BWLA commentary: section 3, OKT with Kronecker factors; section 5, the same
// transform applied to the activations). fp32 arithmetic, bf16 output.
//
// One wave per token, four tokens per workgroup. H^T and R^T sit in LDS for the
// whole workgroup; each wave stages its token transposed (X^T) in LDS, forms
// T = X R^T with lane (a, b) computing the 8 x 8 block rows 8a.., columns 8b..,
// writes T back to its LDS slot and forms Y = H T the same way.
#include "common.h"
#include "kernels.h"

namespace brq {

__global__ __launch_bounds__(256) void k_kron(const uint16_t* __restrict__ x, int M, const float* __restrict__ H,
                                              const float* __restrict__ R, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) float Ht[64 * 64];  // Ht[c][a] = H[a][c]
  __shared__ __attribute__((aligned(16))) float Rt[64 * 64];  // Rt[d][b] = R[b][d]
  __shared__ __attribute__((aligned(16))) float buf[4][64 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    Ht[c * 64 + r] = H[i];
    Rt[c * 64 + r] = R[i];
  }
  const int t = blockIdx.x * 4 + wave;
  const bool live = t < M;
  float* B = buf[wave];
  if (live) {
    // X^T: B[d][a] = x[t][64a + d]; lane reads run a = lane of 64 values
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * 4096 + lane * 64);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = src[q];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int d = q * 8 + 2 * h;
        B[d * 64 + lane] = bf16_to_f32(w[h] & 0xffffu);
        B[(d + 1) * 64 + lane] = bf16_to_f32(w[h] >> 16);
      }
    }
  }
  __syncthreads();
  const int ab = (lane >> 3) * 8, bb = (lane & 7) * 8;
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  if (live) {
    // T[a][b] = sum_d X[a][d] R[b][d]
    for (int d = 0; d < 64; ++d) {
      const float4 x0 = *reinterpret_cast<const float4*>(&B[d * 64 + ab]);
      const float4 x1 = *reinterpret_cast<const float4*>(&B[d * 64 + ab + 4]);
      const float4 r0 = *reinterpret_cast<const float4*>(&Rt[d * 64 + bb]);
      const float4 r1 = *reinterpret_cast<const float4*>(&Rt[d * 64 + bb + 4]);
      const float xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const float rb[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xa[i], rb[j], acc[i][j]);
    }
  }
  __syncthreads();
  if (live) {
    // T row-major: B[c][b]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<float4*>(&B[(ab + i) * 64 + bb]) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
      *reinterpret_cast<float4*>(&B[(ab + i) * 64 + bb + 4]) = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
    }
  }
  __syncthreads();
  if (!live) return;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  // Y[a][b] = sum_c H[a][c] T[c][b]
  for (int c = 0; c < 64; ++c) {
    const float4 h0 = *reinterpret_cast<const float4*>(&Ht[c * 64 + ab]);
    const float4 h1 = *reinterpret_cast<const float4*>(&Ht[c * 64 + ab + 4]);
    const float4 t0 = *reinterpret_cast<const float4*>(&B[c * 64 + bb]);
    const float4 t1 = *reinterpret_cast<const float4*>(&B[c * 64 + bb + 4]);
    const float ha[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
    const float tb[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(ha[i], tb[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      o[h] = (uint32_t)f32_to_bf16_bits(acc[i][2 * h]) | ((uint32_t)f32_to_bf16_bits(acc[i][2 * h + 1]) << 16);
    *reinterpret_cast<uint4*>(y + (size_t)t * 4096 + (ab + i) * 64 + bb) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_kron(const uint16_t* x, int M, const float* H, const float* R, uint16_t* y, hipStream_t st) {
  hipLaunchKernelGGL(k_kron, dim3((M + 3) / 4), dim3(256), 0, st, x, M, H, R, y);
  return hipGetLastError();
}

}  // namespace brq
