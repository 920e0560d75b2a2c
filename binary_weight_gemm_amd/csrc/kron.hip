// Kronecker-factored orthogonal activation rotation x' = (H (x) R) x, computed
// per token as X' = H X R^T with X the token reshaped row-major to [64][64]
// (BWLA commentary: section 3, OKT with Kronecker factors; section 5, the same
// transform applied to the activations). fp32 arithmetic, bf16 output.
//
// One workgroup per compute unit (persistent): H^T and R^T are staged in LDS
// once per workgroup (rows padded to 65 floats so the transposing stores and
// the column reads spread over all banks); each of its six waves then takes
// tokens in turn. For a token, the wave stages X^T in its own LDS slot, forms
// T = X R^T with lane (a, b) computing the 8 x 8 block rows 8a.., columns 8b..,
// writes T back to its slot and forms Y = H T the same way. No barrier is
// needed between tokens: a wave only touches its own slot.
#include "common.h"
#include "kernels.h"

namespace brq {

constexpr int KRON_WAVES = 6;
constexpr int KRON_LD = 65;  // padded row length of H^T and R^T

__global__ __launch_bounds__(64 * KRON_WAVES) void k_kron(const uint16_t* __restrict__ x, int M,
                                                         const float* __restrict__ H, const float* __restrict__ R,
                                                         uint16_t* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) float kl[];
  float* Ht = kl;                       // Ht[c][a] = H[a][c], row length KRON_LD
  float* Rt = kl + 64 * KRON_LD;        // Rt[d][b] = R[b][d]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* B = kl + 2 * 64 * KRON_LD + wave * 64 * 64;  // this wave's 64 x 64 slot
  for (int i = tid; i < 64 * 64; i += blockDim.x) {
    const int r = i >> 6, c = i & 63;
    Ht[c * KRON_LD + r] = H[i];
    Rt[c * KRON_LD + r] = R[i];
  }
  __syncthreads();
  const int ab = (lane >> 3) * 8, bb = (lane & 7) * 8;
  const int nwaves = gridDim.x * KRON_WAVES;
  for (int t = blockIdx.x * KRON_WAVES + wave; t < M; t += nwaves) {
    // X^T: B[d][a] = x[t][64a + d]; lane reads run a = lane of 64 values
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * 4096 + lane * 64);
    uint4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = src[q];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int d = q * 8 + 2 * h;
        B[d * 64 + lane] = bf16_to_f32(w[h] & 0xffffu);
        B[(d + 1) * 64 + lane] = bf16_to_f32(w[h] >> 16);
      }
    }
    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    // T[a][b] = sum_d X[a][d] R[b][d]
    for (int d = 0; d < 64; ++d) {
      const float4 x0 = *reinterpret_cast<const float4*>(&B[d * 64 + ab]);
      const float4 x1 = *reinterpret_cast<const float4*>(&B[d * 64 + ab + 4]);
      float rb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) rb[j] = Rt[d * KRON_LD + bb + j];
      const float xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xa[i], rb[j], acc[i][j]);
    }
    // T row-major: B[c][b] (every lane of this wave has finished reading X^T:
    // LDS operations of one wave complete in order)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<float4*>(&B[(ab + i) * 64 + bb]) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
      *reinterpret_cast<float4*>(&B[(ab + i) * 64 + bb + 4]) = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    // Y[a][b] = sum_c H[a][c] T[c][b]
    for (int c = 0; c < 64; ++c) {
      float ha[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ha[i] = Ht[c * KRON_LD + ab + i];
      const float4 t0 = *reinterpret_cast<const float4*>(&B[c * 64 + bb]);
      const float4 t1 = *reinterpret_cast<const float4*>(&B[c * 64 + bb + 4]);
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
}

hipError_t launch_kron(const uint16_t* x, int M, const float* H, const float* R, uint16_t* y, hipStream_t st) {
  const size_t lds = (size_t)(2 * 64 * KRON_LD + KRON_WAVES * 64 * 64) * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_kron),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const int need = (M + KRON_WAVES - 1) / KRON_WAVES;
  const int grid = need < cus ? need : cus;
  hipLaunchKernelGGL(k_kron, dim3(grid), dim3(64 * KRON_WAVES), lds, st, x, M, H, R, y);
  return hipGetLastError();
}

}  // namespace brq
