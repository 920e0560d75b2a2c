// Reference kernels of the benchmark (not part of the product path): a plain
// streaming read, to measure the HBM rate this device reaches at a given size,
// and a loop of independent fp16 matrix-core products, to measure the rate its
// matrix cores reach. Built into libbrq_ref.so, loaded only by bench.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every thread reads UNR 16-byte words, all loads issued before any use; the
// XOR of the words goes to one store per workgroup so nothing is dropped.
template <int UNR>
__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, size_t n16, uint32_t* __restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * 256 * UNR + threadIdx.x;
  uint4 v[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const size_t i = base + (size_t)u * 256;
    v[u] = p[i < n16 ? i : 0];
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < UNR; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  x = __reduce_or_sync(0xffffffffffffffffull, x);
  if (threadIdx.x == 0 && x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

// ITERS rounds of 8 independent 32x32x16 fp16 products per wave.
__global__ __launch_bounds__(256) void k_mfma_loop(int iters, float* __restrict__ sink) {
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (threadIdx.x + i));
    b[i] = (_Float16)(0.002f * (threadIdx.x - i));
  }
  f32x16 c[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[q][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 8; ++q) c[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[q], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[q][i];
  if (s == 12345.f) sink[blockIdx.x] = s;
}

extern "C" {

// read `bytes` (a multiple of 16) from p; sink holds at least
// brq_ref_stream_blocks(bytes) words
unsigned brq_ref_stream_blocks(size_t bytes) { return (unsigned)((bytes / 16 + 256 * 8 - 1) / (256 * 8)); }

int brq_ref_stream_read(const void* p, size_t bytes, void* sink, void* stream) {
  const size_t n16 = bytes / 16;
  hipLaunchKernelGGL(k_stream_read<8>, dim3(brq_ref_stream_blocks(bytes)), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(p), n16, static_cast<uint32_t*>(sink));
  return (int)hipGetLastError();
}

// `blocks` workgroups of 4 waves, each wave 8 * iters products of 32x32x16
// (32768 flops each); sink holds `blocks` floats
int brq_ref_mfma_loop(int blocks, int iters, void* sink, void* stream) {
  hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, static_cast<float*>(sink));
  return (int)hipGetLastError();
}

}  // extern "C"
