// Kronecker-factored orthogonal activation rotation x' = (H (x) R) x, computed
// per token as X' = H X R^T with X the token reshaped row-major to [n1][n2]
// (BWLA commentary: section 3, OKT with Kronecker factors; section 5, the same
// transform applied to the activations). bf16 output.
//
// X is n1 x n2 with n1, n2 in {32, 64, 96} (hidden sizes 1024 .. 6144; the
// prefill workload is 64 x 64). Both products run on the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16, fp32 accumulate). x is bf16 already; the
// fp32 factors H and R and the fp32 intermediate T = X R^T enter as three
// bf16 pieces each (v = p0 + p1 + p2, each piece the round-to-nearest of what
// is left, 24 significant bits together). T = sum_p X R_p^T (three products)
// and Y = sum_{p+q<=2} H_p T_q (six products): a product of two pieces is
// exact in fp32 and the dropped terms are below 2^-24 of the largest, so Y
// matches fp32 arithmetic to a few units of 2^-24 before its bf16 rounding.
//
// One wave per token (the waves of the grid take tokens in turn). The piece
// fragments of R and H are laid out in LDS once per workgroup in the per-lane
// operand order (fragment f, lane l at 16 (64 f + l) bytes: conflict-free
// 16-byte reads). X is read straight from global memory as the A operand
// (lane l: row 32i + l%32, k = 16s + 8(l/32) .. +7: 16 contiguous bytes).
// T's accumulator layout (lane l, item r: row 8(r/4) + 4(l/32) + r%4, column
// l%32) becomes the B operand of the second product (lane l: column l%32, k =
// 8(l/32) .. +7 of a 16-row step) with one permlane32 swap per pair of items:
// of the rows 16u .. 16u+15 of a tile, lanes 0-31 hold 0-3 and 8-11 and lanes
// 32-63 hold 4-7 and 12-15; swapping the upper lanes' first half with the
// lower lanes' second half leaves rows 0-7 in lanes 0-31 and 8-15 in 32-63.
#include "common.h"
#include "kernels.h"

namespace brq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// v = p0 + p1 + p2 (bf16 bits): each piece rounds what the previous left
// (exact remainders in fp32)
__device__ __forceinline__ void split3_bf16(float v, uint32_t& p0, uint32_t& p1, uint32_t& p2) {
  p0 = f32_to_bf16_bits(v);
  const float r0 = v - bf16_to_f32(p0);
  p1 = f32_to_bf16_bits(r0);
  const float r1 = r0 - bf16_to_f32(p1);
  p2 = f32_to_bf16_bits(r1);
}

constexpr int KRON_WAVES = 4;

// LDS bytes of the factor fragments for n1 = 32 A, n2 = 32 B: R has B row
// tiles of 2 B k-steps, H has A row tiles of 2 A k-steps, three pieces each,
// one 16-byte word per lane
constexpr size_t kron_lds(int A, int B) { return (size_t)(2 * B * B + 2 * A * A) * 3 * 64 * 16; }

// A = n1 / 32 row tiles of X (and of H), B = n2 / 32 row tiles of R (column
// tiles of T and Y)
template <int A, int B>
__global__ __launch_bounds__(64 * KRON_WAVES) void k_kron(const uint16_t* __restrict__ x, int M,
                                                         const float* __restrict__ H, const float* __restrict__ R,
                                                         uint16_t* __restrict__ y) {
  constexpr int N1 = 32 * A, N2 = 32 * B, SR = 2 * B, SH = 2 * A;  // k-steps of 16 per product
  constexpr int RF = B * SR;                                        // R fragment groups (before H's)
  extern __shared__ __attribute__((aligned(16))) uint4 kf[];        // [(RF + A*SH) * 3][64]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // fragment group g for lane l: R (g < RF: row tile g / SR, k-step g % SR)
  // or H (row tile (g - RF) / SH, k-step (g - RF) % SH); row 32 tile + l%32,
  // k = 16 s + 8 (l/32) + e, e = 0..7, as three piece fragments
  for (int idx = tid; idx < (RF + A * SH) * 64; idx += blockDim.x) {
    const int l = idx & 63, g = idx >> 6;
    const bool isr = g < RF;
    const int gg = isr ? g : g - RF, st = isr ? SR : SH, n = isr ? N2 : N1;
    const int tile = gg / st, ks = gg % st;
    const float* src = (isr ? R : H) + (32 * tile + (l & 31)) * n + 16 * ks + 8 * (l >> 5);
    uint32_t pc[3][4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t a0, a1, a2, b0, b1, b2;
      split3_bf16(src[2 * e2], a0, a1, a2);
      split3_bf16(src[2 * e2 + 1], b0, b1, b2);
      pc[0][e2] = a0 | (b0 << 16);
      pc[1][e2] = a1 | (b1 << 16);
      pc[2][e2] = a2 | (b2 << 16);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) kf[(g * 3 + p) * 64 + l] = make_uint4(pc[p][0], pc[p][1], pc[p][2], pc[p][3]);
  }
  __syncthreads();
  const int h = lane >> 5, c = lane & 31;
  const int nwaves = gridDim.x * KRON_WAVES;
  for (int t = blockIdx.x * KRON_WAVES + wave; t < M; t += nwaves) {
    // the fragments are read from LDS for every token: an opaque offset keeps
    // the compiler from hoisting all of them into registers, which would leave
    // room for one wave per SIMD only
    int lo = lane;
    asm volatile("" : "+v"(lo));
    const u32x4* fr = reinterpret_cast<const u32x4*>(kf) + lo;
    auto rfrag = [&](int j, int s, int p) { return fr[((j * SR + s) * 3 + p) * 64]; };
    auto hfrag = [&](int i, int s, int p) { return fr[((RF + i * SH + s) * 3 + p) * 64]; };
    const uint16_t* xt = x + (size_t)t * (N1 * N2);
    u32x4 xa[A][SR];
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
      for (int s = 0; s < SR; ++s) xa[i][s] = *reinterpret_cast<const u32x4*>(xt + (32 * i + c) * N2 + 16 * s + 8 * h);
    // Y = H T, one row tile of T at a time (T rows 32 ti .. are the k-steps
    // s = 2 ti, 2 ti + 1 of the second product), so that only one row tile of
    // T and its pieces are live at once
    f32x16 Y[A][B];
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
      for (int j = 0; j < B; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) Y[i][j][r] = 0.f;
#pragma unroll
    for (int ti = 0; ti < A; ++ti) {
      // T rows 32 ti .. 32 ti + 31 = X rows of that tile times R^T
      f32x16 T[B];
#pragma unroll
      for (int j = 0; j < B; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) T[j][r] = 0.f;
#pragma unroll
      for (int j = 0; j < B; ++j)
#pragma unroll
        for (int s = 0; s < SR; ++s)
#pragma unroll
          for (int p = 0; p < 3; ++p) T[j] = mfma32_bf16(xa[ti][s], rfrag(j, s, p), T[j]);
      // those rows as B operand pieces: piece q of column tile j, step 2 ti + u
      u32x4 tb[3][B][2];
#pragma unroll
      for (int j = 0; j < B; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float v[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(T[j][8 * u + q]),
                                                             __float_as_uint(T[j][8 * u + 4 + q]), false, false);
            v[q] = __uint_as_float(sw[0]);
            v[4 + q] = __uint_as_float(sw[1]);
          }
          uint32_t pc[3][4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t a0, a1, a2, b0, b1, b2;
            split3_bf16(v[2 * e2], a0, a1, a2);
            split3_bf16(v[2 * e2 + 1], b0, b1, b2);
            pc[0][e2] = a0 | (b0 << 16);
            pc[1][e2] = a1 | (b1 << 16);
            pc[2][e2] = a2 | (b2 << 16);
          }
#pragma unroll
          for (int q = 0; q < 3; ++q) tb[q][j][u] = u32x4{pc[q][0], pc[q][1], pc[q][2], pc[q][3]};
        }
      // Y += H_p T_q over the piece pairs p + q <= 2, steps 2 ti and 2 ti + 1
#pragma unroll
      for (int i = 0; i < A; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int p = 0; p < 3; ++p) {
            const u32x4 a = hfrag(i, 2 * ti + u, p);
#pragma unroll
            for (int q = 0; q + p < 3; ++q)
#pragma unroll
              for (int j = 0; j < B; ++j) Y[i][j] = mfma32_bf16(a, tb[q][j][u], Y[i][j]);
          }
    }
    // bf16 out: lane l holds column 32 j + l%32 of rows 32 i + 8 (r/4) + 4 h +
    // r%4. Neighbouring lanes trade one item of each pair (r, r+1): the even
    // lane then writes columns c, c+1 of row r, the odd lane columns c-1, c of
    // row r+1, four bytes each
    uint16_t* yt = y + (size_t)t * (N1 * N2);
    const bool odd = c & 1;
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
      for (int j = 0; j < B; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float a = Y[i][j][r], b = Y[i][j][r + 1];
          const float got = __shfl_xor(odd ? a : b, 1);
          const int row = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3) + (odd ? 1 : 0);
          const uint32_t lo = f32_to_bf16_bits(odd ? got : a), hi = f32_to_bf16_bits(odd ? b : got);
          *reinterpret_cast<uint32_t*>(yt + row * N2 + 32 * j + (c & ~1)) = lo | (hi << 16);
        }
  }
}

bool kron_supported(int64_t n1, int64_t n2) {
  const bool f1 = n1 == 32 || n1 == 64 || n1 == 96, f2 = n2 == 32 || n2 == 64 || n2 == 96;
  return f1 && f2 && (n1 / 32) * (n2 / 32) <= 6;
}

template <int A, int B>
static void run_kron(const uint16_t* x, int M, const float* H, const float* R, uint16_t* y, hipStream_t st) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  // as many workgroups per compute unit as their fragments fit the 160 KiB of
  // LDS (three at most), so that a workgroup's fragment set-up hides behind
  // the others' tokens
  constexpr size_t lds = kron_lds(A, B);
  constexpr int per_cu = (int)((160 * 1024) / lds) < 3 ? (int)((160 * 1024) / lds) : 3;
  if (lds > 64 * 1024) (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_kron<A, B>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int need = (M + KRON_WAVES - 1) / KRON_WAVES;
  const int grid = need < per_cu * cus ? need : per_cu * cus;
  hipLaunchKernelGGL((k_kron<A, B>), dim3(grid), dim3(64 * KRON_WAVES), lds, st, x, M, H, R, y);
}

hipError_t launch_kron(const uint16_t* x, int M, int n1, int n2, const float* H, const float* R, uint16_t* y,
                       hipStream_t st) {
  switch ((n1 / 32) * 4 + n2 / 32) {
    case 1 * 4 + 1: run_kron<1, 1>(x, M, H, R, y, st); break;
    case 1 * 4 + 2: run_kron<1, 2>(x, M, H, R, y, st); break;
    case 1 * 4 + 3: run_kron<1, 3>(x, M, H, R, y, st); break;
    case 2 * 4 + 1: run_kron<2, 1>(x, M, H, R, y, st); break;
    case 2 * 4 + 2: run_kron<2, 2>(x, M, H, R, y, st); break;
    case 2 * 4 + 3: run_kron<2, 3>(x, M, H, R, y, st); break;
    case 3 * 4 + 1: run_kron<3, 1>(x, M, H, R, y, st); break;
    case 3 * 4 + 2: run_kron<3, 2>(x, M, H, R, y, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace brq
