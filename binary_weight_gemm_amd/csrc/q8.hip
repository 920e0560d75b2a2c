// The DBF chain over sign-magnitude Q8 activations, the prompt-processing
// formulation of "LLM binarization, Episode 01: DBF" (section 5, item 4): each
// activation row is denormalised to one shared exponent and encoded in 8 bits
// (a sign and seven magnitude bits), the binary product of a row is an exact
// integer reduction of weight signs times activation codes, and one shared
// scale follows. The pages evaluate that reduction with XOR + AND + POPCOUNT +
// SHIFT + ADD over bitplanes; on gfx950 the same integer comes from the int8
// matrix cores (v_mfma_i32_32x32x32_i8) with the weights as +-1 bytes, exact
// in int32.
//
//   k_q8_rows: one workgroup per row: v = x * d_in (bf16 x fp16, exact in
//     fp32) or v = h_s (fp32); e = the smallest integer with max|v| <= 127 *
//     2^e; q = round-half-even(v / 2^e) as int8, natural order.
//   k_tile_q8: 128 x 128 output tiles of the product of the codes with a +-1
//     sign plane, 64-wide k-steps, four waves of 64 x 64 (2 x 2 MFMAs of 32 x
//     32 x 32); the sign words of a k-step become +-1 bytes in LDS (a byte
//     permute with the 0x00 / 0xFF selectors per four signs). Epilogue:
//     h_s = fp32(d_mid * (acc * 2^e)) (stage 1) or y = d_out * (acc * 2^e).
#include "common.h"
#include "kernels.h"

namespace brq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// ---- quantisation of rows ---------------------------------------------------

template <bool FROM_BF16>
__global__ __launch_bounds__(256) void k_q8_rows(const void* __restrict__ src, const uint16_t* __restrict__ d_in,
                                                 int K, int8_t* __restrict__ q, int* __restrict__ rexp) {
  __shared__ uint32_t s_max[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  // value k of the row (exact in fp32)
  auto val = [&](int k) -> float {
    if (FROM_BF16) {
      const uint16_t* x = reinterpret_cast<const uint16_t*>(src) + (size_t)t * K;
      return bf16_to_f32(x[k]) * f16_bits_to_f32(d_in[k]);
    }
    return reinterpret_cast<const float*>(src)[(size_t)t * K + k];
  };
  uint32_t mx = 0;
  for (int k = tid; k < K; k += 256) mx = max(mx, __float_as_uint(val(k)) & 0x7fffffffu);
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) s_max[tid >> 6] = mx;
  __syncthreads();
  mx = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const float m = __uint_as_float(mx);
  int e = 0;
  if (m > 0.f) {
    const int E = ilogbf(m);  // 2^E <= m < 2^(E+1)
    e = (m <= __builtin_amdgcn_ldexpf(127.f, E - 6)) ? E - 6 : E - 5;
  }
  if (tid == 0) rexp[t] = e;
  for (int k = tid; k < K; k += 256)
    q[(size_t)t * K + k] = (int8_t)(int)__builtin_rintf(__builtin_amdgcn_ldexpf(val(k), -e));
}

// ---- product of codes with a sign plane --------------------------------------

// four sign bits (bit i -> weight i) as four bytes: 0xFF (bit set: -1) or 0x01
__device__ __forceinline__ uint32_t signs4_to_bytes(uint32_t nib) {
  const uint32_t spread = (nib * 0x00204081u) & 0x01010101u;  // bit i -> byte i
  // byte permute: selector 0x0C gives 0x00, 0x0D gives 0xFF
  const uint32_t mask = __builtin_amdgcn_perm(0u, 0u, 0x0C0C0C0Cu + spread);
  return mask | 0x01010101u;
}

template <bool STAGE2>
__global__ __launch_bounds__(256) void k_tile_q8(const int8_t* __restrict__ a, const int* __restrict__ rexp, int M,
                                                 int N, int K, const uint32_t* __restrict__ signs,
                                                 const uint16_t* __restrict__ diag, void* __restrict__ out,
                                                 int out_bf16) {
  constexpr int BM = 128, BN = 128, BK = 64, LDB = BK + 16;  // LDS row: 64 bytes + 16 against bank conflicts
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * LDB];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * LDB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int tiles_n = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
  const int nk = K / BK;
  const int KW = K >> 5;  // sign dwords per weight row

  // staging: thread tid moves A bytes [row tid/2][32 (tid%2) .. +32) (two
  // 16-byte loads) and the sign dword of column tid/2, k-half tid%2
  const int srow = tid >> 1, shalf = tid & 1;
  const int gm = m0 + srow < M ? m0 + srow : M - 1;  // rows past M repeat the last (never stored)
  const int gn = n0 + srow < N ? n0 + srow : N - 1;  // columns past N repeat the last (never stored)
  const int8_t* asrc = a + (size_t)gm * K + 32 * shalf;
  const uint32_t* wsrc = signs + (size_t)gn * KW + shalf;
  const int lofs = srow * LDB + 32 * shalf;
  uint4 ra0 = *reinterpret_cast<const uint4*>(asrc), ra1 = *reinterpret_cast<const uint4*>(asrc + 16);
  uint32_t rw = *wsrc;
#define Q8_STORE_STAGE(buf)                                                                                   \
  {                                                                                                          \
    uint4* da = reinterpret_cast<uint4*>(&As[buf][lofs]);                                                    \
    da[0] = ra0;                                                                                             \
    da[1] = ra1;                                                                                             \
    uint4* db = reinterpret_cast<uint4*>(&Bs[buf][lofs]);                                                    \
    db[0] = make_uint4(signs4_to_bytes(rw & 0xFu), signs4_to_bytes((rw >> 4) & 0xFu),                        \
                       signs4_to_bytes((rw >> 8) & 0xFu), signs4_to_bytes((rw >> 12) & 0xFu));               \
    db[1] = make_uint4(signs4_to_bytes((rw >> 16) & 0xFu), signs4_to_bytes((rw >> 20) & 0xFu),               \
                       signs4_to_bytes((rw >> 24) & 0xFu), signs4_to_bytes(rw >> 28));                       \
  }

  i32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  Q8_STORE_STAGE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      ra0 = *reinterpret_cast<const uint4*>(asrc + (kt + 1) * BK);
      ra1 = *reinterpret_cast<const uint4*>(asrc + (kt + 1) * BK + 16);
      rw = wsrc[(kt + 1) * 2];
    }
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      // lane l: row (column) l%32 of its 32-tile, bytes k = 32 ks + 16 (l/32) .. +15
      const int kofs = 32 * ks + 16 * (lane >> 5);
      i32x4 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const i32x4*>(&As[cur][(wr * 64 + 32 * i + (lane & 31)) * LDB + kofs]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const i32x4*>(&Bs[cur][(wc * 64 + 32 * j + (lane & 31)) * LDB + kofs]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) Q8_STORE_STAGE(cur ^ 1);
    __syncthreads();
  }
#undef Q8_STORE_STAGE

  // epilogue: lane l holds, in item r, row 8(r/4) + 4(l/32) + r%4 of column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wc * 64 + 32 * j + (lane & 31);
      if (col >= N) continue;
      const float dg = f16_bits_to_f32(diag[col]);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wr * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= M) continue;
        const float v = dg * __builtin_amdgcn_ldexpf((float)acc[i][j][r], rexp[row]);
        if (STAGE2)
          store_out(out, (size_t)row * N + col, v, out_bf16);
        else
          reinterpret_cast<float*>(out)[(size_t)row * N + col] = v;
      }
    }
}

// workspace: q1 int8 [M][n], e1 [M], h_s fp32 [M][r], q2 int8 [M][r], e2 [M]
size_t dbf_q8_ws_bytes(int64_t M, int64_t m, int64_t n, int64_t r) {
  (void)m;
  return align256((size_t)M * n) + align256((size_t)M * 4) + align256((size_t)M * r * 4) + align256((size_t)M * r) +
         align256((size_t)M * 4);
}

hipError_t launch_dbf_q8(const uint16_t* x, int M, int m, int n, int r, const uint16_t* d_in, const uint64_t* v,
                         const uint16_t* d_mid, const uint64_t* u, const uint16_t* d_out, void* y, int y_bf16,
                         void* ws, hipStream_t st) {
  char* p = reinterpret_cast<char*>(ws);
  auto take = [&](size_t bytes) { char* q = p; p += align256(bytes); return q; };
  int8_t* q1 = reinterpret_cast<int8_t*>(take((size_t)M * n));
  int* e1 = reinterpret_cast<int*>(take((size_t)M * 4));
  float* hs = reinterpret_cast<float*>(take((size_t)M * r * 4));
  int8_t* q2 = reinterpret_cast<int8_t*>(take((size_t)M * r));
  int* e2 = reinterpret_cast<int*>(take((size_t)M * 4));
  const uint32_t* v32 = reinterpret_cast<const uint32_t*>(v);
  const uint32_t* u32 = reinterpret_cast<const uint32_t*>(u);
  hipLaunchKernelGGL(k_q8_rows<true>, dim3(M), dim3(256), 0, st, x, d_in, n, q1, e1);
  const int t1 = ((M + 127) / 128) * ((r + 127) / 128);
  hipLaunchKernelGGL(k_tile_q8<false>, dim3(t1), dim3(256), 0, st, q1, e1, M, r, n, v32, d_mid, hs, 0);
  hipLaunchKernelGGL(k_q8_rows<false>, dim3(M), dim3(256), 0, st, hs, nullptr, r, q2, e2);
  const int t2 = ((M + 127) / 128) * ((m + 127) / 128);
  hipLaunchKernelGGL(k_tile_q8<true>, dim3(t2), dim3(256), 0, st, q2, e2, M, m, r, u32, d_out, y, y_bf16);
  return hipGetLastError();
}

}  // namespace brq
