// The DBF chain over sign-magnitude Q8 activations, the prompt-processing
// formulation of "LLM binarization, Episode 01: DBF" (section 5, item 4): each
// activation row is denormalised to one shared exponent and encoded in 8 bits
// (a sign and seven magnitude bits), the binary product of a row is an exact
// integer reduction of weight signs times activation codes, and one shared
// scale follows. The pages evaluate that reduction over bitplanes with masked
// population counts; on gfx950 the same integer comes from the int8 matrix
// cores (v_mfma_i32_32x32x32_i8) with the weights as +-1 bytes, exact in int32
// (section 5, item 1 names that form of the reduction).
//
//   k_q8_rows_reg / k_q8_rows: one workgroup per row: v = x * d_in (bf16 x
//     fp16, exact in fp32), v = h_s (fp32), or h_s from int32 K-slice sums;
//     e = the smallest integer with max|v| <= 127 * 2^e; q = round-half-even
//     (v / 2^e) as int8, stored in the k order shared with the weight bytes.
//   k_tile_q8: output tiles of 128 columns by 128 rows (four waves of 64 x
//     64) or 64 rows (32 x 64) of the product of the codes with a +-1 sign
//     plane on MFMAs of 32 x 32 x 32; codes and packed sign dwords move to
//     LDS by direct loads, three stages of 128 k deep; each lane turns a sign
//     dword into its four dwords of +-1 bytes with one AND and one byte
//     permute each. Epilogue: h_s = fp32(d_mid * (acc * 2^e)) (first
//     product), y = d_out * (acc * 2^e) (second), or the raw int32 sums of a
//     K-slice.
//   k_q8_out: y from the K-slice sums of the second product.
#include "common.h"
#include "kernels.h"

namespace brq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// Codes and weight bytes share a k order inside every 32-wide group: byte
// p = 4 d + j of the group holds k = 8 j + d (dword d gathers k = d, d + 8,
// d + 16, d + 24). In that order dword d of the weight bytes of a 32-bit sign
// word w is one byte permute of the selector w & (0x01010101 << d): a
// selector byte is 0 (bit clear: byte 0 of 0x00FFFF01, 0x01) or 2^d (set:
// 1 -> byte 1, 2 -> byte 2, 4 -> byte 4 = the low byte of 0x000000FF, 8 -> the
// sign of bit 15 of 0x00FFFF01, 16 and above -> 0xFF), so -1 or +1.
__device__ __forceinline__ int q8_pos(int k) { return (k & ~31) + 4 * (k & 7) + ((k >> 3) & 3); }


// ---- quantisation of rows ---------------------------------------------------

enum { SRC_XDIN, SRC_F32, SRC_PART };

// SRC_XDIN: v = x * d_in (bf16 x fp16, exact in fp32); SRC_F32: v = h_s;
// SRC_PART: v = h_s = fp32(d_mid * (s * 2^e1)), s the sum of the nsplit int32
// K-slice partials of the first product (exact: |s| < 2^24)
template <int SRC>
__global__ __launch_bounds__(256) void k_q8_rows(const void* __restrict__ src, const uint16_t* __restrict__ diag,
                                                 const int* __restrict__ rexp_in, int nsplit, int M, int K,
                                                 int8_t* __restrict__ q, int* __restrict__ rexp) {
  __shared__ uint32_t s_max[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int e_in = SRC == SRC_PART ? rexp_in[t] : 0;
  auto val = [&](int k) -> float {
    if (SRC == SRC_XDIN) {
      const uint16_t* x = reinterpret_cast<const uint16_t*>(src) + (size_t)t * K;
      return bf16_to_f32(x[k]) * f16_bits_to_f32(diag[k]);
    }
    if (SRC == SRC_F32) return reinterpret_cast<const float*>(src)[(size_t)t * K + k];
    const int* part = reinterpret_cast<const int*>(src) + (size_t)t * K + k;
    int sum = 0;
    for (int s = 0; s < nsplit; ++s) sum += part[(size_t)s * M * K];
    return f16_bits_to_f32(diag[k]) * __builtin_amdgcn_ldexpf((float)sum, e_in);
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
    q[(size_t)t * K + q8_pos(k)] = (int8_t)(int)__builtin_rintf(__builtin_amdgcn_ldexpf(val(k), -e));
}

// The same quantisation with the row held in registers: thread tid takes the
// 8-element groups tid, tid + 256, ... (NG of them, K <= 2048 NG), read with
// 16-byte loads and written as 8-byte codes.
template <int SRC, int NG>
__global__ __launch_bounds__(256) void k_q8_rows_reg(const void* __restrict__ src, const uint16_t* __restrict__ diag,
                                                     const int* __restrict__ rexp_in, int nsplit, int M, int K,
                                                     int8_t* __restrict__ q, int* __restrict__ rexp) {
  __shared__ uint32_t s_max[4];
  __shared__ __attribute__((aligned(16))) int8_t s_code[NG * 2048];
  const int t = blockIdx.x, tid = threadIdx.x;
  f32x4 v[NG][2];
  uint32_t mx = 0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int k = (g * 256 + tid) * 8;
    v[g][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    v[g][1] = v[g][0];
    if (k >= K) continue;
    const size_t o = (size_t)t * K + k;
    if (SRC == SRC_XDIN) {
      const uint4 xb = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(src) + o);
      const uint4 db = *reinterpret_cast<const uint4*>(diag + k);
      const uint32_t xw[4] = {xb.x, xb.y, xb.z, xb.w}, dw[4] = {db.x, db.y, db.z, db.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[g][h >> 1][2 * (h & 1)] = bf16_to_f32(xw[h] & 0xFFFFu) * f16_bits_to_f32(dw[h] & 0xFFFFu);
        v[g][h >> 1][2 * (h & 1) + 1] = bf16_to_f32(xw[h] >> 16) * f16_bits_to_f32(dw[h] >> 16);
      }
    } else if (SRC == SRC_F32) {
      const float* hs = reinterpret_cast<const float*>(src) + o;
      v[g][0] = *reinterpret_cast<const f32x4*>(hs);
      v[g][1] = *reinterpret_cast<const f32x4*>(hs + 4);
    } else {
      const int* part = reinterpret_cast<const int*>(src) + o;
      i32x4 s0 = *reinterpret_cast<const i32x4*>(part), s1 = *reinterpret_cast<const i32x4*>(part + 4);
      for (int sl = 1; sl < nsplit; ++sl) {
        s0 += *reinterpret_cast<const i32x4*>(part + (size_t)sl * M * K);
        s1 += *reinterpret_cast<const i32x4*>(part + (size_t)sl * M * K + 4);
      }
      const int e_in = rexp_in[t];
      const uint4 db = *reinterpret_cast<const uint4*>(diag + k);
      const uint32_t dw[4] = {db.x, db.y, db.z, db.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int a0 = (h < 2 ? s0 : s1)[2 * (h & 1)], a1 = (h < 2 ? s0 : s1)[2 * (h & 1) + 1];
        v[g][h >> 1][2 * (h & 1)] = f16_bits_to_f32(dw[h] & 0xFFFFu) * __builtin_amdgcn_ldexpf((float)a0, e_in);
        v[g][h >> 1][2 * (h & 1) + 1] = f16_bits_to_f32(dw[h] >> 16) * __builtin_amdgcn_ldexpf((float)a1, e_in);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = max(mx, __float_as_uint(v[g][h][c]) & 0x7fffffffu);
  }
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
  // the codes go to their positions in the shared k order through LDS (byte
  // p of a 32-wide group gathers from four threads), then out 8 bytes a thread
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int k = (g * 256 + tid) * 8;
    if (k >= K) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      s_code[q8_pos(k + i)] = (int8_t)(int)__builtin_rintf(__builtin_amdgcn_ldexpf(v[g][i >> 2][i & 3], -e));
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int k = (g * 256 + tid) * 8;
    if (k >= K) continue;
    *reinterpret_cast<uint2*>(q + (size_t)t * K + k) = *reinterpret_cast<const uint2*>(&s_code[k]);
  }
}

template <int SRC>
static void launch_q8_rows(const void* src, const uint16_t* diag, const int* rexp_in, int nsplit, int M, int K,
                           int8_t* q, int* rexp, hipStream_t st) {
  const int ng = (K + 2047) / 2048;
  const dim3 g(M), b(256);
  if (ng <= 1)
    hipLaunchKernelGGL((k_q8_rows_reg<SRC, 1>), g, b, 0, st, src, diag, rexp_in, nsplit, M, K, q, rexp);
  else if (ng <= 2)
    hipLaunchKernelGGL((k_q8_rows_reg<SRC, 2>), g, b, 0, st, src, diag, rexp_in, nsplit, M, K, q, rexp);
  else if (ng <= 4)
    hipLaunchKernelGGL((k_q8_rows_reg<SRC, 4>), g, b, 0, st, src, diag, rexp_in, nsplit, M, K, q, rexp);
  else if (ng <= 8)
    hipLaunchKernelGGL((k_q8_rows_reg<SRC, 8>), g, b, 0, st, src, diag, rexp_in, nsplit, M, K, q, rexp);
  else
    hipLaunchKernelGGL(k_q8_rows<SRC>, g, b, 0, st, src, diag, rexp_in, nsplit, M, K, q, rexp);
}

// y = fp32(d_out * (s * 2^e2)), s the sum of the nsplit int32 partials of the
// second product; four consecutive outputs per thread
__global__ __launch_bounds__(256) void k_q8_out(const int* __restrict__ part, int nsplit, int M, int N,
                                                const int* __restrict__ rexp, const uint16_t* __restrict__ diag,
                                                void* __restrict__ y, int y_bf16) {
  const size_t MN = (size_t)M * N;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  if ((N & 3) == 0) {  // the four share a row; 16-byte loads
    i32x4 sum = *reinterpret_cast<const i32x4*>(part + i);
    for (int s = 1; s < nsplit; ++s) sum += *reinterpret_cast<const i32x4*>(part + (size_t)s * MN + i);
    const int row = (int)(i / N), col = (int)(i % N), e = rexp[row];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_out(y, i + j, f16_bits_to_f32(diag[col + j]) * __builtin_amdgcn_ldexpf((float)sum[j], e), y_bf16);
    return;
  }
  for (int j = 0; j < 4 && i + j < MN; ++j) {
    int sum = 0;
    for (int s = 0; s < nsplit; ++s) sum += part[(size_t)s * MN + i + j];
    const int row = (int)((i + j) / N), col = (int)((i + j) % N);
    store_out(y, i + j, f16_bits_to_f32(diag[col]) * __builtin_amdgcn_ldexpf((float)sum, rexp[row]), y_bf16);
  }
}

// ---- product of codes with a sign plane --------------------------------------

enum { OUT_HS, OUT_Y, OUT_PART };

// chunk slot of row r in a stage row of eight 16-byte chunks: 8 consecutive
// rows (one 128-byte bank line each) and 16 consecutive rows (pairs sharing
// a 256-byte line) both land on distinct slots
__device__ __forceinline__ int q8_swz8(int r) { return (r ^ (r >> 3)) & 7; }

// OUT_HS: h_s = fp32(diag * (acc * 2^e)) as fp32 [M][N]; OUT_Y: the same
// value as y_dtype; OUT_PART: the raw int32 sums of K-slice blockIdx.y into
// part[blockIdx.y][M][N]
// BM = 128 (waves of 64 x 64) or 64 (waves of 32 x 64), 128 columns per tile
template <int OUT, int BM>
__global__ __launch_bounds__(256) void k_tile_q8(const int8_t* __restrict__ a, const int* __restrict__ rexp, int M,
                                                 int N, int K, const uint32_t* __restrict__ signs,
                                                 const uint16_t* __restrict__ diag, void* __restrict__ out,
                                                 int out_bf16) {
  // Stages of 128 k move global -> LDS by direct loads (no registers), three
  // stages deep, so that the loads run two stages ahead of the products even
  // at one workgroup per compute unit. A stage holds the code tile (128 rows
  // of 128 bytes; the 16-byte chunk c of row r sits at chunk c ^ q8_swz8(r),
  // which keeps the fragment reads of 32 rows on distinct banks) and the
  // packed sign dwords of the tile's columns (4 per column); the +-1 weight
  // fragments are built in registers.
  constexpr int BN = 128, BKS = 128;  // BKS: k per stage
  constexpr int NI = BM / 64;         // 32-row blocks per wave
  constexpr int WROWS = BM / 2;       // rows per wave row
  constexpr int ALD = BM / 32;        // code loads per wave and stage (8 rows each)
  static_assert(ALD == 4 || ALD == 2, "tile height 128 or 64");
  // bytes, dwords per stage; the LDS arrays are sized for 128-row tiles
  // whatever BM (shared arrays of a size that depends on a template parameter
  // leave the host compiler without a launch stub for the kernel)
  constexpr int A_ST = 128 * BKS, W_ST = BN * 4;
  // one variable per stage buffer: each gets its own alias scope, so that the
  // fragment reads of one buffer need not wait for the direct loads into
  // another (the stage loop is unrolled so that every access names its buffer)
  __shared__ __attribute__((aligned(16))) int8_t A0[A_ST], A1[A_ST], A2[A_ST];
  __shared__ __attribute__((aligned(16))) uint32_t W0[W_ST], W1[W_ST], W2[W_ST];
#define Q8_ABUF(b) ((b) == 0 ? A0 : (b) == 1 ? A1 : A2)
#define Q8_WBUF(b) ((b) == 0 ? W0 : (b) == 1 ? W1 : W2)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  // tile id -> (row tile, column tile). Workgroups go to the 8 XCDs in turn
  // (id % 8); the first 8 floor(T / 8) ids are renumbered so that each XCD
  // takes a contiguous run of tiles, i.e. few activation row blocks per L2
  const int tiles_n = (N + BN - 1) / BN, ntiles = gridDim.x, per = ntiles >> 3;
  int bid = blockIdx.x;
  if (bid < 8 * per) bid = (bid & 7) * per + (bid >> 3);
  const int m0 = (bid / tiles_n) * BM, n0 = (bid % tiles_n) * BN;
  const int ns = K / BKS / gridDim.y;  // stages of this K-slice
  const int k0 = blockIdx.y * ns * BKS;
  const int KW = K >> 5;  // sign dwords per weight row

  // epilogue operands, fetched before the k-loop: the row exponents of the
  // tile (LDS, visible after the first barrier) and this lane's column scales
  __shared__ int s_rexp[128];
  float dgv[2] = {0.f, 0.f};
  if (OUT != OUT_PART) {
    if (tid < BM) s_rexp[tid] = rexp[m0 + tid < M ? m0 + tid : M - 1];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = n0 + wc * 64 + 32 * j + (lane & 31);
      dgv[j] = f16_bits_to_f32(diag[c < N ? c : N - 1]);
    }
  }
  // direct loads of a stage. Codes: wave w, load i writes rows (BM/4) w + 8 i
  // .. +7 (1 KB); lane L takes row (BM/4) w + 8 i + L/8, physical chunk L%8,
  // i.e. logical chunk (L%8) ^ q8_swz8(row). Signs: load t of wave w writes dword
  // slots 256 t + 64 w + L: column slot/4, dword slot%4 of the stage.
  const int8_t* a_src[ALD];
#pragma unroll
  for (int i = 0; i < ALD; ++i) {
    const int r = (BM / 4) * wave + 8 * i + (lane >> 3);
    const int gr = m0 + r < M ? m0 + r : M - 1;  // rows past M repeat the last (never stored)
    a_src[i] = a + (size_t)gr * K + k0 + 16 * ((lane & 7) ^ q8_swz8(r));
  }
  const uint32_t* w_src[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int slot = 256 * t + 64 * wave + lane, c = n0 + (slot >> 2);
    w_src[t] = signs + (size_t)(c < N ? c : N - 1) * KW + (k0 >> 5) + (slot & 3);
  }
  auto issue = [&](int p, int buf) {  // stage p (clamped to the slice) into buffer buf
    const int q = p < ns ? p : ns - 1;
#pragma unroll
    for (int i = 0; i < ALD; ++i)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a_src[i] + (size_t)q * BKS),
                                       Q8_ABUF(buf) + ((BM / 4) * wave + 8 * i) * BKS, 16, 0, 0);
#pragma unroll
    for (int t = 0; t < 2; ++t)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(w_src[t] + 4 * q),
                                       Q8_WBUF(buf) + 256 * t + 64 * wave, 4, 0, 0);
  };

  // weight fragments: lane l takes column 32 j + l%32 of its wave's 64, and
  // of the 32-wide group of a sub-step the bytes 16 (l/32) .. +15, i.e.
  // dwords d = 4 (l/32) .. +3 of the expanded sign dword
  uint32_t msk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) msk[i] = 0x01010101u << (4 * (lane >> 5) + i);
  auto bfrag = [&](uint32_t w) {
    return i32x4{(int)__builtin_amdgcn_perm(0x000000FFu, 0x00FFFF01u, w & msk[0]),
                 (int)__builtin_amdgcn_perm(0x000000FFu, 0x00FFFF01u, w & msk[1]),
                 (int)__builtin_amdgcn_perm(0x000000FFu, 0x00FFFF01u, w & msk[2]),
                 (int)__builtin_amdgcn_perm(0x000000FFu, 0x00FFFF01u, w & msk[3])};
  };

  i32x16 acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // fragment reads: lane l takes row wr BM/2 + 32 i + l%32, logical chunk
  // 2 u + l/32 of sub-step u
  int a_row[NI], a_swz[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = wr * WROWS + 32 * i + (lane & 31);
    a_row[i] = r * BKS;
    a_swz[i] = q8_swz8(r);
  }
  // one stage: 4 sub-steps of 32 k, each 4 MFMAs; the fragment reads and
  // the weight expansion of sub-step u + 1 are placed between the MFMAs of
  // sub-step u (scheduling-group barriers), so that one wave per SIMD keeps
  // its matrix core busy while they complete
  auto compute = [&](int buf) {
    const int8_t* ab = Q8_ABUF(buf);
    const uint32_t* wb = Q8_WBUF(buf);
    uint4 sw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) sw[j] = *reinterpret_cast<const uint4*>(wb + 4 * (wc * 64 + 32 * j + (lane & 31)));
    auto wdw = [&](int j, int u) { return u == 0 ? sw[j].x : u == 1 ? sw[j].y : u == 2 ? sw[j].z : sw[j].w; };
    i32x4 af[2][NI], bf[2][2];  // [buffer][block]
#pragma unroll
    for (int i = 0; i < NI; ++i)
      af[0][i] = *reinterpret_cast<const i32x4*>(ab + a_row[i] + 16 * ((lane >> 5) ^ a_swz[i]));
#pragma unroll
    for (int j = 0; j < 2; ++j) bf[0][j] = bfrag(wdw(j, 0));
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = u & 1, n = c ^ 1;
      if (u < 3) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          af[n][i] = *reinterpret_cast<const i32x4*>(ab + a_row[i] + 16 * ((2 * (u + 1) + (lane >> 5)) ^ a_swz[i]));
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[n][j] = bfrag(wdw(j, u + 1));
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[c][i], bf[c][j], acc[i][j], 0, 0, 0);
      if (u < 3) {
#pragma unroll
        for (int m = 0; m < 2 * NI; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // one MFMA
          if (m < NI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);               // four VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // stage p computes from buffer p % 3. Before it, each wave waits for its
  // own loads of stage p (those of stage p + 1, ALD + 2 per wave, may stay in
  // flight) and meets the others at a barrier: stage p is then complete in
  // LDS and every wave is done with stage p - 1, whose buffer takes p + 2.
  auto stage = [&](int p, int d) {  // d = p % 3, a constant after unrolling
    // s_waitcnt vmcnt(ALD + 2) expcnt(7) lgkmcnt(0) as a builtin, which the
    // compiler's own wait placement takes into account; the barrier in asm
    // with a memory clobber keeps the LDS accesses on their side of it
    if constexpr (ALD == 4)
      __builtin_amdgcn_s_waitcnt(0x0076);
    else
      __builtin_amdgcn_s_waitcnt(0x0074);
    asm volatile("s_barrier" ::: "memory");
    issue(p + 2, (d + 2) % 3);
    compute(d);
  };
  issue(0, 0);
  issue(1, 1);
  // whole rounds of three stages with no branch inside, then the last one or two
  int p = 0;
  for (; p + 3 <= ns; p += 3) {
#pragma unroll
    for (int d = 0; d < 3; ++d) stage(p + d, d);
  }
  if (p < ns) stage(p, 0);
  if (p + 1 < ns) stage(p + 1, 1);
  __builtin_amdgcn_s_waitcnt(0);  // nothing in flight when the workgroup ends
#undef Q8_ABUF
#undef Q8_WBUF

  // epilogue: lane l holds, in item r, row 8(r/4) + 4(l/32) + r%4 of column
  // l%32. A bf16 y trades one item of each pair (r, r + 1) (adjacent rows)
  // with the neighbouring lane: the even lane then writes columns c, c + 1 of
  // row r, the odd lane columns c - 1, c of row r + 1, four bytes each.
  const bool odd = lane & 1;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wc * 64 + 32 * j + (lane & 31);
      const int rbase = wr * WROWS + 32 * i + 4 * (lane >> 5);  // tile row of item 0
      if (OUT == OUT_Y) {
        if (out_bf16) {
          const int col0 = col & ~1;  // the pair's first column
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const int tr = rbase + 8 * (r >> 2) + (r & 3);
            const float a0 = dgv[j] * __builtin_amdgcn_ldexpf((float)acc[i][j][r], s_rexp[tr]);
            const float a1 = dgv[j] * __builtin_amdgcn_ldexpf((float)acc[i][j][r + 1], s_rexp[tr + 1]);
            const float got = __shfl_xor(odd ? a0 : a1, 1);
            const int row = m0 + tr + (odd ? 1 : 0);
            if (row >= M || col0 >= N) continue;
            const uint32_t lo = f32_to_bf16_bits(odd ? got : a0), hi = f32_to_bf16_bits(odd ? a1 : got);
            uint16_t* yp = reinterpret_cast<uint16_t*>(out);
            const size_t e = (size_t)row * N + col0;
            if (col0 + 1 >= N) {  // odd N: the last column alone
              yp[e] = (uint16_t)lo;
            } else if ((e & 1) == 0) {
              *reinterpret_cast<uint32_t*>(yp + e) = lo | (hi << 16);
            } else {  // odd N, odd row: the pair straddles a 4-byte boundary
              yp[e] = (uint16_t)lo;
              yp[e + 1] = (uint16_t)hi;
            }
          }
          continue;
        }
      }
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = rbase + 8 * (r >> 2) + (r & 3);
        const int row = m0 + tr;
        if (row >= M) continue;
        const size_t o = (size_t)row * N + col;
        if (OUT == OUT_PART) {
          reinterpret_cast<int*>(out)[(size_t)blockIdx.y * M * N + o] = acc[i][j][r];
        } else {
          const float v = dgv[j] * __builtin_amdgcn_ldexpf((float)acc[i][j][r], s_rexp[tr]);
          reinterpret_cast<float*>(out)[o] = v;
        }
      }
    }
}

// K-slices of a product with `tiles` output tiles and nk 64-wide k-steps (nk
// even): doubled while the grid stays within 128 workgroups and every slice
// keeps an even number of k-steps (the loop runs whole pairs), at least 8.
// The int32 partials cost a write and a read of ks M N words, so few slices
// are taken (measured at 512 x 4096 x 4096 x 2048: 128 beats 64, 256, 512)
int q8_ksplit(int tiles, int nk) {
  int ks = 1;
  while (tiles * ks * 2 <= 128 && nk % (4 * ks) == 0 && nk / (2 * ks) >= 8) ks *= 2;
  return ks;
}

// tile height and K-slices of an M x N product with reduction length K:
// 64-row tiles when 128-row tiles would not give every compute unit one
struct Q8Plan {
  int bm, ks, tiles;
};
static Q8Plan q8_plan(int64_t M, int64_t N, int64_t K) {
  const int tn = (int)((N + 127) / 128);
  const int bm = ((M + 127) / 128) * tn < 256 ? 64 : 128;
  const int tiles = (int)((M + bm - 1) / bm) * tn;
  return Q8Plan{bm, q8_ksplit(tiles, (int)(K / 64)), tiles};
}

// workspace: q1 int8 [M][n], e1 [M], h_s fp32 [M][r], q2 int8 [M][r], e2 [M],
// int32 K-slice partials [max(ks1 r, ks2 m)][M]
static void q8_splits(int64_t M, int64_t m, int64_t n, int64_t r, int& ks1, int& ks2) {
  ks1 = q8_plan(M, r, n).ks;
  ks2 = q8_plan(M, m, r).ks;
}

template <int OUT>
static void launch_tile_q8(const Q8Plan& pl, const int8_t* a, const int* rexp, int M, int N, int K,
                           const uint32_t* signs, const uint16_t* diag, void* out, int out_bf16, hipStream_t st) {
  const dim3 g(pl.tiles, pl.ks), b(256);
  if (pl.bm == 64)
    hipLaunchKernelGGL((k_tile_q8<OUT, 64>), g, b, 0, st, a, rexp, M, N, K, signs, diag, out, out_bf16);
  else
    hipLaunchKernelGGL((k_tile_q8<OUT, 128>), g, b, 0, st, a, rexp, M, N, K, signs, diag, out, out_bf16);
}

size_t dbf_q8_ws_bytes(int64_t M, int64_t m, int64_t n, int64_t r) {
  int ks1, ks2;
  q8_splits(M, m, n, r, ks1, ks2);
  size_t part = 0;
  if (ks1 > 1) part = (size_t)ks1 * M * r * 4;
  if (ks2 > 1 && (size_t)ks2 * M * m * 4 > part) part = (size_t)ks2 * M * m * 4;
  return align256((size_t)M * n) + align256((size_t)M * 4) + align256((size_t)M * r * 4) + align256((size_t)M * r) +
         align256((size_t)M * 4) + align256(part);
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
  int* part = reinterpret_cast<int*>(p);
  const uint32_t* v32 = reinterpret_cast<const uint32_t*>(v);
  const uint32_t* u32 = reinterpret_cast<const uint32_t*>(u);
  const Q8Plan p1 = q8_plan(M, r, n), p2 = q8_plan(M, m, r);
  launch_q8_rows<SRC_XDIN>(x, d_in, nullptr, 1, M, n, q1, e1, st);
  if (p1.ks == 1) {
    launch_tile_q8<OUT_HS>(p1, q1, e1, M, r, n, v32, d_mid, hs, 0, st);
    launch_q8_rows<SRC_F32>(hs, nullptr, nullptr, 1, M, r, q2, e2, st);
  } else {
    launch_tile_q8<OUT_PART>(p1, q1, e1, M, r, n, v32, d_mid, part, 0, st);
    launch_q8_rows<SRC_PART>(part, d_mid, e1, p1.ks, M, r, q2, e2, st);
  }
  if (p2.ks == 1) {
    launch_tile_q8<OUT_Y>(p2, q2, e2, M, m, r, u32, d_out, y, y_bf16, st);
  } else {
    launch_tile_q8<OUT_PART>(p2, q2, e2, M, m, r, u32, d_out, part, 0, st);
    const size_t quads = ((size_t)M * m + 3) / 4;
    hipLaunchKernelGGL(k_q8_out, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, part, p2.ks, M, m, e2, d_out,
                       y, y_bf16);
  }
  return hipGetLastError();
}

}  // namespace brq
