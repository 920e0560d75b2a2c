// Activation staging and the few-row (decode) group-128 product.
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} (+-x[m][k]): the activation x
// binary-weight product of "Banyan ..." (Abstract) on the group-128 format of
// "Behaviour-Relearned Quantization" (item 02), for M <= 64 activation rows.
#include "dec_core.h"
#include "kernels.h"

namespace brq {

// One thread per run of 32: load 32 bf16 values, write them in the permuted
// order slot 2b+h <- k = 16h+b, as fp16.
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
    const uint32_t a = f32_to_f16_bits(bf16_to_f32(lo16));
    const uint32_t c = f32_to_f16_bits(bf16_to_f32(hi16));
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
  hipLaunchKernelGGL(k_prep, dim3((unsigned)((runs + 255) / 256)), dim3(256), 0, st, x, runs, xp);
  return hipGetLastError();
}


// One-launch product for M <= 8: wave w owns chunks w*CPW .. w*CPW+CPW-1 of
// the reduction. It issues the loads of its activation slice (all MAXR row
// slots), of its sign words and of its scales before any wait, converts the
// slice into its own LDS region (no workgroup barrier: only this wave reads
// it) and runs its MFMAs as soon as its own data is in. SC16: the scales of
// the wave's 8 groups arrive as one 16-byte load per lane (needs CPW == 2 and
// G % 8 == 0); otherwise one 2-byte load per chunk. Only the lanes that hold
// rows m < M take part in the cross-wave sum (LDS, fixed wave order).
template <int CPW, int MAXR, bool SC16>
__global__ __launch_bounds__(1024) void k_gemm_dec_lds(const uint16_t* __restrict__ x, int M, int N, int K,
                                                       const uint4* __restrict__ signs,
                                                       const uint16_t* __restrict__ scales, void* __restrict__ y,
                                                       int y_bf16) {
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int n = blockIdx.x * 16 + j;
  const int G = K >> 7;
  const int nchunks = (G + 3) >> 2;
  const bool rok = n < N;
  const int nr = rok ? n : 0;  // clamped row; masked by bp.ok
  const uint4* wsig = signs + (size_t)nr * G;
  const uint16_t* wsc = scales + (size_t)nr * G;
  const int c0 = wave * CPW;
  uint4* xw = smem + (size_t)wave * CPW * MAXR * 64;
  f32x4* red = reinterpret_cast<f32x4*>(smem + (size_t)nw * CPW * MAXR * 64);
  f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
  if (c0 < nchunks) {  // uniform across the wave
    WaveStage<ST_BF16, CPW, MAXR> ws;
    ws.load(M, K, c0, [&](int m) { return x + (size_t)m * K; });
    BPre<1, CPW> bp;
    uint4 sq = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int g = 4 * (c0 + c) + kb;
      const bool ok = rok && g < G;
      const int gi = ok ? g : 0;
      bp.ok[0][c] = ok;
      bp.d[0][c] = wsig[gi];
      if (!SC16) bp.s[0][c] = wsc[gi];
    }
    if (SC16) sq = *reinterpret_cast<const uint4*>(wsc + 4 * c0);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    ws.store(xw);
    if (SC16) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        // halfword 4c + kb of the 8 scales
        const uint32_t wv = (kb & 2) ? ((c == 0) ? sq.y : sq.w) : ((c == 0) ? sq.x : sq.z);
        bp.s[0][c] = (kb & 1) ? (wv >> 16) : (wv & 0xffffu);
      }
    }
    const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
    auto aop = [&](int tt, int g, int i) -> u32x4 {
      const int m = min(j, M - 1);
      return xs[(((g >> 2) - c0) * MAXR + m) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_GROUP, 1, 1, CPW, true>(bp, nullptr, G, c0, 1, aop, acc);
  }
  // lane (kb, j) holds rows 4*kb .. 4*kb+3 of column j
  const bool holds = 4 * kb < M;
  if (wave > 0 && holds) red[(wave - 1) * 64 + lane] = acc[0][0];
  __syncthreads();
  if (wave != 0 || !holds || !rok) return;
#pragma unroll
  for (int w = 1; w < 16; ++w)
    if (w < nw) acc[0][0] += red[(w - 1) * 64 + lane];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * kb + i;
    if (m < M) store_out(y, (size_t)m * N + n, acc[0][0][i], y_bf16);
  }
}

// ---- M = 1 on the fp8 x fp4 matrix cores ----------------------------------
// A weight operand of +-1 needs only its sign, and fp4 (e2m1) has no infinity
// or NaN: OR-ing 0b0111 onto a nibble whose top bit is a sign bit gives +-6.0.
// So one shift-or turns a 32-bit sign word into 8 fp4 operands (dword t of a
// lane's 32-k block holds, in nibble q, the sign of k = 4q + t). The
// activation row is split per wave into two fp8 (e4m3) pieces, p0 = RNE(v)
// and p1 = RNE((v - p0)*16) with v = x*2^-a and 2^a chosen from the slice
// maximum so |v| < 256. A bf16 value has 8 significant bits and each piece
// carries 4, so the pieces add up to x exactly for every element within 2^13
// of the slice maximum; smaller ones are off by at most 2^-21 of the maximum.
// Rows 0/1 of v_mfma_scale_f32_16x16x128_f8f6f4 take them with block
// exponents a and a-4. One MFMA covers one scale group of 16 columns; the
// group scale and the 1/6 are applied in fp32 afterwards. (These matrix cores
// add every 8 products with about 13 significant bits relative to the largest
// of them, which bounds the accuracy more than a third piece would help.)
//
// Layout facts of that MFMA (fp8 A, fp4 B): A lane l supplies row l%16 with
// bytes 0..15 = k 16*(l/16).. and bytes 16..31 = k 64+16*(l/16)..; B lane l
// supplies column l%16 with nibble p = k 32*(l/16)+p; the A block exponent of
// (row r, k block b) comes from lane r + 16b; D as for the 16x16 f16 MFMA.
// A lane loads group 4c+kb of its column; four permlane swaps transpose the
// 4 x 4 (group, word) block of the four lanes of a column so that MFMA i gets
// word kb of group 4c+i.
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int F4_CHUNK = 4 * 2 * 128;  // LDS bytes of one chunk: 4 groups x 2 pieces x 128

// (group, word) transpose across the four 16-lane rows: on entry register w
// of row g holds word w of group g; on exit register i of row b holds word b
// of group i.
__device__ __forceinline__ void transpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = d[0];
  r3 = d[1];
}

template <int CPW, int NT>
__global__ __launch_bounds__(1024) void k_gemm_dec_f4(const uint16_t* __restrict__ x, int N, int K,
                                                      const uint4* __restrict__ signs,
                                                      const uint16_t* __restrict__ scales, void* __restrict__ y,
                                                      int y_bf16) {
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int G = K >> 7;
  const int nchunks = (G + 3) >> 2;
  const int c0 = wave * CPW;
  uint8_t* xw = reinterpret_cast<uint8_t*>(smem) + (size_t)wave * CPW * F4_CHUNK;  // [chunk][group][piece][128]
  float* red = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem) + (size_t)nw * CPW * F4_CHUNK);
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  if (c0 < nchunks) {  // uniform across the wave
    // ---- loads: activations (8 per lane per chunk), sign words, 4 scales per chunk
    uint4 xv[CPW];
    uint4 sg[NT][CPW];
    uint2 sc[NT][CPW];
    bool cok[NT];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int k0 = (c0 + c) * 512 + 8 * lane;
      xv[c] = *reinterpret_cast<const uint4*>(x + (k0 < K ? k0 : 0));
    }
    size_t row[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = (blockIdx.x * NT + t) * 16 + j;
      cok[t] = n < N;
      row[t] = (size_t)(n < N ? n : 0) * G;
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int g = 4 * (c0 + c) + kb, gs = 4 * (c0 + c);
        sg[t][c] = signs[row[t] + (g < G ? g : 0)];
        sc[t][c] = *reinterpret_cast<const uint2*>(scales + row[t] + (gs < G ? gs : 0));
      }
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    // ---- block exponents from the slice maximum
    uint32_t mx = 0;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint32_t w4[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) mx = max(mx, max(w4[h] & 0x7fffu, (w4[h] >> 16) & 0x7fffu));
    }
    mx = wave_max_u32(mx);
    int sh = (int)(mx >> 7) - 7;  // E8M0 exponent of piece 0: 2^(e_max - 7)
    sh = sh < 5 ? 5 : (sh > 253 ? 253 : sh);
    const float mh = __uint_as_float((uint32_t)(254 - sh) << 23);  // 2^(127 - sh)
    // ---- pieces in the operand order: lane L's 8 values are k = 8L .. 8L+7 of
    // the chunk (group L/16, word (L%16)/4); value e lands at in-word position
    // 8*(e%4) + 2*(L%4) + e/4
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint32_t w4[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h = (e & 1) ? (w4[e >> 1] & 0xffff0000u) : (w4[e >> 1] << 16);
        v[e] = __uint_as_float(h) * mh;
      }
      uint8_t* base = xw + c * F4_CHUNK + (lane >> 4) * 256 + 32 * ((lane & 15) >> 2) + 2 * (lane & 3);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int p0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[t], v[t + 4], 0, false);
        const float r0 = (v[t] - __builtin_amdgcn_cvt_f32_fp8(p0, 0)) * 16.f;
        const float r1 = (v[t + 4] - __builtin_amdgcn_cvt_f32_fp8(p0, 1)) * 16.f;
        const int p1 = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
        *reinterpret_cast<uint16_t*>(base + 8 * t) = (uint16_t)p0;
        *reinterpret_cast<uint16_t*>(base + 128 + 8 * t) = (uint16_t)p1;
      }
    }
    // A row j holds piece min(j, 1) (rows past 1 repeat piece 1 and are not
    // used) with block exponent sh - 4 * piece
    const int prow = j < 1 ? j : 1;
    const int sa = sh - 4 * prow;
    // ---- products
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint8_t* ab = xw + c * F4_CHUNK + prow * 128 + 16 * kb;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint32_t w0 = sg[t][c].x, w1 = sg[t][c].y, w2 = sg[t][c].z, w3 = sg[t][c].w;
        transpose4(w0, w1, w2, w3);
        const uint32_t wi[4] = {w0, w1, w2, w3};
        const uint32_t s4[4] = {sc[t][c].x & 0xffffu, sc[t][c].x >> 16, sc[t][c].y & 0xffffu, sc[t][c].y >> 16};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(ab + i * 256);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(ab + i * 256 + 64);
          i32x8 A, B;
          A[0] = a0[0]; A[1] = a0[1]; A[2] = a0[2]; A[3] = a0[3];
          A[4] = a1[0]; A[5] = a1[1]; A[6] = a1[2]; A[7] = a1[3];
          B[0] = (int)((wi[i] << 3) | 0x77777777u);
          B[1] = (int)((wi[i] << 2) | 0x77777777u);
          B[2] = (int)((wi[i] << 1) | 0x77777777u);
          B[3] = (int)(wi[i] | 0x77777777u);
          B[4] = 0; B[5] = 0; B[6] = 0; B[7] = 0;
          const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0,
                                                                           sa, 0, 127);
          const bool ok = cok[t] && (4 * (c0 + c) + i < G);
          const float s = ok ? f16_bits_to_f32(s4[i]) : 0.f;
          acc[t] = fmaf(s, d[0] + d[1], acc[t]);
        }
      }
    }
  }
  // lanes 0..15 hold the partial sums of columns j of the NT tiles
  if (wave > 0 && kb == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[((wave - 1) * NT + t) * 16 + j] = acc[t];
  }
  __syncthreads();
  if (wave != 0 || kb != 0) return;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float v = acc[t];
    for (int w = 1; w < nw; ++w) v += red[((w - 1) * NT + t) * 16 + j];
    const int n = (blockIdx.x * NT + t) * 16 + j;
    if (n < N) store_out(y, (size_t)n, v / 6.0f, y_bf16);
  }
}

// staged row slots for M activation rows
static int dec_maxr(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

// staging budget of the one-launch path: up to 128 KiB of LDS (beyond 64 KiB
// the kernel needs the per-function opt-in below)
constexpr int64_t kDecLdsBig = 128 * 1024;

// Split of the one-launch path: chunks of 512 over at most 16 waves, two
// chunks per wave when there are at least four (one chunk each below), more
// only when 16 waves of two do not cover K. The staged slices
// (waves * cpw * maxr KiB) must fit the LDS budget.
static bool dec_lds_split(int64_t M, int64_t K, DecSplit& sp) {
  if (M > 8) return false;
  const int64_t chunks = (K / 128 + 3) / 4;
  int64_t cpw = chunks >= 4 ? 2 : 1;
  if ((chunks + cpw - 1) / cpw > 16) cpw = (chunks + 15) / 16;
  if (cpw > 8) return false;
  sp.cpw = (int)cpw;
  sp.waves = (int)((chunks + cpw - 1) / cpw);
  return (int64_t)sp.waves * sp.cpw * dec_maxr(M) * 1024 <= kDecLdsBig;
}

bool gemm_dec_in_lds(int64_t M, int64_t K) {
  DecSplit sp;
  return dec_lds_split(M, K, sp);
}

template <int MAXR>
static void gemm_dec_lds(const uint16_t* x, int M, int N, int K, const uint4* s4, const uint16_t* scales, void* y,
                         int y_bf16, hipStream_t st) {
  DecSplit sp;
  dec_lds_split(M, K, sp);
  const size_t lds = (size_t)sp.waves * sp.cpw * MAXR * 1024 + (size_t)(sp.waves - 1) * 64 * 16;
  const dim3 grid((N + 15) / 16), block(64 * sp.waves);
  auto opt_in = [&](const void* fn) {
    if (lds > 64 * 1024) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  };
  if (sp.cpw == 2 && (K / 128) % 8 == 0) {
    opt_in(reinterpret_cast<const void*>(&k_gemm_dec_lds<2, MAXR, true>));
    hipLaunchKernelGGL((k_gemm_dec_lds<2, MAXR, true>), grid, block, lds, st, x, M, N, K, s4, scales, y, y_bf16);
  } else {
    BRQ_CPW_SWITCH(sp.cpw, opt_in(reinterpret_cast<const void*>(&k_gemm_dec_lds<CPW, MAXR, false>));
                   hipLaunchKernelGGL((k_gemm_dec_lds<CPW, MAXR, false>), grid, block, lds, st, x, M, N, K, s4,
                                      scales, y, y_bf16));
  }
}

// The fp8 x fp4 path takes M = 1 when the scale groups come in whole chunks
// of four (K % 512 == 0); it splits K like the one-launch fp16 path. Two
// column tiles per workgroup when that still leaves well over one workgroup
// per compute unit (the activation pieces are then shared by both tiles).
static void gemm_dec_f4(const uint16_t* x, int N, int K, const uint4* s4, const uint16_t* scales, void* y,
                        int y_bf16, hipStream_t st) {
  // one chunk per wave up to 16 waves (the less a wave computes after its
  // last sign word lands, the shorter the tail), two beyond
  const int chunks = K / 512;
  DecSplit sp;
  sp.cpw = chunks <= 16 ? 1 : (chunks + 15) / 16;
  sp.waves = (chunks + sp.cpw - 1) / sp.cpw;
  const int tiles = (N + 15) / 16;
  const int nt = tiles >= 768 ? 2 : 1;
  const size_t lds = (size_t)sp.waves * sp.cpw * F4_CHUNK + (size_t)(sp.waves - 1) * nt * 16 * 4;
  const dim3 grid((tiles + nt - 1) / nt), block(64 * sp.waves);
  if (nt == 2) {
    BRQ_CPW_SWITCH(sp.cpw, hipLaunchKernelGGL((k_gemm_dec_f4<CPW, 2>), grid, block, lds, st, x, N, K, s4, scales, y,
                                              y_bf16));
  } else {
    BRQ_CPW_SWITCH(sp.cpw, hipLaunchKernelGGL((k_gemm_dec_f4<CPW, 1>), grid, block, lds, st, x, N, K, s4, scales, y,
                                              y_bf16));
  }
}

hipError_t launch_gemm_dec(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                           void* y, int y_bf16, void* ws, hipStream_t st) {
  const uint4* s4 = reinterpret_cast<const uint4*>(signs);
  if (M == 1 && K % 512 == 0 && gemm_dec_in_lds(M, K)) {
    gemm_dec_f4(x, N, K, s4, scales, y, y_bf16, st);
    return hipGetLastError();
  }
  if (gemm_dec_in_lds(M, K)) {
    if (M == 1) gemm_dec_lds<1>(x, M, N, K, s4, scales, y, y_bf16, st);
    else if (M <= 2) gemm_dec_lds<2>(x, M, N, K, s4, scales, y, y_bf16, st);
    else if (M <= 4) gemm_dec_lds<4>(x, M, N, K, s4, scales, y, y_bf16, st);
    else gemm_dec_lds<8>(x, M, N, K, s4, scales, y, y_bf16, st);
    return hipGetLastError();
  }
  return launch_gemm_mid(x, M, N, K, signs, scales, y, y_bf16, ws, st);
}

}  // namespace brq
