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

// ALDS: every wave stages its own K-slice of x (bf16 -> permuted fp16) in LDS
// after issuing its loads (one launch, no workspace); MAXR is the row bound
// of that path. Otherwise `xa` is the permuted fp16 staging written by k_prep
// and A operands are read from global memory.
template <int TT, int CPW, bool ALDS, int MAXR>
__global__ __launch_bounds__(1024) void k_gemm_dec(const uint16_t* __restrict__ xa, int M, int N, int K,
                                                   const uint4* __restrict__ signs,
                                                   const uint16_t* __restrict__ scales, void* __restrict__ y,
                                                   int y_bf16) {
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15;
  const int n = blockIdx.x * 16 + j;
  const int G = K >> 7;
  const int nchunks = (G + 3) >> 2;
  const int nr = n < N ? n : 0;  // clamped row; masked by rok
  const uint4* wsig[1] = {signs + (size_t)nr * G};
  const uint16_t* wsc[1] = {scales + (size_t)nr * G};
  const bool rok[1] = {n < N};
  f32x4 acc[1][TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[0][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  BPre<1, CPW> bp;
  if (ALDS) {
    // one round: wave w owns chunks w*CPW .. w*CPW+CPW-1
    const int c0 = wave * CPW;
    uint4* xw = smem + (size_t)wave * CPW * MAXR * 64;
    if (c0 < nchunks) {
      WaveStage<ST_BF16, CPW, MAXR> ws;
      ws.load(M, K, c0, [&](int m) { return xa + (size_t)m * K; });
      b_prefetch<BM_GROUP, 1, CPW>(wsig, wsc, rok, G, c0, 1, bp);
      __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
      ws.store(xw);
    }
    __syncthreads();
    if (c0 < nchunks) {
      const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
      auto aop = [&](int tt, int g, int i) -> u32x4 {
        const int m = min(16 * tt + j, M - 1);
        return xs[(((g >> 2) - c0) * MAXR + m) * 64 + (g & 3) * 16 + i];
      };
      b_compute<BM_GROUP, 1, TT, CPW>(bp, nullptr, G, c0, 1, aop, acc);
    }
    __syncthreads();  // the reduction below reuses the staging area
  } else {
    for (int base = 0; base < nchunks; base += nw * CPW) {
      const int c0 = base + wave * CPW;
      b_prefetch<BM_GROUP, 1, CPW>(wsig, wsc, rok, G, c0, 1, bp);
      auto aop = [&](int tt, int g, int i) -> u32x4 {
        const int m = min(16 * tt + j, M - 1);
        return reinterpret_cast<const u32x4*>(xa + (size_t)m * K)[g * 16 + i];
      };
      b_compute<BM_GROUP, 1, TT, CPW>(bp, nullptr, G, c0, 1, aop, acc);
    }
  }
  reduce_waves<1, TT>(acc, reinterpret_cast<f32x4*>(smem));
  if (wave != 0 || n >= N) return;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * tt + 4 * (lane >> 4) + i;
      if (m < M) store_out(y, (size_t)m * N + n, acc[0][tt][i], y_bf16);
    }
}

// staged row slots for M activation rows
static int dec_maxr(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

// LDS path: one round of at most 8 waves x 8 chunks covers K, and the
// per-wave slices of all row slots (waves * cpw * maxr KiB) fit the staging
// budget.
static bool dec_lds_split(int64_t M, int64_t K, DecSplit& sp) {
  const int64_t chunks = (K / 128 + 3) / 4;
  if (M > 8 || chunks > 64) return false;
  sp = dec_split((int)(K / 128), 4);
  if ((int64_t)sp.waves * sp.cpw < chunks) sp = dec_split((int)(K / 128), 8);
  if ((int64_t)sp.waves * sp.cpw < chunks) return false;
  return (int64_t)sp.waves * sp.cpw * dec_maxr(M) * 1024 <= kDecLdsBytes;
}

bool gemm_dec_in_lds(int64_t M, int64_t K) {
  DecSplit sp;
  return dec_lds_split(M, K, sp);
}

template <int TT, bool ALDS, int MAXR>
static void gemm_dec_tt(const uint16_t* xa, int M, int N, int K, const uint4* s4, const uint16_t* scales, void* y,
                        int y_bf16, hipStream_t st) {
  DecSplit sp2 = dec_split(K / 128, 16);
  if (ALDS) dec_lds_split(M, K, sp2);
  size_t lds = (size_t)(sp2.waves - 1) * TT * 64 * 16;
  const size_t stage = (size_t)sp2.waves * sp2.cpw * MAXR * 1024;
  if (ALDS && stage > lds) lds = stage;
  const dim3 grid((N + 15) / 16), block(64 * sp2.waves);
  BRQ_CPW_SWITCH(sp2.cpw, hipLaunchKernelGGL((k_gemm_dec<TT, CPW, ALDS, MAXR>), grid, block, lds, st, xa, M, N, K,
                                             s4, scales, y, y_bf16));
}

hipError_t launch_gemm_dec(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                           void* y, int y_bf16, void* ws, hipStream_t st) {
  const uint4* s4 = reinterpret_cast<const uint4*>(signs);
  const int TT = (M + 15) / 16;
  if (gemm_dec_in_lds(M, K)) {
    if (M == 1) gemm_dec_tt<1, true, 1>(x, M, N, K, s4, scales, y, y_bf16, st);
    else if (M <= 2) gemm_dec_tt<1, true, 2>(x, M, N, K, s4, scales, y, y_bf16, st);
    else if (M <= 4) gemm_dec_tt<1, true, 4>(x, M, N, K, s4, scales, y, y_bf16, st);
    else gemm_dec_tt<1, true, 8>(x, M, N, K, s4, scales, y, y_bf16, st);
    return hipGetLastError();
  }
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws);
  hipError_t e = launch_prep_bf16(x, M, K, xp, st);
  if (e != hipSuccess) return e;
  switch (TT) {
    case 1: gemm_dec_tt<1, false, 1>(xp, M, N, K, s4, scales, y, y_bf16, st); break;
    case 2: gemm_dec_tt<2, false, 1>(xp, M, N, K, s4, scales, y, y_bf16, st); break;
    case 3: gemm_dec_tt<3, false, 1>(xp, M, N, K, s4, scales, y, y_bf16, st); break;
    default: gemm_dec_tt<4, false, 1>(xp, M, N, K, s4, scales, y, y_bf16, st); break;
  }
  return hipGetLastError();
}

}  // namespace brq
