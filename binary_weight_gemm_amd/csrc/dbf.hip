// Double Binary Factorization chain y = D_out U D_mid V D_in x
// ("LLM binarization, Episode 01: DBF": section 1, the representation with
// V in {-1,+1}^(r x n), U in {-1,+1}^(m x r) and three diagonals; section 4,
// the deployed order x_s = D_in x, h = V x_s, h_s = D_mid h, y_core = U h_s,
// y = D_out y_core).
//
// Stage 1 folds D_in into the weight operand: V[j][k] * d_in[k] is the exact
// fp16 value +-d_in[k], so the first product reads x unscaled. Its epilogue
// applies D_mid in fp32 and stores h_s as fp32 rows. Stage 2 multiplies U
// (+-1 operands) by h_s split into two fp16 pieces of h_s * 2^s (hi, lo: two
// activation rows per token), adds the pieces, undoes the power of two and
// applies D_out in fp32. The scale 2^s puts the largest |h_s| of the staged
// slice (decode: per wave; tiled: per row, set by k_dbf_split) near 2^14, so
// the pieces keep about 22 significant bits whatever the magnitude of D_mid.
#include "dec_core.h"
#include "f4.h"
#include "kernels.h"
#include "tile.h"

namespace brq {

// Decode path, stage 1: every wave stages its K-slice of x (bf16 -> permuted
// fp16) and of d_in (permuted) in LDS after issuing its loads; D_in rides on
// the weight operand (+-d_in[k]).
template <int TT, int CPW, int MAXR>
__global__ __launch_bounds__(1024) void k_dbf1_dec(const uint16_t* __restrict__ x, int M, int r, int n,
                                                   const uint4* __restrict__ v, const uint16_t* __restrict__ d_in,
                                                   const uint16_t* __restrict__ d_mid, float* __restrict__ hs) {
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int col = blockIdx.x * 16 + j;  // row of V = output column of stage 1
  const int G = n >> 7;
  const int nchunks = (G + 3) >> 2;
  const uint4* wsig[1] = {v + (size_t)(col < r ? col : 0) * G};
  const uint16_t* wsc[1] = {nullptr};
  const bool rok[1] = {col < r};
  const int c0 = wave * CPW;
  // LDS: x slices of all waves (MAXR row slots), then the d_in slices
  uint4* xw = smem + (size_t)wave * CPW * MAXR * 64;
  uint4* dw = smem + (size_t)(blockDim.x / 64) * CPW * MAXR * 64 + (size_t)wave * CPW * 64;
  BPre<1, CPW> bp;
  f32x4 acc[1][TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[0][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  WaveStage<ST_BF16, CPW, MAXR> sx;
  if (c0 < nchunks) {
    WaveStage<ST_F16, CPW, 1> sd;
    sx.load(M, n, c0, [&](int m) { return x + (size_t)m * n; });
    sd.load(1, n, c0, [&](int) { return d_in; });
    b_prefetch<BM_PERK, 1, CPW>(wsig, wsc, rok, G, c0, 1, bp);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    sx.store(xw);
    sd.store(dw);
  }
  __syncthreads();
  if (c0 < nchunks) {
    const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
    const u32x4* kp = reinterpret_cast<const u32x4*>(dw) - (size_t)c0 * 64;
    auto aop = [&](int tt, int g, int i) -> u32x4 {
      const int m = min(16 * tt + j, M - 1);
      return xs[(((g >> 2) - c0) * MAXR + m) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_PERK, 1, TT, CPW>(bp, kp, G, c0, 1, aop, acc);
    static_assert(TT == 1, "one tile of up to 8 rows");
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][0][i] = __builtin_amdgcn_ldexpf(acc[0][0][i], sx.unscale(i));
  }
  __syncthreads();
  reduce_waves<1, TT>(acc, reinterpret_cast<f32x4*>(smem));
  if (wave != 0 || col >= r) return;
  const float dm = f16_bits_to_f32(d_mid[col]);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * tt + 4 * (lane >> 4) + i;
      if (m < M) hs[(size_t)m * r + col] = acc[0][tt][i] * dm;
    }
}

// Decode path, stage 1 for one row with n % 512 == 0: x_s = D_in x in fp32
// (a bf16 times an fp16 value, exact), per wave slice as six fixed-point
// digit rows under the slice's largest power of two (the single-row scheme
// of the group-128 product on fp32 values: bits below 2^-23 of the slice
// maximum are dropped), V as +-6 fp4 operands on the fp8 x fp4 matrix cores,
// one 512-wide chunk per wave up to 16 waves; D_mid in the epilogue.
constexpr int DBF_F4_GROUP = 7 * 128;           // six digit rows of 128 codes and a zero row
constexpr int DBF_F4_CHUNK = 4 * DBF_F4_GROUP;  // four groups of 128

template <int CPW>
__global__ __launch_bounds__(1024) void k_dbf1_f4(const uint16_t* __restrict__ x, int r, int n,
                                                  const uint4* __restrict__ v, const uint16_t* __restrict__ d_in,
                                                  const uint16_t* __restrict__ d_mid, float* __restrict__ hs) {
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int G = n >> 7, nchunks = G >> 2;
  const int c0 = wave * CPW;
  const int col = blockIdx.x * 16 + j;  // row of V = output column of stage 1
  uint8_t* xw = reinterpret_cast<uint8_t*>(smem) + (size_t)wave * CPW * DBF_F4_CHUNK;
  float* red = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem) + (size_t)nw * CPW * DBF_F4_CHUNK);
  float acc = 0.f;
  if (c0 < nchunks) {  // uniform across the wave
    uint4 xv[CPW], dv[CPW], sg[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int k0 = (c0 + c) * 512 + 8 * lane;
      xv[c] = *reinterpret_cast<const uint4*>(x + (k0 < n ? k0 : 0));
      dv[c] = *reinterpret_cast<const uint4*>(d_in + (k0 < n ? k0 : 0));
    }
    const size_t row = (size_t)(col < r ? col : 0) * G;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int g = 4 * (c0 + c) + kb;
      sg[c] = v[row + (g < G ? g : 0)];
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    // x_s of the lane's 8 values per chunk; slots past the last chunk hold zeros
    f32x4 xs[CPW][2];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint32_t xw4[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
      const uint32_t dw4[4] = {dv[c].x, dv[c].y, dv[c].z, dv[c].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t xb = (i & 1) ? (xw4[i >> 1] >> 16) : (xw4[i >> 1] & 0xffffu);
        const uint32_t db = (i & 1) ? (dw4[i >> 1] >> 16) : (dw4[i >> 1] & 0xffffu);
        xs[c][i >> 2][i & 3] = c0 + c < nchunks ? bf16_to_f32(xb) * f16_bits_to_f32(db) : 0.f;
      }
    }
    float S;
    const uint32_t ebs = f4_slice_exponent_f32<CPW>(xs, S);
    uint8_t* base = xw + (lane >> 4) * DBF_F4_GROUP + 32 * ((lane & 15) >> 2) + 2 * (lane & 3);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if (lane < 32)  // the zero row of each group: 16 bytes per lane
        *reinterpret_cast<uint4*>(xw + c * DBF_F4_CHUNK + (lane >> 3) * DBF_F4_GROUP + 6 * 128 + 16 * (lane & 7)) =
            make_uint4(0u, 0u, 0u, 0u);
      f4_digits_f32(xs[c], S, base + c * DBF_F4_CHUNK, 0);
    }
    // MFMA rows 0..5 read the digit rows, 6..15 the zero row (block exponent 0)
    const int prow = j < 6 ? j : 6;
    const int sa = prow < 6 ? (int)ebs - 2 - 4 * prow : 127;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if (c0 + c >= nchunks) break;  // uniform across the wave
      const uint8_t* ab = xw + c * DBF_F4_CHUNK + prow * 128 + 16 * kb;
      uint32_t w0 = sg[c].x, w1 = sg[c].y, w2 = sg[c].z, w3 = sg[c].w;
      f4_transpose4(w0, w1, w2, w3);
      const uint32_t wi[4] = {w0, w1, w2, w3};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 d = f4_group_mfma(ab + i * DBF_F4_GROUP, wi[i], sa);
        acc += (d[0] + d[1]) + (d[2] + d[3]);
      }
    }
  }
  // digit rows 4 and 5 (lanes 16..31) join rows 0..3 (lanes 0..15); waves meet in LDS in wave order
  acc += __shfl_down(acc, 16, 64);
  if (wave > 0 && kb == 0) red[(wave - 1) * 16 + j] = acc;
  __syncthreads();
  if (wave != 0 || kb != 0 || col >= r) return;
  float s = acc;
  for (int w = 1; w < nw; ++w) s += red[(w - 1) * 16 + j];
  hs[col] = (s / 6.0f) * f16_bits_to_f32(d_mid[col]);
}

// launches k_dbf1_f4 where it applies (one row, n % 512 == 0, at most two
// chunks per wave over 16 waves); false otherwise
static bool dbf1_f4(const uint16_t* x, int r, int n, const uint4* v, const uint16_t* d_in, const uint16_t* d_mid,
                    float* hs, hipStream_t st) {
  if (n % 512 != 0) return false;
  const int chunks = n / 512;
  const int cpw = chunks <= 16 ? 1 : 2;
  if (chunks > 16 * cpw) return false;
  const int waves = (chunks + cpw - 1) / cpw;
  const size_t lds = (size_t)waves * cpw * DBF_F4_CHUNK + (size_t)(waves - 1) * 16 * 4;
  const dim3 grid((r + 15) / 16), block(64 * waves);
  if (cpw == 1) {
    hipLaunchKernelGGL((k_dbf1_f4<1>), grid, block, lds, st, x, r, n, v, d_in, d_mid, hs);
  } else {
    if (lds > 64 * 1024)
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_dbf1_f4<2>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((k_dbf1_f4<2>), grid, block, lds, st, x, r, n, v, d_in, d_mid, hs);
  }
  return true;
}

// Decode path, stage 2: every h_s row is staged in LDS as two scaled fp16
// pieces (two A rows per token, per-wave slices, WaveStageF32); U operands are
// +-1; each wave scales its partials back; D_out in the epilogue.
template <int TT, int CPW, int MAXR>
__global__ __launch_bounds__(1024) void k_dbf2_dec(const float* __restrict__ hs, int M, int m, int r,
                                                   const uint4* __restrict__ u, const uint16_t* __restrict__ d_out,
                                                   void* __restrict__ y, int y_bf16) {
  static_assert(TT == 1, "one tile of piece rows (up to 8 tokens)");
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int col = blockIdx.x * 16 + j;  // row of U = output column
  const int G = r >> 7;
  const int nchunks = (G + 3) >> 2;
  const int rows = 2 * M;
  const uint4* wsig[1] = {u + (size_t)(col < m ? col : 0) * G};
  const uint16_t* wsc[1] = {nullptr};
  const bool rok[1] = {col < m};
  const int c0 = wave * CPW;
  uint4* xw = smem + (size_t)wave * CPW * MAXR * 64;
  BPre<1, CPW> bp;
  f32x4 acc[1][TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[0][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  WaveStageF32<CPW, MAXR / 2> sh;
  if (c0 < nchunks) {
    sh.load(M, r, c0, [&](int t) { return hs + (size_t)t * r; });
    b_prefetch<BM_ONE, 1, CPW>(wsig, wsc, rok, G, c0, 1, bp);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    sh.store(xw);
  }
  __syncthreads();
  if (c0 < nchunks) {
    const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
    auto aop = [&](int tt, int g, int i) -> u32x4 {
      const int pr = min(16 * tt + j, rows - 1);  // piece row: token pr/2, piece pr%2
      return xs[(((g >> 2) - c0) * MAXR + pr) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_ONE, 1, TT, CPW>(bp, nullptr, G, c0, 1, aop, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][0][i] = __builtin_amdgcn_ldexpf(acc[0][0][i], sh.unscale(i));
  }
  __syncthreads();
  reduce_waves<1, TT>(acc, reinterpret_cast<f32x4*>(smem));
  if (wave != 0 || col >= m) return;
  const float dg = f16_bits_to_f32(d_out[col]);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 * tt + 2 * (lane >> 4) + h;
      if (t < M) store_out(y, (size_t)t * m + col, (acc[0][tt][2 * h] + acc[0][tt][2 * h + 1]) * dg, y_bf16);
    }
}

// Decode path in one launch (the joint kernel of section 7 of the DBF post):
// workgroup b computes stage 1 for rows 16b .. 16b+15 of V (if b < r/16)
// and, after a grid-wide wait for every workgroup's h_s, stage 2 for rows
// 16b .. 16b+15 of U (if b < m/16). Its U sign words are loaded before stage 1
// starts, so the second product issues no weight load after the wait. The
// stage bodies and their sums are those of k_dbf1_dec and k_dbf2_dec (the
// results are the same bits); h_s crosses the wait through the coherence
// point (gsync.h). The launch is sized so that every workgroup is resident.
template <int CPW1, int CPW2, int MAXR1, int MAXR2>
__global__ __launch_bounds__(1024) void k_dbf_fused(const uint16_t* __restrict__ x, int M, int m, int n, int r,
                                                    int waves1, int waves2, const uint4* __restrict__ v,
                                                    const uint16_t* __restrict__ d_in,
                                                    const uint16_t* __restrict__ d_mid, const uint4* __restrict__ u,
                                                    const uint16_t* __restrict__ d_out, float* __restrict__ hs,
                                                    void* __restrict__ y, int y_bf16, uint32_t* __restrict__ slot,
                                                    uint32_t spin) {
  extern __shared__ uint4 smem[];
  const uint32_t epoch = grid_epoch(slot);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int col = blockIdx.x * 16 + j;
  const bool do1 = (int)blockIdx.x * 16 < r, do2 = (int)blockIdx.x * 16 < m;  // uniform per workgroup
  const int G1 = n >> 7, nch1 = (G1 + 3) >> 2, c01 = wave * CPW1;
  const int G2 = r >> 7, nch2 = (G2 + 3) >> 2, c02 = wave * CPW2;
  // waves of each stage: those of the two-launch kernels (the rest idle)
  const bool act1 = do1 && wave < waves1 && c01 < nch1, act2 = do2 && wave < waves2 && c02 < nch2;
  uint4* xw = smem + (size_t)wave * CPW1 * MAXR1 * 64;
  uint4* dw = smem + (size_t)waves1 * CPW1 * MAXR1 * 64 + (size_t)wave * CPW1 * 64;
  BPre<1, CPW2> bp2;
  const uint16_t* nsc[1] = {nullptr};
  if (act2) {  // stage 2 weight words first: they do not depend on stage 1
    const uint4* wsig2[1] = {u + (size_t)(col < m ? col : 0) * G2};
    const bool rok2[1] = {col < m};
    b_prefetch<BM_ONE, 1, CPW2>(wsig2, nsc, rok2, G2, c02, 1, bp2);
  }
  f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
  WaveStage<ST_BF16, CPW1, MAXR1> sx;
  BPre<1, CPW1> bp1;
  if (act1) {
    const uint4* wsig[1] = {v + (size_t)(col < r ? col : 0) * G1};
    const bool rok[1] = {col < r};
    WaveStage<ST_F16, CPW1, 1> sd;
    sx.load(M, n, c01, [&](int q) { return x + (size_t)q * n; });
    sd.load(1, n, c01, [&](int) { return d_in; });
    b_prefetch<BM_PERK, 1, CPW1>(wsig, nsc, rok, G1, c01, 1, bp1);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    sx.store(xw);
    sd.store(dw);
  }
  __syncthreads();
  if (act1) {
    const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
    const u32x4* kp = reinterpret_cast<const u32x4*>(dw) - (size_t)c01 * 64;
    auto aop = [&](int, int g, int i) -> u32x4 {
      const int q = min(j, M - 1);
      return xs[(((g >> 2) - c01) * MAXR1 + q) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_PERK, 1, 1, CPW1>(bp1, kp, G1, c01, 1, aop, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][0][i] = __builtin_amdgcn_ldexpf(acc[0][0][i], sx.unscale(i));
  }
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(smem);
  if (do1) {  // the partials of stage 1's waves, added in wave order as reduce_waves does
    if (wave > 0 && wave < waves1) red[(wave - 1) * 64 + lane] = acc[0][0];
    __syncthreads();
    if (wave == 0) {
      for (int w = 1; w < waves1; ++w) acc[0][0] += red[(w - 1) * 64 + lane];
      if (col < r) {
        const float dm = f16_bits_to_f32(d_mid[col]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = 4 * (lane >> 4) + i;
          if (q < M) coh_storef(hs + (size_t)q * r + col, acc[0][0][i] * dm);
        }
      }
    }
  }
  // ---- every workgroup's h_s is at the coherence point after this
  const bool ok = grid_wait(slot, epoch, spin);
  if (!do2) return;  // uniform per workgroup
  if (!ok) {
    if (wave == 0 && lane < 16 && col < m)
      for (int t = 0; t < M; ++t) store_out(y, (size_t)t * m + col, __builtin_nanf(""), y_bf16);
    return;
  }
  // ---- stage 2: h_s as scaled fp16 piece rows, U operands +-1, D_out
  acc[0][0] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int rows = 2 * M;
  uint4* pw = smem + (size_t)wave * CPW2 * MAXR2 * 64;
  WaveStageF32<CPW2, MAXR2 / 2> sh;
  if (act2) {
    sh.template load<true>(M, r, c02, [&](int t) { return hs + (size_t)t * r; });
    sh.store(pw);
    const u32x4* xs = reinterpret_cast<const u32x4*>(pw);
    auto aop = [&](int, int g, int i) -> u32x4 {
      const int pr = min(j, rows - 1);  // piece row: token pr/2, piece pr%2
      return xs[(((g >> 2) - c02) * MAXR2 + pr) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_ONE, 1, 1, CPW2>(bp2, nullptr, G2, c02, 1, aop, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][0][i] = __builtin_amdgcn_ldexpf(acc[0][0][i], sh.unscale(i));
  }
  __syncthreads();
  if (wave > 0 && wave < waves2) red[(wave - 1) * 64 + lane] = acc[0][0];
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < waves2; ++w) acc[0][0] += red[(w - 1) * 64 + lane];
  if (col >= m) return;
  const float dg = f16_bits_to_f32(d_out[col]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 2 * (lane >> 4) + h;
    if (t < M) store_out(y, (size_t)t * m + col, (acc[0][0][2 * h] + acc[0][0][2 * h + 1]) * dg, y_bf16);
  }
}

// Decode path: per-wave staging of the x slice plus d_in (stage 1) and of the
// 2M h_s piece rows (stage 2) within the LDS budget, M <= 8.
static bool dbf_split(int64_t rows, int64_t K, DecSplit& sp) {
  const int64_t chunks = (K / 128 + 3) / 4;
  if (chunks > 64) return false;
  sp = dec_split((int)(K / 128), 4);
  if ((int64_t)sp.waves * sp.cpw < chunks) sp = dec_split((int)(K / 128), 8);
  if ((int64_t)sp.waves * sp.cpw < chunks) return false;
  return (int64_t)sp.waves * sp.cpw * rows * 1024 <= kDecLdsBytes;
}

static int dbf_maxr(int64_t M) { return M <= 1 ? 1 : M <= 4 ? 4 : 8; }

static bool dbf_decode_path(int64_t M, int64_t n, int64_t r) {
  DecSplit a, b;
  return M <= 8 && dbf_split(dbf_maxr(M) + 1, n, a) && dbf_split(2 * dbf_maxr(M), r, b);
}

// Single-launch chains: on when the caller asked for them (mode 2); by default
// (mode 0) off, two graph launches having measured faster on this chip (the
// grid-wide wait costs about what the kernel boundary does, and the first
// stage's workgroups are as slow either way).
static bool dbf_fusion_wanted(int M) {
  (void)M;
  return fusion_mode() == 2;
}

// Tiled path, between the stages: one workgroup per h_s row adds the row's
// S K-slice partials (slice order), finds the row's largest magnitude, writes
// the row as fp16 pieces of h_s * 2^s (rows 2t and 2t+1, permuted operand
// order) with the largest near 2^14, and records -s.
template <int QPT>
__global__ __launch_bounds__(256) void k_dbf_split(const float* __restrict__ hs, int M, int r, int S,
                                                   uint16_t* __restrict__ hp, int* __restrict__ rexp) {
  __shared__ uint32_t s_max[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* row = hs + (size_t)t * r;
  const size_t slice = (size_t)M * r;
  const int quads = r >> 3;  // 8 values (4 permuted pairs) per quad; quads <= 256 * QPT
  // thread tid holds quads tid + 256 i: values k .. k+3 and k+16 .. k+19 of
  // the row, the S (<= 8) partials added in slice order; every load is issued
  // before the sums (slices past S re-read slice 0 and are not added)
  f32x4 a[QPT], b[QPT];
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int q = tid + 256 * i;
    const int k = q < quads ? 32 * (q >> 2) + 4 * (q & 3) : 0;
    f32x4 pa[8], pb[8];
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      const size_t off = (sl < S ? sl : 0) * slice + k;
      pa[sl] = *reinterpret_cast<const f32x4*>(row + off);
      pb[sl] = *reinterpret_cast<const f32x4*>(row + off + 16);
    }
    a[i] = pa[0];
    b[i] = pb[0];
#pragma unroll
    for (int sl = 1; sl < 8; ++sl)
      if (sl < S) {
        a[i] += pa[sl];
        b[i] += pb[sl];
      }
  }
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < QPT; ++i)
    if (tid + 256 * i < quads) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        mx = max(mx, max(__float_as_uint(a[i][e]) & 0x7fffffffu, __float_as_uint(b[i][e]) & 0x7fffffffu));
    }
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) s_max[tid >> 6] = mx;
  __syncthreads();
  mx = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const int s = 14 - ((int)(mx >> 23) - 127);  // 0 -> s = 141, harmless: every value is 0
  if (tid == 0) rexp[t] = -s;
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int q = tid + 256 * i;
    if (q >= quads) continue;
    uint32_t oh[4], ol[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint16_t ha, la, hb, lb;
      split_f16(__builtin_amdgcn_ldexpf(a[i][e], s), ha, la);
      split_f16(__builtin_amdgcn_ldexpf(b[i][e], s), hb, lb);
      oh[e] = (uint32_t)ha | ((uint32_t)hb << 16);
      ol[e] = (uint32_t)la | ((uint32_t)lb << 16);
    }
    // pairs (k+e, k+16+e) are words 4(q&3)+e of run q>>2: 8 fp16 from 8*q
    *reinterpret_cast<uint4*>(hp + (size_t)(2 * t) * r + 8 * q) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
    *reinterpret_cast<uint4*>(hp + (size_t)(2 * t + 1) * r + 8 * q) = make_uint4(ol[0], ol[1], ol[2], ol[3]);
  }
}

// Rows too long to keep in registers (r > 16384): the same in two passes over
// the row, the partials added again in the second.
__global__ __launch_bounds__(256) void k_dbf_split_wide(const float* __restrict__ hs, int M, int r, int S,
                                                   uint16_t* __restrict__ hp, int* __restrict__ rexp) {
  __shared__ uint32_t s_max[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* row = hs + (size_t)t * r;
  const size_t slice = (size_t)M * r;
  const int quads = r >> 3;  // 8 values (4 permuted pairs) per quad
  // values k .. k+3 and k+16 .. k+19 of the row, partials added in slice order
  auto get = [&](int k, f32x4& a, f32x4& b) {
    a = *reinterpret_cast<const f32x4*>(row + k);
    b = *reinterpret_cast<const f32x4*>(row + k + 16);
    for (int sl = 1; sl < S; ++sl) {
      a += *reinterpret_cast<const f32x4*>(row + sl * slice + k);
      b += *reinterpret_cast<const f32x4*>(row + sl * slice + k + 16);
    }
  };
  uint32_t mx = 0;
  for (int q = tid; q < quads; q += 256) {
    const int k = 32 * (q >> 2) + 4 * (q & 3);
    f32x4 a, b;
    get(k, a, b);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mx = max(mx, max(__float_as_uint(a[i]) & 0x7fffffffu, __float_as_uint(b[i]) & 0x7fffffffu));
  }
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) s_max[tid >> 6] = mx;
  __syncthreads();
  mx = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const int s = 14 - ((int)(mx >> 23) - 127);  // 0 -> s = 141, harmless: every value is 0
  if (tid == 0) rexp[t] = -s;
  for (int q = tid; q < quads; q += 256) {
    const int k = 32 * (q >> 2) + 4 * (q & 3);
    f32x4 a, b;
    get(k, a, b);
    uint32_t oh[4], ol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t ha, la, hb, lb;
      split_f16(__builtin_amdgcn_ldexpf(a[i], s), ha, la);
      split_f16(__builtin_amdgcn_ldexpf(b[i], s), hb, lb);
      oh[i] = (uint32_t)ha | ((uint32_t)hb << 16);
      ol[i] = (uint32_t)la | ((uint32_t)lb << 16);
    }
    // pairs (k+i, k+16+i) are words 4(q&3)+i of run q>>2: 8 fp16 from 8*q
    *reinterpret_cast<uint4*>(hp + (size_t)(2 * t) * r + 8 * q) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
    *reinterpret_cast<uint4*>(hp + (size_t)(2 * t + 1) * r + 8 * q) = make_uint4(ol[0], ol[1], ol[2], ol[3]);
  }
}

// workspace: h_s fp32 [M][r]; the tiled path holds one such partial per
// K-slice of stage 1, then the pieces [2M][r] and their exponents [M], then
// the staged rows of x [M][n] fp16 and their staging exponents [M]
size_t dbf_ws_bytes(int64_t M, int64_t m, int64_t n, int64_t r) {
  (void)m;
  if (dbf_decode_path(M, n, r)) return align256((size_t)M * r * 4);
  const size_t hs = align256((size_t)dbf1_ksplit((int)M, (int)r, (int)n) * M * r * 4);
  return hs + align256((size_t)2 * M * r * 2) + align256((size_t)M * 4) + align256((size_t)M * n * 2) +
         align256((size_t)M * 4);
}

// Single-launch decode chain: taken when the caller asked for it (or the
// library's default does) and every workgroup (one per 16 rows of the longer
// of V and U) fits the device at once. Returns false when not taken.
template <int MAXR1, int MAXR2>
static bool dbf_fused(const uint16_t* x, int M, int m, int n, int r, const uint16_t* d_in, const uint64_t* v,
                      const uint16_t* d_mid, const uint64_t* u, const uint16_t* d_out, void* y, int y_bf16,
                      float* hs, hipStream_t st, hipError_t& err) {
  if (!dbf_fusion_wanted(M)) return false;
  DecSplit s1, s2;
  dbf_split(MAXR1 + 1, n, s1);
  dbf_split(MAXR2, r, s2);
  const int waves = s1.waves > s2.waves ? s1.waves : s2.waves;
  const int64_t blocks = ((int64_t)(r > m ? r : m) + 15) / 16;
  size_t lds = (size_t)s1.waves * s1.cpw * (MAXR1 + 1) * 1024;
  const size_t l2 = (size_t)s2.waves * s2.cpw * MAXR2 * 1024, rd = (size_t)(waves - 1) * 64 * 16;
  lds = lds > l2 ? lds : l2;
  lds = lds > rd ? lds : rd;
  const void* fn = nullptr;
#define BRQ_FUSED_FN(C1, C2) reinterpret_cast<const void*>(&k_dbf_fused<C1, C2, MAXR1, MAXR2>)
  if (s1.cpw == 1 && s2.cpw == 1) fn = BRQ_FUSED_FN(1, 1);
  else if (s1.cpw == 2 && s2.cpw == 1) fn = BRQ_FUSED_FN(2, 1);
  else if (s1.cpw == 1 && s2.cpw == 2) fn = BRQ_FUSED_FN(1, 2);
  else if (s1.cpw == 2 && s2.cpw == 2) fn = BRQ_FUSED_FN(2, 2);
#undef BRQ_FUSED_FN
  if (!fn || !grid_fits(fn, 64 * waves, lds, blocks)) return false;
  uint32_t* slot = nullptr;
  err = grid_slot(&slot);
  if (err != hipSuccess) return true;
  const uint4* v4 = reinterpret_cast<const uint4*>(v);
  const uint4* u4 = reinterpret_cast<const uint4*>(u);
  const uint32_t spin = grid_spin_limit();
#define BRQ_FUSED(C1, C2)                                                                                    \
  hipLaunchKernelGGL((k_dbf_fused<C1, C2, MAXR1, MAXR2>), dim3((unsigned)blocks), dim3(64 * waves), lds, st, x, M, \
                     m, n, r, s1.waves, s2.waves, v4, d_in, d_mid, u4, d_out, hs, y, y_bf16, slot, spin)
  if (s1.cpw == 1 && s2.cpw == 1) BRQ_FUSED(1, 1);
  else if (s1.cpw == 2 && s2.cpw == 1) BRQ_FUSED(2, 1);
  else if (s1.cpw == 1 && s2.cpw == 2) BRQ_FUSED(1, 2);
  else BRQ_FUSED(2, 2);
#undef BRQ_FUSED
  err = hipGetLastError();
  return true;
}

template <int MAXR1, int MAXR2>
static hipError_t dbf_decode(const uint16_t* x, int M, int m, int n, int r, const uint16_t* d_in, const uint64_t* v,
                             const uint16_t* d_mid, const uint64_t* u, const uint16_t* d_out, void* y, int y_bf16,
                             float* hs, hipStream_t st) {
  hipError_t fe = hipSuccess;
  if (dbf_fused<MAXR1, MAXR2>(x, M, m, n, r, d_in, v, d_mid, u, d_out, y, y_bf16, hs, st, fe)) return fe;
  DecSplit s1, s2;
  dbf_split(MAXR1 + 1, n, s1);
  dbf_split(MAXR2, r, s2);
  const size_t l1 = (size_t)s1.waves * s1.cpw * (MAXR1 + 1) * 1024, r1 = (size_t)(s1.waves - 1) * 64 * 16;
  const size_t l2 = (size_t)s2.waves * s2.cpw * MAXR2 * 1024, r2 = (size_t)(s2.waves - 1) * 64 * 16;
  const uint4* v4 = reinterpret_cast<const uint4*>(v);
  const uint4* u4 = reinterpret_cast<const uint4*>(u);
  if (!(MAXR1 == 1 && dbf1_f4(x, r, n, v4, d_in, d_mid, hs, st)))
    BRQ_CPW_SWITCH(s1.cpw, hipLaunchKernelGGL((k_dbf1_dec<1, CPW, MAXR1>), dim3((r + 15) / 16), dim3(64 * s1.waves),
                                              l1 > r1 ? l1 : r1, st, x, M, r, n, v4, d_in, d_mid, hs));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  BRQ_CPW_SWITCH(s2.cpw, hipLaunchKernelGGL((k_dbf2_dec<1, CPW, MAXR2>), dim3((m + 15) / 16), dim3(64 * s2.waves),
                                            l2 > r2 ? l2 : r2, st, hs, M, m, r, u4, d_out, y, y_bf16));
  return hipGetLastError();
}

hipError_t launch_dbf(const uint16_t* x, int M, int m, int n, int r, const uint16_t* d_in,
                      const uint64_t* v, const uint16_t* d_mid, const uint64_t* u,
                      const uint16_t* d_out, void* y, int y_bf16, void* ws, hipStream_t st) {
  char* base = reinterpret_cast<char*>(ws);
  float* hs = reinterpret_cast<float*>(base);
  if (dbf_decode_path(M, n, r)) {
    if (M == 1) return dbf_decode<1, 2>(x, M, m, n, r, d_in, v, d_mid, u, d_out, y, y_bf16, hs, st);
    if (M <= 4) return dbf_decode<4, 8>(x, M, m, n, r, d_in, v, d_mid, u, d_out, y, y_bf16, hs, st);
    return dbf_decode<8, 16>(x, M, m, n, r, d_in, v, d_mid, u, d_out, y, y_bf16, hs, st);
  }
  const int ks = dbf1_ksplit(M, r, n);
  base += align256((size_t)ks * M * r * 4);
  uint16_t* hp = reinterpret_cast<uint16_t*>(base);
  base += align256((size_t)2 * M * r * 2);
  int* rexp = reinterpret_cast<int*>(base);
  base += align256((size_t)M * 4);
  uint16_t* xp = reinterpret_cast<uint16_t*>(base);
  base += align256((size_t)M * n * 2);
  int* xexp = reinterpret_cast<int*>(base);
  // x staged as fp16 with a power of two per row (undone in stage 1's epilogue)
  hipError_t e = launch_prep_rows(x, M, n, xp, xexp, 1, st);
  if (e != hipSuccess) return e;
  TileArgs a1{};
  a1.a = xp; a1.M = M; a1.N = r; a1.K = n; a1.signs = v; a1.kmag = d_in; a1.diag = d_mid; a1.rexp = xexp;
  a1.out = hs; a1.ksplit = ks;
  e = launch_tile_dbf1(a1, st);
  if (e != hipSuccess) return e;
  const int qpt = (r / 8 + 255) / 256;  // quads of 8 values per thread
  if (qpt <= 1)
    hipLaunchKernelGGL(k_dbf_split<1>, dim3(M), dim3(256), 0, st, hs, M, r, ks, hp, rexp);
  else if (qpt <= 2)
    hipLaunchKernelGGL(k_dbf_split<2>, dim3(M), dim3(256), 0, st, hs, M, r, ks, hp, rexp);
  else if (qpt <= 4)
    hipLaunchKernelGGL(k_dbf_split<4>, dim3(M), dim3(256), 0, st, hs, M, r, ks, hp, rexp);
  else if (qpt <= 8)
    hipLaunchKernelGGL(k_dbf_split<8>, dim3(M), dim3(256), 0, st, hs, M, r, ks, hp, rexp);
  else
    hipLaunchKernelGGL(k_dbf_split_wide, dim3(M), dim3(256), 0, st, hs, M, r, ks, hp, rexp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  TileArgs a2{};
  a2.a = hp; a2.M = 2 * M; a2.N = m; a2.K = r; a2.signs = u; a2.diag = d_out; a2.rexp = rexp;
  a2.out = y; a2.out_bf16 = y_bf16;
  return launch_tile_dbf2(a2, st);
}

}  // namespace brq
