// Product for 8 < M <= 64 activation rows (the decode-batch regime between one
// vector and the prefill tiles, "LLM binarization, Episode 01: DBF", section 4:
// each matrix is now applied to a handful of vectors).
//
// A staging launch writes x as fp16 in the permuted operand order. The product splits the work into
// 128-column tiles x K-slices: a workgroup (4 waves, 32 columns each) streams
// its slice in k-steps of 128 (one scale group) through a ring of LDS stages
// filled by direct loads -- all M rows of x (16*TT rows), the 16-byte sign
// records and the scales of its 128 columns -- so the loads of a k-step are in
// flight STAGES-1 k-steps ahead. Every wave multiplies all rows (TT tiles of
// 16) by its two 16-column groups with v_mfma_f32_16x16x32_f16 on +-scale
// fp16 weight operands: one activation operand serves two MFMAs and one weight
// operand serves TT.
//
// With several K-slices each workgroup writes its fp32 partial tile to the
// workspace and a third launch adds the slices in slice order (deterministic).
// (Meeting inside the product launch instead -- last-arriving workgroup adds
// the tile -- needs a device-scope release per workgroup, which writes back
// the whole L2 of its chiplet and cost far more than the extra launch.)
#include "common.h"
#include "kernels.h"

namespace brq {

namespace {

constexpr int MID_NB = 2;              // 16-column groups per wave
constexpr int MID_BN = 64 * MID_NB;    // columns per workgroup
constexpr int MID_SIG = MID_BN * 16;   // sign bytes per stage
constexpr int MID_SC = 4 * 256;        // scale dwords per stage: 64 lanes x 4 B per wave

// ring depth: more stages in flight where a stage is small
__host__ __device__ constexpr int mid_stages(int tt) { return tt == 1 ? 8 : tt == 2 ? 6 : 4; }
__host__ __device__ constexpr int mid_stage_bytes(int tt) { return 16 * tt * 256 + MID_SIG + MID_SC; }

struct MidPlan {
  int tiles, slices, kps;  // column tiles, K-slices, k-steps per slice
};

// About two workgroups per compute unit for the rows that stream weights
// (TT <= 2), one for the rows that are matrix-core bound (fewer partial tiles).
MidPlan mid_plan(int64_t M, int64_t N, int64_t K) {
  MidPlan p;
  const int nk = (int)(K / 128);
  const int target = M <= 32 ? 512 : 256;
  p.tiles = (int)((N + MID_BN - 1) / MID_BN);
  int s = (target + p.tiles - 1) / p.tiles;
  if (s > nk) s = nk;
  if (s < 1) s = 1;
  p.kps = (nk + s - 1) / s;
  p.slices = (nk + p.kps - 1) / p.kps;  // no empty slice
  return p;
}

}  // namespace

template <int TT>
__global__ __launch_bounds__(256) void k_mid(const uint16_t* __restrict__ xp, int M, int N, int K,
                                             const uint32_t* __restrict__ signs, const uint16_t* __restrict__ scales,
                                             void* __restrict__ y, int y_bf16, float* __restrict__ part, int kps,
                                             int S) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int ROWS = 16 * TT, SB = mid_stage_bytes(TT), STAGES = mid_stages(TT);
  constexpr int NB = MID_NB, BN = MID_BN;
  constexpr int OPS = TT + NB + 1;  // direct loads per wave per k-step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int tile = blockIdx.x, sl = blockIdx.y;
  const int nk = K >> 7;
  const int kt0 = sl * kps, kt1 = kt0 + kps < nk ? kt0 + kps : nk, nks = kt1 - kt0;
  const int n0 = tile * BN;
  const int cw = n0 + 16 * NB * wave;  // first column of this wave
  const int KW = K >> 5;               // 32-bit sign words per weight row

  // ---- direct loads of one k-step into a stage
  // activations: wave w loads rows 4*TT*w + 4i + L/16 (i < TT), 16-byte chunk
  // L%16 of the k-step to LDS slot (L%16) ^ (row%16); rows past M repeat M-1
  // (their products are never stored).
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(xp);
  const uint8_t* ap[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const int r = 4 * TT * wave + 4 * i + (lane >> 4);
    const int rg = r < M ? r : M - 1;
    const int chunk = (lane & 15) ^ (r & 15);
    ap[i] = xb + (size_t)rg * K * 2 + chunk * 16;
  }
  // signs of group g: lane L loads word L%4 of column cw + 16g + L/4; columns
  // past N repeat N-1 (never stored)
  const uint32_t* sig[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    const int c = cw + 16 * g + (lane >> 2);
    sig[g] = signs + (size_t)(c < N ? c : N - 1) * KW + (lane & 3);
  }
  // scales: lane L loads the aligned dword holding the scale of column
  // cw + L % (16*NB) (lanes past 16*NB repeat); the reader picks the half
  const int scc = cw + (lane & (16 * NB - 1));
  const size_t sc_idx = (size_t)(scc < N ? scc : N - 1) * nk;
  const uint32_t* scw = reinterpret_cast<const uint32_t*>(scales);
  auto issue = [&](int kt, int st) {
    uint8_t* base = lds + st * SB;
#pragma unroll
    for (int i = 0; i < TT; ++i)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(ap[i] + (size_t)kt * 256),
                                       base + (4 * TT * wave + 4 * i) * 256, 16, 0, 0);
#pragma unroll
    for (int g = 0; g < NB; ++g)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(sig[g] + 4 * kt),
                                       base + ROWS * 256 + (NB * wave + g) * 256, 4, 0, 0);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(scw + ((sc_idx + kt) >> 1)),
                                     base + ROWS * 256 + MID_SIG + wave * 256, 4, 0, 0);
  };

  f32x4 acc[TT][NB];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int g = 0; g < NB; ++g) acc[t][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int bsh = 4 * kb;  // the lane's k block takes pairs 4*kb .. 4*kb+3 of each half-run
  // the reader's scale halves: column cw + 16g + j at step kt sits in the high
  // half when its element index is odd
  int sc_odd[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    const int c = cw + 16 * g + j;
    sc_odd[g] = (int)(((size_t)(c < N ? c : N - 1) * nk) & 1);
  }

  // prologue: the first STAGES-1 k-steps in flight (steps past the slice
  // repeat its last step and are never used)
#pragma unroll
  for (int q = 0; q < STAGES - 1; ++q) issue(kt0 + (q < nks ? q : nks - 1), q);

  for (int q = 0; q < nks; ++q) {
    const int st = q % STAGES;
    // this wave's loads of step q landed (the STAGES-2 younger steps may still
    // be in flight), then every wave's loads landed and every wave is done
    // with the stage the next issue overwrites. A plain s_barrier: the
    // workgroup fence of __syncthreads would make the compiler drain every
    // direct load in flight, the prefetches included.
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((STAGES - 2) * OPS) : "memory");
    {
      const int qn = q + STAGES - 1;
      issue(kt0 + (qn < nks ? qn : nks - 1), qn % STAGES);
    }
    const uint8_t* base = lds + st * SB;
    u32x4 w4[NB];
    uint32_t S[NB];
    const int kodd = (kt0 + q) & 1;
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      w4[g] = *reinterpret_cast<const u32x4*>(base + ROWS * 256 + (NB * wave + g) * 256 + j * 16);
      const uint32_t d = *reinterpret_cast<const uint32_t*>(base + ROWS * 256 + MID_SIG + wave * 256 + (16 * g + j) * 4);
      // element sc_idx + kt sits in the high half iff its index is odd
      const uint32_t h = (sc_odd[g] ^ kodd) ? (d >> 16) : (d & 0xffffu);
      S[g] = h | (h << 16);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int slot = ((4 * s + kb) ^ j) * 16;  // chunk 4s+kb of row 16t+j
      u32x4 a[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) a[t] = *reinterpret_cast<const u32x4*>(base + (16 * t + j) * 256 + slot);
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        const uint32_t w = w4[g][s] >> bsh;
        u32x4 b;
#pragma unroll
        for (int u = 0; u < 4; ++u) b[u] = ((w << (15 - u)) & 0x80008000u) | S[g];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t][g] = mfma16(a[t], b, acc[t][g]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // nothing in flight when the workgroup ends

  // lane (kb, j) holds rows 16t + 4kb + i of column cw + 16g + j
  if (S == 1) {
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      const int col = cw + 16 * g + j;
      if (col < N) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * kb + i;
            if (m < M) store_out(y, (size_t)m * N + col, acc[t][g][i], y_bf16);
          }
      }
    }
    return;
  }
  // this slice's partial tile [M][BN] at part[(tile*S + sl)*M*BN ...]; a
  // second launch adds the slices
  float* mine = part + ((size_t)tile * S + sl) * M * BN;
#pragma unroll
  for (int g = 0; g < NB; ++g)
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * t + 4 * kb + i;
        if (m < M) mine[m * BN + 16 * (NB * wave + g) + j] = acc[t][g][i];
      }
}

// y = the sum of the S partial tiles, in slice order (deterministic); one
// thread per four columns of a tile row.
__global__ __launch_bounds__(256) void k_mid_sum(const float* __restrict__ part, int M, int N, int tiles, int S,
                                                 void* __restrict__ y, int y_bf16) {
  const int n4 = M * MID_BN / 4;  // float4s per partial tile
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)tiles * n4) return;
  const int tile = (int)(e / n4), r = (int)(e - (int64_t)tile * n4);
  const f32x4* all = reinterpret_cast<const f32x4*>(part) + (size_t)tile * S * n4 + r;
  f32x4 v = all[0];
  int s2 = 1;
  for (; s2 + 4 <= S; s2 += 4) {
    const f32x4 p0 = all[(size_t)s2 * n4], p1 = all[(size_t)(s2 + 1) * n4];
    const f32x4 p2 = all[(size_t)(s2 + 2) * n4], p3 = all[(size_t)(s2 + 3) * n4];
    v += p0;
    v += p1;
    v += p2;
    v += p3;
  }
  for (; s2 < S; ++s2) v += all[(size_t)s2 * n4];
  const int m = (4 * r) / MID_BN, c = tile * MID_BN + 4 * r - m * MID_BN;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (c + i < N) store_out(y, (size_t)m * N + c + i, v[i], y_bf16);
}

size_t mid_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const MidPlan p = mid_plan(M, N, K);
  size_t b = align256((size_t)M * K * 2);
  if (p.slices > 1) b += align256((size_t)p.tiles * p.slices * M * MID_BN * 4);
  return b;
}

template <int TT>
static hipError_t mid_launch(const uint16_t* xp, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                             void* y, int y_bf16, float* part, const MidPlan& p, hipStream_t st) {
  const int lds = mid_stages(TT) * mid_stage_bytes(TT);
  if (lds > 64 * 1024) {  // per-function opt-in beyond 64 KiB of dynamic LDS
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mid<TT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_mid<TT>, dim3(p.tiles, p.slices), dim3(256), lds, st, xp, M, N, K,
                     reinterpret_cast<const uint32_t*>(signs), scales, y, y_bf16, part, p.kps, p.slices);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.slices == 1) return e;
  const int64_t n = (int64_t)p.tiles * M * MID_BN / 4;
  hipLaunchKernelGGL(k_mid_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, M, N, p.tiles, p.slices, y,
                     y_bf16);
  return hipGetLastError();
}

hipError_t launch_gemm_mid(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                           void* y, int y_bf16, void* ws, hipStream_t st) {
  const MidPlan p = mid_plan(M, N, K);
  char* base = reinterpret_cast<char*>(ws);
  uint16_t* xp = reinterpret_cast<uint16_t*>(base);
  float* part = reinterpret_cast<float*>(base + align256((size_t)M * K * 2));
  const hipError_t e = launch_prep_bf16(x, M, K, xp, st);
  if (e != hipSuccess) return e;
  switch ((M + 15) / 16) {
    case 1: return mid_launch<1>(xp, M, N, K, signs, scales, y, y_bf16, part, p, st);
    case 2: return mid_launch<2>(xp, M, N, K, signs, scales, y, y_bf16, part, p, st);
    case 3: return mid_launch<3>(xp, M, N, K, signs, scales, y, y_bf16, part, p, st);
    default: return mid_launch<4>(xp, M, N, K, signs, scales, y, y_bf16, part, p, st);
  }
}

}  // namespace brq
