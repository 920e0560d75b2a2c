// Prefill product y = x . Wq^T for many activation rows (M > 64) on the fp16
// matrix cores ("LLM binarization, Episode 01: DBF", section 4: one matrix
// applied to many vectors amortises the weight unpack over the rows).
//
// x is first written by k_prep as fp16 in the permuted operand order (the
// pair order of the shift-and-or weight unpack, see common.h), so the main
// kernel moves activation tiles global -> LDS with direct loads
// (global_load_lds_dwordx4), never through registers.
//
// Block tile 256 x 256 x 64, four waves in 2 x 2, each wave 128 x 128 of
// v_mfma_f32_32x32x16_f16 tiles (16 accumulators of 16 fp32). LDS per stage:
// A 256 rows x 128 B, B 256 columns x 128 B, two stages (128 KiB). Rows of
// both tiles hold eight 16-byte chunks stored at slot (chunk ^ ((row/2)%8)),
// so the 32-row fragment reads of a wave spread over all banks.
// Per k-step of 64: the direct loads of step k+1 and the sign words of step
// k+1 are issued first; the 64 MFMAs of step k run; the sign words of step k+1
// are unpacked (one shift + one and-or per pair) into the other B stage; one
// barrier.
//
// Layout facts of the 32x32x16 MFMA: A lane l supplies row l%32 and 8
// consecutive k of block l/32; B lane l supplies column l%32 and the same k
// block; D lane l holds, in item r, row 8*(r/4) + 4*(l/32) + r%4 of column l%32.
#include "common.h"
#include "kernels.h"

namespace brq {

namespace {

constexpr int PF_BM = 256, PF_BN = 256, PF_BK = 64;
constexpr int PF_ROWB = PF_BK * 2;               // bytes per LDS row
constexpr int PF_TILE = PF_BM * PF_ROWB;         // bytes per A (or B) stage

__device__ __forceinline__ int pf_slot(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

}  // namespace

template <bool OUT_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_pf(const uint16_t* __restrict__ xp, int M, int N, int K,
                                            const uint32_t* __restrict__ signs, const uint16_t* __restrict__ scales,
                                            void* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* As = lds;                   // [2][PF_TILE]
  uint8_t* Bs = lds + 2 * PF_TILE;     // [2][PF_TILE]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;

  // tile id -> (tm, tn): consecutive ids of one XCD (id % 8) cover a
  // contiguous range of tiles, so an XCD streams few activation row-blocks
  const int tiles_m = (M + PF_BM - 1) / PF_BM, tiles_n = (N + PF_BN - 1) / PF_BN;
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  const int m0 = (bid / tiles_n) * PF_BM, n0 = (bid % tiles_n) * PF_BN;
  const int nk = K / PF_BK;
  const int G = K >> 7, KW = K >> 5;  // groups, 32-bit sign words per row

  // ---- A: this wave's 8 direct-load instructions cover rows 64*wave .. +63
  // lane L of instruction i: row 64*wave + 8*i + L/8, LDS slot L%8 which holds
  // chunk (L%8) ^ swz(row)
  const uint16_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rl = 64 * wave + 8 * i + (lane >> 3);
    const int gm = m0 + rl < M ? m0 + rl : M - 1;
    const int chunk = (lane & 7) ^ ((rl >> 1) & 7);
    a_src[i] = xp + (size_t)gm * K + chunk * 8;
  }
  auto issue_a = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(a_src[i] + kt * PF_BK, As + buf * PF_TILE + (64 * wave + 8 * i) * PF_ROWB,
                                       16, 0, 0);
  };

  // ---- B: thread t unpacks column n0 + t (one 64-bit sign word per k-step)
  const int bn = n0 + tid;
  const bool bok = bn < N;
  const int bnr = bok ? bn : N - 1;
  const uint32_t* b_sig = signs + (size_t)bnr * KW;
  const uint16_t* b_sc = scales + (size_t)bnr * G;
  uint2 bw;
  uint32_t bs;
  auto load_b = [&](int kt) {
    bw = *reinterpret_cast<const uint2*>(b_sig + 2 * kt);
    bs = b_sc[kt >> 1];
  };
  auto store_b = [&](int buf) {
    const uint32_t S = bok ? (bs | (bs << 16)) : 0u;
    uint8_t* row = Bs + buf * PF_TILE + tid * PF_ROWB;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t dw = (c < 4) ? bw.x : bw.y;
      u32x4 o;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int bit = 4 * (c & 3) + t;
        o[t] = ((dw << (15 - bit)) & 0x80008000u) | S;
      }
      *reinterpret_cast<u32x4*>(row + pf_slot(tid, c) * 16) = o;
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment read offsets (bytes inside a stage); the k chunk of sub-step ks
  // is 2*ks + l/32
  const int fr = lane & 31, fh = lane >> 5;
  int a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_off[i] = (wr * 128 + 32 * i + fr) * PF_ROWB;
    b_off[i] = (wc * 128 + 32 * i + fr) * PF_ROWB;
  }
  const int swz = (fr >> 1) & 7;  // rows of a fragment start at multiples of 32

  // fragments of sub-step ks live in af[ks&1], bfr[ks&1]; the reads of sub-step
  // ks+1 are issued before the 16 MFMAs of sub-step ks
  u32x4 af[2][4], bfr[2][4];
  auto read_frags = [&](const uint8_t* Ac, const uint8_t* Bc, int ks, int set) {
    const int slot = ((2 * ks + fh) ^ swz) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) af[set][i] = *reinterpret_cast<const u32x4*>(Ac + a_off[i] + slot);
#pragma unroll
    for (int j = 0; j < 4; ++j) bfr[set][j] = *reinterpret_cast<const u32x4*>(Bc + b_off[j] + slot);
  };

  // prologue: stage 0 complete
  issue_a(0, 0);
  load_b(0);
  __builtin_amdgcn_s_waitcnt(0);
  store_b(0);
  __syncthreads();

  // One k-step per iteration. Stage `cur` holds step kt. The direct loads and
  // the sign words of step kt+1 are issued first (pinned there by a scheduling
  // barrier), the 64 MFMAs of step kt run, then the sign words are unpacked
  // into stage cur^1. The body has no branches: the loads of the last step
  // repeat step nk-1 into the idle stage.
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const int k1 = kt + 1 < nk ? kt + 1 : kt;
    const uint8_t* Ac = As + cur * PF_TILE;
    const uint8_t* Bc = Bs + cur * PF_TILE;
    issue_a(k1, cur ^ 1);
    load_b(k1);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(Ac, Bc, 0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) read_frags(Ac, Bc, ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[ks & 1][i], bfr[ks & 1][j], acc[i][j]);
    }
    __builtin_amdgcn_sched_barrier(0);  // the sign words are consumed only after the MFMAs
    store_b(cur ^ 1);
    __builtin_amdgcn_s_waitcnt(0);  // direct loads of step kt+1 landed
    __syncthreads();
  }

  // ---- epilogue: lane writes column fr of each 32 x 32 tile, rows in runs of 4
  const bool full = (m0 + PF_BM <= M) && (n0 + PF_BN <= N);
  auto put = [&](size_t idx, float v) {
    if (OUT_BF16)
      reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16_bits(v);
    else
      reinterpret_cast<float*>(y)[idx] = v;
  };
  if (full) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t base = (size_t)(m0 + wr * 128 + 32 * i + 4 * fh) * N + (n0 + wc * 128 + 32 * j + fr);
#pragma unroll
        for (int r = 0; r < 16; ++r) put(base + (size_t)(8 * (r >> 2) + (r & 3)) * N, acc[i][j][r]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wc * 128 + 32 * j + fr;
        const int rbase = m0 + wr * 128 + 32 * i + 4 * fh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + 8 * (r >> 2) + (r & 3);
          if (row < M && col < N) put((size_t)row * N + col, acc[i][j][r]);
        }
      }
  }
}

size_t pf_lds_bytes() { return 4 * (size_t)PF_TILE; }

hipError_t launch_gemm_pf(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                          void* y, int y_bf16, void* ws, hipStream_t st) {
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws);
  hipError_t e = launch_prep_bf16(x, M, K, xp, st);
  if (e != hipSuccess) return e;
  // 128 KiB of dynamic LDS needs the per-function opt-in (set on every call:
  // the attribute is per device and cheap to repeat)
  const void* fn = y_bf16 ? reinterpret_cast<const void*>(&k_pf<true>) : reinterpret_cast<const void*>(&k_pf<false>);
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)pf_lds_bytes());
  if (e != hipSuccess) return e;
  const int tiles = ((M + PF_BM - 1) / PF_BM) * ((N + PF_BN - 1) / PF_BN);
  if (y_bf16)
    hipLaunchKernelGGL(k_pf<true>, dim3(tiles), dim3(256), pf_lds_bytes(), st, xp, M, N, K,
                       reinterpret_cast<const uint32_t*>(signs), scales, y);
  else
    hipLaunchKernelGGL(k_pf<false>, dim3(tiles), dim3(256), pf_lds_bytes(), st, xp, M, N, K,
                       reinterpret_cast<const uint32_t*>(signs), scales, y);
  return hipGetLastError();
}

}  // namespace brq
