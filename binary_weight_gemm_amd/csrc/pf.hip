// Prefill product y = x . Wq^T for many activation rows (M > 64) on the fp16
// matrix cores ("LLM binarization, Episode 01: DBF", section 4: one matrix
// applied to many vectors amortises the weight unpack over the rows).
//
// x is first written by k_prep_rows as fp16 in the permuted operand order
// (the pair order of the shift-and-or weight unpack, see common.h), each row
// scaled by a power of two that the epilogue undoes, so the main
// kernel moves activation tiles global -> LDS with direct loads
// (global_load_lds_dwordx4), never through registers.
//
// Block tile 256 x 256, k-step 128 (one scale group), four waves in 2 x 2,
// each wave 128 x 128 of v_mfma_f32_32x32x16_f16 tiles (16 accumulators of
// 16 fp32). Only the activations go through LDS: 256 rows x 256 B per stage,
// two stages (128 KiB); a row holds sixteen 16-byte chunks, chunk c at slot
// c ^ (row % 16), so that the 16 lanes of one LDS pass hit 16 different slots.
// The weight operand never touches LDS: every lane loads, for each of its four
// 32-column tiles, the four sign words of its column for the k-step (16 bytes)
// and the group scale, and builds the MFMA operands in registers (one shift
// and one and-or per pair of weights).
//
// Schedule of one k-step (8 sub-steps of 16 k, 16 MFMAs each): while the
// MFMAs of sub-step s run, the activation fragments of sub-step s+1 are read
// from LDS and its weight operands are built. In the middle of sub-step 7 every
// wave waits for its own direct loads of the next stage and meets the others
// at one barrier; right after it the direct loads and sign/scale loads two
// k-steps ahead are issued (one full k-step before they are needed), and the
// first fragments of the next k-step are read.
//
// Layout facts of the 32x32x16 MFMA: A lane l supplies row l%32 and 8
// consecutive k of block l/32; B lane l supplies column l%32 and the same k
// block; D lane l holds, in item r, row 8*(r/4) + 4*(l/32) + r%4 of column l%32.
#include "common.h"
#include "kernels.h"

namespace brq {

namespace {

constexpr int PF_BM = 256, PF_BK = 128;
constexpr int PF_ROWB = PF_BK * 2;        // bytes per LDS row
constexpr int PF_TILE = PF_BM * PF_ROWB;  // bytes per activation stage

}  // namespace

// BN = 256 (NJ = 4 column tiles of 32 per wave) or 128 (NJ = 2, used for the
// columns of a last partial round of 256-wide tiles, see launch_gemm_pf). The
// launch covers column tiles starting at column n_base, tiles_n of them.
// LR: one more k-step after the last adds a rank-r weight correction,
// (x V^T) U^T: its activation operand is lr_t [M][128] fp16 (x V^T as hi
// parts in k 0..63 and lo parts in k 64..127, natural order), staged like an
// activation k-step, and its weight operand is lr_u [N][64] fp16 (U padded
// with zeros), factor index k % 64, loaded straight into registers.
template <bool OUT_BF16, int BN, bool LR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_pf(
    const uint16_t* __restrict__ xp, int M, int N, int K, const uint32_t* __restrict__ signs,
    const uint16_t* __restrict__ scales, void* __restrict__ y, int n_base, int tiles_n,
    const uint16_t* __restrict__ lr_t, const uint16_t* __restrict__ lr_u, const int* __restrict__ rexp) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // [2][PF_TILE]
  constexpr int NJ = BN / 64;  // 32-column tiles per wave

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int fr = lane & 31, fh = lane >> 5;

  // tile id -> (tm, tn): consecutive ids of one XCD (id % 8) cover a
  // contiguous range of tiles, so an XCD streams few activation row-blocks
  const int tiles_m = (M + PF_BM - 1) / PF_BM;
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  const int m0 = (bid / tiles_n) * PF_BM, n0 = n_base + (bid % tiles_n) * BN;
  // staging exponents of this wave's 128 output rows (lane l: rows l and 64 + l
  // of the half); the rows were staged as x * 2^s, undone in the epilogue
  int rs0 = 0, rs1 = 0;
  if (rexp) {
    const int ra = m0 + wr * 128 + lane, rb = ra + 64;
    rs0 = rexp[ra < M ? ra : M - 1];
    rs1 = rexp[rb < M ? rb : M - 1];
  }
  const int nk = K / PF_BK;  // k-steps = scale groups
  const int KW = K >> 5;     // 32-bit sign words per weight row

  // ---- activations: this wave's 16 direct loads cover rows 64*wave .. +63;
  // lane L of load i: row 64*wave + 4*i + L/16, LDS slot L%16, which holds
  // chunk (L%16) ^ (row%16). Offsets are in bytes from the tile's first row
  // (rows past M repeat row M-1).
  uint32_t a_off[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rl = 64 * wave + 4 * i + (lane >> 4);
    const int gl = m0 + rl < M ? rl : M - 1 - m0;
    const int chunk = (lane & 15) ^ (rl & 15);
    a_off[i] = (uint32_t)gl * (uint32_t)(K * 2) + (uint32_t)(chunk * 16);
  }
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(xp) + (size_t)m0 * K * 2;
  // direct loads i0 .. i0+3 of k-step kt into `stage`
  auto issue_a4 = [&](int kt, int stage, int i0) {
#pragma unroll
    for (int i = i0; i < i0 + 4; ++i)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(xb + a_off[i] + (size_t)kt * PF_ROWB),
                                       lds + stage * PF_TILE + (64 * wave + 4 * i) * PF_ROWB, 16, 0, 0);
  };

  // ---- weights: column tile j of this wave is columns n0 + wc*BN/2 + 32j ..,
  // lane column fr; the lane's k block (fh) selects pairs 4*fh .. 4*fh+3 of
  // each half-run, so its sign words are pre-shifted right by 4*fh.
  const uint32_t* b_sig[NJ];
  const uint16_t* b_sc[NJ];
  bool b_ok[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = n0 + wc * (BN / 2) + 32 * j + fr;
    b_ok[j] = c < N;
    const int cc = c < N ? c : N - 1;
    b_sig[j] = signs + (size_t)cc * KW;
    b_sc[j] = scales + (size_t)cc * nk;
  }
  uint4 wn[NJ];       // sign words of the next k-step (in flight)
  uint32_t sn[NJ];    // its scales
  auto load_b = [&](int kt) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      wn[j] = *reinterpret_cast<const uint4*>(b_sig[j] + 4 * kt);
      sn[j] = b_sc[j][kt];
    }
  };
  uint32_t wsh[NJ][4];  // pre-shifted sign words of the current k-step
  uint32_t S[NJ];       // magnitude pair (scale | scale << 16), 0 past N
  const int bshift = 4 * fh;
  auto take_b = [&]() {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      wsh[j][0] = wn[j].x >> bshift;
      wsh[j][1] = wn[j].y >> bshift;
      wsh[j][2] = wn[j].z >> bshift;
      wsh[j][3] = wn[j].w >> bshift;
      S[j] = b_ok[j] ? (sn[j] | (sn[j] << 16)) : 0u;
    }
  };
  // weight operand of tile j, sub-step ks: pairs b = 8*(ks%2) + t of run ks/2
  u32x4 bo[2][NJ];
  auto build_b = [&](int ks, int buf) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t w = wsh[j][ks >> 1];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int b = 8 * (ks & 1) + t;
        bo[buf][j][t] = ((w << (15 - b)) & 0x80008000u) | S[j];
      }
    }
  };

  // ---- activation fragments: row wr*128 + 32i + fr, chunk 2*ks + fh at slot
  // (2*ks + fh) ^ (row % 16) = (2*ks) ^ (fh ^ fr % 16)
  const int a_row = (wr * 128 + fr) * PF_ROWB;
  const int a_x = (fh ^ (fr & 15)) * 16;
  u32x4 af[2][4];
  auto read_a = [&](int stage, int ks, int buf) {
    const uint8_t* p = lds + stage * PF_TILE + a_row + ((32 * ks) ^ a_x);
#pragma unroll
    for (int i = 0; i < 4; ++i) af[buf][i] = *reinterpret_cast<const u32x4*>(p + i * 32 * PF_ROWB);
  };

  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto mfmas = [&](int buf, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(af[buf][i], bo[buf][j], acc[i][j]);
  };

  // One k-step per iteration; stage cur holds k-step kt. During sub-steps
  // 0..3 the direct loads of k-step kt+1 go into the other stage (free since
  // the last barrier), 4 per sub-step, and the sign/scale words of kt+1 are
  // requested in sub-step 0. Each sub-step region below is ordered by
  // scheduling-group barriers so that the LDS reads, the operand build and the
  // loads sit between the MFMAs instead of in front of them.
  issue_a4(0, 0, 0);
  issue_a4(0, 0, 4);
  issue_a4(0, 0, 8);
  issue_a4(0, 0, 12);
  load_b(0);
  __builtin_amdgcn_s_waitcnt(0);
  take_b();
  __syncthreads();
  read_a(0, 0, 0);
  build_b(0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const int nx = kt + 1 < nk ? kt + 1 : kt;  // past the end: repeat the last step (unused)
#pragma unroll
    for (int ks = 0; ks < 7; ++ks) {
      const int b = ks & 1;
      read_a(cur, ks + 1, b ^ 1);
      build_b(ks + 1, b ^ 1);
      if (ks < 4) issue_a4(nx, cur ^ 1, 4 * ks);
      if (ks == 0) load_b(nx);
      mfmas(b, 0, 4);
#pragma unroll
      for (int m = 0; m < 4 * NJ; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
        if (m < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        if (ks < 4 && m < 4) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one direct load
        if (ks == 0 && m >= 4 && m < 4 + 2 * NJ) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // sign/scale load
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);      // three VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // sub-step 7: half of its MFMAs, then the k-step boundary
    mfmas(1, 0, 2);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);  // own direct loads of the next stage and its weights landed
    __syncthreads();                // every wave's loads landed and every wave is done with stage cur
    take_b();
    read_a(cur ^ 1, 0, 0);
    build_b(0, 0);
    mfmas(1, 2, 4);
#pragma unroll
    for (int m = 0; m < 2 * NJ; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(0);  // nothing in flight when the workgroup ends

  if constexpr (LR) {
    __syncthreads();  // every wave is done with the stages
    // the tile's rows of x V^T into stage 0, laid out like an activation k-step
    const uint8_t* tb = reinterpret_cast<const uint8_t*>(lr_t) + (size_t)m0 * PF_ROWB;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rl = 64 * wave + 4 * i + (lane >> 4);
      const int gl = m0 + rl < M ? rl : M - 1 - m0;
      const int chunk = (lane & 15) ^ (rl & 15);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(tb + (size_t)gl * PF_ROWB + chunk * 16),
                                       lds + (64 * wave + 4 * i) * PF_ROWB, 16, 0, 0);
    }
    // weight operand of tile j, sub-step ks: U[col][16*(ks%4) + 8*fh .. +7]
    u32x4 bu[NJ][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = n0 + wc * (BN / 2) + 32 * j + fr;
      const uint16_t* ur = lr_u + (size_t)(c < N ? c : N - 1) * 64 + 8 * fh;
#pragma unroll
      for (int q = 0; q < 4; ++q) bu[j][q] = *reinterpret_cast<const u32x4*>(ur + 16 * q);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      read_a(0, ks, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(af[0][i], bu[j][ks & 3], acc[i][j]);
    }
  }

  // ---- undo the rows' staging scales (rare: rows outside [2^-8, 2^15))
  if (__any((rs0 | rs1) != 0)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = 32 * i + 4 * fh + 8 * (r >> 2) + (r & 3);  // row within the wave's half
        const int sr = __shfl(i < 2 ? rs0 : rs1, q & 63, 64);
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j][r] = __builtin_amdgcn_ldexpf(acc[i][j][r], -sr);
      }
  }

  // ---- epilogue: lane writes column fr of each 32 x 32 tile, rows in runs of 4
  const bool full = (m0 + PF_BM <= M) && (n0 + BN <= N);
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
      for (int j = 0; j < NJ; ++j) {
        const size_t base = (size_t)(m0 + wr * 128 + 32 * i + 4 * fh) * N + (n0 + wc * (BN / 2) + 32 * j + fr);
#pragma unroll
        for (int r = 0; r < 16; ++r) put(base + (size_t)(8 * (r >> 2) + (r & 3)) * N, acc[i][j][r]);
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int col = n0 + wc * (BN / 2) + 32 * j + fr;
        const int rbase = m0 + wr * 128 + 32 * i + 4 * fh;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + 8 * (r >> 2) + (r & 3);
          if (row < M && col < N) put((size_t)row * N + col, acc[i][j][r]);
        }
      }
  }
}

size_t pf_lds_bytes() { return 2 * (size_t)PF_TILE; }

template <bool OUT_BF16, int BN, bool LR>
static hipError_t pf_launch(const uint16_t* xp, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                            void* y, int n_base, int tiles_n, const uint16_t* lr_t, const uint16_t* lr_u,
                            const int* rexp, hipStream_t st) {
  // 128 KiB of dynamic LDS needs the per-function opt-in (set on every call:
  // the attribute is per device and cheap to repeat)
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pf<OUT_BF16, BN, LR>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)pf_lds_bytes());
  if (e != hipSuccess) return e;
  const int tiles = ((M + PF_BM - 1) / PF_BM) * tiles_n;
  hipLaunchKernelGGL((k_pf<OUT_BF16, BN, LR>), dim3(tiles), dim3(256), pf_lds_bytes(), st, xp, M, N, K,
                     reinterpret_cast<const uint32_t*>(signs), scales, y, n_base, tiles_n, lr_t, lr_u, rexp);
  return hipGetLastError();
}

// Tile plan. One 256x256 tile per compute unit at a time (128 KiB of LDS), so
// the tiles run in rounds of `cus`. When the last round is at most half full,
// its columns are given to 256x128 tiles instead: a full round of half-size
// tiles, so the launch takes rounds + 1/2 tile-times instead of rounds + 1
// (C5, 4096 x 14336: 768 tiles of 256 wide, then 256 tiles of 128 wide over
// the last 2048 columns).
void pf_plan(int M, int N, int cus, int& big_n, int& small_n) {
  const int tiles_m = (M + PF_BM - 1) / PF_BM, tiles_n = (N + 255) / 256;
  const int64_t total = (int64_t)tiles_m * tiles_n;
  const int64_t rest = total % cus;
  big_n = tiles_n;
  small_n = 0;
  if (total < cus || rest == 0 || 2 * rest > cus) return;
  const int cols = (int)((rest + tiles_m - 1) / tiles_m);  // 256-wide column tiles in the last round
  big_n = tiles_n - cols;
  small_n = (N - big_n * 256 + 127) / 128;
  if ((int64_t)tiles_m * small_n > cus) {  // the 128-wide tiles would not fit one round
    big_n = tiles_n;
    small_n = 0;
  }
}

template <bool LR>
static hipError_t pf_run(const uint16_t* xp, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                         void* y, int y_bf16, const uint16_t* lr_t, const uint16_t* lr_u, const int* rexp,
                         hipStream_t st) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;  // MI355X
  int big_n, small_n;
  pf_plan(M, N, cus, big_n, small_n);
  hipError_t e = hipSuccess;
  if (big_n > 0) {
    e = y_bf16 ? pf_launch<true, 256, LR>(xp, M, N, K, signs, scales, y, 0, big_n, lr_t, lr_u, rexp, st)
               : pf_launch<false, 256, LR>(xp, M, N, K, signs, scales, y, 0, big_n, lr_t, lr_u, rexp, st);
    if (e != hipSuccess) return e;
  }
  if (small_n > 0)
    e = y_bf16 ? pf_launch<true, 128, LR>(xp, M, N, K, signs, scales, y, big_n * 256, small_n, lr_t, lr_u, rexp,
                                          st)
               : pf_launch<false, 128, LR>(xp, M, N, K, signs, scales, y, big_n * 256, small_n, lr_t, lr_u, rexp,
                                           st);
  return e;
}

// workspace: the staged rows (fp16 [M][K]), then one staging exponent per row
size_t pf_ws_bytes(int64_t M, int64_t K) { return align256((size_t)M * K * 2) + align256((size_t)M * 4); }

hipError_t launch_gemm_pf(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                          void* y, int y_bf16, void* ws, hipStream_t st) {
  uint16_t* xp = reinterpret_cast<uint16_t*>(ws);
  int* rexp = reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + align256((size_t)M * K * 2));
  // the rows are staged with a power-of-two scale per row, undone in the epilogue
  const hipError_t e = launch_prep_rows(x, M, K, xp, rexp, 1, st);
  if (e != hipSuccess) return e;
  return pf_run<false>(xp, M, N, K, signs, scales, y, y_bf16, nullptr, nullptr, rexp, st);
}

hipError_t launch_gemm_pf_lr(const uint16_t* xp, const int* rexp, int M, int N, int K, const uint64_t* signs,
                             const uint16_t* scales, const uint16_t* lr_t, const uint16_t* lr_u, void* y, int y_bf16,
                             hipStream_t st) {
  // xp and rexp from launch_prep_rows; lr_t was formed from the same scaled
  // rows, so the epilogue undoes one power of two for both terms
  return pf_run<true>(xp, M, N, K, signs, scales, y, y_bf16, lr_t, lr_u, rexp, st);
}

}  // namespace brq
