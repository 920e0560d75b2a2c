// Product for 8 < M <= 64 activation rows (the decode-batch regime between one
// vector and the prefill tiles, "LLM binarization, Episode 01: DBF", section 4:
// each matrix is now applied to a handful of vectors).
//
// A workgroup owns 64 output columns and a range of at most 32 k-steps (one
// k-step = 128 k = one scale group); its eight waves take every eighth k-step
// of the range (wave w: steps w, w+8, ...), each for all 64 columns and all M
// rows (two waves per SIMD hide each other's waits).
//  - The workgroup's sign records (16 B per column and k-step) and fp16
//    scales are loaded once, by all waves together, into LDS tables where
//    each column's consecutive k-steps are contiguous, as they are in memory
//    (every load instruction covers long contiguous runs); one barrier.
//  - The activation rows stream global -> LDS with direct loads
//    (global_load_lds_dwordx4) through a ring owned by each wave; a stage
//    holds 1/sub of a k-step of every row (about 4 KiB), chunk c of staged row
//    r at slot c ^ ((r / sub) % (16 / sub)), so the 16 lanes of one LDS pass
//    hit 16 different bank groups.
//  - v_mfma_f32_16x16x32_bf16 multiplies the bf16 rows as they are by +-1
//    weights (both exact, so a k-step's four MFMAs give the group's signed sums
//    of x in fp32 for x of any magnitude), and each group sum is added times
//    its fp16 scale into the fp32 result. A lane's 8 k of a 32-k sub-step are
//    consecutive in both operands: byte kb of the sub-step's sign word, with a
//    copy shifted up by 15, gives each weight pair by one shift and one and-or.
// At the end the waves' results meet in LDS and are added in wave order.
//
// When the k-steps are split over several workgroups (K-slices), each writes
// its fp32 partial result to the workspace and a second launch adds the
// slices in slice order (deterministic). The split is chosen so that the grid
// is about one workgroup per compute unit, each wave has a k-step where K
// allows it, and no workgroup has more than 32.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace brq {

namespace {

constexpr int MID_BN = 64;  // columns of a workgroup (four 16-column groups, each in every wave)
constexpr int MID_NB = 4;   // 16-column groups per wave
constexpr int MID_KPS = 32; // most k-steps of a workgroup

struct MidPlan {
  int tiles, splits, kps;  // column tiles, K-slices, k-steps per K-slice
};

// About one workgroup per compute unit (at least 256 workgroups where K
// allows one k-step per wave), and at most MID_KPS k-steps per workgroup.
MidPlan mid_plan(int64_t N, int64_t K) {
  MidPlan p;
  const int nk = (int)(K / 128);
  p.tiles = (int)((N + MID_BN - 1) / MID_BN);
  const int need = (nk + MID_KPS - 1) / MID_KPS;
  const int fill = std::max(1, 256 / p.tiles);
  const int most = std::max(1, nk / 8);  // one k-step for each of the 8 waves
  const int s = std::max(need, std::min(fill, most));
  p.kps = (nk + s - 1) / s;
  p.splits = (nk + p.kps - 1) / p.kps;
  return p;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// wait until at most N vector memory operations are outstanding (a larger
// count waits as for 63: later loads complete after earlier ones); compiler
// fences keep every memory access on its side (s_waitcnt immediate: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void vm_wait() {
  constexpr int n = N < 63 ? N : 63;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void lgkm_wait0() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// f(integral_constant<int, I>) for I = B .. E-1, in order
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace

// The KW waves' results meet in LDS (reused: every wave is past its last
// step) and are added in wave order: the four values (t, g, 0..3) of lane L
// of wave w at red[((w * TT * NB + t * NB + g) * 64 + L) * 4 ..]; then y (one
// K-slice) or this slice's partial result. A thread takes a lane slot (t, g,
// L): rows 16t + 4(L / 16) .. +3 of column 16g + L % 16.
template <int TT, int KW>
__device__ __forceinline__ void mid_reduce_store(const f32x4 (&acc)[TT][MID_NB], uint8_t* lds, void* y, int y_bf16,
                                                 float* part, int M, int N, int n0, int sl, int S, int lane,
                                                 int ks) {
  constexpr int NB = MID_NB, TG = TT * NB;
  f32x4* red = reinterpret_cast<f32x4*>(lds);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int g = 0; g < NB; ++g) red[(ks * TG + t * NB + g) * 64 + lane] = acc[t][g];
  __syncthreads();
  const int np = gridDim.x * MID_BN;
  for (int o = threadIdx.x; o < TG * 64; o += 64 * KW) {
    const int tg = o >> 6, ln = o & 63;
    f32x4 v = red[tg * 64 + ln];
#pragma unroll
    for (int w = 1; w < KW; ++w) v += red[(w * TG + tg) * 64 + ln];
    const int n = n0 + 16 * (tg % NB) + (ln & 15), r0 = 16 * (tg / NB) + 4 * (ln >> 4);
    if (n >= N) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = r0 + e;
      if (row >= M) break;
      if (S == 1) store_out(y, (size_t)row * N + n, v[e], y_bf16);
      else part[((size_t)sl * M + row) * np + n] = v[e];
    }
  }
}

// Eight waves per workgroup (two per SIMD, which hide each other's waits). A
// ring stage holds 1/sub of a k-step of the TT row tiles (sub = 1, 2, 4: 256,
// 128 or 64 bytes of each row), about 4 KiB, so that three or four stages per
// wave fit beside the tables.
__host__ __device__ constexpr int midt_kw(int) { return 8; }
__host__ __device__ constexpr int midt_sub(int tt) { return tt == 1 ? 1 : tt == 2 ? 2 : 4; }
__host__ __device__ constexpr int midt_da(int tt) { return tt == 3 ? 4 : 3; }
__host__ __device__ constexpr int midt_sb(int tt) { return tt * 16 * 256 / midt_sub(tt); }
// Tables in two halves (local k-steps 0..15 and 16..31), each 64 columns x 16
// steps: sign records (16 KiB) then the 4-byte words holding the fp16 scales
// (4 KiB). Entry (column c, step s) of a half sits at slot s ^ (c % 16) of
// column c's 16 slots, so that 16 lanes reading 16 columns at one step hit 16
// different bank groups, while every direct load instruction (64 slots, four
// columns) reads four contiguous 256-byte runs of memory. A wave's steps are
// ks, ks + 8 (first half) and ks + 16, ks + 24 (second half): its first two
// steps run while the second half is still arriving.
constexpr int MIDT_HALF = 16 * 1024 + 4 * 1024;
constexpr int MIDT_TAB = 2 * MIDT_HALF;
// the tables and rings, or (reused at the end) the waves' results: kw x tt x
// 16 rows x 64 columns of fp32
__host__ __device__ constexpr int midt_lds_bytes(int tt) {
  return MIDT_TAB + midt_kw(tt) * midt_da(tt) * midt_sb(tt) > midt_kw(tt) * tt * 4096
             ? MIDT_TAB + midt_kw(tt) * midt_da(tt) * midt_sb(tt)
             : midt_kw(tt) * tt * 4096;
}
static_assert(midt_lds_bytes(1) <= 160 * 1024 && midt_lds_bytes(2) <= 160 * 1024 && midt_lds_bytes(3) <= 160 * 1024 &&
                  midt_lds_bytes(4) <= 160 * 1024,
              "tables and rings exceed the LDS");

// Issue order of a wave's direct loads: table half 0 (4 loads), the
// activations of units 0 .. DA-1 (unit = k-step i * sub + h; la loads each),
// table half 1 (4 loads), then after the products of unit p the activations
// of unit p + DA (while the wave has that unit). Loads complete in order, so
// an operation has landed once at most (the loads issued after it) are
// outstanding. midt_pos* give issue positions (loads issued up to and
// including the operation; before unit u's products for midt_pos_now).
__host__ __device__ constexpr int midt_pos_a(int tt, int units, int u) {  // after A(u)
  const int da = midt_da(tt), la = 4 * tt / midt_sub(tt), pro = da < units ? da : units;
  if (u < da) return 4 + (u + 1) * la;
  return 4 + pro * la + 4 + (u - da + 1) * la;
}
__host__ __device__ constexpr int midt_pos_h1(int tt, int units) {
  const int da = midt_da(tt), la = 4 * tt / midt_sub(tt), pro = da < units ? da : units;
  return 4 + pro * la + 4;
}
__host__ __device__ constexpr int midt_pos_now(int tt, int units, int u) {
  const int da = midt_da(tt), la = 4 * tt / midt_sub(tt);
  int n = midt_pos_h1(tt, units);
  for (int p = 0; p < u; ++p)
    if (p + da < units) n += la;
  return n;
}

struct MidTab {
  const uint8_t* xb;      // activations
  uint32_t xo[4], xl[4];  // activation row offsets (full tiles; the last tile), per load of a tile
  uint32_t cpar;          // bit g: parity of (column 16g + j) * G + the wave's first k-step
  int q0, K, j, kb, sl0;  // first global / local k-step of the wave
};

template <int TT, int CNT>
__device__ __forceinline__ void midt_steps(f32x4 (&acc)[TT][MID_NB], const MidTab& L, uint8_t* lds, uint8_t* aring,
                                           const uint4* __restrict__ recs, const uint16_t* __restrict__ scales, int N,
                                           int G, int n0, int kt0, int nks, int lane, int ks) {
  constexpr int DA = midt_da(TT), SB = midt_sb(TT), NB = MID_NB, KW = midt_kw(TT), SUB = midt_sub(TT);
  constexpr int RB = 256 / SUB, LPT = 4 / SUB;  // bytes per staged row, direct loads per row tile
  constexpr int UNITS = CNT * SUB;
  const int j = L.j, kb = L.kb;
  auto load_a = [&](int u) {
    const int i = u / SUB, h = u % SUB;
    const uint8_t* src = L.xb + (size_t)(L.q0 + KW * i) * 256 + h * RB;
    uint8_t* dst = aring + (u % DA) * SB;
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int r = 0; r < LPT; ++r) {
        const void* g = t < TT - 1 ? src + (size_t)t * 32 * L.K + L.xo[r] : src + L.xl[r];
        __builtin_amdgcn_global_load_lds(g, dst + (16 * t + (16 / LPT) * r) * RB, 16, 0, 0);
      }
  };
  // a table half: instruction i (0..15; wave i % 8 issues it) fills slots
  // 64i .. 64i+63, i.e. columns 4i .. 4i+3; slot p of column c holds step
  // p ^ (c % 16) (steps past the slice repeat its last, columns past N repeat
  // N - 1). The scale of an entry is taken as the aligned 4-byte word that
  // holds it (the scale array is 16-byte aligned, so the word of its last
  // scale lies in the same 16-byte block, never on another page). Only direct
  // loads here: the compiler would make any wait for a register load also
  // wait for every direct load.
  static_assert(KW == 8, "table halves assume eight waves");
  const uint32_t* sw = reinterpret_cast<const uint32_t*>(scales);
  auto load_half = [&](int hf) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = ks + KW * k, e = 64 * i + lane, c = e >> 4, st = 16 * hf + ((e & 15) ^ (c & 15));
      const int n = n0 + c < N ? n0 + c : N - 1;
      const size_t rq = (size_t)n * G + kt0 + (st < nks ? st : nks - 1);
      uint8_t* base = lds + hf * MIDT_HALF;
      __builtin_amdgcn_global_load_lds(recs + rq, base + 64 * i * 16, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(sw + (rq >> 1), base + 16384 + 64 * i * 4, 4, 0, 0);
    }
  };
  load_half(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);  // issue order: half 0, first stages, half 1
#pragma unroll
  for (int u = 0; u < DA && u < UNITS; ++u) load_a(u);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  load_half(1);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  // half 0 of every wave has landed: a bare barrier (__syncthreads would also
  // wait for the loads still in flight)
  vm_wait<midt_pos_h1(TT, UNITS) - 4>();
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  auto half1_ready = [&]() {
    vm_wait<midt_pos_now(TT, UNITS, 2 * SUB < UNITS ? 2 * SUB : UNITS) - midt_pos_h1(TT, UNITS)>();
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  uint32_t one2;  // bf16 +1.0 pairs in a register: the and-or is then one instruction
  asm("v_mov_b32 %0, 0x3f803f80" : "=v"(one2));
  // slot of chunk c of a staged row r: c ^ ((r / sub) % (16 / sub)) (the 16
  // lanes of one pass, rows j, hit 16 different 16-byte bank groups)
  const int swz = (j / SUB) & (16 / SUB - 1);

  u32x4 R[NB];
  uint32_t C[NB];
  f32x4 gs[TT][NB];
  static_for<0, UNITS>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    constexpr int i = u / SUB, h = u % SUB;
    if constexpr (u == 2 * SUB) half1_ready();  // steps 2, 3 read the second half
    vm_wait<midt_pos_now(TT, UNITS, u) - midt_pos_a(TT, UNITS, u)>();  // unit u's activations are in LDS
    if constexpr (h == 0) {
      // step sl = ks + 8i: table half sl / 16, slot (sl % 16) ^ j of column 16g + j
      const int sl = L.sl0 + KW * i;
      const uint8_t* hb = lds + (i >> 1) * MIDT_HALF;
      const int slot = (sl & 15) ^ j;
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        R[g] = *reinterpret_cast<const u32x4*>(hb + ((16 * g + j) * 16 + slot) * 16);
        // the scale: half (parity of column * G + step) of its word; steps of a
        // wave are KW apart (even), so the parity is the wave's first step's
        C[g] = reinterpret_cast<const uint32_t*>(hb + 16384)[(16 * g + j) * 16 + slot] >> (16 * ((L.cpar >> g) & 1));
      }
    }
    const uint8_t* as = aring + (u % DA) * SB + j * RB;
#pragma unroll
    for (int s2 = 0; s2 < 4 / SUB; ++s2) {
      const int s = h * (4 / SUB) + s2;  // 32-k sub-step of the k-step
      const int slot = ((4 * s2 + kb) ^ swz) * 16;
      u32x4 a[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) a[t] = *reinterpret_cast<const u32x4*>(as + t * 16 * RB + slot);
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        // the lane's 8 weights: bits 8kb .. 8kb+7 of word s; pair w = bits 2w, 2w+1
        const uint32_t w8 = __builtin_amdgcn_ubfe(R[g][s], 8 * kb, 8);
        const uint32_t w16 = w8 | (w8 << 15);
        u32x4 b;
#pragma unroll
        for (int w = 0; w < 4; ++w) b[w] = ((w16 << (15 - 2 * w)) & 0x80008000u) | one2;
#pragma unroll
        for (int t = 0; t < TT; ++t) gs[t][g] = mfma16_bf16(a[t], b, s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : gs[t][g]);
      }
    }
    if constexpr (h == SUB - 1) {
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        const float sc = f16_bits_to_f32(C[g]);
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][g][e] = fmaf(sc, gs[t][g][e], acc[t][g][e]);
      }
    }
    lgkm_wait0();  // this unit's ring reads are done before a direct load refills the stage
    if (u + DA < UNITS) load_a(u + DA);
    __builtin_amdgcn_sched_barrier(0);
  });
  if constexpr (UNITS <= 2 * SUB) half1_ready();  // every wave meets both barriers
  __builtin_amdgcn_s_waitcnt(0);
}

// Offsets of activations are 32-bit: M * K * 2 bytes are below 4 GiB on this
// path (mid_fits).
template <int TT>
__global__ __launch_bounds__(64 * midt_kw(TT)) void k_midt(const uint16_t* __restrict__ x, int M, int N, int K,
                                                           const uint4* __restrict__ recs,
                                                           const uint16_t* __restrict__ scales, void* __restrict__ y,
                                                           int y_bf16, float* __restrict__ part, int kps, int S) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int DA = midt_da(TT), SB = midt_sb(TT), NB = MID_NB, KW = midt_kw(TT), SUB = midt_sub(TT);
  constexpr int LPT = 4 / SUB, RPL = 16 / LPT;  // direct loads per row tile, rows per load
  const int lane = threadIdx.x & 63;
  const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // the wave (uniform)
  const int G = K >> 7;
  // workgroup -> (column tile, K-slice): consecutive workgroups go to
  // different chiplets (XCDs, eight); when the slices divide the chiplets and
  // their tiles evenly, each chiplet takes the tiles of one slice only, so its
  // L2 holds one slice of the activations instead of all of them
  int tile = blockIdx.x, sl = blockIdx.y;
  {
    const int tiles = gridDim.x, gx = 8 / S;
    if (S > 1 && S <= 8 && 8 % S == 0 && tiles % gx == 0) {
      const int id = blockIdx.x + tiles * blockIdx.y, xcd = id % 8, slot = id / 8;
      sl = xcd / gx;
      tile = xcd % gx + gx * slot;
    }
  }
  const int kt0 = sl * kps, nks = min(kps, G - kt0);
  const int cnt = nks > ks ? (nks - ks + KW - 1) / KW : 0;  // this wave's k-steps
  const int n0 = tile * MID_BN;

  MidTab L;
  L.j = lane & 15;
  L.kb = lane >> 4;
  L.K = K;
  L.q0 = kt0 + ks;
  L.sl0 = ks;
  L.xb = reinterpret_cast<const uint8_t*>(x);
  // direct load r of a row tile moves rows RPL*r .. RPL*r + RPL-1 of it: lane
  // takes row RPL*r + lane / (16/SUB) and puts the chunk that belongs at slot
  // lane % (16/SUB) there (the swizzle above)
#pragma unroll
  for (int r = 0; r < LPT; ++r) {
    const int cpr = 16 / SUB;  // chunks per staged row
    const int rr = RPL * r + lane / cpr, p = lane % cpr, rl = 16 * (TT - 1) + rr;
    const int c = p ^ ((rr / SUB) & (cpr - 1));
    L.xo[r] = (uint32_t)rr * (uint32_t)K * 2u + (uint32_t)(c * 16);
    L.xl[r] = (uint32_t)(rl < M ? rl : M - 1) * (uint32_t)K * 2u + (uint32_t)(c * 16);
  }
  L.cpar = 0;
#pragma unroll
  for (int g = 0; g < NB; ++g) {
    const int n = n0 + 16 * g + L.j < N ? n0 + 16 * g + L.j : N - 1;
    L.cpar |= (((uint32_t)n * (uint32_t)G + (uint32_t)L.q0) & 1u) << g;
  }
  f32x4 acc[TT][NB];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int g = 0; g < NB; ++g) acc[t][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint8_t* const aring = lds + MIDT_TAB + ks * DA * SB;
#define BRQ_MIDT(C) midt_steps<TT, C>(acc, L, lds, aring, recs, scales, N, G, n0, kt0, nks, lane, ks)
  switch (cnt) {  // uniform across the wave; every wave loads its share of the tables
    case 0: BRQ_MIDT(0); break;
    case 1: BRQ_MIDT(1); break;
    case 2: BRQ_MIDT(2); break;
    case 3: BRQ_MIDT(3); break;
    case 4: BRQ_MIDT(4); break;
    case 5: if constexpr (KW == 4) BRQ_MIDT(5); break;
    case 6: if constexpr (KW == 4) BRQ_MIDT(6); break;
    case 7: if constexpr (KW == 4) BRQ_MIDT(7); break;
    default: if constexpr (KW == 4) BRQ_MIDT(8); break;
  }
#undef BRQ_MIDT
  mid_reduce_store<TT, KW>(acc, lds, y, y_bf16, part, M, N, n0, sl, S, lane, ks);
}

// y = the sum of the S partial results part[s][M][np], in slice order
// (deterministic); one thread per four columns of a row.
__global__ __launch_bounds__(256) void k_mid_sum(const float* __restrict__ part, int M, int N, int np, int S,
                                                 void* __restrict__ y, int y_bf16) {
  const int n4 = np / 4;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)M * n4) return;
  const int m = (int)(e / n4), c = 4 * (int)(e - (int64_t)m * n4);
  const f32x4* p = reinterpret_cast<const f32x4*>(part + (size_t)m * np + c);
  const size_t step = (size_t)M * n4;
  f32x4 v = p[0];
  for (int s = 1; s < S; ++s) v += p[s * step];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (c + i < N) store_out(y, (size_t)m * N + c + i, v[i], y_bf16);
}

bool mid_fits(int64_t M, int64_t N, int64_t K) {
  return (uint64_t)M * (uint64_t)K * 2u < (1ull << 32) && (uint64_t)N * (uint64_t)(K / 8) < (1ull << 32);
}

size_t mid_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const MidPlan p = mid_plan(N, K);
  return p.splits > 1 ? align256((size_t)p.splits * M * p.tiles * MID_BN * 4) : 0;
}

template <typename Kern>
static hipError_t mid_run(Kern kern, int threads, int lds, const uint16_t* x, int M, int N, int K,
                          const uint64_t* signs, const uint16_t* scales, void* y, int y_bf16, float* part,
                          const MidPlan& p, hipStream_t st) {
  if (lds > 64 * 1024) {  // per-function opt-in beyond 64 KiB of dynamic LDS
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(p.tiles, p.splits), dim3(threads), lds, st, x, M, N, K,
                     reinterpret_cast<const uint4*>(signs), scales, y, y_bf16, part, p.kps, p.splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int np = p.tiles * MID_BN;
  const int64_t n = (int64_t)M * np / 4;
  hipLaunchKernelGGL(k_mid_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, M, N, np, p.splits, y,
                     y_bf16);
  return hipGetLastError();
}

template <int TT>
static hipError_t midt_launch(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                              void* y, int y_bf16, float* part, const MidPlan& p, hipStream_t st) {
  return mid_run(&k_midt<TT>, 64 * midt_kw(TT), midt_lds_bytes(TT), x, M, N, K, signs, scales, y, y_bf16, part,
                 p, st);
}

hipError_t launch_gemm_mid(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                           void* y, int y_bf16, void* ws, hipStream_t st) {
  const MidPlan p = mid_plan(N, K);
  float* part = reinterpret_cast<float*>(ws);
  switch ((M + 15) / 16) {
    case 1: return midt_launch<1>(x, M, N, K, signs, scales, y, y_bf16, part, p, st);
    case 2: return midt_launch<2>(x, M, N, K, signs, scales, y, y_bf16, part, p, st);
    case 3: return midt_launch<3>(x, M, N, K, signs, scales, y, y_bf16, part, p, st);
    default: return midt_launch<4>(x, M, N, K, signs, scales, y, y_bf16, part, p, st);
  }
}

}  // namespace brq
