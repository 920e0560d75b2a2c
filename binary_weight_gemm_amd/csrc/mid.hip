// Product for 8 < M <= 64 activation rows (the decode-batch regime between one
// vector and the prefill tiles, "LLM binarization, Episode 01: DBF", section 4:
// each matrix is now applied to a handful of vectors).
//
// The work is split into 128-column tiles x K-slices of at most 8 k-steps
// (one 128-byte line of every sign row). A workgroup (4 waves, 32 columns
// each) first issues direct loads of all sign records of its slice into LDS
// and reads its scales; the activations stream through registers: each wave
// loads its share of the bf16 rows PREF k-steps ahead and writes them, as
// they are, in the permuted operand order to one of two LDS stages. Every
// wave multiplies all rows (TT tiles of 16) by its two 16-column groups with
// v_mfma_f32_16x16x32_bf16 on +-1 weight operands (bf16 activations and +-1
// are exact, so a k-step's MFMAs give the group's signed sums of x in fp32,
// for x of any magnitude) and adds each group sum times its fp16 scale into
// the fp32 result: one activation operand serves two MFMAs and one weight
// operand serves TT.
//
// With several K-slices each workgroup writes its fp32 partial tile to the
// workspace and a second launch adds the slices in slice order (deterministic).
// (Meeting inside the product launch instead -- last-arriving workgroup adds
// the tile -- needs a device-scope release per workgroup, which writes back
// the whole L2 of its chiplet and cost far more than the extra launch.)
#include "common.h"
#include "kernels.h"

namespace brq {

namespace {

constexpr int MID_NB = 2;            // 16-column groups per wave
constexpr int MID_BN = 64 * MID_NB;  // columns per workgroup
constexpr int MID_KPS = 8;           // most k-steps per slice: 8 x 16 B = one 128-byte line of a sign row

// k-steps of activations in flight in registers
__host__ __device__ constexpr int mid_pref(int tt) { return tt <= 2 ? 4 : 2; }
// dynamic LDS: the slice's sign records, its scale pairs, two activation stages
__host__ __device__ constexpr int mid_lds_bytes(int tt) {
  return MID_BN * MID_KPS * 16 + MID_BN * MID_KPS * 4 + 2 * 16 * tt * 256;
}

struct MidPlan {
  int tiles, slices, kps;  // column tiles, K-slices, k-steps per slice
};

// Slices of 8 k-steps (each column's sign records of a slice are one 128-byte
// line), halved while the grid has fewer than 256 workgroups.
MidPlan mid_plan(int64_t N, int64_t K) {
  MidPlan p;
  const int nk = (int)(K / 128);
  p.tiles = (int)((N + MID_BN - 1) / MID_BN);
  int kps = MID_KPS;
  while (kps > 1 && (int64_t)p.tiles * ((nk + kps - 1) / kps) < 256) kps /= 2;
  p.kps = kps;
  p.slices = (nk + kps - 1) / kps;
  return p;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

}  // namespace

template <int TT>
__global__ __launch_bounds__(256) void k_mid(const uint16_t* x, int M, int N, int K,
                                             const uint32_t* __restrict__ signs, const uint16_t* __restrict__ scales,
                                             void* __restrict__ y, int y_bf16, float* __restrict__ part, int kps,
                                             int S) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int PREF = mid_pref(TT), SB = 16 * TT * 256;
  constexpr int NB = MID_NB, BN = MID_BN;
  uint8_t* const l_sig = lds;                                                 // [2*kps blocks][1 KiB]
  uint32_t* const l_sc = reinterpret_cast<uint32_t*>(lds + BN * MID_KPS * 16);  // [kps][BN] scale pairs
  uint8_t* const l_a = lds + BN * MID_KPS * 20;                               // [2][16*TT rows][256 B]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int tile = blockIdx.x, sl = blockIdx.y;
  const int nk = K >> 7;
  const int kt0 = sl * kps, kt1 = kt0 + kps < nk ? kt0 + kps : nk, nks = kt1 - kt0;
  const int n0 = tile * BN;
  const int KW = K >> 5;  // 32-bit sign words per weight row

  // ---- the slice's sign records, one direct load per 64 x 16 B: block i
  // holds columns C*i .. C*i+C-1 (C = 64/kps) for all kps steps, lane L ->
  // column C*i + L % C, step L / C, at byte 16*L of the block. A column's
  // records of the slice are contiguous in memory (one line when kps = 8).
  // Columns past N repeat N-1 and steps past K repeat the last (never used).
  {
    const int C = 64 / kps;
    const int c = lane % C, q = lane / C;
    const int kt = kt0 + q < nk ? kt0 + q : nk - 1;
    for (int i = wave; i < 2 * kps; i += 4) {
      const int n = n0 + C * i + c < N ? n0 + C * i + c : N - 1;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(signs + (size_t)n * KW + 4 * kt), l_sig + i * 1024,
                                       16, 0, 0);
    }
  }

  // ---- the slice's scales: thread e -> (column e % BN, step e / BN)
  uint32_t scv[MID_KPS * BN / 256];
#pragma unroll
  for (int i = 0; i < MID_KPS * BN / 256; ++i) {
    const int e = tid + 256 * i, c = e % BN, q = e / BN;
    const int n = n0 + c < N ? n0 + c : N - 1;
    const int kt = kt0 + q < nk ? kt0 + q : nk - 1;
    scv[i] = q < kps ? scales[(size_t)n * nk + kt] : 0u;
  }

  // ---- activations: lane (rr = L/16, c = L%16) of wave w stages rows
  // r = 4*TT*w + 4i + rr (i < TT; rows past M repeat M-1, never stored),
  // permuted 16-byte chunk c of each k-step: run c/4, pairs b = 4(c%4) + u,
  // i.e. bf16 elements 4(c%4)+u (low halves) and 16+4(c%4)+u (high halves)
  // of the run -- two 8-byte loads. The chunk goes to LDS slot c ^ (r%16).
  const int rr = lane >> 4, cc = lane & 15;
  const uint8_t* xr[TT];
  uint32_t a_dst[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const int r = 4 * TT * wave + 4 * i + rr;
    const int rg = r < M ? r : M - 1;
    xr[i] = reinterpret_cast<const uint8_t*>(x) + (size_t)rg * K * 2 + (cc >> 2) * 64 + (cc & 3) * 8;
    a_dst[i] = (uint32_t)(r * 256 + ((cc ^ (r & 15)) * 16));
  }
  uint2 ra[PREF][TT][2];
  // (x is not __restrict__: the prefetch loads must stay ahead of the
  // barriers, which are memory clobbers)
  auto load_step = [&](uint2 (&dst)[TT][2], int q) {
    const size_t off = (size_t)(kt0 + (q < nks ? q : nks - 1)) * 256;
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      dst[i][0] = *reinterpret_cast<const uint2*>(xr[i] + off);
      dst[i][1] = *reinterpret_cast<const uint2*>(xr[i] + off + 32);
    }
  };
  auto stage_step = [&](const uint2 (&src)[TT][2], int st) {
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const uint2 lo = src[i][0], hi = src[i][1];
      u32x4 o;
      // pair (element b, element 16 + b): low halves, then high halves
      o[0] = __builtin_amdgcn_perm(hi.x, lo.x, 0x05040100u);
      o[1] = __builtin_amdgcn_perm(hi.x, lo.x, 0x07060302u);
      o[2] = __builtin_amdgcn_perm(hi.y, lo.y, 0x05040100u);
      o[3] = __builtin_amdgcn_perm(hi.y, lo.y, 0x07060302u);
      *reinterpret_cast<u32x4*>(l_a + st * SB + a_dst[i]) = o;
    }
  };
#pragma unroll
  for (int d = 0; d < PREF; ++d) load_step(ra[d], d);

#pragma unroll
  for (int i = 0; i < MID_KPS * BN / 256; ++i) {
    const int e = tid + 256 * i;
    l_sc[e] = scv[i] | (scv[i] << 16);
  }
  stage_step(ra[0], 0);
  load_step(ra[0], PREF);
  // every older load of this wave -- its sign records included -- landed
  // (only the activation loads of steps 1 .. PREF may be in flight), then
  // every wave's stage-0 writes and sign records are in
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * TT * PREF) : "memory");

  f32x4 acc[TT][NB];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int g = 0; g < NB; ++g) acc[t][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int bsh = 4 * kb;  // the lane's k block takes pairs 4*kb .. 4*kb+3 of each half-run
  // where this lane's columns sit in the sign blocks
  int sg_off[NB];
  {
    const int C = 64 / kps;
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      const int cl = 16 * (NB * wave + g) + j;
      sg_off[g] = (cl / C) * 1024 + (cl % C) * 16;
    }
  }
  const int sg_step = (64 / kps) * 16;

  // one k-step: stage step q+1 into the other LDS stage (every wave finished
  // reading it before the last barrier) and refill its registers with step
  // q+1+PREF (both unconditional: past the slice they repeat its last step,
  // unused), then multiply step q. d = q % PREF picks the registers.
  auto step = [&](const int q, const int d) {
    stage_step(ra[(d + 1) % PREF], (q + 1) & 1);
    load_step(ra[(d + 1) % PREF], q + 1 + PREF);
    const uint8_t* base = l_a + (q & 1) * SB;
    u32x4 a[4][TT];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < TT; ++t)  // chunk 4s+kb of row 16t+j
        a[s][t] = *reinterpret_cast<const u32x4*>(base + (16 * t + j) * 256 + (((4 * s + kb) ^ j) * 16));
    u32x4 w4[NB];
    float sc[NB];
#pragma unroll
    for (int g = 0; g < NB; ++g) {
      w4[g] = *reinterpret_cast<const u32x4*>(l_sig + sg_off[g] + q * sg_step);
      sc[g] = f16_bits_to_f32(l_sc[q * BN + 16 * (NB * wave + g) + j] & 0xffffu);
    }
    f32x4 gs[TT][NB];  // the k-step's (one scale group's) signed sums
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int g = 0; g < NB; ++g) {
        const uint32_t w = w4[g][s] >> bsh;
        u32x4 b;  // bf16 +-1 pairs
#pragma unroll
        for (int u = 0; u < 4; ++u) b[u] = ((w << (15 - u)) & 0x80008000u) | 0x3f803f80u;
#pragma unroll
        for (int t = 0; t < TT; ++t)
          gs[t][g] = mfma16_bf16(a[s][t], b, s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : gs[t][g]);
      }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
      for (int g = 0; g < NB; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][g][i] = fmaf(sc[g], gs[t][g][i], acc[t][g][i]);
    // the next stage's writes are in and every wave is done with this one
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // whole rounds of PREF steps with no branch inside, so that the compiler's
  // wait before each staging counts the PREF-1 younger steps in flight
  int q = 0;
  for (; q + PREF <= nks; q += PREF) {
#pragma unroll
    for (int d = 0; d < PREF; ++d) step(q + d, d);
  }
#pragma unroll
  for (int d = 0; d < PREF - 1; ++d)
    if (q + d < nks) step(q + d, d);
  __builtin_amdgcn_s_waitcnt(0);  // nothing in flight when the workgroup ends

  // lane (kb, j) holds rows 16t + 4kb + i of column cw + 16g + j
  const int cw = n0 + 16 * NB * wave;
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
  const MidPlan p = mid_plan(N, K);
  return p.slices > 1 ? align256((size_t)p.tiles * p.slices * M * MID_BN * 4) : 0;
}

template <int TT>
static hipError_t mid_launch(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                             void* y, int y_bf16, float* part, const MidPlan& p, hipStream_t st) {
  const int lds = mid_lds_bytes(TT);
  if (lds > 64 * 1024) {  // per-function opt-in beyond 64 KiB of dynamic LDS
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_mid<TT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_mid<TT>, dim3(p.tiles, p.slices), dim3(256), lds, st, x, M, N, K,
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
  const MidPlan p = mid_plan(N, K);
  float* part = reinterpret_cast<float*>(ws);
  switch ((M + 15) / 16) {
    case 1: return mid_launch<1>(x, M, N, K, signs, scales, y, y_bf16, part, p, st);
    case 2: return mid_launch<2>(x, M, N, K, signs, scales, y, y_bf16, part, p, st);
    case 3: return mid_launch<3>(x, M, N, K, signs, scales, y, y_bf16, part, p, st);
    default: return mid_launch<4>(x, M, N, K, signs, scales, y, y_bf16, part, p, st);
  }
}

}  // namespace brq
