// Routed mixture-of-experts SwiGLU layer on group-128 experts.
//
// Each selected (token, slot) route carries an expert id and a route weight
// ("LLM binarization, Episode 01: DBF", section 4); gate/up read the token's
// hidden vector, shared by all its routes, and down reads the route's own
// intermediate, compacted in expert-major order (section 5, items 8 and 10:
// expert-major route-specific inputs, shared gate/up inputs not duplicated,
// empty experts skipped). 256 experts with 8 routed and an f32 router follow
// the "BTL-4 Compact" news item.
//
// Launches, all on the caller's stream, no host read-back (T > 4; the
// decode path for T <= 4 is described further down):
//  1. top-k per token (descending fp32 logit, ties to the lower expert index)
//     and the softmax over the k selected logits, one wave per token.
//  2. route: per-expert counts and offsets, one record per active expert and
//     the expert-major route list (one workgroup; for T <= 8 the same
//     workgroup does step 1 first, in one launch).
//  3. gate/up: one workgroup per (blocks of 16 intermediate columns, active
//     expert); both products share every activation operand; SwiGLU in fp32;
//     the result is stored as an fp32 row per route. Where H is a multiple
//     of 512 (up to 8192) on the fp8 x fp4 matrix cores with the routes as
//     fixed-point digit rows (k_moe_gateup_f4, f4.h), else on fp16 tiles.
//  4. down: one workgroup per (4 blocks of 16 hidden columns, active expert);
//     stages the fp32 rows as scaled fp16 hi/lo pieces (WaveStageF32) and
//     writes the route's fp32 output.
//  5. combine: y_t = sum over slots j, in slot order, of w_tj * out(t, j).
#include <type_traits>

#include "dec_core.h"
#include "f4.h"
#include "kernels.h"

namespace brq {

constexpr int MOE_MAX_E = 1024;
constexpr int MOE_MAX_T = 256;
constexpr int MOE_MAX_R = MOE_MAX_T * 16;

struct MoeWs {
  int* ids;          // [T][k]
  float* wts;        // [T][k]
  int* off;          // [E+1]
  int4* blk;         // [E] (expert, first route, routes, 0) of the a-th active expert; zeros after the last
  int* route_tok;    // [R] token of each expert-major route position
  int* route_pos;    // [T][k] expert-major position of route (t, j)
  float* ap;         // [R][I] fp32 SwiGLU output (staged by the down launch as scaled pieces)
  float* o;          // [R][H]
};

static MoeWs moe_carve(void* ws, int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  MoeWs w;
  char* p = reinterpret_cast<char*>(ws);
  const int64_t R = T * k;
  auto take = [&](size_t bytes) { char* q = p; p += align256(bytes); return q; };
  w.ids = reinterpret_cast<int*>(take((size_t)R * 4));
  w.wts = reinterpret_cast<float*>(take((size_t)R * 4));
  w.off = reinterpret_cast<int*>(take((size_t)(E + 1) * 4));
  w.blk = reinterpret_cast<int4*>(take((size_t)E * 16));
  w.route_tok = reinterpret_cast<int*>(take((size_t)R * 4));
  w.route_pos = reinterpret_cast<int*>(take((size_t)R * 4));
  w.ap = reinterpret_cast<float*>(take((size_t)R * I * 4));
  w.o = reinterpret_cast<float*>(take((size_t)R * H * 4));
  return w;
}

size_t moe_ws_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  const int64_t R = T * k;
  return 2 * align256((size_t)R * 4) + align256((size_t)(E + 1) * 4) + align256((size_t)E * 16) +
         2 * align256((size_t)R * 4) + align256((size_t)R * I * 4) + align256((size_t)R * H * 4);
}

// exclusive prefix sum over the block (blockDim.x <= 1024); returns the total
__device__ int block_exclusive_scan(int v, int* s_part, int& excl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) s_part[wave] = inc;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < nw; ++w) {
    const int p = s_part[w];
    if (w < wave) before += p;
    total += p;
  }
  excl = before + inc - v;
  __syncthreads();
  return total;
}

// ---- wave-level top-k -------------------------------------------------------
// A routing candidate is a 64-bit key: the fp32 logit mapped to an unsigned
// integer of the same order in the high word, the complement of the expert
// index in the low word. The largest key is the largest logit and, among equal
// logits, the lower expert index. -0 is folded to +0 first so that the two
// zeros tie as they do in a plain fp32 comparison. Key 0 marks "no candidate".
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  v = (v == 0.f) ? 0.f : v;
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(~(uint32_t)e);
}
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)(~(uint32_t)key); }

// DPP move of a 64-bit value (lanes without a source, or outside ROWMASK, read 0)
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWMASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWMASK, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Largest key of the wave, returned to every lane: quad swaps, half-row and row
// mirrors, then the row broadcasts carry the maximum to lane 63.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  v = max64(v, dpp64<0xB1, 0xf>(v));   // quad_perm [1,0,3,2]
  v = max64(v, dpp64<0x4E, 0xf>(v));   // quad_perm [2,3,0,1]
  v = max64(v, dpp64<0x141, 0xf>(v));  // row_half_mirror
  v = max64(v, dpp64<0x140, 0xf>(v));  // row_mirror
  v = max64(v, dpp64<0x142, 0xa>(v));  // row_bcast15 into rows 1 and 3
  v = max64(v, dpp64<0x143, 0xc>(v));  // row_bcast31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Sum over lanes 0..15 (row 0), returned to every lane.
__device__ __forceinline__ float row0_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
}

// Top-k routing of one token by one wave: the k largest keys in descending
// order (k <= 16), then the softmax over the selected logits. Lane j < k
// returns slot j's expert and weight.
template <int PER>
__device__ __forceinline__ void wave_route(const float* __restrict__ lg, int E, int k, int& id, float& wt) {
  const int lane = threadIdx.x & 63;
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(lg[e], e) : 0ull;
  }
  float sel = 0.f, top = 0.f;
  id = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t m = key[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) m = max64(m, key[i]);
    const uint64_t w = wave_max_key(m);
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = (key[i] == w) ? 0ull : key[i];
    if (j == 0) top = key_logit(w);
    if (lane == j) { sel = key_logit(w); id = key_expert(w); }
  }
  const float ex = lane < k ? expf(sel - top) : 0.f;
  wt = ex / row0_sum(ex);
}

// Top-k of every token, one wave per token, four tokens per workgroup.
__global__ __launch_bounds__(256) void k_moe_topk(const float* __restrict__ logits, int T, int E, int k, MoeWs ws,
                                                  int32_t* __restrict__ ids_user, float* __restrict__ w_user) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int id;
  float w;
  if (E <= 256) wave_route<4>(logits + (size_t)t * E, E, k, id, w);
  else wave_route<16>(logits + (size_t)t * E, E, k, id, w);
  if (lane < k) {
    ws.ids[t * k + lane] = id;
    ws.wts[t * k + lane] = w;
    if (ids_user) ids_user[t * k + lane] = id;
    if (w_user) w_user[t * k + lane] = w;
  }
}

// One workgroup of 1024 threads builds the expert-major lists from the ids.
// Routes of one expert are ordered by token (slots of one token name distinct
// experts): the rank of route (t, j) inside its expert is the number of earlier
// tokens in the expert's token bitmap. TOPK: the workgroup's sixteen waves
// first route the tokens themselves (T <= MOE_ROUTE_T, one token per wave, as
// k_moe_topk does), so that routing and lists take one launch.
constexpr int MOE_ROUTE_T = 8;
template <bool TOPK>
__global__ __launch_bounds__(1024) void k_moe_route(const float* __restrict__ logits, int T, int E, int k, MoeWs ws,
                                                    int32_t* __restrict__ ids_user, float* __restrict__ w_user) {
  __shared__ int s_ids[MOE_MAX_R];
  __shared__ int s_cnt[MOE_MAX_E];
  __shared__ int s_off[MOE_MAX_E];
  __shared__ unsigned long long s_map[MOE_MAX_E * (MOE_MAX_T / 64)];
  __shared__ int s_part[16];
  const int tid = threadIdx.x;
  const int words = (T + 63) >> 6;
  if constexpr (TOPK) {
    const int lane = tid & 63, t = tid >> 6;
    if (t < T) {
      int id;
      float w;
      if (E <= 256) wave_route<4>(logits + (size_t)t * E, E, k, id, w);
      else wave_route<16>(logits + (size_t)t * E, E, k, id, w);
      if (lane < k) {
        s_ids[t * k + lane] = id;
        ws.ids[t * k + lane] = id;
        ws.wts[t * k + lane] = w;
        if (ids_user) ids_user[t * k + lane] = id;
        if (w_user) w_user[t * k + lane] = w;
      }
    }
  }
  for (int e = tid; e < E; e += blockDim.x) {
    s_cnt[e] = 0;
    for (int q = 0; q < words; ++q) s_map[e * words + q] = 0ull;
  }
  __syncthreads();
  for (int r = tid; r < T * k; r += blockDim.x) {
    const int t = r / k;
    int id;
    if constexpr (TOPK) {
      id = s_ids[r];
    } else {
      id = ws.ids[r];
      s_ids[r] = id;
    }
    atomicAdd(&s_cnt[id], 1);
    atomicOr(&s_map[id * words + (t >> 6)], 1ull << (t & 63));
  }
  __syncthreads();
  // offsets (exclusive scan of counts) and the ascending list of active experts
  int cnt = 0, off = 0, aidx = 0;
  if (tid < E) cnt = s_cnt[tid];
  const int R = block_exclusive_scan(cnt, s_part, off);
  const int na = block_exclusive_scan(cnt > 0 ? 1 : 0, s_part, aidx);
  if (tid < E) {
    s_off[tid] = off;
    ws.off[tid] = off;
    // one 16-byte record per active expert, so that a gate/up or down
    // workgroup learns its expert, routes and count in one load
    if (cnt > 0) ws.blk[aidx] = make_int4(tid, off, cnt, 0);
    if (tid >= na) ws.blk[tid] = make_int4(0, 0, 0, 0);
  }
  if (tid == 0) ws.off[E] = R;
  __syncthreads();
  for (int r = tid; r < T * k; r += blockDim.x) {
    const int e = s_ids[r], t = r / k;
    int rank = 0;
    for (int q = 0; q < (t >> 6); ++q) rank += __popcll(s_map[e * words + q]);
    rank += __popcll(s_map[e * words + (t >> 6)] & ((1ull << (t & 63)) - 1ull));
    const int pos = s_off[e] + rank;
    ws.route_tok[pos] = t;
    ws.route_pos[r] = pos;
  }
}

// top-k and expert-major lists: one launch for up to MOE_ROUTE_T tokens,
// else a wave per token in k_moe_topk and the lists in a second launch
static void moe_route(const float* logits, int T, int E, int k, const MoeWs& ws, int32_t* ids, float* w,
                      hipStream_t st) {
  if (T <= MOE_ROUTE_T) {
    hipLaunchKernelGGL(k_moe_route<true>, dim3(1), dim3(1024), 0, st, logits, T, E, k, ws, ids, w);
  } else {
    hipLaunchKernelGGL(k_moe_topk, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E, k, ws, ids, w);
    hipLaunchKernelGGL(k_moe_route<false>, dim3(1), dim3(1024), 0, st, nullptr, T, E, k, ws, nullptr, nullptr);
  }
}

// The sign and scale words look invariant across the token tiles of a
// workgroup; an empty asm that "rewrites" them per tile keeps the compiler
// from hoisting every block's weight operands out of the tile loop (CB x 16 x
// 4 registers) and from waiting for the words before the first tile's
// activation loads are issued.
template <int NB, int CPW>
__device__ __forceinline__ void pin_signs(BPre<NB, CPW>& bp) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      asm volatile("" : "+v"(bp.d[nb][c].x), "+v"(bp.d[nb][c].y), "+v"(bp.d[nb][c].z), "+v"(bp.d[nb][c].w),
                   "+v"(bp.s[nb][c]));
}

// reduce_waves over CB column blocks of NB accumulators each (wave order)
template <int CB, int NB>
__device__ __forceinline__ void reduce_waves_cb(f32x4 (&acc)[CB][NB][1], f32x4* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (nw == 1) return;
  if (wave > 0) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[(((wave - 1) * CB + cb) * NB + nb) * 64 + lane] = acc[cb][nb][0];
  }
  __syncthreads();
  if (wave == 0) {
    for (int w = 1; w < nw; ++w)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[cb][nb][0] += red[(((w - 1) * CB + cb) * NB + nb) * 64 + lane];
  }
}

// gate/up: one workgroup per (CB blocks of 16 intermediate columns, active
// expert). The sign words of all CB blocks are loaded first; the expert's
// tokens are staged once per tile of up to tile_rows tokens (each wave its own
// K-slice, bf16 -> permuted scaled fp16) and multiplied by every block, so a
// workgroup keeps CB blocks' loads in flight and pays one staging per tile.
// The tile body is specialised by the expert's count (1/2/4/8/16 staged rows,
// section 7 item 1 of the DBF post: kernels chosen by the observed per-expert
// counts), picked per workgroup at run time.
template <int CPW, int MAXR, int CB>
__global__ __launch_bounds__(512) void k_moe_gateup(const uint16_t* __restrict__ x, int H, int I,
                                                    const uint4* __restrict__ gs, const uint16_t* __restrict__ gsc,
                                                    const uint4* __restrict__ us, const uint16_t* __restrict__ usc,
                                                    MoeWs ws) {
  extern __shared__ uint4 smem[];
  const int4 bk = ws.blk[blockIdx.y];
  const int e = bk.x, r0 = bk.y, cnt = bk.z;
  if (cnt == 0) return;  // past the last active expert
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15;
  const int G = H >> 7, nchunks = (G + 3) >> 2;
  const int c0 = wave * CPW;
  BPre<2, CPW> bp[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = (blockIdx.x * CB + cb) * 16 + j;
    const size_t row = (size_t)e * I + (n < I ? n : 0);
    const uint4* wsig[2] = {gs + row * G, us + row * G};
    const uint16_t* wsc[2] = {gsc + row * G, usc + row * G};
    const bool rok[2] = {n < I, n < I};
    // unconditional (indices clamped): a conditional prefetch makes the
    // compiler wait for each block's words before issuing the next block's
    b_prefetch<BM_GROUP, 2, CPW>(wsig, wsc, rok, G, c0, 1, bp[cb]);
  }
  // one tile of up to MAXR tokens; the first is peeled off the loop so that
  // its activation loads issue while the sign words are still in flight
  auto run_tile = [&](const int tb) {
    const int rows = (cnt - tb) < MAXR ? (cnt - tb) : MAXR;
    f32x4 acc[CB][2][1];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb][0][0] = acc[cb][1][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    // stage and multiply `rows` tokens with SR staged row slots (SR >= rows)
    auto tile = [&](auto sr) {
      constexpr int SR = decltype(sr)::value;
      uint4* xw = smem + (size_t)wave * CPW * SR * 64;
      WaveStage<ST_BF16, CPW, SR> sx;
      if (c0 < nchunks) {
        sx.load(rows, H, c0, [&](int rr) { return x + (size_t)ws.route_tok[r0 + tb + rr] * H; });
        sx.store(xw);
      }
      __syncthreads();
      if (c0 < nchunks) {
        const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
        auto aop = [&](int, int g, int i) -> u32x4 {
          const int m = min(j, rows - 1);
          return xs[(((g >> 2) - c0) * SR + m) * 64 + (g & 3) * 16 + i];
        };
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          pin_signs(bp[cb]);
          b_compute<BM_GROUP, 2, 1, CPW>(bp[cb], nullptr, G, c0, 1, aop, acc[cb]);
        }
        // back from the rows' staging scales (exact powers of two)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int u = sx.unscale(i);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            acc[cb][0][0][i] = __builtin_amdgcn_ldexpf(acc[cb][0][0][i], u);
            acc[cb][1][0][i] = __builtin_amdgcn_ldexpf(acc[cb][1][0][i], u);
          }
        }
      }
    };
    // the staged row slots follow the expert's count: 1, 2, 4, 8 or MAXR rows
    // (each variant stages, converts and unscales only the rows it holds)
    if (rows <= 1) tile(std::integral_constant<int, 1>{});
    else if (MAXR > 2 && rows <= 2) tile(std::integral_constant<int, (MAXR > 2 ? 2 : MAXR)>{});
    else if (MAXR > 4 && rows <= 4) tile(std::integral_constant<int, (MAXR > 4 ? 4 : MAXR)>{});
    else if (MAXR > 8 && rows <= 8) tile(std::integral_constant<int, (MAXR > 8 ? 8 : MAXR)>{});
    else tile(std::integral_constant<int, MAXR>{});
    __syncthreads();
    reduce_waves_cb<CB, 2>(acc, reinterpret_cast<f32x4*>(smem));
    if (wave == 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int n = (blockIdx.x * CB + cb) * 16 + j;
        if (n >= I) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int p = 4 * (lane >> 4) + i;
          if (p < rows) {
            const float g = acc[cb][0][0][i], u = acc[cb][1][0][i];
            ws.ap[(size_t)(r0 + tb + p) * I + n] = g / (1.0f + expf(-g)) * u;
          }
        }
      }
    }
    __syncthreads();
  };
  run_tile(0);  // an active expert has at least one route
  for (int tb = MAXR; tb < cnt; tb += MAXR) run_tile(tb);
  (void)nw;
}

// gate/up on the fp8 x fp4 matrix cores (grouped path, H % 512 == 0): the
// expert's token rows as fixed-point digit rows (f4.h), two routes per
// product (digit rows 0..5 and 8..13, the zero row for the others), the +-1
// weights as +-6 fp4 operands built by one shift-or per eight weights. One
// workgroup per (NT blocks of 16 intermediate columns, active expert), one
// 512-wide chunk of the hidden vector per wave (CPW per wave beyond 8
// chunks); the routes are taken in pairs, each pair's digits rebuilt in the
// wave's LDS region chunk by chunk; the waves' sums meet in LDS in wave
// order, and SwiGLU (fp32) writes the routes' intermediate rows.
constexpr int MOE_F4_ROWS = 13;  // digit rows of a route pair, then the zero row
constexpr int MOE_F4_GROUP = MOE_F4_ROWS * 128;
constexpr int MOE_F4_CHUNK = 4 * MOE_F4_GROUP;

template <int CPW, int NT>
__global__ __launch_bounds__(512) void k_moe_gateup_f4(const uint16_t* __restrict__ x, int H, int I,
                                                       const uint4* __restrict__ gs, const uint16_t* __restrict__ gsc,
                                                       const uint4* __restrict__ us, const uint16_t* __restrict__ usc,
                                                       MoeWs ws) {
  extern __shared__ uint4 smem[];
  const int4 bk = ws.blk[blockIdx.y];
  const int e = bk.x, r0 = bk.y, cnt = bk.z;
  if (cnt == 0) return;  // past the last active expert
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int G = H >> 7, nchunks = G >> 2;
  const int c0 = wave * CPW;
  uint8_t* xw = reinterpret_cast<uint8_t*>(smem) + (size_t)wave * MOE_F4_CHUNK;
  float* red = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem) + (size_t)nw * MOE_F4_CHUNK);
  // the first pair's token rows, then every weight word, all before any wait
  auto load_x = [&](int q0, uint4 (&xv)[2][CPW]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rr = q0 + h < cnt ? q0 + h : cnt - 1;  // a missing second route: zeroed below
      const uint16_t* xr = x + (size_t)ws.route_tok[r0 + rr] * H;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int k0 = (c0 + c) * 512 + 8 * lane;
        xv[h][c] = *reinterpret_cast<const uint4*>(xr + (k0 < H ? k0 : 0));
      }
    }
  };
  uint4 xv[2][CPW];
  load_x(0, xv);
  uint4 sg[2][NT][CPW];
  uint2 sc[2][NT][CPW];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = (blockIdx.x * NT + t) * 16 + j;
    const size_t row = ((size_t)e * I + (n < I ? n : 0)) * G;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int g = 4 * (c0 + c) + kb, g4 = 4 * (c0 + c);
      sg[0][t][c] = gs[row + (g < G ? g : 0)];
      sg[1][t][c] = us[row + (g < G ? g : 0)];
      sc[0][t][c] = *reinterpret_cast<const uint2*>(gsc + row + (g4 < G ? g4 : 0));
      sc[1][t][c] = *reinterpret_cast<const uint2*>(usc + row + (g4 < G ? g4 : 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (lane < 32)  // the zero row of each group: 16 bytes per lane, never overwritten
    *reinterpret_cast<uint4*>(xw + (lane >> 3) * MOE_F4_GROUP + 12 * 128 + 16 * (lane & 7)) =
        make_uint4(0u, 0u, 0u, 0u);
  // MFMA row j reads digit row j of the pair's first route (j < 6), digit row
  // j - 8 of its second (8 <= j < 14, LDS rows 6..11) or the zero row
  const int prow = j < 6 ? j : (j >= 8 && j < 14) ? j - 2 : 12;
  uint8_t* base = xw + (lane >> 4) * MOE_F4_GROUP + 32 * ((lane & 15) >> 2) + 2 * (lane & 3);
  for (int q0 = 0; q0 < cnt; q0 += 2) {
    if (q0 > 0) load_x(q0, xv);
    // slots past the last chunk, and a missing second route, hold zeros
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        if (c0 + c >= nchunks || q0 + h >= cnt) xv[h][c] = make_uint4(0u, 0u, 0u, 0u);
    float S0, S1;
    const uint32_t e0 = f4_slice_exponent<CPW>(xv[0], S0), e1 = f4_slice_exponent<CPW>(xv[1], S1);
    // the zero row (prow 12) takes scale 2^0 (ebs - 26 is the E8M0 NaN code at ebs = 25)
    const int sa = prow == 12 ? 127 : j < 8 ? (int)e0 - 2 - 4 * j : (int)e1 - 2 - 4 * (j - 8);
    float acc[2][NT];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][t] = 0.f;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if (c0 + c >= nchunks) break;  // uniform across the wave
      f4_digits(xv[0][c], S0, base, 0);
      f4_digits(xv[1][c], S1, base, 6);
      const uint8_t* ab = xw + prow * 128 + 16 * kb;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          uint32_t w0 = sg[m][t][c].x, w1 = sg[m][t][c].y, w2 = sg[m][t][c].z, w3 = sg[m][t][c].w;
          f4_transpose4(w0, w1, w2, w3);
          const uint32_t wi[4] = {w0, w1, w2, w3};
          const uint32_t s4[4] = {sc[m][t][c].x & 0xffffu, sc[m][t][c].x >> 16, sc[m][t][c].y & 0xffffu,
                                  sc[m][t][c].y >> 16};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 d = f4_group_mfma(ab + i * MOE_F4_GROUP, wi[i], sa);
            acc[m][t] = fmaf(f16_bits_to_f32(s4[i]), (d[0] + d[1]) + (d[2] + d[3]), acc[m][t]);
          }
        }
    }
    // digit rows 4 and 5 join rows 0..3: lanes 0..15 hold the first route's
    // sums, lanes 32..47 the second's
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][t] += __shfl_down(acc[m][t], 16, 64);
    const bool holds = (kb & 1) == 0;
    if (wave > 0 && holds) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[(((wave - 1) * 2 + m) * NT + t) * 32 + (kb >> 1) * 16 + j] = acc[m][t];
    }
    __syncthreads();
    if (wave == 0 && holds) {
      const int p = q0 + (kb >> 1);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float v[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          v[m] = acc[m][t];
          for (int w = 1; w < nw; ++w) v[m] += red[(((w - 1) * 2 + m) * NT + t) * 32 + (kb >> 1) * 16 + j];
          v[m] = v[m] / 6.0f;
        }
        const int n = (blockIdx.x * NT + t) * 16 + j;
        if (p < cnt && n < I) ws.ap[(size_t)(r0 + p) * I + n] = v[0] / (1.0f + expf(-v[0])) * v[1];
      }
    }
    __syncthreads();  // red and the digit regions are free for the next pair
  }
}

// down: one workgroup per (CB blocks of 16 hidden columns, active expert); the
// routes' fp32 intermediates are staged per wave as scaled fp16 hi/lo pieces
// (WaveStageF32), up to 8 routes (16 piece rows) a tile, and multiplied by
// every block; each wave scales its partials back before the waves meet.
template <int CPW, int CB, int RT>
__global__ __launch_bounds__(512) void k_moe_down(int H, int I, const uint4* __restrict__ ds,
                                                  const uint16_t* __restrict__ dsc, MoeWs ws) {
  extern __shared__ uint4 smem[];
  const int4 bk = ws.blk[blockIdx.y];
  const int e = bk.x, r0 = bk.y, cnt = bk.z;
  if (cnt == 0) return;  // past the last active expert
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int G = I >> 7, nchunks = (G + 3) >> 2;
  const int c0 = wave * CPW;
  BPre<1, CPW> bp[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = (blockIdx.x * CB + cb) * 16 + j;
    const size_t row = (size_t)e * H + (n < H ? n : 0);
    const uint4* wsig[1] = {ds + row * G};
    const uint16_t* wsc[1] = {dsc + row * G};
    const bool rok[1] = {n < H};
    b_prefetch<BM_GROUP, 1, CPW>(wsig, wsc, rok, G, c0, 1, bp[cb]);  // unconditional, as in gate/up
  }
  // one tile of up to RT routes; the first is peeled off the loop (as in gate/up)
  auto run_tile = [&](const int tb) {
    const int routes = (cnt - tb) < RT ? (cnt - tb) : RT;
    const int rows = 2 * routes;
    f32x4 acc[CB][1][1];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb][0][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    // stage and multiply the `rows` piece rows with SR staged slots (SR >= rows)
    auto tile = [&](auto sr) {
      constexpr int SR = decltype(sr)::value;
      uint4* xw = smem + (size_t)wave * CPW * SR * 64;
      WaveStageF32<CPW, SR / 2> sa;
      if (c0 < nchunks) {
        sa.load(routes, I, c0, [&](int m) { return ws.ap + (size_t)(r0 + tb + m) * I; });
        sa.store(xw);
      }
      __syncthreads();
      if (c0 < nchunks) {
        const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
        auto aop = [&](int, int g, int i) -> u32x4 {
          const int pr = min(j, rows - 1);
          return xs[(((g >> 2) - c0) * SR + pr) * 64 + (g & 3) * 16 + i];
        };
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          pin_signs(bp[cb]);
          b_compute<BM_GROUP, 1, 1, CPW>(bp[cb], nullptr, G, c0, 1, aop, acc[cb]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int us = sa.unscale(i);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[cb][0][0][i] = __builtin_amdgcn_ldexpf(acc[cb][0][0][i], us);
        }
      }
    };
    if (rows <= 4) tile(std::integral_constant<int, 4>{});
    else if (RT <= 4 || rows <= 8) tile(std::integral_constant<int, 8>{});
    else tile(std::integral_constant<int, 16>{});
    __syncthreads();
    reduce_waves_cb<CB, 1>(acc, reinterpret_cast<f32x4*>(smem));
    if (wave == 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int n = (blockIdx.x * CB + cb) * 16 + j;
        if (n >= H) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int q = 2 * (lane >> 4) + h;
          if (q < routes) ws.o[(size_t)(r0 + tb + q) * H + n] = acc[cb][0][0][2 * h] + acc[cb][0][0][2 * h + 1];
        }
      }
    }
    __syncthreads();
  };
  run_tile(0);
  for (int tb = RT; tb < cnt; tb += RT) run_tile(tb);
}

// One thread per 4 consecutive hidden columns of a token: the slots' positions
// and weights are loaded first (k <= 16, unrolled), then one 16-byte load per
// slot; y = sum over j in slot order of w_tj * out(t, j), one fma per slot.
__global__ __launch_bounds__(256) void k_moe_combine(int T, int H, int k, MoeWs ws, void* __restrict__ y,
                                                     int y_bf16) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int h4 = H >> 2;
  if (q >= (int64_t)T * h4) return;
  const int t = (int)(q / h4), n = 4 * (int)(q % h4);
  int pos[16];
  float wt[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int jj = j < k ? j : 0;  // clamped, unconditional loads
    pos[j] = ws.route_pos[t * k + jj];
    wt[j] = ws.wts[t * k + jj];
  }
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= k) break;
    const f32x4 o = *reinterpret_cast<const f32x4*>(ws.o + (size_t)pos[j] * H + n);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(wt[j], o[i], acc[i]);
  }
  const size_t base = (size_t)t * H + n;
  if (y_bf16) {
    uint2 b;
    b.x = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
    b.y = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + base) = b;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(y) + base) = acc;
  }
}

// ---- decode path (few tokens): two launches --------------------------------
//  A: every workgroup routes all T tokens itself (one wave per token), finds
//     the a-th active expert (ascending ids) and its routes, and runs gate/up +
//     SwiGLU for them; the result of route r = t*k + j is stored at piece rows
//     2r, 2r+1 (token-major). Workgroup (0, 0) also publishes ids and weights.
//  B: one workgroup per (16 hidden columns, token), one wave per slot: wave j
//     multiplies expert ids[t][j]'s down rows by route (t, j)'s intermediate;
//     wave 0 adds w_tj * out_j over the slots in slot order.
constexpr int MOE_SMALL_T = 4;
// 16-column blocks per gate/up (down) workgroup: fewer where each wave holds
// more chunks of sign words, so that the prefetched words stay in registers
constexpr int moe_cb_gu(int cpw) { return cpw == 1 ? 4 : cpw == 2 ? 2 : 1; }
constexpr int moe_cb_dn(int cpw) { return cpw == 1 ? 4 : cpw == 2 ? 2 : 1; }

// The want-th distinct expert (ascending id) among the R = T*k <= 64 routes
// in s_ids, and its routes in ascending (token, slot) order, by one wave with
// no serial loop: lane q holds route q; a distinct expert's rank is the
// number of set bits of s_bits (the routed experts) below its id, from an
// exclusive prefix of the words' bit counts (lane w holding word w, E/32 <= 32
// words). Lane 0 writes the expert (-1 if fewer than want+1 are routed) and
// its route count.
__device__ __forceinline__ void route_pick(const int* s_ids, const uint32_t* s_bits, int R, int E, int k, int want,
                                           int* s_tok, int* s_slot, int& s_e, int& s_cnt) {
  const int lane = threadIdx.x & 63;
  const uint32_t bw = lane < ((E + 31) >> 5) ? s_bits[lane] : 0u;
  int inc = __popc(bw);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  const int excl = inc - __popc(bw);
  const int id = lane < R ? s_ids[lane] : 0;
  const int before = __shfl(excl, id >> 5, 64);
  const uint32_t word = (uint32_t)__shfl((int)bw, id >> 5, 64);
  const int rank = before + __popc(word & ((1u << (id & 31)) - 1u));
  const bool mine = lane < R && rank == want;
  const uint64_t bm = __ballot(mine);
  const int cnt = __popcll(bm);
  const int e = cnt ? __shfl(id, __ffsll((unsigned long long)bm) - 1, 64) : -1;
  if (mine) {
    const int pos = __popcll(bm & ((1ull << lane) - 1ull));
    const int t = lane / k;
    s_tok[pos] = t;
    s_slot[pos] = lane - t * k;
  }
  if (lane == 0) {
    s_e = e;
    s_cnt = cnt;
  }
}

template <int CPW, int MAXR>
__global__ __launch_bounds__(512) void k_moe_a_small(const uint16_t* __restrict__ x, const float* __restrict__ logits,
                                                     int T, int E, int k, int H, int I,
                                                     const uint4* __restrict__ gs, const uint16_t* __restrict__ gsc,
                                                     const uint4* __restrict__ us, const uint16_t* __restrict__ usc,
                                                     MoeWs ws, int32_t* __restrict__ ids_user,
                                                     float* __restrict__ w_user) {
  extern __shared__ uint4 smem[];
  __shared__ int s_ids[MOE_SMALL_T * 16];
  __shared__ float s_w[MOE_SMALL_T * 16];
  __shared__ uint32_t s_bits[MOE_MAX_E / 32];
  __shared__ int s_tok[MOE_SMALL_T], s_slot[MOE_SMALL_T];
  __shared__ int s_e, s_cnt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  for (int i = tid; i < MOE_MAX_E / 32; i += blockDim.x) s_bits[i] = 0u;
  for (int t = wave; t < T; t += nw) {
    int id;
    float w;
    if (E <= 256) wave_route<4>(logits + (size_t)t * E, E, k, id, w);
    else wave_route<16>(logits + (size_t)t * E, E, k, id, w);
    if (lane < k) {
      s_ids[t * k + lane] = id;
      s_w[t * k + lane] = w;
    }
  }
  __syncthreads();
  for (int r = tid; r < T * k; r += blockDim.x) atomicOr(&s_bits[s_ids[r] >> 5], 1u << (s_ids[r] & 31));
  __syncthreads();
  if (wave == 0) route_pick(s_ids, s_bits, T * k, E, k, blockIdx.y, s_tok, s_slot, s_e, s_cnt);
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int r = tid; r < T * k; r += blockDim.x) {
      ws.ids[r] = s_ids[r];
      ws.wts[r] = s_w[r];
      if (ids_user) ids_user[r] = s_ids[r];
      if (w_user) w_user[r] = s_w[r];
    }
  }
  __syncthreads();
  const int e = s_e, cnt = s_cnt;
  if (e < 0) return;
  const int j = lane & 15, kb = lane >> 4;
  const int n = blockIdx.x * 16 + j;
  const int G = H >> 7, nchunks = (G + 3) >> 2;
  const int c0 = wave * CPW;
  const bool rok = n < I;
  const size_t row = (size_t)e * I + (rok ? n : 0);
  const uint4* wsig[2] = {gs + row * G, us + row * G};
  const uint16_t* wsc[2] = {gsc + row * G, usc + row * G};
  const bool rk[2] = {rok, rok};
  uint4* xw = smem + (size_t)wave * CPW * MAXR * 64;
  f32x4* red = reinterpret_cast<f32x4*>(smem + (size_t)nw * CPW * MAXR * 64);
  f32x4 acc[2][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}, {f32x4{0.f, 0.f, 0.f, 0.f}}};
  if (c0 < nchunks) {
    WaveStage<ST_BF16, CPW, MAXR> sx;
    sx.load(cnt, H, c0, [&](int q) { return x + (size_t)s_tok[q] * H; });
    BPre<2, CPW> bp;
    b_prefetch<BM_GROUP, 2, CPW>(wsig, wsc, rk, G, c0, 1, bp);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    sx.store(xw);
    const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
    auto aop = [&](int, int g, int i) -> u32x4 {
      const int m = min(j, cnt - 1);
      return xs[(((g >> 2) - c0) * MAXR + m) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_GROUP, 2, 1, CPW, true>(bp, nullptr, G, c0, 1, aop, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[0][0][i] = __builtin_amdgcn_ldexpf(acc[0][0][i], sx.unscale(i));
      acc[1][0][i] = __builtin_amdgcn_ldexpf(acc[1][0][i], sx.unscale(i));
    }
  }
  const bool holds = 4 * kb < cnt;
  if (wave > 0 && holds) {
    red[(2 * (wave - 1)) * 64 + lane] = acc[0][0];
    red[(2 * (wave - 1) + 1) * 64 + lane] = acc[1][0];
  }
  __syncthreads();
  if (wave != 0 || !holds || !rok) return;
  for (int w = 1; w < nw; ++w) {
    acc[0][0] += red[(2 * (w - 1)) * 64 + lane];
    acc[1][0] += red[(2 * (w - 1) + 1) * 64 + lane];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 4 * kb + i;
    if (q < cnt) {
      const float g = acc[0][0][i], u = acc[1][0][i];
      ws.ap[((size_t)s_tok[q] * k + s_slot[q]) * I + n] = g / (1.0f + expf(-g)) * u;
    }
  }
}

template <int CPW>
__global__ __launch_bounds__(1024) void k_moe_b_token(int H, int I, int k, const uint4* __restrict__ ds,
                                                      const uint16_t* __restrict__ dsc, MoeWs ws,
                                                      void* __restrict__ y, int y_bf16) {
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, slot = threadIdx.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int t = blockIdx.y;
  const int n = blockIdx.x * 16 + j;
  const int r = t * k + slot;
  const int e = ws.ids[r];
  const int G = I >> 7;
  const bool rok = n < H;
  const size_t row = (size_t)e * H + (rok ? n : 0);
  const uint4* wsig[1] = {ds + row * G};
  const uint16_t* wsc[1] = {dsc + row * G};
  const bool rk[1] = {rok};
  uint4* xw = smem + (size_t)slot * CPW * 2 * 64;
  float* part = reinterpret_cast<float*>(smem + (size_t)k * CPW * 2 * 64);  // [k][16]
  f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
  WaveStageF32<CPW, 1> sa;  // the route's fp32 row as two scaled piece rows
  {
    sa.load(1, I, 0, [&](int) { return ws.ap + (size_t)r * I; });
    BPre<1, CPW> bp;
    b_prefetch<BM_GROUP, 1, CPW>(wsig, wsc, rk, G, 0, 1, bp);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    sa.store(xw);
    const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
    auto aop = [&](int, int g, int i) -> u32x4 {
      const int p = min(j, 1);
      return xs[((g >> 2) * 2 + p) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_GROUP, 1, 1, CPW, true>(bp, nullptr, G, 0, 1, aop, acc);
  }
  // lanes 0..15 hold piece rows 0 and 1 of column j
  if (kb == 0) part[slot * 16 + j] = __builtin_amdgcn_ldexpf(acc[0][0][0] + acc[0][0][1], sa.unscale(0));
  __syncthreads();
  if (slot != 0 || kb != 0 || !rok) return;
  float sum = 0.f;
  for (int q = 0; q < k; ++q) sum = fmaf(ws.wts[t * k + q], part[q * 16 + j], sum);
  store_out(y, (size_t)t * H + n, sum, y_bf16);
}

// The decode path in one launch (the persistent gate/up -> SwiGLU -> down
// kernel of section 7 of the DBF post): every workgroup routes the T <= 4
// tokens itself; workgroup (x, a) then does the gate/up work of
// k_moe_a_small's workgroup (x, a) and, after a grid-wide wait, workgroup
// number b = a * gridDim.x + x < (H/16) * T does the down work of
// k_moe_b_token's workgroup (b % (H/16), b / (H/16)). The down weight words
// are loaded right after routing, before the gate/up products, so the second
// half issues no weight load after the wait. Arithmetic and sum orders are
// those of the two-launch path (the same bits); the SwiGLU rows cross the
// wait through the coherence point (gsync.h). WA waves do gate/up, k waves
// (one per slot) do down.
template <int CPW, int MAXR, int CPWB>
__global__ __launch_bounds__(1024) void k_moe_fused_small(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ logits, int T, int E, int k,
                                                          int H, int I, int WA, const uint4* __restrict__ gs,
                                                          const uint16_t* __restrict__ gsc,
                                                          const uint4* __restrict__ us,
                                                          const uint16_t* __restrict__ usc,
                                                          const uint4* __restrict__ ds,
                                                          const uint16_t* __restrict__ dsc, MoeWs ws,
                                                          int32_t* __restrict__ ids_user, float* __restrict__ w_user,
                                                          void* __restrict__ y, int y_bf16, uint32_t* __restrict__ slot,
                                                          uint32_t spin) {
  extern __shared__ uint4 smem[];
  __shared__ int s_ids[MOE_SMALL_T * 16];
  __shared__ float s_w[MOE_SMALL_T * 16];
  __shared__ uint32_t s_bits[MOE_MAX_E / 32];
  __shared__ int s_tok[MOE_SMALL_T], s_slot[MOE_SMALL_T];
  __shared__ int s_e, s_cnt;
  const uint32_t epoch = grid_epoch(slot);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  // ---- routing of every token (as k_moe_a_small)
  for (int i = tid; i < MOE_MAX_E / 32; i += blockDim.x) s_bits[i] = 0u;
  for (int t = wave; t < T; t += nw) {
    int id;
    float w;
    if (E <= 256) wave_route<4>(logits + (size_t)t * E, E, k, id, w);
    else wave_route<16>(logits + (size_t)t * E, E, k, id, w);
    if (lane < k) {
      s_ids[t * k + lane] = id;
      s_w[t * k + lane] = w;
    }
  }
  __syncthreads();
  for (int q = tid; q < T * k; q += blockDim.x) atomicOr(&s_bits[s_ids[q] >> 5], 1u << (s_ids[q] & 31));
  __syncthreads();
  if (wave == 0) route_pick(s_ids, s_bits, T * k, E, k, blockIdx.y, s_tok, s_slot, s_e, s_cnt);
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int q = tid; q < T * k; q += blockDim.x) {
      if (ids_user) ids_user[q] = s_ids[q];
      if (w_user) w_user[q] = s_w[q];
    }
  }
  __syncthreads();
  // ---- down weight words of this workgroup's second half (wave = slot)
  const int HB = (H + 15) / 16;
  const int b2 = blockIdx.y * gridDim.x + blockIdx.x;
  const bool do2 = b2 < HB * T;  // uniform per workgroup
  const int t2 = do2 ? b2 / HB : 0;
  const int n2 = (b2 - t2 * HB) * 16 + j;
  const bool act2 = do2 && wave < k;  // uniform per wave
  const int GI = I >> 7;
  BPre<1, CPWB> bpd;
  if (act2) {
    const int e2 = s_ids[t2 * k + wave];
    const bool rok = n2 < H;
    const size_t row = (size_t)e2 * H + (rok ? n2 : 0);
    const uint4* wsig[1] = {ds + row * GI};
    const uint16_t* wsc[1] = {dsc + row * GI};
    const bool rk[1] = {rok};
    b_prefetch<BM_GROUP, 1, CPWB>(wsig, wsc, rk, GI, 0, 1, bpd);
  }
  // ---- gate/up of (16 intermediate columns, active expert), as k_moe_a_small
  const int e = s_e, cnt = s_cnt;
  const int n = blockIdx.x * 16 + j;
  const int G = H >> 7, nchunks = (G + 3) >> 2;
  const int c0 = wave * CPW;
  const bool rok = n < I;
  uint4* xw = smem + (size_t)wave * CPW * MAXR * 64;
  f32x4* red = reinterpret_cast<f32x4*>(smem + (size_t)WA * CPW * MAXR * 64);
  f32x4 acc[2][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}, {f32x4{0.f, 0.f, 0.f, 0.f}}};
  if (e >= 0 && wave < WA && c0 < nchunks) {
    const size_t row = (size_t)e * I + (rok ? n : 0);
    const uint4* wsig[2] = {gs + row * G, us + row * G};
    const uint16_t* wsc[2] = {gsc + row * G, usc + row * G};
    const bool rk[2] = {rok, rok};
    WaveStage<ST_BF16, CPW, MAXR> sx;
    sx.load(cnt, H, c0, [&](int q) { return x + (size_t)s_tok[q] * H; });
    BPre<2, CPW> bp;
    b_prefetch<BM_GROUP, 2, CPW>(wsig, wsc, rk, G, c0, 1, bp);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    sx.store(xw);
    const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
    auto aop = [&](int, int g, int i) -> u32x4 {
      const int m = min(j, cnt - 1);
      return xs[(((g >> 2) - c0) * MAXR + m) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_GROUP, 2, 1, CPW, true>(bp, nullptr, G, c0, 1, aop, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[0][0][i] = __builtin_amdgcn_ldexpf(acc[0][0][i], sx.unscale(i));
      acc[1][0][i] = __builtin_amdgcn_ldexpf(acc[1][0][i], sx.unscale(i));
    }
  }
  const bool holds = 4 * kb < cnt;
  if (e >= 0 && wave > 0 && wave < WA && holds) {
    red[(2 * (wave - 1)) * 64 + lane] = acc[0][0];
    red[(2 * (wave - 1) + 1) * 64 + lane] = acc[1][0];
  }
  __syncthreads();
  if (e >= 0 && wave == 0 && holds && rok) {
    for (int w = 1; w < WA; ++w) {
      acc[0][0] += red[(2 * (w - 1)) * 64 + lane];
      acc[1][0] += red[(2 * (w - 1) + 1) * 64 + lane];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 4 * kb + i;
      if (q < cnt) {
        const float g = acc[0][0][i], uu = acc[1][0][i];
        coh_storef(ws.ap + ((size_t)s_tok[q] * k + s_slot[q]) * I + n, g / (1.0f + expf(-g)) * uu);
      }
    }
  }
  // ---- every route's SwiGLU row is at the coherence point after this
  const bool ok = grid_wait(slot, epoch, spin);
  if (!do2) return;
  if (!ok) {
    if (wave == 0 && lane < 16 && n2 < H) store_out(y, (size_t)t2 * H + n2, __builtin_nanf(""), y_bf16);
    return;
  }
  // ---- down of (16 hidden columns, token t2), one wave per slot, as k_moe_b_token
  uint4* pw = smem + (size_t)wave * CPWB * 2 * 64;
  float* part = reinterpret_cast<float*>(smem + (size_t)k * CPWB * 2 * 64);  // [k][16]
  if (act2) {
    const int r2 = t2 * k + wave;
    f32x4 ad[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
    WaveStageF32<CPWB, 1> sa;
    sa.template load<true>(1, I, 0, [&](int) { return ws.ap + (size_t)r2 * I; });
    sa.store(pw);
    const u32x4* xs = reinterpret_cast<const u32x4*>(pw);
    auto aop = [&](int, int g, int i) -> u32x4 {
      const int p = min(j, 1);
      return xs[((g >> 2) * 2 + p) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_GROUP, 1, 1, CPWB, true>(bpd, nullptr, GI, 0, 1, aop, ad);
    if (kb == 0) part[wave * 16 + j] = __builtin_amdgcn_ldexpf(ad[0][0][0] + ad[0][0][1], sa.unscale(0));
  }
  __syncthreads();
  if (wave != 0 || kb != 0 || n2 >= H) return;
  float sum = 0.f;
  for (int q = 0; q < k; ++q) sum = fmaf(s_w[t2 * k + q], part[q * 16 + j], sum);
  store_out(y, (size_t)t2 * H + n2, sum, y_bf16);
}

// Single-launch layers: on when the caller asked for them (mode 2); by
// default (mode 0) off: two graph launches measured as fast or faster on this
// chip (the grid-wide wait costs about what the kernel boundary does).
static bool moe_fusion_wanted(int T) {
  (void)T;
  return fusion_mode() == 2;
}

// The decode path applies when the per-wave staging of both launches fits.
static bool moe_small_path(int T, int H, int I, int k, DecSplit& sa, int& maxr, int& cpwb) {
  if (T > MOE_SMALL_T) return false;
  maxr = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
  sa = dec_split(H / 128, 8);
  const int chunks_b = (I / 128 + 3) / 4;
  cpwb = chunks_b;
  if (chunks_b > 4) return false;
  if ((int64_t)sa.waves * sa.cpw * maxr * 1024 + (int64_t)(sa.waves - 1) * 2 * 64 * 16 > kDecLdsBytes) return false;
  return (int64_t)k * cpwb * 2 * 1024 + (int64_t)k * 16 * 4 <= kDecLdsBytes;
}

// token rows per gate/up tile: staged row slots per chunk, so that
// waves * cpw * slots KiB fit the staging budget; 4 when an expert expects at
// most 3 routes (T*k/E), which quarters the staging LDS and lets more
// workgroups share a compute unit
static int moe_tile_rows(const DecSplit& sp, int T, int E, int k) {
  const int64_t chunks = (int64_t)sp.waves * sp.cpw;
  const int r = chunks <= 4 ? 16 : chunks <= 16 ? 4 : 1;
  return (r > 4 && (int64_t)T * k <= 3 * (int64_t)E) ? 4 : r;
}

using MoeFusedFn = void (*)(const uint16_t*, const float*, int, int, int, int, int, int, const uint4*,
                           const uint16_t*, const uint4*, const uint16_t*, const uint4*, const uint16_t*, MoeWs,
                           int32_t*, float*, void*, int, uint32_t*, uint32_t);
template <int C, int MR>
static MoeFusedFn moe_fused_fn_cb(int cpwb) {
  switch (cpwb) {
    case 1: return &k_moe_fused_small<C, MR, 1>;
    case 2: return &k_moe_fused_small<C, MR, 2>;
    case 3: return &k_moe_fused_small<C, MR, 3>;
    default: return &k_moe_fused_small<C, MR, 4>;
  }
}
template <int C>
static MoeFusedFn moe_fused_fn_mr(int maxr, int cpwb) {
  return maxr == 1 ? moe_fused_fn_cb<C, 1>(cpwb) : maxr == 2 ? moe_fused_fn_cb<C, 2>(cpwb) : moe_fused_fn_cb<C, 4>(cpwb);
}
static MoeFusedFn moe_fused_fn(int cpw, int maxr, int cpwb) {
  return cpw == 1 ? moe_fused_fn_mr<1>(maxr, cpwb) : moe_fused_fn_mr<2>(maxr, cpwb);
}

// Single-launch decode layer: taken when the caller asked for it (or the
// library's default does) and every workgroup fits the device at once.
// Returns false when not taken.
static bool moe_fused(const uint16_t* x, const float* logits, int T, int H, int I, int E, int k, int maxact,
                      const DecSplit& sa, int maxr, int cpwb, const uint64_t* gate_s, const uint16_t* gate_sc,
                      const uint64_t* up_s, const uint16_t* up_sc, const uint64_t* down_s, const uint16_t* down_sc,
                      void* y, int y_bf16, int32_t* ids, float* w, const MoeWs& ws, hipStream_t st,
                      hipError_t& err) {
  if (!moe_fusion_wanted(T)) return false;
  const int waves = sa.waves > k ? sa.waves : k;
  const int gx = (I + 15) / 16, hb = (H + 15) / 16;
  int gy = maxact;
  if ((int64_t)gx * gy < (int64_t)hb * T) gy = (int)(((int64_t)hb * T + gx - 1) / gx);
  const size_t la = (size_t)sa.waves * sa.cpw * maxr * 1024 + (size_t)(sa.waves - 1) * 2 * 64 * 16;
  const size_t lb = (size_t)k * cpwb * 2 * 1024 + (size_t)k * 16 * 4;
  const size_t lds = la > lb ? la : lb;
  // instantiated for 1 or 2 chunks per gate/up wave (H <= 8192), 1, 2 or 4
  // staged token rows and 1 .. 4 down chunks (I <= 2048)
  if (sa.cpw > 2 || maxr > 4 || cpwb > 4) return false;
  MoeFusedFn fn = moe_fused_fn(sa.cpw, maxr, cpwb);
  if (!grid_fits(reinterpret_cast<const void*>(fn), 64 * waves, lds, (int64_t)gx * gy)) return false;
  uint32_t* slot = nullptr;
  err = grid_slot(&slot);
  if (err != hipSuccess) return true;
  const uint32_t spin = grid_spin_limit();
  const uint4* g4 = reinterpret_cast<const uint4*>(gate_s);
  const uint4* u4 = reinterpret_cast<const uint4*>(up_s);
  const uint4* d4 = reinterpret_cast<const uint4*>(down_s);
  hipLaunchKernelGGL(fn, dim3(gx, gy), dim3(64 * waves), lds, st, x, logits, T, E, k, H, I, sa.waves, g4, gate_sc, u4,
                     up_sc, d4, down_sc, ws, ids, w, y, y_bf16, slot, spin);
  err = hipGetLastError();
  return true;
}

hipError_t launch_moe(const uint16_t* x, const float* logits, int T, int H, int I, int E, int top_k,
                      const uint64_t* gate_s, const uint16_t* gate_sc, const uint64_t* up_s,
                      const uint16_t* up_sc, const uint64_t* down_s, const uint16_t* down_sc, void* y,
                      int y_bf16, int32_t* ids, float* w, void* ws_ptr, hipStream_t st) {
  MoeWs ws = moe_carve(ws_ptr, T, H, I, E, top_k);
  const int maxact = (T * top_k < E) ? T * top_k : E;
  {
    DecSplit sa;
    int maxr, cpwb;
    if (moe_small_path(T, H, I, top_k, sa, maxr, cpwb)) {
      hipError_t fe = hipSuccess;
      if (moe_fused(x, logits, T, H, I, E, top_k, maxact, sa, maxr, cpwb, gate_s, gate_sc, up_s, up_sc, down_s,
                    down_sc, y, y_bf16, ids, w, ws, st, fe))
        return fe;
      const size_t la = (size_t)sa.waves * sa.cpw * maxr * 1024 + (size_t)(sa.waves - 1) * 2 * 64 * 16;
      const dim3 ga((I + 15) / 16, maxact), ba(64 * sa.waves);
      const uint4* g4 = reinterpret_cast<const uint4*>(gate_s);
      const uint4* u4 = reinterpret_cast<const uint4*>(up_s);
#define BRQ_A(MR)                                                                                            \
  BRQ_CPW_SWITCH(sa.cpw, hipLaunchKernelGGL((k_moe_a_small<CPW, MR>), ga, ba, la, st, x, logits, T, E, top_k, H, \
                                            I, g4, gate_sc, u4, up_sc, ws, ids, w))
      if (maxr == 1) { BRQ_A(1); } else if (maxr == 2) { BRQ_A(2); } else if (maxr == 4) { BRQ_A(4); } else { BRQ_A(8); }
#undef BRQ_A
      hipError_t e1 = hipGetLastError();
      if (e1 != hipSuccess) return e1;
      const size_t lb = (size_t)top_k * cpwb * 2 * 1024 + (size_t)top_k * 16 * 4;
      const dim3 gb((H + 15) / 16, T), bb(64 * top_k);
      const uint4* d4 = reinterpret_cast<const uint4*>(down_s);
      switch (cpwb) {
        case 1: hipLaunchKernelGGL((k_moe_b_token<1>), gb, bb, lb, st, H, I, top_k, d4, down_sc, ws, y, y_bf16); break;
        case 2: hipLaunchKernelGGL((k_moe_b_token<2>), gb, bb, lb, st, H, I, top_k, d4, down_sc, ws, y, y_bf16); break;
        case 3: hipLaunchKernelGGL((k_moe_b_token<3>), gb, bb, lb, st, H, I, top_k, d4, down_sc, ws, y, y_bf16); break;
        default: hipLaunchKernelGGL((k_moe_b_token<4>), gb, bb, lb, st, H, I, top_k, d4, down_sc, ws, y, y_bf16); break;
      }
      return hipGetLastError();
    }
  }
  moe_route(logits, T, E, top_k, ws, ids, w, st);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const DecSplit sg = dec_split(H / 128, 8), sd = dec_split(I / 128, 8);
  const int tr = moe_tile_rows(sg, T, E, top_k);
  const int rt = 8;  // routes per down tile (4 is built too: more registers, less LDS)
  const int cbg = moe_cb_gu(sg.cpw), cbd = moe_cb_dn(sd.cpw);
  size_t lg = (size_t)sg.waves * sg.cpw * tr * 1024, rg = (size_t)(sg.waves - 1) * 2 * cbg * 64 * 16;
  size_t ld = (size_t)sd.waves * sd.cpw * 2 * rt * 1024, rd = (size_t)(sd.waves - 1) * cbd * 64 * 16;
  const unsigned gx = (unsigned)((I + 16 * cbg - 1) / (16 * cbg));
  const unsigned dx = (unsigned)((H + 16 * cbd - 1) / (16 * cbd));
  // gate/up on the digit path where the hidden vector comes in whole 512-wide
  // chunks, at most two per wave (H <= 8192)
  if (H % 512 == 0 && sg.cpw <= 2) {
    constexpr int NT = 2;
    const size_t lf = (size_t)sg.waves * MOE_F4_CHUNK + (size_t)(sg.waves - 1) * 2 * NT * 32 * 4;
    const dim3 gf((unsigned)((I + 16 * NT - 1) / (16 * NT)), maxact), bf(64 * sg.waves);
    const uint4* g4 = reinterpret_cast<const uint4*>(gate_s);
    const uint4* u4 = reinterpret_cast<const uint4*>(up_s);
    if (sg.cpw == 1)
      hipLaunchKernelGGL((k_moe_gateup_f4<1, NT>), gf, bf, lf, st, x, H, I, g4, gate_sc, u4, up_sc, ws);
    else
      hipLaunchKernelGGL((k_moe_gateup_f4<2, NT>), gf, bf, lf, st, x, H, I, g4, gate_sc, u4, up_sc, ws);
  } else {
#define BRQ_GATEUP(TR)                                                                                       \
  BRQ_CPW_SWITCH(sg.cpw, hipLaunchKernelGGL((k_moe_gateup<CPW, TR, moe_cb_gu(CPW)>), dim3(gx, maxact),           \
                                            dim3(64 * sg.waves), lg > rg ? lg : rg, st, x, H, I,                \
                                            reinterpret_cast<const uint4*>(gate_s), gate_sc,                    \
                                            reinterpret_cast<const uint4*>(up_s), up_sc, ws))
  if (tr == 16) {
    BRQ_GATEUP(16);
  } else if (tr == 4) {
    BRQ_GATEUP(4);
  } else {
    BRQ_GATEUP(1);
  }
#undef BRQ_GATEUP
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
#define BRQ_DOWN(RT)                                                                                         \
  BRQ_CPW_SWITCH(sd.cpw, hipLaunchKernelGGL((k_moe_down<CPW, moe_cb_dn(CPW), RT>), dim3(dx, maxact),              \
                                            dim3(64 * sd.waves), ld > rd ? ld : rd, st, H, I,                   \
                                            reinterpret_cast<const uint4*>(down_s), down_sc, ws))
  if (rt == 4) {
    BRQ_DOWN(4);
  } else {
    BRQ_DOWN(8);
  }
#undef BRQ_DOWN
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)(((int64_t)T * (H / 4) + 255) / 256)), dim3(256), 0, st, T, H, top_k,
                     ws, y, y_bf16);
  return hipGetLastError();
}

// ===========================================================================
// MoE layer with DBF experts: every routed gate, up and down projection is a
// chain y = D_out U D_mid V D_in x ("LLM binarization, Episode 01: DBF",
// section 4). After top-k and route (as above) four grouped launches run the
// chains, one workgroup per (CB blocks of 16 output columns, active expert),
// waves splitting the reduction axis:
//  stage 0: gate and up V factors on the expert's token rows (the hidden
//           vector shared by the token's experts), D_in folded into the weight
//           operand (+-d_in[k]), D_mid in the epilogue -> h_s (fp32 rows)
//  stage 1: gate and up U factors on the route's own h_s rows (+-1 operands),
//           D_out, SwiGLU -> the intermediate a (fp32 rows)
//  stage 2: down V factor on a (+-d_in), D_mid -> h_s (reusing stage 0's buffer)
//  stage 3: down U factor on h_s (+-1), D_out -> the route's fp32 output
// and the combine launch sums the slots in slot order. Stages 1-3 read their
// fp32 input rows as scaled fp16 hi/lo pieces (WaveStageF32): two MFMA rows
// per route, added and scaled back per wave before the waves' partials meet.
// ===========================================================================

struct DbfStageArgs {
  const uint4* sig[2];     // sign rows of the stage's matrices (all experts)
  const uint16_t* din[2];  // D_in of the matrices (V stages)
  const uint16_t* dg[2];   // epilogue diagonal: D_mid (V stages) or D_out (U stages)
  const float* in[2];      // fp32 input rows (stages 1-3): [R][K]
  float* out;              // fp32 output rows (stages 0 and 2): [R][N] per matrix
};

template <int STAGE, int CPW, int SR, int CB>
__global__ __launch_bounds__(512) void k_moe_dbf(const uint16_t* __restrict__ x, int H, int I, int r, int R,
                                                 DbfStageArgs a, MoeWs ws) {
  constexpr int NMAT = STAGE < 2 ? 2 : 1;
  constexpr bool PERK = STAGE == 0 || STAGE == 2;  // D_in rides on the weight operand
  constexpr bool PIECES = STAGE != 0;              // inputs are fp32 rows, staged as two piece rows per route
  constexpr int NIN = STAGE == 1 ? 2 : 1;          // separate input rows per matrix (stage 1)
  constexpr int RT = PIECES ? SR / 2 : SR;         // routes per tile
  constexpr int BMODE = PERK ? BM_PERK : BM_ONE;
  extern __shared__ uint4 smem[];
  const int4 bk = ws.blk[blockIdx.y];
  const int e = bk.x, r0 = bk.y, cnt = bk.z;
  if (cnt == 0) return;  // past the last active expert
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15;
  const int K = STAGE == 0 ? H : STAGE == 2 ? I : r;  // reduction axis
  const int N = STAGE == 1 ? I : STAGE == 3 ? H : r;  // outputs (rows of the stage's matrices)
  const int G = K >> 7, nchunks = (G + 3) >> 2;
  const int c0 = wave * CPW;
  // LDS: D_in slices of every wave first (kept across tiles), then the input
  // rows of every wave (overwritten per tile), the wave partials alias them
  uint4* dw = smem + (size_t)wave * NMAT * CPW * 64;
  uint4* stage_base = smem + (PERK ? (size_t)nw * NMAT * CPW * 64 : 0);
  uint4* xw = stage_base + (size_t)wave * NIN * CPW * SR * 64;

  // every block's sign words (and D_in) in flight before any wait; the CB
  // blocks of a matrix are one b_compute call, so each activation operand
  // (and D_in operand) is read from LDS once for all of them
  BPre<CB, CPW> bp[NMAT];
#pragma unroll
  for (int q = 0; q < NMAT; ++q) {
    const uint4* wsig[CB];
    const uint16_t* wsc[CB];
    bool rok[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = (blockIdx.x * CB + cb) * 16 + j;
      wsig[cb] = a.sig[q] + ((size_t)e * N + (col < N ? col : 0)) * G;
      wsc[cb] = nullptr;
      rok[cb] = col < N;
    }
    b_prefetch<BMODE, CB, CPW>(wsig, wsc, rok, G, c0, 1, bp[q]);
  }
  if constexpr (PERK) {
    if (c0 < nchunks) {
#pragma unroll
      for (int q = 0; q < NMAT; ++q) {
        WaveStage<ST_F16, CPW, 1> sd;
        sd.load(1, K, c0, [&](int) { return a.din[q] + (size_t)e * K; });
        sd.store(dw + q * CPW * 64);
      }
    }
  }

  // one tile of up to RT routes; the first is peeled off the loop so that its
  // input loads issue while the sign words are still in flight
  auto run_tile = [&](const int tb) {
    const int routes = (cnt - tb) < RT ? (cnt - tb) : RT;
    const int rows = PIECES ? 2 * routes : routes;
    f32x4 acc[NMAT][CB][1];
#pragma unroll
    for (int q = 0; q < NMAT; ++q)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[q][cb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    WaveStageF32<CPW, RT> sf0, sf1;  // the two inputs of stage 1 (gate, up); sf0 elsewhere
    WaveStage<ST_BF16, CPW, SR> sx;  // stage 0: the routes' token rows
    if (c0 < nchunks) {
      if constexpr (PIECES) {
        sf0.load(routes, K, c0, [&](int m) { return a.in[0] + (size_t)(r0 + tb + m) * K; });
        if constexpr (NIN == 2) sf1.load(routes, K, c0, [&](int m) { return a.in[1] + (size_t)(r0 + tb + m) * K; });
        sf0.store(xw);
        if constexpr (NIN == 2) sf1.store(xw + CPW * SR * 64);
      } else {
        sx.load(rows, K, c0, [&](int rr) { return x + (size_t)ws.route_tok[r0 + tb + rr] * H; });
        sx.store(xw);
      }
    }
    __syncthreads();
    if (c0 < nchunks) {
#pragma unroll
      for (int q = 0; q < NMAT; ++q) {
        const u32x4* xs = reinterpret_cast<const u32x4*>(xw + (NIN == 2 ? q : 0) * CPW * SR * 64);
        auto aop = [&](int, int g, int i) -> u32x4 {
          const int m = min(j, rows - 1);
          return xs[(((g >> 2) - c0) * SR + m) * 64 + (g & 3) * 16 + i];
        };
        const u32x4* kp = PERK ? reinterpret_cast<const u32x4*>(dw + q * CPW * 64) - (size_t)c0 * 64 : nullptr;
        pin_signs(bp[q]);
        b_compute<BMODE, CB, 1, CPW>(bp[q], kp, G, c0, 1, aop, acc[q]);
        // back from the wave's scaled pieces or rows (exact powers of two)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int us = !PIECES ? sx.unscale(i) : (NIN == 2 && q == 1) ? sf1.unscale(i) : sf0.unscale(i);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[q][cb][0][i] = __builtin_amdgcn_ldexpf(acc[q][cb][0][i], us);
        }
      }
    }
    __syncthreads();
    reduce_waves_cb<NMAT, CB>(acc, reinterpret_cast<f32x4*>(stage_base));
    if (wave == 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int col = (blockIdx.x * CB + cb) * 16 + j;
        if (col >= N) continue;
        if constexpr (STAGE == 0) {
          // rows are routes: lane (kb, j) holds routes 4kb + i of column col
#pragma unroll
          for (int q = 0; q < NMAT; ++q) {
            const float dm = f16_bits_to_f32(a.dg[q][(size_t)e * N + col]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int p = 4 * (lane >> 4) + i;
              if (p < routes) a.out[(size_t)q * R * r + (size_t)(r0 + tb + p) * r + col] = acc[q][cb][0][i] * dm;
            }
          }
        } else {
          // rows are pieces: route 2kb + h is rows 4kb + 2h (hi) and + 1 (lo)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int p = 2 * (lane >> 4) + h;
            if (p >= routes) continue;
            const size_t route = (size_t)(r0 + tb + p);
            const float v0 = (acc[0][cb][0][2 * h] + acc[0][cb][0][2 * h + 1]) *
                             f16_bits_to_f32(a.dg[0][(size_t)e * N + col]);
            if constexpr (STAGE == 1) {
              const float u = (acc[NMAT - 1][cb][0][2 * h] + acc[NMAT - 1][cb][0][2 * h + 1]) *
                              f16_bits_to_f32(a.dg[1][(size_t)e * N + col]);
              ws.ap[route * I + col] = v0 / (1.0f + expf(-v0)) * u;
            } else if constexpr (STAGE == 2) {
              a.out[route * r + col] = v0;
            } else {
              ws.o[route * H + col] = v0;
            }
          }
        }
      }
    }
    __syncthreads();
  };
  run_tile(0);  // an active expert has at least one route
  for (int tb = RT; tb < cnt; tb += RT) run_tile(tb);
}

// Stage 0 on the fp8 x fp4 matrix cores (H % 512 == 0, at most two chunks
// per wave): the gate and up V factors against x_s = d_in (.) x of the
// routes (bf16 times fp16, exact in fp32), carried as fixed-point digit rows
// of the 24-bit field under each wave slice's largest power of two (bits
// below 2^-23 of the slice maximum dropped, f4.h), two routes per product,
// the V signs as +-6 fp4 operands. One workgroup per (NT blocks of 16 rank
// rows, active expert); h_s = d_mid (.) (the sum / 6) in fp32.
template <int CPW, int NT>
__global__ __launch_bounds__(512) void k_moe_dbf0_f4(const uint16_t* __restrict__ x, int H, int r, int R,
                                                     DbfStageArgs a, MoeWs ws) {
  extern __shared__ uint4 smem[];
  const int4 bk = ws.blk[blockIdx.y];
  const int e = bk.x, r0 = bk.y, cnt = bk.z;
  if (cnt == 0) return;  // past the last active expert
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int G = H >> 7, nchunks = G >> 2;
  const int c0 = wave * CPW;
  uint8_t* xw = reinterpret_cast<uint8_t*>(smem) + (size_t)wave * MOE_F4_CHUNK;
  float* red = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem) + (size_t)nw * MOE_F4_CHUNK);
  auto load_x = [&](int q0, uint4 (&xv)[2][CPW]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rr = q0 + h < cnt ? q0 + h : cnt - 1;
      const uint16_t* xr = x + (size_t)ws.route_tok[r0 + rr] * H;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int k0 = (c0 + c) * 512 + 8 * lane;
        xv[h][c] = *reinterpret_cast<const uint4*>(xr + (k0 < H ? k0 : 0));
      }
    }
  };
  uint4 xv[2][CPW];
  load_x(0, xv);
  uint4 dv[2][CPW];  // d_in of the gate and up chains, the lane's 8 values per chunk
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int k0 = (c0 + c) * 512 + 8 * lane;
      dv[m][c] = *reinterpret_cast<const uint4*>(a.din[m] + (size_t)e * H + (k0 < H ? k0 : 0));
    }
  uint4 sg[2][NT][CPW];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = (blockIdx.x * NT + t) * 16 + j;
    const size_t row = ((size_t)e * r + (n < r ? n : 0)) * G;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const int g = 4 * (c0 + c) + kb;
        sg[m][t][c] = a.sig[m][row + (g < G ? g : 0)];
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (lane < 32)
    *reinterpret_cast<uint4*>(xw + (lane >> 3) * MOE_F4_GROUP + 12 * 128 + 16 * (lane & 7)) =
        make_uint4(0u, 0u, 0u, 0u);
  const int prow = j < 6 ? j : (j >= 8 && j < 14) ? j - 2 : 12;
  uint8_t* base = xw + (lane >> 4) * MOE_F4_GROUP + 32 * ((lane & 15) >> 2) + 2 * (lane & 3);
  for (int q0 = 0; q0 < cnt; q0 += 2) {
    if (q0 > 0) load_x(q0, xv);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        if (c0 + c >= nchunks || q0 + h >= cnt) xv[h][c] = make_uint4(0u, 0u, 0u, 0u);
    float acc[2][NT];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      // x_s = d_in (.) x of both routes for chain m
      f32x4 xs[2][CPW][2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
          const uint32_t xw4[4] = {xv[h][c].x, xv[h][c].y, xv[h][c].z, xv[h][c].w};
          const uint32_t dw4[4] = {dv[m][c].x, dv[m][c].y, dv[m][c].z, dv[m][c].w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t xb = (i & 1) ? (xw4[i >> 1] >> 16) : (xw4[i >> 1] & 0xffffu);
            const uint32_t db = (i & 1) ? (dw4[i >> 1] >> 16) : (dw4[i >> 1] & 0xffffu);
            xs[h][c][i >> 2][i & 3] = bf16_to_f32(xb) * f16_bits_to_f32(db);
          }
        }
      float S0, S1;
      const uint32_t e0 = f4_slice_exponent_f32<CPW>(xs[0], S0), e1 = f4_slice_exponent_f32<CPW>(xs[1], S1);
      // the zero row (prow 12) takes scale 2^0 (ebs - 26 is the E8M0 NaN code at ebs = 25)
      const int sa = prow == 12 ? 127 : j < 8 ? (int)e0 - 2 - 4 * j : (int)e1 - 2 - 4 * (j - 8);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][t] = 0.f;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        if (c0 + c >= nchunks) break;  // uniform across the wave
        f4_digits_f32(xs[0][c], S0, base, 0);
        f4_digits_f32(xs[1][c], S1, base, 6);
        const uint8_t* ab = xw + prow * 128 + 16 * kb;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          uint32_t w0 = sg[m][t][c].x, w1 = sg[m][t][c].y, w2 = sg[m][t][c].z, w3 = sg[m][t][c].w;
          f4_transpose4(w0, w1, w2, w3);
          const uint32_t wi[4] = {w0, w1, w2, w3};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 d = f4_group_mfma(ab + i * MOE_F4_GROUP, wi[i], sa);
            acc[m][t] += (d[0] + d[1]) + (d[2] + d[3]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[m][t] += __shfl_down(acc[m][t], 16, 64);
    const bool holds = (kb & 1) == 0;
    if (wave > 0 && holds) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) red[(((wave - 1) * 2 + m) * NT + t) * 32 + (kb >> 1) * 16 + j] = acc[m][t];
    }
    __syncthreads();
    if (wave == 0 && holds) {
      const int p = q0 + (kb >> 1);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int n = (blockIdx.x * NT + t) * 16 + j;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float v = acc[m][t];
          for (int w = 1; w < nw; ++w) v += red[(((w - 1) * 2 + m) * NT + t) * 32 + (kb >> 1) * 16 + j];
          if (p < cnt && n < r)
            a.out[(size_t)m * R * r + (size_t)(r0 + p) * r + n] =
                (v / 6.0f) * f16_bits_to_f32(a.dg[m][(size_t)e * r + n]);
        }
      }
    }
    __syncthreads();
  }
}

// ---- DBF experts, few tokens (T <= 4): five launches ----------------------
//  route: one workgroup, one wave per token: top-k, then one block record per
//         route in token-major order (route i = t*k + j forms its own block of
//         one route), ids and weights out;
//  stages 0-2: k_moe_dbf on those one-route blocks;
//  stage 3 + combine: one workgroup per (16 hidden columns, token), one wave
//         per slot: the down U factor on the route's h_s (scaled pieces, the
//         wave covers the whole rank), D_out; wave 0 then adds w_tj * out_j
//         in slot order.
__global__ __launch_bounds__(256) void k_moe_route_tok(const float* __restrict__ logits, int T, int E, int k,
                                                       MoeWs ws, int32_t* __restrict__ ids_user,
                                                       float* __restrict__ w_user) {
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  if (t >= T) return;
  int id;
  float w;
  if (E <= 256) wave_route<4>(logits + (size_t)t * E, E, k, id, w);
  else wave_route<16>(logits + (size_t)t * E, E, k, id, w);
  if (lane < k) {
    const int r = t * k + lane;
    ws.ids[r] = id;
    ws.wts[r] = w;
    ws.blk[r] = make_int4(id, r, 1, 0);
    ws.route_tok[r] = t;
    ws.route_pos[r] = r;
    if (ids_user) ids_user[r] = id;
    if (w_user) w_user[r] = w;
  }
}

template <int CPW>
__global__ __launch_bounds__(1024) void k_moe_dbf_down_tok(int H, int r, int k, const uint4* __restrict__ u,
                                                           const uint16_t* __restrict__ d_out,
                                                           const float* __restrict__ hs, MoeWs ws,
                                                           void* __restrict__ y, int y_bf16) {
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, slot = threadIdx.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int t = blockIdx.y;
  const int n = blockIdx.x * 16 + j;
  const int route = t * k + slot;
  const int e = ws.ids[route];
  const int G = r >> 7;
  const bool rok = n < H;
  const size_t row = (size_t)e * H + (rok ? n : 0);
  const uint4* wsig[1] = {u + row * G};
  const uint16_t* wsc[1] = {nullptr};
  const bool rk[1] = {rok};
  uint4* xw = smem + (size_t)slot * CPW * 2 * 64;
  float* part = reinterpret_cast<float*>(smem + (size_t)k * CPW * 2 * 64);  // [k][16]
  f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
  WaveStageF32<CPW, 1> sh;  // the route's h_s row as two scaled piece rows
  {
    sh.load(1, r, 0, [&](int) { return hs + (size_t)route * r; });
    BPre<1, CPW> bp;
    b_prefetch<BM_ONE, 1, CPW>(wsig, wsc, rk, G, 0, 1, bp);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    sh.store(xw);
    const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
    auto aop = [&](int, int g, int i) -> u32x4 {
      const int p = min(j, 1);
      return xs[((g >> 2) * 2 + p) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_ONE, 1, 1, CPW, true>(bp, nullptr, G, 0, 1, aop, acc);
  }
  // lanes 0..15 hold piece rows 0 and 1 of column j
  if (kb == 0)
    part[slot * 16 + j] =
        __builtin_amdgcn_ldexpf(acc[0][0][0] + acc[0][0][1], sh.unscale(0)) * f16_bits_to_f32(d_out[row]);
  __syncthreads();
  if (slot != 0 || kb != 0 || !rok) return;
  float sum = 0.f;
  for (int q = 0; q < k; ++q) sum = fmaf(ws.wts[t * k + q], part[q * 16 + j], sum);
  store_out(y, (size_t)t * H + n, sum, y_bf16);
}

// the few-token path applies when the last launch's staging fits and the
// one-route blocks fit the E block records of the workspace (T*k <= E)
static bool moe_dbf_tok_path(int T, int E, int r, int k, int& cpw, size_t& lds) {
  cpw = (r / 128 + 3) / 4;
  lds = (size_t)k * cpw * 2 * 1024 + (size_t)k * 16 * 4;
  return T <= MOE_SMALL_T && T * k <= E && cpw <= 4 && lds <= (size_t)kDecLdsBytes;
}

size_t moe_dbf_ws_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int64_t r) {
  return moe_ws_bytes(T, H, I, E, k) + align256((size_t)2 * T * k * r * 4);  // h_s: fp32 [2][T*k][r]
}

template <int STAGE, int SR, int CB, int CPW = 1>
static hipError_t moe_dbf_stage_cb(const uint16_t* x, int H, int I, int r, int R, int maxact, const DbfStageArgs& a,
                                   const MoeWs& ws, int waves, hipStream_t st) {
  const int N = STAGE == 1 ? I : STAGE == 3 ? H : r;
  constexpr int NMAT = STAGE < 2 ? 2 : 1;
  constexpr int NIN = STAGE == 1 ? 2 : 1;
  constexpr bool PERK = STAGE == 0 || STAGE == 2;
  const size_t din = PERK ? (size_t)waves * NMAT * CPW * 1024 : 0;
  const size_t stg = (size_t)waves * NIN * CPW * SR * 1024;
  const size_t red = (size_t)(waves - 1) * CB * NMAT * 1024;
  const size_t lds = din + (stg > red ? stg : red);
  const dim3 grid((unsigned)((N + 16 * CB - 1) / (16 * CB)), (unsigned)maxact);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_moe_dbf<STAGE, CPW, SR, CB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_moe_dbf<STAGE, CPW, SR, CB>), grid, dim3(64 * waves), lds, st, x, H, I, r, R, a, ws);
  return hipGetLastError();
}

// One chunk (512 of the reduction axis) per wave up to K = 4096 (8 waves);
// the hidden vector of stage 0 may be up to 8192 long (two chunks per wave,
// token tiles of 4 rows so that the staged rows fit the registers). CB
// blocks of 16 columns per workgroup: 4 when that still gives about four
// workgroups per compute unit for the experts that can be active, fewer
// otherwise (decode at T = 1 has 8).
template <int STAGE, int SR>
static hipError_t moe_dbf_stage(const uint16_t* x, int H, int I, int r, int R, int maxact, const DbfStageArgs& a,
                                const MoeWs& ws, hipStream_t st) {
  const int K = STAGE == 0 ? H : STAGE == 2 ? I : r;
  const int N = STAGE == 1 ? I : STAGE == 3 ? H : r;
  const DecSplit sp = dec_split(K / 128, 8);
  const int64_t blocks = (int64_t)((N + 15) / 16) * maxact;
  if constexpr (STAGE == 0) {
    // the V factors of gate and up on the digit path where the hidden vector
    // comes in whole 512-wide chunks
    if (H % 512 == 0 && sp.cpw <= 2) {
      constexpr int NT = 2;
      const size_t lf = (size_t)sp.waves * MOE_F4_CHUNK + (size_t)(sp.waves - 1) * 2 * NT * 32 * 4;
      const dim3 gf((unsigned)((N + 16 * NT - 1) / (16 * NT)), (unsigned)maxact), bf(64 * sp.waves);
      if (sp.cpw == 1) hipLaunchKernelGGL((k_moe_dbf0_f4<1, NT>), gf, bf, lf, st, x, H, r, R, a, ws);
      else hipLaunchKernelGGL((k_moe_dbf0_f4<2, NT>), gf, bf, lf, st, x, H, r, R, a, ws);
      return hipGetLastError();
    }
    if (sp.cpw == 2) {
      if (blocks >= 4096) return moe_dbf_stage_cb<STAGE, 4, 4, 2>(x, H, I, r, R, maxact, a, ws, sp.waves, st);
      if (blocks >= 2048) return moe_dbf_stage_cb<STAGE, 4, 2, 2>(x, H, I, r, R, maxact, a, ws, sp.waves, st);
      return moe_dbf_stage_cb<STAGE, 4, 1, 2>(x, H, I, r, R, maxact, a, ws, sp.waves, st);
    }
  }
  if (sp.cpw != 1) return hipErrorInvalidValue;  // outside the accepted shapes
  if (blocks >= 4096) return moe_dbf_stage_cb<STAGE, SR, 4>(x, H, I, r, R, maxact, a, ws, sp.waves, st);
  if (blocks >= 2048) return moe_dbf_stage_cb<STAGE, SR, 2>(x, H, I, r, R, maxact, a, ws, sp.waves, st);
  return moe_dbf_stage_cb<STAGE, SR, 1>(x, H, I, r, R, maxact, a, ws, sp.waves, st);
}

hipError_t launch_moe_dbf(const uint16_t* x, const float* logits, int T, int H, int I, int E, int top_k, int r,
                          const DbfFactors& gate, const DbfFactors& up, const DbfFactors& down, void* y, int y_bf16,
                          int32_t* ids, float* w, void* ws_ptr, hipStream_t st) {
  MoeWs ws = moe_carve(ws_ptr, T, H, I, E, top_k);
  float* hbuf = reinterpret_cast<float*>(reinterpret_cast<char*>(ws_ptr) + moe_ws_bytes(T, H, I, E, top_k));
  const int R = T * top_k;
  int cpw3;
  size_t lds3;
  const bool tok = moe_dbf_tok_path(T, E, r, top_k, cpw3, lds3);
  const int maxact = tok ? R : (R < E ? R : E);
  if (tok) {
    hipLaunchKernelGGL(k_moe_route_tok, dim3(1), dim3(256), 0, st, logits, T, E, top_k, ws, ids, w);
  } else {
    moe_route(logits, T, E, top_k, ws, ids, w, st);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  auto u4 = [](const uint64_t* p) { return reinterpret_cast<const uint4*>(p); };
  // token tiles of 4 when experts expect at most 3 routes, as in the group-128 layer
  const bool small = (int64_t)R <= 3 * (int64_t)E;
  DbfStageArgs a0{{u4(gate.v), u4(up.v)}, {gate.d_in, up.d_in}, {gate.d_mid, up.d_mid}, {nullptr, nullptr}, hbuf};
  DbfStageArgs a1{{u4(gate.u), u4(up.u)}, {nullptr, nullptr}, {gate.d_out, up.d_out},
                  {hbuf, hbuf + (size_t)R * r}, nullptr};
  DbfStageArgs a2{{u4(down.v), nullptr}, {down.d_in, nullptr}, {down.d_mid, nullptr},
                  {ws.ap, nullptr}, hbuf};
  DbfStageArgs a3{{u4(down.u), nullptr}, {nullptr, nullptr}, {down.d_out, nullptr}, {hbuf, nullptr}, nullptr};
  if (tok) {
    err = moe_dbf_stage<0, 4>(x, H, I, r, R, maxact, a0, ws, st);
    if (err == hipSuccess) err = moe_dbf_stage<1, 8>(x, H, I, r, R, maxact, a1, ws, st);
    if (err == hipSuccess) err = moe_dbf_stage<2, 8>(x, H, I, r, R, maxact, a2, ws, st);
    if (err != hipSuccess) return err;
    const dim3 g3((H + 15) / 16, T), b3(64 * top_k);
    const uint4* du = u4(down.u);
    switch (cpw3) {
      case 1: hipLaunchKernelGGL((k_moe_dbf_down_tok<1>), g3, b3, lds3, st, H, r, top_k, du, down.d_out, hbuf, ws, y, y_bf16); break;
      case 2: hipLaunchKernelGGL((k_moe_dbf_down_tok<2>), g3, b3, lds3, st, H, r, top_k, du, down.d_out, hbuf, ws, y, y_bf16); break;
      case 3: hipLaunchKernelGGL((k_moe_dbf_down_tok<3>), g3, b3, lds3, st, H, r, top_k, du, down.d_out, hbuf, ws, y, y_bf16); break;
      default: hipLaunchKernelGGL((k_moe_dbf_down_tok<4>), g3, b3, lds3, st, H, r, top_k, du, down.d_out, hbuf, ws, y, y_bf16); break;
    }
    return hipGetLastError();
  }
  if (small) {
    err = moe_dbf_stage<0, 4>(x, H, I, r, R, maxact, a0, ws, st);
    if (err == hipSuccess) err = moe_dbf_stage<1, 8>(x, H, I, r, R, maxact, a1, ws, st);
    if (err == hipSuccess) err = moe_dbf_stage<2, 8>(x, H, I, r, R, maxact, a2, ws, st);
    if (err == hipSuccess) err = moe_dbf_stage<3, 8>(x, H, I, r, R, maxact, a3, ws, st);
  } else {
    err = moe_dbf_stage<0, 16>(x, H, I, r, R, maxact, a0, ws, st);
    if (err == hipSuccess) err = moe_dbf_stage<1, 16>(x, H, I, r, R, maxact, a1, ws, st);
    if (err == hipSuccess) err = moe_dbf_stage<2, 16>(x, H, I, r, R, maxact, a2, ws, st);
    if (err == hipSuccess) err = moe_dbf_stage<3, 16>(x, H, I, r, R, maxact, a3, ws, st);
  }
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)(((int64_t)T * (H / 4) + 255) / 256)), dim3(256), 0, st, T, H, top_k,
                     ws, y, y_bf16);
  return hipGetLastError();
}

}  // namespace brq
