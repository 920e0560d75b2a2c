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
// Launches, all on the caller's stream, no host read-back:
//  1. route: top-k per token (descending fp32 logit, ties to the lower expert
//     index), softmax over the k selected logits, per-expert counts and
//     offsets, the list of active experts and the expert-major route list;
//     the other workgroups stage x in the permuted fp16 operand order.
//  2. gate/up: one workgroup per (16 intermediate columns, active expert);
//     both products share every activation operand; SwiGLU in fp32; the
//     result is stored as an fp16 hi/lo pair per route, permuted.
//  3. down: one workgroup per (16 hidden columns, active expert); writes the
//     route's fp32 output.
//  4. combine: y_t = sum over slots j, in slot order, of w_tj * out(t, j).
#include "dec_core.h"
#include "kernels.h"

namespace brq {

constexpr int MOE_MAX_E = 1024;
constexpr int MOE_MAX_T = 256;
constexpr int MOE_MAX_R = MOE_MAX_T * 16;

struct MoeWs {
  int* ids;          // [T][k]
  float* wts;        // [T][k]
  int* off;          // [E+1]
  int* act;          // [E]
  int* nact;         // [1]
  int* route_tok;    // [R] token of each expert-major route position
  int* route_pos;    // [T][k] expert-major position of route (t, j)
  uint16_t* ap;      // [2R][I] permuted fp16 hi/lo of the SwiGLU output
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
  w.act = reinterpret_cast<int*>(take((size_t)E * 4));
  w.nact = reinterpret_cast<int*>(take(4));
  w.route_tok = reinterpret_cast<int*>(take((size_t)R * 4));
  w.route_pos = reinterpret_cast<int*>(take((size_t)R * 4));
  w.ap = reinterpret_cast<uint16_t*>(take((size_t)2 * R * I * 2));
  w.o = reinterpret_cast<float*>(take((size_t)R * H * 4));
  return w;
}

size_t moe_ws_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  const int64_t R = T * k;
  return 2 * align256((size_t)R * 4) + align256((size_t)(E + 1) * 4) + align256((size_t)E * 4) + align256(4) +
         2 * align256((size_t)R * 4) + align256((size_t)2 * R * I * 2) + align256((size_t)R * H * 4);
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

// One workgroup of 1024 threads. Top-k: one wave per token. Routes of one
// expert are ordered by token (slots of one token name distinct experts): the
// rank of route (t, j) inside its expert is the number of earlier tokens in the
// expert's token bitmap.
__global__ __launch_bounds__(1024) void k_moe_route(const float* __restrict__ logits, int T, int E, int k, MoeWs ws,
                                                    int32_t* __restrict__ ids_user, float* __restrict__ w_user) {
  __shared__ int s_ids[MOE_MAX_R];
  __shared__ int s_cnt[MOE_MAX_E];
  __shared__ int s_off[MOE_MAX_E];
  __shared__ unsigned long long s_map[MOE_MAX_E * (MOE_MAX_T / 64)];
  __shared__ int s_part[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int words = (T + 63) >> 6;
  for (int e = tid; e < E; e += blockDim.x) {
    s_cnt[e] = 0;
    for (int q = 0; q < words; ++q) s_map[e * words + q] = 0ull;
  }
  __syncthreads();
  const int per_lane = (E + 63) / 64;
  for (int t = wave; t < T; t += nw) {
    float v[MOE_MAX_E / 64];
#pragma unroll
    for (int i = 0; i < MOE_MAX_E / 64; ++i) {
      const int e = lane + 64 * i;
      v[i] = (i < per_lane && e < E) ? logits[(size_t)t * E + e] : 0.f;
    }
    uint32_t taken = 0;
    float sel0 = 0.f, mysel = 0.f;
    int myid = 0;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < MOE_MAX_E / 64; ++i) {
        const int e = lane + 64 * i;
        if (i < per_lane && e < E && !((taken >> i) & 1u)) {
          if (be == 0x7fffffff || v[i] > bv || (v[i] == bv && e < be)) { bv = v[i]; be = e; }
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oe = __shfl_xor(be, o, 64);
        if (oe != 0x7fffffff && (be == 0x7fffffff || ov > bv || (ov == bv && oe < be))) { bv = ov; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (j == 0) sel0 = bv;  // the largest selected logit
      if (j == lane) { mysel = bv; myid = be; }
    }
    // softmax over the k selected logits (lane j holds slot j)
    const float ex = lane < k ? expf(mysel - sel0) : 0.f;
    float esum = ex;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) esum += __shfl_xor(esum, o, 64);
    if (lane < k) {
      const float w = ex / esum;
      ws.ids[t * k + lane] = myid;
      ws.wts[t * k + lane] = w;
      s_ids[t * k + lane] = myid;
      if (ids_user) ids_user[t * k + lane] = myid;
      if (w_user) w_user[t * k + lane] = w;
      atomicAdd(&s_cnt[myid], 1);
      atomicOr(&s_map[myid * words + (t >> 6)], 1ull << (t & 63));
    }
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
    if (cnt > 0) ws.act[aidx] = tid;
  }
  if (tid == 0) {
    ws.off[E] = R;
    *ws.nact = na;
  }
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

// gate/up: one workgroup per (16 intermediate columns, active expert). The
// expert's sign words are loaded once; its tokens are staged, a tile of up to
// tile_rows at a time, each wave staging its own K-slice (bf16 -> permuted
// fp16).
template <int CPW, int MAXR>
__global__ __launch_bounds__(512) void k_moe_gateup(const uint16_t* __restrict__ x, int H, int I,
                                                    const uint4* __restrict__ gs, const uint16_t* __restrict__ gsc,
                                                    const uint4* __restrict__ us, const uint16_t* __restrict__ usc,
                                                    MoeWs ws) {
  extern __shared__ uint4 smem[];
  if ((int)blockIdx.y >= *ws.nact) return;
  const int e = ws.act[blockIdx.y];
  const int r0 = ws.off[e], cnt = ws.off[e + 1] - r0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int n = blockIdx.x * 16 + j;
  const int G = H >> 7, nchunks = (G + 3) >> 2;
  const int c0 = wave * CPW;
  const size_t row = (size_t)e * I + (n < I ? n : 0);
  const uint4* wsig[2] = {gs + row * G, us + row * G};
  const uint16_t* wsc[2] = {gsc + row * G, usc + row * G};
  const bool rok[2] = {n < I, n < I};
  BPre<2, CPW> bp;
  if (c0 < nchunks) b_prefetch<BM_GROUP, 2, CPW>(wsig, wsc, rok, G, c0, 1, bp);
  const int pc = perm_pos(n);
  for (int tb = 0; tb < cnt; tb += MAXR) {
    const int rows = (cnt - tb) < MAXR ? (cnt - tb) : MAXR;
    uint4* xw = smem + (size_t)wave * CPW * MAXR * 64;
    if (c0 < nchunks) {
      WaveStage<ST_BF16, CPW, MAXR> sx;
      sx.load(rows, H, c0, [&](int rr) { return x + (size_t)ws.route_tok[r0 + tb + rr] * H; });
      sx.store(xw);
    }
    __syncthreads();
    f32x4 acc[2][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}, {f32x4{0.f, 0.f, 0.f, 0.f}}};
    if (c0 < nchunks) {
      const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
      auto aop = [&](int, int g, int i) -> u32x4 {
        const int m = min(j, rows - 1);
        return xs[(((g >> 2) - c0) * MAXR + m) * 64 + (g & 3) * 16 + i];
      };
      b_compute<BM_GROUP, 2, 1, CPW>(bp, nullptr, G, c0, 1, aop, acc);
    }
    __syncthreads();
    reduce_waves<2, 1>(acc, reinterpret_cast<f32x4*>(smem));
    if (wave == 0 && n < I) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = 4 * (lane >> 4) + i;
        if (p < rows) {
          const float g = acc[0][0][i], u = acc[1][0][i];
          const float a = g / (1.0f + expf(-g)) * u;
          uint16_t hi, lo;
          split_f16(a, hi, lo);
          ws.ap[(size_t)(2 * (r0 + tb + p)) * I + pc] = hi;
          ws.ap[(size_t)(2 * (r0 + tb + p) + 1) * I + pc] = lo;
        }
      }
    }
    __syncthreads();
  }
}

// down: one workgroup per (16 hidden columns, active expert); the routes'
// fp16 hi/lo intermediates are staged per wave, 8 routes (16 piece rows) a
// tile.
template <int CPW>
__global__ __launch_bounds__(512) void k_moe_down(int H, int I, const uint4* __restrict__ ds,
                                                  const uint16_t* __restrict__ dsc, MoeWs ws) {
  extern __shared__ uint4 smem[];
  if ((int)blockIdx.y >= *ws.nact) return;
  const int e = ws.act[blockIdx.y];
  const int r0 = ws.off[e], cnt = ws.off[e + 1] - r0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int n = blockIdx.x * 16 + j;
  const int G = I >> 7, nchunks = (G + 3) >> 2;
  const int c0 = wave * CPW;
  const size_t row = (size_t)e * H + (n < H ? n : 0);
  const uint4* wsig[1] = {ds + row * G};
  const uint16_t* wsc[1] = {dsc + row * G};
  const bool rok[1] = {n < H};
  BPre<1, CPW> bp;
  if (c0 < nchunks) b_prefetch<BM_GROUP, 1, CPW>(wsig, wsc, rok, G, c0, 1, bp);
  for (int tb = 0; tb < cnt; tb += 8) {
    const int routes = (cnt - tb) < 8 ? (cnt - tb) : 8;
    const int rows = 2 * routes;
    uint4* xw = smem + (size_t)wave * CPW * 16 * 64;
    if (c0 < nchunks) {
      WaveStage<ST_COPY, CPW, 16> sa;
      sa.load(rows, I, c0, [&](int pr) { return ws.ap + (size_t)(2 * (r0 + tb) + pr) * I; });
      sa.store(xw);
    }
    __syncthreads();
    f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
    if (c0 < nchunks) {
      const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
      auto aop = [&](int, int g, int i) -> u32x4 {
        const int pr = min(j, rows - 1);
        return xs[(((g >> 2) - c0) * 16 + pr) * 64 + (g & 3) * 16 + i];
      };
      b_compute<BM_GROUP, 1, 1, CPW>(bp, nullptr, G, c0, 1, aop, acc);
    }
    __syncthreads();
    reduce_waves<1, 1>(acc, reinterpret_cast<f32x4*>(smem));
    if (wave == 0 && n < H) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = 2 * (lane >> 4) + h;
        if (q < routes) ws.o[(size_t)(r0 + tb + q) * H + n] = acc[0][0][2 * h] + acc[0][0][2 * h + 1];
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_moe_combine(int T, int H, int k, MoeWs ws, void* __restrict__ y,
                                                     int y_bf16) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * H) return;
  const int t = (int)(idx / H), n = (int)(idx % H);
  float acc = 0.f;
  for (int j = 0; j < k; ++j) acc = fmaf(ws.wts[t * k + j], ws.o[(size_t)ws.route_pos[t * k + j] * H + n], acc);
  store_out(y, (size_t)idx, acc, y_bf16);
}

// token rows per gate/up tile: staged row slots per chunk, so that
// waves * cpw * slots KiB fit the staging budget
static int moe_tile_rows(const DecSplit& sp) {
  const int64_t chunks = (int64_t)sp.waves * sp.cpw;
  return chunks <= 4 ? 16 : chunks <= 16 ? 4 : 1;
}

hipError_t launch_moe(const uint16_t* x, const float* logits, int T, int H, int I, int E, int top_k,
                      const uint64_t* gate_s, const uint16_t* gate_sc, const uint64_t* up_s,
                      const uint16_t* up_sc, const uint64_t* down_s, const uint16_t* down_sc, void* y,
                      int y_bf16, int32_t* ids, float* w, void* ws_ptr, hipStream_t st) {
  MoeWs ws = moe_carve(ws_ptr, T, H, I, E, top_k);
  const int maxact = (T * top_k < E) ? T * top_k : E;
  hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(1024), 0, st, logits, T, E, top_k, ws, ids, w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const DecSplit sg = dec_split(H / 128, 8), sd = dec_split(I / 128, 8);
  const int tr = moe_tile_rows(sg);
  size_t lg = (size_t)sg.waves * sg.cpw * tr * 1024, rg = (size_t)(sg.waves - 1) * 2 * 64 * 16;
  size_t ld = (size_t)sd.waves * sd.cpw * 16 * 1024, rd = (size_t)(sd.waves - 1) * 64 * 16;
#define BRQ_GATEUP(TR)                                                                                       \
  BRQ_CPW_SWITCH(sg.cpw, hipLaunchKernelGGL((k_moe_gateup<CPW, TR>), dim3((I + 15) / 16, maxact),                \
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
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  BRQ_CPW_SWITCH(sd.cpw, hipLaunchKernelGGL((k_moe_down<CPW>), dim3((H + 15) / 16, maxact), dim3(64 * sd.waves),
                                            ld > rd ? ld : rd, st, H, I, reinterpret_cast<const uint4*>(down_s),
                                            down_sc, ws));
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)(((int64_t)T * H + 255) / 256)), dim3(256), 0, st, T, H, top_k,
                     ws, y, y_bf16);
  return hipGetLastError();
}

}  // namespace brq
