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
constexpr int MOE_MAX_R = 4096;  // 256 tokens x 16 slots

struct MoeWs {
  uint16_t* xp;      // [T][H] permuted fp16
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
  w.xp = reinterpret_cast<uint16_t*>(take((size_t)T * H * 2));
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
  return align256((size_t)T * H * 2) + 2 * align256((size_t)R * 4) + align256((size_t)(E + 1) * 4) +
         align256((size_t)E * 4) + align256(4) + 2 * align256((size_t)R * 4) +
         align256((size_t)2 * R * I * 2) + align256((size_t)R * H * 4);
}

__global__ __launch_bounds__(256) void k_moe_route(const float* __restrict__ logits, int T, int E, int k,
                                                   const uint16_t* __restrict__ x, int64_t xruns, MoeWs ws,
                                                   int32_t* __restrict__ ids_user, float* __restrict__ w_user) {
  if (blockIdx.x > 0) {
    // ---- stage x in the permuted fp16 operand order (one run of 32 per thread)
    const int64_t t = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x;
    if (t >= xruns) return;
    const uint32_t* s = reinterpret_cast<const uint32_t*>(x + t * 32);
    uint32_t o[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const uint32_t lo = (b & 1) ? (s[b >> 1] >> 16) : (s[b >> 1] & 0xffffu);
      const uint32_t hi = (b & 1) ? (s[8 + (b >> 1)] >> 16) : (s[8 + (b >> 1)] & 0xffffu);
      o[b] = (uint32_t)f32_to_f16_bits(bf16_to_f32(lo)) | ((uint32_t)f32_to_f16_bits(bf16_to_f32(hi)) << 16);
    }
    uint4* d = reinterpret_cast<uint4*>(ws.xp + t * 32);
    d[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d[1] = make_uint4(o[4], o[5], o[6], o[7]);
    d[2] = make_uint4(o[8], o[9], o[10], o[11]);
    d[3] = make_uint4(o[12], o[13], o[14], o[15]);
    return;
  }
  __shared__ int s_ids[MOE_MAX_R];
  __shared__ int s_cnt[MOE_MAX_E];
  __shared__ int s_off[MOE_MAX_E + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = T * k;
  const int per_lane = (E + 63) / 64;

  // ---- top-k per token: one wave per token ---------------------------------
  for (int t = wave; t < T; t += 4) {
    float v[MOE_MAX_E / 64];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < MOE_MAX_E / 64; ++i) {
      const int e = lane + 64 * i;
      v[i] = (i < per_lane && e < E) ? logits[(size_t)t * E + e] : 0.f;
    }
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
    }
  }
  for (int e = tid; e < E; e += 256) s_cnt[e] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += 256) atomicAdd(&s_cnt[s_ids[r]], 1);
  __syncthreads();
  if (tid == 0) {
    int acc = 0, na = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = acc;
      ws.off[e] = acc;
      if (s_cnt[e] > 0) ws.act[na++] = e;
      acc += s_cnt[e];
    }
    s_off[E] = acc;
    ws.off[E] = acc;
    *ws.nact = na;
  }
  __syncthreads();
  // expert-major route list, routes of one expert in (token, slot) order
  for (int e = tid; e < E; e += 256) {
    if (s_cnt[e] == 0) continue;
    int c = s_off[e];
    for (int r = 0; r < R; ++r)
      if (s_ids[r] == e) {
        ws.route_tok[c] = r / k;
        ws.route_pos[r] = c;
        ++c;
      }
  }
}

__global__ __launch_bounds__(1024) void k_moe_gateup(int H, int I, const uint4* __restrict__ gs,
                                                     const uint16_t* __restrict__ gsc, const uint4* __restrict__ us,
                                                     const uint16_t* __restrict__ usc, MoeWs ws) {
  __shared__ f32x4 red[15 * 2 * 64];
  if ((int)blockIdx.y >= *ws.nact) return;
  const int e = ws.act[blockIdx.y];
  const int r0 = ws.off[e], cnt = ws.off[e + 1] - r0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15;
  const int n = blockIdx.x * 16 + j;
  const int G = H >> 7;
  const size_t row = (size_t)e * I + n;
  const uint4* wsig[2] = {n < I ? gs + row * G : nullptr, n < I ? us + row * G : nullptr};
  const uint16_t* wsc[2] = {n < I ? gsc + row * G : nullptr, n < I ? usc + row * G : nullptr};
  const int pc = perm_pos(n);
  for (int tb = 0; tb < cnt; tb += 16) {
    const u32x4* arow[1] = {tb + j < cnt ? reinterpret_cast<const u32x4*>(ws.xp + (size_t)ws.route_tok[r0 + tb + j] * H)
                                         : nullptr};
    f32x4 acc[2][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}, {f32x4{0.f, 0.f, 0.f, 0.f}}};
    dec_core<BM_GROUP, 2, 1>(wsig, wsc, nullptr, arow, G, wave, nw, acc);
    reduce_waves<2, 1>(acc, red);
    if (wave == 0 && n < I) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = tb + 4 * (lane >> 4) + i;
        if (p < cnt) {
          const float g = acc[0][0][i], u = acc[1][0][i];
          const float a = g / (1.0f + expf(-g)) * u;
          uint16_t hi, lo;
          split_f16(a, hi, lo);
          ws.ap[(size_t)(2 * (r0 + p)) * I + pc] = hi;
          ws.ap[(size_t)(2 * (r0 + p) + 1) * I + pc] = lo;
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(1024) void k_moe_down(int H, int I, const uint4* __restrict__ ds,
                                                   const uint16_t* __restrict__ dsc, MoeWs ws) {
  __shared__ f32x4 red[15 * 64];
  if ((int)blockIdx.y >= *ws.nact) return;
  const int e = ws.act[blockIdx.y];
  const int r0 = ws.off[e], cnt = ws.off[e + 1] - r0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15;
  const int n = blockIdx.x * 16 + j;
  const int G = I >> 7;
  const size_t row = (size_t)e * H + n;
  const uint4* wsig[1] = {n < H ? ds + row * G : nullptr};
  const uint16_t* wsc[1] = {n < H ? dsc + row * G : nullptr};
  for (int tb = 0; tb < cnt; tb += 8) {
    const int p = tb + (j >> 1);
    const u32x4* arow[1] = {p < cnt ? reinterpret_cast<const u32x4*>(ws.ap + (size_t)(2 * (r0 + p) + (j & 1)) * I)
                                    : nullptr};
    f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
    dec_core<BM_GROUP, 1, 1>(wsig, wsc, nullptr, arow, G, wave, nw, acc);
    reduce_waves<1, 1>(acc, red);
    if (wave == 0 && n < H) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = tb + 2 * (lane >> 4) + h;
        if (q < cnt) ws.o[(size_t)(r0 + q) * H + n] = acc[0][0][2 * h] + acc[0][0][2 * h + 1];
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

hipError_t launch_moe(const uint16_t* x, const float* logits, int T, int H, int I, int E, int top_k,
                      const uint64_t* gate_s, const uint16_t* gate_sc, const uint64_t* up_s,
                      const uint16_t* up_sc, const uint64_t* down_s, const uint16_t* down_sc, void* y,
                      int y_bf16, int32_t* ids, float* w, void* ws_ptr, hipStream_t st) {
  MoeWs ws = moe_carve(ws_ptr, T, H, I, E, top_k);
  const int64_t xruns = (int64_t)T * H / 32;
  const int maxact = (T * top_k < E) ? T * top_k : E;
  hipLaunchKernelGGL(k_moe_route, dim3((unsigned)(1 + (xruns + 255) / 256)), dim3(256), 0, st, logits, T, E, top_k,
                     x, xruns, ws, ids, w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_moe_gateup, dim3((I + 15) / 16, maxact), dim3(64 * dec_waves(H / 128)), 0, st, H, I,
                     reinterpret_cast<const uint4*>(gate_s), gate_sc, reinterpret_cast<const uint4*>(up_s), up_sc,
                     ws);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_moe_down, dim3((H + 15) / 16, maxact), dim3(64 * dec_waves(I / 128)), 0, st, H, I,
                     reinterpret_cast<const uint4*>(down_s), down_sc, ws);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)(((int64_t)T * H + 255) / 256)), dim3(256), 0, st, T, H, top_k,
                     ws, y, y_bf16);
  return hipGetLastError();
}

}  // namespace brq
