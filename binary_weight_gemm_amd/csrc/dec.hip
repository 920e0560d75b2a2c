// Activation staging and the few-row (decode) group-128 product.
//
// y[m][n] = sum_g scale[n][g] * sum_{k in g} (+-x[m][k]): the activation x
// binary-weight product of "Banyan ..." (Abstract) on the group-128 format of
// "Behaviour-Relearned Quantization" (item 02), for M <= 64 activation rows.
#include "dec_core.h"
#include "kernels.h"

namespace brq {

// Activation staging for the tiled products: bf16 rows -> fp16 in the
// permuted operand order (slot 2b+h of each run of 32 <- k = 16h+b).
// One workgroup per row: the row's runs of 32 stay in registers (up to 4 per
// thread, K <= 32768) while the row's largest |x| is found; when it lies
// outside [2^-8, 2^15) the row is staged as fp16(x * 2^s) with s = 14 - its
// exponent (the largest value then in [2^14, 2^15), every bf16 value exact in
// fp16 or on its subnormal grid far below 2^-24 of the maximum), else s = 0;
// s goes to rexp[row] for the product's epilogue to undo. scale = 0 keeps
// every s at 0 (callers that add unscaled terms into the same accumulator).
__global__ __launch_bounds__(256) void k_prep_rows(const uint16_t* __restrict__ src, int K,
                                                   uint16_t* __restrict__ dst, int* __restrict__ rexp, int scale) {
  __shared__ uint32_t s_max[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int runs = K >> 5;
  const uint16_t* xr = src + (size_t)row * K;
  uint16_t* dr = dst + (size_t)row * K;
  uint4 q[4][4];
  uint32_t mx = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = tid + 256 * u;
    const uint4* s4 = reinterpret_cast<const uint4*>(xr + 32 * (t < runs ? t : 0));
#pragma unroll
    for (int h = 0; h < 4; ++h) q[u][h] = s4[h];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (tid + 256 * u >= runs) continue;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t w4[4] = {q[u][h].x, q[u][h].y, q[u][h].z, q[u][h].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max(w4[e] & 0x7fffu, (w4[e] >> 16) & 0x7fffu));
    }
  }
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) s_max[tid >> 6] = mx;
  __syncthreads();
  mx = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const int e = (int)(mx >> 7) - 127;  // exponent of the row's largest |x| (-127: all zero)
  const int sc = (scale && mx != 0 && (e >= 15 || e < -8)) ? 14 - e : 0;
  if (tid == 0) rexp[row] = sc;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = tid + 256 * u;
    if (t >= runs) continue;
    const uint32_t v[16] = {q[u][0].x, q[u][0].y, q[u][0].z, q[u][0].w, q[u][1].x, q[u][1].y, q[u][1].z, q[u][1].w,
                            q[u][2].x, q[u][2].y, q[u][2].z, q[u][2].w, q[u][3].x, q[u][3].y, q[u][3].z, q[u][3].w};
    uint32_t o[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      // element b lives in word b/2 (half b%2); element 16+b in word 8+b/2
      const uint32_t lo = (b & 1) ? (v[b >> 1] & 0xffff0000u) : (v[b >> 1] << 16);
      const uint32_t hi = (b & 1) ? (v[8 + (b >> 1)] & 0xffff0000u) : (v[8 + (b >> 1)] << 16);
      o[b] = (uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(__uint_as_float(lo), sc)) |
             ((uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(__uint_as_float(hi), sc)) << 16);
    }
    uint4* d = reinterpret_cast<uint4*>(dr + 32 * t);
    d[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d[1] = make_uint4(o[4], o[5], o[6], o[7]);
    d[2] = make_uint4(o[8], o[9], o[10], o[11]);
    d[3] = make_uint4(o[12], o[13], o[14], o[15]);
  }
}

// Rows longer than 32768 values: the same in two passes over the row (the
// largest |x| first, then the staging), runs of 32 per thread in turn; dst
// NULL: only the exponents.
__global__ __launch_bounds__(256) void k_prep_rows_long(const uint16_t* __restrict__ src, int K,
                                                        uint16_t* __restrict__ dst, int* __restrict__ rexp) {
  __shared__ uint32_t s_max[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int runs = K >> 5;
  const uint16_t* xr = src + (size_t)row * K;
  uint32_t mx = 0;
  for (int t = tid; t < runs; t += 256) {
    const uint4* s4 = reinterpret_cast<const uint4*>(xr + 32 * t);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint4 q = s4[h];
      const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max(w4[e] & 0x7fffu, (w4[e] >> 16) & 0x7fffu));
    }
  }
  mx = wave_max_u32(mx);
  if ((tid & 63) == 0) s_max[tid >> 6] = mx;
  __syncthreads();
  mx = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const int e = (int)(mx >> 7) - 127;
  const int sc = (mx != 0 && (e >= 15 || e < -8)) ? 14 - e : 0;
  if (tid == 0) rexp[row] = sc;
  if (!dst) return;
  uint16_t* dr = dst + (size_t)row * K;
  for (int t = tid; t < runs; t += 256) {
    const uint4* s4 = reinterpret_cast<const uint4*>(xr + 32 * t);
    const uint4 q0 = s4[0], q1 = s4[1], q2 = s4[2], q3 = s4[3];
    const uint32_t v[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                            q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
    uint32_t o[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const uint32_t lo = (b & 1) ? (v[b >> 1] & 0xffff0000u) : (v[b >> 1] << 16);
      const uint32_t hi = (b & 1) ? (v[8 + (b >> 1)] & 0xffff0000u) : (v[8 + (b >> 1)] << 16);
      o[b] = (uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(__uint_as_float(lo), sc)) |
             ((uint32_t)f32_to_f16_bits(__builtin_amdgcn_ldexpf(__uint_as_float(hi), sc)) << 16);
    }
    uint4* d = reinterpret_cast<uint4*>(dr + 32 * t);
    d[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d[1] = make_uint4(o[4], o[5], o[6], o[7]);
    d[2] = make_uint4(o[8], o[9], o[10], o[11]);
    d[3] = make_uint4(o[12], o[13], o[14], o[15]);
  }
}

hipError_t launch_prep_rows(const uint16_t* x, int64_t rows, int64_t K, uint16_t* xp, int* rexp, int scale,
                            hipStream_t st) {
  if (K <= 32768 && xp)
    hipLaunchKernelGGL(k_prep_rows, dim3((unsigned)rows), dim3(256), 0, st, x, (int)K, xp, rexp, scale);
  else
    hipLaunchKernelGGL(k_prep_rows_long, dim3((unsigned)rows), dim3(256), 0, st, x, (int)K, xp, rexp);
  return hipGetLastError();
}



// One-launch product for M <= 8: wave w owns chunks w*CPW .. w*CPW+CPW-1 of
// the reduction. It issues the loads of its activation slice (all MAXR row
// slots), of its sign words and of its scales before any wait, converts the
// slice into its own LDS region (no workgroup barrier: only this wave reads
// it) and runs its MFMAs as soon as its own data is in. SC16: the scales of
// the wave's 8 groups arrive as one 16-byte load per lane (needs CPW == 2 and
// G % 8 == 0); otherwise one 2-byte load per chunk. Only the lanes that hold
// rows m < M take part in the cross-wave sum (LDS, fixed wave order).
template <int CPW, int MAXR, bool SC16>
__global__ __launch_bounds__(1024) void k_gemm_dec_lds(const uint16_t* __restrict__ x, int M, int N, int K,
                                                       const uint4* __restrict__ signs,
                                                       const uint16_t* __restrict__ scales, void* __restrict__ y,
                                                       int y_bf16) {
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int n = blockIdx.x * 16 + j;
  const int G = K >> 7;
  const int nchunks = (G + 3) >> 2;
  const bool rok = n < N;
  const int nr = rok ? n : 0;  // clamped row; masked by bp.ok
  const uint4* wsig = signs + (size_t)nr * G;
  const uint16_t* wsc = scales + (size_t)nr * G;
  const int c0 = wave * CPW;
  uint4* xw = smem + (size_t)wave * CPW * MAXR * 64;
  f32x4* red = reinterpret_cast<f32x4*>(smem + (size_t)nw * CPW * MAXR * 64);
  f32x4 acc[1][1] = {{f32x4{0.f, 0.f, 0.f, 0.f}}};
  if (c0 < nchunks) {  // uniform across the wave
    WaveStage<ST_BF16, CPW, MAXR> ws;
    ws.load(M, K, c0, [&](int m) { return x + (size_t)m * K; });
    BPre<1, CPW> bp;
    uint4 sq = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int g = 4 * (c0 + c) + kb;
      const bool ok = rok && g < G;
      const int gi = ok ? g : 0;
      bp.ok[0][c] = ok;
      bp.d[0][c] = wsig[gi];
      if (!SC16) bp.s[0][c] = wsc[gi];
    }
    if (SC16) sq = *reinterpret_cast<const uint4*>(wsc + 4 * c0);
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    ws.store(xw);
    if (SC16) {
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        // halfword 4c + kb of the 8 scales
        const uint32_t wv = (kb & 2) ? ((c == 0) ? sq.y : sq.w) : ((c == 0) ? sq.x : sq.z);
        bp.s[0][c] = (kb & 1) ? (wv >> 16) : (wv & 0xffffu);
      }
    }
    const u32x4* xs = reinterpret_cast<const u32x4*>(xw);
    auto aop = [&](int tt, int g, int i) -> u32x4 {
      const int m = min(j, M - 1);
      return xs[(((g >> 2) - c0) * MAXR + m) * 64 + (g & 3) * 16 + i];
    };
    b_compute<BM_GROUP, 1, 1, CPW, true>(bp, nullptr, G, c0, 1, aop, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][0][i] = __builtin_amdgcn_ldexpf(acc[0][0][i], ws.unscale(i));
  }
  // lane (kb, j) holds rows 4*kb .. 4*kb+3 of column j
  const bool holds = 4 * kb < M;
  if (wave > 0 && holds) red[(wave - 1) * 64 + lane] = acc[0][0];
  __syncthreads();
  if (wave != 0 || !holds || !rok) return;
#pragma unroll
  for (int w = 1; w < 16; ++w)
    if (w < nw) acc[0][0] += red[(w - 1) * 64 + lane];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * kb + i;
    if (m < M) store_out(y, (size_t)m * N + n, acc[0][0][i], y_bf16);
  }
}

// ---- M = 1 on the fp8 x fp4 matrix cores ----------------------------------
// A weight operand of +-1 needs only its sign, and fp4 (e2m1) has no infinity
// or NaN: OR-ing 0b0111 onto a nibble whose top bit is a sign bit gives +-6.0.
// So one shift-or turns a 32-bit sign word into 8 fp4 operands (dword t of a
// lane's 32-k block holds, in nibble q, the sign of k = 4q + t).
//
// These matrix cores add each run of 8 products after aligning them to the
// largest one and truncating whatever falls more than 13 bits below it, so
// floating-point pieces of the activations would lose the low bits of small
// values next to large ones. The activations therefore enter as fixed-point
// digits, which makes every product and every partial sum exact: per wave
// slice, with 2^e the largest power of two in the slice (biased exponent
// ebs), each |x| is written as X * 2^(ebs - 150) with X = its 8-bit
// significand shifted into a 24-bit field (bits shifted out below are
// dropped: less than 2^-23 of the slice maximum), and the six 4-bit digits of
// X (most significant first) go to A rows 0..5 as sign-magnitude e4m3 codes.
// X is formed as the truncating fp32 -> u32 conversion of |x| * 2^(150 - ebs)
// (exact: a power-of-two scaling of a bf16 value, below 2^24), the same
// integer as shifting the 8-bit significand right by ebs - e.
// An e4m3 code c in 0..15 is the value c * 2^-9 (subnormals and the first
// normal binade), so the code of a digit is the digit itself plus the sign
// bit. Row p carries block exponent ebs - 2 - 4p and the weights 135, which
// puts row p's product at 6 * sum(+-digit_p) * 2^(ebs - 130 - 4p): integers
// times one power of two, exact in fp32. Rows 6..15 read an all-zero LDS row,
// so every lane simply adds its four output rows. One MFMA covers one scale
// group of 16 columns; the group scale and the 1/6 are applied in fp32
// afterwards.
//
// Layout facts of that MFMA (fp8 A, fp4 B): A lane l supplies row l%16 with
// bytes 0..15 = k 16*(l/16).. and bytes 16..31 = k 64+16*(l/16)..; B lane l
// supplies column l%16 with nibble p = k 32*(l/16)+p; the A block exponent of
// (row r, k block b) comes from lane r + 16b; D as for the 16x16 f16 MFMA.
// A lane loads group 4c+kb of its column; four permlane swaps transpose the
// 4 x 4 (group, word) block of the four lanes of a column so that MFMA i gets
// word kb of group i.
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int F4_DIGITS = 6;
constexpr int F4_GROUP = (F4_DIGITS + 1) * 128;  // LDS bytes of one group: six digit rows of 128 codes, a zero row
constexpr int F4_CHUNK = 4 * F4_GROUP;     // LDS bytes of one chunk of four groups

// (group, word) transpose across the four 16-lane rows: on entry register w
// of row g holds word w of group g; on exit register i of row b holds word b
// of group i.
__device__ __forceinline__ void transpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3) {
  auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = c[0];
  r1 = c[1];
  r2 = d[0];
  r3 = d[1];
}

template <int CPW, int NT>
__global__ __launch_bounds__(1024) void k_gemm_dec_f4(const uint16_t* __restrict__ x, int N, int K,
                                                      const uint4* __restrict__ signs,
                                                      const uint16_t* __restrict__ scales, void* __restrict__ y,
                                                      int y_bf16) {
  extern __shared__ uint4 smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int G = K >> 7;
  const int nchunks = (G + 3) >> 2;
  const int c0 = wave * CPW;
  uint8_t* xw = reinterpret_cast<uint8_t*>(smem) + (size_t)wave * CPW * F4_CHUNK;  // [chunk][group][digit][128]
  float* red = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem) + (size_t)nw * CPW * F4_CHUNK);
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  if (c0 < nchunks) {  // uniform across the wave
    // ---- loads: activations (8 per lane per chunk), sign words, 4 scales per chunk
    uint4 xv[CPW];
    uint4 sg[NT][CPW];
    uint2 sc[NT][CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int k0 = (c0 + c) * 512 + 8 * lane;
      xv[c] = *reinterpret_cast<const uint4*>(x + (k0 < K ? k0 : 0));
    }
    size_t row[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = (blockIdx.x * NT + t) * 16 + j;
      row[t] = (size_t)(n < N ? n : 0) * G;
    }
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int g = 4 * (c0 + c) + kb, gs = 4 * (c0 + c);
        sg[t][c] = signs[row[t] + (g < G ? g : 0)];
        sc[t][c] = *reinterpret_cast<const uint2*>(scales + row[t] + (gs < G ? gs : 0));
      }
    __builtin_amdgcn_sched_barrier(0);  // every load above issues before any wait below
    // a slot past the last chunk (the last wave when CPW does not divide the
    // chunk count) holds zeros: no digits, no part in the exponent
#pragma unroll
    for (int c = 0; c < CPW; ++c)
      if (c0 + c >= nchunks) xv[c] = make_uint4(0u, 0u, 0u, 0u);
    // ---- slice exponent: biased exponent of the largest |x| of the wave slice
    uint32_t mx = 0;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint32_t w4[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) mx = max(mx, max(w4[h] & 0x7fffu, (w4[h] >> 16) & 0x7fffu));
    }
    mx = wave_max_u32(mx);
    // at least 24, so that a zero (or bf16 subnormal, dropped: below 2^-126)
    // shifts its implicit bit out of the field entirely
    const uint32_t ebs = max(mx >> 7, 24u);
    const float S = __uint_as_float((277u - ebs) << 23);  // 2^(150 - ebs), a normal fp32 for ebs in 24..254
    // ---- digit codes in the operand order: lane L's 8 values are k = 8L .. 8L+7
    // of the chunk (group L/16, word (L%16)/4); value e lands at in-word
    // position 8*(e%4) + 2*(L%4) + e/4 of each digit row
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const uint32_t w4[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wp = (e & 1) ? (w4[e >> 1] & 0xffff0000u) : (w4[e >> 1] << 16);  // the bf16 as fp32
        const uint32_t X = (uint32_t)(fabsf(__uint_as_float(wp)) * S);  // 24-bit magnitude field
        const uint32_t sr = (wp >> 31) * 0x808080u;                        // sign bit of each code byte
        lo[e] = (X & 0x0f0f0fu) | sr;         // nibbles 0, 2, 4 -> bytes 0, 1, 2
        hi[e] = ((X >> 4) & 0x0f0f0fu) | sr;  // nibbles 1, 3, 5 -> bytes 0, 1, 2
      }
      if (lane < 32)  // the zero row of each group: 16 bytes per lane
        *reinterpret_cast<uint4*>(xw + c * F4_CHUNK + (lane >> 3) * F4_GROUP + F4_DIGITS * 128 + 16 * (lane & 7)) =
            make_uint4(0u, 0u, 0u, 0u);
      uint8_t* base = xw + c * F4_CHUNK + (lane >> 4) * F4_GROUP + 32 * ((lane & 15) >> 2) + 2 * (lane & 3);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // values t and t+4 side by side: byte permutes pair their codes per nibble
        const uint32_t l02 = __builtin_amdgcn_perm(lo[t + 4], lo[t], 0x05010400u);
        const uint32_t l4 = __builtin_amdgcn_perm(lo[t + 4], lo[t], 0x0c0c0602u);
        const uint32_t h13 = __builtin_amdgcn_perm(hi[t + 4], hi[t], 0x05010400u);
        const uint32_t h5 = __builtin_amdgcn_perm(hi[t + 4], hi[t], 0x0c0c0602u);
        // digit p (most significant first) is nibble 5 - p
        auto put = [&](int nib, uint32_t v16) {
          *reinterpret_cast<uint16_t*>(base + (F4_DIGITS - 1 - nib) * 128 + 8 * t) = (uint16_t)v16;
        };
        put(0, l02);
        put(2, l02 >> 16);
        put(4, l4);
        put(1, h13);
        put(3, h13 >> 16);
        put(5, h5);
      }
    }
    const int prow = j < F4_DIGITS ? j : F4_DIGITS;  // lanes 6..15 read the zero row
    // the zero row takes scale 2^0: at ebs = 25 its digit form ebs - 26
    // would be the E8M0 NaN code 0xff
    const int sa = prow < F4_DIGITS ? (int)ebs - 2 - 4 * prow : 127;
    // ---- products (the last wave's slots past the last chunk take no part)
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      if (c0 + c >= nchunks) break;  // uniform across the wave
      const uint8_t* ab = xw + c * F4_CHUNK + prow * 128 + 16 * kb;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint32_t w0 = sg[t][c].x, w1 = sg[t][c].y, w2 = sg[t][c].z, w3 = sg[t][c].w;
        transpose4(w0, w1, w2, w3);
        const uint32_t wi[4] = {w0, w1, w2, w3};
        const uint32_t s4[4] = {sc[t][c].x & 0xffffu, sc[t][c].x >> 16, sc[t][c].y & 0xffffu, sc[t][c].y >> 16};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(ab + i * F4_GROUP);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(ab + i * F4_GROUP + 64);
          i32x8 A, B;
          A[0] = a0[0]; A[1] = a0[1]; A[2] = a0[2]; A[3] = a0[3];
          A[4] = a1[0]; A[5] = a1[1]; A[6] = a1[2]; A[7] = a1[3];
          B[0] = (int)((wi[i] << 3) | 0x77777777u);
          B[1] = (int)((wi[i] << 2) | 0x77777777u);
          B[2] = (int)((wi[i] << 1) | 0x77777777u);
          B[3] = (int)(wi[i] | 0x77777777u);
          B[4] = 0; B[5] = 0; B[6] = 0; B[7] = 0;
          const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 4, 0,
                                                                           sa, 0, 135);
          // K % 512 == 0: every group of the chunk exists; columns past N read
          // row 0 (finite) and are never stored. Lanes 0..15 hold digit rows
          // 0..3 of column j, lanes 16..31 rows 4..7 (6, 7 zero), the rest zeros.
          acc[t] = fmaf(f16_bits_to_f32(s4[i]), (d[0] + d[1]) + (d[2] + d[3]), acc[t]);
        }
      }
    }
  }
  // digit rows 4 and 5 (lanes 16..31) join rows 0..3 (lanes 0..15)
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] += __shfl_down(acc[t], 16, 64);
  if (wave > 0 && kb == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[((wave - 1) * NT + t) * 16 + j] = acc[t];
  }
  __syncthreads();
  if (wave != 0 || kb != 0) return;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float v = acc[t];
    for (int w = 1; w < nw; ++w) v += red[((w - 1) * NT + t) * 16 + j];
    const int n = (blockIdx.x * NT + t) * 16 + j;
    if (n < N) store_out(y, (size_t)n, v / 6.0f, y_bf16);
  }
}

// staged row slots for M activation rows
static int dec_maxr(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

// staging budget of the one-launch path: up to 128 KiB of LDS (beyond 64 KiB
// the kernel needs the per-function opt-in below)
constexpr int64_t kDecLdsBig = 128 * 1024;

// Split of the one-launch path: chunks of 512 over at most 16 waves, two
// chunks per wave when there are at least four (one chunk each below), more
// only when 16 waves of two do not cover K. The staged slices
// (waves * cpw * maxr KiB) must fit the LDS budget.
static bool dec_lds_split(int64_t M, int64_t K, DecSplit& sp) {
  if (M > 8) return false;
  const int64_t chunks = (K / 128 + 3) / 4;
  int64_t cpw = chunks >= 4 ? 2 : 1;
  if ((chunks + cpw - 1) / cpw > 16) cpw = (chunks + 15) / 16;
  if (cpw > 8) return false;
  sp.cpw = (int)cpw;
  sp.waves = (int)((chunks + cpw - 1) / cpw);
  return (int64_t)sp.waves * sp.cpw * dec_maxr(M) * 1024 <= kDecLdsBig;
}

bool gemm_dec_in_lds(int64_t M, int64_t K) {
  DecSplit sp;
  return dec_lds_split(M, K, sp);
}

template <int MAXR>
static void gemm_dec_lds(const uint16_t* x, int M, int N, int K, const uint4* s4, const uint16_t* scales, void* y,
                         int y_bf16, hipStream_t st) {
  DecSplit sp;
  dec_lds_split(M, K, sp);
  const size_t lds = (size_t)sp.waves * sp.cpw * MAXR * 1024 + (size_t)(sp.waves - 1) * 64 * 16;
  const dim3 grid((N + 15) / 16), block(64 * sp.waves);
  auto opt_in = [&](const void* fn) {
    if (lds > 64 * 1024) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  };
  if (sp.cpw == 2 && (K / 128) % 8 == 0) {
    opt_in(reinterpret_cast<const void*>(&k_gemm_dec_lds<2, MAXR, true>));
    hipLaunchKernelGGL((k_gemm_dec_lds<2, MAXR, true>), grid, block, lds, st, x, M, N, K, s4, scales, y, y_bf16);
  } else {
    BRQ_CPW_SWITCH(sp.cpw, opt_in(reinterpret_cast<const void*>(&k_gemm_dec_lds<CPW, MAXR, false>));
                   hipLaunchKernelGGL((k_gemm_dec_lds<CPW, MAXR, false>), grid, block, lds, st, x, M, N, K, s4,
                                      scales, y, y_bf16));
  }
}

// The fp8 x fp4 path takes M = 1 when the scale groups come in whole chunks
// of four (K % 512 == 0) and the digit rows of the workgroup's slices fit the
// LDS (K <= 23040: up to 45 chunks of 3.5 KiB); longer rows take the fp16 one-launch
// path. Two column tiles per workgroup when that still leaves well over one
// workgroup per compute unit (the activation digits are then shared by both
// tiles). One chunk per wave up to 16 waves (the less a wave computes after
// its last sign word lands, the shorter the tail), more beyond.
constexpr size_t kF4Lds = 160 * 1024;

static bool f4_split(int64_t K, int64_t N, DecSplit& sp, int& nt, size_t& lds) {
  if (K % 512 != 0) return false;
  const int64_t chunks = K / 512;
  const int64_t cpw = chunks <= 16 ? 1 : (chunks + 15) / 16;
  if (cpw > 8) return false;
  sp.cpw = (int)cpw;
  sp.waves = (int)((chunks + cpw - 1) / cpw);
  const int64_t tiles = (N + 15) / 16;
  nt = tiles >= 768 ? 2 : 1;
  lds = (size_t)sp.waves * sp.cpw * F4_CHUNK + (size_t)(sp.waves - 1) * nt * 16 * 4;
  return lds <= kF4Lds;
}

static void gemm_dec_f4(const uint16_t* x, int N, int K, const uint4* s4, const uint16_t* scales, void* y,
                        int y_bf16, hipStream_t st) {
  DecSplit sp;
  int nt;
  size_t lds;
  f4_split(K, N, sp, nt, lds);
  const int tiles = (N + 15) / 16;
  const dim3 grid((tiles + nt - 1) / nt), block(64 * sp.waves);
  auto opt_in = [&](const void* fn) {
    if (lds > 64 * 1024) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  };
  if (nt == 2) {
    BRQ_CPW_SWITCH(sp.cpw, opt_in(reinterpret_cast<const void*>(&k_gemm_dec_f4<CPW, 2>));
                   hipLaunchKernelGGL((k_gemm_dec_f4<CPW, 2>), grid, block, lds, st, x, N, K, s4, scales, y, y_bf16));
  } else {
    BRQ_CPW_SWITCH(sp.cpw, opt_in(reinterpret_cast<const void*>(&k_gemm_dec_f4<CPW, 1>));
                   hipLaunchKernelGGL((k_gemm_dec_f4<CPW, 1>), grid, block, lds, st, x, N, K, s4, scales, y, y_bf16));
  }
}

hipError_t launch_gemm_dec(const uint16_t* x, int M, int N, int K, const uint64_t* signs, const uint16_t* scales,
                           void* y, int y_bf16, void* ws, hipStream_t st) {
  const uint4* s4 = reinterpret_cast<const uint4*>(signs);
  DecSplit sp;
  int nt;
  size_t lds;
  if (M == 1 && f4_split(K, N, sp, nt, lds)) {
    gemm_dec_f4(x, N, K, s4, scales, y, y_bf16, st);
    return hipGetLastError();
  }
  if (gemm_dec_in_lds(M, K)) {
    if (M == 1) gemm_dec_lds<1>(x, M, N, K, s4, scales, y, y_bf16, st);
    else if (M <= 2) gemm_dec_lds<2>(x, M, N, K, s4, scales, y, y_bf16, st);
    else if (M <= 4) gemm_dec_lds<4>(x, M, N, K, s4, scales, y, y_bf16, st);
    else gemm_dec_lds<8>(x, M, N, K, s4, scales, y, y_bf16, st);
    return hipGetLastError();
  }
  if (!mid_fits(M, N, K)) return launch_gemm_pf(x, M, N, K, signs, scales, y, y_bf16, ws, st);
  return launch_gemm_mid(x, M, N, K, signs, scales, y, y_bf16, ws, st);
}

}  // namespace brq
