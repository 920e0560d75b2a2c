// Internal launchers of libbrq (host side). Arguments are validated by the
// C-ABI layer before any of these is called; each returns hipGetLastError()
// after its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace brq {

// ---- S1 quantiser --------------------------------------------------------
hipError_t launch_pack(const float* w, int64_t rows, int64_t cols, uint64_t* signs,
                       uint16_t* scales /* NULL: SIGN1 plane only */, hipStream_t st);

// ---- activation staging --------------------------------------------------
// bf16 [rows][K] -> fp16 [rows][K] in the permuted operand order (slot 2b+h of
// each run of 32 <- k = 16h+b), one workgroup per row, each row scaled by 2^rexp[row] (a power of
// two, 0 for rows whose largest |x| is in [2^-8, 2^15); scale = 0: always 0)
// so that every bf16 value is exact in fp16 whatever the row's range. xp
// NULL: only the exponents (scale must be 1 then).
hipError_t launch_prep_rows(const uint16_t* x, int64_t rows, int64_t K, uint16_t* xp, int* rexp, int scale,
                            hipStream_t st);
// fp16 vector [K] -> fp16 [K] in the permuted operand order.

// ---- group-128 product ----------------------------------------------------
// Few activation rows (M <= 64): split-K inside a workgroup, 16 output columns
// per workgroup. x: bf16 [M][K]. When M*K*2 <= kDecLdsBytes the activations
// are staged in LDS by the product kernel itself (one launch, no workspace);
// otherwise the split-K path below takes them.
constexpr int64_t kDecLdsBytes = 64 * 1024;
bool gemm_dec_in_lds(int64_t M, int64_t K);
hipError_t launch_gemm_dec(const uint16_t* x, int M, int N, int K, const uint64_t* signs,
                           const uint16_t* scales, void* y, int y_bf16, void* ws, hipStream_t st);
// Rows not taken by the one-launch path (M <= 64): bf16 matrix-core product
// over 64-column tiles, K split over the waves of a workgroup and, where the
// grid needs it, over workgroups (+ a slice-sum launch); `ws` holds
// mid_ws_bytes(M, N, K) bytes (the K-slice partials). Shapes whose activations
// or sign plane reach 4 GiB (mid_fits false) take the prefill path.
bool mid_fits(int64_t M, int64_t N, int64_t K);
size_t mid_ws_bytes(int64_t M, int64_t N, int64_t K);
size_t pf_ws_bytes(int64_t M, int64_t K);
// workspace of launch_gemm_dec (M <= 64)
inline size_t gemm_dec_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (gemm_dec_in_lds(M, K)) return 0;
  return mid_fits(M, N, K) ? mid_ws_bytes(M, N, K) : pf_ws_bytes(M, K);
}
hipError_t launch_gemm_mid(const uint16_t* x, int M, int N, int K, const uint64_t* signs,
                           const uint16_t* scales, void* y, int y_bf16, void* ws, hipStream_t st);
// Many activation rows (prefill): x staged to `ws` (pf_ws_bytes) as permuted
// fp16 with a power-of-two scale per row, then the 256 x 256 direct-to-LDS
// matrix-core kernel, which undoes the scales in its epilogue (pf_ws_bytes
// above).
hipError_t launch_gemm_pf(const uint16_t* x, int M, int N, int K, const uint64_t* signs,
                          const uint16_t* scales, void* y, int y_bf16, void* ws, hipStream_t st);
// The product on rows already staged by launch_prep_rows (xp, rexp), with one
// extra k-step per tile that adds a rank-r correction: lr_t [M][128] fp16
// ((x 2^rexp) V^T as hi | lo), lr_u [N][64] fp16 (U padded).
hipError_t launch_gemm_pf_lr(const uint16_t* xp, const int* rexp, int M, int N, int K, const uint64_t* signs,
                             const uint16_t* scales, const uint16_t* lr_t, const uint16_t* lr_u, void* y, int y_bf16,
                             hipStream_t st);
// y = x . (Wq + U V)^T, r <= 64; `ws` holds lr_ws_bytes(M, N, K) bytes.
size_t lr_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_lr(const uint16_t* x, int M, int N, int K, const uint64_t* signs,
                          const uint16_t* scales, const uint16_t* v, const uint16_t* u, int r, void* y,
                          int y_bf16, void* ws, hipStream_t st);

// ---- DBF chain -------------------------------------------------------------
// stage 1: h_s[M][r] (fp32) = D_mid (V (D_in x))
// stage 2: y[M][m] = D_out (U h_s), h_s taken as scaled fp16 pieces
hipError_t launch_dbf(const uint16_t* x, int M, int m, int n, int r, const uint16_t* d_in,
                      const uint64_t* v, const uint16_t* d_mid, const uint64_t* u,
                      const uint16_t* d_out, void* y, int y_bf16, void* ws, hipStream_t st);
size_t dbf_ws_bytes(int64_t M, int64_t m, int64_t n, int64_t r);
// the same chain over Q8 activation codes (int8 matrix cores, exact integer
// reductions, one exponent per row)
hipError_t launch_dbf_q8(const uint16_t* x, int M, int m, int n, int r, const uint16_t* d_in, const uint64_t* v,
                         const uint16_t* d_mid, const uint64_t* u, const uint16_t* d_out, void* y, int y_bf16,
                         void* ws, hipStream_t st);
size_t dbf_q8_ws_bytes(int64_t M, int64_t m, int64_t n, int64_t r);

// ---- routed MoE ------------------------------------------------------------
size_t moe_ws_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k);
// The layer with DBF experts (one record of five tensors per projection).
struct DbfFactors {
  const uint16_t* d_in;
  const uint64_t* v;
  const uint16_t* d_mid;
  const uint64_t* u;
  const uint16_t* d_out;
};
size_t moe_dbf_ws_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k, int64_t r);
hipError_t launch_moe_dbf(const uint16_t* x, const float* logits, int T, int H, int I, int E, int top_k, int r,
                          const DbfFactors& gate, const DbfFactors& up, const DbfFactors& down, void* y,
                          int y_bf16, int32_t* ids, float* w, void* ws, hipStream_t st);
hipError_t launch_moe(const uint16_t* x, const float* logits, int T, int H, int I, int E,
                      int top_k, const uint64_t* gate_s, const uint16_t* gate_sc,
                      const uint64_t* up_s, const uint16_t* up_sc, const uint64_t* down_s,
                      const uint16_t* down_sc, void* y, int y_bf16, int32_t* ids, float* w,
                      void* ws, hipStream_t st);

// ---- Kronecker rotation ----------------------------------------------------
// factor sizes n1, n2 in {32, 64, 96} with n1 * n2 <= 6144
bool kron_supported(int64_t n1, int64_t n2);
hipError_t launch_kron(const uint16_t* x, int M, int n1, int n2, const float* H, const float* R, uint16_t* y,
                       hipStream_t st);

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Status reporting shared by the entry points (abi.hip): report(s, msg) sets
// the calling thread's last-error text for a non-OK status and returns s;
// device_ok() checks that the current device is a gfx950.
}  // namespace brq
#include "../../include/brq.h"
namespace brq {
brq_status report(brq_status s, const char* msg);
brq_status device_ok();

}  // namespace brq
