// C-ABI entry points of libbrq: argument validation on the host, then dispatch
// to the gfx950 kernels. Every check that can fail runs before the first HIP
// call, so invalid arguments never touch the device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/brq.h"
#include "kernels.h"
#include "gsync.h"

namespace {

thread_local std::string g_last_error;

brq_status fail(brq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

brq_status ok() {
  g_last_error.clear();
  return BRQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every index inside 32-bit element counts per row

// gfx950 check, cached per device id
std::mutex g_dev_mu;
int g_dev_state[64];  // 0 unknown, 1 gfx950, 2 other

// launch-failure injection (brq_debug_fail_launches): calls still to fail
std::atomic<int> g_inject{0};

bool take_injected() {
  int n = g_inject.load(std::memory_order_relaxed);
  while (n > 0)
    if (g_inject.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) return true;
  return false;
}

// Every entry point calls this after its arguments passed and right before it
// enqueues anything.
brq_status check_device() {
  if (take_injected()) return fail(BRQ_E_HIP, "injected launch failure (brq_debug_fail_launches)");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(BRQ_E_DEVICE, "no current HIP device");
  }
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_state[dev] == 1) return BRQ_OK;
    if (g_dev_state[dev] == 2) return fail(BRQ_E_DEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(BRQ_E_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
  }
  const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    g_dev_state[dev] = good ? 1 : 2;
  }
  if (!good) return fail(BRQ_E_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return BRQ_OK;
}

brq_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BRQ_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// An enum argument from a C caller can hold any int; reading it as the C++
// enum type is only defined for the enumerators' range, so the raw value is
// taken from the argument's bytes and checked as an int.
template <class E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool dtype_ok(const brq_dtype& d) {
  const int v = enum_value(d);
  return v == BRQ_BF16 || v == BRQ_F32;
}

size_t gemm_ws(int64_t M, int64_t N, int64_t K) {
  if (M <= 64) return brq::gemm_dec_ws_bytes(M, N, K);
  return brq::pf_ws_bytes(M, K);
}

}  // namespace

namespace brq {
// for entry points defined in other source files of the library
brq_status report(brq_status s, const char* msg) { return s == BRQ_OK ? ok() : fail(s, "%s", msg); }
brq_status device_ok() { return check_device(); }
}  // namespace brq

extern "C" {

int brq_abi_version(void) { return BRQ_ABI_VERSION; }

const char* brq_status_str(brq_status s) {
  switch (enum_value(s)) {
    case BRQ_OK: return "BRQ_OK";
    case BRQ_E_NULL: return "BRQ_E_NULL";
    case BRQ_E_SHAPE: return "BRQ_E_SHAPE";
    case BRQ_E_ALIGN: return "BRQ_E_ALIGN";
    case BRQ_E_DTYPE: return "BRQ_E_DTYPE";
    case BRQ_E_WORKSPACE: return "BRQ_E_WORKSPACE";
    case BRQ_E_DEVICE: return "BRQ_E_DEVICE";
    case BRQ_E_HIP: return "BRQ_E_HIP";
  }
  return "BRQ_E_UNKNOWN";
}

const char* brq_last_error(void) { return g_last_error.c_str(); }

brq_status brq_debug_fail_launches(int32_t count) {
  if (count < 0) return fail(BRQ_E_SHAPE, "brq_debug_fail_launches: count %d < 0", (int)count);
  g_inject.store(count, std::memory_order_relaxed);
  return ok();
}

brq_status brq_set_decode_fusion(brq_fusion mode, uint32_t spin_limit) {
  const int m = enum_value(mode);
  if (m != BRQ_FUSION_DEFAULT && m != BRQ_FUSION_OFF && m != BRQ_FUSION_ON)
    return fail(BRQ_E_SHAPE, "brq_set_decode_fusion: unknown mode %d", m);
  brq::set_fusion(m, spin_limit);
  return ok();
}

size_t brq_sign_words(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 64 || cols % 64) return 0;
  return (size_t)rows * (size_t)(cols / 64);
}

size_t brq_scale_count(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 128 || cols % 128) return 0;
  return (size_t)rows * (size_t)(cols / 128);
}

brq_status brq_pack(const float* w, int64_t rows, int64_t cols, uint64_t* signs, uint16_t* scales,
                    void* stream) {
  if (!w || !signs) return fail(BRQ_E_NULL, "brq_pack: w and signs must not be NULL");
  if (rows < 1 || rows > kMaxDim) return fail(BRQ_E_SHAPE, "brq_pack: rows=%lld out of range", (long long)rows);
  const int64_t mult = scales ? 128 : 64;
  if (cols < mult || cols > kMaxDim || cols % mult)
    return fail(BRQ_E_SHAPE, "brq_pack: cols=%lld must be a positive multiple of %lld", (long long)cols,
                (long long)mult);
  if (!aligned(w, 16) || !aligned(signs, 16) || (scales && !aligned(scales, 16)))
    return fail(BRQ_E_ALIGN, "brq_pack: buffers must be 16-byte aligned");
  brq_status s = check_device();
  if (s != BRQ_OK) return s;
  return hip_result(brq::launch_pack(w, rows, cols, signs, scales, (hipStream_t)stream), "brq_pack");
}

size_t brq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 128 || K % 128) return 0;
  return gemm_ws(M, N, K);
}

brq_status brq_gemm(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint64_t* signs,
                    const uint16_t* scales, void* y, brq_dtype y_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !signs || !scales || !y) return fail(BRQ_E_NULL, "brq_gemm: x, signs, scales and y must not be NULL");
  if (M < 1 || N < 1 || M > kMaxDim || N > kMaxDim)
    return fail(BRQ_E_SHAPE, "brq_gemm: M=%lld N=%lld out of range", (long long)M, (long long)N);
  if (K < 128 || K > kMaxDim || K % 128)
    return fail(BRQ_E_SHAPE, "brq_gemm: K=%lld must be a positive multiple of 128", (long long)K);
  if (!dtype_ok(y_dtype)) return fail(BRQ_E_DTYPE, "brq_gemm: unknown y_dtype %d", enum_value(y_dtype));
  if (!aligned(x, 16) || !aligned(signs, 16) || !aligned(scales, 16) || !aligned(y, 16))
    return fail(BRQ_E_ALIGN, "brq_gemm: x, signs, scales and y must be 16-byte aligned");
  const size_t need = gemm_ws(M, N, K);
  if (need && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(BRQ_E_WORKSPACE, "brq_gemm: workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  brq_status s = check_device();
  if (s != BRQ_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const int yb = y_dtype == BRQ_BF16;
  if (M <= 64)
    return hip_result(brq::launch_gemm_dec(x, (int)M, (int)N, (int)K, signs, scales, y, yb, ws, st), "brq_gemm");
  return hip_result(brq::launch_gemm_pf(x, (int)M, (int)N, (int)K, signs, scales, y, yb, ws, st), "brq_gemm");
}

size_t brq_gemm_lr_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t r) {
  if (M < 1 || N < 1 || K < 128 || K % 128 || r < 1 || r > 64) return 0;
  return brq::lr_ws_bytes(M, N, K);
}

brq_status brq_gemm_lr(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint64_t* signs,
                       const uint16_t* scales, const uint16_t* v, const uint16_t* u, int64_t r, void* y,
                       brq_dtype y_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !signs || !scales || !v || !u || !y)
    return fail(BRQ_E_NULL, "brq_gemm_lr: x, signs, scales, v, u and y must not be NULL");
  if (M < 1 || N < 1 || M > kMaxDim || N > kMaxDim)
    return fail(BRQ_E_SHAPE, "brq_gemm_lr: M=%lld N=%lld out of range", (long long)M, (long long)N);
  if (K < 128 || K > kMaxDim || K % 128)
    return fail(BRQ_E_SHAPE, "brq_gemm_lr: K=%lld must be a positive multiple of 128", (long long)K);
  if (r < 1 || r > 64) return fail(BRQ_E_SHAPE, "brq_gemm_lr: rank r=%lld must be in 1..64", (long long)r);
  if (!dtype_ok(y_dtype)) return fail(BRQ_E_DTYPE, "brq_gemm_lr: unknown y_dtype %d", enum_value(y_dtype));
  if (!aligned(x, 16) || !aligned(signs, 16) || !aligned(scales, 16) || !aligned(y, 16) || !aligned(v, 2) ||
      !aligned(u, 2))
    return fail(BRQ_E_ALIGN, "brq_gemm_lr: x, signs, scales and y must be 16-byte aligned, v and u 2-byte");
  const size_t need = brq::lr_ws_bytes(M, N, K);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(BRQ_E_WORKSPACE, "brq_gemm_lr: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                ws_bytes);
  brq_status s = check_device();
  if (s != BRQ_OK) return s;
  return hip_result(brq::launch_gemm_lr(x, (int)M, (int)N, (int)K, signs, scales, v, u, (int)r, y,
                                        y_dtype == BRQ_BF16, ws, (hipStream_t)stream),
                    "brq_gemm_lr");
}

size_t brq_dbf_workspace_bytes(int64_t M, int64_t m, int64_t n, int64_t r) {
  if (M < 1 || m < 1 || n < 128 || r < 128 || n % 128 || r % 128) return 0;
  return brq::dbf_ws_bytes(M, m, n, r);
}

brq_status brq_dbf_gemm(const uint16_t* x, int64_t M, int64_t m, int64_t n, int64_t r, const uint16_t* d_in,
                        const uint64_t* v, const uint16_t* d_mid, const uint64_t* u, const uint16_t* d_out,
                        void* y, brq_dtype y_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !d_in || !v || !d_mid || !u || !d_out || !y)
    return fail(BRQ_E_NULL, "brq_dbf_gemm: x, d_in, v, d_mid, u, d_out and y must not be NULL");
  if (M < 1 || m < 1 || M > kMaxDim || m > kMaxDim)
    return fail(BRQ_E_SHAPE, "brq_dbf_gemm: M=%lld m=%lld out of range", (long long)M, (long long)m);
  if (n < 128 || r < 128 || n > kMaxDim || r > kMaxDim || n % 128 || r % 128)
    return fail(BRQ_E_SHAPE, "brq_dbf_gemm: n=%lld and r=%lld must be positive multiples of 128", (long long)n,
                (long long)r);
  if (!dtype_ok(y_dtype)) return fail(BRQ_E_DTYPE, "brq_dbf_gemm: unknown y_dtype %d", enum_value(y_dtype));
  if (!aligned(x, 16) || !aligned(v, 16) || !aligned(u, 16) || !aligned(y, 16) || !aligned(d_in, 16) ||
      !aligned(d_mid, 2) || !aligned(d_out, 2))
    return fail(BRQ_E_ALIGN, "brq_dbf_gemm: x, v, u, y and d_in must be 16-byte aligned");
  const size_t need = brq::dbf_ws_bytes(M, m, n, r);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(BRQ_E_WORKSPACE, "brq_dbf_gemm: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                ws_bytes);
  brq_status s = check_device();
  if (s != BRQ_OK) return s;
  return hip_result(brq::launch_dbf(x, (int)M, (int)m, (int)n, (int)r, d_in, v, d_mid, u, d_out, y,
                                    y_dtype == BRQ_BF16, ws, (hipStream_t)stream),
                    "brq_dbf_gemm");
}

// longest Q8 reduction: 127 * 131072 < 2^24, so every integer sum converts to
// fp32 exactly
constexpr int64_t kMaxQ8Red = 131072;

size_t brq_dbf_q8_workspace_bytes(int64_t M, int64_t m, int64_t n, int64_t r) {
  if (M < 1 || m < 1 || n < 128 || r < 128 || n % 128 || r % 128 || M > kMaxDim || m > kMaxDim || n > kMaxQ8Red ||
      r > kMaxQ8Red)
    return 0;
  return brq::dbf_q8_ws_bytes(M, m, n, r);
}

brq_status brq_dbf_gemm_q8(const uint16_t* x, int64_t M, int64_t m, int64_t n, int64_t r, const uint16_t* d_in,
                           const uint64_t* v, const uint16_t* d_mid, const uint64_t* u, const uint16_t* d_out,
                           void* y, brq_dtype y_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !d_in || !v || !d_mid || !u || !d_out || !y)
    return fail(BRQ_E_NULL, "brq_dbf_gemm_q8: x, d_in, v, d_mid, u, d_out and y must not be NULL");
  if (M < 1 || m < 1 || M > kMaxDim || m > kMaxDim)
    return fail(BRQ_E_SHAPE, "brq_dbf_gemm_q8: M=%lld m=%lld out of range", (long long)M, (long long)m);
  if (n < 128 || r < 128 || n > kMaxQ8Red || r > kMaxQ8Red || n % 128 || r % 128)
    return fail(BRQ_E_SHAPE, "brq_dbf_gemm_q8: n=%lld and r=%lld must be multiples of 128 in [128, 131072]",
                (long long)n, (long long)r);
  const int64_t wide = m > r ? m : r;
  if (((M + 127) / 128) * ((wide + 127) / 128) > (int64_t)INT32_MAX)
    return fail(BRQ_E_SHAPE, "brq_dbf_gemm_q8: M=%lld with max(m, r)=%lld needs more than 2^31 tiles", (long long)M,
                (long long)wide);
  if (!dtype_ok(y_dtype)) return fail(BRQ_E_DTYPE, "brq_dbf_gemm_q8: unknown y_dtype %d", enum_value(y_dtype));
  if (!aligned(x, 16) || !aligned(v, 16) || !aligned(u, 16) || !aligned(y, 4) || !aligned(d_in, 16) ||
      !aligned(d_mid, 16) || !aligned(d_out, 2))
    return fail(BRQ_E_ALIGN, "brq_dbf_gemm_q8: x, v, u, d_in and d_mid must be 16-byte aligned, y 4-byte");
  const size_t need = brq::dbf_q8_ws_bytes(M, m, n, r);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(BRQ_E_WORKSPACE, "brq_dbf_gemm_q8: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                ws_bytes);
  brq_status s = check_device();
  if (s != BRQ_OK) return s;
  return hip_result(brq::launch_dbf_q8(x, (int)M, (int)m, (int)n, (int)r, d_in, v, d_mid, u, d_out, y,
                                       y_dtype == BRQ_BF16, ws, (hipStream_t)stream),
                    "brq_dbf_gemm_q8");
}

size_t brq_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k) {
  if (T < 1 || T > 256 || H < 128 || I < 128 || H > 32768 || I > 2048 || H % 128 || I % 128 || E < 1 ||
      E > 1024 || top_k < 1 ||
      top_k > 16 || top_k > E)
    return 0;
  return brq::moe_ws_bytes(T, H, I, E, top_k);
}

brq_status brq_moe_ffn(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t I, int64_t E,
                       int64_t top_k, const uint64_t* gate_s, const uint16_t* gate_sc, const uint64_t* up_s,
                       const uint16_t* up_sc, const uint64_t* down_s, const uint16_t* down_sc, void* y,
                       brq_dtype y_dtype, int32_t* ids, float* w, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !logits || !gate_s || !gate_sc || !up_s || !up_sc || !down_s || !down_sc || !y)
    return fail(BRQ_E_NULL, "brq_moe_ffn: inputs, weights and y must not be NULL");
  if (T < 1 || T > 256) return fail(BRQ_E_SHAPE, "brq_moe_ffn: T=%lld must be in [1, 256]", (long long)T);
  if (E < 1 || E > 1024) return fail(BRQ_E_SHAPE, "brq_moe_ffn: E=%lld must be in [1, 1024]", (long long)E);
  if (top_k < 1 || top_k > 16 || top_k > E)
    return fail(BRQ_E_SHAPE, "brq_moe_ffn: top_k=%lld must be in [1, min(E, 16)]", (long long)top_k);
  if (H < 128 || I < 128 || H > 32768 || I > 2048 || H % 128 || I % 128)
    return fail(BRQ_E_SHAPE, "brq_moe_ffn: H=%lld and I=%lld must be multiples of 128, H <= 32768, I <= 2048",
                (long long)H, (long long)I);
  if (!dtype_ok(y_dtype)) return fail(BRQ_E_DTYPE, "brq_moe_ffn: unknown y_dtype %d", enum_value(y_dtype));
  if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(gate_s, 16) || !aligned(up_s, 16) || !aligned(down_s, 16) ||
      !aligned(gate_sc, 16) || !aligned(up_sc, 16) || !aligned(down_sc, 16) || !aligned(y, 16) ||
      (ids && !aligned(ids, 4)) || (w && !aligned(w, 4)))
    return fail(BRQ_E_ALIGN, "brq_moe_ffn: weight planes, scales, x and y must be 16-byte aligned");
  const size_t need = brq::moe_ws_bytes(T, H, I, E, top_k);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(BRQ_E_WORKSPACE, "brq_moe_ffn: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                ws_bytes);
  brq_status s = check_device();
  if (s != BRQ_OK) return s;
  return hip_result(brq::launch_moe(x, logits, (int)T, (int)H, (int)I, (int)E, (int)top_k, gate_s, gate_sc, up_s,
                                    up_sc, down_s, down_sc, y, y_dtype == BRQ_BF16, ids, w, ws, (hipStream_t)stream),
                    "brq_moe_ffn");
}

size_t brq_moe_dbf_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t top_k, int64_t r) {
  if (T < 1 || T > 256 || E < 1 || E > 1024 || top_k < 1 || top_k > 16 || top_k > E) return 0;
  if (H < 128 || I < 128 || r < 128 || H % 128 || I % 128 || r % 128 || H > 8192 || I > 2048 || r > 2048) return 0;
  return brq::moe_dbf_ws_bytes(T, H, I, E, top_k, r);
}

brq_status brq_moe_dbf_ffn(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t I, int64_t E,
                           int64_t top_k, int64_t r, const brq_dbf_factors* gate, const brq_dbf_factors* up,
                           const brq_dbf_factors* down, void* y, brq_dtype y_dtype, int32_t* ids, float* w, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!x || !logits || !gate || !up || !down || !y)
    return fail(BRQ_E_NULL, "brq_moe_dbf_ffn: x, logits, the three records and y must not be NULL");
  const brq_dbf_factors* recs[3] = {gate, up, down};
  for (const brq_dbf_factors* f : recs)
    if (!f->d_in || !f->v || !f->d_mid || !f->u || !f->d_out)
      return fail(BRQ_E_NULL, "brq_moe_dbf_ffn: every tensor of the gate, up and down records must be set");
  if (T < 1 || T > 256) return fail(BRQ_E_SHAPE, "brq_moe_dbf_ffn: T=%lld must be in [1, 256]", (long long)T);
  if (E < 1 || E > 1024) return fail(BRQ_E_SHAPE, "brq_moe_dbf_ffn: E=%lld must be in [1, 1024]", (long long)E);
  if (top_k < 1 || top_k > 16 || top_k > E)
    return fail(BRQ_E_SHAPE, "brq_moe_dbf_ffn: top_k=%lld must be in [1, min(E, 16)]", (long long)top_k);
  if (H < 128 || I < 128 || r < 128 || H % 128 || I % 128 || r % 128 || H > 8192 || I > 2048 || r > 2048)
    return fail(BRQ_E_SHAPE,
                "brq_moe_dbf_ffn: H=%lld, I=%lld, r=%lld must be multiples of 128 with H <= 8192, I <= 2048, "
                "r <= 2048",
                (long long)H, (long long)I, (long long)r);
  if (!dtype_ok(y_dtype)) return fail(BRQ_E_DTYPE, "brq_moe_dbf_ffn: unknown y_dtype %d", enum_value(y_dtype));
  bool al = aligned(x, 16) && aligned(logits, 4) && aligned(y, 16) && (!ids || aligned(ids, 4)) && (!w || aligned(w, 4));
  for (const brq_dbf_factors* f : recs)
    al = al && aligned(f->v, 16) && aligned(f->u, 16) && aligned(f->d_in, 16) && aligned(f->d_mid, 2) &&
         aligned(f->d_out, 2);
  if (!al)
    return fail(BRQ_E_ALIGN, "brq_moe_dbf_ffn: x, y, sign planes and d_in must be 16-byte aligned, diagonals 2-byte");
  const size_t need = brq::moe_dbf_ws_bytes(T, H, I, E, top_k, r);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(BRQ_E_WORKSPACE, "brq_moe_dbf_ffn: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                ws_bytes);
  brq_status s = check_device();
  if (s != BRQ_OK) return s;
  auto rec = [](const brq_dbf_factors* f) { return brq::DbfFactors{f->d_in, f->v, f->d_mid, f->u, f->d_out}; };
  return hip_result(brq::launch_moe_dbf(x, logits, (int)T, (int)H, (int)I, (int)E, (int)top_k, (int)r, rec(gate),
                                        rec(up), rec(down), y, y_dtype == BRQ_BF16, ids, w, ws, (hipStream_t)stream),
                    "brq_moe_dbf_ffn");
}

brq_status brq_kron_rotate(const uint16_t* x, int64_t M, const float* H, int64_t n1, const float* R, int64_t n2,
                           uint16_t* y, void* stream) {
  if (!x || !H || !R || !y) return fail(BRQ_E_NULL, "brq_kron_rotate: x, H, R and y must not be NULL");
  if (M < 1 || M > kMaxDim) return fail(BRQ_E_SHAPE, "brq_kron_rotate: M=%lld out of range", (long long)M);
  if (!brq::kron_supported(n1, n2))
    return fail(BRQ_E_SHAPE,
                "brq_kron_rotate: n1=%lld n2=%lld, factor sizes must be 32, 64 or 96 with n1 * n2 <= 6144",
                (long long)n1, (long long)n2);
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(H, 4) || !aligned(R, 4))
    return fail(BRQ_E_ALIGN, "brq_kron_rotate: x and y must be 16-byte aligned");
  const char* xb = reinterpret_cast<const char*>(x);
  const char* yb = reinterpret_cast<const char*>(y);
  const size_t bytes = (size_t)M * (size_t)(n1 * n2) * 2;
  if (xb < yb + bytes && yb < xb + bytes) return fail(BRQ_E_SHAPE, "brq_kron_rotate: x and y overlap");
  brq_status s = check_device();
  if (s != BRQ_OK) return s;
  return hip_result(brq::launch_kron(x, (int)M, (int)n1, (int)n2, H, R, y, (hipStream_t)stream),
                    "brq_kron_rotate");
}

}  // extern "C"
