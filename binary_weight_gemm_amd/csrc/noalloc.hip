// brq_moe_ffn_noalloc: the routed MoE layer of brq_moe_ffn with its workspace
// taken from a scratch array that the library holds on each GPU, for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc). Same kernels as brq_moe_ffn.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends. Host
// code never passes the variable's name to a kernel (on the host that name is
// a stand-in, not a device address); the first call on a device looks its
// address up with hipGetSymbolAddress, with that device current, and keeps it
// per device. No call here allocates or frees device memory.
//
// Every call on one GPU uses that GPU's array and leaves its contents behind;
// the MoE kernels write every workspace value before they read it, so nothing
// needs clearing between calls. Calls that overlap on one GPU (other streams,
// other host threads) race on the array: callers serialise them.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/brq.h"
#include "kernels.h"

static constexpr size_t kScratchBytes = BRQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];

// device address of this device's scratch array (looked up once per device)
brq_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return brq::report(BRQ_E_DEVICE, "brq_moe_ffn_noalloc: no current HIP device");
  }
  if (dev >= kMaxDevices) return brq::report(BRQ_E_DEVICE, "brq_moe_ffn_noalloc: device index above 63");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      char msg[256];
      snprintf(msg, sizeof(msg), "brq_moe_ffn_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
               hipGetErrorString(e));
      return brq::report(BRQ_E_HIP, msg);
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return BRQ_OK;
}

}  // namespace

extern "C" brq_status brq_moe_ffn_noalloc(const uint16_t* x, const float* logits, int64_t T, int64_t H, int64_t I,
                                          int64_t E, int64_t top_k, const uint64_t* gate_s, const uint16_t* gate_sc,
                                          const uint64_t* up_s, const uint16_t* up_sc, const uint64_t* down_s,
                                          const uint16_t* down_sc, void* y, brq_dtype y_dtype, int32_t* ids,
                                          float* w, void* stream) {
  const size_t need = brq_moe_workspace_bytes(T, H, I, E, top_k);
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  auto al4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; };
  const bool args_ok = need != 0 && x && logits && gate_s && gate_sc && up_s && up_sc && down_s && down_sc && y &&
                       (y_dtype == BRQ_BF16 || y_dtype == BRQ_F32) && al16(x) && al4(logits) && al16(gate_s) &&
                       al16(up_s) && al16(down_s) && al16(gate_sc) && al16(up_sc) && al16(down_sc) && al16(y) &&
                       al4(ids) && al4(w);
  if (!args_ok)  // the full entry point validates in the same order and names the argument; nothing is enqueued
    return brq_moe_ffn(x, logits, T, H, I, E, top_k, gate_s, gate_sc, up_s, up_sc, down_s, down_sc, y, y_dtype, ids,
                       w, nullptr, 0, stream);
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "brq_moe_ffn_noalloc: T=%lld H=%lld I=%lld top_k=%lld need %zu bytes of workspace, more than the "
             "%zu-byte scratch array; call brq_moe_ffn with a workspace instead",
             (long long)T, (long long)H, (long long)I, (long long)top_k, need, kScratchBytes);
    return brq::report(BRQ_E_WORKSPACE, msg);
  }
  brq_status s = brq::device_ok();
  if (s != BRQ_OK) return s;
  void* ws = nullptr;
  s = scratch_ptr(&ws);
  if (s != BRQ_OK) return s;
  return brq_moe_ffn(x, logits, T, H, I, E, top_k, gate_s, gate_sc, up_s, up_sc, down_s, down_sc, y, y_dtype, ids, w,
                     ws, kScratchBytes, stream);
}
