// The library's grid-wait memory (gsync.h): a file-scope __device__ array of
// wait slots, zero when the code object loads, one copy per GPU. Host code
// never passes the array's name to a kernel (on the host that name is a
// stand-in, not a device address); the first use on a device looks its
// address up with hipGetSymbolAddress, with that device current, and keeps it
// per device. Launches take the slots in turn, so two single-launch chains in
// flight at the same time (on different streams) use different slots unless
// 128 others were issued in between. A captured graph keeps the slot it was
// captured with; every launch leaves a slot ready for the next one.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gsync.h"

static constexpr int kSlots = 128;  // 128 x 2176 bytes = 272 KiB per GPU
static __device__ __align__(256) uint32_t grid_wait_mem[kSlots * brq::kWaitSlotWords] = {};

namespace brq {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint32_t* g_base[kMaxDevices];
std::atomic<uint32_t> g_next[kMaxDevices];
int g_cus[kMaxDevices];
std::atomic<int> g_mode{0};
std::atomic<uint32_t> g_spin{kGridSpinLimit};
}  // namespace

hipError_t grid_slot(uint32_t** slot) {
  *slot = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_base[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(grid_wait_mem));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_base[dev] = static_cast<uint32_t*>(p);
    }
  }
  *slot = g_base[dev] + (size_t)(g_next[dev].fetch_add(1u) % kSlots) * kWaitSlotWords;
  return hipSuccess;
}

bool grid_fits(const void* kernel, int threads, size_t lds, int64_t blocks) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return false;
  }
  int cus;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_cus[dev]) {
      int v = 0;
      if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
        (void)hipGetLastError();
        return false;
      }
      g_cus[dev] = v;
    }
    cus = g_cus[dev];
  }
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, lds) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return (int64_t)per * cus >= blocks;
}

int fusion_mode() { return g_mode.load(std::memory_order_relaxed); }
uint32_t grid_spin_limit() { return g_spin.load(std::memory_order_relaxed); }
void set_fusion(int mode, uint32_t spin_limit) {
  g_mode.store(mode, std::memory_order_relaxed);
  g_spin.store(spin_limit == 0 || spin_limit > kGridSpinLimit ? kGridSpinLimit : spin_limit,
               std::memory_order_relaxed);
}

}  // namespace brq
