// Grid-wide wait inside one launch, for the single-launch decode chains (a
// chain's second product needs every workgroup's part of the first; section
// 7 of "LLM binarization, Episode 01: DBF" proposes such a joint kernel with a
// grid-wide synchronisation between the products).
//
// Each launch gets one slot of the library's own wait memory (a __device__
// array, zero when the code object loads; the host hands out the slots in
// turn). A slot holds eight arrival counters, one top counter and eight
// release flags, each on its own 128-byte line, so that no address takes more
// than a few dozen of the workgroups' atomics (256 workgroups on one address
// wait about three times as long on this chip):
//  * workgroup w arrives at counter w % 8; every counter that has members
//    advances by exactly 128 per launch (the group's first workgroup adds the
//    rest), so it is a multiple of 128 between launches and the old value an
//    arrival returns tells it whether it came last in its group;
//  * the last of each group arrives at the top counter, which advances by 8
//    per launch in the same way; its last arrival writes flag value f + 1 into
//    the eight flags, f being the flag value every workgroup read when it
//    started (no flag changes before every workgroup has arrived);
//  * the others poll flag w % 8 until it reads f + 1.
// Data crosses the wait only through agent-scope atomic stores and loads,
// which this chip serves at the device's coherence point past the chiplet
// L2s, and every wave waits for its stores to complete before the workgroup
// arrives, so a reader that sees the flag also sees the data. This is the
// agent-scope release/acquire pattern without the cache-wide L2 write-back and
// invalidate that plainly stored data would need (those cost several
// microseconds on 256 workgroups).
//
// The wait is bounded: after `spin_limit` polls it gives up and returns false,
// and the caller writes NaN to its outputs. Launches that use it are sized so
// that every workgroup is resident at once (grid_fits), so the bound is a
// guard, not a path. Two such launches running at the same time on one device
// (two streams) can hold compute units the other needs; the library issues
// them only when the caller asked for single-launch chains or when its own
// default does (brq_set_decode_fusion).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace brq {

constexpr uint32_t kGridSpinLimit = 1u << 22;
constexpr int kWaitSlotWords = 17 * 32;  // 17 lines of 128 bytes

__device__ __forceinline__ uint32_t coh_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coh_storef(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes of fp32 values written by other workgroups of the launch, as two
// 8-byte agent-scope loads
__device__ __forceinline__ float4 coh_load4(const float* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float4(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                     __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
}

// Flag value of the slot when the workgroup starts (read before any arrival).
__device__ __forceinline__ uint32_t grid_epoch(const uint32_t* slot) {
  return coh_load(slot + 32 * 9);  // flag 0; all eight flags hold the same value between launches
}

__device__ __forceinline__ bool grid_wait(uint32_t* slot, uint32_t epoch, uint32_t spin_limit) {
  __shared__ int s_ok;
  // each wave waits until its stores have completed, then the workgroup
  // meets, so the arrival below follows every store of the workgroup
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t nwg = gridDim.x * gridDim.y;
    const uint32_t wg = blockIdx.y * gridDim.x + blockIdx.x;
    const uint32_t q = wg & 7u;
    const uint32_t members = (nwg - q + 7u) >> 3;
    const uint32_t groups = nwg < 8u ? nwg : 8u;
    uint32_t* arrive = slot + 32 * q;
    uint32_t* top = slot + 32 * 8;
    uint32_t* flag = slot + 32 * (9 + q);
    const uint32_t inc = wg < 8u ? 128u - (members - 1u) : 1u;
    const uint32_t old = atomicAdd(arrive, inc);
    if (old + inc == (old & ~127u) + 128u) {  // last of its group
      const uint32_t tinc = q == 0 ? 8u - (groups - 1u) : 1u;
      const uint32_t told = atomicAdd(top, tinc);
      if (told + tinc == (told & ~7u) + 8u)  // last group: release everyone
        for (int p = 0; p < 8; ++p) coh_store(slot + 32 * (9 + p), epoch + 1u);
    }
    uint32_t it = 0;
    int ok = 1;
    while ((int32_t)(coh_load(flag) - (epoch + 1u)) < 0) {
      if (++it > spin_limit) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    s_ok = ok;
  }
  __syncthreads();
  return s_ok != 0;
}

// ---- host side (gsync.hip) ---------------------------------------------------
// The wait slot for the next single-launch chain on the current device.
hipError_t grid_slot(uint32_t** slot);
// Whether `blocks` workgroups of `kernel` (`threads` each, `lds` bytes of
// dynamic LDS) can all be resident on the current device at once.
bool grid_fits(const void* kernel, int threads, size_t lds, int64_t blocks);
// Single-launch chains: 0 = the library's default per path, 1 = never, 2 =
// wherever the launch fits (brq_set_decode_fusion); and the poll bound.
int fusion_mode();
uint32_t grid_spin_limit();
void set_fusion(int mode, uint32_t spin_limit);

}  // namespace brq
