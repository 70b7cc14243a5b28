// coherent.h - hand-off of data between workgroups inside one launch.
//
// The L2 caches of the XCDs are not coherent with each other.  Data that one
// workgroup produces and a workgroup on another XCD consumes within the same
// launch is therefore written with agent-coherent stores and read with
// agent-coherent loads (the sc1 cache policy: the store writes through to
// the device-coherent level, the load does not return a stale L2 copy).
// This avoids the release fence's L2 write-back, which costs about 20 ns per
// workgroup serialised across the device.  Counters are relaxed agent-scope
// atomics; a producer waits for its own stores (vmcnt) before it counts
// itself done.  Every wait is bounded and reports a timeout instead of
// hanging.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "i4d_internal.h"

namespace i4d {

__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint16_t ld_coh(const uint16_t* p) {
  return __hip_atomic_load(const_cast<uint16_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte agent-coherent load at byte offset `off` of a buffer of `bytes`
// bytes (a raw buffer load: offsets at or beyond `bytes` return zeros)
__device__ __forceinline__ u32x4_t ld_coh16(const void* base, uint32_t off, uint32_t bytes) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16 /* sc1 */);
}

// 16-byte agent-coherent store at byte offset `off` of a buffer of `bytes`
// bytes (the sc1 policy of the relaxed agent-scope stores above)
__device__ __forceinline__ void st_coh16(void* base, uint32_t off, uint32_t bytes, u32x4_t v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 16 /* sc1 */);
}

// Flagged words: 8 bytes holding 4 bytes of data and the flag of the launch
// that wrote them, stored and loaded as one 64-bit access (single-copy
// atomic).  A reader that sees its launch's flag has that launch's data,
// so the hand-off needs neither a counter nor the producer's wait for its
// stores: the consumer polls the data itself.  The flag is the launch's
// epoch + 1, so words of an earlier launch, and zeroed memory, never match.
__device__ __forceinline__ void st_flag(uint64_t* p, uint32_t data, uint32_t flag) {
  __hip_atomic_store(p, ((uint64_t)flag << 32) | data, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_flag(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool flag_is(uint64_t w, uint32_t flag) { return (uint32_t)(w >> 32) == flag; }
// polls of flagged words before a wait counts as timed out
constexpr int kPollLimit = 1 << 20;
// a timed-out poll: the sticky word of the launch and the cache's error word
__device__ __forceinline__ void poll_timeout(unsigned* sync_err, int32_t* err_word) {
  if ((threadIdx.x & 63) == 0) {
    if (sync_err) atomicOr(sync_err, 1u);
    if (err_word) atomicOr(err_word, I4D_DEVERR_SYNC);
  }
}

// wait until this wave's stores (and loads) have completed
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ unsigned atomic_add_agent(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// bounded spin until *p >= target; false (and the error bit set) on timeout
__device__ __forceinline__ bool spin_geq(unsigned* p, unsigned target, unsigned* err, unsigned bit) {
  for (int it = 0; it < (1 << 21); ++it) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  atomicOr(err, bit);
  return false;
}

}  // namespace i4d
