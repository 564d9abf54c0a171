// Device-wide hand-offs between workgroups of one launch, for the kernels
// whose workgroups wait on each other's results (the streaming boundary and
// the single-pass pre).
//
// The L2 caches of the part's compute dies are not coherent with each other.
// Data meant for another workgroup is written with device-coherent stores (the
// sc1 cache policy) and read with device-coherent loads; a writer waits for
// its stores to complete (s_waitcnt 0) before it bumps a counter, and a reader
// polls that counter with a device-coherent load before it reads.  No
// cache-wide writeback or invalidate is needed (__threadfence does both, and
// costs tens to hundreds of microseconds here).  Counters live in the caller's
// workspace and are zero at rest: each kernel returns them to zero before it
// ends.
#pragma once

#include <hip/hip_runtime.h>

namespace mhc {

constexpr int kCoherent = 16;            // buffer cache-policy bit sc1: device-coherent access
constexpr int kSpinLimit = 1 << 22;      // polls (with a short sleep) before a wait gives up
constexpr unsigned kOob = 0x40000000u;   // a buffer offset past every resource's end

// Buffer resource over `bytes` bytes from base: accesses past the end read 0
// and write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ unsigned ld_dev(const unsigned* p) {
    return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned* p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
    st_dev(reinterpret_cast<unsigned*>(p), __float_as_uint(v));
}
__device__ __forceinline__ unsigned add_dev(unsigned* p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-coherent load of a float at byte offset off of a buffer resource
// (0 past its end).  Unlike an atomic load, several can be in flight at once
// (the compiler waits for each atomic load before the next iteration of a loop).
__device__ __forceinline__ float ld_coh(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kCoherent));
}

// Spin (one thread) until *p is nonzero; false if the bound ran out.
__device__ __forceinline__ bool wait_flag(const unsigned* p) {
    for (int n = 0; n < kSpinLimit; ++n) {
        if (ld_dev(p) != 0u) return true;
        __builtin_amdgcn_s_sleep(20);  // about half a microsecond: few polls on the counters' lines
    }
    return false;
}

// Spin (one thread) until *p >= target; false if the bound ran out.
__device__ __forceinline__ bool wait_count(const unsigned* p, unsigned target) {
    for (int n = 0; n < kSpinLimit; ++n) {
        if (ld_dev(p) >= target) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}

}  // namespace mhc
