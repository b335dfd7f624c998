// lds_sync.hpp -- bounded waits on LDS counters between the waves of one
// workgroup (the weight-streaming and decode kernels): a loading wave
// announces that its direct-to-LDS loads of a K segment landed, the waves
// that multiply wait for the announcement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_i8.hpp"

namespace q8 {

// Waves of the streaming and decode kernels that ran for more than
// SG_WAVE_LIMIT_TICKS (see sg_wait_ge), counted per device since the
// library was loaded there; q8_wait_timeouts reads it.
__device__ unsigned int sg_wait_timeouts;

// 10 ms of the 100 MHz real-time counter: far beyond any call of these
// kernels (well under 1 ms), and below the time one bounded wait takes to
// give up (2^20 polls of at least a 64-clock sleep, about 30 ms).
constexpr uint64_t SG_WAVE_LIMIT_TICKS = 1000000;

// Spin (short sleeps) until an LDS counter reaches target; bounded (about
// 2^20 polls, tens of milliseconds) so a broken invariant gives wrong
// output, not a hung device.  A wave whose wait gave up has run far longer
// than any call takes, and counts itself in sg_wait_timeouts at its end (a
// clock read at its start and end, outside the waits: recording inside the
// poll loop changed its code and cost 5-15% on W8A16 calls).  The poll is
// a ds_read written out (and waited for inside the same statement): a
// compiler-visible LDS read would first drain the loading waves' in-flight
// direct loads.
__device__ __forceinline__ void sg_wait_ge(int* c, int target) {
    const uint32_t a = (uint32_t)(uintptr_t)(Q8_LDS int*)c;
    for (int it = 0; it < (1 << 20); ++it) {
        int v;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
        if (__builtin_amdgcn_readfirstlane(v) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// Increment an LDS counter (one lane).  A returnless ds_add written out, so
// that the compiler does not drain this wave's direct-to-LDS loads first (it
// cannot tell the counter from their targets); the caller has waited for
// exactly the loads the signal announces.
__device__ __forceinline__ void sg_signal(int* c) {
    const uint32_t a = (uint32_t)(uintptr_t)(Q8_LDS int*)c;
    asm volatile("ds_add_u32 %0, %1" ::"v"(a), "v"(1) : "memory");
}

// s_waitcnt vmcnt(n) for a run-time n in [0, 63]; other counters untouched.
__device__ __forceinline__ void sg_wait_vm(int n) {
    switch (n) {
#define Q8_W(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
#define Q8_W8(b) Q8_W(b) Q8_W(b + 1) Q8_W(b + 2) Q8_W(b + 3) Q8_W(b + 4) Q8_W(b + 5) Q8_W(b + 6) Q8_W(b + 7)
        Q8_W8(0) Q8_W8(8) Q8_W8(16) Q8_W8(24) Q8_W8(32) Q8_W8(40) Q8_W8(48) Q8_W8(56)
#undef Q8_W8
#undef Q8_W
        default: __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); break;
    }
}

}  // namespace q8
