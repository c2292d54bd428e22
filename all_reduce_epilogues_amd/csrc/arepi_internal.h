// arepi_internal.h -- shared host/device helpers of the gfx950 kernels behind
// include/arepi.h.  Nothing here is visible through the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "../../include/arepi.h"

namespace arepi {

// ---- host-side error reporting ------------------------------------------------

// Records the message for arepi_last_error() and returns `code`.
int fail(int code, const std::string &msg);
// Clears the message (successful call).
int ok();
// Turns a HIP launch error into AREPI_ELAUNCH with the runtime's message.
int check_launch(const char *what);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bound of a spin wait as passed to the kernels: > 0 is a number of polls;
// < 0 is a wall-clock budget of -bound ticks of the device's constant-rate
// clock (s_memrealtime).  default_spin_bound() is about one second of that
// clock on the current device (its rate read once per device).
int64_t default_spin_bound();
inline int64_t spin_bound(int64_t spin_limit) { return spin_limit > 0 ? spin_limit : default_spin_bound(); }

// ---- device-side helpers ------------------------------------------------------

// One step of a bounded wait started at wall-clock time t0: true when the
// bound (spin_bound's encoding) is used up; n counts the polls.
__device__ __forceinline__ uint64_t spin_clock() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ bool spin_expired(int64_t bound, int64_t &n, uint64_t t0) {
    if (bound > 0) return ++n > bound;
    return (int64_t)(spin_clock() - t0) > -bound;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (nontemporal) 16-byte load/store: the nt cache policy, for data
// touched once per kernel.
__device__ __forceinline__ uint4 load16_nt(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store16_nt(void *p, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

// gfx9 buffer-resource word 3 (raw, untyped 32-bit data format).
constexpr int kBufferDword3 = 0x00020000;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Cache-policy operand of the direct-to-LDS load builtins for a streaming
// (nt) load on gfx950 (checked against the emitted assembly).
constexpr int kAuxNontemporal = 2;

// Two fp32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// Widen 8 bf16 (one 16-byte pack) to fp32.
__device__ __forceinline__ void unpack8(const uint4 q, float f[8]) {
    f[0] = bf_lo(q.x); f[1] = bf_hi(q.x);
    f[2] = bf_lo(q.y); f[3] = bf_hi(q.y);
    f[4] = bf_lo(q.z); f[5] = bf_hi(q.z);
    f[6] = bf_lo(q.w); f[7] = bf_hi(q.w);
}

__device__ __forceinline__ uint4 pack8(const float f[8]) {
    uint4 q;
    q.x = pack_bf16x2(f[0], f[1]);
    q.y = pack_bf16x2(f[2], f[3]);
    q.z = pack_bf16x2(f[4], f[5]);
    q.w = pack_bf16x2(f[6], f[7]);
    return q;
}

// Scoped relaxed atomic load / release fetch-or / acquire fence.  `system`
// selects system scope (a producer on another device), otherwise agent scope.
__device__ __forceinline__ uint32_t load_relaxed(const uint32_t *p, bool system) {
    return system ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
                  : __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fetch_or_relaxed(uint32_t *p, uint32_t v, bool system) {
    if (system)
        __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else
        __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fetch_and_relaxed(uint32_t *p, uint32_t v, bool system) {
    if (system)
        __hip_atomic_fetch_and(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else
        __hip_atomic_fetch_and(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire(bool system) {
    if (system)
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
    else
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ void fence_release(bool system) {
    if (system)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
    else
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

// Device-coherent 8-byte load/store (relaxed atomics at the given scope): the
// access is not satisfied from a non-coherent cache level, so a value written
// by another XCD (or device) becomes visible to a polling reader.
__device__ __forceinline__ uint64_t load64_coherent(const uint64_t *p, bool system) {
    return system ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
                  : __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store64_coherent(uint64_t *p, uint64_t v, bool system) {
    if (system)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace arepi
