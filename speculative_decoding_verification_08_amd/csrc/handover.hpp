// Tagged hand-over words between workgroups of one launch (or of two
// launches in stream order).  A word is 64 bits: the call's tag above a
// 32-bit value, written with a device-scope atomic store (no wait) and read
// with a device-scope atomic load, so it is seen across XCDs.  A reader
// checks the tag, so a word left by an earlier call of any shape is never
// taken for fresh; tags are never 0, so a workspace zeroed once before its
// first use needs no clearing between calls.  Waits are
// bounded by the 100 MHz wall clock.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {
namespace {

constexpr uint64_t kWaitTicks = 200000000ull;  // 2 s of the 100 MHz wall clock

__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t bits) {
    return (static_cast<uint64_t>(tag) << 32) | bits;
}
// Publish without waiting (a device-scope store; readers check the tag).
__device__ __forceinline__ void publish(uint64_t *p, uint32_t tag, uint32_t bits) {
    __hip_atomic_store(p, tagged(tag, bits), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_f32(uint64_t *p, uint32_t tag, float v) {
    publish(p, tag, __float_as_uint(v));
}
__device__ __forceinline__ uint64_t fetch(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool current(uint64_t w, uint32_t tag) {
    return static_cast<uint32_t>(w >> 32) == tag;
}
__device__ __forceinline__ float word_f32(uint64_t w) {
    return __uint_as_float(static_cast<uint32_t>(w));
}
// A hand-over word read through the caches, without waiting: it may be stale
// (an earlier value of this call's word, or a word of an earlier call), never
// wrong, and a stale word only costs the skip it would have allowed.  The
// device-scope read measured no better and delays the item more.
__device__ __forceinline__ uint64_t plain_word(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Bounded wait (from t0) until one word carries the call's tag.  One lane
// polls one word with a pause between reads, so waiting workgroups add little
// traffic beside the streaming ones; the caller then reads everything it
// needs once.
__device__ __forceinline__ void wait_word(const uint64_t *p, uint32_t tag, uint64_t t0) {
    while (!current(fetch(p), tag) && wall_clock64() - t0 <= kWaitTicks)
        __builtin_amdgcn_s_sleep(4);
}

// A bounded wait ran out: count it in the workspace header (the failure
// word, third of the header's 32-bit words), one thread per failed output.
__device__ __forceinline__ void count_failure(uint32_t *hdr) {
    __hip_atomic_fetch_add(hdr + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace
}  // namespace sv
