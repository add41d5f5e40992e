// Division by a divisor fixed for a launch: the host makes the multiplier,
// the kernels' item decodes divide with one multiply, one add and one shift
// (a runtime integer division costs tens of instructions ahead of a
// workgroup's first load).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// q = (mulhi(n, m) + n) >> s, exact for n < 2^31 (Granlund and Montgomery's
// method with a 33-bit multiplier whose top bit is implicit).
struct FastDiv {
    uint32_t m = 0, s = 0;
};
inline FastDiv make_fastdiv(uint32_t d) {  // d >= 1
    FastDiv f;
    if (d == 0) return f;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    f.s = l;
    f.m = static_cast<uint32_t>(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    return f;
}
__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    const uint32_t hi = static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> 32);
    return (hi + n) >> f.s;  // hi < n for n < 2^31, so the sum does not wrap
}

}  // namespace sv
