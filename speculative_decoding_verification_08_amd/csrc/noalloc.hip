// The chain verify for callers that cannot allocate device memory: its
// workspace is an array in the library's own device memory, one copy per GPU.
#include <hip/hip_runtime.h>

#include <mutex>

#include "spec_verify.h"

namespace sv {
namespace {

// The largest workspace the array serves: 8 MiB covers B = 256 sequences of
// K = 8 drafts over a 152k fp32 vocabulary (5.3 MiB).
constexpr size_t kScratchBytes = SPEC_VERIFY_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the array is a whole number of 256-byte blocks");
constexpr int kMaxDevices = 64;

// Static storage, so every copy starts zeroed; each GPU that the library runs
// on holds its copy until the process ends.  In host code this name is a
// stand-in, not a device address: kernels and copies take the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

struct DeviceScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// The current device's copy of the array, looked up on the first call made on
// that device (with that device current) and kept; nullptr if the lookup
// failed.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        void *p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.err == hipSuccess && p != nullptr) d.ptr = p;
    });
    return d.ptr;
}

}  // namespace
}  // namespace sv

extern "C" spec_status spec_verify_chain_noalloc(
    const void *target_logits, const void *draft_logits, spec_dtype dtype,
    const int32_t *draft_tokens, const float *u_accept, const float *u_sample, int32_t B, int32_t K,
    int32_t V, float temperature, int32_t *out_tokens, int32_t *out_accepted, float *out_diag,
    hipStream_t stream) {
    size_t need = 0;
    const spec_status st = spec_verify_workspace_bytes(SPEC_MODE_CHAIN, B, K, V, dtype, &need);
    if (st != SPEC_OK) return st;
    if (need > sv::kScratchBytes) return SPEC_ERR_SCRATCH_LIMIT;
    if (B == 0) return SPEC_OK;
    void *ws = sv::device_scratch();
    if (ws == nullptr) return SPEC_ERR_LAUNCH;
    // Nothing in the array needs clearing between calls: every word one
    // workgroup hands another carries its call's tag.
    return spec_verify_chain(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample,
                             B, K, V, temperature, out_tokens, out_accepted, out_diag, ws,
                             sv::kScratchBytes, stream);
}
