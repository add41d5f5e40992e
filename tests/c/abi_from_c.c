/*
 * The library's C ABI used from plain C (no C++, no Python): workspace sizes
 * and the argument checks that return before anything is enqueued, so it
 * runs without a GPU.  Built and run by tests/test_abi_host.py.
 */
#include <stdint.h>
#include <stdio.h>

#include "spec_verify.h"

#define FAKE ((void *)(uintptr_t)(1u << 20))

static int failures = 0;

static void expect(int cond, const char *what)
{
    if (!cond) {
        printf("FAILED: %s\n", what);
        ++failures;
    }
}

int main(void)
{
    size_t n = 0;
    expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, 64, 5, 128256, SPEC_DTYPE_BF16, &n) == SPEC_OK &&
               n > 0 && n % 256 == 0,
           "chain workspace size");
    expect(spec_verify_workspace_bytes(SPEC_MODE_TOPK, 512, 8, 128256, SPEC_DTYPE_BF16, &n) == SPEC_OK &&
               n == 256u + 512u * 16u * 128u,
           "top-k workspace size");
    expect(spec_verify_workspace_bytes(SPEC_MODE_TOPK, 2, 9, 100, SPEC_DTYPE_F32, &n) == SPEC_ERR_INVALID_ARG,
           "top-k k > 8 rejected");
    expect(spec_verify_chain(NULL, NULL, SPEC_DTYPE_BF16, NULL, NULL, NULL, 0, 3, 100, 1.0f, NULL, NULL,
                             NULL, NULL, 0, NULL) == SPEC_OK,
           "B = 0 is a no-op");
    expect(spec_verify_chain(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 2, 3, 100, 0.0f, FAKE, FAKE,
                             NULL, FAKE, 1 << 20, NULL) == SPEC_ERR_INVALID_ARG,
           "T = 0 rejected by the chain verify");
    expect(spec_verify_greedy(FAKE, SPEC_DTYPE_BF16, FAKE, 2, 3, 100, FAKE, FAKE, FAKE, 16, NULL) ==
               SPEC_ERR_WORKSPACE,
           "small workspace reported");
    expect(spec_draft_topk(FAKE, SPEC_DTYPE_BF16, 2, 100, 0, FAKE, NULL, FAKE, 1 << 20, NULL) ==
               SPEC_ERR_INVALID_ARG,
           "top-k k = 0 rejected");
    expect(spec_kv_commit(FAKE, FAKE, 2, 3, 8, 16, 64, NULL, 0, FAKE, FAKE, FAKE, NULL) == SPEC_ERR_INVALID_ARG,
           "KV commit with overlapping scratch and cache rejected");
    expect(spec_tree_mask(FAKE, NULL, 2, 300, FAKE, FAKE, NULL) == SPEC_ERR_INVALID_ARG,
           "tree mask over 256 nodes rejected");
    expect(spec_verify_status_string(SPEC_ERR_WORKSPACE)[0] != '\0', "status text");
    if (failures == 0)
        printf("C ABI checks passed\n");
    return failures != 0;
}
