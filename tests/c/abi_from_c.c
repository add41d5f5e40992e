/*
 * The library's C ABI used from plain C (no C++, no Python): workspace sizes
 * and the argument checks that return before anything is enqueued, so it
 * runs without a GPU.  Built against the library by tests/test_abi_host.py,
 * and against a host-only build of the ABI under the address and
 * undefined-behaviour sanitizers by tests/test_sanitized_host.py (where the
 * kernel launchers are stand-ins that count calls: none may happen).
 */
#include <stdint.h>
#include <stdio.h>

#include "spec_verify.h"

#define FAKE ((void *)(uintptr_t)(1u << 20))
#define FAKE_AT(off) ((void *)((uintptr_t)(1u << 20) + (off)))
#define BIG ((size_t)1 << 30)

/* Present only in the sanitized build (the launcher stand-ins). */
extern int abi_stub_launches __attribute__((weak));

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

    /* Workspace sizes at and past every limit. */
    expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, 0, 0, 1, SPEC_DTYPE_F32, &n) == SPEC_OK && n > 0,
           "empty chain workspace");
    expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, 2, 4, SPEC_VERIFY_MAX_CHAIN_V_BF16, SPEC_DTYPE_BF16,
                                       &n) == SPEC_OK,
           "chain at the bf16 vocabulary limit");
    expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, 2, 4, SPEC_VERIFY_MAX_CHAIN_V_BF16 + 1,
                                       SPEC_DTYPE_BF16, &n) == SPEC_ERR_INVALID_ARG,
           "chain past the bf16 vocabulary limit");
    expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, 2, 4, SPEC_VERIFY_MAX_CHAIN_V_F32 + 1, SPEC_DTYPE_F32,
                                       &n) == SPEC_ERR_INVALID_ARG,
           "chain past the fp32 vocabulary limit");
    expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, -1, 4, 100, SPEC_DTYPE_F32, &n) == SPEC_ERR_INVALID_ARG,
           "negative B");
    expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, 2, 65, 100, SPEC_DTYPE_F32, &n) == SPEC_ERR_INVALID_ARG,
           "K past the limit");
    expect(spec_verify_workspace_bytes(SPEC_MODE_TREE, 2, 257, 100, SPEC_DTYPE_F32, &n) == SPEC_ERR_INVALID_ARG,
           "tree past 256 nodes");
    expect(spec_verify_workspace_bytes(SPEC_MODE_GREEDY, 2, 4, SPEC_VERIFY_MAX_V + 1, SPEC_DTYPE_F32, &n) ==
               SPEC_ERR_INVALID_ARG,
           "greedy past the vocabulary limit");
    expect(spec_verify_workspace_bytes((spec_mode)7, 2, 4, 100, SPEC_DTYPE_F32, &n) == SPEC_ERR_INVALID_ARG,
           "unknown mode");
    expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, 2, 4, 100, (spec_dtype)5, &n) == SPEC_ERR_INVALID_ARG,
           "unknown dtype");
    expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, 2000000000, 64, 1 << 18, SPEC_DTYPE_F32, &n) ==
               SPEC_ERR_INVALID_ARG,
           "grid past 2^31 workgroups");

    /* Chain verify and its phases: every argument check. */
    {
        float T[] = {0.0f, -1.0f, 1.0f / 0.0f, 0.0f / 0.0f};
        for (int i = 0; i < 4; ++i)
            expect(spec_verify_chain(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, T[i], FAKE, FAKE,
                                     NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
                   "chain temperature not positive and finite");
        expect(spec_verify_chain(NULL, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, 1.0f, FAKE, FAKE,
                                 NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "chain without target");
        expect(spec_verify_chain(FAKE_AT(8), FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, 1.0f, FAKE,
                                 FAKE, NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "chain with misaligned target");
        expect(spec_verify_chain(FAKE, NULL, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, 1.0f, FAKE, FAKE,
                                 NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "chain without draft");
        expect(spec_verify_chain(FAKE, FAKE, SPEC_DTYPE_BF16, NULL, FAKE, FAKE, 4, 3, 1000, 1.0f, FAKE, FAKE,
                                 NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "chain without tokens");
        expect(spec_verify_chain(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, NULL, 4, 3, 1000, 1.0f, FAKE, FAKE,
                                 NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "chain without u_sample");
        expect(spec_verify_chain(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, 1.0f, NULL, FAKE,
                                 NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "chain without out_tokens");
        expect(spec_verify_chain(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, 1.0f, FAKE, FAKE,
                                 FAKE_AT(4), FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "chain with misaligned diag");
        expect(spec_verify_chain(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, 1.0f, FAKE, FAKE,
                                 NULL, NULL, BIG, NULL) == SPEC_ERR_WORKSPACE,
               "chain without workspace");
        expect(spec_verify_workspace_bytes(SPEC_MODE_CHAIN, 4, 3, 1000, SPEC_DTYPE_BF16, &n) == SPEC_OK &&
                   spec_verify_chain(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 4, 3, 1000, 1.0f, FAKE, FAKE,
                                     NULL, FAKE, n - 1, NULL) == SPEC_ERR_WORKSPACE,
               "chain workspace one byte short");
        expect(spec_verify_chain(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 4, 65, 1000, 1.0f, FAKE, FAKE,
                                 NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "chain K past the limit");
        expect(spec_verify_chain_stats(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, 4, 3, 1000, 0.0f, FAKE, BIG, NULL) ==
                   SPEC_ERR_INVALID_ARG,
               "statistics phase at T = 0");
        expect(spec_verify_chain_sample(FAKE, FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, NULL, 4, 3, 1000, 1.0f, FAKE,
                                        FAKE, NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "sample phase without u_sample");
        expect(spec_verify_chain_noalloc(FAKE, FAKE, SPEC_DTYPE_F32, FAKE, FAKE, FAKE, 4096, 64, 1 << 17, 1.0f,
                                         FAKE, FAKE, NULL, NULL) == SPEC_ERR_SCRATCH_LIMIT,
               "allocation-free chain past its array");
        expect(spec_verify_chain_noalloc(FAKE, FAKE, SPEC_DTYPE_F32, FAKE, FAKE, FAKE, 2, 4, 0, 1.0f, FAKE, FAKE,
                                         NULL, NULL) == SPEC_ERR_INVALID_ARG,
               "allocation-free chain with V = 0");
        expect(spec_verify_chain_noalloc(FAKE, FAKE, SPEC_DTYPE_F32, FAKE, FAKE, FAKE, 0, 4, 100, 1.0f, FAKE,
                                         FAKE, NULL, NULL) == SPEC_OK,
               "allocation-free chain with B = 0");
    }

    /* Greedy chain and static tree. */
    {
        int32_t good[] = {-1, 0, 0, 1};
        int32_t bad[][3] = {{0, 0, 1}, {-1, 1, 0}, {-1, 0, 2}, {-1, -1, 0}, {-1, 0, 5}};
        expect(spec_verify_greedy(NULL, SPEC_DTYPE_BF16, FAKE, 2, 4, 100, FAKE, FAKE, FAKE, BIG, NULL) ==
                   SPEC_ERR_INVALID_ARG,
               "greedy without logits");
        expect(spec_verify_greedy(FAKE, SPEC_DTYPE_BF16, NULL, 2, 4, 100, FAKE, FAKE, FAKE, BIG, NULL) ==
                   SPEC_ERR_INVALID_ARG,
               "greedy without tokens");
        expect(spec_verify_tree_greedy(FAKE, SPEC_DTYPE_BF16, FAKE, good, 0, 4, 100, FAKE, NULL, FAKE, FAKE, BIG,
                                       NULL) == SPEC_OK,
               "tree with B = 0");
        for (int i = 0; i < 5; ++i)
            expect(spec_verify_tree_greedy(FAKE, SPEC_DTYPE_BF16, FAKE, bad[i], 2, 3, 100, FAKE, NULL, FAKE, FAKE,
                                           BIG, NULL) == SPEC_ERR_INVALID_ARG,
                   "tree whose parents do not form a tree");
        expect(spec_verify_tree_greedy(FAKE, SPEC_DTYPE_BF16, FAKE, good, 2, 4, 100, FAKE, NULL, FAKE, FAKE, 8,
                                       NULL) == SPEC_ERR_WORKSPACE,
               "tree workspace too small");
        expect(spec_verify_tree_greedy_dyn(FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, NULL, 2, 8, 100, FAKE, NULL, FAKE,
                                           FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "per-sequence trees without node counts");
        expect(spec_verify_tree_greedy_dyn(FAKE, SPEC_DTYPE_BF16, FAKE, FAKE, FAKE, 2, 300, 100, FAKE, NULL, FAKE,
                                           FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
               "per-sequence trees past 256 nodes");
    }

    /* Top-k, KV commit and tree mask. */
    expect(spec_draft_topk(FAKE, SPEC_DTYPE_BF16, 0, 100, 4, FAKE, NULL, FAKE, BIG, NULL) == SPEC_OK,
           "top-k with no rows");
    expect(spec_draft_topk(FAKE_AT(8), SPEC_DTYPE_BF16, 2, 100, 4, FAKE, NULL, FAKE, BIG, NULL) ==
               SPEC_ERR_INVALID_ARG,
           "top-k with misaligned logits");
    expect(spec_draft_topk(FAKE, SPEC_DTYPE_BF16, 2, 4, 5, FAKE, NULL, FAKE, BIG, NULL) == SPEC_ERR_INVALID_ARG,
           "top-k with k > V");
    expect(spec_draft_topk(FAKE, SPEC_DTYPE_BF16, 2, 100, 4, FAKE, NULL, FAKE, 16, NULL) == SPEC_ERR_WORKSPACE,
           "top-k workspace too small");
    expect(spec_kv_commit(FAKE, FAKE_AT((size_t)1 << 32), 0, 3, 8, 16, 64, NULL, 0, FAKE, FAKE, FAKE_AT(128),
                          NULL) == SPEC_ERR_INVALID_ARG,
           "KV commit with no planes");
    expect(spec_kv_commit(FAKE, FAKE_AT((size_t)1 << 32), 2, 3, 8, 16, 72, NULL, 0, FAKE, FAKE, FAKE_AT(128),
                          NULL) == SPEC_ERR_INVALID_ARG,
           "KV commit rows not a multiple of 16 bytes");
    expect(spec_kv_commit(FAKE, FAKE_AT((size_t)1 << 32), 2, 3, 8, 16, 64, NULL, 0, FAKE, FAKE_AT(64),
                          FAKE_AT(64), NULL) == SPEC_ERR_INVALID_ARG,
           "KV commit whose new lengths alias the old");
    expect(spec_kv_commit(FAKE, FAKE_AT((size_t)1 << 32), 2, 0, 8, 16, 64, NULL, 0, FAKE, FAKE, FAKE_AT(128),
                          NULL) == SPEC_OK,
           "KV commit with B = 0");
    expect(spec_tree_mask(FAKE, NULL, 2, 0, FAKE, FAKE, NULL) == SPEC_ERR_INVALID_ARG, "tree mask with N = 0");
    expect(spec_tree_mask(FAKE, FAKE_AT(2), 2, 10, FAKE, FAKE, NULL) == SPEC_ERR_INVALID_ARG,
           "tree mask with misaligned counts");
    expect(spec_tree_mask(FAKE, NULL, 0, 10, FAKE, FAKE, NULL) == SPEC_OK, "tree mask with B = 0");
    for (int s = 0; s <= 4; ++s)
        expect(spec_verify_status_string((spec_status)s)[0] != '\0', "status text of every status");

    if (&abi_stub_launches != NULL)
        expect(abi_stub_launches == 0, "an argument check reached a kernel launch");
    if (failures == 0)
        printf("C ABI checks passed\n");
    return failures != 0;
}
