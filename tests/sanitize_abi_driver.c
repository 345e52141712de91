/*
 * Host-side driver of liborr's C ABI for the sanitizer test
 * (tests/test_sanitizers.py): every call below is rejected by the argument
 * checks, or fails at a site named by ORR_FAULT_INJECT, before any device
 * work, so it runs without a GPU. Built and run with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the library's host code and on this driver;
 * any report aborts the run. Exit status 0 and "abi driver ok" mean every
 * call returned the expected status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "orr.h"

static int failures = 0;

static void expect(const char *what, orr_status got, orr_status want) {
    const char *msg = orr_last_error();
    if (got != want) {
        fprintf(stderr, "%s: got %d (%s), want %d\n", what, (int)got, msg, (int)want);
        failures++;
    }
    if (want != ORR_OK && strlen(msg) == 0) {
        fprintf(stderr, "%s: empty error message\n", what);
        failures++;
    }
}

int main(void) {
    const float *P = (const float *)(uintptr_t)256; /* placeholders, never dereferenced */
    float *A = (float *)(uintptr_t)256;
    void *WS = (void *)(uintptr_t)256;
    const size_t WSB = (size_t)1 << 30;
    orr_tree *t = (orr_tree *)(uintptr_t)1;
    orr_timings tm;
    int64_t bounds[9];
    uint32_t *U = (uint32_t *)(uintptr_t)256;

    if (orr_abi_version() != ORR_ABI_VERSION) failures++;
    for (int s = -1; s <= 8; s++)
        if (!orr_status_string((orr_status)s)) failures++;
    for (int k = -1; k <= 3; k++)
        if (!orr_traversal_name((orr_traversal)k)) failures++;
    /* workspace sizes over the whole admissible range, and outside it */
    const int64_t ns[] = {0, 1, 2, 63, 64, 65, 1000, 1 << 20, 2147483647LL, 2147483648LL, -1};
    const int32_t caps[] = {0, 1, 2, 32, 256, 257};
    for (size_t a = 0; a < sizeof ns / sizeof ns[0]; a++)
        for (size_t b = 0; b < sizeof caps / sizeof caps[0]; b++) {
            size_t w = orr_workspace_bytes(ns[a], caps[b]);
            int ok = ns[a] >= 1 && ns[a] <= ORR_MAX_N && caps[b] >= 1 && caps[b] <= ORR_MAX_LEAF_CAP;
            /* node indices are 32-bit: n + 21 floor(n / (cap + 1)) + 1 < 2^32 */
            if (ok && ns[a] + 21 * (ns[a] / (caps[b] + 1)) + 1 > 4294967295LL) ok = 0;
            if ((w != 0) != ok) {
                fprintf(stderr, "workspace_bytes(%lld, %d) = %zu\n", (long long)ns[a], caps[b], w);
                failures++;
            }
        }

    /* argument checks */
    expect("eval n=0", orr_eval_forces(P, P, 0, 0.05f, 0.5f, 32, ORR_TRAVERSAL_COHERENT, A, U, U, U, U, WS, WSB, NULL,
                                       NULL), ORR_ERR_RANGE);
    expect("eval eps tiny", orr_eval_forces(P, P, 100, 1e-20f, 0.5f, 32, ORR_TRAVERSAL_COHERENT, A, U, U, U, U, WS, WSB,
                                            NULL, NULL), ORR_ERR_RANGE);
    expect("eval theta nan", orr_eval_forces(P, P, 100, 0.05f, 0.0f / 0.0f, 32, ORR_TRAVERSAL_COHERENT, A, U, U, U, U,
                                             WS, WSB, NULL, NULL), ORR_ERR_RANGE);
    expect("eval traversal", orr_eval_forces(P, P, 100, 0.05f, 0.5f, 32, (orr_traversal)7, A, U, U, U, U, WS, WSB, NULL,
                                             NULL), ORR_ERR_INVALID_ARG);
    expect("eval unaligned", orr_eval_forces(P, P, 100, 0.05f, 0.5f, 32, ORR_TRAVERSAL_COHERENT, A, U, U, U, U,
                                             (char *)WS + 8, WSB, NULL, NULL), ORR_ERR_INVALID_ARG);
    expect("eval small ws", orr_eval_forces(P, P, 100, 0.05f, 0.5f, 32, ORR_TRAVERSAL_COHERENT, A, U, U, U, U, WS, 64,
                                            NULL, NULL), ORR_ERR_WORKSPACE);
    expect("noalloc too big", orr_eval_forces_noalloc(P, P, 1100000, 0.05f, 0.5f, 32, ORR_TRAVERSAL_COHERENT, A, U, U,
                                                      U, U, NULL), ORR_ERR_WORKSPACE);
    orr_tree *out = (orr_tree *)(uintptr_t)1;
    expect("build null out", orr_build_tree(P, P, 100, 32, WS, WSB, NULL, NULL), ORR_ERR_INVALID_ARG);
    expect("build cap", orr_build_tree(P, P, 100, 300, WS, WSB, NULL, &out), ORR_ERR_RANGE);
    if (out != NULL) failures++;
    expect("walk null", orr_tree_walk(NULL, 0.05f, 0.5f, ORR_TRAVERSAL_COHERENT, A, U, U, U, U, &tm),
           ORR_ERR_INVALID_ARG);
    expect("walk eps", orr_tree_walk(t, -1.0f, 0.5f, ORR_TRAVERSAL_COHERENT, A, U, U, U, U, NULL), ORR_ERR_RANGE);
    expect("grouped width", orr_tree_walk_grouped(t, 0.05f, 0.5f, 3, A, U, U, U, U), ORR_ERR_RANGE);
    expect("descend width", orr_tree_walk_descend(t, 0.05f, 0.5f, 128, A, U, U, U, U), ORR_ERR_RANGE);
    expect("width walk null", orr_tree_walk_width(NULL, 0.05f, 0.5f, 64, A, U, U, U, U), ORR_ERR_INVALID_ARG);
    expect("min walk null", orr_tree_walk_min_advance(NULL, 0.05f, 0.5f, A, U, U, U, U), ORR_ERR_INVALID_ARG);
    expect("range null", orr_tree_walk_range(NULL, 0.05f, 0.5f, ORR_TRAVERSAL_COHERENT, 0, 64, A, U, U, U, U),
           ORR_ERR_INVALID_ARG);
    expect("bounds k", orr_tree_shard_bounds(t, 0, bounds), ORR_ERR_RANGE);
    expect("info null", orr_tree_info_get(NULL, NULL), ORR_ERR_INVALID_ARG);
    expect("check null", orr_tree_check(NULL), ORR_ERR_INVALID_ARG);
    expect("workspace check small", orr_workspace_check(WS, 16, NULL), ORR_ERR_WORKSPACE);
    expect("export null", orr_tree_export(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL), ORR_ERR_INVALID_ARG);
    expect("direct n", orr_direct_forces(P, P, 0, 0.05f, A, NULL), ORR_ERR_RANGE);
    expect("direct targets null", orr_direct_forces_targets(P, P, 10, 0.05f, NULL, 4, A, NULL), ORR_ERR_INVALID_ARG);
    expect("direct fp64 eps", orr_direct_forces_fp64_targets(P, P, 10, -1.0, (const int64_t *)P, 4, (double *)A, NULL),
           ORR_ERR_RANGE);
    expect("selftest range", orr_selftest_inv_sqrt(5, 1, (uint64_t *)U, U, NULL), ORR_ERR_INVALID_ARG);
    orr_tree_free(NULL);

    /* fault injection: the first device work of each call fails instead */
    setenv("ORR_FAULT_INJECT", "cube", 1);
    expect("eval cube", orr_eval_forces(P, P, 1000, 0.05f, 0.5f, 32, ORR_TRAVERSAL_COHERENT, A, U, U, U, U, WS, WSB,
                                        NULL, NULL), ORR_ERR_HIP);
    expect("build cube", orr_build_tree(P, P, 1000, 32, WS, WSB, NULL, &out), ORR_ERR_HIP);
    setenv("ORR_FAULT_INJECT", "events", 1);
    expect("eval events", orr_eval_forces(P, P, 1000, 0.05f, 0.5f, 32, ORR_TRAVERSAL_COHERENT, A, U, U, U, U, WS, WSB,
                                          NULL, &tm), ORR_ERR_HIP);
    setenv("ORR_FAULT_INJECT", "alloc", 1);
    expect("build alloc", orr_build_tree(P, P, 1000, 32, WS, WSB, NULL, &out), ORR_ERR_HOST_MEMORY);
    setenv("ORR_FAULT_INJECT", "scratch", 1);
    expect("noalloc scratch", orr_eval_forces_noalloc(P, P, 1000, 0.05f, 0.5f, 32, ORR_TRAVERSAL_COHERENT, A, U, U, U,
                                                      U, NULL), ORR_ERR_HIP);
    setenv("ORR_FAULT_INJECT", "sync", 1);
    expect("workspace check sync", orr_workspace_check(WS, WSB, NULL), ORR_ERR_HIP);
    setenv("ORR_FAULT_INJECT", "direct", 1);
    expect("direct", orr_direct_forces(P, P, 100, 0.05f, A, NULL), ORR_ERR_HIP);
    unsetenv("ORR_FAULT_INJECT");

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("abi driver ok\n");
    return 0;
}
