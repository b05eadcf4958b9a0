/* Drives the host side of the C ABI (include/pamm.h) under AddressSanitizer
 * and UndefinedBehaviorSanitizer: the sampler on many shapes, the workspace
 * size queries, the status strings, and every argument error of every entry
 * point, none of which reaches the HIP runtime or a GPU.  Pointers passed to
 * the compute entry points are aligned addresses that are never dereferenced
 * (argument checks reject the call first).  Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pamm.h"

static int fails = 0;
#define EXPECT(c) do { if (!(c)) { fprintf(stderr, "FAILED %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)
#define P(a) ((void *)(uintptr_t)(a))

int main(void) {
    EXPECT(pamm_abi_version() == PAMM_ABI_VERSION);
    for (int s = -2; s < 12; ++s) EXPECT(pamm_status_string(s) != NULL && strlen(pamm_status_string(s)) > 0);
    /* sampler: heap buffers of exactly k entries, so any overrun is caught */
    const int64_t shapes[][2] = {{1, 1}, {7, 3}, {100, 100}, {32768, 64}, {131072, 256}, {5000, 4096}, {10, 0}};
    for (size_t t = 0; t < sizeof shapes / sizeof shapes[0]; ++t) {
        int64_t n = shapes[t][0], k = shapes[t][1];
        int32_t *g = malloc(sizeof(int32_t) * (size_t)(k ? k : 1));
        EXPECT(pamm_sample_generators(n, k, 42 + t, g) == PAMM_OK);
        for (int64_t j = 1; j < k; ++j) EXPECT(g[j - 1] < g[j]);
        free(g);
    }
    int32_t g4[4];
    EXPECT(pamm_sample_generators(3, 4, 0, g4) == PAMM_ERR_SHAPE);
    EXPECT(pamm_sample_generators(3, -1, 0, g4) == PAMM_ERR_SHAPE);
    EXPECT(pamm_sample_generators(3, 2, 0, NULL) == PAMM_ERR_NULL);
    EXPECT(pamm_sample_generators((int64_t)1 << 32, 2, 0, g4) == PAMM_ERR_SHAPE);
    /* workspace sizes, including odd and empty shapes */
    EXPECT(pamm_compress_workspace_size(0, 8, 0, PAMM_BF16) == 0);
    EXPECT(pamm_compress_workspace_size(1024, 32, 300, PAMM_BF16) > 0);
    EXPECT(pamm_wgrad_workspace_size(32768, 64, 4096, 12288, PAMM_BF16) > 0);
    EXPECT(pamm_wgrad_workspace_size(-1, 64, 4096, 12288, PAMM_BF16) == 0);
    EXPECT(pamm_wgrad_workspace_size(1, 1, 1, 1, PAMM_F32) > 0);
    const uintptr_t A = 0x10000;  /* aligned, never dereferenced */
    /* compress */
    EXPECT(pamm_compress(P(A), 64, 32, 32, 5, P(A), 4, 0.1f, P(A), P(A), P(A), NULL, 0, NULL) == PAMM_ERR_DTYPE);
    EXPECT(pamm_compress(P(A), 64, 32, 16, 1, P(A), 4, 0.1f, P(A), P(A), P(A), NULL, 0, NULL) == PAMM_ERR_SHAPE);
    EXPECT(pamm_compress(P(A), 64, 32, 32, 1, P(A), 65, 0.1f, P(A), P(A), P(A), NULL, 0, NULL) == PAMM_ERR_SHAPE);
    EXPECT(pamm_compress(P(A), 64, 32, 32, 1, P(A), 4, -1.f, P(A), P(A), P(A), NULL, 0, NULL) == PAMM_ERR_VALUE);
    EXPECT(pamm_compress(NULL, 64, 32, 32, 1, P(A), 4, 0.1f, P(A), P(A), P(A), NULL, 0, NULL) == PAMM_ERR_NULL);
    EXPECT(pamm_compress(P(A + 2), 64, 32, 32, 1, P(A), 4, 0.1f, P(A), P(A), P(A), NULL, 0, NULL) == PAMM_ERR_ALIGN);
    EXPECT(pamm_compress(P(A), 1024, 32, 32, 1, P(A), 300, 0.1f, P(A), P(A), P(A), NULL, 0, NULL) == PAMM_ERR_WORKSPACE);
    EXPECT(pamm_compress(NULL, 0, 32, 32, 1, NULL, 0, 0.1f, NULL, NULL, NULL, NULL, 0, NULL) == PAMM_OK);
    /* wgrad and its no-allocation twin */
    size_t ws = pamm_wgrad_workspace_size(64, 4, 32, 48, PAMM_BF16);
    EXPECT(pamm_wgrad(P(A), P(A), P(A), 64, 4, 32, P(A), 48, 48, 9, P(A), 48, 0, 0, P(A), ws, NULL) == PAMM_ERR_DTYPE);
    EXPECT(pamm_wgrad(P(A), P(A), P(A), 64, 65, 32, P(A), 48, 48, 1, P(A), 48, 0, 0, P(A), ws, NULL) == PAMM_ERR_SHAPE);
    EXPECT(pamm_wgrad(P(A), P(A), P(A), 64, 4, 32, P(A), 48, 40, 1, P(A), 48, 0, 0, P(A), ws, NULL) == PAMM_ERR_SHAPE);
    EXPECT(pamm_wgrad(P(A), P(A), P(A), 64, 4, 32, NULL, 48, 48, 1, P(A), 48, 0, 0, P(A), ws, NULL) == PAMM_ERR_NULL);
    EXPECT(pamm_wgrad(P(A), P(A), P(A), 64, 4, 32, P(A), 48, 48, 1, P(A + 4), 48, 0, 0, P(A), ws, NULL) == PAMM_ERR_ALIGN);
    EXPECT(pamm_wgrad(P(A), P(A), P(A), 64, 4, 32, P(A), 48, 48, 1, P(A), 48, 0, 0, NULL, 0, NULL) == PAMM_ERR_WORKSPACE);
    EXPECT(pamm_wgrad(P(A), P(A), P(A), 64, 4, 32, P(A), 48, 48, 1, P(A), 48, 0, 0, P(A), ws - 1, NULL) == PAMM_ERR_WORKSPACE);
    EXPECT(pamm_wgrad(P(A), P(A), P(A), 64, 4, 64, P(A), 48, 48, 1, P(A), 48, 0, 1, P(A), ws, NULL) == PAMM_ERR_SHAPE);
    EXPECT(pamm_wgrad_noalloc(P(A), P(A), P(A), 64, 4, 32, P(A), 48, 48, 9, P(A), 48, 0, 0, NULL) == PAMM_ERR_DTYPE);
    EXPECT(pamm_wgrad_noalloc(P(A), P(A), P(A), 64, 4, 32, P(A), 48, 48, 1, NULL, 48, 0, 0, NULL) == PAMM_ERR_NULL);
    EXPECT(pamm_wgrad_noalloc(P(A), P(A), P(A), 65536, 4096, 4096, P(A), 12288, 12288, 1, P(A), 12288, 0, 0, NULL) ==
           PAMM_ERR_TOO_LARGE);
    /* the fused projection + compression */
    size_t fw = pamm_forward_compress_workspace_size(64, 32, 4, PAMM_BF16);
    EXPECT(fw > 0);
    EXPECT(pamm_forward_compress(P(A), 64, 32, 32, 0, P(A), 48, 32, NULL, P(A), 48, P(A), 4, 0.1f, P(A), P(A), P(A),
                                 P(A), fw, NULL) == PAMM_ERR_UNSUPPORTED);
    EXPECT(pamm_forward_compress(P(A), 64, 32, 32, 1, NULL, 48, 32, NULL, P(A), 48, P(A), 4, 0.1f, P(A), P(A), P(A),
                                 P(A), fw, NULL) == PAMM_ERR_NULL);
    EXPECT(pamm_forward_compress(P(A), 64, 32, 32, 1, P(A), 48, 16, NULL, P(A), 48, P(A), 4, 0.1f, P(A), P(A), P(A),
                                 P(A), fw, NULL) == PAMM_ERR_SHAPE);
    EXPECT(pamm_forward_compress(P(A), 64, 32, 32, 1, P(A), 48, 32, P(A + 1), P(A), 48, P(A), 4, 0.1f, P(A), P(A),
                                 P(A), P(A), fw, NULL) == PAMM_ERR_ALIGN);
    EXPECT(pamm_forward_compress(P(A), 64, 32, 32, 1, P(A), 48, 32, NULL, P(A), 48, P(A), 4, 0.1f, P(A), P(A), P(A),
                                 P(A), fw - 1, NULL) == PAMM_ERR_WORKSPACE);
    /* decompress */
    EXPECT(pamm_decompress(P(A), P(A), P(A), 64, 4, 32, 3, P(A), 32, NULL) == PAMM_ERR_DTYPE);
    EXPECT(pamm_decompress(P(A), P(A), P(A), 64, 4, 32, 1, P(A), 16, NULL) == PAMM_ERR_SHAPE);
    EXPECT(pamm_decompress(P(A), P(A), P(A), 64, 4, 32, 1, NULL, 32, NULL) == PAMM_ERR_NULL);
    EXPECT(pamm_decompress(P(A), P(A), P(A), 64, 4, 32, 1, P(A + 8), 32, NULL) == PAMM_ERR_ALIGN);
    EXPECT(pamm_decompress(NULL, NULL, NULL, 0, 0, 32, 1, NULL, 32, NULL) == PAMM_OK);
    if (fails) { fprintf(stderr, "%d failures\n", fails); return 1; }
    printf("ABI sanitizer driver ok\n");
    return 0;
}
