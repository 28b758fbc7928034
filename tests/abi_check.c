/* A C caller of libgtattn: compiles against include/gtattn.h as C11 (and as
 * C++), links the library and checks argument rejection paths, which return
 * before any device work.  Prints "ok" and exits 0 when every check holds. */
#include <gtattn.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

static void expect(int got, int want, const char* what) {
    if (got != want) {
        printf("%s: got %d (%s), want %d; last error: %s\n", what, got, gt_status_string(got), want, gt_last_error());
        ++failures;
    }
}

int main(void) {
    const void* p = (const void*)(uintptr_t)256; /* never dereferenced: rejected first */
    float* fp = (float*)(uintptr_t)256;
    expect(gt_sparse_mha_fwd(NULL, NULL, NULL, NULL, NULL, NULL, -1, 0, 8, 64, GT_F32, NULL), GT_EINVAL, "N < 0");
    expect(gt_sparse_mha_fwd(NULL, NULL, NULL, NULL, NULL, NULL, 0, 0, 8, 64, GT_F32, NULL), GT_OK, "N = 0");
    expect(gt_sparse_mha_fwd((const int64_t*)p, NULL, p, p, p, (void*)fp, 4, 4, 8, 64, GT_F32, NULL), GT_EINVAL,
           "NULL indices with E > 0");
    expect(gt_sddmm((const int64_t*)p, (const int32_t*)p, p, p, fp, 4, 4, 8, 257, GT_F32, NULL), GT_EUNSUPPORTED,
           "D > 256");
    expect(gt_spmm((const int64_t*)p, (const int32_t*)p, fp, p, (void*)fp, 4, 4, 8, 64, 9, NULL), GT_EUNSUPPORTED,
           "unknown dtype");
    expect(gt_edge_softmax((const int64_t*)p, fp, fp, 4, 4, 0, NULL), GT_EINVAL, "H < 1");
    if (strlen(gt_last_error()) == 0) {
        printf("gt_last_error is empty after a rejection\n");
        ++failures;
    }
    expect(gt_config_set(GT_CFG_CHUNK_EDGES, -1), GT_EINVAL, "chunk of -1 edges");
    expect((int)gt_config_get(GT_CFG_CHUNK_EDGES), 0, "default chunk (automatic)");
    expect((int)gt_config_chunk_edges(1000, 0), 512, "automatic chunk, small graph");
    expect((int)gt_config_chunk_edges((int64_t)1 << 23, 0), 2048, "automatic chunk, large graph");
    expect((int)gt_config_chunk_edges((int64_t)1 << 23, 1), 512, "automatic chunk, softmax");
    expect((int)gt_config_get(77), -1, "unknown key");
    expect(gt_profile_begin(0), GT_EINVAL, "profile capacity 0");
    expect(strcmp(gt_status_string(GT_OK), "ok"), 0, "status string");
    if (failures) return 1;
    printf("ok\n");
    return 0;
}
