/*
 * Host-only exercise of the C ABI's argument validation (include/mxfp4.h), built together with
 * a host-sanitized libmxfp4 (AddressSanitizer and UndefinedBehaviorSanitizer on the host code).
 * Every call here is invalid in some way or a pure size query, so none of them reaches a device
 * or launches anything; each must return the documented status. Exit status 0 = every check
 * held (a sanitizer report aborts the run with a non-zero status).
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/mxfp4.h"

static int failures = 0;

#define EXPECT(call, want)                                                                    \
    do {                                                                                      \
        int got_ = (int)(call);                                                               \
        if (got_ != (int)(want)) {                                                            \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
                    got_, (int)(want));                                                       \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

int main(void)
{
    /* fake, aligned, never-dereferenced addresses: every call below fails validation first */
    static _Alignas(256) uint8_t host_buf[4096];
    void *p = host_buf;
    uint8_t *q = host_buf;
    float *c = (float *)host_buf;
    const int64_t big = INT64_MAX, neg = -1;

    /* quantize */
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, 64, 64, 64, 2, 16, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2, NULL),
           MXFP4_ERR_ARG);                                       /* axis */
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, 64, 64, 64, 1, 24, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2, NULL),
           MXFP4_ERR_ARG);                                       /* hadamard size */
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, 64, 64, 64, 1, MXFP4_RHT, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2,
                          NULL), MXFP4_ERR_ARG);                 /* randomized without a size */
    EXPECT(mxfp4_quantize(p, (mxfp4_dtype_t)7, 64, 64, 64, 1, 16, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2, NULL),
           MXFP4_ERR_ARG);                                       /* dtype */
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, 64, 64, 64, 1, 16, (mxfp4_rounding_t)5, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2,
                          NULL), MXFP4_ERR_ARG);                 /* rounding */
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, 64, 48, 64, 1, 16, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2, NULL),
           MXFP4_ERR_SHAPE);                                     /* length not a multiple of 32 */
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, neg, 64, 64, 1, 16, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2, NULL),
           MXFP4_ERR_SHAPE);
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, big, big, big, 1, 16, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2, NULL),
           MXFP4_ERR_SHAPE);
    EXPECT(mxfp4_quantize(NULL, MXFP4_IN_BF16, 64, 64, 64, 1, 16, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2, NULL),
           MXFP4_ERR_NULL);
    EXPECT(mxfp4_quantize(host_buf + 2, MXFP4_IN_BF16, 64, 64, 64, 1, 16, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2,
                          NULL), MXFP4_ERR_ALIGN);
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, 64, 64, 60, 1, 16, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2, NULL),
           MXFP4_ERR_ARG);                                       /* ldx < cols */
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, 64, 64, 64, 1, 16, MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 16, q, 2, NULL),
           MXFP4_ERR_ARG);                                       /* ldq < L / 2 */
    EXPECT(mxfp4_quantize(p, MXFP4_IN_BF16, 64, 64, 64, 1, 16, MXFP4_RNE, 0, 0, (mxfp4_layout_t)3, q, 32, q, 2, NULL),
           MXFP4_ERR_ARG);

    /* quantize_dual */
    mxfp4_quant_out_t o1 = {MXFP4_RNE, 0, 0, MXFP4_LAYOUT_ROWS, q, 32, q, 2};
    mxfp4_quant_out_t o0 = {MXFP4_SR_PHILOX, 1, 1, MXFP4_LAYOUT_ROWS, q, 32, q, 2};
    EXPECT(mxfp4_quantize_dual(p, MXFP4_IN_BF16, 64, 64, 64, 16, NULL, &o0, NULL), MXFP4_ERR_NULL);
    EXPECT(mxfp4_quantize_dual(p, MXFP4_IN_BF16, 48, 64, 64, 16, &o1, &o0, NULL), MXFP4_ERR_SHAPE);
    o0.rounding = (mxfp4_rounding_t)9;
    EXPECT(mxfp4_quantize_dual(p, MXFP4_IN_BF16, 64, 64, 64, 16, &o1, &o0, NULL), MXFP4_ERR_ARG);

    /* grouped dual quantize */
    mxfp4_dual_item_t di[MXFP4_DUAL_GROUP_MAX + 1];
    for (int i = 0; i <= MXFP4_DUAL_GROUP_MAX; ++i) {
        di[i].x = p; di[i].dtype = MXFP4_IN_BF16; di[i].rows = 64; di[i].cols = 64; di[i].ldx = 64;
        di[i].axis1 = o1; di[i].axis0 = o1;
    }
    EXPECT(mxfp4_quantize_dual_grouped(di, MXFP4_DUAL_GROUP_MAX + 1, 16, NULL), MXFP4_ERR_ARG);
    EXPECT(mxfp4_quantize_dual_grouped(di, -1, 16, NULL), MXFP4_ERR_ARG);
    EXPECT(mxfp4_quantize_dual_grouped(NULL, 2, 16, NULL), MXFP4_ERR_NULL);
    EXPECT(mxfp4_quantize_dual_grouped(NULL, 0, 16, NULL), MXFP4_OK);
    di[1].dtype = MXFP4_IN_F32;
    EXPECT(mxfp4_quantize_dual_grouped(di, 2, 16, NULL), MXFP4_ERR_ARG);          /* mixed dtypes */
    di[1].dtype = MXFP4_IN_BF16;
    di[1].rows = 48;
    EXPECT(mxfp4_quantize_dual_grouped(di, 2, 16, NULL), MXFP4_ERR_SHAPE);        /* rows % 32 */
    di[1].rows = 64;
    EXPECT(mxfp4_quantize_dual_grouped(di, 2, 24, NULL), MXFP4_ERR_ARG);          /* hadamard size */
    di[1].axis0.q = NULL;
    EXPECT(mxfp4_quantize_dual_grouped(di, 2, 16, NULL), MXFP4_ERR_NULL);
    di[1].axis0.q = q;
    di[0].rows = 0; di[1].rows = 0;
    EXPECT(mxfp4_quantize_dual_grouped(di, 2, 16, NULL), MXFP4_OK);               /* nothing to do */

    /* gemm and gemm_ex */
    EXPECT(mxfp4_gemm(q, 32, q, 2, q, 32, q, 2, 8, 8, 48, 1.0f, c, 8, MXFP4_LAYOUT_ROWS, NULL, 0, NULL),
           MXFP4_ERR_SHAPE);                                     /* K not a multiple of 32 */
    EXPECT(mxfp4_gemm(q, 32, q, 2, q, 32, q, 2, 8, 8, 64, 1.0f, c, 4, MXFP4_LAYOUT_ROWS, NULL, 0, NULL),
           MXFP4_ERR_ARG);                                       /* ldc < N */
    EXPECT(mxfp4_gemm(q, 16, q, 2, q, 32, q, 2, 8, 8, 64, 1.0f, c, 8, MXFP4_LAYOUT_ROWS, NULL, 0, NULL),
           MXFP4_ERR_ARG);                                       /* lda < K / 2 */
    EXPECT(mxfp4_gemm(q, 32, q, 2, q, 32, q, 2, 8, 8, 64, 1.0f, NULL, 8, MXFP4_LAYOUT_ROWS, NULL, 0, NULL),
           MXFP4_ERR_NULL);
    EXPECT(mxfp4_gemm(q + 1, 32, q, 2, q, 32, q, 2, 8, 8, 64, 1.0f, c, 8, MXFP4_LAYOUT_ROWS, NULL, 0, NULL),
           MXFP4_ERR_ALIGN);
    EXPECT(mxfp4_gemm(q, 32, q, 2, q, 32, q, 2, 8, 8, 256, 1.0f, c, 8, MXFP4_LAYOUT_TILED, NULL, 0, NULL),
           MXFP4_ERR_SHAPE);                                     /* tiled needs K % 512 */
    EXPECT(mxfp4_gemm(q, 0, q, 0, q, 0, q, 0, (int64_t)1 << 30, 256, (int64_t)1 << 20, 1.0f, c, 256, MXFP4_LAYOUT_TILED,
                      NULL, 0, NULL), MXFP4_ERR_SHAPE);          /* tiled offsets beyond 32 bits */
    EXPECT(mxfp4_gemm(q, 32, q, 2, q, 32, q, 2, neg, 8, 64, 1.0f, c, 8, MXFP4_LAYOUT_ROWS, NULL, 0, NULL),
           MXFP4_ERR_SHAPE);
    EXPECT(mxfp4_gemm_ex(q, 32, q, 2, q, 32, q, 2, 8, 8, 64, 1.0f, 0.5f, c, (mxfp4_out_dtype_t)4, 8, MXFP4_LAYOUT_ROWS,
                         NULL, 0, NULL), MXFP4_ERR_ARG);
    EXPECT(mxfp4_gemm_ex(q, 32, q, 2, q, 32, q, 2, 8, 8, 64, 1.0f, 0.5f, host_buf + 1, MXFP4_OUT_BF16, 8,
                         MXFP4_LAYOUT_ROWS, NULL, 0, NULL), MXFP4_ERR_ALIGN);

    /* grouped gemm */
    mxfp4_gemm_item_t items[MXFP4_GEMM_GROUP_MAX + 1];
    for (int i = 0; i <= MXFP4_GEMM_GROUP_MAX; ++i) {
        items[i].aq = q; items[i].as = q; items[i].bq = q; items[i].bs = q;
        items[i].c = c + 64 * i;                                 /* 8 x 8 outputs, disjoint */
    }
    EXPECT(mxfp4_gemm_grouped(items, MXFP4_GEMM_GROUP_MAX + 1, 32, 2, 32, 2, 8, 8, 64, 1.0f, 8, MXFP4_LAYOUT_ROWS,
                              NULL), MXFP4_ERR_ARG);             /* too many products */
    EXPECT(mxfp4_gemm_grouped(items, -1, 32, 2, 32, 2, 8, 8, 64, 1.0f, 8, MXFP4_LAYOUT_ROWS, NULL), MXFP4_ERR_ARG);
    EXPECT(mxfp4_gemm_grouped(NULL, 2, 32, 2, 32, 2, 8, 8, 64, 1.0f, 8, MXFP4_LAYOUT_ROWS, NULL), MXFP4_ERR_NULL);
    EXPECT(mxfp4_gemm_grouped(NULL, 0, 32, 2, 32, 2, 8, 8, 64, 1.0f, 8, MXFP4_LAYOUT_ROWS, NULL), MXFP4_OK);
    EXPECT(mxfp4_gemm_grouped(items, 2, 32, 2, 32, 2, 8, 8, 48, 1.0f, 8, MXFP4_LAYOUT_ROWS, NULL),
           MXFP4_ERR_SHAPE);                                     /* K not a multiple of 32 */
    EXPECT(mxfp4_gemm_grouped(items, 2, 32, 2, 32, 2, 8, 8, 64, 1.0f, 8, MXFP4_LAYOUT_TILED, NULL),
           MXFP4_ERR_SHAPE);                                     /* tiled needs K % 512 */
    items[1].bs = NULL;
    EXPECT(mxfp4_gemm_grouped(items, 2, 32, 2, 32, 2, 8, 8, 64, 1.0f, 8, MXFP4_LAYOUT_ROWS, NULL), MXFP4_ERR_NULL);
    items[1].bs = q;
    items[1].c = c + 60;                                         /* overlaps the first output's last row */
    EXPECT(mxfp4_gemm_grouped(items, 2, 32, 2, 32, 2, 8, 8, 64, 1.0f, 8, MXFP4_LAYOUT_ROWS, NULL), MXFP4_ERR_ARG);
    items[1].c = c;
    EXPECT(mxfp4_gemm_grouped(items, 2, 32, 2, 32, 2, 8, 8, 64, 1.0f, 8, MXFP4_LAYOUT_ROWS, NULL), MXFP4_ERR_ARG);
    EXPECT(mxfp4_gemm_grouped(items, 2, 32, 2, 32, 2, 0, 8, 64, 1.0f, 8, MXFP4_LAYOUT_ROWS, NULL),
           MXFP4_OK);                                            /* empty output: nothing to write */

    /* size queries: invalid sizes give 0, valid ones a sane count */
    EXPECT(mxfp4_gemm_workspace_bytes(neg, 8, 64) == 0, 1);
    EXPECT(mxfp4_gemm_workspace_bytes(big, big, big) == 0, 1);
    EXPECT(mxfp4_linear_workspace_bytes(MXFP4_FPROP, neg, 64, 64) == 0, 1);
    EXPECT(mxfp4_linear_workspace_bytes((mxfp4_pass_t)9, 64, 64, 64) == 0, 1);
    EXPECT(mxfp4_linear_workspace_bytes(MXFP4_WGRAD, 8192, 4096, 4096) > 0, 1);
    EXPECT(mxfp4_linear_step_workspace_bytes(big, 1, 1) == 0, 1);
    size_t cb = 0, sb = 0;
    EXPECT(mxfp4_tiled_sizes(300, 1024, &cb, &sb), MXFP4_OK);
    EXPECT(cb == (size_t)512 * 512 && sb == (size_t)512 * 32, 1);
    EXPECT(mxfp4_tiled_sizes(300, 1000, &cb, &sb), MXFP4_ERR_SHAPE);
    EXPECT(mxfp4_tiled_sizes(300, 1024, NULL, &sb), MXFP4_ERR_NULL);

    /* linear calls and the training step */
    mxfp4_linear_cfg_t cfg = {16, MXFP4_RNE, MXFP4_SR_PHILOX, 7};
    EXPECT(mxfp4_linear_fprop(p, p, 64, 64, 64, NULL, p, 4096, c, NULL), MXFP4_ERR_NULL);
    EXPECT(mxfp4_linear_fprop(p, p, 64, 48, 64, &cfg, p, 4096, c, NULL), MXFP4_ERR_SHAPE);
    EXPECT(mxfp4_linear_dgrad(p, p, 64, 64, 64, &cfg, p, 16, c, NULL), MXFP4_ERR_WORKSPACE);
    EXPECT(mxfp4_linear_wgrad(p, p, 64, 64, 64, &cfg, host_buf + 8, 1u << 20, c, NULL), MXFP4_ERR_ALIGN);
    cfg.hadamard = 8;
    EXPECT(mxfp4_linear_wgrad(p, p, 64, 64, 64, &cfg, p, 1u << 20, c, NULL), MXFP4_ERR_ARG);
    mxfp4_step_cfg_t step = {16, MXFP4_RNE, MXFP4_RNE, MXFP4_SR_PHILOX, 7};
    EXPECT(mxfp4_linear_forward(p, p, 64, 64, 48, &step, p, 1u << 20, c, NULL), MXFP4_ERR_SHAPE);
    EXPECT(mxfp4_linear_forward(p, p, 64, 64, 64, &step, p, 16, c, NULL), MXFP4_ERR_WORKSPACE);
    EXPECT(mxfp4_linear_backward(p, 64, 64, 64, NULL, p, 1u << 20, c, c, NULL), MXFP4_ERR_NULL);
    step.wgrad = (mxfp4_rounding_t)3;
    EXPECT(mxfp4_linear_backward(p, 64, 64, 64, &step, p, 1u << 20, c, c, NULL), MXFP4_ERR_ARG);
    EXPECT(mxfp4_linear_fprop_noalloc(p, p, 8192, 14336, 4096, &cfg, c, NULL), MXFP4_ERR_WORKSPACE);
    EXPECT(mxfp4_linear_fprop_noalloc(p, p, -64, 64, 64, &cfg, c, NULL), MXFP4_ERR_SHAPE);

    /* status strings and the ABI version */
    for (int s = -2; s <= 9; ++s) {
        const char *msg = mxfp4_status_string((mxfp4_status_t)s);
        EXPECT(msg != NULL && strlen(msg) > 0, 1);
    }
    EXPECT(mxfp4_abi_version(), MXFP4_ABI_VERSION);

    if (failures) {
        fprintf(stderr, "%d validation checks failed\n", failures);
        return 1;
    }
    printf("abi validation: all checks passed\n");
    return 0;
}
