/*
 * A plain C99 caller of the library's public header: it must compile as C,
 * link against libswiglu_q.so and get the documented status codes back from
 * the host-side validation (no call here reaches the GPU: every one either
 * fails validation or has M == 0).  Built and run by tests/test_abi.py.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "swiglu_q.h"

static int failures = 0;

static void expect(int got, int want, const char *what) {
    if (got != want) {
        fprintf(stderr, "%s: got %d (%s), want %d (%s)\n", what, got, swiglu_q_strerror(got), want,
                swiglu_q_strerror(want));
        ++failures;
    }
}

int main(void) {
    /* fake, 256-byte aligned device addresses: validation never dereferences them */
    char *p = (char *)(uintptr_t)(1u << 20);
    const uint32_t *w = (const uint32_t *)p;
    int t;

    if (swiglu_q_version() == NULL || swiglu_q_version()[0] == '\0') {
        fprintf(stderr, "empty version string\n");
        ++failures;
    }
    for (int s = SWQ_OK; s <= SWQ_ERR_WORKSPACE; ++s)
        if (swiglu_q_strerror(s) == NULL || strlen(swiglu_q_strerror(s)) == 0) {
            fprintf(stderr, "no text for status %d\n", s);
            ++failures;
        }

    /* forward: M == 0 is a no-op; every other case fails before any HIP call */
    expect(swiglu_q_forward(p, w, p, p, w, p, p, 0, 256, 64, 4, 64, 4, 64, SWQ_MATCH, p, NULL), SWQ_OK, "M = 0");
    expect(swiglu_q_forward(NULL, w, p, p, w, p, p, 4, 256, 64, 4, 64, 4, 64, SWQ_MATCH, p, NULL), SWQ_ERR_NULL,
           "x = NULL");
    expect(swiglu_q_forward(p, w, p, p, w, p, p, 4, 256, 64, 3, 64, 4, 64, SWQ_MATCH, p, NULL), SWQ_ERR_UNSUPPORTED,
           "3-bit gate");
    expect(swiglu_q_forward(p, w, p, p, w, p, p, 4, 96, 64, 4, 64, 4, 64, SWQ_MATCH, p, NULL), SWQ_ERR_SHAPE,
           "H not a multiple of gs");
    expect(swiglu_q_forward(p, w, p, p, w, p, p, 4, 256, 64, 4, 64, 4, 64, 7, p, NULL), SWQ_ERR_UNSUPPORTED,
           "unknown mode");
    expect(swiglu_q_forward(p + 8, w, p, p, w, p, p, 4, 256, 64, 4, 64, 4, 64, SWQ_MATCH, p, NULL), SWQ_ERR_ALIGN,
           "x misaligned");
    expect(swiglu_q_forward(p, w, p, p, w, p, p, 4, 256, 64, 4, 64, 4, 64, SWQ_F32, p + 2, NULL), SWQ_ERR_ALIGN,
           "f32 out misaligned");

    /* linear */
    expect(swiglu_q_linear(p, w, p, p, 0, 256, 65, 4, 64, SWQ_LINEAR_BF16, p, NULL), SWQ_OK, "linear M = 0");
    expect(swiglu_q_linear(p, w, p, p, 4, 256, 0, 4, 64, SWQ_LINEAR_BF16, p, NULL), SWQ_ERR_SHAPE, "linear N = 0");
    expect(swiglu_q_linear(p, w, p, p, 4, 256, 65, 4, 64, 2, p, NULL), SWQ_ERR_UNSUPPORTED, "linear out mode");
    expect(swiglu_q_linear(p, NULL, p, p, 4, 256, 65, 4, 64, SWQ_LINEAR_F32, p, NULL), SWQ_ERR_NULL,
           "linear W = NULL");

    /* whole MLP */
    expect(swiglu_q_mlp(p, w, p, p, w, p, p, w, p, p, NULL, 0, 256, 512, 256, 4, 64, 4, 64, 4, 64,
                        SWQ_LINEAR_BF16, p, NULL), SWQ_OK, "mlp M = 0");
    expect(swiglu_q_mlp(p, w, p, p, w, p, p, NULL, p, p, p, 4, 256, 512, 256, 4, 64, 4, 64, 4, 64,
                        SWQ_LINEAR_BF16, p, NULL), SWQ_ERR_NULL, "mlp Wd = NULL");
    expect(swiglu_q_mlp(p, w, p, p, w, p, p, w, p, p, p, 4, 256, 480, 256, 4, 64, 4, 64, 4, 64,
                        SWQ_LINEAR_BF16, p, NULL), SWQ_ERR_SHAPE, "mlp I not a multiple of gs_d");
    expect(swiglu_q_mlp(p, w, p, p, w, p, p, w, p, p, p + 1, 4, 256, 512, 256, 4, 64, 4, 64, 4, 64,
                        SWQ_LINEAR_BF16, p, NULL), SWQ_ERR_ALIGN, "mlp residual misaligned");

    /* debug hook */
    expect(swiglu_q_debug_gemm(p, w, p, p, w, p, p, 4, 256, 64, 4, 64, 4, 64, 5, (float *)p, (float *)p, NULL),
           SWQ_ERR_UNSUPPORTED, "debug path");

    /* support predicate, threshold, workspace size */
    expect(swiglu_q_supported(2048, 4, 64, 4, 64, SWQ_MATCH), 1, "supported 4/64");
    expect(swiglu_q_supported(2048, 2, 32, 8, 128, SWQ_F32), 1, "supported 2/32 + 8/128");
    expect(swiglu_q_supported(2048, 5, 64, 4, 64, SWQ_MATCH), 0, "5-bit unsupported");
    t = swiglu_q_get_m_threshold();
    swiglu_q_set_m_threshold(9);
    expect(swiglu_q_get_m_threshold(), 9, "threshold round trip");
    expect(swiglu_q_path_for(8, 2048, 5632), SWQ_PATH_GEMV, "path of M = 8 under T = 9");
    expect(swiglu_q_path_for(9, 2048, 5632), SWQ_PATH_MFMA, "path of M = 9 under T = 9");
    expect(swiglu_q_path_for(0, 2048, 5632), -1, "path of M = 0");
    swiglu_q_set_m_threshold(-1);
    expect(swiglu_q_get_m_threshold(), t, "default rule restored");
    if (swiglu_q_workspace_bytes(512, 2048, 8192, 4, 64, 4, 64) <= 0) {
        fprintf(stderr, "no workspace size for a valid shape\n");
        ++failures;
    }
    expect((int)swiglu_q_workspace_bytes(512, 2048, 8192, 3, 64, 4, 64), 0, "workspace of an invalid spec");

    if (failures == 0) printf("c abi ok\n");
    return failures == 0 ? 0 : 1;
}
