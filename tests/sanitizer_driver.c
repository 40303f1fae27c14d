/*
 * Host-side driver for the sanitizer test (tests/test_host_sanitizers.py):
 * calls every entry point of include/ssm.h on the paths that return before
 * any device work (size queries, argument checks, workspace checks) and
 * compares each return code with the expected one.  Built with AddressSanitizer
 * and UndefinedBehaviorSanitizer around the library's host code; exits 0 and
 * prints "ok <count> checks" when every code matches and no sanitizer fired.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssm.h"

static int checks = 0, failures = 0;

static void expect(int got, int want, const char* what) {
    ++checks;
    if (got != want) {
        ++failures;
        fprintf(stderr, "mismatch: %s returned %d, expected %d\n", what, got, want);
    }
}

/* an aligned address that no path below dereferences */
#define FAKE ((void*)(uintptr_t)0x10000000)
#define FAKE_OFF(n) ((void*)((uintptr_t)0x10000000 + (n)))

int main(void) {
    size_t bytes = 0;
    int64_t M = 0, nfft = 0;
    int32_t form = 0;

    /* workspace sizes: every op, valid shapes including the multi-pass lengths */
    const int64_t Ls[] = {1, 2, 100, 1000, 1024, 3000, 16384, 16385, 40000, 65536};
    for (size_t i = 0; i < sizeof Ls / sizeof Ls[0]; ++i) {
        for (int op = SSM_OP_KERNEL_GEN; op <= SSM_OP_FORWARD_COMPLEX; ++op)
            expect(ssm_workspace_bytes(op, 3, 5, 64, 2, Ls[i], &bytes), SSM_OK, "workspace bytes");
        expect(ssm_workspace_bytes(SSM_OP_DISCRETIZE, 1, 5, 64, 2, Ls[i], &bytes), SSM_OK, "workspace discretize");
    }
    expect(ssm_workspace_bytes(SSM_OP_HIPPO, 0, 0, 1024, 0, 0, &bytes), SSM_OK, "workspace hippo");
    expect(ssm_workspace_bytes(SSM_OP_HIPPO, 0, 0, 1025, 0, 0, &bytes), SSM_ERR_UNSUPPORTED, "workspace hippo cap");
    expect(ssm_workspace_bytes(SSM_OP_HIPPO, 0, 0, 0, 0, 0, &bytes), SSM_ERR_INVALID_ARGUMENT, "workspace hippo N");
    expect(ssm_workspace_bytes(SSM_OP_FORWARD, 1, 1, 1, 1, 1, NULL), SSM_ERR_INVALID_ARGUMENT, "workspace null");
    expect(ssm_workspace_bytes(99, 1, 1, 1, 1, 1, &bytes), SSM_ERR_INVALID_ARGUMENT, "workspace op");
    expect(ssm_workspace_bytes(SSM_OP_FORWARD, 1, 0, 1, 1, 1, &bytes), SSM_ERR_INVALID_ARGUMENT, "workspace H");
    expect(ssm_workspace_bytes(SSM_OP_FORWARD, 1, 1, 1, 5, 1, &bytes), SSM_ERR_UNSUPPORTED, "workspace r");
    expect(ssm_workspace_bytes(SSM_OP_FORWARD, 1, 1, 1, 1, 65537, &bytes), SSM_ERR_UNSUPPORTED, "workspace L");
    expect(ssm_workspace_bytes(SSM_OP_DISCRETIZE, 1, 1, 4097, 1, 8, &bytes), SSM_ERR_UNSUPPORTED, "workspace N");

    /* transform lengths, launch forms, status strings */
    for (int64_t L = 1; L <= 5000; L += 37) expect(ssm_transform_lengths(L, &M, &nfft), SSM_OK, "lengths");
    expect(ssm_transform_lengths(0, &M, &nfft), SSM_ERR_INVALID_ARGUMENT, "lengths L");
    expect(ssm_transform_lengths(5, NULL, &nfft), SSM_ERR_INVALID_ARGUMENT, "lengths null");
    expect(ssm_forward_form(8, 256, 1024, &form), SSM_OK, "form");
    expect(ssm_forward_form(0, 256, 1024, &form), SSM_ERR_INVALID_ARGUMENT, "form batch");
    for (int code = -1; code < 32; ++code) expect(ssm_status_string(code) != NULL, 1, "status string");

    /* entry points: rejections before any device work */
    const ssm_c64* c = (const ssm_c64*)FAKE;
    ssm_c64* co = (ssm_c64*)FAKE;
    const float* f = (const float*)FAKE;
    float* fo = (float*)FAKE;
    int32_t* st = (int32_t*)FAKE;
    expect(ssm_discretize(0, 4, 1, 16, c, c, c, c, c, f, co, NULL, co, st, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT,
           "discretize H");
    expect(ssm_discretize(2, 4, 1, 16, NULL, c, c, c, c, f, co, NULL, co, st, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT,
           "discretize null");
    expect(ssm_discretize(2, 4097, 1, 16, c, c, c, c, c, f, co, NULL, co, st, NULL, 0, NULL), SSM_ERR_UNSUPPORTED,
           "discretize N");
    expect(ssm_kernel_gen(2, 4, 5, 16, c, c, c, c, c, f, co, NULL, st, FAKE, 1 << 30, NULL), SSM_ERR_UNSUPPORTED,
           "kernel_gen r");
    expect(ssm_kernel_gen(2, 4, 1, 16, c, c, c, c, c, f, co, NULL, st, FAKE, 64, NULL), SSM_ERR_WORKSPACE,
           "kernel_gen workspace");
    expect(ssm_fftconv(2, 3, 0, f, 1, NULL, f, fo, FAKE, 1 << 30, NULL), SSM_ERR_INVALID_ARGUMENT, "fftconv L");
    expect(ssm_fftconv(2, 3, 16, f, 1, NULL, (const float*)FAKE_OFF(2), fo, FAKE, 1 << 30, NULL),
           SSM_ERR_INVALID_ARGUMENT, "fftconv align");
    expect(ssm_forward(2, 3, 4, 1, 16, c, c, c, c, c, f, NULL, f, fo, NULL, NULL, FAKE, 64, NULL), SSM_ERR_WORKSPACE,
           "forward workspace");
    expect(ssm_forward(2, 3, 4, 1, 16, c, c, c, c, c, f, NULL, f, NULL, NULL, NULL, FAKE, 1 << 30, NULL),
           SSM_ERR_INVALID_ARGUMENT, "forward null y");
    expect(ssm_forward_noalloc(2, 0, 4, 1, 16, c, c, c, c, c, f, NULL, f, fo, NULL, NULL, NULL),
           SSM_ERR_INVALID_ARGUMENT, "noalloc H");
    expect(ssm_forward_noalloc(2, 1024, 4, 1, 16384, c, c, c, c, c, f, NULL, f, fo, NULL, NULL, NULL),
           SSM_ERR_SCRATCH_LIMIT, "noalloc scratch limit");
    expect(ssm_forward_complex(2, 3, 4, 1, 16, c, c, c, c, c, f, NULL, f, fo, NULL, NULL, NULL, FAKE, 1 << 30, NULL),
           SSM_ERR_INVALID_ARGUMENT, "complex null y_im");
    expect(ssm_forward_complex(2, 3, 4, 5, 16, c, c, c, c, c, f, NULL, f, fo, fo, NULL, NULL, FAKE, 1 << 30, NULL),
           SSM_ERR_UNSUPPORTED, "complex r");
    expect(ssm_step(2, 3, 257, 1, 16, c, c, c, c, c, f, NULL, f, fo, co, NULL, 0, NULL), SSM_ERR_UNSUPPORTED,
           "step N");
    expect(ssm_step(2, 3, 4, 1, 0, c, c, c, c, c, f, NULL, f, fo, co, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT,
           "step T");
    expect(ssm_step(2, 3, 4, 1, 16, c, c, c, c, c, f, NULL, f, fo, (ssm_c64*)FAKE_OFF(4), NULL, 0, NULL),
           SSM_ERR_INVALID_ARGUMENT, "step align");
    expect(ssm_step(2, 3, 4, 1, 16, c, c, c, c, c, f, NULL, f, fo, co, NULL, 48, NULL), SSM_ERR_INVALID_ARGUMENT,
           "step lanes");
    expect(ssm_workspace_bytes(SSM_OP_STEP_PREPARED, 0, 5, 256, 4, 0, &bytes), SSM_OK, "workspace prepared");
    expect(ssm_workspace_bytes(SSM_OP_STEP_PREPARED, 0, 5, 257, 4, 0, &bytes), SSM_ERR_UNSUPPORTED,
           "workspace prepared N");
    expect(ssm_step_prepare(3, 4, 1, c, c, c, c, c, f, FAKE, 64, NULL, NULL), SSM_ERR_WORKSPACE, "prepare bytes");
    expect(ssm_step_prepare(3, 4, 1, c, c, c, c, c, f, FAKE_OFF(64), 1 << 20, NULL, NULL), SSM_ERR_INVALID_ARGUMENT,
           "prepare align");
    expect(ssm_step_prepare(3, 4, 5, c, c, c, c, c, f, FAKE, 1 << 20, NULL, NULL), SSM_ERR_UNSUPPORTED, "prepare r");
    expect(ssm_step_prepared(2, 3, 4, 1, 16, FAKE, 64, NULL, f, fo, co, NULL, 0, NULL), SSM_ERR_WORKSPACE,
           "prepared bytes");
    expect(ssm_step_prepared(2, 3, 4, 1, 0, FAKE, 1 << 20, NULL, f, fo, co, NULL, 0, NULL), SSM_ERR_INVALID_ARGUMENT,
           "prepared T");
    expect(ssm_step_prepared(2, 3, 4, 1, 16, NULL, 1 << 20, NULL, f, fo, co, NULL, 0, NULL),
           SSM_ERR_INVALID_ARGUMENT, "prepared null");
    expect(ssm_step_prepared(2, 3, 65, 1, 16, FAKE, 1 << 20, NULL, f, fo, co, NULL, 16, NULL),
           SSM_ERR_INVALID_ARGUMENT, "prepared lanes");
    expect(ssm_hippo_dplr(3, 8, 1.0, 0, NULL, 0, NULL, co, co, NULL, NULL, NULL, FAKE, 1 << 30, NULL),
           SSM_ERR_INVALID_ARGUMENT, "hippo kind");
    expect(ssm_hippo_dplr(SSM_HIPPO_LEGT, 8, -1.0, 0, NULL, 0, NULL, co, co, NULL, NULL, NULL, FAKE, 1 << 30, NULL),
           SSM_ERR_INVALID_ARGUMENT, "hippo theta");
    expect(ssm_hippo_dplr(SSM_HIPPO_LEGS, 1025, 1.0, 0, NULL, 0, NULL, co, co, NULL, NULL, NULL, FAKE, 1 << 30, NULL),
           SSM_ERR_UNSUPPORTED, "hippo N");
    expect(ssm_hippo_dplr(SSM_HIPPO_LEGS, 8, 1.0, 2, NULL, 0, NULL, co, co, NULL, NULL, NULL, FAKE, 1 << 30, NULL),
           SSM_ERR_INVALID_ARGUMENT, "hippo null B");
    expect(ssm_hippo_dplr(SSM_HIPPO_LEGS, 8, 1.0, 0, NULL, 0, NULL, co, co, NULL, NULL, NULL, FAKE, 100, NULL),
           SSM_ERR_WORKSPACE, "hippo workspace");

    if (failures) {
        fprintf(stderr, "%d of %d checks failed\n", failures, checks);
        return 1;
    }
    printf("ok %d checks\n", checks);
    return 0;
}
