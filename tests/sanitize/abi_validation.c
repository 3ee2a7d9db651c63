/* Host-only driver for the C ABI's argument checks, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer together with csrc/abi.cpp. Every call here is invalid (or a pure size
 * query), so no HIP call is reached and no GPU is needed. Pointers are fake, never dereferenced
 * addresses: the checks only compare their values. Exits 0 when every call returns the documented
 * status; a sanitizer report aborts the run. */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssm_scan.h"

#define PTR(off) ((void *)(uintptr_t)(0x7F0000000000ull + (uint64_t)(off)))
#define G (1ull << 30)

static int failures = 0;

static void expect(int got, int want, const char *what) {
    if (got != want) {
        printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, ssm_last_error_message());
        ++failures;
    } else if (want != SSM_OK && ssm_last_error_message()[0] == '\0') {
        printf("FAIL %s: no error message\n", what);
        ++failures;
    }
}

typedef struct {
    void *u, *delta, *A, *B, *C, *D, *z, *bias, *out, *last;
    int64_t nb, nd, L, N;
    int io;
    unsigned flags;
    void *ws;
    size_t ws_bytes;
} scan_args;

static scan_args scan_ok(void) {
    scan_args a = {PTR(0), PTR(G), PTR(2 * G), PTR(3 * G), PTR(4 * G), NULL, NULL, NULL, PTR(5 * G), NULL,
                   1, 64, 128, 16, SSM_DTYPE_F32, 0, PTR(8 * G), (size_t)1 << 30};
    return a;
}

static int scan(const scan_args *a) {
    return ssm_scan_fwd_ex(a->u, a->delta, (const float *)a->A, a->B, a->C, (const float *)a->D, a->z,
                           (const float *)a->bias, 1, a->out, (float *)a->last, a->nb, a->nd, a->L, a->N, a->io,
                           a->flags, a->ws, a->ws_bytes, NULL);
}

static void scan_cases(void) {
    scan_args a;
    void **fields[] = {&a.u, &a.delta, &a.A, &a.B, &a.C, &a.out};
    for (unsigned i = 0; i < sizeof(fields) / sizeof(fields[0]); ++i) {
        a = scan_ok();
        *fields[i] = NULL;
        expect(scan(&a), SSM_ERR_NULL_POINTER, "scan null");
    }
    const int64_t shapes[][4] = {{0, 64, 128, 16}, {1, 0, 128, 16}, {1, 64, 0, 16}, {1, 64, 128, 0},
                                 {1, 64, 128, 17}, {-3, 64, 128, 16}, {1ll << 40, 1ll << 40, 1, 16},
                                 {INT64_MAX, INT64_MAX, INT64_MAX, 16}, {1, INT64_MAX, 2, 16},
                                 {1, 1, INT64_MAX, 16}, {INT64_MIN, 1, 1, 16}};
    for (unsigned i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
        a = scan_ok();
        a.nb = shapes[i][0]; a.nd = shapes[i][1]; a.L = shapes[i][2]; a.N = shapes[i][3];
        expect(scan(&a), SSM_ERR_BAD_SHAPE, "scan shape");
    }
    a = scan_ok(); a.io = 2; expect(scan(&a), SSM_ERR_BAD_DTYPE, "scan dtype");
    a = scan_ok(); a.io = -1; expect(scan(&a), SSM_ERR_BAD_DTYPE, "scan dtype");
    void **all[] = {&a.u, &a.delta, &a.A, &a.B, &a.C, &a.D, &a.z, &a.bias, &a.out, &a.last};
    for (unsigned i = 0; i < sizeof(all) / sizeof(all[0]); ++i) {
        a = scan_ok();
        *all[i] = (char *)PTR((6 + i) * G) + 4;
        expect(scan(&a), SSM_ERR_MISALIGNED, "scan misaligned");
    }
    a = scan_ok(); a.out = a.u; expect(scan(&a), SSM_ERR_BAD_SHAPE, "scan out aliases u");
    a = scan_ok(); a.last = (char *)a.B + 64; expect(scan(&a), SSM_ERR_BAD_SHAPE, "scan last_state inside B");
    const unsigned flags[] = {4u, 8u, 0x80000000u, SSM_FLAG_ZOH | 4u, SSM_FLAG_OUT_F32 | 16u};
    for (unsigned i = 0; i < sizeof(flags) / sizeof(flags[0]); ++i) {
        a = scan_ok(); a.flags = flags[i];
        expect(scan(&a), SSM_ERR_BAD_FLAGS, "scan flags");
    }
    const size_t need = ssm_scan_fwd_workspace_size(1, 64, 128);
    a = scan_ok(); a.ws = NULL; expect(scan(&a), SSM_ERR_WORKSPACE, "scan workspace NULL");
    a = scan_ok(); a.ws_bytes = need - 1; expect(scan(&a), SSM_ERR_WORKSPACE, "scan workspace small");
    a = scan_ok(); a.ws = (char *)a.ws + 8; expect(scan(&a), SSM_ERR_MISALIGNED, "scan workspace misaligned");
    a = scan_ok(); a.ws = (char *)a.out - 1024; a.ws_bytes = need;
    expect(scan(&a), SSM_ERR_WORKSPACE, "scan workspace overlaps out");
    /* the plain entry point takes the same path */
    a = scan_ok();
    expect(ssm_scan_fwd(a.u, a.delta, (const float *)a.A, a.B, a.C, NULL, NULL, NULL, 1, a.out, NULL, 1, 64, 128, 99,
                        0, a.ws, a.ws_bytes, NULL), SSM_ERR_BAD_SHAPE, "scan plain shape");
    if (!strstr(ssm_last_error_message(), "dstate=99")) {
        printf("FAIL scan plain shape: message '%s'\n", ssm_last_error_message());
        ++failures;
    }
    /* the allocation-free variant: validation, then the size limit of its array, before any HIP call */
    a = scan_ok();
    expect(ssm_scan_fwd_noalloc(a.u, a.delta, (const float *)a.A, a.B, a.C, NULL, NULL, NULL, 1, a.out, NULL,
                                1, 2048, 65536, 16, 1, 0, NULL), SSM_ERR_WORKSPACE, "noalloc beyond its array");
    expect(ssm_scan_fwd_noalloc(NULL, a.delta, (const float *)a.A, a.B, a.C, NULL, NULL, NULL, 1, a.out, NULL,
                                1, 64, 128, 16, 1, 0, NULL), SSM_ERR_NULL_POINTER, "noalloc null");
    expect(ssm_scan_fwd_noalloc(a.u, a.delta, (const float *)a.A, a.B, a.C, NULL, NULL, NULL, 1, a.out, NULL,
                                1, 64, 128, 16, 1, 64u, NULL), SSM_ERR_BAD_FLAGS, "noalloc flags");
}

static void size_cases(void) {
    const int64_t bad[][3] = {{0, 64, 128}, {1, 0, 128}, {1, 64, 0}, {-1, 64, 128}, {1ll << 40, 1ll << 40, 1},
                              {INT64_MAX, INT64_MAX, INT64_MAX}, {INT64_MIN, INT64_MIN, INT64_MIN}, {1, 1, INT64_MAX}};
    for (unsigned i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
        if (ssm_scan_fwd_workspace_size(bad[i][0], bad[i][1], bad[i][2]) != 0 ||
            ssm_scan_bwd_workspace_size(bad[i][0], bad[i][1], bad[i][2]) != 0 ||
            ssm_scan_segment_tokens(bad[i][0], bad[i][1], bad[i][2]) > 64) {
            printf("FAIL size query %u\n", i);
            ++failures;
        }
    }
    const int64_t good[][3] = {{1, 64, 128}, {4, 5120, 2048}, {1, 2048, 65536}, {3, 7, 5}};
    for (unsigned i = 0; i < sizeof(good) / sizeof(good[0]); ++i) {
        const size_t f = ssm_scan_fwd_workspace_size(good[i][0], good[i][1], good[i][2]);
        if (f == 0 || ssm_scan_bwd_workspace_size(good[i][0], good[i][1], good[i][2]) <= f ||
            ssm_scan_segment_tokens(good[i][0], good[i][1], good[i][2]) != 64) {
            printf("FAIL size query good %u\n", i);
            ++failures;
        }
    }
    if (ssm_scan_fwd_noalloc_max_workspace() != ((size_t)64 << 20)) { printf("FAIL noalloc max\n"); ++failures; }
    for (int s = -5; s < 40; ++s)
        if (!ssm_status_string(s) || !ssm_status_string(s)[0]) { printf("FAIL status string %d\n", s); ++failures; }
    if (ssm_abi_version() != SSM_ABI_VERSION) { printf("FAIL abi version\n"); ++failures; }
    const int def = ssm_set_wait_limit(7);
    if (ssm_set_wait_limit(0) != 7 || ssm_set_wait_limit(-1) != def) { printf("FAIL wait limit\n"); ++failures; }
    ssm_set_wait_limit(0);
}

static void other_entry_points(void) {
    void *p[16];
    for (int i = 0; i < 16; ++i) p[i] = PTR((uint64_t)i * G);
    /* backward */
#define BWD(u, dl, A, B, C, z, dout, du, dd, dA, dB, dC, dz, nb, nd, L, N, io, ws, wsb)                               \
    ssm_scan_bwd(u, dl, (const float *)(A), B, C, NULL, z, NULL, 1, dout, du, dd, (float *)(dA), (float *)(dB),   \
                 (float *)(dC), NULL, dz, NULL, nb, nd, L, N, io, ws, wsb, NULL)
    const size_t bw = ssm_scan_bwd_workspace_size(1, 64, 128);
    expect(BWD(NULL, p[1], p[2], p[3], p[4], NULL, p[5], p[6], p[7], p[8], p[9], p[10], NULL, 1, 64, 128, 16, 0, p[12], bw),
           SSM_ERR_NULL_POINTER, "bwd null u");
    expect(BWD(p[0], p[1], p[2], p[3], p[4], p[11], p[5], p[6], p[7], p[8], p[9], p[10], NULL, 1, 64, 128, 16, 0, p[12], bw),
           SSM_ERR_NULL_POINTER, "bwd z without dz");
    expect(BWD(p[0], p[1], p[2], p[3], p[4], NULL, p[5], p[6], p[7], p[8], p[9], p[10], NULL, INT64_MAX, 64, 128, 16, 0,
               p[12], bw), SSM_ERR_BAD_SHAPE, "bwd shape");
    expect(BWD(p[0], p[1], p[2], p[3], p[4], NULL, p[5], p[6], p[7], p[8], p[9], p[10], NULL, 1, 64, 128, 16, 9, p[12], bw),
           SSM_ERR_BAD_DTYPE, "bwd dtype");
    expect(BWD(p[0], p[1], p[2], p[3], p[4], NULL, p[5], p[1], p[7], p[8], p[9], p[10], NULL, 1, 64, 128, 16, 0, p[12], bw),
           SSM_ERR_BAD_SHAPE, "bwd du aliases delta");
    expect(BWD(p[0], p[1], p[2], p[3], p[4], NULL, p[5], p[6], p[7], p[8], p[9], p[10], NULL, 1, 64, 128, 16, 0, p[12], bw - 1),
           SSM_ERR_WORKSPACE, "bwd workspace small");
    /* decode update */
#define UPD(st, x, dl, A, B, C, z, out, nb, nd, N, io, fl)                                                             \
    ssm_state_update_ex((float *)(st), x, dl, (const float *)(A), B, C, NULL, z, out, nb, nd, N, io, fl, NULL)
    expect(UPD(NULL, p[1], p[2], p[3], p[4], p[5], NULL, p[6], 2, 64, 16, 1, 0), SSM_ERR_NULL_POINTER, "update null");
    expect(UPD(p[0], p[1], p[2], p[3], p[4], p[5], NULL, p[6], 2, 64, 17, 1, 0), SSM_ERR_BAD_SHAPE, "update N");
    expect(UPD(p[0], p[1], p[2], p[3], p[4], p[5], NULL, p[6], INT64_MAX, INT64_MAX, 16, 1, 0), SSM_ERR_BAD_SHAPE,
           "update huge");
    expect(UPD(p[0], p[1], p[2], p[3], p[4], p[5], NULL, p[6], 2, 64, 16, 5, 0), SSM_ERR_BAD_DTYPE, "update dtype");
    expect(UPD(p[0], p[1], p[2], p[3], p[4], p[5], (char *)p[7] + 2, p[6], 2, 64, 16, 1, 0), SSM_ERR_MISALIGNED,
           "update misaligned z");
    expect(UPD(p[0], p[1], p[2], p[3], p[4], p[5], NULL, p[0], 2, 64, 16, 1, 0), SSM_ERR_BAD_SHAPE, "update out in state");
    expect(UPD(p[0], p[1], p[2], p[3], p[4], p[5], NULL, p[6], 2, 64, 16, 1, 4u), SSM_ERR_BAD_FLAGS, "update flags");
    /* convolution and its decode window */
    expect(ssm_causal_conv1d(NULL, (const float *)p[1], NULL, 1, p[2], 2, 64, 100, 4, 0, NULL), SSM_ERR_NULL_POINTER,
           "conv null");
    const int64_t widths[] = {0, 9, 12, -1, INT64_MAX};
    for (unsigned i = 0; i < sizeof(widths) / sizeof(widths[0]); ++i)
        expect(ssm_causal_conv1d(p[0], (const float *)p[1], NULL, 1, p[2], 2, 64, 100, widths[i], 0, NULL),
               SSM_ERR_BAD_SHAPE, "conv width");
    expect(ssm_causal_conv1d(p[0], (const float *)p[1], NULL, 1, p[2], INT64_MAX, INT64_MAX, INT64_MAX, 4, 0, NULL),
           SSM_ERR_BAD_SHAPE, "conv huge");
    expect(ssm_causal_conv1d(p[0], (const float *)p[1], NULL, 1, (char *)p[0] + 64, 2, 64, 100, 4, 0, NULL),
           SSM_ERR_BAD_SHAPE, "conv out in x");
    expect(ssm_conv_window_update((float *)p[0], p[1], (const float *)p[2], NULL, 1, p[3], 2, 64, 9, 1, NULL),
           SSM_ERR_BAD_SHAPE, "window width");
    expect(ssm_conv_window_update((float *)p[0], p[1], (const float *)p[2], NULL, 1, p[0], 2, 64, 4, 1, NULL),
           SSM_ERR_BAD_SHAPE, "window out in window");
    expect(ssm_conv_window_update((float *)p[0], p[1], (const float *)p[2], NULL, 1, p[3], 2, 64, 4, -1, NULL),
           SSM_ERR_BAD_DTYPE, "window dtype");
}

static void ssd_cases(void) {
    void *p[8];
    for (int i = 0; i < 8; ++i) p[i] = PTR((uint64_t)i * G);
#define SSD(x, a, b, c, y, fs, nb, L, H, P, N, ng, io, fl)                                                             \
    ssm_ssd_scan(x, (const float *)(a), b, c, y, (float *)(fs), nb, L, H, P, N, ng, io, fl, NULL, 0, NULL)
    expect(SSD(NULL, p[1], p[2], p[3], p[4], NULL, 2, 100, 8, 64, 128, 1, 1, 0u), SSM_ERR_NULL_POINTER, "ssd null");
    const int64_t shapes[][6] = {{0, 100, 8, 64, 128, 1}, {2, 100, 6, 64, 128, 4}, {2, 100, 8, 72, 128, 1},
                                 {2, 100, 8, 64, 136, 1}, {INT64_MAX, INT64_MAX, 8, 64, 128, 1},
                                 {1, INT64_MAX, INT64_MAX, 64, 128, 1}, {2, 100, 8, 64, 128, INT64_MAX}};
    for (unsigned i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        expect(SSD(p[0], p[1], p[2], p[3], p[4], NULL, shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3],
                   shapes[i][4], shapes[i][5], 1, 0u), SSM_ERR_BAD_SHAPE, "ssd shape");
    expect(SSD(p[0], p[1], p[2], p[3], p[4], NULL, 2, 100, 8, 64, 128, 1, 7, 0u), SSM_ERR_BAD_DTYPE, "ssd dtype");
    expect(SSD(p[0], p[1], p[2], p[3], p[4], NULL, 2, 100, 8, 64, 128, 1, 1, SSM_FLAG_ZOH), SSM_ERR_BAD_FLAGS, "ssd flags");
    expect(SSD(p[0], p[1], p[2], p[3], (char *)p[0] + 64, NULL, 2, 100, 8, 64, 128, 1, 1, 0u), SSM_ERR_BAD_SHAPE,
           "ssd y in x");
    expect(SSD(p[0], p[1], p[2], p[3], p[4], (char *)p[2] + 4, 2, 100, 8, 64, 128, 1, 1, 0u), SSM_ERR_MISALIGNED,
           "ssd final state misaligned");
    const size_t need = ssm_ssd_scan_workspace_size(2, 100, 8, 64, 128, 1);
    expect(need > 0 ? SSM_OK : SSM_ERR_WORKSPACE, SSM_OK, "ssd workspace size");
    expect(ssm_ssd_scan(p[0], (const float *)p[1], p[2], p[3], p[4], NULL, 2, 100, 8, 64, 128, 1, 1, 0u, p[6], need - 1,
                        NULL), SSM_ERR_WORKSPACE, "ssd workspace small");
    expect(ssm_ssd_scan(p[0], (const float *)p[1], p[2], p[3], p[4], NULL, 2, 100, 8, 64, 128, 1, 1, 0u, (char *)p[4] + 64,
                        need, NULL), SSM_ERR_WORKSPACE, "ssd workspace in y");
    expect(ssm_ssd_scan(p[0], (const float *)p[1], p[2], p[3], p[4], NULL, 2, 100, 8, 64, 128, 1, 1, 0u, NULL, need,
                        NULL), SSM_ERR_WORKSPACE, "ssd NULL workspace with bytes");
}

/* Each thread's last error message is its own. */
static void *thread_body(void *arg) {
    const int shape = *(const int *)arg;
    scan_args a = scan_ok();
    for (int i = 0; i < 2000; ++i) {
        if (shape) a.N = 99; else a.u = NULL;
        const int st = scan(&a);
        const char *m = ssm_last_error_message();
        if (st != (shape ? SSM_ERR_BAD_SHAPE : SSM_ERR_NULL_POINTER) ||
            !strstr(m, shape ? "dstate=99" : "u")) {
            printf("FAIL thread-local message: %d '%s'\n", st, m);
            return (void *)1;
        }
    }
    return NULL;
}

int main(void) {
    scan_cases();
    size_cases();
    other_entry_points();
    ssd_cases();
    pthread_t t[4];
    int kinds[4] = {0, 1, 0, 1};
    for (int i = 0; i < 4; ++i) pthread_create(&t[i], NULL, thread_body, &kinds[i]);
    for (int i = 0; i < 4; ++i) {
        void *r = NULL;
        pthread_join(t[i], &r);
        if (r) ++failures;
    }
    if (failures) {
        printf("%d failures\n", failures);
        return 1;
    }
    printf("abi validation ok\n");
    return 0;
}
