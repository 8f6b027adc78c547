/*
 * A plain C caller of the library's C ABI (include/gqa_decode.h): no Python, no
 * torch, only hipMalloc'd buffers and the declared entry points.  Test
 * infrastructure: it links the CPU oracle (oracle/oracle.c) to check results.
 *
 *   gqa_c_caller host   argument checks, plans, tuning and status strings
 *                       (host code only: needs no GPU)
 *   gqa_c_caller gpu    gqa_decode, gqa_paged_decode, gqa_decode_noalloc,
 *                       gqa_decode_partials + gqa_decode_combine, gqa_decode_fp8
 *                       and gqa_decode_mq on small ragged cases against the
 *                       oracle, elementwise |gpu - oracle| <= 2e-3 + 2e-3 |oracle|
 *
 * Exit status 0 when every check passes, 1 otherwise.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gqa_decode.h"

/* the oracle's entry points (oracle/oracle.c) */
int oracle_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seq_lens, int B,
                  int Hq, int Hkv, int D, int S_max, float scale, double *out);
int oracle_paged_decode(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                        const int32_t *seq_lens, const int32_t *page_table, int B, int Hq, int Hkv, int D,
                        int page_size, int num_pages, int max_pages, float scale, double *out);
int oracle_decode_fp8(const uint16_t *q, const uint8_t *k, const uint8_t *v, const int32_t *seq_lens, int B,
                      int Hq, int Hkv, int D, int S_max, float scale, float k_scale, float v_scale, int chunk,
                      double *out);
int oracle_decode_mq(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int32_t *seq_lens, int B,
                     int M, int Hq, int Hkv, int D, int S_max, float scale, int chunk, double *out);

static int failures = 0;

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fprintf(stderr, "\n");                        \
            ++failures;                                   \
        }                                                 \
    } while (0)

/* Inputs: a counter-based generator (splitmix64 of a seed and an index), each
 * draw mapped to a value in [-2, 2) and rounded to bf16 (nearest, ties to even). */
static uint64_t splitmix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static void fill_bf16(uint16_t *dst, size_t n, uint64_t seed) {
    for (size_t i = 0; i < n; ++i) {
        const double x = (double)(splitmix64(seed * 0x100000001B3ull + i) >> 11) / 9007199254740992.0;
        dst[i] = f32_to_bf16((float)(4.0 * x - 2.0));
    }
}

/* E4M3 bytes from the same generator, the two NaN codes (0x7F, 0xFF) replaced by +-448. */
static void fill_e4m3(uint8_t *dst, size_t n, uint64_t seed) {
    for (size_t i = 0; i < n; ++i) {
        const uint8_t x = (uint8_t)(splitmix64(seed * 0x100000001B3ull + i) >> 56);
        dst[i] = (x & 0x7F) == 0x7F ? (uint8_t)(x - 1) : x;
    }
}

static int compare(const float *got, const double *ref, size_t n, const char *what) {
    size_t bad = 0;
    double worst = 0.0;
    for (size_t i = 0; i < n; ++i) {
        const double err = fabs((double)got[i] - ref[i]);
        if (!(err <= 2e-3 + 2e-3 * fabs(ref[i]))) ++bad;
        if (err > worst || err != err) worst = err;
    }
    printf("%-44s n=%zu max_abs_err=%.3g bad=%zu\n", what, n, worst, bad);
    CHECK(bad == 0, "%s: %zu of %zu elements outside the tolerance", what, bad, n);
    return bad == 0;
}

#define HIP_OK(call)                                                           \
    do {                                                                       \
        hipError_t e_ = (call);                                                \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

static void *dev_copy(const void *host, size_t bytes) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes > 0 ? bytes : 16));
    if (bytes > 0) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static void *zeroed_workspace(size_t bytes) {
    void *ws = NULL;
    HIP_OK(hipMalloc(&ws, bytes > 0 ? bytes : 16));
    HIP_OK(hipMemset(ws, 0, bytes > 0 ? bytes : 16)); /* the counter header starts at zero */
    return ws;
}

/* ------------------------------------------------------------------ host mode */
static void host_checks(void) {
    gqa_plan_t plan;
    /* pure host planning, explicit CU count */
    CHECK(gqa_decode_plan(1, 24, 4, 256, 4096, 0, 0, 256, &plan) == GQA_OK, "plan GQA-6");
    CHECK(plan.partition == 0 && plan.grid == 256 && plan.split_tokens == 4 * plan.tile_tokens, "GQA-6 plan shape");
    CHECK(gqa_decode_plan(32, 32, 8, 128, 8192, 32, 0, 256, &plan) == GQA_OK && plan.partition == 1,
          "paged batch plan: even shares");
    CHECK(gqa_decode_plan(1, 8, 3, 128, 100, 0, 0, 256, &plan) == GQA_ERR_SHAPE, "Hq %% Hkv");
    CHECK(gqa_decode_plan(1, 8, 2, 96, 100, 0, 0, 256, &plan) == GQA_ERR_UNSUPPORTED, "head_dim 96");
    CHECK(gqa_decode_plan(1, 8, 2, 128, 100, 0, 0, 256, NULL) == GQA_ERR_NULL, "NULL plan");

    /* argument checks run before any device work */
    char buf[64] __attribute__((aligned(16)));
    const void *p = buf;
    float *out = (float *)buf;
    const int32_t *lens = (const int32_t *)buf;
    CHECK(gqa_decode(NULL, p, p, lens, 1, 8, 2, 128, 64, 0.1f, out, NULL, 0, 0, NULL) == GQA_ERR_NULL, "NULL q");
    CHECK(gqa_decode(p, p, p, lens, 1, 8, 3, 128, 64, 0.1f, out, NULL, 0, 0, NULL) == GQA_ERR_SHAPE, "Hq %% Hkv");
    CHECK(gqa_decode(p, p, p, lens, 1, 8, 2, 96, 64, 0.1f, out, NULL, 0, 0, NULL) == GQA_ERR_UNSUPPORTED,
          "head_dim 96");
    CHECK(gqa_decode(p, p, p, lens, 1, 8, 2, 128, 64, 0.1f, (float *)(buf + 4), NULL, 0, 0, NULL) == GQA_ERR_ALIGN,
          "misaligned out");
    CHECK(gqa_paged_decode(p, p, p, lens, lens, 1, 8, 2, 128, 24, 4, 4, 0.1f, out, NULL, 0, 0, NULL) ==
              GQA_ERR_UNSUPPORTED,
          "page size 24");
    CHECK(gqa_decode(NULL, NULL, NULL, NULL, 0, 8, 2, 128, 64, 0.1f, NULL, NULL, 0, 0, NULL) == GQA_OK,
          "B = 0 is a no-op");

    /* the tuning: read, replace, reject out-of-range fields, restore */
    gqa_tuning_t t0, t;
    gqa_decode_get_tuning(&t0);
    t = t0;
    t.fold = 2;
    CHECK(gqa_decode_set_tuning(&t) == GQA_OK, "set tuning");
    CHECK(gqa_decode_plan(1, 24, 4, 256, 4096, 0, 0, 256, &plan) == GQA_OK && plan.fused == 1, "fold=2 plan");
    t.qk_mode = 7;
    CHECK(gqa_decode_set_tuning(&t) == GQA_ERR_SHAPE, "qk_mode 7 rejected");
    CHECK(gqa_decode_set_tuning(NULL) == GQA_ERR_NULL, "NULL tuning");
    CHECK(gqa_decode_set_tuning(&t0) == GQA_OK, "restore tuning");

    for (int s = 0; s <= 7; ++s) CHECK(gqa_status_string((gqa_status_t)s) != NULL, "status string %d", s);
    printf("host checks: %s\n", failures == 0 ? "ok" : "FAILED");
}

/* ------------------------------------------------------------------ GPU mode */
static void contiguous_case(int B, int Hq, int Hkv, int D, int S_max, const int32_t *lens, float scale,
                            uint64_t seed, int noalloc) {
    const size_t nq = (size_t)B * Hq * D, nkv = (size_t)B * Hkv * S_max * D, no = nq;
    uint16_t *q = malloc(nq * 2), *k = malloc(nkv * 2), *v = malloc(nkv * 2);
    float *got = malloc(no * 4);
    double *ref = malloc(no * 8);
    fill_bf16(q, nq, seed);
    fill_bf16(k, nkv, seed + 1);
    fill_bf16(v, nkv, seed + 2);
    void *dq = dev_copy(q, nq * 2), *dk = dev_copy(k, nkv * 2), *dv = dev_copy(v, nkv * 2);
    void *dl = dev_copy(lens, (size_t)B * 4);
    float *dout = NULL;
    HIP_OK(hipMalloc((void **)&dout, no * 4));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    gqa_status_t s;
    char what[96];
    if (noalloc) {
        s = gqa_decode_noalloc(dq, dk, dv, dl, B, Hq, Hkv, D, S_max, scale, dout, 0, stream);
        snprintf(what, sizeof what, "gqa_decode_noalloc B=%d Hq=%d Hkv=%d D=%d", B, Hq, Hkv, D);
    } else {
        const size_t ws_bytes = gqa_decode_workspace_bytes(B, Hq, Hkv, D, S_max, 0, 0);
        CHECK(ws_bytes != (size_t)-1, "workspace query");
        void *ws = NULL;
        HIP_OK(hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 16));
        HIP_OK(hipMemset(ws, 0, ws_bytes > 0 ? ws_bytes : 16)); /* the counter header starts at zero */
        s = gqa_decode(dq, dk, dv, dl, B, Hq, Hkv, D, S_max, scale, dout, ws, ws_bytes, 0, stream);
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipFree(ws));
        snprintf(what, sizeof what, "gqa_decode B=%d Hq=%d Hkv=%d D=%d", B, Hq, Hkv, D);
    }
    CHECK(s == GQA_OK, "%s returned %s", what, gqa_status_string(s));
    HIP_OK(hipStreamSynchronize(stream));
    HIP_OK(hipMemcpy(got, dout, no * 4, hipMemcpyDeviceToHost));
    CHECK(oracle_decode(q, k, v, lens, B, Hq, Hkv, D, S_max, scale, ref) == 0, "oracle");
    if (s == GQA_OK) compare(got, ref, no, what);
    HIP_OK(hipStreamDestroy(stream));
    hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dl), hipFree(dout);
    free(q), free(k), free(v), free(got), free(ref);
}

static void paged_case(int B, int Hq, int Hkv, int D, int page_size, int max_pages, const int32_t *lens,
                       float scale, uint64_t seed) {
    int num_pages = 0;
    for (int b = 0; b < B; ++b) num_pages += (lens[b] + page_size - 1) / page_size;
    num_pages += 3;
    const size_t nq = (size_t)B * Hq * D, nkv = (size_t)num_pages * Hkv * page_size * D;
    uint16_t *q = malloc(nq * 2), *k = malloc(nkv * 2), *v = malloc(nkv * 2);
    int32_t *table = malloc((size_t)B * max_pages * 4);
    float *got = malloc(nq * 4);
    double *ref = malloc(nq * 8);
    fill_bf16(q, nq, seed);
    fill_bf16(k, nkv, seed + 1);
    fill_bf16(v, nkv, seed + 2);
    /* pages handed out back to front, unused entries -1 */
    int next = num_pages - 1;
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < max_pages; ++i)
            table[(size_t)b * max_pages + i] = i < (lens[b] + page_size - 1) / page_size ? next-- : -1;
    void *dq = dev_copy(q, nq * 2), *dk = dev_copy(k, nkv * 2), *dv = dev_copy(v, nkv * 2);
    void *dl = dev_copy(lens, (size_t)B * 4), *dt = dev_copy(table, (size_t)B * max_pages * 4);
    float *dout = NULL;
    HIP_OK(hipMalloc((void **)&dout, nq * 4));
    const size_t ws_bytes = gqa_decode_workspace_bytes(B, Hq, Hkv, D, max_pages * page_size, page_size, 0);
    void *ws = NULL;
    HIP_OK(hipMalloc(&ws, ws_bytes > 0 ? ws_bytes : 16));
    HIP_OK(hipMemset(ws, 0, ws_bytes > 0 ? ws_bytes : 16));
    const gqa_status_t s = gqa_paged_decode(dq, dk, dv, dl, dt, B, Hq, Hkv, D, page_size, num_pages, max_pages,
                                            scale, dout, ws, ws_bytes, 0, NULL);
    char what[96];
    snprintf(what, sizeof what, "gqa_paged_decode B=%d Hq=%d Hkv=%d D=%d ps=%d", B, Hq, Hkv, D, page_size);
    CHECK(s == GQA_OK, "%s returned %s", what, gqa_status_string(s));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got, dout, nq * 4, hipMemcpyDeviceToHost));
    CHECK(oracle_paged_decode(q, k, v, lens, table, B, Hq, Hkv, D, page_size, num_pages, max_pages, scale, ref) == 0,
          "oracle");
    if (s == GQA_OK) compare(got, ref, nq, what);
    hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dl), hipFree(dt), hipFree(dout), hipFree(ws);
    free(q), free(k), free(v), free(table), free(got), free(ref);
}

/* The two kernels apart: gqa_decode_partials, then gqa_decode_combine on the same workspace. */
static void two_step_case(int B, int Hq, int Hkv, int D, int S_max, const int32_t *lens, float scale,
                          uint64_t seed) {
    const size_t nq = (size_t)B * Hq * D, nkv = (size_t)B * Hkv * S_max * D;
    uint16_t *q = malloc(nq * 2), *k = malloc(nkv * 2), *v = malloc(nkv * 2);
    float *got = malloc(nq * 4);
    double *ref = malloc(nq * 8);
    fill_bf16(q, nq, seed);
    fill_bf16(k, nkv, seed + 1);
    fill_bf16(v, nkv, seed + 2);
    void *dq = dev_copy(q, nq * 2), *dk = dev_copy(k, nkv * 2), *dv = dev_copy(v, nkv * 2);
    void *dl = dev_copy(lens, (size_t)B * 4);
    float *dout = NULL;
    HIP_OK(hipMalloc((void **)&dout, nq * 4));
    const size_t ws_bytes = gqa_decode_workspace_bytes(B, Hq, Hkv, D, S_max, 0, 0);
    void *ws = zeroed_workspace(ws_bytes);
    gqa_status_t s = gqa_decode_partials(dq, dk, dv, dl, B, Hq, Hkv, D, S_max, scale, dout, ws, ws_bytes, 0, NULL);
    CHECK(s == GQA_OK, "gqa_decode_partials returned %s", gqa_status_string(s));
    if (s == GQA_OK) {
        s = gqa_decode_combine(ws, ws_bytes, dl, B, Hq, Hkv, D, S_max, 0, 0, dout, NULL);
        CHECK(s == GQA_OK, "gqa_decode_combine returned %s", gqa_status_string(s));
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got, dout, nq * 4, hipMemcpyDeviceToHost));
    CHECK(oracle_decode(q, k, v, lens, B, Hq, Hkv, D, S_max, scale, ref) == 0, "oracle");
    char what[96];
    snprintf(what, sizeof what, "partials + combine B=%d Hq=%d Hkv=%d D=%d", B, Hq, Hkv, D);
    if (s == GQA_OK) compare(got, ref, nq, what);
    hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dl), hipFree(dout), hipFree(ws);
    free(q), free(k), free(v), free(got), free(ref);
}

/* An E4M3 cache with per-tensor scales; the workspace from the E4M3 plan on this device. */
static void fp8_case(int B, int Hq, int Hkv, int D, int S_max, const int32_t *lens, float scale, float k_scale,
                     float v_scale, uint64_t seed) {
    const size_t nq = (size_t)B * Hq * D, nkv = (size_t)B * Hkv * S_max * D;
    uint16_t *q = malloc(nq * 2);
    uint8_t *k = malloc(nkv), *v = malloc(nkv);
    float *got = malloc(nq * 4);
    double *ref = malloc(nq * 8);
    fill_bf16(q, nq, seed);
    fill_e4m3(k, nkv, seed + 1);
    fill_e4m3(v, nkv, seed + 2);
    void *dq = dev_copy(q, nq * 2), *dk = dev_copy(k, nkv), *dv = dev_copy(v, nkv);
    void *dl = dev_copy(lens, (size_t)B * 4);
    float *dout = NULL;
    HIP_OK(hipMalloc((void **)&dout, nq * 4));
    int dev = 0, cus = 0;
    HIP_OK(hipGetDevice(&dev));
    HIP_OK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    gqa_plan_t plan;
    CHECK(gqa_decode_plan_fp8(B, Hq, Hkv, D, S_max, 0, 0, cus, &plan) == GQA_OK, "E4M3 plan");
    void *ws = zeroed_workspace(plan.workspace_bytes);
    const gqa_status_t s = gqa_decode_fp8(dq, dk, dv, dl, B, Hq, Hkv, D, S_max, scale, k_scale, v_scale, dout, ws,
                                          plan.workspace_bytes, 0, NULL);
    char what[96];
    snprintf(what, sizeof what, "gqa_decode_fp8 B=%d Hq=%d Hkv=%d D=%d", B, Hq, Hkv, D);
    CHECK(s == GQA_OK, "%s returned %s", what, gqa_status_string(s));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got, dout, nq * 4, hipMemcpyDeviceToHost));
    CHECK(oracle_decode_fp8(q, k, v, lens, B, Hq, Hkv, D, S_max, scale, k_scale, v_scale, 0, ref) == 0, "oracle");
    if (s == GQA_OK) compare(got, ref, nq, what);
    hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dl), hipFree(dout), hipFree(ws);
    free(q), free(k), free(v), free(got), free(ref);
}

/* M query tokens per sequence (the last M positions, causal); q and out [B][M][Hq][D]. */
static void mq_case(int B, int M, int Hq, int Hkv, int D, int S_max, const int32_t *lens, float scale,
                    uint64_t seed) {
    const size_t nq = (size_t)B * M * Hq * D, nkv = (size_t)B * Hkv * S_max * D;
    uint16_t *q = malloc(nq * 2), *k = malloc(nkv * 2), *v = malloc(nkv * 2);
    float *got = malloc(nq * 4);
    double *ref = malloc(nq * 8);
    fill_bf16(q, nq, seed);
    fill_bf16(k, nkv, seed + 1);
    fill_bf16(v, nkv, seed + 2);
    void *dq = dev_copy(q, nq * 2), *dk = dev_copy(k, nkv * 2), *dv = dev_copy(v, nkv * 2);
    void *dl = dev_copy(lens, (size_t)B * 4);
    float *dout = NULL;
    HIP_OK(hipMalloc((void **)&dout, nq * 4));
    const size_t ws_bytes = gqa_decode_workspace_bytes(B, M * Hq, Hkv, D, S_max, 0, 0);
    void *ws = zeroed_workspace(ws_bytes);
    const gqa_status_t s = gqa_decode_mq(dq, dk, dv, dl, B, M, Hq, Hkv, D, S_max, scale, dout, ws, ws_bytes, 0, NULL);
    char what[96];
    snprintf(what, sizeof what, "gqa_decode_mq B=%d M=%d Hq=%d Hkv=%d D=%d", B, M, Hq, Hkv, D);
    CHECK(s == GQA_OK, "%s returned %s", what, gqa_status_string(s));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(got, dout, nq * 4, hipMemcpyDeviceToHost));
    CHECK(oracle_decode_mq(q, k, v, lens, B, M, Hq, Hkv, D, S_max, scale, 0, ref) == 0, "oracle");
    if (s == GQA_OK) compare(got, ref, nq, what);
    hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dl), hipFree(dout), hipFree(ws);
    free(q), free(k), free(v), free(got), free(ref);
}

static void gpu_checks(void) {
    int n = 0;
    HIP_OK(hipGetDeviceCount(&n));
    CHECK(n > 0, "no GPU");
    if (n == 0) return;
    const int32_t l1[3] = {700, 0, 1};
    contiguous_case(3, 16, 4, 128, 700, l1, 0.08838834764831845f, 11, 0);        /* even shares / small job */
    const int32_t l2[1] = {4096};
    contiguous_case(1, 24, 4, 256, 4096, l2, 0.0625f, 12, 0);                   /* the GQA-6 layer */
    const int32_t l3[2] = {512, 77};
    contiguous_case(2, 8, 2, 64, 512, l3, 0.125f, 13, 0);
    contiguous_case(1, 24, 4, 256, 4096, l2, 0.0625f, 14, 1);                   /* no-alloc entry point */
    contiguous_case(3, 16, 4, 128, 700, l1, 0.08838834764831845f, 15, 1);
    const int32_t l4[4] = {1000, 33, 0, 512};
    paged_case(4, 32, 8, 128, 32, 32, l4, 0.08838834764831845f, 16);
    paged_case(4, 8, 2, 64, 16, 64, l4, 0.125f, 17);
    const int32_t l5[5] = {3000, 1, 0, 2048, 777};
    two_step_case(5, 32, 8, 128, 3000, l5, 0.08838834764831845f, 18);         /* even shares */
    two_step_case(1, 24, 4, 256, 4096, l2, 0.0625f, 19);                       /* fixed splits */
    fp8_case(3, 16, 4, 128, 700, l1, 0.08838834764831845f, 1.0f / 16, 1.0f / 16, 20);
    fp8_case(1, 24, 4, 256, 4096, l2, 0.0625f, 1.0f / 32, 1.0f / 8, 21);
    const int32_t l6[3] = {900, 2, 64};                                         /* len 2 < M: row 0 is zero */
    mq_case(3, 3, 16, 4, 128, 900, l6, 0.08838834764831845f, 22);             /* M * G = 12 query rows */
    printf("gpu checks: %s\n", failures == 0 ? "ok" : "FAILED");
}

int main(int argc, char **argv) {
    const char *mode = argc > 1 ? argv[1] : "host";
    if (strcmp(mode, "host") == 0) {
        host_checks();
    } else if (strcmp(mode, "gpu") == 0) {
        host_checks();
        gpu_checks();
    } else {
        fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
        return 2;
    }
    return failures == 0 ? 0 : 1;
}
