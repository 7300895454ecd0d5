/*
 * bt_c_client.c -- drives libbt.so through its C ABI from plain C (the HIP runtime only
 * for device memory, copies and a stream; no Python, no torch) and checks every result
 * against the C oracle (oracle/bt_oracle.c, linked in). Test infrastructure: built by
 * tests/c_abi/__init__.py, run by tests/test_c_client.py.
 *
 * For each case (M tokens, N output rows, K inputs) it packs seeded weights
 * W ~ N(0, 0.02), quantizes seeded activations X ~ N(0, 1), and runs every product entry
 * point that takes the case: bt_ternary_gemm (and bt_ternary_gemm_ws where the plan splits
 * K), bt_ternary_gemv_algo with each kernel choice that accepts M and K, bt_ternary_linear
 * and bt_ternary_linear_static. The bar is the library's contract: gamma, the codes, q,
 * s_x, sum q and acc bit-exact; Y within |dY| <= 1e-5 |Y| + 1e-6 of the oracle's.
 *
 * Exit status: 0 every check passed; 1 a result differs from the oracle; 2 an entry point
 * returned an unexpected status or the HIP runtime failed; 77 no GPU (nothing was run).
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bt.h"

int oracle_absmean(const float *W, int64_t N, int64_t K, float *gamma_out);
int oracle_ternarize(const float *W, int64_t N, int64_t K, float gamma, int8_t *T);
int oracle_quant_act(const float *X, int64_t M, int64_t K, int8_t *Q, float *s_x, int32_t *qsum);
int oracle_ternary_matmul(const int8_t *T, const int8_t *Q, int64_t M, int64_t N, int64_t K, int32_t *acc);
int oracle_scale_epilogue(const int32_t *acc, float gamma, const float *s_x, int64_t M, int64_t N, float *Y);

static int failures = 0;

#define HIP_CHECK(call)                                                                      \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess) {                                                              \
            fprintf(stderr, "HIP error %d (%s) at %s:%d\n", (int)e_, hipGetErrorString(e_), \
                    __FILE__, __LINE__);                                                     \
            exit(2);                                                                         \
        }                                                                                    \
    } while (0)

static void expect_status(bt_status got, bt_status want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d (%s), expected %d; last error: %s\n", what, (int)got, bt_status_str(got),
                (int)want, bt_last_error());
        exit(2);
    }
}

/* splitmix64 and Box-Muller: a seeded normal generator of the test's own. */
static uint64_t rng_state;

static uint64_t splitmix64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform01(void) { return ((splitmix64() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

static float *normal_array(int64_t n, double sigma, uint64_t seed)
{
    float *a = malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!a)
        exit(2);
    rng_state = seed;
    for (int64_t i = 0; i < n; i += 2) {
        const double r = sqrt(-2.0 * log(uniform01())), t = 6.283185307179586 * uniform01();
        a[i] = (float)(sigma * r * cos(t));
        if (i + 1 < n)
            a[i + 1] = (float)(sigma * r * sin(t));
    }
    return a;
}

static void *dev_alloc(size_t bytes)
{
    void *p = NULL;
    HIP_CHECK(hipMalloc(&p, bytes ? bytes : 256));
    return p;
}

static void *host_alloc(size_t bytes)
{
    void *p = calloc(bytes ? bytes : 1, 1);
    if (!p)
        exit(2);
    return p;
}

static void check(int ok, const char *what, int64_t M, int64_t N, int64_t K)
{
    if (!ok) {
        fprintf(stderr, "MISMATCH %s at M=%lld N=%lld K=%lld\n", what, (long long)M, (long long)N, (long long)K);
        ++failures;
    }
}

/* acc bit-exact and Y within the contract's tolerance, on the first M rows. */
static void check_product(const char *what, hipStream_t s, const float *dY, const int32_t *dacc, const float *Yref,
                          const int32_t *accref, int64_t M, int64_t N, int64_t K)
{
    const size_t mn = (size_t)(M * N);
    float *Y = host_alloc(mn * sizeof(float));
    int32_t *acc = host_alloc(mn * sizeof(int32_t));
    HIP_CHECK(hipStreamSynchronize(s));
    HIP_CHECK(hipMemcpy(Y, dY, mn * sizeof(float), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(acc, dacc, mn * sizeof(int32_t), hipMemcpyDeviceToHost));
    char label[160];
    snprintf(label, sizeof label, "%s acc", what);
    check(memcmp(acc, accref, mn * sizeof(int32_t)) == 0, label, M, N, K);
    int yok = 1;
    for (size_t i = 0; i < mn; ++i) {
        const double d = fabs((double)Y[i] - (double)Yref[i]);
        if (!(d <= 1e-5 * fabs((double)Yref[i]) + 1e-6))
            yok = 0;
    }
    snprintf(label, sizeof label, "%s Y", what);
    check(yok, label, M, N, K);
    free(Y);
    free(acc);
}

static void run_case(hipStream_t s, int64_t M, int64_t N, int64_t K, uint64_t seed)
{
    const int64_t rb = bt_act_row_bytes(K);
    float *W = normal_array(N * K, 0.02, seed);
    float *X = normal_array(M * K, 1.0, seed ^ 0x5DEECE66Dull);

    /* the oracle's results */
    float gamma_ref = 0.0f;
    int8_t *Tref = host_alloc((size_t)(N * K));
    int8_t *Qref = host_alloc((size_t)(M * K));
    float *sref = host_alloc((size_t)M * sizeof(float));
    int32_t *qsref = host_alloc((size_t)M * sizeof(int32_t));
    int32_t *accref = host_alloc((size_t)(M * N) * sizeof(int32_t));
    float *Yref = host_alloc((size_t)(M * N) * sizeof(float));
    if (oracle_absmean(W, N, K, &gamma_ref) || oracle_ternarize(W, N, K, gamma_ref, Tref) ||
        oracle_quant_act(X, M, K, Qref, sref, qsref) || oracle_ternary_matmul(Tref, Qref, M, N, K, accref) ||
        oracle_scale_epilogue(accref, gamma_ref, sref, M, N, Yref)) {
        fprintf(stderr, "oracle rejected M=%lld N=%lld K=%lld\n", (long long)M, (long long)N, (long long)K);
        exit(2);
    }

    /* device buffers, owned here */
    float *dW = dev_alloc((size_t)(N * K) * sizeof(float));
    float *dX = dev_alloc((size_t)(M * K) * sizeof(float));
    void *dWp = dev_alloc(bt_packed_weight_bytes(N, K));
    float *dscale = dev_alloc(sizeof(float));
    void *dpws = dev_alloc(bt_pack_workspace_bytes(N, K));
    int8_t *dT = dev_alloc((size_t)(N * K));
    int8_t *dXq = dev_alloc((size_t)(M * rb));
    float *dsx = dev_alloc((size_t)M * sizeof(float));
    int32_t *dxs = dev_alloc((size_t)M * sizeof(int32_t));
    float *dY = dev_alloc((size_t)(M * N) * sizeof(float));
    int32_t *dacc = dev_alloc((size_t)(M * N) * sizeof(int32_t));
    HIP_CHECK(hipMemcpy(dW, W, (size_t)(N * K) * sizeof(float), hipMemcpyHostToDevice));
    HIP_CHECK(hipMemcpy(dX, X, (size_t)(M * K) * sizeof(float), hipMemcpyHostToDevice));

    /* weights: gamma and every code */
    expect_status(bt_pack_weights(dW, N, K, dWp, dscale, dpws, s), BT_OK, "bt_pack_weights");
    expect_status(bt_unpack_weights(dWp, N, K, dT, s), BT_OK, "bt_unpack_weights");
    HIP_CHECK(hipStreamSynchronize(s));
    float gamma = 0.0f;
    int8_t *T = host_alloc((size_t)(N * K));
    HIP_CHECK(hipMemcpy(&gamma, dscale, sizeof(float), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(T, dT, (size_t)(N * K), hipMemcpyDeviceToHost));
    check(memcmp(&gamma, &gamma_ref, sizeof(float)) == 0, "gamma", M, N, K);
    check(memcmp(T, Tref, (size_t)(N * K)) == 0, "codes", M, N, K);

    /* activations: q (and zero padding), s_x, sum q */
    expect_status(bt_quant_act(dX, M, K, dXq, dsx, dxs, s), BT_OK, "bt_quant_act");
    HIP_CHECK(hipStreamSynchronize(s));
    int8_t *Xq = host_alloc((size_t)(M * rb));
    float *sx = host_alloc((size_t)M * sizeof(float));
    int32_t *xs = host_alloc((size_t)M * sizeof(int32_t));
    HIP_CHECK(hipMemcpy(Xq, dXq, (size_t)(M * rb), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(sx, dsx, (size_t)M * sizeof(float), hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(xs, dxs, (size_t)M * sizeof(int32_t), hipMemcpyDeviceToHost));
    int qok = 1;
    for (int64_t m = 0; m < M; ++m) {
        if (memcmp(Xq + m * rb, Qref + m * K, (size_t)K) != 0)
            qok = 0;
        for (int64_t k = K; k < rb; ++k)
            if (Xq[m * rb + k] != 0)
                qok = 0;
    }
    check(qok, "q", M, N, K);
    check(memcmp(sx, sref, (size_t)M * sizeof(float)) == 0, "s_x", M, N, K);
    check(memcmp(xs, qsref, (size_t)M * sizeof(int32_t)) == 0, "sum q", M, N, K);

    /* the prefill product, and its split-K form where the plan splits */
    expect_status(bt_ternary_gemm(dWp, dscale, dXq, dsx, dxs, M, N, K, dY, dacc, s), BT_OK, "bt_ternary_gemm");
    check_product("bt_ternary_gemm", s, dY, dacc, Yref, accref, M, N, K);
    const size_t gws = bt_gemm_workspace_bytes(M, N, K);
    if (gws > 0) {
        void *dgws = dev_alloc(gws);
        HIP_CHECK(hipMemsetAsync(dgws, 0, gws, s)); /* the split-K counters start at zero */
        for (int rep = 0; rep < 2; ++rep) {         /* the second call reuses the reset counters */
            expect_status(bt_ternary_gemm_ws(dWp, dscale, dXq, dsx, dxs, M, N, K, dY, dacc, dgws, gws, s), BT_OK,
                          "bt_ternary_gemm_ws");
            check_product("bt_ternary_gemm_ws", s, dY, dacc, Yref, accref, M, N, K);
        }
        HIP_CHECK(hipFree(dgws));
    }

    /* the decode product: every kernel choice that accepts the case */
    if (M <= BT_GEMV_MAX_M) {
        static const struct {
            int32_t algo;
            const char *name;
        } algos[] = {{BT_GEMV_AUTO, "gemv auto"}, {BT_GEMV_MFMA, "gemv mfma"}, {BT_GEMV_STAGED, "gemv staged"},
                     {BT_GEMV_DOT4, "gemv dot4"}, {BT_GEMV_LUT, "gemv lut"}};
        for (size_t a = 0; a < sizeof algos / sizeof algos[0]; ++a) {
            const bt_status st =
                bt_ternary_gemv_algo(dWp, dscale, dXq, dsx, dxs, M, N, K, dY, dacc, algos[a].algo, s);
            if (st == BT_ERR_UNSUPPORTED && algos[a].algo != BT_GEMV_AUTO && algos[a].algo != BT_GEMV_MFMA)
                continue; /* a kernel that does not take this M or K says so */
            expect_status(st, BT_OK, algos[a].name);
            check_product(algos[a].name, s, dY, dacc, Yref, accref, M, N, K);
        }
    }

    /* the whole layer from fp32 activations: with a workspace, and with the static scratch */
    const size_t lws = bt_linear_workspace_bytes(M, N, K);
    void *dlws = lws ? dev_alloc(lws) : NULL;
    expect_status(bt_ternary_linear(dWp, dscale, dX, M, N, K, dY, dacc, dlws, s), BT_OK, "bt_ternary_linear");
    check_product("bt_ternary_linear", s, dY, dacc, Yref, accref, M, N, K);
    if (lws <= (size_t)BT_STATIC_SCRATCH_BYTES) {
        expect_status(bt_ternary_linear_static(dWp, dscale, dX, M, N, K, dY, dacc, s), BT_OK,
                      "bt_ternary_linear_static");
        check_product("bt_ternary_linear_static", s, dY, dacc, Yref, accref, M, N, K);
    }
    printf("case M=%lld N=%lld K=%lld: %s\n", (long long)M, (long long)N, (long long)K,
           lws ? "quantizer + product route" : "fused route");
    fflush(stdout);

    if (dlws)
        HIP_CHECK(hipFree(dlws));
    void *dev[] = {dW, dX, dWp, dscale, dpws, dT, dXq, dsx, dxs, dY, dacc};
    for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i)
        HIP_CHECK(hipFree(dev[i]));
    void *host[] = {W, X, Tref, Qref, sref, qsref, accref, Yref, T, Xq, sx, xs};
    for (size_t i = 0; i < sizeof host / sizeof host[0]; ++i)
        free(host[i]);
}

/* Argument errors are reported before anything is enqueued, with a message. */
static void run_errors(hipStream_t s)
{
    void *d = dev_alloc(1 << 16);
    expect_status(bt_ternary_gemm(NULL, (const float *)d, (const int8_t *)d, (const float *)d, (const int32_t *)d,
                                  4, 64, 64, (float *)d, NULL, s),
                  BT_ERR_NULL, "bt_ternary_gemm with a NULL weight pointer");
    check(strlen(bt_last_error()) > 0, "bt_last_error after BT_ERR_NULL", 4, 64, 64);
    expect_status(bt_quant_act((const float *)d, 1, (int64_t)BT_MAX_K + 1, (int8_t *)d, (float *)d, (int32_t *)d, s),
                  BT_ERR_SHAPE, "bt_quant_act with K above BT_MAX_K");
    expect_status(bt_ternary_gemv(d, (const float *)d, (const int8_t *)d, (const float *)d, (const int32_t *)d,
                                  BT_GEMV_MAX_M + 1, 64, 64, (float *)d, NULL, s),
                  BT_ERR_UNSUPPORTED, "bt_ternary_gemv above its token limit");
    /* M == 0 is a no-op that succeeds */
    expect_status(bt_ternary_linear(d, (const float *)d, (const float *)d, 0, 64, 64, (float *)d, NULL, NULL, s),
                  BT_OK, "bt_ternary_linear with M = 0");
    HIP_CHECK(hipStreamSynchronize(s));
    HIP_CHECK(hipFree(d));
    printf("argument errors: ok\n");
}

int main(void)
{
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        printf("no GPU: nothing run\n");
        return 77;
    }
    HIP_CHECK(hipSetDevice(0));
    hipStream_t s;
    HIP_CHECK(hipStreamCreate(&s));
    static const int64_t cases[][3] = {
        {128, 512, 256},   /* the tiny matmul: X [128,256], W [512,256] */
        {1, 3840, 2560},   /* 2B-class QKV at one token (fused route) */
        {4, 2560, 6912},   /* 2B-class down at four tokens (fused route) */
        {16, 2560, 2560},  /* sixteen tokens (quantizer + staged GEMV) */
        {5, 200, 301},     /* ragged rows and columns, K % 4 != 0 */
        {256, 2560, 2560}, /* prefill, few tiles (the small-M form, one workgroup per CU) */
        {300, 3500, 2600}, /* prefill, the small-M form at two workgroups per CU */
        {700, 3000, 4000}, /* prefill with K split over workgroups */
    };
    for (size_t c = 0; c < sizeof cases / sizeof cases[0]; ++c)
        run_case(s, cases[c][0], cases[c][1], cases[c][2], 1000 + c);
    run_errors(s);
    HIP_CHECK(hipStreamDestroy(s));
    if (failures) {
        printf("%d mismatches against the oracle\n", failures);
        return 1;
    }
    printf("all checks passed\n");
    return 0;
}
