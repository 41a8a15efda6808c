/*
 * A plain C caller of libqknorm.so, with no Python in the process: device memory from the HIP
 * runtime's C API, the fused QK-Norm and the fold + deferred projection called through
 * include/qknorm.h, every output checked against the fp64 oracle (liboracle.so, test
 * infrastructure), and the error path of a bad call. Exit status 0 when everything holds.
 *
 * Operations: layerwise QK-Norm ("SwiftQK: Fast and Communication-Efficient Tensor Parallelism
 * for Query-Key Normalization", abstract) and the deferred norm-then-project ("FlashNorm: Fast
 * Normalization for Transformers", abstract, items (i) and (ii)).
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qknorm.h"

/* the oracle's entry points (oracle/oracle.c); 1 = bf16 storage */
void oracle_rmsnorm_rows(int64_t T, int64_t d, double eps, int xdt, const void* x, int64_t ldx,
                         int gdt, const void* gamma, double* y, int64_t ldy);
void oracle_fold_weight(int64_t K, int64_t N, int wdt, const void* w, int64_t ldw, int gdt,
                        const void* gamma, double* wf, int64_t ldwf);
void oracle_round_bf16_array(int64_t n, const double* src, uint16_t* dst);
void oracle_normproj(int64_t T, int64_t K, int64_t N, double eps, int xdt, const void* x,
                     int64_t ldx, int wdt, const void* wf, int64_t ldw, double* y, int64_t ldy);

static uint64_t rng_state = 0x243F6A8885A308D3ull;

/* splitmix64, then a Box-Muller normal draw */
static double uniform01(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return ((double)(z >> 11) + 0.5) / 9007199254740992.0;
}

static double normal(double mu, double sd)
{
    return mu + sd * sqrt(-2.0 * log(uniform01())) * cos(6.283185307179586 * uniform01());
}

static uint16_t to_bf16(double v)
{
    uint16_t b;
    oracle_round_bf16_array(1, &v, &b);
    return b;
}

static double from_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint16_t* random_bf16(int64_t n, double mu, double sd)
{
    uint16_t* a = malloc((size_t)n * sizeof *a);
    for (int64_t i = 0; i < n; ++i) a[i] = to_bf16(normal(mu, sd));
    return a;
}

static int failures = 0;

#define HIP_OK(call)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess) {                                                               \
            fprintf(stderr, "%s failed: %d\n", #call, (int)e_);                               \
            exit(2);                                                                          \
        }                                                                                     \
    } while (0)

static void* to_device(const void* host, size_t bytes)
{
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

/* bf16 outputs of the row operation: within 8e-3 relative and 2 bf16 ulp of the fp64 value */
static void check_rows(const char* what, const uint16_t* got, const double* ref, int64_t n)
{
    int64_t bad = 0;
    for (int64_t i = 0; i < n; ++i) {
        double g = from_bf16(got[i]), r = ref[i], err = fabs(g - r);
        int ex;
        frexp(r, &ex);
        double ulp = r != 0.0 ? ldexp(1.0, ex - 8) : 0.0;
        double tol = fmin(8e-3 * fabs(r), 2.0 * ulp);
        if (err > tol) ++bad;
    }
    printf("%s: %lld of %lld outside the tolerance\n", what, (long long)bad, (long long)n);
    failures += bad != 0;
}

/* projection outputs: |got - ref| <= 8e-3 |ref| + 2^-13 r_t sum_k |x W'| */
static void check_projection(const char* what, const uint16_t* got, const double* ref,
                             const uint16_t* x, const uint16_t* wf, int64_t T, int64_t K,
                             int64_t N, double eps)
{
    int64_t bad = 0;
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += from_bf16(x[t * K + k]) * from_bf16(x[t * K + k]);
        double r = 1.0 / sqrt(s / (double)K + eps);
        for (int64_t n = 0; n < N; ++n) {
            double a = 0.0;
            for (int64_t k = 0; k < K; ++k)
                a += fabs(from_bf16(x[t * K + k]) * from_bf16(wf[k * N + n]));
            double g = from_bf16(got[t * N + n]), e = ref[t * N + n];
            if (fabs(g - e) > 8e-3 * fabs(e) + ldexp(r * a, -13)) ++bad;
        }
    }
    printf("%s: %lld of %lld outside the tolerance\n", what, (long long)bad, (long long)(T * N));
    failures += bad != 0;
}

static void fused_case(int64_t T, int64_t dq, int64_t dk)
{
    const double eps = 1e-6;
    uint16_t *q = random_bf16(T * dq, 0.0, 2.0), *k = random_bf16(T * dk, 0.0, 2.0);
    uint16_t *gq = random_bf16(dq, 1.0, 0.05), *gk = random_bf16(dk, 1.0, 0.05);
    void *dq_in = to_device(q, (size_t)(T * dq * 2)), *dk_in = to_device(k, (size_t)(T * dk * 2));
    void *dgq = to_device(gq, (size_t)dq * 2), *dgk = to_device(gk, (size_t)dk * 2);
    void *dq_out = NULL, *dk_out = NULL;
    HIP_OK(hipMalloc(&dq_out, (size_t)(T * dq * 2)));
    HIP_OK(hipMalloc(&dk_out, (size_t)(T * dk * 2)));
    int st = qknorm_fused(T, (float)eps, QKN_BF16, QKN_BF16, dq_in, dq, dq_out, dq, dgq, dq, dk_in,
                          dk, dk_out, dk, dgk, dk, NULL);
    if (st != QKN_OK) {
        printf("qknorm_fused: %s\n", qkn_status_string(st));
        ++failures;
        return;
    }
    HIP_OK(hipDeviceSynchronize());
    uint16_t *yq = malloc((size_t)(T * dq * 2)), *yk = malloc((size_t)(T * dk * 2));
    HIP_OK(hipMemcpy(yq, dq_out, (size_t)(T * dq * 2), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(yk, dk_out, (size_t)(T * dk * 2), hipMemcpyDeviceToHost));
    double *rq = malloc((size_t)(T * dq) * sizeof(double)), *rk = malloc((size_t)(T * dk) * sizeof(double));
    oracle_rmsnorm_rows(T, dq, eps, 1, q, dq, 1, gq, rq, dq);
    oracle_rmsnorm_rows(T, dk, eps, 1, k, dk, 1, gk, rk, dk);
    char what[96];
    snprintf(what, sizeof what, "qknorm_fused Q [%lld, %lld]", (long long)T, (long long)dq);
    check_rows(what, yq, rq, T * dq);
    snprintf(what, sizeof what, "qknorm_fused K [%lld, %lld]", (long long)T, (long long)dk);
    check_rows(what, yk, rk, T * dk);
    HIP_OK(hipFree(dq_in)); HIP_OK(hipFree(dk_in)); HIP_OK(hipFree(dgq)); HIP_OK(hipFree(dgk));
    HIP_OK(hipFree(dq_out)); HIP_OK(hipFree(dk_out));
    free(q); free(k); free(gq); free(gk); free(yq); free(yk); free(rq); free(rk);
}

static void projection_case(int64_t T, int64_t K, int64_t N)
{
    const double eps = 1e-6;
    uint16_t *x = random_bf16(T * K, 0.0, 1.0), *w = random_bf16(K * N, 0.0, 0.02);
    uint16_t* g = random_bf16(K, 1.0, 0.05);
    void *dx = to_device(x, (size_t)(T * K * 2)), *dw = to_device(w, (size_t)(K * N * 2));
    void* dg = to_device(g, (size_t)K * 2);
    void *dwf = NULL, *dy = NULL;
    HIP_OK(hipMalloc(&dwf, (size_t)(K * N * 2)));
    HIP_OK(hipMalloc(&dy, (size_t)(T * N * 2)));
    int st = normproj_fold_weight(K, N, QKN_BF16, QKN_BF16, dw, N, dg, dwf, N, NULL);
    if (st == QKN_OK)
        st = normproj_deferred(T, K, N, (float)eps, QKN_BF16, dx, K, dwf, N, dy, N, NULL);
    if (st != QKN_OK) {
        printf("fold / deferred: %s\n", qkn_status_string(st));
        ++failures;
        return;
    }
    HIP_OK(hipDeviceSynchronize());
    uint16_t *wf = malloc((size_t)(K * N * 2)), *y = malloc((size_t)(T * N * 2));
    HIP_OK(hipMemcpy(wf, dwf, (size_t)(K * N * 2), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(y, dy, (size_t)(T * N * 2), hipMemcpyDeviceToHost));
    /* the fold: bit-exact against the fp64 product rounded once to bf16 */
    double* wf_ref = malloc((size_t)(K * N) * sizeof(double));
    uint16_t* wf_bits = malloc((size_t)(K * N * 2));
    oracle_fold_weight(K, N, 1, w, N, 1, g, wf_ref, N);
    oracle_round_bf16_array(K * N, wf_ref, wf_bits);
    int fold_ok = memcmp(wf, wf_bits, (size_t)(K * N * 2)) == 0;
    printf("normproj_fold_weight [%lld, %lld]: %s\n", (long long)K, (long long)N,
           fold_ok ? "bit-exact" : "MISMATCH");
    failures += !fold_ok;
    double* ref = malloc((size_t)(T * N) * sizeof(double));
    oracle_normproj(T, K, N, eps, 1, x, K, 1, wf_bits, N, ref, N);
    char what[96];
    snprintf(what, sizeof what, "normproj_deferred T=%lld K=%lld N=%lld", (long long)T,
             (long long)K, (long long)N);
    check_projection(what, y, ref, x, wf_bits, T, K, N, eps);
    HIP_OK(hipFree(dx)); HIP_OK(hipFree(dw)); HIP_OK(hipFree(dg)); HIP_OK(hipFree(dwf));
    HIP_OK(hipFree(dy));
    free(x); free(w); free(g); free(wf); free(y); free(wf_ref); free(wf_bits); free(ref);
}

int main(void)
{
    int dev_count = 0;
    HIP_OK(hipGetDeviceCount(&dev_count));
    if (dev_count < 1) {
        fprintf(stderr, "no GPU\n");
        return 2;
    }
    fused_case(64, 4096, 512);   /* team shapes 3 and 0 */
    fused_case(37, 520, 4100);   /* masked shape, generic path past 2048 vectors */
    projection_case(8, 256, 512);     /* matrix-vector form */
    projection_case(300, 512, 264);   /* tiled matrix-core form, ragged */

    /* a bad call returns its status before touching the device */
    int st = qknorm_fused(4, 1e-6f, QKN_BF16, QKN_BF16, NULL, 64, NULL, 64, NULL, 64, NULL, 0,
                          NULL, 0, NULL, 0, NULL);
    printf("null pointers: %s\n", qkn_status_string(st));
    failures += st != QKN_ERR_NULL;

    printf(failures ? "c abi check FAILED\n" : "c abi check ok\n");
    return failures ? 1 : 0;
}
