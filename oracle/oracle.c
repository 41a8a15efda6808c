/*
 * Plain, slow fp64 CPU oracle for layerwise QK-Norm, its scalar-statistics split, the
 * folded / deferred norm-then-project, the pre-attention RMSNorm elimination ahead of QK-Norm,
 * and the folded / deferred LayerNorm-then-project.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg load this library. The GPU library never links, includes or calls it, and the two share
 * no source, header, table or helper.
 *
 * Definition (RMSNorm with a per-column weight gamma and epsilon inside the root):
 *
 *     r      = 1 / sqrt( (1/d) * sum_j x[j]^2 + eps )
 *     y[i]   = x[i] * gamma[i] * r
 *
 * "Layerwise" QK-Norm applies it to each token's full heads*head_dim Q and K projection
 * vectors, because the normalisation factor depends on the whole vector ("SwiftQK: Fast and
 * Communication-Efficient Tensor Parallelism for Query-Key Normalization", abstract).
 *
 * Everything is evaluated in IEEE double precision with plain left-to-right loops; inputs are
 * widened exactly (bf16 bits << 16 -> float -> double). No fast-math, no blocking, no
 * reordering beyond what the definitions state.
 *
 * Parity pins: every function here is pinned by the CPU tests (hand-derived worked examples,
 * closed forms, invariants, brute force on tiny rows, decomposition equality, the fold and
 * elimination identities, and library special cases). None is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* storage codes understood by the oracle (its own; unrelated to any other library's) */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Exact widening of one stored element to double. */
static double oracle_elem(int dtype, const void* base, int64_t idx)
{
    if (dtype == ORACLE_F64) return ((const double*)base)[idx];
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    /* bf16: the 16 stored bits are the upper half of a float32 */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value (ties to even) and return its bits.
 * bf16 keeps 8 significant bits and float32's exponent range (normal min 2^-126, subnormal
 * spacing 2^-133). Values at or beyond max + half a spacing round to infinity. */
uint16_t oracle_bf16_rne(double v)
{
    float f;
    uint32_t bits;
    if (isnan(v)) return 0x7FC0;
    if (isinf(v)) return v > 0 ? 0x7F80 : 0xFF80;
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    int e = ilogb(a);                 /* a = m * 2^e, 1 <= m < 2 */
    if (e < -126) e = -126;           /* subnormal range: fixed spacing 2^-133 */
    double q = nearbyint(ldexp(a, 7 - e));   /* default rounding mode: nearest, ties even */
    double r = ldexp(q, e - 7);
    /* largest finite bf16 is (2 - 2^-7) * 2^127 */
    if (r > ldexp(255.0, 120)) return v > 0 ? 0x7F80 : 0xFF80;
    f = (float)(v > 0 ? r : -r);      /* exactly representable */
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(bits >> 16);
}

void oracle_round_bf16_array(int64_t n, const double* src, uint16_t* dst)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_bf16_rne(src[i]);
}

/* Sum of squares of one row, left to right. */
static double row_sumsq(int dtype, const void* x, int64_t off, int64_t d)
{
    double s = 0.0;
    for (int64_t i = 0; i < d; ++i) {
        double v = oracle_elem(dtype, x, off + i);
        s += v * v;
    }
    return s;
}

/*
 * RMSNorm of each of T rows of width d (the monolithic definition above).
 * gamma == NULL means gamma = 1. y is [T, d] doubles with row stride ldy.
 */
void oracle_rmsnorm_rows(int64_t T, int64_t d, double eps, int xdt, const void* x, int64_t ldx,
                         int gdt, const void* gamma, double* y, int64_t ldy)
{
    for (int64_t t = 0; t < T; ++t) {
        double s = row_sumsq(xdt, x, t * ldx, d);
        double r = 1.0 / sqrt(s / (double)d + eps);
        for (int64_t i = 0; i < d; ++i) {
            double g = gamma ? oracle_elem(gdt, gamma, i) : 1.0;
            y[t * ldy + i] = oracle_elem(xdt, x, t * ldx + i) * g * r;
        }
    }
}

/*
 * Partial statistic of one column slice: s[t] = sum over the slice's d_local columns of x^2.
 * This is the per-rank scalar that SwiftQK exchanges instead of the activation vector
 * ("SwiftQK: ...", abstract: scalar partial-sum aggregation).
 */
void oracle_partial_sumsq(int64_t T, int64_t d_local, int xdt, const void* x, int64_t ldx,
                          double* s)
{
    for (int64_t t = 0; t < T; ++t) s[t] = row_sumsq(xdt, x, t * ldx, d_local);
}

/*
 * Scale one column slice with aggregated statistics (same abstract: aggregate the scalars,
 * then the element-wise scale). For row t:
 *     S = s_own[t] + sum_{e=0}^{n_ext-1} s_ext[e * ld_ext + t]
 *     r = 1 / sqrt(S / d_full + eps)          (mean over the FULL vector width)
 *     y = x * gamma * r                       over the d_local columns of the slice
 * s_own and s_ext are read with their own storage codes (f32 or f64).
 */
void oracle_apply_with_stats(int64_t T, int64_t d_local, int64_t d_full, double eps,
                             int xdt, const void* x, int64_t ldx, int gdt, const void* gamma,
                             int sdt, const void* s_own, int64_t n_ext, int edt,
                             const void* s_ext, int64_t ld_ext, double* y, int64_t ldy)
{
    for (int64_t t = 0; t < T; ++t) {
        double S = oracle_elem(sdt, s_own, t);
        for (int64_t e = 0; e < n_ext; ++e) S += oracle_elem(edt, s_ext, e * ld_ext + t);
        double r = 1.0 / sqrt(S / (double)d_full + eps);
        for (int64_t i = 0; i < d_local; ++i) {
            double g = gamma ? oracle_elem(gdt, gamma, i) : 1.0;
            y[t * ldy + i] = oracle_elem(xdt, x, t * ldx + i) * g * r;
        }
    }
}

/*
 * FlashNorm step (i): fold the norm weights into the next linear layer,
 *     W'[k][n] = gamma[k] * W[k][n]        (W' = diag(gamma) W, W is [K, N], y = x W)
 * ("FlashNorm: Fast Normalization for Transformers", abstract, item (i)).
 * wf is [K, N] doubles, row-major with row stride ldwf.
 */
void oracle_fold_weight(int64_t K, int64_t N, int wdt, const void* w, int64_t ldw,
                        int gdt, const void* gamma, double* wf, int64_t ldwf)
{
    for (int64_t k = 0; k < K; ++k) {
        double g = gamma ? oracle_elem(gdt, gamma, k) : 1.0;
        for (int64_t n = 0; n < N; ++n) wf[k * ldwf + n] = g * oracle_elem(wdt, w, k * ldw + n);
    }
}

/*
 * FlashNorm step (ii): deferred scaling. For row t of x [T, K] and the folded W' [K, N]:
 *     r      = 1 / sqrt( (1/K) sum_k x[t][k]^2 + eps )
 *     acc[n] = sum_k x[t][k] * W'[k][n]
 *     y[t][n] = acc[n] * r
 * (same abstract, item (ii): the scalar 1/RMS is applied to the product's output).
 */
void oracle_normproj(int64_t T, int64_t K, int64_t N, double eps, int xdt, const void* x,
                     int64_t ldx, int wdt, const void* wf, int64_t ldw, double* y, int64_t ldy)
{
    for (int64_t t = 0; t < T; ++t) {
        double s = row_sumsq(xdt, x, t * ldx, K);
        double r = 1.0 / sqrt(s / (double)K + eps);
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += oracle_elem(xdt, x, t * ldx + k) * oracle_elem(wdt, wf, k * ldw + n);
            y[t * ldy + n] = acc * r;
        }
    }
}

/*
 * The unfused order the fold replaces: RMSNorm first (with gamma), then the product with the
 * unfolded W [K, N]:   y[t][n] = sum_k (x[t][k] * gamma[k] * r_t) * W[k][n].
 */
void oracle_normproj_unfused(int64_t T, int64_t K, int64_t N, double eps, int xdt,
                             const void* x, int64_t ldx, int gdt, const void* gamma, int wdt,
                             const void* w, int64_t ldw, double* y, int64_t ldy)
{
    for (int64_t t = 0; t < T; ++t) {
        double s = row_sumsq(xdt, x, t * ldx, K);
        double r = 1.0 / sqrt(s / (double)K + eps);
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double g = gamma ? oracle_elem(gdt, gamma, k) : 1.0;
                double xn = oracle_elem(xdt, x, t * ldx + k) * g * r;
                acc += xn * oracle_elem(wdt, w, k * ldw + n);
            }
            y[t * ldy + n] = acc;
        }
    }
}

/* Plain product y = a @ b over fp64 (a [T, K] any storage, b [K, N] any storage). Used for
 * the unfused baseline whose intermediate is stored in bf16. */
void oracle_matmul(int64_t T, int64_t K, int64_t N, int adt, const void* a, int64_t lda,
                   int bdt, const void* b, int64_t ldb, double* y, int64_t ldy)
{
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += oracle_elem(adt, a, t * lda + k) * oracle_elem(bdt, b, k * ldb + n);
            y[t * ldy + n] = acc;
        }
}

/* ------------------------------------------------------------------------------------------
 * Eliminating the pre-attention RMSNorm by scale invariance ("FlashNorm: Fast Normalization
 * for Transformers", abstract: when a second RMSNorm follows the linear layer, the first one
 * changes nothing and can go, as ahead of attention with Q/K normalisation).
 *
 * The chain being simplified, for one token x [K]:
 *     h = x * gamma_pre * r1,  r1 = 1 / sqrt(mean(x^2) + eps_pre)     (pre-attention RMSNorm)
 *     q = h Wq,  k = h Wk                                               (Wq [K, nq], Wk [K, nk])
 *     yq = RMSNorm(q; gamma_q, eps_qk) over all nq columns, yk likewise over nk (layerwise)
 *
 * With W' = diag(gamma_pre) W and p = x W', q = r1 * p, so
 *     yq = p * gamma_q / sqrt(mean(p^2) + eps_qk / r1^2) = p * gamma_q / sqrt(mean(p^2) + eps_qk * (mean(x^2) + eps_pre)).
 * Dropping r1 and keeping eps_qk is therefore exact only when eps_qk = 0 (the second norm then
 * cancels any per-token scale); with exact = 1 the eliminated form uses the per-token
 * epsilon eps_qk * (mean(x^2) + eps_pre) and equals the chain for every epsilon.
 * ------------------------------------------------------------------------------------------ */

/* RMSNorm of one fp64 vector in place-free form: out[i] = v[i] * g[i] / sqrt(mean(v^2) + eps). */
static void rms_vec(int64_t d, const double* v, int gdt, const void* gamma, double eps,
                    double* out)
{
    double s = 0.0;
    for (int64_t i = 0; i < d; ++i) s += v[i] * v[i];
    double r = 1.0 / sqrt(s / (double)d + eps);
    for (int64_t i = 0; i < d; ++i) {
        double g = gamma ? oracle_elem(gdt, gamma, i) : 1.0;
        out[i] = v[i] * g * r;
    }
}

/* Plain vector-matrix product out[n] = sum_k v[k] * W[k][n], W [K, N] with row stride ldw. */
static void vecmat(int64_t K, int64_t N, const double* v, int wdt, const void* w, int64_t ldw,
                   double* out)
{
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += v[k] * oracle_elem(wdt, w, k * ldw + n);
        out[n] = acc;
    }
}

/*
 * The unsimplified chain: pre-norm, both projections, layerwise QK-Norm of each.
 * work must hold K + nq + nk doubles. yq [T, nq] and yk [T, nk] are dense.
 */
void oracle_qk_chain(int64_t T, int64_t K, int64_t nq, int64_t nk, double eps_pre,
                     double eps_qk, int xdt, const void* x, int64_t ldx, int g1dt,
                     const void* gamma_pre, int wdt, const void* wq, int64_t ldwq,
                     const void* wk, int64_t ldwk, int gdt, const void* gamma_q,
                     const void* gamma_k, double* work, double* yq, double* yk)
{
    double* h = work;
    double* q = work + K;
    double* k = q + nq;
    for (int64_t t = 0; t < T; ++t) {
        double s = row_sumsq(xdt, x, t * ldx, K);
        double r1 = 1.0 / sqrt(s / (double)K + eps_pre);
        for (int64_t i = 0; i < K; ++i) {
            double g = gamma_pre ? oracle_elem(g1dt, gamma_pre, i) : 1.0;
            h[i] = oracle_elem(xdt, x, t * ldx + i) * g * r1;
        }
        vecmat(K, nq, h, wdt, wq, ldwq, q);
        vecmat(K, nk, h, wdt, wk, ldwk, k);
        rms_vec(nq, q, gdt, gamma_q, eps_qk, yq + t * nq);
        rms_vec(nk, k, gdt, gamma_k, eps_qk, yk + t * nk);
    }
}

/*
 * The eliminated form: p = x W'q and x W'k with the pre-norm weight already folded in
 * (W' [K, n]) and no pre-norm, then layerwise QK-Norm of each. exact = 0 uses eps_qk as is;
 * exact = 1 uses eps_qk * (mean(x^2) + eps_pre) per token (the identity above).
 * work must hold nq + nk doubles.
 */
void oracle_qk_eliminated(int64_t T, int64_t K, int64_t nq, int64_t nk, double eps_qk,
                          double eps_pre, int exact, int xdt, const void* x, int64_t ldx,
                          int wdt, const void* wqf, int64_t ldwq, const void* wkf, int64_t ldwk,
                          int gdt, const void* gamma_q, const void* gamma_k, double* work,
                          double* yq, double* yk)
{
    double* q = work;
    double* k = work + nq;
    for (int64_t t = 0; t < T; ++t) {
        double eps = eps_qk;
        if (exact) eps = eps_qk * (row_sumsq(xdt, x, t * ldx, K) / (double)K + eps_pre);
        for (int64_t n = 0; n < nq; ++n) {
            double acc = 0.0;
            for (int64_t i = 0; i < K; ++i)
                acc += oracle_elem(xdt, x, t * ldx + i) * oracle_elem(wdt, wqf, i * ldwq + n);
            q[n] = acc;
        }
        for (int64_t n = 0; n < nk; ++n) {
            double acc = 0.0;
            for (int64_t i = 0; i < K; ++i)
                acc += oracle_elem(xdt, x, t * ldx + i) * oracle_elem(wdt, wkf, i * ldwk + n);
            k[n] = acc;
        }
        rms_vec(nq, q, gdt, gamma_q, eps, yq + t * nq);
        rms_vec(nk, k, gdt, gamma_k, eps, yk + t * nk);
    }
}

/* ------------------------------------------------------------------------------------------
 * LayerNorm ahead of a projection, with the same two steps ("FlashNorm", abstract: the method
 * carries over to LayerNorm). The pages give no formulas for it; the derivation used:
 *
 *     LN(x) = (x - mu) * r * gamma + beta,  mu = mean(x),  r = 1 / sqrt(mean((x - mu)^2) + eps)
 *     LN(x) W = r * (x W' - mu * c) + b,    W' = diag(gamma) W,  c[n] = sum_k W'[k][n],
 *                                           b[n] = sum_k beta[k] W[k][n]
 *
 * so gamma folds into W exactly as for RMSNorm, beta becomes an output bias, and the mean
 * enters as one rank-one correction with the column sums of the folded weight.
 * ------------------------------------------------------------------------------------------ */

/* Mean and (population) variance of one row, two passes. */
static void row_mean_var(int dtype, const void* x, int64_t off, int64_t d, double* mu,
                         double* var)
{
    double s = 0.0;
    for (int64_t i = 0; i < d; ++i) s += oracle_elem(dtype, x, off + i);
    double m = s / (double)d;
    double v = 0.0;
    for (int64_t i = 0; i < d; ++i) {
        double c = oracle_elem(dtype, x, off + i) - m;
        v += c * c;
    }
    *mu = m;
    *var = v / (double)d;
}

/* LayerNorm of each row; gamma / beta may be NULL (1 / 0). */
void oracle_layernorm_rows(int64_t T, int64_t d, double eps, int xdt, const void* x,
                           int64_t ldx, int gdt, const void* gamma, int bdt, const void* beta,
                           double* y, int64_t ldy)
{
    for (int64_t t = 0; t < T; ++t) {
        double mu, var;
        row_mean_var(xdt, x, t * ldx, d, &mu, &var);
        double r = 1.0 / sqrt(var + eps);
        for (int64_t i = 0; i < d; ++i) {
            double g = gamma ? oracle_elem(gdt, gamma, i) : 1.0;
            double b = beta ? oracle_elem(bdt, beta, i) : 0.0;
            y[t * ldy + i] = (oracle_elem(xdt, x, t * ldx + i) - mu) * r * g + b;
        }
    }
}

/* Column sums c[n] = sum_k W[k][n] of a [K, N] matrix. */
void oracle_colsum(int64_t K, int64_t N, int wdt, const void* w, int64_t ldw, double* c)
{
    for (int64_t n = 0; n < N; ++n) {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += oracle_elem(wdt, w, k * ldw + n);
        c[n] = s;
    }
}

/* Deferred LayerNorm-then-project: y[t][n] = r_t * (sum_k x[t][k] W'[k][n] - mu_t * c[n]) + b[n]
 * with mu_t, r_t from x as in LN; bias may be NULL. */
void oracle_normproj_layernorm(int64_t T, int64_t K, int64_t N, double eps, int xdt,
                               const void* x, int64_t ldx, int wdt, const void* wf, int64_t ldw,
                               int cdt, const void* colsum, int bdt, const void* bias, double* y,
                               int64_t ldy)
{
    for (int64_t t = 0; t < T; ++t) {
        double mu, var;
        row_mean_var(xdt, x, t * ldx, K, &mu, &var);
        double r = 1.0 / sqrt(var + eps);
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += oracle_elem(xdt, x, t * ldx + k) * oracle_elem(wdt, wf, k * ldw + n);
            double b = bias ? oracle_elem(bdt, bias, n) : 0.0;
            y[t * ldy + n] = r * (acc - mu * oracle_elem(cdt, colsum, n)) + b;
        }
    }
}

/* The unfused order: LayerNorm (with gamma, beta) first, then the product with W [K, N]. */
void oracle_layernorm_proj_unfused(int64_t T, int64_t K, int64_t N, double eps, int xdt,
                                   const void* x, int64_t ldx, int gdt, const void* gamma,
                                   int bdt, const void* beta, int wdt, const void* w,
                                   int64_t ldw, double* y, int64_t ldy)
{
    for (int64_t t = 0; t < T; ++t) {
        double mu, var;
        row_mean_var(xdt, x, t * ldx, K, &mu, &var);
        double r = 1.0 / sqrt(var + eps);
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double g = gamma ? oracle_elem(gdt, gamma, k) : 1.0;
                double b = beta ? oracle_elem(bdt, beta, k) : 0.0;
                double xn = (oracle_elem(xdt, x, t * ldx + k) - mu) * r * g + b;
                acc += xn * oracle_elem(wdt, w, k * ldw + n);
            }
            y[t * ldy + n] = acc;
        }
    }
}
