/*
 * qknorm.h - C ABI of libqknorm.so: layerwise QK-Norm and deferred norm-then-project on
 * AMD Instinct MI355X (gfx950).
 *
 * Operations (sources are the pages' titles and the part that states the operation):
 *
 *   RMSNorm of a row x of width d with per-column weight gamma and epsilon inside the root:
 *       r = 1 / sqrt( (1/d) * sum_i x_i^2 + eps ),     y_i = x_i * gamma_i * r
 *   Layerwise QK-Norm applies it to each token's full (heads * head_dim) Q and K projection
 *   vectors; the factor depends on the full vector ("SwiftQK: Fast and Communication-Efficient
 *   Tensor Parallelism for Query-Key Normalization", abstract).
 *
 * Conventions shared by every call:
 *   - Tensors are row-major [T, d] with a row stride ld (in elements, ld >= d). A tensor
 *     whose extent ((T - 1) * ld + d elements) exceeds 2^56 bytes is QKN_ERR_SHAPE, so that no
 *     size arithmetic can wrap.
 *   - Every pointer argument is a DEVICE pointer that the caller allocates and owns; the
 *     library allocates no memory. It keeps no workspace between calls, except the one
 *     device array per GPU that normproj_deferred_layernorm_noalloc uses.
 *   - `stream` is a hipStream_t passed as void*; NULL selects the null stream. Calls enqueue
 *     work and return; they never synchronise the host. There is no global mutable state
 *     except a thread-local copy of the last HIP error (and the device addresses of that
 *     array, looked up once per GPU under a lock), so calls are thread-safe.
 *   - dtype codes: QKN_F32 (float) and QKN_BF16 (bfloat16). Outputs have the input's dtype;
 *     arithmetic is fp32 with one rounding at the output (round to nearest even for bf16).
 *     Row statistics are fp32 sums: a row whose sum of squares exceeds the fp32 range gets
 *     r = 0 (outputs 0); squares below it are lost, which eps makes immaterial.
 *   - Arguments are validated before any HIP call; a non-zero status is returned without
 *     touching the device. T == 0 is a valid no-op. Launch failures return QKN_ERR_HIP and
 *     the raw hipError_t is kept for qkn_last_hip_error(). No exception crosses the ABI.
 *   - An output may alias its own input exactly (same pointer, same ld): the row is read in
 *     full before it is written. Any other overlap between an output and an input or another
 *     output is QKN_ERR_ALIAS.
 *   - Misaligned pointers and strides are accepted: 16-byte accesses run where every operand
 *     allows them, element accesses otherwise. Elements must sit at their natural alignment:
 *     2 bytes for bf16, 4 for fp32 (statistics included), 8 for the shard stage's 64-bit
 *     mailbox words; an element off it is QKN_ERR_ALIGN.
 *   - Projection weights (W, the folded W', the stacked Q/K weights) are row-major [K, N] with
 *     row stride ldw >= N, the layout y = x W reads them in.
 *   - Results are deterministic: fixed reduction orders, no atomic read-modify-write (the shard
 *     mailbox words are plain device-coherent 64-bit stores and loads).
 */
#ifndef QKNORM_H
#define QKNORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKN_API __attribute__((visibility("default")))

enum { QKN_F32 = 0, QKN_BF16 = 1 };

enum {
    QKN_OK = 0,
    QKN_ERR_NULL = 1,  /* a required pointer is NULL                                   */
    QKN_ERR_SHAPE = 2, /* negative or inconsistent sizes / strides                     */
    QKN_ERR_DTYPE = 3, /* unknown dtype code, or a dtype the operation does not support */
    QKN_ERR_EPS = 4,   /* eps is negative, NaN or infinite                               */
    QKN_ERR_ALIAS = 5, /* an output partially overlaps an input or another output        */
    QKN_ERR_ALIGN = 6, /* a pointer is not aligned to what the call requires            */
    QKN_ERR_HIP = 7,   /* the HIP runtime reported an error; see qkn_last_hip_error()    */
    QKN_ERR_SCRATCH = 8 /* the input exceeds the static workspace of a *_noalloc call     */
};

/*
 * qknorm_fused - layerwise QK-Norm of Q and K in ONE launch.
 *
 * ("SwiftQK: ...", abstract: RMSNorm over each token's full Q and K vectors.)
 * For every token t < T:  q_out[t,:] = RMSNorm(q[t, 0:dq]; gamma_q, eps)
 *                         k_out[t,:] = RMSNorm(k[t, 0:dk]; gamma_k, eps)
 *   T           tokens (>= 0)
 *   eps         finite, >= 0
 *   dtype       QKN_F32 or QKN_BF16: storage of q, k, q_out, k_out
 *   gamma_dtype QKN_F32 or QKN_BF16: storage of gamma_q [dq] and gamma_k [dk]
 *   q, ldq      input [T, dq], row stride ldq >= dq;  q_out, ldq_out likewise
 *   k, ...      the same for K. K is optional: pass k == k_out == gamma_k == NULL and dk == 0
 *               to normalise Q alone.
 * Sum of squares and scaling are fp32; the sum is reduced in a fixed order.
 */
QKN_API int qknorm_fused(int64_t T, float eps, int dtype, int gamma_dtype,
                         const void* q, int64_t ldq, void* q_out, int64_t ldq_out,
                         const void* gamma_q, int64_t dq,
                         const void* k, int64_t ldk, void* k_out, int64_t ldk_out,
                         const void* gamma_k, int64_t dk, void* stream);

/*
 * qknorm_partial_sumsq - first half of the scalar-statistics split (one GPU's shard stage).
 *
 * ("SwiftQK: ...", abstract: ranks exchange scalar partial sums instead of activation vectors.)
 * psq_q[t] = sum_{i < dq_local} q[t,i]^2 and psq_k[t] likewise, in fp32, one launch for both.
 *   q [T, dq_local] with stride ldq (the shard's column slice), psq_q [T] fp32 output.
 *   K is optional (k == psq_k == NULL, dk_local == 0).
 */
QKN_API int qknorm_partial_sumsq(int64_t T, int dtype,
                                 const void* q, int64_t ldq, int64_t dq_local, float* psq_q,
                                 const void* k, int64_t ldk, int64_t dk_local, float* psq_k,
                                 void* stream);

/*
 * qknorm_apply_with_stats - second half: aggregate the statistics, then scale the slice.
 *
 * ("SwiftQK: ...", abstract: scalar aggregation, then the element-wise scale.) For row t:
 *   S = psq[t] + ext[0*ld_ext + t] + ... + ext[(n_ext-1)*ld_ext + t]   (fp32, in this order)
 *   r = 1 / sqrt(S / d_full + eps)        -- mean over the FULL width d_full, not the slice
 *   out[t, i] = x[t, i] * gamma[i] * r    for i < d_local
 *   n_ext       number of peers' partials (>= 0; 0 means the slice is the whole row)
 *   psq_*       [T] fp32 own partials (e.g. from qknorm_partial_sumsq)
 *   ext_*       [n_ext, T] fp32, peer-major, row stride ld_ext >= T (may be NULL if n_ext==0)
 *   d_*_full    full row width, >= d_*_local >= 1
 *   gamma_*     the slice's own gamma values [d_local]
 *   K is optional (k, k_out, gamma_k, psq_k, ext_k NULL and dk_local == 0).
 */
QKN_API int qknorm_apply_with_stats(int64_t T, float eps, int dtype, int gamma_dtype,
                                    int64_t n_ext,
                                    const void* q, int64_t ldq, void* q_out, int64_t ldq_out,
                                    const void* gamma_q, int64_t dq_local, int64_t dq_full,
                                    const float* psq_q, const float* ext_q, int64_t ld_ext_q,
                                    const void* k, int64_t ldk, void* k_out, int64_t ldk_out,
                                    const void* gamma_k, int64_t dk_local, int64_t dk_full,
                                    const float* psq_k, const float* ext_k, int64_t ld_ext_k,
                                    void* stream);

/*
 * qknorm_shard_fused - the shard stage in ONE pass over this rank's slice.
 *
 * ("SwiftQK: ...", abstract: ranks exchange per-row scalars only, and waiting for the peers'
 * scalars is hidden behind element-wise work in one persistent kernel that cannot deadlock.)
 * Computes what qknorm_partial_sumsq followed by qknorm_apply_with_stats computes, reading x
 * once. Exchanged partials travel as mailbox WORDS: uint64 = (epoch << 32) | the
 * fp32 bits of the value, each stored and loaded as one aligned 64-bit device-coherent access,
 * so a word that carries the current epoch carries its value (no separate flags). Per row:
 *   1. s_own = sum of squares of the slice's row; if psq_*_out != NULL it is published there
 *      as a word ([T], 8-byte aligned);
 *   2. if epoch != 0, waits until mail_*[e * ld_mail + row] carries `epoch` for every peer
 *      e < n_ext (at most max_spin polls per row block, then sets *timed_out = 1 and carries
 *      on: the rows of that block are then unspecified); with epoch == 0 the mailbox is taken
 *      as complete and its tags are not looked at;
 *   3. S = s_own + value(mail[0][row]) + ... + value(mail[n_ext-1][row])  (fp32, this order),
 *      out = x * gamma * (1 / sqrt(S / d_full + eps)).
 * mail_* are the mailboxes the peers fill ([n_ext, T] words, row stride ld_mail >= T,
 * 8-byte aligned), for instance by qknorm_shard_publish. A new pass over the same mailbox uses
 * a new epoch (mailboxes start zeroed, epoch 0 never matches a wait).
 *   persistent  1: every workgroup (one per row block, dispatched in ascending order) reserves
 *               LDS it does not use, so that at most three quarters of the workgroups the
 *               registers allow are resident on a CU at once; a producer of the words running
 *               on another stream of the SAME device then always finds a quarter of the slots
 *               and of the LDS free (required then), provided its work is not queued behind
 *               this pass: streams are mapped onto a few hardware queues, and a producer
 *               submitted later to a stream that shares the pass's queue starts only after the
 *               pass ends (the pass then times out). Submitting the producer's work before the
 *               pass avoids that on any mapping;
 *               0: no reservation, for producers that do not run on this device, such as the
 *               peer ranks under tensor parallelism; every rank must then launch the same grid
 *               so that row blocks are dispatched in the same ascending order everywhere.
 *               Ignored when epoch == 0 (nothing waits). Both policies stream at the same rate.
 *   n_ext     0..64
 *   timed_out device int (required when epoch != 0), set to 1 on a timeout, never cleared
 *   slices    any strides and widths d_local <= 2048 bf16 / 1024 fp32 (QKN_ERR_SHAPE); 16-byte
 *             accesses where the slices are 16-byte aligned with ld * sizeof(dtype) and d_local
 *             multiples of 16 bytes, element accesses otherwise
 * Other arguments as for qknorm_apply_with_stats; K optional in the same way.
 */
QKN_API int qknorm_shard_fused(int64_t T, float eps, int dtype, int gamma_dtype, int64_t n_ext,
                               const void* q, int64_t ldq, void* q_out, int64_t ldq_out,
                               const void* gamma_q, int64_t dq_local, int64_t dq_full,
                               uint64_t* psq_q_out, const uint64_t* mail_q, int64_t ld_mail_q,
                               const void* k, int64_t ldk, void* k_out, int64_t ldk_out,
                               const void* gamma_k, int64_t dk_local, int64_t dk_full,
                               uint64_t* psq_k_out, const uint64_t* mail_k, int64_t ld_mail_k,
                               uint32_t epoch, int persistent, int64_t max_spin, int* timed_out,
                               void* stream);

/*
 * qknorm_shard_publish - a peer's side of the mailbox of qknorm_shard_fused.
 *
 * For every peer e < n_ext and row t: mail_*[e * ld_mail + t] = (epoch << 32) | bits of
 * part_*[e * ld_part + t], one device-coherent 64-bit store each. Under tensor parallelism
 * each rank writes its own slot of every peer's mailbox this way (its psq words); on one GPU
 * this call stands in for the peers.
 * part_* [n_ext, T] fp32 (row stride ld_part >= T); mail_* 8-byte aligned words; K optional
 * (part_k == mail_k == NULL).
 */
QKN_API int qknorm_shard_publish(int64_t T, int64_t n_ext, const float* part_q, int64_t ld_part_q,
                                 uint64_t* mail_q, int64_t ld_mail_q, const float* part_k,
                                 int64_t ld_part_k, uint64_t* mail_k, int64_t ld_mail_k,
                                 uint32_t epoch, void* stream);

/*
 * normproj_fold_weight - fold the norm weights into the following projection (once, offline).
 *
 * ("FlashNorm: Fast Normalization for Transformers", abstract, item (i).)
 * For the projection y = x W with W [K, N] row-major (stride ldw >= N):
 *   w_fold[k * ldw_fold + n] = bf16( gamma[k] * W[k, n] )     (fp32 product, one rounding)
 * i.e. W' = diag(gamma) W in the layout of W, [K, N] row-major (stride ldw_fold >= N), the
 * operand normproj_deferred takes. gamma == NULL means gamma = 1 (a plain copy). w_fold may be
 * w itself with the same stride (in place); any other overlap is QKN_ERR_ALIAS.
 *   dtype       storage of W and w_fold: QKN_BF16 only
 *   gamma_dtype QKN_F32 or QKN_BF16
 */
QKN_API int normproj_fold_weight(int64_t K, int64_t N, int dtype, int gamma_dtype,
                                 const void* w, int64_t ldw, const void* gamma,
                                 void* w_fold, int64_t ldw_fold, void* stream);

/*
 * normproj_deferred - RMSNorm followed by the projection, with the scale deferred.
 *
 * ("FlashNorm: ...", abstract, item (ii): the scalar 1/RMS is applied to the output of the
 * matrix product, so the reduction and the product proceed together.) For t < T, n < N:
 *   r_t     = 1 / sqrt( (1/K) sum_k x[t,k]^2 + eps )         (fp32, from the same x tiles)
 *   y[t,n]  = bf16( r_t * sum_k x[t,k] * w_fold[k,n] )        (bf16 products, fp32 accumulate)
 *   x       [T, K] bf16, stride ldx >= K
 *   w_fold  W' [K, N] bf16 row-major (e.g. from normproj_fold_weight), stride ldw >= N
 *   y       [T, N] bf16, stride ldy >= N; must not overlap x or w_fold
 *   dtype   QKN_BF16 only
 * Any K, strides and 2-byte-aligned pointers. With K, ldx, ldw (and N, for T > 16) multiples
 * of 8 and x, w_fold 16-byte aligned, T <= 16 runs a streaming matrix-vector kernel and larger
 * T the pipelined matrix-core (MFMA) kernels; other operands take an element-load
 * matrix-core kernel.
 */
QKN_API int normproj_deferred(int64_t T, int64_t K, int64_t N, float eps, int dtype,
                              const void* x, int64_t ldx, const void* w_fold, int64_t ldw,
                              void* y, int64_t ldy, void* stream);

/*
 * normproj_unfused - the order the fold replaces, kept as the measured baseline.
 *
 * ("FlashNorm: ...", abstract: the RMS reduction blocks the following product.)
 *   xn[t,k] = bf16( x[t,k] * gamma[k] * r_t )      (an RMSNorm launch, caller's buffer xn)
 *   y[t,n]  = bf16( sum_k xn[t,k] * w[k,n] )        (a plain matrix-core launch)
 *   w  the UNFOLDED weight W [K, N] bf16 row-major, stride ldw >= N
 *   xn [T, K] bf16 (stride ldxn) is scratch owned by the caller.
 * Same dtype and alignment rules as normproj_deferred.
 */
QKN_API int normproj_unfused(int64_t T, int64_t K, int64_t N, float eps, int dtype,
                             int gamma_dtype, const void* x, int64_t ldx, const void* gamma,
                             const void* w, int64_t ldw, void* xn, int64_t ldxn,
                             void* y, int64_t ldy, void* stream);

/*
 * normproj_fold_layernorm - the fold for LayerNorm followed by the projection (once, offline).
 *
 * ("FlashNorm: ...", abstract: the folding and deferral carry over to LayerNorm. The pages
 * give no formulas; the ones used follow from LN(x) W = r (x W' - mu c) + beta W.)
 *   w_fold      as normproj_fold_weight: W' = diag(gamma) W, bf16 [K, N] row-major
 *   colsum[n] = sum_k W'[k, n]  over the bf16 values of w_fold exactly as stored (fp64 sum,
 *               rounded once to fp32), [N] fp32
 *   bias[n]   = sum_k beta[k] W[k, n]  (fp64 sum, rounded once), [N] fp32; may be NULL
 * gamma / beta may be NULL (1 / 0); both use gamma_dtype. Outputs must not overlap each other
 * or the inputs. Layout and alignment rules of normproj_fold_weight.
 */
QKN_API int normproj_fold_layernorm(int64_t K, int64_t N, int dtype, int gamma_dtype,
                                    const void* w, int64_t ldw, const void* gamma,
                                    const void* beta, void* w_fold, int64_t ldw_fold,
                                    float* colsum, float* bias, void* stream);

/*
 * normproj_deferred_layernorm - LayerNorm followed by the projection, normalisation deferred.
 *
 * (Same passage.) For t < T, n < N, with the row statistics in fp32 (sums of x - x[t,0] and of
 * its square):
 *   mu_t    = (1/K) sum_k x[t,k]
 *   r_t     = 1 / sqrt( (1/K) sum_k (x[t,k] - mu_t)^2 + eps )
 *   y[t,n]  = bf16( r_t * (sum_k x[t,k] w_fold[k,n] - mu_t colsum[n]) + bias[n] )
 *   colsum, bias  [N] fp32 from normproj_fold_layernorm; bias may be NULL (zero)
 *   row_stats     optional [T, 2] fp32 workspace (caller-owned, must not overlap any other
 *                 argument). When given, 8-byte aligned, and the product runs on the pipelined
 *                 matrix-core kernels (T > 16; N, ldy, K, ldx, ldw multiples of 8; x, w_fold and
 *                 y 16-byte aligned; K a multiple of 64, or of 32 for large shapes), (mu_t, r_t)
 *                 are computed by one streaming pass over x into row_stats and the product
 *                 applies them in its epilogue; otherwise (and when NULL) the product
 *                 accumulates them from the x tiles it multiplies, and row_stats is left
 *                 untouched. The pass costs one read of x; accumulating
 *                 inside the product repeats the work once per 128- or 256-column block of y.
 * Other arguments, dtype and alignment rules as normproj_deferred.
 */
QKN_API int normproj_deferred_layernorm(int64_t T, int64_t K, int64_t N, float eps, int dtype,
                                        const void* x, int64_t ldx, const void* w_fold,
                                        int64_t ldw, const float* colsum, const float* bias,
                                        void* y, int64_t ldy, float* row_stats, void* stream);

/*
 * normproj_deferred_layernorm_noalloc - normproj_deferred_layernorm for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc) and have no workspace of their own to pass.
 *
 * Computes exactly what normproj_deferred_layernorm computes with a row_stats workspace (the
 * same kernels and results), with the workspace taken from a device array the library holds:
 * 2 * 131072 fp32 (1 MiB) per GPU, kept until the process ends. It calls no allocator.
 *   T           at most 131072 rows (QKN_ERR_SCRATCH beyond; nothing is launched)
 * Every call on one GPU shares that GPU's array and overwrites it before reading it, so calls
 * that overlap in time on one GPU (other streams, other threads) race and must be ordered by
 * the caller. The first call on a device looks up the array's device address (a HIP call).
 * Other arguments and rules as normproj_deferred_layernorm.
 */
QKN_API int normproj_deferred_layernorm_noalloc(int64_t T, int64_t K, int64_t N, float eps,
                                                int dtype, const void* x, int64_t ldx,
                                                const void* w_fold, int64_t ldw,
                                                const float* colsum, const float* bias, void* y,
                                                int64_t ldy, void* stream);

/*
 * normproj_layernorm_unfused - LayerNorm launch then plain projection (measured baseline).
 *   xn[t,k] = bf16( (x[t,k] - mu_t) r_t gamma[k] + beta[k] )   (caller's scratch xn [T, K])
 *   y[t,n]  = bf16( sum_k xn[t,k] w[k,n] )
 * w is the unfolded weight W [K, N] row-major. gamma / beta (gamma_dtype, may be NULL) must be
 * aligned to their element size. Other rules as normproj_unfused.
 */
QKN_API int normproj_layernorm_unfused(int64_t T, int64_t K, int64_t N, float eps, int dtype,
                                       int gamma_dtype, const void* x, int64_t ldx,
                                       const void* gamma, const void* beta,
                                       const void* w, int64_t ldw, void* xn,
                                       int64_t ldxn, void* y, int64_t ldy, void* stream);

/*
 * qknorm_project_eliminated - Q/K projection and layerwise QK-Norm with the pre-attention
 * RMSNorm removed.
 *
 * ("FlashNorm: ...", abstract: RMS is unchanged by scaling its input, so with a second RMSNorm
 * after the linear layer the first one has no effect and can be removed, e.g. ahead of
 * attention with Q/K normalisation.) The pre-norm weight is folded into the stacked projection
 * w_qk = [W'q | W'k] ([K, nq + nk] bf16 row-major, stride ldw >= nq + nk: normproj_fold_weight
 * of the stacked weight [Wq | Wk] with the pre-norm's gamma):
 *   p[t,:]       = x[t,:] w_qk                  exact == 0: no pre-norm at all
 *                = r1_t x[t,:] w_qk             exact == 1: r1_t = 1/sqrt(mean(x_t^2) + eps_pre)
 *   y[t, 0:nq]   = p[t,0:nq] gamma_q / sqrt(mean(p[t,0:nq]^2) + eps_qk)
 *   y[t, nq:]    = p[t,nq:] gamma_k / sqrt(mean(p[t,nq:]^2) + eps_qk)
 * With exact == 0 the result equals the pre-norm -> projection -> QK-Norm chain with eps_qk
 * replaced per token by eps_qk / (mean(x_t^2) + eps_pre): identical when eps_qk == 0, and for
 * eps_qk > 0 the two differ by that epsilon alone (negligible once mean(p^2) >> eps_qk * mean(x^2)).
 * exact == 1 keeps the pre-norm's scale (deferred to the product's output) and equals the
 * chain for every epsilon.
 *   x    [T, K] bf16 (stride ldx)     y  [T, nq + nk] bf16 (stride ldy), also holds p (bf16)
 *   gamma_q [nq], gamma_k [nk] in gamma_dtype; nk == 0 normalises Q only (gamma_k unused)
 * Two launches: the matrix-core product, then the fused Q+K row kernel in place on y.
 * Alignment rules of normproj_deferred; y must not overlap x, w_qk or the gammas.
 */
QKN_API int qknorm_project_eliminated(int64_t T, int64_t K, int64_t nq, int64_t nk,
                                      float eps_qk, float eps_pre, int exact, int gamma_dtype,
                                      const void* x, int64_t ldx, const void* w_qk, int64_t ldw,
                                      const void* gamma_q, const void* gamma_k, void* y,
                                      int64_t ldy, void* stream);

/*
 * qknorm_project_unfused - the chain qknorm_project_eliminated simplifies, in one call
 * (measured baseline): pre-attention RMSNorm launch, plain product, layerwise QK-Norm launch.
 *
 * ("FlashNorm: ...", abstract: the RMSNorm ahead of a linear layer whose output is normalised
 * again; this is that chain computed as written.)
 *   xn[t,k]     = bf16( x[t,k] gamma_pre[k] / sqrt(mean(x_t^2) + eps_pre) )   (caller's xn)
 *   p[t,:]      = bf16( xn[t,:] w )                                            (kept in y)
 *   y[t, 0:nq]  = p[t,0:nq] gamma_q / sqrt(mean(p[t,0:nq]^2) + eps_qk)
 *   y[t, nq:]   = p[t,nq:] gamma_k / sqrt(mean(p[t,nq:]^2) + eps_qk)
 * w [K, nq + nk] bf16 row-major is the unfolded stacked weight [Wq | Wk] (stride ldw >= nq + nk).
 * The intermediates xn and p are written with
 * ordinary stores, because the next launch reads them straight back (as p is in
 * qknorm_project_eliminated), so the two entry points differ by the pre-norm alone.
 *   x [T, K] bf16 (ldx); xn [T, K] bf16 scratch (ldxn, caller-owned, must not
 *   overlap any other argument); y [T, nq + nk] bf16 (ldy)
 *   gamma_pre [K], gamma_q [nq], gamma_k [nk] in gamma_dtype; nk == 0 normalises Q only
 * Three launches. Alignment rules of normproj_unfused; y must not overlap x, w or the
 * gammas. Every argument is checked before the first launch.
 */
QKN_API int qknorm_project_unfused(int64_t T, int64_t K, int64_t nq, int64_t nk, float eps_qk,
                                   float eps_pre, int gamma_dtype, const void* x, int64_t ldx,
                                   const void* gamma_pre, const void* w, int64_t ldw,
                                   const void* gamma_q, const void* gamma_k, void* xn,
                                   int64_t ldxn, void* y, int64_t ldy, void* stream);

/*
 * qkn_device_copy - plain streaming copy of nbytes (16-byte vectors where aligned).
 * Used to calibrate measured bandwidth and memory counters against a kernel of known traffic.
 * dst and src must not overlap.
 */
QKN_API int qkn_device_copy(void* dst, const void* src, int64_t nbytes, void* stream);

/* Static description of a status code (never NULL). */
QKN_API const char* qkn_status_string(int status);

/* Raw hipError_t of the last QKN_ERR_HIP returned on the calling thread (0 if none). */
QKN_API int qkn_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QKNORM_H */
