// Host-side launch interface between the C-ABI layer (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkn {

// What a row launch computes for each row of its tensors.
enum RowMode : int {
    kFused = 0,    // sum of squares -> 1/rms over the row -> x * gamma * (1/rms)
    kPartial = 1,  // sum of squares of the slice -> psq_out[row]
    kApply = 2,    // psq_in[row] + ext[..][row] -> 1/rms over d_full -> x * gamma * (1/rms)
};

// One tensor (Q or K) of a row launch.
struct RowSeg {
    const void* x;       // [T, d] input, row stride ldx elements
    void* y;             // [T, d] output (kFused / kApply), row stride ldy
    const void* g;       // gamma [d] (kFused / kApply)
    int64_t ldx, ldy;
    int64_t d;           // columns processed
    float inv_dfull;     // 1 / width the mean is taken over (d for kFused, d_full for kApply)
    const float* psq_in; // kApply: own partial [T]
    const float* ext;    // kApply: peers' partials [n_ext, T], row stride ld_ext
    int64_t ld_ext;
    int64_t n_ext;
    float* psq_out;      // kPartial: [T]
};

struct RowJob {
    RowSeg seg[2];       // seg[1] is used only when nseg == 2
    int nseg;
    int64_t T;
    float eps;
    int mode;            // RowMode
    int bf16;            // storage of x / y: 1 = bf16, 0 = fp32
    int gamma_bf16;      // storage of gamma: 1 = bf16, 0 = fp32
    int keep_cached;     // 1: the caller reads y back next, so a one-tensor fused job stores
                         // it with ordinary stores (kept in the caches) instead of
                         // non-temporal ones
};

// Chooses the register-resident kernel (one wavefront per row group, 16-byte accesses) when
// every tensor is 16-byte aligned and fits in registers; otherwise a workgroup-per-row
// two-pass kernel (16-byte or element accesses).
hipError_t launch_rows(const RowJob& job, hipStream_t stream);

// W [K, N] (stride ldw) -> w_fold [K, N] (stride ldwf) = bf16(gamma[k] * W[k, n]).
hipError_t launch_fold(int64_t K, int64_t N, const void* w, int64_t ldw, const void* gamma,
                       int gamma_bf16, void* w_fold, int64_t ldwf, hipStream_t stream);

// Epilogue of the projection acc = x [T, K] . w with w = W' row-major [K, N].
enum Epi : int {
    kEpiPlain = 0,      // y = bf16(acc)
    kEpiRms = 1,        // y = bf16(acc / rms(x row))
    kEpiLayerNorm = 2,  // y = bf16(r * (acc - mean(x row) * colsum[n]) + bias[n]), r = 1/std
    kEpiLayerNormStats = 3,  // the same with (mean, r) of each row read from rowstats [T, 2]
};
// Flag or-ed into the epilogue: the caller reads y again right away, so the tiled kernels
// store it with ordinary stores (it stays in the caches) instead of non-temporal ones.
constexpr int kEpiKeepCached = 16;
// rowstats is read by kEpiLayerNormStats only, which runs on the pipelined kernels alone
// (normproj_pipelined() must hold).
hipError_t launch_normproj(int64_t T, int64_t K, int64_t N, float eps, int epi,
                           const void* x, int64_t ldx, const void* w, int64_t ldw, void* y,
                           int64_t ldy, const float* colsum, const float* bias,
                           const float* rowstats, hipStream_t stream);

// Whether launch_normproj runs one of the pipelined matrix-core kernels for this shape and
// these operands.
bool normproj_pipelined(int64_t T, int64_t K, int64_t N, const void* x, int64_t ldx,
                        const void* w, int64_t ldw, int64_t ldy, const void* y);

// rowstats[t] = (mean of x row t, 1 / sqrt(var + eps)) in fp32, K % 8 == 0, rows 16-byte aligned.
hipError_t launch_layernorm_stats(int64_t T, int64_t K, float eps, const void* x, int64_t ldx,
                                  float* rowstats, hipStream_t stream);

// colsum[n] = sum_k bf16(gamma[k] * W[k, n]), bias[n] = sum_k beta[k] * W[k, n] (bias may be
// null; gamma / beta null mean 1 / 0; gamma and beta share one storage type).
hipError_t launch_fold_stats(int64_t K, int64_t N, const void* w, int64_t ldw, const void* gamma,
                             const void* beta, int gb_bf16, float* colsum, float* bias,
                             hipStream_t stream);

// y [T, K] = bf16(LayerNorm(x) * gamma + beta), any alignment (16-byte accesses where x, y,
// gamma and beta allow them).
hipError_t launch_layernorm_rows(int64_t T, int64_t K, float eps, const void* x, int64_t ldx,
                                 const void* gamma, const void* beta, int gb_bf16, void* y,
                                 int64_t ldy, hipStream_t stream);

hipError_t launch_copy(void* dst, const void* src, int64_t nbytes, hipStream_t stream);

// Single-launch shard stage (partial sums, publication, wait for peers, aggregation, scale)
// with an epoch-tagged mailbox: each exchanged partial is one 64-bit word (epoch << 32 | fp32).
struct ShardSeg {
    const void* x;
    void* y;
    const void* g;
    int64_t ldx, ldy, d;      // slice width d
    float inv_dfull;
    uint64_t* psq_out;        // [T] own partials as words, or null
    const uint64_t* mail;     // [n_ext][ld_mail] peers' partials as words
    int64_t ld_mail;
};
struct ShardArgs {
    ShardSeg seg[2];
    int nseg;
    int64_t T;
    float eps;
    int64_t n_ext;
    int bf16, gamma_bf16;
    uint32_t epoch;           // 0: mailbox complete before launch, no tag checks, no waiting
    int persistent;           // 1: at most 3/4 of the resident workgroups at once, 0: no cap
    int64_t max_spin;
    int* timed_out;
};
hipError_t launch_shard_fused(const ShardArgs& args, hipStream_t stream);
hipError_t launch_shard_publish(int64_t T, int64_t n_ext, int nseg, const float* const* src,
                                const int64_t* ld_src, uint64_t* const* dst,
                                const int64_t* ld_dst, uint32_t epoch, hipStream_t stream);

}  // namespace qkn
