// Norm-then-project on gfx950 with the RMS scale deferred to the product's output
// ("FlashNorm: Fast Normalization for Transformers", abstract, items (i) and (ii)), plus the
// one-time weight fold and a plain streaming copy used for calibration.
//
// Matrix-core kernel: y[t, n] = r_t * sum_k x[t, k] * w[n, k] with both operands K-contiguous
// (the fold writes W' transposed). A 256-thread workgroup owns a 128 x 128 output tile; its
// four wavefronts each own 64 x 64 as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16. Tiles of
// 128 x 64 of x and W' are staged through LDS (row pitch padded by 16 bytes so the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks), with the next tile's global loads
// in flight while the current tile feeds the matrix cores. The same x vectors that go to LDS
// are squared and summed by the VALU, so 1/rms is ready at the epilogue without another pass
// over x: the reduction runs beside the product instead of before it.
//
// Small T (<= 16) is a matrix-vector product bound by streaming W' once: a wavefront per pair
// of output columns, fp32 dot products reduced across the wave.

#include "device.h"
#include "launch.h"

namespace qkn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;             // LDS row pitch in bf16 elements (144 bytes)
constexpr int kThreads = 256;
constexpr int kChunksPerRow = kBK / 8;      // 16-byte chunks per tile row
constexpr int kLoadsPerThread = kBM * kChunksPerRow / kThreads;  // 4

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <bool NORM>
__global__ __launch_bounds__(kThreads) void normproj_mfma_kernel(
    int64_t T, int64_t K, int64_t N, float eps, float inv_k, const uint16_t* __restrict__ x,
    int64_t ldx, const uint16_t* __restrict__ w, int64_t ldw, uint16_t* __restrict__ y,
    int64_t ldy, int nbm, int nbn)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kPitch];
    __shared__ float rstd[kBM];

    // Blocks are handed to the 8 XCDs round-robin; give each XCD a contiguous range of tiles
    // (whole row panels of x) so that panel is fetched into one XCD's L2 only.
    const int nb = nbm * nbn;
    int bid = (int)blockIdx.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    const int tm = bid / nbn;
    const int tn = bid % nbn;
    const int64_t m0 = (int64_t)tm * kBM;
    const int64_t n0 = (int64_t)tn * kBN;

    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;

    // Global -> register staging: chunk c of this thread is tile row (tid/8 + 32c), k-chunk tid%8.
    const int ld_row = tid / kChunksPerRow;
    const int ld_kc = tid % kChunksPerRow;
    u32x4 ra[kLoadsPerThread], rb[kLoadsPerThread];
    float ssq[kLoadsPerThread] = {0.0f, 0.0f, 0.0f, 0.0f};

    auto load_tiles = [&](int64_t k0) {
        const int64_t k = k0 + ld_kc * 8;
#pragma unroll
        for (int c = 0; c < kLoadsPerThread; ++c) {
            const int r = ld_row + c * (kThreads / kChunksPerRow);
            const int64_t gm = m0 + r, gn = n0 + r;
            ra[c] = (gm < T && k < K) ? *(const u32x4*)(x + gm * ldx + k) : u32x4{0u, 0u, 0u, 0u};
            rb[c] = (gn < N && k < K) ? *(const u32x4*)(w + gn * ldw + k) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_tiles = [&]() {
#pragma unroll
        for (int c = 0; c < kLoadsPerThread; ++c) {
            const int r = ld_row + c * (kThreads / kChunksPerRow);
            *(u32x4*)(As + r * kPitch + ld_kc * 8) = ra[c];
            *(u32x4*)(Bs + r * kPitch + ld_kc * 8) = rb[c];
            if constexpr (NORM) {
                const u32x4 v = ra[c];
                float s = ssq[c];
                s = fmaf(bf16_lo(v.x), bf16_lo(v.x), s); s = fmaf(bf16_hi(v.x), bf16_hi(v.x), s);
                s = fmaf(bf16_lo(v.y), bf16_lo(v.y), s); s = fmaf(bf16_hi(v.y), bf16_hi(v.y), s);
                s = fmaf(bf16_lo(v.z), bf16_lo(v.z), s); s = fmaf(bf16_hi(v.z), bf16_hi(v.z), s);
                s = fmaf(bf16_lo(v.w), bf16_lo(v.w), s); s = fmaf(bf16_hi(v.w), bf16_hi(v.w), s);
                ssq[c] = s;
            }
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int64_t nk = (K + kBK - 1) / kBK;
    load_tiles(0);
    store_tiles();
    __syncthreads();

    // MFMA operand fragments: lane holds row (lane % 32) of a 32-row block, 8 consecutive k
    // starting at 8 * (lane / 32) within each 16-wide k step.
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    for (int64_t kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) load_tiles((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            u32x4 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                af[i] = *(const u32x4*)(As + (wm * 64 + i * 32 + frag_row) * kPitch + ks * 16 + frag_k);
                bfr[i] = *(const u32x4*)(Bs + (wn * 64 + i * 32 + frag_row) * kPitch + ks * 16 + frag_k);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
        __syncthreads();
        if (kt + 1 < nk) {
            store_tiles();
            __syncthreads();
        }
    }

    if constexpr (NORM) {
        // Combine the 8 threads that share each tile row, then 1/rms per row.
#pragma unroll
        for (int c = 0; c < kLoadsPerThread; ++c) {
            const float s = sum8(ssq[c]);
            if (ld_kc == 0) rstd[ld_row + c * (kThreads / kChunksPerRow)] = rsqrtf(s * inv_k + eps);
        }
        __syncthreads();
    }

    // Accumulator layout of a 32x32 block: lane holds column lane % 32, and for e in 0..15 the
    // row 8 * (e / 4) + 4 * (lane / 32) + e % 4.
    const int out_col = lane & 31;
    const int out_row = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t gn = n0 + wn * 64 + j * 32 + out_col;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = wm * 64 + i * 32 + 8 * (e / 4) + out_row + (e % 4);
                const int64_t gm = m0 + r;
                float v = acc[i][j][e];
                if constexpr (NORM) v *= rstd[r];
                if (gm < T && gn < N) y[gm * ldy + gn] = to_bf16(v);
            }
        }
    }
}

// Matrix-vector form for T <= 16: each wavefront produces kCols adjacent output columns for
// every token; W' rows are streamed once, x rows come from cache.
constexpr int kGemvCols = 2;
constexpr int kGemvMaxT = 16;

template <bool NORM>
__global__ __launch_bounds__(kThreads) void normproj_gemv_kernel(
    int T, int64_t K, int64_t N, float eps, float inv_k, const uint16_t* __restrict__ x,
    int64_t ldx, const uint16_t* __restrict__ w, int64_t ldw, uint16_t* __restrict__ y,
    int64_t ldy)
{
    const int lane = lane_id();
    const int64_t n_base = ((int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave) * kGemvCols;
    if (n_base >= N) return;

    float acc[kGemvMaxT][kGemvCols];
    float ssq[kGemvMaxT];
#pragma unroll
    for (int t = 0; t < kGemvMaxT; ++t) {
        ssq[t] = 0.0f;
#pragma unroll
        for (int c = 0; c < kGemvCols; ++c) acc[t][c] = 0.0f;
    }

    for (int64_t k = (int64_t)lane * 8; k < K; k += kWave * 8) {
        float wf[kGemvCols][8];
#pragma unroll
        for (int c = 0; c < kGemvCols; ++c) {
            const int64_t n = n_base + c;
            const u32x4 v = n < N ? load_stream(w + n * ldw + k) : u32x4{0u, 0u, 0u, 0u};
            wf[c][0] = bf16_lo(v.x); wf[c][1] = bf16_hi(v.x);
            wf[c][2] = bf16_lo(v.y); wf[c][3] = bf16_hi(v.y);
            wf[c][4] = bf16_lo(v.z); wf[c][5] = bf16_hi(v.z);
            wf[c][6] = bf16_lo(v.w); wf[c][7] = bf16_hi(v.w);
        }
#pragma unroll
        for (int t = 0; t < kGemvMaxT; ++t) {
            if (t < T) {
                const u32x4 v = *(const u32x4*)(x + (int64_t)t * ldx + k);
                float xf[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                               bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if constexpr (NORM) ssq[t] = fmaf(xf[e], xf[e], ssq[t]);
#pragma unroll
                    for (int c = 0; c < kGemvCols; ++c) acc[t][c] = fmaf(xf[e], wf[c][e], acc[t][c]);
                }
            }
        }
    }

#pragma unroll
    for (int t = 0; t < kGemvMaxT; ++t) {
        if (t < T) {
            float rs = 1.0f;
            if constexpr (NORM) rs = rsqrtf(wave_sum(ssq[t]) * inv_k + eps);
#pragma unroll
            for (int c = 0; c < kGemvCols; ++c) {
                const float v = wave_sum(acc[t][c]) * rs;
                if (lane == c && n_base + c < N) y[(int64_t)t * ldy + n_base + c] = to_bf16(v);
            }
        }
    }
}

// W [K, N] -> w_fold [N, K] = bf16(gamma[k] * W[k, n]) through a 64 x 64 LDS tile.
__global__ __launch_bounds__(kThreads) void fold_kernel(int64_t K, int64_t N,
                                                        const uint16_t* __restrict__ w,
                                                        int64_t ldw, const void* gamma,
                                                        int gamma_bf16,
                                                        uint16_t* __restrict__ wf, int64_t ldwf)
{
    __shared__ uint16_t tile[64][66];
    const int64_t k0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    const int tx = (int)threadIdx.x % 64, ty = (int)threadIdx.x / 64;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = i * 4 + ty;  // k within tile
        const int64_t k = k0 + r, n = n0 + tx;
        uint16_t out = 0;
        if (k < K && n < N) {
            float g = 1.0f;
            if (gamma) g = gamma_bf16 ? __uint_as_float((uint32_t)((const uint16_t*)gamma)[k] << 16)
                                      : ((const float*)gamma)[k];
            out = to_bf16(g * __uint_as_float((uint32_t)w[k * ldw + n] << 16));
        }
        tile[tx][r] = out;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = i * 4 + ty;  // n within tile
        const int64_t n = n0 + r, k = k0 + tx;
        if (k < K && n < N) wf[n * ldwf + k] = tile[r][tx];
    }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(char* __restrict__ dst,
                                                        const char* __restrict__ src,
                                                        int64_t nbytes, int vec)
{
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t done = 0;
    if (vec) {
        const int64_t n16 = nbytes / 16;
        for (int64_t i = tid; i < n16; i += stride)
            store_stream(dst + i * 16, load_stream(src + i * 16));
        done = n16 * 16;
    }
    for (int64_t i = done + tid; i < nbytes; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_normproj(int64_t T, int64_t K, int64_t N, float eps, bool norm,
                           const void* x, int64_t ldx, const void* w, int64_t ldw, void* y,
                           int64_t ldy, hipStream_t st)
{
    if (T == 0 || N == 0) return hipSuccess;
    const float inv_k = (float)(1.0 / (double)K);
    const uint16_t* xp = (const uint16_t*)x;
    const uint16_t* wp = (const uint16_t*)w;
    uint16_t* yp = (uint16_t*)y;
    if (T <= kGemvMaxT) {
        const int64_t cols_per_block = (kThreads / kWave) * kGemvCols;
        const int64_t nblk = (N + cols_per_block - 1) / cols_per_block;
        if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
        if (norm)
            hipLaunchKernelGGL(normproj_gemv_kernel<true>, dim3((unsigned)nblk), dim3(kThreads), 0,
                               st, (int)T, K, N, eps, inv_k, xp, ldx, wp, ldw, yp, ldy);
        else
            hipLaunchKernelGGL(normproj_gemv_kernel<false>, dim3((unsigned)nblk), dim3(kThreads), 0,
                               st, (int)T, K, N, eps, inv_k, xp, ldx, wp, ldw, yp, ldy);
        return hipGetLastError();
    }
    const int64_t nbm = (T + kBM - 1) / kBM, nbn = (N + kBN - 1) / kBN;
    if (nbm * nbn > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(nbm * nbn));
    if (norm)
        hipLaunchKernelGGL(normproj_mfma_kernel<true>, grid, dim3(kThreads), 0, st, T, K, N, eps,
                           inv_k, xp, ldx, wp, ldw, yp, ldy, (int)nbm, (int)nbn);
    else
        hipLaunchKernelGGL(normproj_mfma_kernel<false>, grid, dim3(kThreads), 0, st, T, K, N, eps,
                           inv_k, xp, ldx, wp, ldw, yp, ldy, (int)nbm, (int)nbn);
    return hipGetLastError();
}

hipError_t launch_fold(int64_t K, int64_t N, const void* w, int64_t ldw, const void* gamma,
                       int gamma_bf16, void* w_fold, int64_t ldwf, hipStream_t st)
{
    if (K == 0 || N == 0) return hipSuccess;
    const int64_t gx = (N + 63) / 64, gy = (K + 63) / 64;
    if (gx > 0x7fffffff || gy > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fold_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0, st, K, N,
                       (const uint16_t*)w, ldw, gamma, gamma_bf16, (uint16_t*)w_fold, ldwf);
    return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, int64_t nbytes, hipStream_t st)
{
    if (nbytes == 0) return hipSuccess;
    const int vec = (((uintptr_t)dst | (uintptr_t)src) & 15u) == 0;
    int64_t nblk = (nbytes / 16 + kThreads - 1) / kThreads;
    if (nblk < 1) nblk = 1;
    if (nblk > 65536) nblk = 65536;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, st, (char*)dst,
                       (const char*)src, nbytes, vec);
    return hipGetLastError();
}

}  // namespace qkn
