// Norm-then-project on gfx950 with the RMS scale deferred to the product's output
// ("FlashNorm: Fast Normalization for Transformers", abstract, items (i) and (ii)), plus the
// one-time weight fold and a plain streaming copy used for calibration.
//
// y[t, n] = r_t * sum_k x[t, k] * w[n, k] with both operands K-contiguous (the fold writes W'
// transposed), on v_mfma_f32_32x32x16_bf16. The 1/rms factor comes from the same x values that
// feed the matrix cores, squared and summed on the VALU while the MFMAs run, so no extra pass
// over x is needed and the reduction proceeds beside the product instead of before it.
//
// Pipelined kernel (K a multiple of the k-tile, N of 8): a workgroup owns a BM x BN output tile.
// Its k-tiles of x and W' stream into an NST-deep LDS ring by direct global->LDS DMA
// (global_load_lds_dwordx4, 1 KB per wavefront instruction), NST-1 tiles ahead of the one being
// multiplied; each tile row's 16-byte chunks are XOR-swizzled so the fragment reads of 16
// consecutive rows fall in 16 distinct bank groups. Wavefronts own WM x WN sub-tiles of 32 x 32
// MFMA blocks; those in the first column also accumulate the rows' sums of squares from the x
// fragments they already hold. The epilogue scales by 1/rms, rounds to bf16 and stages the tile
// through LDS so each lane stores 16 contiguous bytes. Blocks are remapped so that each XCD
// works on a contiguous range of row panels (one L2 holds each x panel).
//
// Generic kernel (any K % 8 == 0, any N): 128 x 128 tiles through padded LDS rows with register
// staging of the next k-tile.
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

// ------------------------------------------------------------------------------------------
// Pipelined kernel.

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS at lds_off + 16 * lane. Issued through
// inline assembly so that the compiler does not wait for it before unrelated LDS reads; the
// kernel awaits completion with s_waitcnt vmcnt (vector loads complete in issue order). One
// wait state separates the M0 write from the DMA (a gfx9-family hazard). M0 is declared
// clobbered; no other instruction in these kernels uses it (checked in the generated code).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_off)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds_off)), "v"(gsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4] = 7 (no wait), lgkmcnt[11:8] = 15
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Physical 16-byte chunk of logical chunk kc in tile row r. ds_read_b128 is served 16 lanes
// (256 bytes, 64 banks) at a time and the fragment reads touch 16 consecutive rows at one
// logical chunk: rows of 128 B (k-tile 64) pair up per 256 B, so kc is xored with
// (r >> 1) & 7; rows of 64 B (k-tile 32) come four per 256 B: (r >> 2) & 3.
template <int BK>
__device__ __forceinline__ int swz(int kc, int r)
{
    return BK == 64 ? (kc ^ ((r >> 1) & 7)) : (kc ^ ((r >> 2) & 3));
}

template <int BM, int BN, int WM, int WN, int NST, int BK, bool NORM>
__global__ __launch_bounds__(WM * WN * 64) void normproj_pipe_kernel(
    int64_t T, int64_t K, int64_t N, float eps, float inv_k, const uint16_t* __restrict__ x,
    int64_t ldx, const uint16_t* __restrict__ w, int64_t ldw, uint16_t* __restrict__ y,
    int64_t ldy, int nbm, int nbn)
{
    constexpr int NW = WM * WN, NT = NW * kWave;
    constexpr int ROWB = BK * 2;            // bytes per tile row
    constexpr int RPC = 1024 / ROWB;        // tile rows per 1 KB DMA chunk
    constexpr int LPR = ROWB / 16;          // lanes per tile row within a chunk
    constexpr int STAGE_A = BM * ROWB, STAGE = (BM + BN) * ROWB;
    constexpr int CA = BM / RPC, CT = (BM + BN) / RPC;
    static_assert(CT % NW == 0, "DMA chunks must divide among the wavefronts");
    constexpr int CPW = CT / NW;            // DMA instructions per wavefront per k-tile
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int CP = BN + 8;              // epilogue tile pitch (bf16)
    constexpr int PIPE = NST * STAGE, CTILE = BM * CP * 2;
    constexpr int SMEM = PIPE > CTILE ? PIPE : CTILE;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];
    __shared__ float rs_lds[BM];

    const int tid = (int)threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;
    const int nb = nbm * nbn;
    int bid = (int)blockIdx.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    const int64_t m0 = (int64_t)(bid / nbn) * BM, n0 = (int64_t)(bid % nbn) * BN;

    // Source of each DMA chunk this lane fetches (fixed across k). Out-of-range rows are clamped
    // to the last valid row: they only feed output rows / columns that are never stored.
    const int lrow = lane / LPR;
    const uint16_t* src[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int chunk = wave * CPW + c;
        const int trow = (chunk < CA ? chunk : chunk - CA) * RPC + lrow;
        const int lkc = swz<BK>(lane % LPR, trow);  // the logical chunk landing at lane % LPR
        if (chunk < CA) {
            const int64_t r = m0 + trow < T ? m0 + trow : T - 1;
            src[c] = x + r * ldx + lkc * 8;
        } else {
            const int64_t r = n0 + trow < N ? n0 + trow : N - 1;
            src[c] = w + r * ldw + lkc * 8;
        }
    }
    auto issue = [&](int slot, int64_t k0) {
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int chunk = wave * CPW + c;
            char* dst = smem + slot * STAGE + chunk * 1024;
            dma16((const void*)(src[c] + k0), (uint32_t)(uintptr_t)(lds_void*)dst);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    float ssq[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) ssq[i] = 0.0f;

    const int nk = (int)(K / BK);
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nk) issue(s, (int64_t)s * BK);

    const int frow = lane & 31, fk = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        // k-tile kt must have landed; up to NST-2 later tiles stay in flight
        const int later = (nk - 1 - kt) < (NST - 2) ? (nk - 1 - kt) : (NST - 2);
        if constexpr (NST >= 4) {
            if (later >= 2) wait_vmcnt<2 * CPW>();
            else if (later == 1) wait_vmcnt<CPW>();
            else wait_vmcnt<0>();
        } else if constexpr (NST == 3) {
            if (later >= 1) wait_vmcnt<CPW>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();  // every wavefront's DMA has landed; slot (kt-1) % NST is free again
        if (kt + NST - 1 < nk) issue((kt + NST - 1) % NST, (int64_t)(kt + NST - 1) * BK);
        const char* As = smem + (kt % NST) * STAGE;
        const char* Bs = As + STAGE_A;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            u32x4 af[TM], bfr[TN];
            const int kc = ks * 2 + fk;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + frow;
                af[i] = *(const u32x4*)(As + r * ROWB + (swz<BK>(kc, r) << 4));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 32 + frow;
                bfr[j] = *(const u32x4*)(Bs + r * ROWB + (swz<BK>(kc, r) << 4));
            }
            if constexpr (NORM) {
                if (wn == 0) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        const u32x4 v = af[i];
                        float s = ssq[i];
                        s = fmaf(bf16_lo(v.x), bf16_lo(v.x), s); s = fmaf(bf16_hi(v.x), bf16_hi(v.x), s);
                        s = fmaf(bf16_lo(v.y), bf16_lo(v.y), s); s = fmaf(bf16_hi(v.y), bf16_hi(v.y), s);
                        s = fmaf(bf16_lo(v.z), bf16_lo(v.z), s); s = fmaf(bf16_hi(v.z), bf16_hi(v.z), s);
                        s = fmaf(bf16_lo(v.w), bf16_lo(v.w), s); s = fmaf(bf16_hi(v.w), bf16_hi(v.w), s);
                        ssq[i] = s;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
    }

    if constexpr (NORM) {
        // lanes l and l + 32 summed the two halves of each 16-wide k step of the same row
        if (wn == 0) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const float s = ssq[i] + __shfl_xor(ssq[i], 32);
                if (lane < 32) rs_lds[wm * WTM + i * 32 + lane] = rsqrtf(s * inv_k + eps);
            }
        }
    }
    __syncthreads();  // all DMA consumed (the last k-tile waited for vmcnt 0); 1/rms visible

    // accumulator layout of a 32 x 32 block: lane holds column lane % 32 and, for e in 0..15,
    // row 8 * (e / 4) + 4 * (lane / 32) + e % 4
    uint16_t* ct = (uint16_t*)smem;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = wm * WTM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int c = wn * WTN + j * 32 + (lane & 31);
                float v = acc[i][j][e];
                if constexpr (NORM) v *= rs_lds[r];
                ct[r * CP + c] = to_bf16(v);
            }
    __syncthreads();
    constexpr int C8 = BN / 8;
    for (int idx = tid; idx < BM * C8; idx += NT) {
        const int r = idx / C8, c8 = idx % C8;
        const int64_t gm = m0 + r, gn = n0 + c8 * 8;
        if (gm < T && gn < N) *(u32x4*)(y + gm * ldy + gn) = *(const u32x4*)(ct + r * CP + c8 * 8);
    }
}

// ------------------------------------------------------------------------------------------
// Generic kernel.

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

template <int BM, int BN, int WM, int WN, int NST, int BK>
hipError_t launch_pipe(int64_t T, int64_t K, int64_t N, float eps, float inv_k, bool norm,
                       const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                       uint16_t* y, int64_t ldy, hipStream_t st)
{
    const int64_t nbm = (T + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    if (nbm * nbn > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(nbm * nbn)), block(WM * WN * kWave);
    if (norm)
        hipLaunchKernelGGL((normproj_pipe_kernel<BM, BN, WM, WN, NST, BK, true>), grid, block, 0,
                           st, T, K, N, eps, inv_k, x, ldx, w, ldw, y, ldy, (int)nbm, (int)nbn);
    else
        hipLaunchKernelGGL((normproj_pipe_kernel<BM, BN, WM, WN, NST, BK, false>), grid, block, 0,
                           st, T, K, N, eps, inv_k, x, ldx, w, ldw, y, ldy, (int)nbm, (int)nbn);
    return hipGetLastError();
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
    const bool pipe_ok = N % 8 == 0 && ldy % 8 == 0 && ((uintptr_t)y & 15u) == 0;
    const int64_t big_tiles = ((T + 255) / 256) * ((N + 255) / 256);
    if (pipe_ok && K % 32 == 0 && big_tiles >= 512) {
        // many output tiles: 256 x 256 per workgroup of 8 wavefronts, k-tiles of 32, 4 stages
        return launch_pipe<256, 256, 4, 2, 4, 32>(T, K, N, eps, inv_k, norm, xp, ldx, wp, ldw, yp,
                                                  ldy, st);
    }
    if (pipe_ok && K % 64 == 0) {
        // 128 x 128 per workgroup of 4 wavefronts, k-tiles of 64, 2 stages (2 workgroups per CU)
        return launch_pipe<128, 128, 2, 2, 2, 64>(T, K, N, eps, inv_k, norm, xp, ldx, wp, ldw, yp,
                                                  ldy, st);
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
