// Row kernels for layerwise QK-Norm on gfx950: the fused launch (sum of squares, 1/rms and
// the gamma scale of Q and K rows in one launch), and the two halves of the scalar-statistics
// split (per-row partial sums of squares; aggregation of own + peers' partials followed by the
// scale). RMSNorm over a token's full Q / K vector is the operation of "SwiftQK: Fast and
// Communication-Efficient Tensor Parallelism for Query-Key Normalization" (abstract).
//
// Team path. A 256-thread workgroup is 4 wavefronts. A "team" of WPR wavefronts owns RR rows
// of one tensor; each lane of the team holds NVW 16-byte vectors of each row, so a row is read
// from HBM once, kept in registers, and written once. Per team the lane loads its gamma
// vectors first (cache hits), then the rows (non-temporal), sums squares in fp32, reduces
// across the wavefront with DPP row operations and four lane reads, and across the team's
// wavefronts through LDS in a fixed order; then it scales and stores what it still holds.
// Shapes keep the per-lane footprint at 1-3 vectors so that many wavefronts are in flight: wide
// rows are split over the 4 wavefronts of a workgroup, narrow rows get one wavefront (or
// several rows per wavefront for the read-mostly split kernels). Q and K are separate block
// ranges of one grid, each with its own shape.
//
// Generic path. One workgroup per row and two passes over it (the second re-reads the row,
// mostly from cache), 16-byte or element accesses. Used for misaligned tensors and for rows
// wider than 2048 vectors.
#pragma once

#include <utility>

#include "device.h"
#include "launch.h"

namespace qkn {

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * kWave;

// Team shapes, indexed by the smallest class whose capacity (vectors of 16 bytes per row)
// holds the row.
constexpr int kShapeCount = 7;
constexpr int kShapeWpr[kShapeCount] = {1, 2, 4, 4, 4, 4, 4};   // wavefronts per row
constexpr int kShapeNvw[kShapeCount] = {1, 1, 1, 2, 3, 4, 8};   // vectors per lane per row
constexpr int kShapeCap[kShapeCount] = {64, 128, 256, 512, 768, 1024, 2048};

// Rows per team: one, except for single-wavefront rows in the split kernels, which batch rows
// (4 for the read-only partial sums, 2 for aggregation + scale).
__host__ __device__ constexpr int shape_rr(int mode, int sh)
{
    return sh != 0 ? 1 : mode == kPartial ? 4 : mode == kApply ? 2 : 1;
}
__host__ __device__ constexpr int shape_rows_per_block(int mode, int sh)
{
    return (kWavesPerBlock / kShapeWpr[sh]) * shape_rr(mode, sh);
}

template <bool BF>
struct Io {
    static constexpr int kEpv = BF ? 8 : 4;   // elements per 16-byte vector
    static constexpr int kEs = BF ? 2 : 4;    // element size in bytes
};

template <bool BF>
__device__ __forceinline__ void unpack(const u32x4& v, float* f)
{
    if constexpr (BF) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    } else {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
}

template <bool BF>
__device__ __forceinline__ u32x4 pack(const float* f)
{
    u32x4 v;
    if constexpr (BF) {
        v.x = pack_bf16x2(f[0], f[1]);
        v.y = pack_bf16x2(f[2], f[3]);
        v.z = pack_bf16x2(f[4], f[5]);
        v.w = pack_bf16x2(f[6], f[7]);
    } else {
        v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
        v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
    }
    return v;
}

// gamma for the EPV columns of one 16-byte x vector, kept in registers as stored:
// kGv 16-byte words (bf16 x: 8 values = 16 B bf16 or 32 B fp32; fp32 x: 4 values = 8 B bf16
// or 16 B fp32).
template <bool BF, bool GBF>
struct Gamma {
    static constexpr int kEpv = Io<BF>::kEpv;
    static constexpr int kGv = (kEpv * (GBF ? 2 : 4) + 15) / 16;

    // col is a multiple of kEpv; gamma is 16-byte aligned.
    __device__ __forceinline__ static void load(const void* g, int64_t col, u32x4* raw)
    {
        if constexpr (GBF && !BF) {
            const u32x2 v = *(const u32x2*)((const uint16_t*)g + col);
            raw[0] = u32x4{v.x, v.y, 0u, 0u};
        } else if constexpr (GBF) {
            raw[0] = *(const u32x4*)((const uint16_t*)g + col);
        } else {
#pragma unroll
            for (int h = 0; h < kGv; ++h) raw[h] = *(const u32x4*)((const float*)g + col + 4 * h);
        }
    }

    __device__ __forceinline__ static uint32_t word(const u32x4& v, int c)
    {
        return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
    }

    // value e (a compile-time constant after unrolling) of the EPV held in raw
    __device__ __forceinline__ static float at(const u32x4* raw, int e)
    {
        if constexpr (GBF) {
            const uint32_t w = word(raw[0], e >> 1);
            return (e & 1) ? bf16_hi(w) : bf16_lo(w);
        } else {
            return __uint_as_float(word(raw[e >> 2], e & 3));
        }
    }
};

// The rows of block `blk` of one tensor under team shape SH; NTS: non-temporal output stores.
// FULL: the row width fills the shape exactly (d == kShapeCap[SH] * EPV), so no vector is past
// the end of the row and the loads and stores need no column mask.
template <int MODE, bool BF, bool GBF, int SH, bool NTS, bool FULL>
__device__ __forceinline__ void run_team(const RowSeg& s, int64_t T, float eps, int64_t blk,
                                         float* red)
{
    constexpr int WPR = kShapeWpr[SH];
    constexpr int NVW = kShapeNvw[SH];
    constexpr int RR = shape_rr(MODE, SH);
    constexpr int TEAMS = kWavesPerBlock / WPR;
    constexpr int EPV = Io<BF>::kEpv;
    constexpr int ES = Io<BF>::kEs;
    using G = Gamma<BF, GBF>;

    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int tm = wave / WPR, wt = wave % WPR;
    const int64_t row0 = (blk * TEAMS + tm) * RR;
    // with one row per workgroup the grid has exactly T blocks: every row exists
    constexpr bool kRowsExact = TEAMS * RR == 1;
    auto col_in = [&](int64_t col) { return FULL || col < s.d; };
    auto row_in = [&](int r) { return kRowsExact || row0 + r < T; };

    // gamma first: its cache hits are back before the row loads are.
    u32x4 graw[NVW][G::kGv];
    if constexpr (MODE != kPartial) {
#pragma unroll
        for (int j = 0; j < NVW; ++j) {
            const int64_t col = (int64_t)((wt * NVW + j) * kWave + lane) * EPV;
            if (col_in(col)) {
                G::load(s.g, col, graw[j]);
            } else {
#pragma unroll
                for (int h = 0; h < G::kGv; ++h) graw[j][h] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }

    // Own + peers' statistics of row row0 + lane (lanes 0..RR-1): the own partial and the first
    // 8 peers are loaded before the rows, so all of them are in flight together.
    constexpr int kPeerChunk = 8;
    const bool stat_lane = lane < RR && row0 + lane < T;
    float own = 0.0f, peer[kPeerChunk];
    if constexpr (MODE == kApply) {
#pragma unroll
        for (int u = 0; u < kPeerChunk; ++u) peer[u] = 0.0f;
        if (stat_lane) {
            const int64_t t = row0 + lane;
            own = s.psq_in[t];
#pragma unroll
            for (int u = 0; u < kPeerChunk; ++u)
                if (u < s.n_ext) peer[u] = s.ext[u * s.ld_ext + t];
        }
    }

    u32x4 v[RR][NVW];
#pragma unroll
    for (int r = 0; r < RR; ++r) {
        const bool row_ok = row_in(r);
        const char* xr = (const char*)s.x + (row0 + r) * s.ldx * ES;
#pragma unroll
        for (int j = 0; j < NVW; ++j) {
            const int64_t col = (int64_t)((wt * NVW + j) * kWave + lane) * EPV;
            v[r][j] = (row_ok && col_in(col)) ? load_stream(xr + col * ES) : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // S = own + peer 0 + peer 1 + ... in that order (fp32)
    float S = 0.0f;
    if constexpr (MODE == kApply) {
        S = own;
#pragma unroll
        for (int u = 0; u < kPeerChunk; ++u)
            if (u < s.n_ext) S += peer[u];
        if (stat_lane) {
            const int64_t t = row0 + lane;
            for (int64_t e = kPeerChunk; e < s.n_ext; ++e) S += s.ext[e * s.ld_ext + t];
        }
    }

    float rs[RR];
    if constexpr (MODE != kApply) {
        float tot[RR];
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int j = 0; j < NVW; ++j) {
                if constexpr (BF) {
                    // two bf16 per instruction, squares exact, one rounding per pair
                    a0 = sumsq_bf16x2(v[r][j].x, a0);
                    a1 = sumsq_bf16x2(v[r][j].y, a1);
                    a0 = sumsq_bf16x2(v[r][j].z, a0);
                    a1 = sumsq_bf16x2(v[r][j].w, a1);
                } else {
                    float f[EPV];
                    unpack<BF>(v[r][j], f);
#pragma unroll
                    for (int e = 0; e < EPV; e += 2) {
                        a0 = fmaf(f[e], f[e], a0);
                        a1 = fmaf(f[e + 1], f[e + 1], a1);
                    }
                }
            }
            tot[r] = wave_sum(a0 + a1);
        }
        if constexpr (WPR > 1) {
            if (lane == 0) {
#pragma unroll
                for (int r = 0; r < RR; ++r) red[(tm * RR + r) * WPR + wt] = tot[r];
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                float t = 0.0f;
#pragma unroll
                for (int w = 0; w < WPR; ++w) t += red[(tm * RR + r) * WPR + w];
                tot[r] = t;
            }
        }
        if constexpr (MODE == kPartial) {
            if (wt == 0) {
                float o = tot[0];
#pragma unroll
                for (int r = 1; r < RR; ++r) o = (lane == r) ? tot[r] : o;
                if (lane < RR && row0 + lane < T) s.psq_out[row0 + lane] = o;
            }
            return;
        }
#pragma unroll
        for (int r = 0; r < RR; ++r) rs[r] = rsqrtf(tot[r] * s.inv_dfull + eps);
    } else {
        const float rl = rsqrtf(S * s.inv_dfull + eps);
#pragma unroll
        for (int r = 0; r < RR; ++r) rs[r] = lane_read(rl, r);
    }

    if constexpr (MODE != kPartial) {
        // Keep the rows packed across the reduction; otherwise the compiler keeps the fp32
        // values widened for the sum of squares alive and doubles the register footprint.
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int j = 0; j < NVW; ++j) asm volatile("" : "+v"(v[r][j]));

#pragma unroll
        for (int r = 0; r < RR; ++r) {
            if (row_in(r)) {
                char* yr = (char*)s.y + (row0 + r) * s.ldy * ES;
#pragma unroll
                for (int j = 0; j < NVW; ++j) {
                    const int64_t col = (int64_t)((wt * NVW + j) * kWave + lane) * EPV;
                    if (col_in(col)) {
                        float f[EPV], o[EPV];
                        unpack<BF>(v[r][j], f);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) o[e] = (f[e] * G::at(graw[j], e)) * rs[r];
                        if constexpr (NTS) store_stream(yr + col * ES, pack<BF>(o));
                        else *(u32x4*)(yr + col * ES) = pack<BF>(o);
                    }
                }
            }
        }
    }
}

// Row block handled by the i-th of n workgroups of one tensor. Aggregation + scale reads the
// own and the peers' partials, 4 bytes per row each: a 128-byte line of them spans G row
// blocks. Workgroup i runs on XCD i % 8 (the tensors' block ranges start at multiples of 8
// when the rows fill whole groups), so within each group of 8 G workgroups those on one XCD
// take G consecutive blocks: each line of partials is then fetched into one L2 only. The other
// modes read no partials and keep the plain order.
template <int MODE, int SH>
__device__ __forceinline__ int64_t block_order(int64_t i, int64_t n)
{
    if constexpr (MODE != kApply) {
        return i;
    } else {
        constexpr int G = 32 / shape_rows_per_block(MODE, SH);
        const int64_t full = n / (8 * G) * (8 * G);
        if (i >= full) return i;
        const int r = (int)(i % (8 * G));
        return i - r + (r & 7) * G + (r >> 3);
    }
}

// Blocks [0, nblk0) serve seg[0] with shape SH0, the rest seg[1] with shape SH1; FULL: both
// tensors' widths fill their shapes exactly.
template <int MODE, bool BF, bool GBF, int SH0, int SH1, bool NTS = true, bool FULL = false>
__global__ __launch_bounds__(kBlock) void rows_team_kernel(RowJob job, int nblk0)
{
    __shared__ float red[32];
    const int b = (int)blockIdx.x;
    if (b < nblk0)
        run_team<MODE, BF, GBF, SH0, NTS, FULL>(job.seg[0], job.T, job.eps,
                                                block_order<MODE, SH0>(b, nblk0), red);
    else
        run_team<MODE, BF, GBF, SH1, NTS, FULL>(job.seg[1], job.T, job.eps,
                                                block_order<MODE, SH1>(b - nblk0,
                                                                       (int)gridDim.x - nblk0),
                                                red);
}

// ------------------------------------------------------------------------------------------
// Generic path: one workgroup per row, two passes.

template <bool BF>
__device__ __forceinline__ float load_elem(const void* p, int64_t i)
{
    if constexpr (BF) return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
    else return ((const float*)p)[i];
}

template <bool BF>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v)
{
    if constexpr (BF) ((uint16_t*)p)[i] = to_bf16(v);
    else ((float*)p)[i] = v;
}

template <int MODE, bool BF, bool GBF, bool VEC>
__global__ __launch_bounds__(kBlock) void rows_generic_kernel(RowJob job)
{
    constexpr int EPV = Io<BF>::kEpv;
    constexpr int ES = Io<BF>::kEs;
    __shared__ float red[kWavesPerBlock];
    __shared__ float total;

    const int64_t b = blockIdx.x;
    const bool second = b >= job.T;
    const RowSeg s = second ? job.seg[1] : job.seg[0];
    const int64_t row = second ? b - job.T : b;
    const char* xr = (const char*)s.x + row * s.ldx * ES;
    const int tid = (int)threadIdx.x;

    float S = 0.0f;
    if constexpr (MODE != kApply) {
        float a = 0.0f;
        if constexpr (VEC) {
            for (int64_t col = (int64_t)tid * EPV; col < s.d; col += (int64_t)kBlock * EPV) {
                float f[EPV];
                unpack<BF>(*(const u32x4*)(xr + col * ES), f);
#pragma unroll
                for (int e = 0; e < EPV; ++e) a = fmaf(f[e], f[e], a);
            }
        } else {
            for (int64_t col = tid; col < s.d; col += kBlock) {
                const float f = load_elem<BF>(xr, col);
                a = fmaf(f, f, a);
            }
        }
        a = wave_sum(a);
        if (lane_id() == 0) red[tid / kWave] = a;
        __syncthreads();
        if (tid == 0) total = (red[0] + red[1]) + (red[2] + red[3]);
        __syncthreads();
        S = total;
        if constexpr (MODE == kPartial) {
            if (tid == 0) s.psq_out[row] = S;
            return;
        }
    } else {
        S = s.psq_in[row];
        for (int64_t e = 0; e < s.n_ext; ++e) S += s.ext[e * s.ld_ext + row];
    }

    if constexpr (MODE != kPartial) {
        const float rs = rsqrtf(S * s.inv_dfull + job.eps);
        char* yr = (char*)s.y + row * s.ldy * ES;
        if constexpr (VEC) {
            for (int64_t col = (int64_t)tid * EPV; col < s.d; col += (int64_t)kBlock * EPV) {
                float f[EPV], o[EPV];
                u32x4 graw[Gamma<BF, GBF>::kGv];
                unpack<BF>(*(const u32x4*)(xr + col * ES), f);
                Gamma<BF, GBF>::load(s.g, col, graw);
#pragma unroll
                for (int e = 0; e < EPV; ++e) o[e] = (f[e] * Gamma<BF, GBF>::at(graw, e)) * rs;
                *(u32x4*)(yr + col * ES) = pack<BF>(o);
            }
        } else {
            for (int64_t col = tid; col < s.d; col += kBlock) {
                const float f = load_elem<BF>(xr, col);
                store_elem<BF>(yr, col, (f * load_elem<GBF>(s.g, col)) * rs);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Host-side selection for one (x storage, gamma storage) pair.

typedef hipError_t (*RowLaunch)(const RowJob&, hipStream_t);

template <int MODE, bool BF, bool GBF, int SH0, int SH1, bool NTS = true, bool FULL = false>
hipError_t launch_team(const RowJob& job, hipStream_t st)
{
    const int64_t per0 = shape_rows_per_block(MODE, SH0);
    const int64_t per1 = shape_rows_per_block(MODE, SH1);
    const int64_t nblk0 = (job.T + per0 - 1) / per0;
    const int64_t nblk1 = job.nseg > 1 ? (job.T + per1 - 1) / per1 : 0;
    if (nblk0 + nblk1 > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rows_team_kernel<MODE, BF, GBF, SH0, SH1, NTS, FULL>),
                       dim3((unsigned)(nblk0 + nblk1)), dim3(kBlock), 0, st, job, (int)nblk0);
    return hipGetLastError();
}

template <int MODE, bool BF, bool GBF, int I, int... J>
RowLaunch pick_second(int j, std::integer_sequence<int, J...>)
{
    RowLaunch r = nullptr;
    ((j == J ? (r = launch_team<MODE, BF, GBF, I, J>, 0) : 0), ...);
    return r;
}

// Fused launches: every pair (i >= j) of shapes; the caller orders the segments so that the
// first has the larger shape. Split launches use one shape (the larger) for both tensors. When
// both tensors share one shape and fill it exactly (full), the unmasked instantiation runs.
template <int MODE, bool BF, bool GBF, int... I>
RowLaunch pick_team(int i, int j, bool full, std::integer_sequence<int, I...>)
{
    RowLaunch r = nullptr;
    if constexpr (MODE != kApply) {
        if (full && i == j) {
            ((i == I ? (r = launch_team<MODE, BF, GBF, I, I, true, true>, 0) : 0), ...);
            return r;
        }
    }
    if constexpr (MODE == kFused) {
        ((i == I ? (r = pick_second<MODE, BF, GBF, I>(j, std::make_integer_sequence<int, I + 1>{}),
                    0)
                 : 0),
         ...);
    } else {
        ((i == I ? (r = launch_team<MODE, BF, GBF, I, I>, 0) : 0), ...);
    }
    return r;
}

// One-tensor fused jobs whose output the caller reads back: ordinary stores.
template <bool BF, bool GBF, int... I>
RowLaunch pick_cached(int i, std::integer_sequence<int, I...>)
{
    RowLaunch r = nullptr;
    ((i == I ? (r = launch_team<kFused, BF, GBF, I, I, false>, 0) : 0), ...);
    return r;
}

template <int MODE, bool BF, bool GBF, bool VEC>
hipError_t launch_generic(const RowJob& job, hipStream_t st)
{
    const int64_t nblk = job.T * job.nseg;
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rows_generic_kernel<MODE, BF, GBF, VEC>), dim3((unsigned)nblk),
                       dim3(kBlock), 0, st, job);
    return hipGetLastError();
}

inline bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

// Smallest team shape holding d columns, or -1 if the row is wider than every shape.
inline int shape_class(int64_t d, int epv)
{
    const int64_t vectors = (d + epv - 1) / epv;
    for (int i = 0; i < kShapeCount; ++i)
        if (vectors <= kShapeCap[i]) return i;
    return -1;
}

template <int MODE, bool BF, bool GBF>
hipError_t dispatch_mode(const RowJob& job_in, hipStream_t st)
{
    constexpr int EPV = Io<BF>::kEpv;
    constexpr int ES = Io<BF>::kEs;
    RowJob job = job_in;
    bool vec = true, fits = true;
    int cls[2] = {0, 0};
    for (int i = 0; i < job.nseg; ++i) {
        const RowSeg& s = job.seg[i];
        vec = vec && aligned16(s.x) && (s.ldx * ES) % 16 == 0 && s.d % EPV == 0;
        if (MODE != kPartial)
            vec = vec && aligned16(s.y) && (s.ldy * ES) % 16 == 0 && aligned16(s.g);
        cls[i] = shape_class(s.d, EPV);
        fits = fits && cls[i] >= 0;
    }
    if (!vec) return launch_generic<MODE, BF, GBF, false>(job, st);
    if (!fits) return launch_generic<MODE, BF, GBF, true>(job, st);
    if (job.nseg == 1) {
        cls[1] = cls[0];
    } else if (cls[1] > cls[0]) {  // the tensors are independent: put the wider one first
        const RowSeg t = job.seg[0];
        job.seg[0] = job.seg[1];
        job.seg[1] = t;
        const int c = cls[0];
        cls[0] = cls[1];
        cls[1] = c;
    }
    const int i = cls[0], j = MODE == kFused ? cls[1] : cls[0];
    // (aggregation + scale keeps the masked form: unmasked it measured 6% slower)
    bool full = MODE != kApply;
    for (int t = 0; t < job.nseg; ++t) full = full && job.seg[t].d == (int64_t)kShapeCap[i] * EPV;
    if constexpr (MODE == kFused) {
        if (job.nseg == 1 && job.keep_cached) {
            RowLaunch f = pick_cached<BF, GBF>(i, std::make_integer_sequence<int, kShapeCount>{});
            return f ? f(job, st) : hipErrorInvalidValue;
        }
    }
    RowLaunch f = pick_team<MODE, BF, GBF>(i, j, full,
                                           std::make_integer_sequence<int, kShapeCount>{});
    return f ? f(job, st) : hipErrorInvalidValue;
}

// Defined (explicitly instantiated) in rows_inst.hip, once per storage pair.
template <bool BF, bool GBF>
hipError_t dispatch_rows(const RowJob& job, hipStream_t st);

}  // namespace qkn
