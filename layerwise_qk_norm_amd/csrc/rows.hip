// Row kernels for layerwise QK-Norm on gfx950: the fused launch (sum of squares, 1/rms and
// the gamma scale of Q and K rows in one launch), and the two halves of the scalar-statistics
// split (per-row partial sums of squares; aggregation of own + peers' partials followed by
// the scale). RMSNorm over a token's full Q / K vector is the operation of "SwiftQK: Fast and
// Communication-Efficient Tensor Parallelism for Query-Key Normalization" (abstract).
//
// Register path: one wavefront owns R rows (R*NV 16-byte vectors per lane). It issues all of
// its loads, sums squares in fp32 per lane, reduces across the wave with DPP row operations and
// four lane reads, and scales and stores the rows it still holds in registers, so each element
// is read from HBM once and written once. Workgroups are 4 independent wavefronts: no LDS and
// no barriers.
//
// Generic path: one workgroup per row, two passes over the row (the second pass re-reads it,
// mostly from cache), element or 16-byte accesses. Used for misaligned tensors and for rows
// wider than the register path holds.

#include "device.h"
#include "launch.h"

namespace qkn {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * kWave;

// Rows per wavefront for a given number of 16-byte vectors per lane and row: narrow rows are
// batched so that every lane keeps about 8 vectors in flight.
__host__ __device__ constexpr int rows_for(int nv) { return nv >= 8 ? 1 : 8 / nv; }

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

// gamma[col .. col+EPV) as fp32; col is a multiple of EPV and gamma is 16-byte aligned.
template <int EPV>
__device__ __forceinline__ void load_gamma(const void* g, int gamma_bf16, int64_t col, float* out)
{
    if (gamma_bf16) {
        const uint16_t* p = (const uint16_t*)g + col;
        if constexpr (EPV == 8) {
            u32x4 v = *(const u32x4*)p;
            unpack<true>(v, out);
        } else {
            u32x2 v = *(const u32x2*)p;
            out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
            out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
        }
    } else {
        const f32x4* p = (const f32x4*)((const float*)g + col);
#pragma unroll
        for (int h = 0; h < EPV / 4; ++h) {
            f32x4 v = p[h];
            out[4 * h + 0] = v.x; out[4 * h + 1] = v.y;
            out[4 * h + 2] = v.z; out[4 * h + 3] = v.w;
        }
    }
}

// One wavefront, rows [row0, row0 + R) of one tensor, NV 16-byte vectors per lane and row.
template <int MODE, bool BF, int NV, int R>
__device__ __forceinline__ void run_group(const RowSeg& s, int64_t T, float eps, int gamma_bf16,
                                          int64_t row0)
{
    constexpr int EPV = Io<BF>::kEpv;
    constexpr int ES = Io<BF>::kEs;
    const int lane = lane_id();

    // Own + peers' statistics for row row0 + lane (lanes 0..R-1), issued first.
    float S = 0.0f;
    if constexpr (MODE == kApply) {
        if (lane < R && row0 + lane < T) {
            const int64_t t = row0 + lane;
            S = s.psq_in[t];
#pragma unroll 8
            for (int64_t e = 0; e < s.n_ext; ++e) S += s.ext[e * s.ld_ext + t];
        }
    }

    u32x4 v[R][NV];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool row_ok = row0 + r < T;
        const char* xr = (const char*)s.x + (row0 + r) * s.ldx * ES;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t col = (int64_t)(j * kWave + lane) * EPV;
            v[r][j] = (row_ok && col < s.d) ? load_stream(xr + col * ES) : u32x4{0u, 0u, 0u, 0u};
        }
    }

    float ss[R];
    if constexpr (MODE != kApply) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                float f[EPV];
                unpack<BF>(v[r][j], f);
#pragma unroll
                for (int e = 0; e < EPV; e += 2) {
                    a0 = fmaf(f[e], f[e], a0);
                    a1 = fmaf(f[e + 1], f[e + 1], a1);
                }
            }
            ss[r] = wave_sum(a0 + a1);
        }
    }

    if constexpr (MODE == kPartial) {
        float o = ss[0];
#pragma unroll
        for (int r = 1; r < R; ++r) o = (lane == r) ? ss[r] : o;
        if (lane < R && row0 + lane < T) s.psq_out[row0 + lane] = o;
        return;
    } else {
        float rs[R];
        if constexpr (MODE == kFused) {
#pragma unroll
            for (int r = 0; r < R; ++r) rs[r] = rsqrtf(ss[r] * s.inv_dfull + eps);
        } else {
            const float rl = rsqrtf(S * s.inv_dfull + eps);
#pragma unroll
            for (int r = 0; r < R; ++r) rs[r] = lane_read(rl, r);
        }

#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t col = (int64_t)(j * kWave + lane) * EPV;
            if (col < s.d) {
                float g[EPV];
                load_gamma<EPV>(s.g, gamma_bf16, col, g);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (row0 + r < T) {
                        float f[EPV], o[EPV];
                        unpack<BF>(v[r][j], f);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) o[e] = (f[e] * g[e]) * rs[r];
                        store_stream((char*)s.y + ((row0 + r) * s.ldy + col) * ES, pack<BF>(o));
                    }
                }
            }
        }
    }
}

// Blocks [0, nblk_q) serve seg[0] (Q), the rest seg[1] (K); each wavefront one row group.
template <int MODE, bool BF, int NVQ, int NVK>
__global__ __launch_bounds__(kBlock) void rows_kernel(RowJob job, int64_t nblk_q)
{
    constexpr int RQ = rows_for(NVQ);
    constexpr int RK = rows_for(NVK);
    const int wave = (int)(threadIdx.x / kWave);
    if ((int64_t)blockIdx.x < nblk_q) {
        const int64_t group = (int64_t)blockIdx.x * kWavesPerBlock + wave;
        if (group * RQ >= job.T) return;
        run_group<MODE, BF, NVQ, RQ>(job.seg[0], job.T, job.eps, job.gamma_bf16, group * RQ);
    } else {
        const int64_t group = ((int64_t)blockIdx.x - nblk_q) * kWavesPerBlock + wave;
        if (group * RK >= job.T) return;
        run_group<MODE, BF, NVK, RK>(job.seg[1], job.T, job.eps, job.gamma_bf16, group * RK);
    }
}

// ------------------------------------------------------------------------------------------
// Generic path: one workgroup per row, two passes.

template <bool BF>
__device__ __forceinline__ float load_elem(const void* p, int64_t i)
{
    if constexpr (BF) return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
    else return ((const float*)p)[i];
}

__device__ __forceinline__ float load_gamma_elem(const void* g, int gamma_bf16, int64_t i)
{
    return gamma_bf16 ? __uint_as_float((uint32_t)((const uint16_t*)g)[i] << 16)
                      : ((const float*)g)[i];
}

template <bool BF>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v)
{
    if constexpr (BF) ((uint16_t*)p)[i] = to_bf16(v);
    else ((float*)p)[i] = v;
}

template <int MODE, bool BF, bool VEC>
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

    const float rs = rsqrtf(S * s.inv_dfull + job.eps);
    char* yr = (char*)s.y + row * s.ldy * ES;
    if constexpr (VEC) {
        for (int64_t col = (int64_t)tid * EPV; col < s.d; col += (int64_t)kBlock * EPV) {
            float f[EPV], g[EPV], o[EPV];
            unpack<BF>(*(const u32x4*)(xr + col * ES), f);
            load_gamma<EPV>(s.g, job.gamma_bf16, col, g);
#pragma unroll
            for (int e = 0; e < EPV; ++e) o[e] = (f[e] * g[e]) * rs;
            *(u32x4*)(yr + col * ES) = pack<BF>(o);
        }
    } else {
        for (int64_t col = tid; col < s.d; col += kBlock) {
            const float f = load_elem<BF>(xr, col);
            store_elem<BF>(yr, col, (f * load_gamma_elem(s.g, job.gamma_bf16, col)) * rs);
        }
    }
}

// ------------------------------------------------------------------------------------------
// Dispatch.

constexpr int kNvMenu[] = {1, 2, 4, 8, 16};
constexpr int kNvCount = 5;

typedef hipError_t (*RegLaunch)(const RowJob&, hipStream_t);

template <int MODE, bool BF, int NVQ, int NVK>
hipError_t launch_reg(const RowJob& job, hipStream_t st)
{
    constexpr int RQ = rows_for(NVQ);
    constexpr int RK = rows_for(NVK);
    const int64_t groups_q = (job.T + RQ - 1) / RQ;
    const int64_t groups_k = job.nseg > 1 ? (job.T + RK - 1) / RK : 0;
    const int64_t nblk_q = (groups_q + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t nblk_k = (groups_k + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t nblk = nblk_q + nblk_k;
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rows_kernel<MODE, BF, NVQ, NVK>), dim3((unsigned)nblk), dim3(kBlock), 0,
                       st, job, nblk_q);
    return hipGetLastError();
}

template <int MODE, bool BF, int IQ>
struct RowTable {
    static constexpr RegLaunch row[kNvCount] = {
        launch_reg<MODE, BF, kNvMenu[IQ], 1>, launch_reg<MODE, BF, kNvMenu[IQ], 2>,
        launch_reg<MODE, BF, kNvMenu[IQ], 4>, launch_reg<MODE, BF, kNvMenu[IQ], 8>,
        launch_reg<MODE, BF, kNvMenu[IQ], 16>};
};

// Fused launches get every (Q width, K width) pair; the split's launches use one width class
// for both tensors (the larger), which keeps the instantiation count small.
template <int MODE, bool BF>
RegLaunch pick_reg(int iq, int ik)
{
    if constexpr (MODE == kFused) {
        switch (iq) {
        case 0: return RowTable<MODE, BF, 0>::row[ik];
        case 1: return RowTable<MODE, BF, 1>::row[ik];
        case 2: return RowTable<MODE, BF, 2>::row[ik];
        case 3: return RowTable<MODE, BF, 3>::row[ik];
        default: return RowTable<MODE, BF, 4>::row[ik];
        }
    } else {
        switch (iq > ik ? iq : ik) {
        case 0: return launch_reg<MODE, BF, 1, 1>;
        case 1: return launch_reg<MODE, BF, 2, 2>;
        case 2: return launch_reg<MODE, BF, 4, 4>;
        case 3: return launch_reg<MODE, BF, 8, 8>;
        default: return launch_reg<MODE, BF, 16, 16>;
        }
    }
}

template <int MODE, bool BF, bool VEC>
hipError_t launch_generic(const RowJob& job, hipStream_t st)
{
    const int64_t nblk = job.T * job.nseg;
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((rows_generic_kernel<MODE, BF, VEC>), dim3((unsigned)nblk), dim3(kBlock),
                       0, st, job);
    return hipGetLastError();
}

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

// Index into kNvMenu of the smallest width class holding d columns, or -1 if none does.
int width_class(int64_t d, int epv)
{
    const int64_t per_vec = (int64_t)kWave * epv;
    const int64_t nv = (d + per_vec - 1) / per_vec;
    for (int i = 0; i < kNvCount; ++i)
        if (nv <= kNvMenu[i]) return i;
    return -1;
}

template <int MODE, bool BF>
hipError_t dispatch(const RowJob& job, hipStream_t st)
{
    constexpr int EPV = Io<BF>::kEpv;
    constexpr int ES = Io<BF>::kEs;
    bool vec = true;
    int cls[2] = {0, 0};
    bool fits = true;
    for (int i = 0; i < job.nseg; ++i) {
        const RowSeg& s = job.seg[i];
        vec = vec && aligned16(s.x) && (s.ldx * ES) % 16 == 0 && s.d % EPV == 0;
        if (MODE != kPartial)
            vec = vec && aligned16(s.y) && (s.ldy * ES) % 16 == 0 && aligned16(s.g);
        cls[i] = width_class(s.d, EPV);
        fits = fits && cls[i] >= 0;
    }
    if (job.nseg == 1) cls[1] = cls[0];
    if (vec && fits) return pick_reg<MODE, BF>(cls[0], cls[1])(job, st);
    if (vec) return launch_generic<MODE, BF, true>(job, st);
    return launch_generic<MODE, BF, false>(job, st);
}

}  // namespace

hipError_t launch_rows(const RowJob& job, hipStream_t stream)
{
    if (job.T == 0) return hipSuccess;
    switch (job.mode) {
    case kFused:
        return job.bf16 ? dispatch<kFused, true>(job, stream) : dispatch<kFused, false>(job, stream);
    case kPartial:
        return job.bf16 ? dispatch<kPartial, true>(job, stream)
                        : dispatch<kPartial, false>(job, stream);
    default:
        return job.bf16 ? dispatch<kApply, true>(job, stream) : dispatch<kApply, false>(job, stream);
    }
}

}  // namespace qkn
