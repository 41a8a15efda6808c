// Single-launch shard stage of layerwise QK-Norm under tensor parallelism: one pass over this
// rank's column slice computes the per-row partial sums of squares, publishes them, waits for
// the peers' partials, aggregates, and scales the slice it still holds in registers ("SwiftQK:
// Fast and Communication-Efficient Tensor Parallelism for Query-Key Normalization", abstract:
// ranks exchange per-row scalars only, and the wait for the peers' scalars is hidden behind
// element-wise work in one persistent kernel that cannot deadlock). Compared with the two
// launches (partial sums, then aggregation + scale) x is read once instead of twice.
//
// Mailbox. Every exchanged partial travels as one 8-byte word: the epoch of the pass in the
// upper half, the fp32 value in the lower half, stored and loaded as a single aligned 64-bit
// access. A reader that sees its epoch in a word has that word's value, so there is no
// separate flag, no wait for store acknowledgements and no workgroup barrier. Because tag and
// value can only change together, even a plain, possibly stale cached load is safe to accept
// when it shows the current epoch: the first look at the mailbox is an ordinary load in flight
// beside the row loads, and only a word that shows an older epoch is polled again, with
// device-scope coherent loads that go through to memory across the XCDs (so a stale line can
// only cost a re-poll, never a wrong value or an endless wait). Words are published with
// device-scope coherent stores. A release/acquire pair would instead write back and
// invalidate whole L2 caches. One GPU simulates its peers with shard_publish_kernel, which
// writes the same words.
//
// Deadlock safety. A reader waits only on data that other work produces, and every wait is
// bounded (max_spin polls, after which the kernel records a timeout and finishes), so it never
// hangs. The grid is always one workgroup per row block, dispatched in ascending order. Two
// residency policies: `persistent` (the name of the flag; no workgroup loops), where every
// workgroup reserves LDS it does not use so that at most three quarters of the workgroups the
// registers allow are resident on a CU at once, leaving a quarter of the slots (and of the LDS)
// to a producer launched on another stream of the same device, provided that stream is not
// queued behind this kernel: HIP maps streams onto a few hardware queues, and two streams that
// share one run their work in submission order, so a producer submitted after the pass to the
// same queue cannot start before it ends (the pass then waits out max_spin and reports the
// timeout); or no reservation, for producers that do not run on this device (the peers under
// tensor parallelism), where progress rests on every rank dispatching row blocks in the same
// ascending order, so that the lowest unfinished block is resident, and has been published,
// everywhere.

#include <atomic>

#include "rows_impl.h"

namespace qkn {
namespace {

constexpr int kShardRowsPerWave = 4;
constexpr int kShardItemRows = kWavesPerBlock * kShardRowsPerWave;  // rows per workgroup item
constexpr int kPeersPerGroup = kWave / kShardRowsPerWave;           // mailbox words per lane pass
constexpr int kMaxPeerGroups = 4;                                   // n_ext <= 64

// kernel-argument view of one tensor's slice
struct ShardTensor {
    const void* x;
    void* y;
    const void* g;
    int64_t ldx, ldy, d;
    float inv_dfull;
    uint64_t* psq_out;     // [T] tagged words, or null
    const uint64_t* mail;  // [n_ext][ld_mail] tagged words
    int64_t ld_mail;
};

struct ShardJob {
    ShardTensor t[2];
    int nseg;
    int64_t T, nib, n_ext;  // nib: row blocks per tensor
    float eps;
    uint32_t epoch;         // 0: the mailbox is complete before launch, tags are not checked
    int persistent;         // 1: at most 3/4 of the resident workgroups at once
    int64_t max_spin;
    int* timed_out;
};

__device__ __forceinline__ uint64_t tagged(float v, uint32_t epoch)
{
    return ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(v);
}

// Registers of one workgroup item in flight: the wavefront's rows and its first look at the
// mailbox words of those rows.
template <int NV, int NG>
struct ShardItem {
    u32x4 v[kShardRowsPerWave][NV];
    uint64_t mw[NG];
    bool mine[NG];
};

// Element accesses for slices the 16-byte vectors cannot serve (a pointer or a row stride off
// 16 bytes, or a width that is not a whole number of vectors): the EPV elements a lane owns,
// one at a time, those at or past d read as 0 and not written. The packing is that of the
// vector path, so the arithmetic is shared.
template <bool BF>
__device__ __forceinline__ u32x4 load_elems(const char* row, int64_t col, int64_t d)
{
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if constexpr (BF) {
        const uint16_t* p = (const uint16_t*)row;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col + e < d)
                w[e >> 1] |= (uint32_t)__builtin_nontemporal_load(p + col + e) << (16 * (e & 1));
    } else {
        const uint32_t* p = (const uint32_t*)row;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (col + e < d) w[e] = __builtin_nontemporal_load(p + col + e);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

template <bool BF>
__device__ __forceinline__ void store_elems(char* row, int64_t col, int64_t d, const u32x4& v)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (BF) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col + e < d)
                __builtin_nontemporal_store((uint16_t)(w[e >> 1] >> (16 * (e & 1))),
                                            (uint16_t*)row + col + e);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (col + e < d) __builtin_nontemporal_store(w[e], (uint32_t*)row + col + e);
    }
}

// gamma for the EPV columns from col, element by element, in Gamma<BF, GBF>'s packing
template <bool BF, bool GBF>
__device__ __forceinline__ void load_gamma_elems(const void* g, int64_t col, int64_t d,
                                                 u32x4* raw)
{
    constexpr int EPV = Io<BF>::kEpv;
    constexpr int GV = Gamma<BF, GBF>::kGv;
    uint32_t w[4 * GV];
#pragma unroll
    for (int i = 0; i < 4 * GV; ++i) w[i] = 0u;
    if constexpr (GBF) {
        const uint16_t* p = (const uint16_t*)g;
#pragma unroll
        for (int e = 0; e < EPV; ++e)
            if (col + e < d) w[e >> 1] |= (uint32_t)p[col + e] << (16 * (e & 1));
    } else {
        const uint32_t* p = (const uint32_t*)g;
#pragma unroll
        for (int e = 0; e < EPV; ++e)
            if (col + e < d) w[e] = p[col + e];
    }
#pragma unroll
    for (int h = 0; h < GV; ++h) raw[h] = u32x4{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
}

// NG: peer groups of 16 the kernel is built for (1 when n_ext <= 16, else 4). VEC: 16-byte
// accesses (slices aligned to 16 bytes, widths a whole number of vectors), else element
// accesses. One workgroup per row block (item).
template <bool BF, bool GBF, int NV, int NG, bool VEC>
__global__ __launch_bounds__(kBlock) void shard_fused_kernel(ShardJob job)
{
    constexpr int EPV = Io<BF>::kEpv;
    constexpr int ES = Io<BF>::kEs;
    constexpr int RR = kShardRowsPerWave;
    using G = Gamma<BF, GBF>;
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t items = job.nib * job.nseg;
    const int ngroups = (int)((job.n_ext + kPeersPerGroup - 1) / kPeersPerGroup);
    const bool check = job.epoch != 0;
    if ((int64_t)blockIdx.x >= items) return;

    // gamma of both tensors, loaded once
    u32x4 graw[2][NV][G::kGv];
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t col = (int64_t)(j * kWave + lane) * EPV;
            if (ts < job.nseg && col < job.t[ts].d) {
                if constexpr (VEC) G::load(job.t[ts].g, col, graw[ts][j]);
                else load_gamma_elems<BF, GBF>(job.t[ts].g, col, job.t[ts].d, graw[ts][j]);
            } else {
#pragma unroll
                for (int h = 0; h < G::kGv; ++h) graw[ts][j][h] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }

    // issue the loads of one item: the first look at the mailbox words (lane l of group g
    // watches peer 16 g + l / RR, row row0 + l % RR; plain loads, see above) and the rows
    auto issue = [&](int64_t item, ShardItem<NV, NG>& it) {
        const int tsel = item >= job.nib ? 1 : 0;
        const ShardTensor& s = job.t[tsel];
        const int64_t row0 = (tsel ? item - job.nib : item) * kShardItemRows + wave * RR;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int64_t e = (int64_t)g * kPeersPerGroup + lane / RR;
            const int64_t t = row0 + lane % RR;
            it.mine[g] = g < ngroups && e < job.n_ext && t < job.T;
            it.mw[g] = it.mine[g] ? s.mail[e * s.ld_mail + t] : 0;
        }
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const bool row_ok = row0 + r < job.T;
            const char* xr = (const char*)s.x + (row0 + r) * s.ldx * ES;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int64_t col = (int64_t)(j * kWave + lane) * EPV;
                if constexpr (VEC)
                    it.v[r][j] = (row_ok && col < s.d) ? load_stream(xr + col * ES)
                                                       : u32x4{0u, 0u, 0u, 0u};
                else
                    it.v[r][j] = (row_ok && col < s.d) ? load_elems<BF>(xr, col, s.d)
                                                       : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };

    // finish one item whose loads were issued into `cur`
    auto process = [&](int64_t item, ShardItem<NV, NG>& cur) {
        const int tsel = item >= job.nib ? 1 : 0;
        const ShardTensor& s = job.t[tsel];
        const int64_t row0 = (tsel ? item - job.nib : item) * kShardItemRows + wave * RR;

        // own partial sums of squares (lane r < RR holds row row0 + r), published as words
        float own = 0.0f;
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                float f[EPV];
                unpack<BF>(cur.v[r][j], f);
#pragma unroll
                for (int e = 0; e < EPV; e += 2) {
                    a0 = fmaf(f[e], f[e], a0);
                    a1 = fmaf(f[e + 1], f[e + 1], a1);
                }
            }
            const float t = wave_sum(a0 + a1);
            own = (lane == r) ? t : own;
        }
        const bool stat_lane = lane < RR && row0 + lane < job.T;
        if (s.psq_out && stat_lane)
            __hip_atomic_store(s.psq_out + row0 + lane, tagged(own, job.epoch), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);

        // wait until every watched word carries this epoch (usually the first look did)
        if (check) {
            bool ok = true;
#pragma unroll
            for (int g = 0; g < NG; ++g)
                ok = ok && (!cur.mine[g] || (uint32_t)(cur.mw[g] >> 32) == job.epoch);
            for (int64_t spin = 0; !__all(ok); ++spin) {
                if (spin >= job.max_spin) {
                    if (lane == 0) *job.timed_out = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
                ok = true;
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    if (cur.mine[g] && (uint32_t)(cur.mw[g] >> 32) != job.epoch) {
                        const int64_t e = (int64_t)g * kPeersPerGroup + lane / RR;
                        cur.mw[g] = __hip_atomic_load(s.mail + e * s.ld_mail + row0 + lane % RR,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        ok = ok && (uint32_t)(cur.mw[g] >> 32) == job.epoch;
                    }
                }
            }
        }

        // S = own + peer 0 + peer 1 + ... (fp32, in that order): lane r < RR gathers the value
        // of peer e from lane (e % 16) * RR + r of group e / 16
        float S = own;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g >= ngroups) break;
            const float val = __uint_as_float((uint32_t)cur.mw[g]);
            const int64_t ne = job.n_ext - (int64_t)g * kPeersPerGroup;
            const int cnt = ne < kPeersPerGroup ? (int)ne : kPeersPerGroup;
            for (int q = 0; q < cnt; ++q) S += __shfl(val, q * RR + (lane % RR));
        }
        const float rl = rsqrtf(S * s.inv_dfull + job.eps);
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            if (row0 + r < job.T) {
                const float rs = lane_read(rl, r);
                char* yr = (char*)s.y + (row0 + r) * s.ldy * ES;
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    const int64_t col = (int64_t)(j * kWave + lane) * EPV;
                    if (col < s.d) {
                        float f[EPV], o[EPV];
                        unpack<BF>(cur.v[r][j], f);
#pragma unroll
                        for (int e = 0; e < EPV; ++e)
                            o[e] = (f[e] * G::at(graw[tsel][j], e)) * rs;
                        if constexpr (VEC) store_stream(yr + col * ES, pack<BF>(o));
                        else store_elems<BF>(yr, col, s.d, pack<BF>(o));
                    }
                }
            }
        }
    };

    ShardItem<NV, NG> a;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        issue(item, a);
        process(item, a);
    }
}

struct PublishJob {
    const float* src[2];
    int64_t ld_src[2];
    uint64_t* dst[2];
    int64_t ld_dst[2];
    int nseg;
    int64_t T, n_ext;
    uint32_t epoch;
};

// One thread per (peer, tensor, row): the peer's partial, tagged with the epoch, as one
// device-coherent 64-bit store.
__global__ __launch_bounds__(kBlock) void shard_publish_kernel(PublishJob job)
{
    const int64_t total = job.n_ext * job.nseg * job.T;
    for (int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * kBlock) {
        const int64_t t = idx % job.T;
        const int tsel = (int)((idx / job.T) % job.nseg);
        const int64_t e = idx / (job.T * job.nseg);
        const float v = job.src[tsel][e * job.ld_src[tsel] + t];
        __hip_atomic_store(job.dst[tsel] + e * job.ld_dst[tsel] + t, tagged(v, job.epoch),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The device a stream's work runs on (the current device for the null stream), or -1.
int stream_device(hipStream_t st)
{
    int dev = -1;
    const hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    return e == hipSuccess ? dev : -1;
}

// LDS per CU of device dev, cached per device id
int device_lds_per_cu(int dev)
{
    static std::atomic<int> cache[64];
    if (dev >= 0 && dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int lds = 0;
    if (dev < 0 ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        lds <= 0)
        lds = 65536;
    if (dev >= 0 && dev < 64) cache[dev].store(lds, std::memory_order_relaxed);
    return lds;
}

template <bool BF, bool GBF, int NV, bool VEC>
hipError_t launch_shard_nv(const ShardJob& job, hipStream_t st)
{
    auto kernel = job.n_ext <= kPeersPerGroup
                      ? shard_fused_kernel<BF, GBF, NV, 1, VEC>
                      : shard_fused_kernel<BF, GBF, NV, kMaxPeerGroups, VEC>;
    const int64_t items = job.nib * job.nseg;
    if (items > 0x7fffffff) return hipErrorInvalidConfiguration;
    size_t lds = 0;
    if (job.epoch != 0 && job.persistent) {
        // Room for a producer on the same device: each workgroup reserves LDS it does not use,
        // sized so that at most three quarters of the workgroups the registers allow are
        // resident on a CU at once. The rest of the grid waits in the dispatcher, which hands
        // out row blocks in ascending order as workgroups finish (a grid that strides over the
        // blocks instead gives every workgroup a fixed share, and the slowest share sets the
        // time).
        static std::atomic<int> occupancy[2] = {{0}, {0}};
        static std::atomic<int> attr_set[2][64];  // per device: the attribute is per context
        const int which = job.n_ext <= kPeersPerGroup ? 0 : 1;
        int occ = occupancy[which].load(std::memory_order_relaxed);
        if (occ <= 0) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kBlock, 0) !=
                    hipSuccess ||
                occ <= 0)
                occ = 1;
            occupancy[which].store(occ, std::memory_order_relaxed);
        }
        const int cap = (occ * 3) / 4 > 0 ? (occ * 3) / 4 : 1;
        const int dev = stream_device(st);
        const int lds_cu = device_lds_per_cu(dev);
        // cap workgroups fit in lds_cu, cap + 1 do not (1 KB steps; the hardware allocates LDS
        // in 1280-byte granules on gfx950, which keeps cap * allocation <= lds_cu for cap <= 7)
        lds = (size_t)((lds_cu / (cap + 1) + 1024) / 1024 * 1024);
        if ((int64_t)lds * cap > lds_cu) lds = (size_t)(lds_cu / cap) / 1024 * 1024;
        if (lds > 65536) {
            // more than 64 KB of dynamic LDS must be allowed explicitly (workgroups with one
            // resident per CU reserve half the LDS)
            const bool known = dev >= 0 && dev < 64 &&
                               attr_set[which][dev].load(std::memory_order_relaxed) != 0;
            if (!known) {
                // the attribute applies to the current device: make it the stream's for the call
                int cur = -1;
                hipError_t e = hipGetDevice(&cur);
                if (e != hipSuccess) return e;
                const bool swap = dev >= 0 && dev != cur;
                if (swap && (e = hipSetDevice(dev)) != hipSuccess) return e;
                e = hipFuncSetAttribute((const void*)kernel,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (swap) {
                    const hipError_t r = hipSetDevice(cur);
                    if (e == hipSuccess) e = r;
                }
                if (e != hipSuccess) return e;
                if (dev >= 0 && dev < 64) attr_set[which][dev].store(1, std::memory_order_relaxed);
            }
        }
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)items), dim3(kBlock), lds, st, job);
    return hipGetLastError();
}

template <bool BF, bool GBF>
hipError_t launch_shard_types(const ShardJob& job, int nv, bool vec, hipStream_t st)
{
    if (vec) {
        switch (nv) {
        case 1: return launch_shard_nv<BF, GBF, 1, true>(job, st);
        case 2: return launch_shard_nv<BF, GBF, 2, true>(job, st);
        default: return launch_shard_nv<BF, GBF, 4, true>(job, st);
        }
    }
    switch (nv) {
    case 1: return launch_shard_nv<BF, GBF, 1, false>(job, st);
    case 2: return launch_shard_nv<BF, GBF, 2, false>(job, st);
    default: return launch_shard_nv<BF, GBF, 4, false>(job, st);
    }
}

}  // namespace

hipError_t launch_shard_fused(const ShardArgs& a, hipStream_t st)
{
    if (a.T == 0) return hipSuccess;
    ShardJob job = {};
    job.nseg = a.nseg;
    job.T = a.T;
    job.nib = (a.T + kShardItemRows - 1) / kShardItemRows;
    job.n_ext = a.n_ext;
    job.eps = a.eps;
    job.epoch = a.epoch;
    job.persistent = a.persistent;
    job.max_spin = a.max_spin;
    job.timed_out = a.timed_out;
    const int epv = a.bf16 ? 8 : 4;
    const int64_t es = a.bf16 ? 2 : 4;
    int64_t vmax = 0;
    bool vec = true;
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
    for (int i = 0; i < a.nseg; ++i) {
        const ShardSeg& r = a.seg[i];
        job.t[i] = {r.x, r.y, r.g, r.ldx, r.ldy, r.d, r.inv_dfull, r.psq_out, r.mail, r.ld_mail};
        const int64_t v = (r.d + epv - 1) / epv;
        vmax = v > vmax ? v : vmax;
        vec = vec && a16(r.x) && a16(r.y) && a16(r.g) && (r.ldx * es) % 16 == 0 &&
              (r.ldy * es) % 16 == 0 && r.d % epv == 0;
    }
    const int64_t per = (int64_t)kWave;
    const int nv = vmax <= per ? 1 : vmax <= 2 * per ? 2 : 4;
    if (a.bf16) return a.gamma_bf16 ? launch_shard_types<true, true>(job, nv, vec, st)
                                    : launch_shard_types<true, false>(job, nv, vec, st);
    return a.gamma_bf16 ? launch_shard_types<false, true>(job, nv, vec, st)
                        : launch_shard_types<false, false>(job, nv, vec, st);
}

hipError_t launch_shard_publish(int64_t T, int64_t n_ext, int nseg, const float* const* src,
                                const int64_t* ld_src, uint64_t* const* dst,
                                const int64_t* ld_dst, uint32_t epoch, hipStream_t st)
{
    if (T == 0 || n_ext == 0) return hipSuccess;
    PublishJob job = {};
    for (int i = 0; i < nseg; ++i) {
        job.src[i] = src[i];
        job.ld_src[i] = ld_src[i];
        job.dst[i] = dst[i];
        job.ld_dst[i] = ld_dst[i];
    }
    job.nseg = nseg;
    job.T = T;
    job.n_ext = n_ext;
    job.epoch = epoch;
    const int64_t total = n_ext * nseg * T;
    int64_t grid = (total + kBlock - 1) / kBlock;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(shard_publish_kernel, dim3((unsigned)grid), dim3(kBlock), 0, st, job);
    return hipGetLastError();
}

}  // namespace qkn
