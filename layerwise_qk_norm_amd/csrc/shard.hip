// Single-launch shard stage of layerwise QK-Norm under tensor parallelism: one pass over this
// rank's column slice computes the per-row partial sums of squares, publishes them, waits for
// the peers' partials, aggregates, and scales the slice it still holds in registers ("SwiftQK:
// Fast and Communication-Efficient Tensor Parallelism for Query-Key Normalization", abstract:
// scalar partial-sum aggregation, with the remaining peer-to-peer reduction overlapped with
// independent element-wise work in a deadlock-safe persistent kernel). Compared with the two
// launches (partial sums, then aggregation + scale) x is read once instead of twice.
//
// Mailbox protocol. Rows are grouped in blocks of kShardFlagRows (16). A peer's partials of
// one row block (Q or K) are valid in the mailbox once its flag holds the current epoch. The
// writer stores the values with device-scope coherence (written through the XCD's L2), waits
// until those stores are acknowledged (s_waitcnt vmcnt(0)), and only then stores the flag; the
// reader polls the flag and reads the mailbox with device-scope coherent loads. This orders the
// data before the flag without the device-wide L2 write-back and invalidation that a
// release/acquire pair costs on a multi-XCD GPU (they made the pass 30x slower). One GPU
// simulates its peers with shard_publish_kernel.
//
// Deadlock safety. A reader waits only on data that other work produces: when it waits, the
// grid is persistent and holds at most three quarters of the workgroups the device can keep
// resident, so a producer launched on another stream of the same device always finds free
// slots; and every wait is bounded (max_spin polls), after which the kernel records a timeout
// and finishes, so it never hangs.

#include <atomic>

#include "rows_impl.h"

namespace qkn {
namespace {

constexpr int kShardRowsPerWave = 4;
constexpr int kShardFlagRows = kWavesPerBlock * kShardRowsPerWave;  // one workgroup item

// kernel-argument view of one tensor's slice
struct ShardTensor {
    const void* x;
    void* y;
    const void* g;
    int64_t ldx, ldy, d;
    float inv_dfull;
    float* psq_out;
    const float* ext;
    int64_t ld_ext;
};

struct ShardJob {
    ShardTensor t[2];
    int nseg;
    int64_t T, nfb, n_ext;
    float eps;
    const uint32_t* peer_ready;  // [n_ext][2][nfb] or null: no waiting
    uint32_t* own_ready;         // [2][nfb] or null: no publication of flags
    uint32_t epoch;
    int64_t max_spin;
    int* timed_out;
};

template <bool BF, bool GBF, int NV>
__global__ __launch_bounds__(kBlock) void shard_fused_kernel(ShardJob job)
{
    constexpr int EPV = Io<BF>::kEpv;
    constexpr int ES = Io<BF>::kEs;
    constexpr int RR = kShardRowsPerWave;
    using G = Gamma<BF, GBF>;
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const int64_t items = job.nfb * job.nseg;

    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int tsel = item >= job.nfb ? 1 : 0;
        const int64_t fb = tsel ? item - job.nfb : item;
        const ShardTensor s = tsel ? job.t[1] : job.t[0];
        const int64_t row0 = fb * kShardFlagRows + wave * RR;

        // first poll of the peers' flags (lane e: peer e), in flight together with the row loads
        const bool poll_lane = job.peer_ready != nullptr && lane < job.n_ext;
        const uint32_t* flag = poll_lane
            ? job.peer_ready + ((int64_t)lane * 2 + tsel) * job.nfb + fb : nullptr;
        uint32_t seen = poll_lane
            ? __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : job.epoch;

        u32x4 graw[NV][G::kGv];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int64_t col = (int64_t)(j * kWave + lane) * EPV;
            if (col < s.d) {
                G::load(s.g, col, graw[j]);
            } else {
#pragma unroll
                for (int h = 0; h < G::kGv; ++h) graw[j][h] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        u32x4 v[RR][NV];
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const bool row_ok = row0 + r < job.T;
            const char* xr = (const char*)s.x + (row0 + r) * s.ldx * ES;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int64_t col = (int64_t)(j * kWave + lane) * EPV;
                v[r][j] = (row_ok && col < s.d) ? load_stream(xr + col * ES) : u32x4{0u, 0u, 0u, 0u};
            }
        }

        // own partial sums of squares (lane r < RR holds row row0 + r) and their publication
        float own = 0.0f;
#pragma unroll
        for (int r = 0; r < RR; ++r) {
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
            const float t = wave_sum(a0 + a1);
            own = (lane == r) ? t : own;
        }
        const bool stat_lane = lane < RR && row0 + lane < job.T;
        if (job.own_ready) {
            if (stat_lane)
                __hip_atomic_store(s.psq_out + row0 + lane, own, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);  // this wavefront's partials are acknowledged ...
            __syncthreads();                // ... for all four wavefronts of the row block ...
            if (threadIdx.x == 0)           // ... before the flag
                __hip_atomic_store(job.own_ready + tsel * job.nfb + fb, job.epoch,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (stat_lane) {
            s.psq_out[row0 + lane] = own;
        }

        // wait for the peers' partials of this row block (usually the first poll already saw them)
        if (job.peer_ready) {
            bool done = seen == job.epoch;
            for (int64_t spin = 0; !__all(done); ++spin) {
                if (spin >= job.max_spin) {
                    if (lane == 0) *job.timed_out = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
                if (!done)
                    done = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                           job.epoch;
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);  // mailbox reads stay after the polls
        }

        // S = own + peer 0 + peer 1 + ... (fp32, in that order)
        float S = own;
        if (stat_lane) {
            const int64_t t = row0 + lane;
            for (int64_t e0 = 0; e0 < job.n_ext; e0 += 8) {
                float p[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float* a = s.ext + (e0 + u) * s.ld_ext + t;
                    p[u] = e0 + u >= job.n_ext ? 0.0f
                           : job.peer_ready ? __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                            : *a;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (e0 + u < job.n_ext) S += p[u];
            }
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
                        unpack<BF>(v[r][j], f);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) o[e] = (f[e] * G::at(graw[j], e)) * rs;
                        store_stream(yr + col * ES, pack<BF>(o));
                    }
                }
            }
        }
        if (job.own_ready) __syncthreads();  // the next item's flag barrier starts clean
    }
}

struct PublishJob {
    const float* src[2];
    int64_t ld_src[2];
    float* dst[2];
    int64_t ld_dst[2];
    int nseg;
    int64_t T, nfb, n_ext;
    uint32_t* ready;
    uint32_t epoch;
};

// One thread per (peer, tensor, row block): copy that block's partials into the mailbox with
// device-coherent stores, wait for their acknowledgement, then store the flag.
__global__ __launch_bounds__(kBlock) void shard_publish_kernel(PublishJob job)
{
    const int64_t total = job.n_ext * job.nseg * job.nfb;
    for (int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * kBlock) {
        const int64_t fb = idx % job.nfb;
        const int tsel = (int)((idx / job.nfb) % job.nseg);
        const int64_t e = idx / (job.nfb * job.nseg);
        const float* src = job.src[tsel] + e * job.ld_src[tsel];
        float* dst = job.dst[tsel] + e * job.ld_dst[tsel];
        const int64_t t1 = (fb + 1) * kShardFlagRows < job.T ? (fb + 1) * kShardFlagRows : job.T;
        for (int64_t t = fb * kShardFlagRows; t < t1; ++t)
            __hip_atomic_store(dst + t, src[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __hip_atomic_store(job.ready + (e * 2 + tsel) * job.nfb + fb, job.epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

template <bool BF, bool GBF, int NV>
hipError_t launch_shard_nv(const ShardJob& job, hipStream_t st)
{
    auto kernel = shard_fused_kernel<BF, GBF, NV>;
    const int64_t items = job.nfb * job.nseg;
    int64_t grid = items;
    if (job.peer_ready) {
        static std::atomic<int> occupancy{0};
        int occ = occupancy.load(std::memory_order_relaxed);
        if (occ <= 0) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kBlock, 0) !=
                    hipSuccess ||
                occ <= 0)
                occ = 1;
            occupancy.store(occ, std::memory_order_relaxed);
        }
        const int64_t cap = ((int64_t)device_cus() * occ * 3) / 4;
        grid = items < cap ? items : (cap > 0 ? cap : 1);
    }
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kBlock), 0, st, job);
    return hipGetLastError();
}

template <bool BF, bool GBF>
hipError_t launch_shard_types(const ShardJob& job, int nv, hipStream_t st)
{
    switch (nv) {
    case 1: return launch_shard_nv<BF, GBF, 1>(job, st);
    case 2: return launch_shard_nv<BF, GBF, 2>(job, st);
    default: return launch_shard_nv<BF, GBF, 4>(job, st);
    }
}

}  // namespace

int64_t shard_flag_rows() { return kShardFlagRows; }

hipError_t launch_shard_fused(const ShardArgs& a, hipStream_t st)
{
    if (a.T == 0) return hipSuccess;
    ShardJob job = {};
    job.nseg = a.nseg;
    job.T = a.T;
    job.nfb = (a.T + kShardFlagRows - 1) / kShardFlagRows;
    job.n_ext = a.n_ext;
    job.eps = a.eps;
    job.peer_ready = a.peer_ready;
    job.own_ready = a.own_ready;
    job.epoch = a.epoch;
    job.max_spin = a.max_spin;
    job.timed_out = a.timed_out;
    const int epv = a.bf16 ? 8 : 4;
    int64_t vmax = 0;
    for (int i = 0; i < a.nseg; ++i) {
        const RowSeg& r = a.seg[i];
        job.t[i] = {r.x, r.y, r.g, r.ldx, r.ldy, r.d, r.inv_dfull, r.psq_out, r.ext, r.ld_ext};
        const int64_t v = (r.d + epv - 1) / epv;
        vmax = v > vmax ? v : vmax;
    }
    const int64_t per = (int64_t)kWave;
    const int nv = vmax <= per ? 1 : vmax <= 2 * per ? 2 : 4;
    if (a.bf16) return a.gamma_bf16 ? launch_shard_types<true, true>(job, nv, st)
                                    : launch_shard_types<true, false>(job, nv, st);
    return a.gamma_bf16 ? launch_shard_types<false, true>(job, nv, st)
                        : launch_shard_types<false, false>(job, nv, st);
}

hipError_t launch_shard_publish(int64_t T, int64_t n_ext, int nseg, const float* const* src,
                                const int64_t* ld_src, float* const* dst, const int64_t* ld_dst,
                                uint32_t* ready, uint32_t epoch, hipStream_t st)
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
    job.nfb = (T + kShardFlagRows - 1) / kShardFlagRows;
    job.n_ext = n_ext;
    job.ready = ready;
    job.epoch = epoch;
    const int64_t total = n_ext * nseg * job.nfb;
    int64_t grid = (total + kBlock - 1) / kBlock;
    if (grid > 1024) grid = 1024;
    hipLaunchKernelGGL(shard_publish_kernel, dim3((unsigned)grid), dim3(kBlock), 0, st, job);
    return hipGetLastError();
}

}  // namespace qkn
