// C-ABI entry points of libqknorm.so: argument validation (before any HIP call) and dispatch
// onto the caller's stream. The operations and conventions are documented in qknorm.h.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/qknorm.h"
#include "launch.h"

// Workspace of normproj_deferred_layernorm_noalloc: (mean, 1/std) of up to kNoallocRows rows,
// one copy per GPU for the life of the process. Host code never passes `scratch` itself to a
// kernel (on the host the name stands for a host-side shadow): it uses the device address
// hipGetSymbolAddress returns, looked up once per device on the first call made on it.
constexpr int64_t kNoallocRows = 131072;
static __device__ __align__(256) float scratch[2 * kNoallocRows];

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return QKN_OK;
    g_last_hip_error = (int)e;
    return QKN_ERR_HIP;
}

bool valid_dtype(int dt) { return dt == QKN_F32 || dt == QKN_BF16; }
int64_t elem_size(int dt) { return dt == QKN_F32 ? 4 : 2; }
bool valid_eps(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

// Largest byte extent a tensor argument may span: 2^56 bytes, far beyond any device, so that
// the extents, the overlap checks and the launches' 64-bit index arithmetic cannot wrap.
constexpr int64_t kMaxExtentBytes = int64_t(1) << 56;

// Whether a [rows, cols] tensor with row stride ld of es-byte elements spans more than
// kMaxExtentBytes (an empty one never does).
bool too_large(int64_t rows, int64_t cols, int64_t ld, int64_t es)
{
    if (rows <= 0 || cols <= 0) return false;
    int64_t e = 0;
    if (__builtin_mul_overflow(rows - 1, ld, &e) || __builtin_add_overflow(e, cols, &e) ||
        __builtin_mul_overflow(e, es, &e))
        return true;
    return e > kMaxExtentBytes;
}

// Bytes touched by a [rows, cols] tensor with row stride ld: the hull [lo, hi) and, per row,
// `width` bytes every `pitch` bytes (one row: width == pitch == hi - lo).
struct Range {
    uintptr_t lo = 0, hi = 0;
    uintptr_t width = 0, pitch = 0;
    bool empty() const { return hi <= lo; }
};

Range span(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t es)
{
    Range r;
    if (p == nullptr || rows <= 0 || cols <= 0) return r;
    r.lo = (uintptr_t)p;
    r.hi = r.lo + (uintptr_t)(((rows - 1) * ld + cols) * es);
    r.width = (uintptr_t)(cols * es);
    r.pitch = rows > 1 ? (uintptr_t)(ld * es) : r.hi - r.lo;
    return r;
}

// Whether two tensors share a byte. Hulls that do not meet never do; two multi-row tensors with
// the same pitch are disjoint when, within every period of that pitch, one's columns end
// before the other's begin (e.g. the Q and K column blocks of one [T, nq + nk] matrix);
// anything else whose hulls meet counts as overlapping.
bool overlap(const Range& a, const Range& b)
{
    if (a.empty() || b.empty() || a.hi <= b.lo || b.hi <= a.lo) return false;
    const bool multi = a.pitch > a.width && b.pitch > b.width;
    if (multi && a.pitch == b.pitch) {
        const Range& first = a.lo <= b.lo ? a : b;
        const Range& second = a.lo <= b.lo ? b : a;
        const uintptr_t off = (second.lo - first.lo) % first.pitch;
        if (off >= first.width && off + second.width <= first.pitch) return false;
    }
    return true;
}

// An output may alias its own input exactly (same base, same stride); any other overlap is an
// error. `others` are ranges the output must not touch at all.
bool out_ok(const void* out, int64_t ld_out, const void* in, int64_t ld_in, const Range& r_out,
            const Range& r_in, const Range* others, int n_others)
{
    const bool exact = out == in && ld_out == ld_in;
    if (!exact && overlap(r_out, r_in)) return false;
    for (int i = 0; i < n_others; ++i)
        if (overlap(r_out, others[i])) return false;
    return true;
}

// Common checks of one row tensor: pointers present, 1 <= d <= ld.
int check_rows(int64_t T, const void* x, int64_t ldx, const void* y, int64_t ldy, int64_t d,
               bool need_y)
{
    if (d < 1 || ldx < d || (need_y && ldy < d)) return QKN_ERR_SHAPE;
    if (too_large(T, d, ldx, 4) || (need_y && too_large(T, d, ldy, 4))) return QKN_ERR_SHAPE;
    if (T > 0 && (x == nullptr || (need_y && y == nullptr))) return QKN_ERR_NULL;
    return QKN_OK;
}

// a pointer off the natural alignment of its elements (null is aligned)
bool misaligned(const void* p, int64_t bytes) { return ((uintptr_t)p % (uintptr_t)bytes) != 0; }

}  // namespace

extern "C" {

QKN_API const char* qkn_status_string(int status)
{
    switch (status) {
    case QKN_OK: return "ok";
    case QKN_ERR_NULL: return "a required pointer is NULL";
    case QKN_ERR_SHAPE: return "invalid or inconsistent sizes or strides";
    case QKN_ERR_DTYPE: return "unsupported dtype code";
    case QKN_ERR_EPS: return "eps must be finite and >= 0";
    case QKN_ERR_ALIAS: return "an output partially overlaps an input or another output";
    case QKN_ERR_ALIGN: return "a pointer is not aligned to what the call requires";
    case QKN_ERR_HIP: return "HIP runtime error (see qkn_last_hip_error)";
    case QKN_ERR_SCRATCH: return "the input exceeds the library's static workspace";
    default: return "unknown status";
    }
}

QKN_API int qkn_last_hip_error(void) { return g_last_hip_error; }

QKN_API int qknorm_fused(int64_t T, float eps, int dtype, int gamma_dtype, const void* q,
                         int64_t ldq, void* q_out, int64_t ldq_out, const void* gamma_q,
                         int64_t dq, const void* k, int64_t ldk, void* k_out, int64_t ldk_out,
                         const void* gamma_k, int64_t dk, void* stream)
{
    if (T < 0) return QKN_ERR_SHAPE;
    if (!valid_dtype(dtype) || !valid_dtype(gamma_dtype)) return QKN_ERR_DTYPE;
    if (!valid_eps(eps)) return QKN_ERR_EPS;
    const bool has_k = !(k == nullptr && k_out == nullptr && gamma_k == nullptr && dk == 0);
    int st = check_rows(T, q, ldq, q_out, ldq_out, dq, true);
    if (st != QKN_OK) return st;
    if (T > 0 && gamma_q == nullptr) return QKN_ERR_NULL;
    if (has_k) {
        st = check_rows(T, k, ldk, k_out, ldk_out, dk, true);
        if (st != QKN_OK) return st;
        if (T > 0 && gamma_k == nullptr) return QKN_ERR_NULL;
    }
    if (T == 0) return QKN_OK;

    const int64_t es = elem_size(dtype), gs = elem_size(gamma_dtype);
    if (misaligned(q, es) || misaligned(q_out, es) || misaligned(gamma_q, gs) ||
        (has_k && (misaligned(k, es) || misaligned(k_out, es) || misaligned(gamma_k, gs))))
        return QKN_ERR_ALIGN;
    const Range rq = span(q, T, dq, ldq, es), rqo = span(q_out, T, dq, ldq_out, es);
    const Range rgq = span(gamma_q, 1, dq, dq, gs);
    Range rk, rko, rgk;
    if (has_k) {
        rk = span(k, T, dk, ldk, es);
        rko = span(k_out, T, dk, ldk_out, es);
        rgk = span(gamma_k, 1, dk, dk, gs);
    }
    const Range others_q[] = {rgq, rk, rko, rgk};
    if (!out_ok(q_out, ldq_out, q, ldq, rqo, rq, others_q, has_k ? 4 : 1)) return QKN_ERR_ALIAS;
    if (has_k) {
        const Range others_k[] = {rgk, rq, rgq};
        if (!out_ok(k_out, ldk_out, k, ldk, rko, rk, others_k, 3)) return QKN_ERR_ALIAS;
    }

    qkn::RowJob job = {};
    job.nseg = has_k ? 2 : 1;
    job.T = T;
    job.eps = eps;
    job.mode = qkn::kFused;
    job.bf16 = dtype == QKN_BF16;
    job.gamma_bf16 = gamma_dtype == QKN_BF16;
    job.seg[0] = {q, q_out, gamma_q, ldq, ldq_out, dq, (float)(1.0 / (double)dq),
                  nullptr, nullptr, 0, 0, nullptr};
    if (has_k)
        job.seg[1] = {k, k_out, gamma_k, ldk, ldk_out, dk, (float)(1.0 / (double)dk),
                      nullptr, nullptr, 0, 0, nullptr};
    return hip_status(qkn::launch_rows(job, (hipStream_t)stream));
}

QKN_API int qknorm_partial_sumsq(int64_t T, int dtype, const void* q, int64_t ldq,
                                 int64_t dq_local, float* psq_q, const void* k, int64_t ldk,
                                 int64_t dk_local, float* psq_k, void* stream)
{
    if (T < 0) return QKN_ERR_SHAPE;
    if (!valid_dtype(dtype)) return QKN_ERR_DTYPE;
    const bool has_k = !(k == nullptr && psq_k == nullptr && dk_local == 0);
    int st = check_rows(T, q, ldq, nullptr, 0, dq_local, false);
    if (st != QKN_OK) return st;
    if (T > 0 && psq_q == nullptr) return QKN_ERR_NULL;
    if (has_k) {
        st = check_rows(T, k, ldk, nullptr, 0, dk_local, false);
        if (st != QKN_OK) return st;
        if (T > 0 && psq_k == nullptr) return QKN_ERR_NULL;
    }
    if (T == 0) return QKN_OK;

    const int64_t es = elem_size(dtype);
    if (misaligned(q, es) || misaligned(k, es) || misaligned(psq_q, 4) || misaligned(psq_k, 4))
        return QKN_ERR_ALIGN;
    const Range rq = span(q, T, dq_local, ldq, es), rk = has_k ? span(k, T, dk_local, ldk, es) : Range();
    const Range rpq = span(psq_q, 1, T, T, 4), rpk = has_k ? span(psq_k, 1, T, T, 4) : Range();
    if (overlap(rpq, rq) || overlap(rpq, rk) || overlap(rpq, rpk) || overlap(rpk, rq) ||
        overlap(rpk, rk))
        return QKN_ERR_ALIAS;

    qkn::RowJob job = {};
    job.nseg = has_k ? 2 : 1;
    job.T = T;
    job.mode = qkn::kPartial;
    job.bf16 = dtype == QKN_BF16;
    job.seg[0] = {q, nullptr, nullptr, ldq, 0, dq_local, 0.0f, nullptr, nullptr, 0, 0, psq_q};
    if (has_k) job.seg[1] = {k, nullptr, nullptr, ldk, 0, dk_local, 0.0f, nullptr, nullptr, 0, 0, psq_k};
    return hip_status(qkn::launch_rows(job, (hipStream_t)stream));
}

QKN_API int qknorm_apply_with_stats(int64_t T, float eps, int dtype, int gamma_dtype,
                                    int64_t n_ext, const void* q, int64_t ldq, void* q_out,
                                    int64_t ldq_out, const void* gamma_q, int64_t dq_local,
                                    int64_t dq_full, const float* psq_q, const float* ext_q,
                                    int64_t ld_ext_q, const void* k, int64_t ldk, void* k_out,
                                    int64_t ldk_out, const void* gamma_k, int64_t dk_local,
                                    int64_t dk_full, const float* psq_k, const float* ext_k,
                                    int64_t ld_ext_k, void* stream)
{
    if (T < 0 || n_ext < 0) return QKN_ERR_SHAPE;
    if (!valid_dtype(dtype) || !valid_dtype(gamma_dtype)) return QKN_ERR_DTYPE;
    if (!valid_eps(eps)) return QKN_ERR_EPS;
    const bool has_k = !(k == nullptr && k_out == nullptr && gamma_k == nullptr &&
                         psq_k == nullptr && ext_k == nullptr && dk_local == 0);
    int st = check_rows(T, q, ldq, q_out, ldq_out, dq_local, true);
    if (st != QKN_OK) return st;
    if (dq_full < dq_local) return QKN_ERR_SHAPE;
    if (n_ext > 0 && (ld_ext_q < T || too_large(n_ext, T, ld_ext_q, 4))) return QKN_ERR_SHAPE;
    if (T > 0 && (gamma_q == nullptr || psq_q == nullptr || (n_ext > 0 && ext_q == nullptr)))
        return QKN_ERR_NULL;
    if (has_k) {
        st = check_rows(T, k, ldk, k_out, ldk_out, dk_local, true);
        if (st != QKN_OK) return st;
        if (dk_full < dk_local) return QKN_ERR_SHAPE;
        if (n_ext > 0 && (ld_ext_k < T || too_large(n_ext, T, ld_ext_k, 4)))
            return QKN_ERR_SHAPE;
        if (T > 0 && (gamma_k == nullptr || psq_k == nullptr || (n_ext > 0 && ext_k == nullptr)))
            return QKN_ERR_NULL;
    }
    if (T == 0) return QKN_OK;

    const int64_t es = elem_size(dtype), gs = elem_size(gamma_dtype);
    if (misaligned(q, es) || misaligned(q_out, es) || misaligned(gamma_q, gs) ||
        misaligned(psq_q, 4) || misaligned(ext_q, 4) ||
        (has_k && (misaligned(k, es) || misaligned(k_out, es) || misaligned(gamma_k, gs) ||
                   misaligned(psq_k, 4) || misaligned(ext_k, 4))))
        return QKN_ERR_ALIGN;
    const Range rq = span(q, T, dq_local, ldq, es), rqo = span(q_out, T, dq_local, ldq_out, es);
    const Range rgq = span(gamma_q, 1, dq_local, dq_local, gs);
    const Range rpq = span(psq_q, 1, T, T, 4);
    const Range req = n_ext > 0 ? span(ext_q, n_ext, T, ld_ext_q, 4) : Range();
    Range rk, rko, rgk, rpk, rek;
    if (has_k) {
        rk = span(k, T, dk_local, ldk, es);
        rko = span(k_out, T, dk_local, ldk_out, es);
        rgk = span(gamma_k, 1, dk_local, dk_local, gs);
        rpk = span(psq_k, 1, T, T, 4);
        rek = n_ext > 0 ? span(ext_k, n_ext, T, ld_ext_k, 4) : Range();
    }
    const Range others_q[] = {rgq, rpq, req, rk, rko, rgk, rpk, rek};
    if (!out_ok(q_out, ldq_out, q, ldq, rqo, rq, others_q, 8)) return QKN_ERR_ALIAS;
    if (has_k) {
        const Range others_k[] = {rgk, rpk, rek, rq, rgq, rpq, req};
        if (!out_ok(k_out, ldk_out, k, ldk, rko, rk, others_k, 7)) return QKN_ERR_ALIAS;
    }

    qkn::RowJob job = {};
    job.nseg = has_k ? 2 : 1;
    job.T = T;
    job.eps = eps;
    job.mode = qkn::kApply;
    job.bf16 = dtype == QKN_BF16;
    job.gamma_bf16 = gamma_dtype == QKN_BF16;
    job.seg[0] = {q, q_out, gamma_q, ldq, ldq_out, dq_local, (float)(1.0 / (double)dq_full),
                  psq_q, ext_q, ld_ext_q, n_ext, nullptr};
    if (has_k)
        job.seg[1] = {k, k_out, gamma_k, ldk, ldk_out, dk_local, (float)(1.0 / (double)dk_full),
                      psq_k, ext_k, ld_ext_k, n_ext, nullptr};
    return hip_status(qkn::launch_rows(job, (hipStream_t)stream));
}

QKN_API int qknorm_shard_fused(int64_t T, float eps, int dtype, int gamma_dtype, int64_t n_ext,
                               const void* q, int64_t ldq, void* q_out, int64_t ldq_out,
                               const void* gamma_q, int64_t dq_local, int64_t dq_full,
                               uint64_t* psq_q_out, const uint64_t* mail_q, int64_t ld_mail_q,
                               const void* k, int64_t ldk, void* k_out, int64_t ldk_out,
                               const void* gamma_k, int64_t dk_local, int64_t dk_full,
                               uint64_t* psq_k_out, const uint64_t* mail_k, int64_t ld_mail_k,
                               uint32_t epoch, int persistent, int64_t max_spin, int* timed_out,
                               void* stream)
{
    if (T < 0 || n_ext < 0 || n_ext > 64 || max_spin < 0) return QKN_ERR_SHAPE;
    if (persistent != 0 && persistent != 1) return QKN_ERR_SHAPE;
    if (!valid_dtype(dtype) || !valid_dtype(gamma_dtype)) return QKN_ERR_DTYPE;
    if (!valid_eps(eps)) return QKN_ERR_EPS;
    const bool has_k = !(k == nullptr && k_out == nullptr && gamma_k == nullptr &&
                         psq_k_out == nullptr && mail_k == nullptr && dk_local == 0);
    const int64_t es = elem_size(dtype), gs = elem_size(gamma_dtype), epv = 16 / es;
    const int64_t dmax = 4 * 64 * epv;
    struct S {
        const void* x; int64_t ldx; void* y; int64_t ldy; const void* g; int64_t dl, df;
        uint64_t* psq; const uint64_t* mail; int64_t ldm;
    } segs[2] = {{q, ldq, q_out, ldq_out, gamma_q, dq_local, dq_full, psq_q_out, mail_q, ld_mail_q},
                 {k, ldk, k_out, ldk_out, gamma_k, dk_local, dk_full, psq_k_out, mail_k, ld_mail_k}};
    const int nseg = has_k ? 2 : 1;
    for (int i = 0; i < nseg; ++i) {
        const S& c = segs[i];
        int st = check_rows(T, c.x, c.ldx, c.y, c.ldy, c.dl, true);
        if (st != QKN_OK) return st;
        if (c.df < c.dl || c.dl > dmax) return QKN_ERR_SHAPE;
        if (n_ext > 0 && (c.ldm < T || too_large(n_ext, T, c.ldm, 8))) return QKN_ERR_SHAPE;
        if (T > 0 && (c.g == nullptr || (n_ext > 0 && c.mail == nullptr))) return QKN_ERR_NULL;
        // elements at their natural alignment, mailbox words at 8 bytes; 16-byte accesses run
        // where every slice allows them, element accesses otherwise
        if (((uintptr_t)c.x % (uintptr_t)es) || ((uintptr_t)c.y % (uintptr_t)es) ||
            ((uintptr_t)c.g % (uintptr_t)gs) || ((uintptr_t)c.psq & 7u) ||
            ((uintptr_t)c.mail & 7u))
            return QKN_ERR_ALIGN;
    }
    if (T > 0 && epoch != 0 && timed_out == nullptr) return QKN_ERR_NULL;
    if (T == 0) return QKN_OK;

    Range r_in[2], r_out[2], r_g[2], r_psq[2], r_mail[2];
    for (int i = 0; i < nseg; ++i) {
        const S& c = segs[i];
        r_in[i] = span(c.x, T, c.dl, c.ldx, es);
        r_out[i] = span(c.y, T, c.dl, c.ldy, es);
        r_g[i] = span(c.g, 1, c.dl, c.dl, gs);
        r_psq[i] = c.psq ? span(c.psq, 1, T, T, 8) : Range();
        r_mail[i] = n_ext > 0 ? span(c.mail, n_ext, T, c.ldm, 8) : Range();
    }
    const Range r_to = timed_out ? span(timed_out, 1, 1, 1, 4) : Range();
    for (int i = 0; i < nseg; ++i) {
        // every written range against every other range (exact in-place output allowed)
        const Range writes[3] = {r_out[i], r_psq[i], r_to};
        for (int a = 0; a < 3; ++a) {
            for (int j = 0; j < nseg; ++j) {
                const bool self_inplace = a == 0 && j == i && segs[i].y == segs[i].x &&
                                          segs[i].ldy == segs[i].ldx;
                if (!self_inplace && overlap(writes[a], r_in[j])) return QKN_ERR_ALIAS;
                if (overlap(writes[a], r_g[j]) || overlap(writes[a], r_mail[j])) return QKN_ERR_ALIAS;
                if (j != i && (overlap(writes[a], r_out[j]) || overlap(writes[a], r_psq[j])))
                    return QKN_ERR_ALIAS;
            }
        }
        if (overlap(r_out[i], r_psq[i]) || overlap(r_out[i], r_to) || overlap(r_psq[i], r_to))
            return QKN_ERR_ALIAS;
    }

    qkn::ShardArgs a = {};
    a.nseg = nseg;
    a.T = T;
    a.eps = eps;
    a.n_ext = n_ext;
    a.bf16 = dtype == QKN_BF16;
    a.gamma_bf16 = gamma_dtype == QKN_BF16;
    a.epoch = epoch;
    a.persistent = persistent;
    a.max_spin = max_spin;
    a.timed_out = timed_out;
    for (int i = 0; i < nseg; ++i) {
        const S& c = segs[i];
        a.seg[i] = {c.x, c.y, c.g, c.ldx, c.ldy, c.dl, (float)(1.0 / (double)c.df), c.psq,
                    c.mail, c.ldm};
    }
    return hip_status(qkn::launch_shard_fused(a, (hipStream_t)stream));
}

QKN_API int qknorm_shard_publish(int64_t T, int64_t n_ext, const float* part_q, int64_t ld_part_q,
                                 uint64_t* mail_q, int64_t ld_mail_q, const float* part_k,
                                 int64_t ld_part_k, uint64_t* mail_k, int64_t ld_mail_k,
                                 uint32_t epoch, void* stream)
{
    if (T < 0 || n_ext < 0) return QKN_ERR_SHAPE;
    const bool has_k = !(part_k == nullptr && mail_k == nullptr);
    if (T == 0 || n_ext == 0) return QKN_OK;
    if (part_q == nullptr || mail_q == nullptr ||
        (has_k && (part_k == nullptr || mail_k == nullptr)))
        return QKN_ERR_NULL;
    if (ld_part_q < T || ld_mail_q < T || (has_k && (ld_part_k < T || ld_mail_k < T)))
        return QKN_ERR_SHAPE;
    if (too_large(n_ext, T, ld_mail_q, 8) || too_large(n_ext, T, ld_part_q, 4) ||
        (has_k && (too_large(n_ext, T, ld_mail_k, 8) || too_large(n_ext, T, ld_part_k, 4))))
        return QKN_ERR_SHAPE;
    if (((uintptr_t)mail_q & 7u) || ((uintptr_t)mail_k & 7u)) return QKN_ERR_ALIGN;
    const Range rq = span(mail_q, n_ext, T, ld_mail_q, 8);
    const Range rk = has_k ? span(mail_k, n_ext, T, ld_mail_k, 8) : Range();
    const Range pq = span(part_q, n_ext, T, ld_part_q, 4);
    const Range pk = has_k ? span(part_k, n_ext, T, ld_part_k, 4) : Range();
    if (overlap(rq, pq) || overlap(rq, pk) || overlap(rq, rk) || overlap(rk, pq) || overlap(rk, pk))
        return QKN_ERR_ALIAS;
    const float* src[2] = {part_q, part_k};
    const int64_t lds[2] = {ld_part_q, ld_part_k};
    uint64_t* dst[2] = {mail_q, mail_k};
    const int64_t ldd[2] = {ld_mail_q, ld_mail_k};
    return hip_status(qkn::launch_shard_publish(T, n_ext, has_k ? 2 : 1, src, lds, dst, ldd, epoch,
                                                (hipStream_t)stream));
}

QKN_API int normproj_fold_weight(int64_t K, int64_t N, int dtype, int gamma_dtype,
                                 const void* w, int64_t ldw, const void* gamma, void* w_fold,
                                 int64_t ldw_fold, void* stream)
{
    if (K < 0 || N < 0 || ldw < N || ldw_fold < N) return QKN_ERR_SHAPE;
    if (too_large(K, N, ldw, 2) || too_large(K, N, ldw_fold, 2)) return QKN_ERR_SHAPE;
    if (dtype != QKN_BF16 || !valid_dtype(gamma_dtype)) return QKN_ERR_DTYPE;
    if (K == 0 || N == 0) return QKN_OK;
    if (w == nullptr || w_fold == nullptr) return QKN_ERR_NULL;
    const Range rw = span(w, K, N, ldw, 2), rf = span(w_fold, K, N, ldw_fold, 2);
    const Range rg = gamma ? span(gamma, 1, K, K, elem_size(gamma_dtype)) : Range();
    // in place (w_fold == w, same stride) is allowed: each element is read, then written
    if (!out_ok(w_fold, ldw_fold, w, ldw, rf, rw, &rg, 1)) return QKN_ERR_ALIAS;
    return hip_status(qkn::launch_fold(K, N, w, ldw, gamma, gamma_dtype == QKN_BF16, w_fold,
                                       ldw_fold, (hipStream_t)stream));
}

namespace {

// x [T, K] (ldx), w [K, N] row-major (ldw), y [T, N] (ldy), all bf16 at any alignment.
int check_normproj(int64_t T, int64_t K, int64_t N, float eps, int dtype, const void* x,
                   int64_t ldx, const void* w, int64_t ldw, const void* y, int64_t ldy)
{
    if (T < 0 || K < 1 || N < 0 || ldx < K || ldw < N || ldy < N) return QKN_ERR_SHAPE;
    if (too_large(T, K, ldx, 2) || too_large(K, N, ldw, 2) || too_large(T, N, ldy, 2))
        return QKN_ERR_SHAPE;
    if (dtype != QKN_BF16) return QKN_ERR_DTYPE;
    if (!valid_eps(eps)) return QKN_ERR_EPS;
    if (T == 0 || N == 0) return QKN_OK;
    if (x == nullptr || w == nullptr || y == nullptr) return QKN_ERR_NULL;
    if (((uintptr_t)x & 1u) || ((uintptr_t)w & 1u) || ((uintptr_t)y & 1u)) return QKN_ERR_ALIGN;
    const Range ry = span(y, T, N, ldy, 2);
    if (overlap(ry, span(x, T, K, ldx, 2)) || overlap(ry, span(w, K, N, ldw, 2)))
        return QKN_ERR_ALIAS;
    return QKN_OK;
}

}  // namespace

QKN_API int normproj_deferred(int64_t T, int64_t K, int64_t N, float eps, int dtype,
                              const void* x, int64_t ldx, const void* w_fold, int64_t ldw,
                              void* y, int64_t ldy, void* stream)
{
    const int st = check_normproj(T, K, N, eps, dtype, x, ldx, w_fold, ldw, y, ldy);
    if (st != QKN_OK || T == 0 || N == 0) return st;
    return hip_status(qkn::launch_normproj(T, K, N, eps, qkn::kEpiRms, x,
                                           ldx, w_fold, ldw, y, ldy, nullptr, nullptr, nullptr,
                                           (hipStream_t)stream));
}

namespace {

// RMSNorm launch into xn (ordinary stores: the product reads xn straight back), then the plain
// product; keep_y: the caller reads y back next as well.
int unfused_rms_product(int64_t T, int64_t K, int64_t N, float eps, int dtype, int gamma_dtype,
                        const void* x, int64_t ldx, const void* gamma, const void* w,
                        int64_t ldw, void* xn, int64_t ldxn, void* y, int64_t ldy, bool keep_y,
                        void* stream)
{
    int st = check_normproj(T, K, N, eps, dtype, x, ldx, w, ldw, y, ldy);
    if (st != QKN_OK) return st;
    if (!valid_dtype(gamma_dtype)) return QKN_ERR_DTYPE;
    if (ldxn < K || too_large(T, K, ldxn, 2)) return QKN_ERR_SHAPE;
    if (T == 0 || N == 0) return QKN_OK;
    if (xn == nullptr || gamma == nullptr) return QKN_ERR_NULL;
    if (((uintptr_t)xn & 1u) != 0) return QKN_ERR_ALIGN;
    const Range rxn = span(xn, T, K, ldxn, 2), rg = span(gamma, 1, K, K, elem_size(gamma_dtype));
    if (overlap(rxn, span(x, T, K, ldx, 2)) || overlap(rxn, span(w, K, N, ldw, 2)) ||
        overlap(rxn, span(y, T, N, ldy, 2)) || overlap(rxn, rg) ||
        overlap(span(y, T, N, ldy, 2), rg))
        return QKN_ERR_ALIAS;

    qkn::RowJob job = {};
    job.nseg = 1;
    job.T = T;
    job.eps = eps;
    job.mode = qkn::kFused;
    job.bf16 = 1;
    job.gamma_bf16 = gamma_dtype == QKN_BF16;
    job.keep_cached = 1;
    job.seg[0] = {x, xn, gamma, ldx, ldxn, K, (float)(1.0 / (double)K), nullptr, nullptr, 0, 0,
                  nullptr};
    hipError_t e = qkn::launch_rows(job, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(qkn::launch_normproj(T, K, N, eps,
                                           qkn::kEpiPlain |
                                               (keep_y ? qkn::kEpiKeepCached : 0),
                                           xn, ldxn, w, ldw, y, ldy, nullptr, nullptr, nullptr,
                                           (hipStream_t)stream));
}

}  // namespace

QKN_API int normproj_unfused(int64_t T, int64_t K, int64_t N, float eps, int dtype,
                             int gamma_dtype, const void* x, int64_t ldx, const void* gamma,
                             const void* w, int64_t ldw, void* xn, int64_t ldxn, void* y,
                             int64_t ldy, void* stream)
{
    return unfused_rms_product(T, K, N, eps, dtype, gamma_dtype, x, ldx, gamma, w, ldw, xn, ldxn,
                               y, ldy, false, stream);
}

QKN_API int normproj_fold_layernorm(int64_t K, int64_t N, int dtype, int gamma_dtype,
                                    const void* w, int64_t ldw, const void* gamma,
                                    const void* beta, void* w_fold, int64_t ldw_fold,
                                    float* colsum, float* bias, void* stream)
{
    if (K < 0 || N < 0 || ldw < N || ldw_fold < N) return QKN_ERR_SHAPE;
    if (too_large(K, N, ldw, 2) || too_large(K, N, ldw_fold, 2)) return QKN_ERR_SHAPE;
    if (dtype != QKN_BF16 || !valid_dtype(gamma_dtype)) return QKN_ERR_DTYPE;
    if (K == 0 || N == 0) return QKN_OK;
    if (w == nullptr || w_fold == nullptr || colsum == nullptr) return QKN_ERR_NULL;
    const int64_t gs = elem_size(gamma_dtype);
    const Range rw = span(w, K, N, ldw, 2), rf = span(w_fold, K, N, ldw_fold, 2);
    const Range rg = gamma ? span(gamma, 1, K, K, gs) : Range();
    const Range rb = beta ? span(beta, 1, K, K, gs) : Range();
    const Range rc = span(colsum, 1, N, N, 4), ro = bias ? span(bias, 1, N, N, 4) : Range();
    const Range ins[] = {rw, rg, rb};
    for (const Range& r : ins)
        if (overlap(rf, r) || overlap(rc, r) || overlap(ro, r)) return QKN_ERR_ALIAS;
    if (overlap(rf, rc) || overlap(rf, ro) || overlap(rc, ro)) return QKN_ERR_ALIAS;
    hipError_t e = qkn::launch_fold(K, N, w, ldw, gamma, gamma_dtype == QKN_BF16, w_fold,
                                    ldw_fold, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(qkn::launch_fold_stats(K, N, w, ldw, gamma, beta, gamma_dtype == QKN_BF16,
                                             colsum, bias, (hipStream_t)stream));
}

namespace {

// Checks of deferred LayerNorm, the optional row-statistics workspace included.
int check_deferred_layernorm(int64_t T, int64_t K, int64_t N, float eps, int dtype,
                             const void* x, int64_t ldx, const void* w_fold, int64_t ldw,
                             const float* colsum, const float* bias, const void* y, int64_t ldy,
                             const float* row_stats)
{
    const int st = check_normproj(T, K, N, eps, dtype, x, ldx, w_fold, ldw, y, ldy);
    if (st != QKN_OK || T == 0 || N == 0) return st;
    if (colsum == nullptr) return QKN_ERR_NULL;
    const Range ry = span(y, T, N, ldy, 2);
    const Range rc = span(colsum, 1, N, N, 4);
    const Range rb = bias ? span(bias, 1, N, N, 4) : Range{};
    if (overlap(ry, rc) || (bias && overlap(ry, rb))) return QKN_ERR_ALIAS;
    if (row_stats) {
        const Range rs = span(row_stats, 1, 2 * T, 2 * T, 4);
        if (overlap(rs, ry) || overlap(rs, span(x, T, K, ldx, 2)) ||
            overlap(rs, span(w_fold, K, N, ldw, 2)) || overlap(rs, rc) ||
            (bias && overlap(rs, rb)))
            return QKN_ERR_ALIAS;
    }
    return QKN_OK;
}

// Deferred LayerNorm after its checks: the statistics pass into row_stats and the product that
// applies them, or (no workspace, or a shape the pass does not serve) the product alone.
int run_deferred_layernorm(int64_t T, int64_t K, int64_t N, float eps, const void* x,
                           int64_t ldx, const void* w_fold, int64_t ldw, const float* colsum,
                           const float* bias, void* y, int64_t ldy, float* row_stats,
                           void* stream)
{
    const hipStream_t s = (hipStream_t)stream;
    // the workspace holds (mean, 1/std) pairs as 8-byte stores: one that is not 8-byte aligned
    // is left unused
    if (row_stats && ((uintptr_t)row_stats & 7u) == 0 &&
        qkn::normproj_pipelined(T, K, N, x, ldx, w_fold, ldw, ldy, y)) {
        // statistics from one streaming pass over x; the product applies them in its epilogue
        const hipError_t e = qkn::launch_layernorm_stats(T, K, eps, x, ldx, row_stats, s);
        if (e != hipSuccess) return hip_status(e);
        return hip_status(qkn::launch_normproj(T, K, N, eps, qkn::kEpiLayerNormStats, x,
                                               ldx, w_fold, ldw, y, ldy, colsum, bias, row_stats,
                                               s));
    }
    return hip_status(qkn::launch_normproj(T, K, N, eps, qkn::kEpiLayerNorm, x, ldx, w_fold,
                                           ldw, y, ldy, colsum, bias, nullptr, s));
}

constexpr int kMaxDevices = 256;
std::atomic<float*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the device that owns `stream` (the current device for the
// null stream).
int noalloc_scratch(void* stream, float** out)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
    float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int cur = 0;
            e = hipGetDevice(&cur);
            if (e != hipSuccess) return hip_status(e);
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (cur != dev) {
                const hipError_t e2 = hipSetDevice(cur);
                if (e == hipSuccess) e = e2;
            }
            if (e != hipSuccess) return hip_status(e);
            if (addr == nullptr) return hip_status(hipErrorInvalidSymbol);
            p = (float*)addr;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return QKN_OK;
}

}  // namespace

QKN_API int normproj_deferred_layernorm(int64_t T, int64_t K, int64_t N, float eps, int dtype,
                                        const void* x, int64_t ldx, const void* w_fold,
                                        int64_t ldw, const float* colsum, const float* bias,
                                        void* y, int64_t ldy, float* row_stats, void* stream)
{
    const int st = check_deferred_layernorm(T, K, N, eps, dtype, x, ldx, w_fold, ldw, colsum,
                                            bias, y, ldy, row_stats);
    if (st != QKN_OK || T == 0 || N == 0) return st;
    return run_deferred_layernorm(T, K, N, eps, x, ldx, w_fold, ldw, colsum, bias, y, ldy,
                                  row_stats, stream);
}

QKN_API int normproj_deferred_layernorm_noalloc(int64_t T, int64_t K, int64_t N, float eps,
                                                int dtype, const void* x, int64_t ldx,
                                                const void* w_fold, int64_t ldw,
                                                const float* colsum, const float* bias, void* y,
                                                int64_t ldy, void* stream)
{
    int st = check_deferred_layernorm(T, K, N, eps, dtype, x, ldx, w_fold, ldw, colsum, bias, y,
                                      ldy, nullptr);
    if (st != QKN_OK || T == 0 || N == 0) return st;
    if (T > kNoallocRows) return QKN_ERR_SCRATCH;
    float* ws = nullptr;
    st = noalloc_scratch(stream, &ws);
    if (st != QKN_OK) return st;
    return run_deferred_layernorm(T, K, N, eps, x, ldx, w_fold, ldw, colsum, bias, y, ldy, ws,
                                  stream);
}

QKN_API int normproj_layernorm_unfused(int64_t T, int64_t K, int64_t N, float eps, int dtype,
                                       int gamma_dtype, const void* x, int64_t ldx,
                                       const void* gamma, const void* beta, const void* w,
                                       int64_t ldw, void* xn, int64_t ldxn, void* y, int64_t ldy,
                                       void* stream)
{
    int st = check_normproj(T, K, N, eps, dtype, x, ldx, w, ldw, y, ldy);
    if (st != QKN_OK) return st;
    if (!valid_dtype(gamma_dtype)) return QKN_ERR_DTYPE;
    if (ldxn < K || too_large(T, K, ldxn, 2)) return QKN_ERR_SHAPE;
    if (T == 0 || N == 0) return QKN_OK;
    if (xn == nullptr) return QKN_ERR_NULL;
    const int64_t gs = elem_size(gamma_dtype);
    if (((uintptr_t)xn & 1u) != 0 || ((uintptr_t)gamma % (uintptr_t)gs) != 0 ||
        ((uintptr_t)beta % (uintptr_t)gs) != 0)
        return QKN_ERR_ALIGN;
    const Range rxn = span(xn, T, K, ldxn, 2), ry = span(y, T, N, ldy, 2);
    const Range rg = span(gamma, 1, K, K, gs), rb = span(beta, 1, K, K, gs);
    if (overlap(rxn, span(x, T, K, ldx, 2)) || overlap(rxn, span(w, K, N, ldw, 2)) ||
        overlap(rxn, ry) || overlap(rxn, rg) || overlap(rxn, rb) || overlap(ry, rg) ||
        overlap(ry, rb))
        return QKN_ERR_ALIAS;
    hipError_t e = qkn::launch_layernorm_rows(T, K, eps, x, ldx, gamma, beta,
                                              gamma_dtype == QKN_BF16, xn, ldxn,
                                              (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(qkn::launch_normproj(T, K, N, eps, qkn::kEpiPlain,
                                           xn, ldxn, w, ldw, y, ldy, nullptr, nullptr, nullptr,
                                           (hipStream_t)stream));
}

namespace {

// Arguments of the layerwise QK-Norm that follows the projection (checked before any launch).
int check_qk_gammas(int64_t T, int64_t nq, int64_t nk, int gamma_dtype, const void* gamma_q,
                    const void* gamma_k, const void* y, int64_t ldy)
{
    if (!valid_dtype(gamma_dtype)) return QKN_ERR_DTYPE;
    if (T == 0) return QKN_OK;
    if (gamma_q == nullptr || (nk > 0 && gamma_k == nullptr)) return QKN_ERR_NULL;
    const int64_t gs = elem_size(gamma_dtype);
    const Range ry = span(y, T, nq + nk, ldy, 2);
    if (overlap(ry, span(gamma_q, 1, nq, nq, gs)) ||
        (nk > 0 && overlap(ry, span(gamma_k, 1, nk, nk, gs))))
        return QKN_ERR_ALIAS;
    return QKN_OK;
}

// Layerwise QK-Norm of the two column blocks of y [T, nq + nk], in place.
hipError_t qk_norm_in_place(int64_t T, int64_t nq, int64_t nk, float eps_qk, int gamma_dtype,
                            const void* gamma_q, const void* gamma_k, void* y, int64_t ldy,
                            void* stream)
{
    qkn::RowJob job = {};
    job.nseg = nk > 0 ? 2 : 1;
    job.T = T;
    job.eps = eps_qk;
    job.mode = qkn::kFused;
    job.bf16 = 1;
    job.gamma_bf16 = gamma_dtype == QKN_BF16;
    uint16_t* yq = (uint16_t*)y;
    job.seg[0] = {yq, yq, gamma_q, ldy, ldy, nq, (float)(1.0 / (double)nq), nullptr, nullptr, 0,
                  0, nullptr};
    if (nk > 0)
        job.seg[1] = {yq + nq, yq + nq, gamma_k, ldy, ldy, nk, (float)(1.0 / (double)nk), nullptr,
                      nullptr, 0, 0, nullptr};
    return qkn::launch_rows(job, (hipStream_t)stream);
}

}  // namespace

QKN_API int qknorm_project_eliminated(int64_t T, int64_t K, int64_t nq, int64_t nk,
                                      float eps_qk, float eps_pre, int exact, int gamma_dtype,
                                      const void* x, int64_t ldx, const void* w_qk, int64_t ldw,
                                      const void* gamma_q, const void* gamma_k, void* y,
                                      int64_t ldy, void* stream)
{
    if (nq < 1 || nk < 0 || nq > kMaxExtentBytes || nk > kMaxExtentBytes) return QKN_ERR_SHAPE;
    if (!valid_eps(eps_pre)) return QKN_ERR_EPS;
    if (exact != 0 && exact != 1) return QKN_ERR_SHAPE;
    const int64_t N = nq + nk;
    int st = check_normproj(T, K, N, eps_qk, QKN_BF16, x, ldx, w_qk, ldw, y, ldy);
    if (st != QKN_OK) return st;
    st = check_qk_gammas(T, nq, nk, gamma_dtype, gamma_q, gamma_k, y, ldy);
    if (st != QKN_OK || T == 0) return st;
    // p = x W' (scaled by the pre-norm's 1/rms when exact), stored in y in bf16
    // (ordinary stores: the row kernel below reads y straight back)
    hipError_t e = qkn::launch_normproj(T, K, N, eps_pre,
                                        (exact ? qkn::kEpiRms : qkn::kEpiPlain) |
                                            qkn::kEpiKeepCached,
                                        x, ldx, w_qk, ldw, y, ldy, nullptr, nullptr, nullptr,
                                        (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(qk_norm_in_place(T, nq, nk, eps_qk, gamma_dtype, gamma_q, gamma_k, y, ldy,
                                       stream));
}

QKN_API int qknorm_project_unfused(int64_t T, int64_t K, int64_t nq, int64_t nk, float eps_qk,
                                   float eps_pre, int gamma_dtype, const void* x, int64_t ldx,
                                   const void* gamma_pre, const void* w, int64_t ldw,
                                   const void* gamma_q, const void* gamma_k, void* xn,
                                   int64_t ldxn, void* y, int64_t ldy, void* stream)
{
    if (nq < 1 || nk < 0 || nq > kMaxExtentBytes || nk > kMaxExtentBytes) return QKN_ERR_SHAPE;
    if (!valid_eps(eps_qk)) return QKN_ERR_EPS;
    const int64_t N = nq + nk;
    // shapes, pointers and aliasing of the norm and the product are checked by
    // unfused_rms_product before its first launch; the QK-Norm's arguments here
    int st = check_normproj(T, K, N, eps_pre, QKN_BF16, x, ldx, w, ldw, y, ldy);
    if (st != QKN_OK) return st;
    st = check_qk_gammas(T, nq, nk, gamma_dtype, gamma_q, gamma_k, y, ldy);
    if (st != QKN_OK) return st;
    if (T > 0 && xn != nullptr && ldxn >= K) {
        const Range rxn = span(xn, T, K, ldxn, 2);
        const int64_t gs = elem_size(gamma_dtype);
        if (overlap(rxn, span(gamma_q, 1, nq, nq, gs)) ||
            (nk > 0 && overlap(rxn, span(gamma_k, 1, nk, nk, gs))))
            return QKN_ERR_ALIAS;
    }
    // the pre-norm and the plain product, p kept in the caches for the QK-Norm launch
    st = unfused_rms_product(T, K, N, eps_pre, QKN_BF16, gamma_dtype, x, ldx, gamma_pre,
                             w, ldw, xn, ldxn, y, ldy, true, stream);
    if (st != QKN_OK || T == 0) return st;
    return hip_status(qk_norm_in_place(T, nq, nk, eps_qk, gamma_dtype, gamma_q, gamma_k, y, ldy,
                                       stream));
}

QKN_API int qkn_device_copy(void* dst, const void* src, int64_t nbytes, void* stream)
{
    if (nbytes < 0 || nbytes > kMaxExtentBytes) return QKN_ERR_SHAPE;
    if (nbytes == 0) return QKN_OK;
    if (dst == nullptr || src == nullptr) return QKN_ERR_NULL;
    if (overlap(span(dst, 1, nbytes, nbytes, 1), span(src, 1, nbytes, nbytes, 1)))
        return QKN_ERR_ALIAS;
    return hip_status(qkn::launch_copy(dst, src, nbytes, (hipStream_t)stream));
}

}  // extern "C"
