// Norm-then-project on gfx950 with the normalisation deferred to the product's output
// ("FlashNorm: Fast Normalization for Transformers", abstract, items (i) and (ii), and its
// extension to LayerNorm), plus the one-time weight folds, the LayerNorm row kernel of the
// unfused baseline and a plain streaming copy used for calibration.
//
// acc[t, n] = sum_k x[t, k] * w[k, n] with x row-major [T, K] and W' row-major [K, N] (the
// layout of the weight the fold scales), on v_mfma_f32_32x32x16_bf16; the W' fragments, which
// hold 8 consecutive k of one column per lane, come from LDS through the gfx950 transpose load
// ds_read_b64_tr_b16. The epilogue is one of
//   plain      y = acc
//   RMSNorm    y = r_t * acc,                          r_t = 1 / sqrt(mean(x_t^2) + eps)
//   LayerNorm  y = r_t * (acc - mu_t * c[n]) + b[n],   r_t = 1 / sqrt(var(x_t) + eps)
// with c the column sums of the folded weight and b = beta W. The row statistics come from the
// same x values that feed the matrix cores, accumulated on the VALU while the MFMAs run, so no
// extra pass over x is needed and the reduction proceeds beside the product instead of before
// it; for LayerNorm they can instead come from one streaming pass over x (layernorm_stats_kernel)
// that the product's epilogue reads. LayerNorm accumulates sum(x - x0) and sum((x - x0)^2) with
// x0 the row's first element, so that the one-pass variance does not cancel for rows whose mean
// is large against their spread.
//
// Pipelined kernel (K a multiple of the k-tile; N, strides and pointers 16-byte friendly): a
// workgroup owns a BM x BN output tile.
// Its k-tiles of x and W' reach LDS by direct global->LDS DMA (global_load_lds_dwordx4, 1 KB per
// wavefront instruction, tile base in scalar registers and a 32-bit offset per lane), either
// through an NST-deep ring of whole k-tiles or, for 256 x 256 tiles with k-tiles of 64 (64 KB
// each, so only two whole k-tiles fit in LDS), through a ring of five 32 KB parts: the x part of
// a k-tile is requested two k-tiles ahead and its W' part one ahead, which keeps one and a half
// k-tiles in flight instead of one. With five parts or with 3 or more whole-tile stages, the
// requests are spread over the k steps of the current k-tile rather than issued in one burst.
// The x
// tile's rows have their 16-byte chunks XOR-swizzled so the fragment reads of 16 consecutive
// rows fall in 16 distinct bank groups; the W' tile's k rows have their 64-byte segments
// swizzled by the row so that the 4 rows a transpose load reads fall in distinct bank groups. Wavefronts own WM x WN sub-tiles of 32 x 32 MFMA blocks, with the W'
// fragment as the MFMA's first operand so that a lane's accumulator holds one output row and
// runs of 4 consecutive columns. The WN wavefronts that hold the same rows' x fragments take
// turns over the k steps to accumulate the row statistics (sums of squares through
// v_dot2c_f32_bf16 for RMSNorm), and their partials are added through LDS in a fixed order.
// The epilogue applies the row scale, rounds to bf16, writes the tile to LDS 8 bytes at a time
// and stores it so each lane writes 16 contiguous bytes, non-temporally unless the caller reads
// the output straight back. Workgroups are remapped so that each XCD works on a block of the
// tile grid whose row and column panels its L2 can share (the split chosen per grid shape).
//
// Element kernel (any K, strides and 2-byte alignment): 128 x 128 tiles staged element by
// element through padded LDS rows.
//
// Small T (<= 16) is a matrix-vector product bound by streaming W' once: 16x16x32 MFMAs with the
// tokens as rows, W' and x staged through per-wavefront LDS by DMA, K split across a
// workgroup's wavefronts (normproj_mvl_kernel).

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

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_at(const uint16_t* p, int64_t i)
{
    return __uint_as_float((uint32_t)p[i] << 16);
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// s + a.lo * a.lo + a.hi * a.hi for a packed pair of bf16 (v_dot2c_f32_bf16: the products of
// bf16 values are exact in fp32, one instruction per two elements).
__device__ __forceinline__ float dot2_sq(uint32_t a, float s)
{
    const bf16x2v v = __builtin_bit_cast(bf16x2v, a);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
}

// Row statistics of 8 bf16 values: RMSNorm sums squares; LayerNorm sums the values and their
// squares after subtracting the row's shift x0 (fp32, so that the variance does not cancel).
template <int EPI>
__device__ __forceinline__ void accum_stats(const u32x4& v, float x0, float& s1, float& s2)
{
    if constexpr (EPI == kEpiLayerNorm) {
        const float e[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                            bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float d = e[j] - x0;
            s1 += d;
            s2 = fmaf(d, d, s2);
        }
    } else {
        s2 = dot2_sq(v.x, s2);
        s2 = dot2_sq(v.y, s2);
        s2 = dot2_sq(v.z, s2);
        s2 = dot2_sq(v.w, s2);
    }
}

// Row scale (and LayerNorm mean) from the row's sums over K columns.
template <int EPI>
__device__ __forceinline__ void row_scale(float s1, float s2, float x0, float inv_k, float eps,
                                          float& rs, float& mu)
{
    if constexpr (EPI == kEpiLayerNorm) {
        const float ms = s1 * inv_k;                          // mean of x - x0
        const float var = fmaxf(fmaf(-ms, ms, s2 * inv_k), 0.0f);
        rs = rsqrtf(var + eps);
        mu = x0 + ms;
    } else {
        rs = rsqrtf(s2 * inv_k + eps);
        mu = 0.0f;
    }
}

// Row statistics accumulated inside the product (RMSNorm, LayerNorm) or read from memory.
template <int EPI>
constexpr bool kStatsInLoop = EPI == kEpiRms || EPI == kEpiLayerNorm;
template <int EPI>
constexpr bool kLayerNormOut = EPI == kEpiLayerNorm || EPI == kEpiLayerNormStats;

template <int EPI>
__device__ __forceinline__ float epilogue(float acc, float rs, float mu, float c, float b)
{
    if constexpr (EPI == kEpiRms) return acc * rs;
    if constexpr (kLayerNormOut<EPI>) return fmaf(rs, fmaf(-mu, c, acc), b);
    return acc;
}

// ------------------------------------------------------------------------------------------
// Pipelined kernel.

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS at lds_off + 16 * lane, addressed as a
// wavefront-uniform 64-bit base in scalar registers plus a 32-bit byte offset per lane (no
// 64-bit address arithmetic per request). Issued through inline assembly so that the compiler
// does not wait for it before unrelated LDS reads; the kernel awaits completion with s_waitcnt
// vmcnt (vector loads complete in issue order). One wait state separates the M0 write from the
// DMA (a gfx9-family hazard). M0 is declared clobbered; no other instruction in these kernels
// uses it (checked in the generated code).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_off)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 ::"s"(__builtin_amdgcn_readfirstlane(lds_off)), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt fields: vmcnt[3:0] and [15:14], expcnt[6:4] = 7 (no wait), lgkmcnt[11:8] = 15
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most `later` k-tiles of CPT DMA requests each are still in flight (0 <= later
// <= L): the requests complete in issue order, so everything issued before them has landed.
template <int CPT, int L>
__device__ __forceinline__ void wait_tiles(int later)
{
    if constexpr (L == 0) {
        wait_vmcnt<0>();
    } else {
        if (later >= L) wait_vmcnt<L * CPT>();
        else wait_tiles<CPT, L - 1>(later);
    }
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

// Physical 16-byte chunk of logical chunk c in k row r of a row-major W' tile. A transpose
// load reads 4 consecutive rows at the same 64 bytes per 16-lane group; xoring the 64-byte
// segment index with r % 4 puts those rows in 4 different 64-byte bank groups.
__device__ __forceinline__ int swz_kn(int c, int r) { return c ^ ((r & 3) << 2); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// ds_read_b64_tr_b16 at LDS address p (8-byte aligned).
__device__ __forceinline__ u32x2 lds_tr16(const char* p)
{
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p));
}

// NTS: non-temporal output stores (the output leaves the library) or ordinary ones.
// W' is row-major [K, N]: its k-tile lands in LDS as BK rows of BN columns and the MFMA
// fragments (8 consecutive k of one column per lane) are read with the LDS transpose load
// ds_read_b64_tr_b16 (gfx950). Within each 16-lane group that instruction hands lane i,
// element j the 16-bit element i % 4 of the 8 bytes that lane 4 j + i / 4 addressed: when lane
// 4 r + c of a group addresses columns 4 c .. 4 c + 3 of row r of a 4-row block, lane i
// receives column i of rows 0..3.
// KG > 1 splits every k-tile's k steps among KG groups of WM x WN wavefronts (group g takes the
// steps s with s % KG == g): each wavefront then holds a KG times larger share of the output
// tile for the same number of wavefronts per CU, which cuts the LDS fragment bytes per MFMA;
// after the last k-tile groups 1..KG-1 hand their accumulators to group 0 through LDS, which
// adds them in group order (a fixed order, so results do not depend on timing).
template <int BM, int BN, int WM, int WN, int NST, int BK, int EPI, bool RING, bool NTS, int KG>
__global__ __launch_bounds__(WM * WN * KG * 64) void normproj_pipe_kernel(
    int64_t T, int64_t K, int64_t N, float eps, float inv_k, const uint16_t* __restrict__ x,
    int64_t ldx, const uint16_t* __restrict__ w, int64_t ldw, uint16_t* __restrict__ y,
    int64_t ldy, int nbm, int nbn, const float* __restrict__ colsum,
    const float* __restrict__ bias, const float* __restrict__ rowstats)
{
    constexpr int NWP = WM * WN;            // wavefront positions on the output tile
    constexpr int NW = NWP * KG, NT = NW * kWave;
    constexpr int ROWB = BK * 2;            // bytes per tile row
    constexpr int RPC = 1024 / ROWB;        // tile rows per 1 KB DMA chunk
    constexpr int LPR = ROWB / 16;          // lanes per tile row within a chunk
    // W' part: BK rows of BN columns (n contiguous)
    constexpr int ROWB_B = BN * 2;
    constexpr int RPC_B = 1024 / ROWB_B, LPR_B = ROWB_B / 16;
    constexpr int PART_A = BM * ROWB, PART_B = BK * ROWB_B, STAGE = PART_A + PART_B;
    constexpr int CA = BM / RPC, CB = BK / RPC_B;
    static_assert(RPC_B >= 1 && LPR_B <= kWave, "W' tile rows");
    static_assert(CA % NW == 0 && CB % NW == 0, "DMA chunks must divide among the wavefronts");
    constexpr int CPA = CA / NW, CPB = CB / NW;  // DMA instructions per wavefront per part
    constexpr int KS = BK / 16;
    static_assert(KS % KG == 0, "k groups take equal shares of the k steps");
    constexpr int KSG = KS / KG;            // k steps per wavefront per k-tile
    static_assert(!RING || (BM == BN && (CPA + CPB) % KSG == 0), "ring: five equal parts");
    constexpr int PIPE = RING ? 5 * PART_A : NST * STAGE;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int CP = BN + 8;              // epilogue tile pitch (bf16)
    // after the k loop the pipeline's LDS holds the output tile (where the k groups' accumulators
    // are exchanged first) and the per-row / per-column epilogue operands
    constexpr int CT_BYTES = BM * CP * 2;
    constexpr int XCH = (KG - 1) * NWP * TM * TN * 16 * kWave * 4;
    constexpr int OFF_RS = CT_BYTES > XCH ? CT_BYTES : XCH, OFF_MU = OFF_RS + BM * 4;
    constexpr int OFF_PART = OFF_MU + BM * 4, OFF_CS = OFF_PART + 2 * WN * KG * BM * 4;
    constexpr int OFF_BS = OFF_CS + BN * 4, EPI_END = OFF_BS + BN * 4;
    constexpr int SMEM = PIPE > EPI_END ? PIPE : EPI_END;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];
    float* rs_lds = (float*)(smem + OFF_RS);
    float* mu_lds = (float*)(smem + OFF_MU);
    float* part_lds = (float*)(smem + OFF_PART);  // per wave column and k group: row sums
    float* cs_lds = (float*)(smem + OFF_CS);
    float* bs_lds = (float*)(smem + OFF_BS);

    const int tid = (int)threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wavefront-uniform
    const int kg = KG == 1 ? 0 : wave / NWP, wp = KG == 1 ? wave : wave % NWP;
    const int wm = wp / WN, wn = wp % WN;
    const int nb = nbm * nbn;
    int bid = (int)blockIdx.x;
    // Workgroup b runs on XCD b % 8. Each XCD takes a block of the tile grid: the row panels
    // split gx ways and the column panels 8 / gx ways, with gx chosen so that the row and column
    // panels one XCD's L2 must hold are fewest (ties go to fewer row panels: x streams from
    // HBM, W' is shared by every row panel); within the block, tiles go row by row. Grids that
    // do not split evenly keep plain contiguous ranges of tiles per XCD.
    int64_t m0, n0;
    int gx = 0;
    {
        int best = 0x7fffffff;
        for (int g = 1; g <= 8; g *= 2)
            if (nbm % g == 0 && nbn % (8 / g) == 0 && nbm / g + nbn / (8 / g) <= best) {
                best = nbm / g + nbn / (8 / g);
                gx = g;
            }
    }
    if (gx) {
        const int xcd = bid & 7, j = bid >> 3;
        const int gy = 8 / gx, rpg = nbm / gx, cpg = nbn / gy;
        m0 = (int64_t)((xcd / gy) * rpg + j / cpg) * BM;
        n0 = (int64_t)((xcd % gy) * cpg + j % cpg) * BN;
    } else {
        if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
        m0 = (int64_t)(bid / nbn) * BM;
        n0 = (int64_t)(bid % nbn) * BN;
    }
    // LDS byte address of the pipeline buffer; DMA destinations are offsets from it, kept in
    // scalar registers
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void*)smem;

    // Sources of the DMA chunks this lane fetches (fixed across k): chunks wave * CPA + c of the
    // x part and wave * CPB + c of the W' part. Out-of-range rows are clamped to the last valid
    // row: they only feed output rows / columns that are never stored.
    // Each request is a wavefront-uniform base (the tile's first row at column k0) plus a 32-bit
    // byte offset per lane (row offset, which a 256-row tile keeps below 2^32 for ld < 2^23).
    const int lrow = lane / LPR;
    uint32_t offa[CPA], offb[CPB];
#pragma unroll
    for (int c = 0; c < CPA; ++c) {
        const int trow = (wave * CPA + c) * RPC + lrow;
        const int64_t r = m0 + trow < T ? m0 + trow : T - 1;
        offa[c] = (uint32_t)(((r - m0) * ldx + swz<BK>(lane % LPR, trow) * 8) * 2);
    }
#pragma unroll
    for (int c = 0; c < CPB; ++c) {
        // k row trow of the tile, 16-byte chunk (8 columns) given by the lane's slot; chunks past
        // N (a multiple of 8) read the last chunk and feed columns never stored
        const int trow = (wave * CPB + c) * RPC_B + lane / LPR_B;
        const int64_t col = n0 + (int64_t)swz_kn(lane % LPR_B, trow) * 8;
        offb[c] = (uint32_t)((trow * ldw + ((col < N ? col : N - 8) - n0)) * 2);
    }
    const uint16_t* xa = x + m0 * ldx;
    const uint16_t* wb = w + n0;

    // part: byte offset of the destination part within the pipeline buffer
    auto dma_a = [&](int c, uint32_t part, int64_t k0) {
        dma16s((const void*)(xa + k0), offa[c], lds0 + part + (uint32_t)(wave * CPA + c) * 1024u);
    };
    auto dma_b = [&](int c, uint32_t part, int64_t k0) {
        dma16s((const void*)(wb + k0 * ldw), offb[c],
               lds0 + part + (uint32_t)(wave * CPB + c) * 1024u);
    };
    auto issue_tile = [&](int slot, int64_t k0) {
        const uint32_t base = (uint32_t)(slot * STAGE);
#pragma unroll
        for (int c = 0; c < CPA; ++c) dma_a(c, base, k0);
#pragma unroll
        for (int c = 0; c < CPB; ++c) dma_b(c, base + PART_A, k0);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    const int frow = lane & 31, fk = lane >> 5;
    // W' fragment reads: lane 4 r + c of its 16-lane group g addresses row 8 (g / 2) + r (+ 4
    // for the second half of the 8 k) at columns 16 (g % 2) + 4 c .. + 3 of 32-column block j;
    // boff[j] is that byte offset within the first k step (later steps add 16 rows, which
    // keeps the row modulo 4 and so the swizzle)
    uint32_t boff[TN];
    {
        const int g = lane >> 4, i = lane & 15;
        const int r = 8 * (g >> 1) + (i >> 2);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = wn * WTN + j * 32 + 16 * (g & 1) + 4 * (i & 3);
            boff[j] = (uint32_t)(r * ROWB_B + (swz_kn(col >> 3, r) << 4) + (col & 7) * 2);
        }
    }
    float s1[TM], s2[TM], x0[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        s1[i] = s2[i] = x0[i] = 0.0f;
        if constexpr (EPI == kEpiLayerNorm) {
            const int64_t r = m0 + wm * WTM + i * 32 + frow;
            x0[i] = bf16_at(x, (r < T ? r : T - 1) * ldx);
        }
    }

    const int nk = (int)(K / BK);
    if constexpr (RING) {
        // part p holds the x part of k-tile t when p == 2t mod 5 and its W' part when
        // p == 2t + 1 mod 5: the x part (streamed from HBM) is requested two k-tiles ahead, the
        // W' part (shared by every row panel, mostly cache-resident) one ahead
#pragma unroll
        for (int c = 0; c < CPA; ++c) dma_a(c, 0u, 0);
#pragma unroll
        for (int c = 0; c < CPB; ++c) dma_b(c, (uint32_t)PART_A, 0);
        if (nk > 1) {
#pragma unroll
            for (int c = 0; c < CPA; ++c) dma_a(c, 2u * PART_A, BK);
        }
    } else {
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
            if (s < nk) issue_tile(s, (int64_t)s * BK);
    }

    int pa = 0;  // ring: part holding the x half of k-tile kt (2 kt mod 5)
    for (int kt = 0; kt < nk; ++kt) {
        constexpr int CPT = CPA + CPB;
        const int pb = pa == 4 ? 0 : pa + 1;        // W' half of k-tile kt
        const int pnb = pa >= 2 ? pa - 2 : pa + 3;  // W' half of k-tile kt + 1
        const int pna = pa >= 1 ? pa - 1 : 4;       // x half of k-tile kt + 2
        if constexpr (RING) {
            // k-tile kt must have landed; the x part of k-tile kt + 1 may stay in flight
            if (kt + 1 < nk) wait_vmcnt<CPA>();
            else wait_vmcnt<0>();
        } else {
            // k-tile kt must have landed; up to NST-2 later tiles stay in flight
            const int later = (nk - 1 - kt) < (NST - 2) ? (nk - 1 - kt) : (NST - 2);
            wait_tiles<CPT, (NST > 2 ? NST - 2 : 0)>(later);
        }
        __syncthreads();  // every wavefront's DMA has landed; the parts of k-tile kt-1 are free
        // whole-tile stages: with NST >= 3 the next k-tile's requests are spread over the k steps
        // (two later k-tiles are still in flight meanwhile); with 2 stages they go out at once
        constexpr bool SPREAD = !RING && NST >= 3 && CPT % KSG == 0;
        if constexpr (!RING && !SPREAD) {
            if (kt + NST - 1 < nk) issue_tile((kt + NST - 1) % NST, (int64_t)(kt + NST - 1) * BK);
        }
        const char* As = RING ? smem + pa * PART_A : smem + (kt % NST) * STAGE;
        const char* Bs = RING ? smem + pb * PART_A : As + PART_A;
#pragma unroll
        for (int q = 0; q < KSG; ++q) {
            const int ks = KG == 1 ? q : q * KG + kg;  // this wavefront's q-th k step
            u32x4 af[TM], bfr[TN];
            const int kc = ks * 2 + fk;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + frow;
                af[i] = *(const u32x4*)(As + r * ROWB + (swz<BK>(kc, r) << 4));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                // rows ks * 16 + ...: the swizzle depends on the row modulo 4 only
                const char* p = Bs + ks * 16 * ROWB_B + boff[j];
                const u32x2 lo = lds_tr16(p), hi = lds_tr16(p + 4 * ROWB_B);
                bfr[j] = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
            if constexpr (kStatsInLoop<EPI>) {
                // the WN wavefronts of a k group holding the same rows take turns over its steps
                if (q % WN == wn) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) accum_stats<EPI>(af[i], x0[i], s1[i], s2[i]);
                }
            }
            // W' fragment as the MFMA's A operand: the accumulator of a 32 x 32 block then holds
            // output row (token) lane % 32 and 4 consecutive columns per group of 4 values
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
            if constexpr (RING) {
                // this k step's share of the next DMA requests, spread over the k steps so the
                // MFMA issue is never held behind a burst of them: the W' part of k-tile kt+1
                // first, then the x part of k-tile kt+2 (parts freed by the barrier above)
                constexpr int PER = CPT / KSG;
#pragma unroll
                for (int h = 0; h < PER; ++h) {
                    const int c = q * PER + h;
                    if (c < CPB) {
                        if (kt + 1 < nk)
                            dma_b(c, (uint32_t)(pnb * PART_A), (int64_t)(kt + 1) * BK);
                    } else {
                        if (kt + 2 < nk)
                            dma_a(c - CPB, (uint32_t)(pna * PART_A), (int64_t)(kt + 2) * BK);
                    }
                }
            }
            if constexpr (SPREAD) {
                constexpr int PER = CPT / KSG;
                const int nt = kt + NST - 1;
                const uint32_t base = (uint32_t)((nt % NST) * STAGE);
#pragma unroll
                for (int h = 0; h < PER; ++h) {
                    const int c = q * PER + h;
                    if (nt < nk) {
                        if (c < CPA) dma_a(c, base, (int64_t)nt * BK);
                        else dma_b(c - CPA, base + PART_A, (int64_t)nt * BK);
                    }
                }
            }
        }
        pa = pa >= 3 ? pa - 3 : pa + 2;
    }
    __syncthreads();  // every wavefront is done with the pipeline's LDS (no DMA is in flight)
    if constexpr (KG > 1) {
        // k groups 1.. store their accumulators (16 bytes per lane, lanes contiguous); group 0
        // adds them in group order
        f32x4* xch = (f32x4*)smem;
        auto slot = [&](int g, int i, int j, int e4) {
            return ((((g - 1) * NWP + wp) * TM + i) * TN * 4 + j * 4 + e4) * kWave + lane;
        };
        if (kg > 0) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4)
                        xch[slot(kg, i, j, e4)] = f32x4{acc[i][j][4 * e4], acc[i][j][4 * e4 + 1],
                                                        acc[i][j][4 * e4 + 2],
                                                        acc[i][j][4 * e4 + 3]};
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int g = 1; g < KG; ++g)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int e4 = 0; e4 < 4; ++e4) {
                            const f32x4 v = xch[slot(g, i, j, e4)];
                            acc[i][j][4 * e4] += v.x;
                            acc[i][j][4 * e4 + 1] += v.y;
                            acc[i][j][4 * e4 + 2] += v.z;
                            acc[i][j][4 * e4 + 3] += v.w;
                        }
        }
        __syncthreads();  // the exchange area becomes the output tile
    }

    if constexpr (kLayerNormOut<EPI>) {
        for (int c = tid; c < BN; c += NT) {
            const int64_t gn = n0 + c;
            cs_lds[c] = gn < N ? colsum[gn] : 0.0f;
            bs_lds[c] = (gn < N && bias) ? bias[gn] : 0.0f;
        }
    }
    if constexpr (EPI == kEpiLayerNormStats) {
        for (int r = tid; r < BM; r += NT) {
            const int64_t gr = m0 + r < T ? m0 + r : T - 1;
            const f32x2 st = *(const f32x2*)(rowstats + 2 * gr);
            mu_lds[r] = st.x;
            rs_lds[r] = st.y;
        }
        __syncthreads();  // row statistics and column terms visible
    }
    if constexpr (kStatsInLoop<EPI>) {
        // lanes l and l + 32 summed the two halves of each 16-wide k step of the same row
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const float q2 = s2[i] + __shfl_xor(s2[i], 32);
            const float q1 = s1[i] + __shfl_xor(s1[i], 32);
            if (lane < 32) {
                part_lds[(0 * WN * KG + kg * WN + wn) * BM + wm * WTM + i * 32 + lane] = q1;
                part_lds[(1 * WN * KG + kg * WN + wn) * BM + wm * WTM + i * 32 + lane] = q2;
            }
        }
        __syncthreads();
        // one thread per tile row: add the wave columns' partials in a fixed order
        for (int r = tid; r < BM; r += NT) {
            float q1 = 0.0f, q2 = 0.0f;
#pragma unroll
            for (int c = 0; c < WN * KG; ++c) {
                q1 += part_lds[(0 * WN * KG + c) * BM + r];
                q2 += part_lds[(1 * WN * KG + c) * BM + r];
            }
            const int64_t gr = m0 + r;
            const float xr0 = EPI == kEpiLayerNorm ? bf16_at(x, (gr < T ? gr : T - 1) * ldx) : 0.0f;
            float rs, mu;
            row_scale<EPI>(q1, q2, xr0, inv_k, eps, rs, mu);
            rs_lds[r] = rs;
            if constexpr (EPI == kEpiLayerNorm) mu_lds[r] = mu;
        }
        __syncthreads();  // row scales visible
    }

    // output row wm*WTM + i*32 + lane%32; columns wn*WTN + j*32 + 8g + 4(lane/32) + 0..3 in
    // accumulator entries 4g .. 4g+3, rounded to bf16 and written 8 bytes at a time
    uint16_t* ct = (uint16_t*)smem;
    if (KG == 1 || kg == 0) {  // group 0 holds the summed accumulators
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * WTM + i * 32 + (lane & 31);
            float rs = 1.0f, mu = 0.0f;
            if constexpr (EPI != kEpiPlain) rs = rs_lds[r];
            if constexpr (kLayerNormOut<EPI>) mu = mu_lds[r];
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
                    if constexpr (EPI == kEpiRms) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] *= rs;
                    }
                    if constexpr (kLayerNormOut<EPI>) {
                        const f32x4 cs = *(const f32x4*)(cs_lds + c);
                        const f32x4 bs = *(const f32x4*)(bs_lds + c);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[e] = epilogue<EPI>(v[e], rs, mu, cs[e], bs[e]);
                    }
                    const u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                    *(u32x2*)(ct + r * CP + c) = pk;
                }
        }
    }
    __syncthreads();
    // each thread stores one 16-byte column chunk of every RSTEP-th row: all its LDS reads are
    // issued before the first global store
    constexpr int C8 = BN / 8;
    static_assert(NT % C8 == 0 && (BM * C8) % NT == 0, "store loop shape");
    constexpr int RSTEP = NT / C8, ITER = BM * C8 / NT;
    const int c8 = tid % C8, r0 = tid / C8;
    const int64_t gn = n0 + c8 * 8;
    u32x4 out[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it)
        out[it] = *(const u32x4*)(ct + (r0 + it * RSTEP) * CP + c8 * 8);
    uint16_t* yp = y + (m0 + r0) * ldy + gn;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        if (m0 + r0 + it * RSTEP < T && gn < N) {
            uint16_t* p = yp + (int64_t)it * RSTEP * ldy;
            if constexpr (NTS) store_stream(p, out[it]);
            else *(u32x4*)p = out[it];
        }
    }
}

// Element kernel: any K, any row strides, any 2-byte alignment of x, W' and y. 128 x 128 tiles, k-tiles of 64; each thread loads 32 elements of x and of W' per
// k-tile with 2-byte loads (consecutive threads on consecutive elements of a row), which it
// stores into padded LDS rows k-contiguous for both operands before the matrix-core loop of
// the generic kernel. Elements past T, N or K are zero. The row statistics are summed from the
// staged x tile in LDS (two threads per row, 32 columns each), elements past K left out.
template <int EPI>
__global__ __launch_bounds__(kThreads) void normproj_elem_kernel(
    int64_t T, int64_t K, int64_t N, float eps, float inv_k, const uint16_t* __restrict__ x,
    int64_t ldx, const uint16_t* __restrict__ w, int64_t ldw, uint16_t* __restrict__ y,
    int64_t ldy, int nbm, int nbn, const float* __restrict__ colsum,
    const float* __restrict__ bias)
{
    constexpr int kPer = kBM * kBK / kThreads;  // 32 elements per thread and operand
    __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kPitch];
    __shared__ float rstd[kBM];
    __shared__ float mean[kBM];
    __shared__ float part[2][2][kBM];

    const int nb = nbm * nbn;
    int bid = (int)blockIdx.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
    const int64_t m0 = (int64_t)(bid / nbn) * kBM;
    const int64_t n0 = (int64_t)(bid % nbn) * kBN;
    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;

    uint16_t ra[kPer], rb[kPer];
    // element e of this thread: x tile row (e * 256 + tid) / 64, column tid % 64; W' element
    // (k, n) with n = (e * 256 + tid) % 128 and k = (e * 256 + tid) / 128 (consecutive threads
    // read consecutive columns), stored transposed (k contiguous) for the fragment reads
    auto load_tiles = [&](int64_t k0) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = e * kThreads + tid;
            const int64_t gm = m0 + idx / kBK, gk = k0 + idx % kBK;
            ra[e] = (gm < T && gk < K) ? x[gm * ldx + gk] : (uint16_t)0;
            const int64_t gn = n0 + idx % kBN, wk = k0 + idx / kBN;
            rb[e] = (gn < N && wk < K) ? w[wk * ldw + gn] : (uint16_t)0;
        }
    };
    auto store_tiles = [&]() {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = e * kThreads + tid;
            As[(idx / kBK) * kPitch + idx % kBK] = ra[e];
            Bs[(idx % kBN) * kPitch + idx / kBN] = rb[e];
        }
    };

    // statistics: thread tid sums row tid / 2, columns 32 (tid % 2) .. + 31 of each x tile
    const int srow = tid >> 1, shalf = tid & 1;
    float s1 = 0.0f, s2 = 0.0f, x0 = 0.0f;
    if constexpr (EPI == kEpiLayerNorm) {
        const int64_t r = m0 + srow;
        x0 = bf16_at(x, (r < T ? r : T - 1) * ldx);
    }
    auto tile_stats = [&](int64_t k0) {
        if constexpr (EPI != kEpiPlain) {
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                const int col = shalf * 32 + c;
                if (k0 + col < K) {
                    const float v = __uint_as_float((uint32_t)As[srow * kPitch + col] << 16);
                    if constexpr (EPI == kEpiLayerNorm) {
                        const float d = v - x0;
                        s1 += d;
                        s2 = fmaf(d, d, s2);
                    } else {
                        s2 = fmaf(v, v, s2);
                    }
                }
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
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    for (int64_t kt = 0; kt < nk; ++kt) {
        store_tiles();
        __syncthreads();
        if (kt + 1 < nk) load_tiles((kt + 1) * kBK);
        tile_stats(kt * kBK);
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
    }

    if constexpr (EPI != kEpiPlain) {
        part[0][shalf][srow] = s1;
        part[1][shalf][srow] = s2;
        __syncthreads();
        if (tid < kBM) {
            const float q1 = part[0][0][tid] + part[0][1][tid];
            const float q2 = part[1][0][tid] + part[1][1][tid];
            const int64_t r = m0 + tid;
            const float xr0 = EPI == kEpiLayerNorm ? bf16_at(x, (r < T ? r : T - 1) * ldx) : 0.0f;
            float rs, mu;
            row_scale<EPI>(q1, q2, xr0, inv_k, eps, rs, mu);
            rstd[tid] = rs;
            mean[tid] = mu;
        }
        __syncthreads();
    }

    // accumulator of a 32 x 32 block: lane holds column lane % 32 and, for e in 0..15, row
    // 8 (e / 4) + 4 (lane / 32) + e % 4
    const int out_col = lane & 31;
    const int out_row = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t gn = n0 + wn * 64 + j * 32 + out_col;
            float cs = 0.0f, bs = 0.0f;
            if constexpr (EPI == kEpiLayerNorm) {
                if (gn < N) {
                    cs = colsum[gn];
                    if (bias) bs = bias[gn];
                }
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = wm * 64 + i * 32 + 8 * (e / 4) + out_row + (e % 4);
                const int64_t gm = m0 + r;
                float v = acc[i][j][e];
                if constexpr (EPI == kEpiRms) v *= rstd[r];
                if constexpr (EPI == kEpiLayerNorm) v = epilogue<EPI>(v, rstd[r], mean[r], cs, bs);
                if (gm < T && gn < N) y[gm * ldy + gn] = to_bf16(v);
            }
        }
    }
}

// Matrix-vector form for T <= 16 on the matrix cores: v_mfma_f32_16x16x32_bf16 with the (up
// to 16) tokens as the M dimension and 16 columns of W' as N. Fragment layout: lane l supplies
// A[l % 16][8 (l / 16) .. + 7] and B[8 (l / 16) .. + 7][l % 16]; it receives
// D[4 (l / 16) + i][l % 16] for i = 0..3.
//
// Each wavefront fetches a step of 64 k of its tiles with the LDS DMA into a region of LDS of
// its own and reads the fragments back from there (x with ds_read_b128, W' with transpose
// loads). The x rows of the step travel the same way, so every global access of the k loop is a
// DMA counted by vmcnt alone and the wavefront keeps S steps in flight under its own waits (no
// barriers: nothing in the loop is shared between wavefronts). A workgroup owns NTILE 16-column
// tiles; its wavefronts split K into interleaved steps and add their partial products (and row
// sums) through LDS in a fixed order. Every workgroup walks K from the start, so that at any
// time the chip reads whole consecutive k rows of W'.
//
// x step layout (16 rows, 2 KB): row r, 16-byte chunk c (8 k values) at byte
// (r & 1) * 1024 + (r >> 1) * 128 + (c ^ mvl_f(r)) * 16. One DMA instruction fills the even
// rows and one the odd rows, each lane fetching the chunk its destination slot stands for; a
// fragment read (16 rows at one chunk per 16-lane phase) then touches 16 distinct 16-byte bank
// groups of the 256-byte bank row. Steps of up to 8 x rows use r * 128 + (c ^ (r >> 1)) * 16.
constexpr int kGemvMaxT = 16;

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma16(const u32x4& a, const u32x4& b, const f32x4v& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int mvl_f(int r) { return ((r >> 2) << 1) | (r & 1); }
__device__ __forceinline__ uint32_t mvl_off16(int r, int c)
{
    return (uint32_t)((r & 1) * 1024 + (r >> 1) * 128 + ((c ^ mvl_f(r)) << 4));
}
__device__ __forceinline__ uint32_t mvl_off8(int r, int c)
{
    return (uint32_t)(r * 128 + ((c ^ (r >> 1)) << 4));
}

// s_waitcnt vmcnt(N) that the compiler may not move LDS reads above.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `later` steps of C DMA instructions each remain in flight (0 <= later <= L).
template <int C, int L>
__device__ __forceinline__ void wait_steps(int later)
{
    if constexpr (L > 0) {
        if (later >= L) {
            wait_vm<C * L>();
            return;
        }
        wait_steps<C, L - 1>(later);
    } else {
        wait_vm<0>();
    }
}

// W' step layout: 64 k rows of the workgroup's 16 NTILE columns, each
// row 32 NTILE contiguous bytes (one 32-byte segment per tile), so a DMA instruction covers
// 32 / NTILE rows with whole 32 NTILE-byte runs of W' rows. A fragment is two transpose loads,
// each 4 rows x 16 columns per 16-lane group; a half-wavefront's two groups read rows 8 apart.
// With one tile, row k sits in slot mvk_slot(k) (32 bytes each), which puts those rows in
// different halves of the 256-byte bank row; with two, row k sits at 64 k and tile j's
// segment at physical segment j ^ mvk_seg<2>(k), so the 8 rows a half-wavefront reads at one
// tile cover the 64 banks once.
__device__ __forceinline__ int mvk_slot(int k) { return k ^ (((k >> 3) & 1) << 2); }
template <int NTILE>
__device__ __forceinline__ int mvk_seg(int k)
{
    static_assert(NTILE == 1 || NTILE == 2, "row-major W' tiles per workgroup");
    return NTILE == 2 ? (k >> 3) & 1 : 0;
}
// Byte offset of row k, tile j, column c (a multiple of 4) within a W' step.
template <int NTILE>
__device__ __forceinline__ uint32_t mvk_off(int k, int j, int c)
{
    if constexpr (NTILE == 1) return (uint32_t)((mvk_slot(k) << 5) + (c << 1));
    else return (uint32_t)(k * 32 * NTILE + ((j ^ mvk_seg<NTILE>(k)) << 5) + (c << 1));
}

template <int EPI, int NTILE, int XR, int WAVES, int S>
__global__ __launch_bounds__(WAVES * 64) void normproj_mvl_kernel(
    int T, int64_t K, int64_t N, float eps, float inv_k, const uint16_t* __restrict__ x,
    int64_t ldx, const uint16_t* __restrict__ w, int64_t ldw, uint16_t* __restrict__ y,
    int64_t ldy, const float* __restrict__ colsum, const float* __restrict__ bias)
{
    constexpr int kCols = 16 * NTILE;
    static_assert(XR == 1 || XR == 2 || XR == 4 || XR == 8 || XR == 16, "x rows per step");
    constexpr int XH = XR == 16 ? 2 : 1;          // DMA instructions for the x rows
    constexpr int XOFF = NTILE * 2048;            // x rows after the W' tiles of a step
    constexpr int STAGE = XOFF + (XR == 16 ? 2048 : XR * 128);  // one step of one wavefront
    constexpr int REGION = S * STAGE;             // a wavefront's LDS
    constexpr int C = 2 * NTILE + XH;             // DMA instructions per step
    static_assert(S >= 2 && C * (S - 1) < 64, "vmcnt range");
    static_assert(REGION >= NTILE * 4 * kWave * 4 + 2 * 16 * 4, "partials fit the region");
    __shared__ __attribute__((aligned(1024))) char smem[WAVES * REGION];

    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    const int r16 = lane & 15, g = lane >> 4;
    // A 128-byte line of a k row of W' holds kShare tiles. Workgroup b runs on XCD b % 8;
    // within each group of 8 kShare workgroups, those on one XCD take kShare adjacent tiles
    // (and walk K in the same order), so each line is fetched into one L2 and served there to
    // the workgroups that share it. Tiles past the last whole group keep their index.
    constexpr int kShare = 4 / NTILE;
    int tile = (int)blockIdx.x;
    if constexpr (kShare > 1) {
        const int full = ((int)gridDim.x / (8 * kShare)) * (8 * kShare);
        if (tile < full) {
            const int r = tile % (8 * kShare);
            tile = tile - r + (r & 7) * kShare + (r >> 3);
        }
    }
    const int64_t n0 = (int64_t)tile * kCols;
    char* region = smem + wave * REGION;
    const uint32_t lds_region = (uint32_t)(uintptr_t)(lds_void*)region;

    // DMA sources, as a row byte offset (from the step's first k row of W', or from x) and a
    // chunk byte offset. Token rows past T read row T - 1: they feed outputs that are never
    // stored. The offsets fit 32 bits for ld < 2^25.
    const int drow = lane >> 3, dc = lane & 7;
    uint32_t wrow[NTILE][2], wch[NTILE][2], xrow[XH], xch[XH];
    // W': instruction i = 2 j + h of a step fills bytes 1024 i .. 1024 i + 1023, rows
    // R i .. R i + R - 1 (R = 32 / NTILE), lane l the row's 16-byte chunk l % (2 NTILE): wk
    // is the k row the lane's slot holds, wrow its byte offset (from the step's first row), wch
    // the byte offset of the lane's 8 columns from column n0 (chunks past N, a multiple of 8,
    // read the last chunk and feed columns never stored)
    int wk[NTILE][2];
#pragma unroll
    for (int j = 0; j < NTILE; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            constexpr int R = 32 / NTILE, LPRW = 2 * NTILE;
            const int slot = (2 * j + h) * R + lane / LPRW, pc = lane % LPRW;
            int col;
            if constexpr (NTILE == 1) {
                wk[j][h] = mvk_slot(slot);
                col = 8 * pc;
            } else {
                wk[j][h] = slot;
                col = 16 * ((pc >> 1) ^ mvk_seg<NTILE>(slot)) + 8 * (pc & 1);
            }
            const int64_t n = n0 + col;
            wrow[j][h] = (uint32_t)(wk[j][h] * ldw * 2);
            wch[j][h] = (uint32_t)(((n < N ? n : N - 8) - n0) * 2);
        }
#pragma unroll
    for (int h = 0; h < XH; ++h) {
        const int r = XH == 1 ? drow : 2 * drow + h;
        xrow[h] = (uint32_t)((r < T ? r : T - 1) * ldx * 2);
        xch[h] = (uint32_t)((XH == 1 ? dc ^ (r >> 1) : dc ^ mvl_f(r)) << 4);
    }
    const uint16_t* wb = w + n0;
    const uint32_t kbytes = (uint32_t)(K * 2);

    float x0 = 0.0f;
    if constexpr (EPI == kEpiLayerNorm) {
        x0 = bf16_at(x, (int64_t)(r16 < T ? r16 : 0) * ldx);
        asm volatile("" ::"v"(x0));  // its load completes before the first DMA is issued
    }

    // Step st into slot `slot`: chunks past K read the row's last chunk and are zeroed at use.
    auto issue = [&](int64_t st, int slot) {
        const uint32_t kb = (uint32_t)st * 128u;
        const bool full = kb + 128u <= kbytes;
        const uint32_t dst = lds_region + (uint32_t)(slot * STAGE);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot's fragment reads are done
        // the step's first k row as the scalar base; rows past K read row K - 1 (zeroed at use)
        const uint16_t* wst = wb + st * 64 * ldw;
#pragma unroll
        for (int j = 0; j < NTILE; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t ro = wrow[j][h];
                if (!full && st * 64 + wk[j][h] >= K) ro = (uint32_t)((K - 1 - st * 64) * ldw * 2);
                dma16s(wst, ro + wch[j][h], dst + (uint32_t)(j * 2048 + h * 1024));
            }
#pragma unroll
        for (int h = 0; h < XH; ++h) {
            const uint32_t c = full ? kb + xch[h] : min(kb + xch[h], kbytes - 16u);
            if (XR >= 8 || lane < XR * 8) dma16s(x, xrow[h] + c, dst + (uint32_t)(XOFF + h * 1024));
        }
    };

    f32x4v acc[NTILE];
#pragma unroll
    for (int j = 0; j < NTILE; ++j) acc[j] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    float s1 = 0.0f, s2 = 0.0f;

    auto consume = [&](int64_t st, int slot) {
        const char* sp = region + slot * STAGE;
        u32x4 a[2], b[NTILE][2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = q * 4 + g;
            a[q] = *(const u32x4*)(sp + XOFF + (XR == 16 ? mvl_off16(r16, c)
                                                          : mvl_off8(r16 & (XR - 1), c)));
#pragma unroll
            for (int j = 0; j < NTILE; ++j) {
                // rows 32 q + 8 g + (r16 >> 2) (+ 4), columns 4 (r16 & 3) .. + 3 of tile j
                const int k0 = 32 * q + 8 * g + (r16 >> 2);
                const u32x2 lo = lds_tr16(sp + mvk_off<NTILE>(k0, j, 4 * (r16 & 3)));
                const u32x2 hi = lds_tr16(sp + mvk_off<NTILE>(k0 + 4, j, 4 * (r16 & 3)));
                b[j][q] = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
        }
        bool kin[2] = {true, true};
        if ((uint32_t)st * 128u + 128u > kbytes) {  // the last, partial step
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                kin[q] = st * 64 + (q * 4 + g) * 8 < K;
                if (!kin[q]) {
                    a[q] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int j = 0; j < NTILE; ++j) b[j][q] = u32x4{0u, 0u, 0u, 0u};
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            // chunks past K take no part in the row sums (a zero would add -x0 to LayerNorm's)
            if constexpr (EPI != kEpiPlain) {
                if (kin[q]) accum_stats<EPI>(a[q], x0, s1, s2);
            }
#pragma unroll
            for (int j = 0; j < NTILE; ++j) acc[j] = mfma16(a[q], b[j][q], acc[j]);
        }
    };

    const int64_t nsteps = (K + 63) / 64;
    const int nmine = wave < nsteps ? (int)((nsteps - 1 - wave) / WAVES) + 1 : 0;
    auto step = [&](int i) { return wave + (int64_t)i * WAVES; };
#pragma unroll
    for (int i = 0; i < S; ++i)
        if (i < nmine) issue(step(i), i);
    for (int i0 = 0; i0 < nmine; i0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int i = i0 + u;
            if (i >= nmine) break;
            const int later = nmine - 1 - i;
            wait_steps<C, S - 1>(later < S - 1 ? later : S - 1);
            consume(step(i), u);
            if (i + S < nmine) issue(step(i + S), u);
        }
    }

    // partial products and row sums into the wavefront's own region (its DMAs are complete)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    float* racc = (float*)region;
    float* rst = racc + NTILE * 4 * kWave;
#pragma unroll
    for (int j = 0; j < NTILE; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) racc[(j * 4 + i) * kWave + lane] = acc[j][i];
    if constexpr (EPI != kEpiPlain) {
        s1 += __shfl_xor(s1, 16);
        s2 += __shfl_xor(s2, 16);
        s1 += __shfl_xor(s1, 32);
        s2 += __shfl_xor(s2, 32);
        if (lane < 16) {
            rst[lane] = s1;
            rst[16 + lane] = s2;
        }
    }
    __syncthreads();
    if (wave != 0) return;

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * g + i;
        if (t >= T) continue;
        float rs = 1.0f, mu = 0.0f;
        if constexpr (EPI != kEpiPlain) {
            float q1 = 0.0f, q2 = 0.0f;
#pragma unroll
            for (int v = 0; v < WAVES; ++v) {
                const float* o = (const float*)(smem + v * REGION) + NTILE * 4 * kWave;
                q1 += o[t];
                q2 += o[16 + t];
            }
            const float xt0 = EPI == kEpiLayerNorm ? bf16_at(x, (int64_t)t * ldx) : 0.0f;
            row_scale<EPI>(q1, q2, xt0, inv_k, eps, rs, mu);
        }
#pragma unroll
        for (int j = 0; j < NTILE; ++j) {
            const int64_t n = n0 + j * 16 + r16;
            if (n >= N) continue;
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < WAVES; ++v)
                sum += ((const float*)(smem + v * REGION))[(j * 4 + i) * kWave + lane];
            float cs = 0.0f, bs = 0.0f;
            if constexpr (EPI == kEpiLayerNorm) {
                cs = colsum[n];
                if (bias) bs = bias[n];
            }
            y[(int64_t)t * ldy + n] = to_bf16(epilogue<EPI>(sum, rs, mu, cs, bs));
        }
    }
}

// W [K, N] -> w_fold [K, N] = bf16(gamma[k] * W[k, n]) (fp32 product, one rounding), in the
// same row-major layout: one workgroup per k row, consecutive threads on consecutive columns.
// In place (w_fold == w) each element is read and then written by the same thread.
__global__ __launch_bounds__(kThreads) void fold_kernel(int64_t K, int64_t N,
                                                        const uint16_t* w, int64_t ldw,
                                                        const void* gamma, int gamma_bf16,
                                                        uint16_t* wf, int64_t ldwf)
{
    const int64_t k = blockIdx.y;
    float g = 1.0f;
    if (gamma) g = gamma_bf16 ? bf16_at((const uint16_t*)gamma, k) : ((const float*)gamma)[k];
    for (int64_t n = (int64_t)blockIdx.x * kThreads + threadIdx.x; n < N;
         n += (int64_t)gridDim.x * kThreads)
        wf[k * ldwf + n] = to_bf16(g * bf16_at(w, k * ldw + n));
}

// Statistics of the LayerNorm fold: c[n] = sum_k W'[k][n] over the folded values exactly as
// fold_kernel stores them (bf16 of gamma[k] * W[k][n]), and b[n] = sum_k beta[k] * W[k][n].
// 64 columns per workgroup, the k range split over 4 thread rows, fp64 sums combined in a
// fixed order and rounded once to fp32.
__global__ __launch_bounds__(kThreads) void fold_stats_kernel(int64_t K, int64_t N,
                                                             const uint16_t* __restrict__ w,
                                                             int64_t ldw, const void* gamma,
                                                             const void* beta, int gb_bf16,
                                                             float* __restrict__ colsum,
                                                             float* __restrict__ bias)
{
    __shared__ double red[2][4][64];
    const int tx = (int)threadIdx.x % 64, ty = (int)threadIdx.x / 64;
    const int64_t n = (int64_t)blockIdx.x * 64 + tx;
    double c = 0.0, b = 0.0;
    if (n < N) {
        for (int64_t k = ty; k < K; k += 4) {
            const float wv = bf16_at(w, k * ldw + n);
            float g = 1.0f, be = 0.0f;
            if (gamma) g = gb_bf16 ? bf16_at((const uint16_t*)gamma, k) : ((const float*)gamma)[k];
            if (beta) be = gb_bf16 ? bf16_at((const uint16_t*)beta, k) : ((const float*)beta)[k];
            c += (double)__uint_as_float((uint32_t)to_bf16(g * wv) << 16);
            b += (double)be * (double)wv;
        }
    }
    red[0][ty][tx] = c;
    red[1][ty][tx] = b;
    __syncthreads();
    if (ty == 0 && n < N) {
        colsum[n] = (float)(((red[0][0][tx] + red[0][1][tx]) + red[0][2][tx]) + red[0][3][tx]);
        if (bias) bias[n] = (float)(((red[1][0][tx] + red[1][1][tx]) + red[1][2][tx]) + red[1][3][tx]);
    }
}

// Eight consecutive values from k (a multiple of 8) of a bf16 or fp32 vector, 16-byte loads.
__device__ __forceinline__ void load8(const void* p, int64_t k, bool bf, float* out)
{
    if (bf) {
        const u32x4 v = *(const u32x4*)((const uint16_t*)p + k);
        out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x); out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
        out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z); out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
    } else {
        const f32x4 a = *(const f32x4*)((const float*)p + k);
        const f32x4 b = *(const f32x4*)((const float*)p + k + 4);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
}

// LayerNorm rows for the unfused baseline: one workgroup per row. Pass 1 sums x - x0 and its
// square (x0 = the row's first element), pass 2 re-reads the row from cache and writes
// bf16((x - mu) * r * gamma + beta). VEC: 16-byte accesses (K % 8 == 0, 16-byte aligned rows,
// gamma and beta); otherwise one element per access.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void layernorm_rows_kernel(
    int64_t K, float eps, float inv_k, const uint16_t* __restrict__ x, int64_t ldx,
    const void* gamma, const void* beta, int gb_bf16, uint16_t* __restrict__ y, int64_t ldy)
{
    __shared__ float red[2][kThreads / kWave];
    const int64_t t = blockIdx.x;
    const uint16_t* xr = x + t * ldx;
    const float x0 = bf16_at(xr, 0);
    float s1 = 0.0f, s2 = 0.0f;
    if constexpr (VEC) {
        for (int64_t k = (int64_t)threadIdx.x * 8; k < K; k += kThreads * 8)
            accum_stats<kEpiLayerNorm>(*(const u32x4*)(xr + k), x0, s1, s2);
    } else {
        for (int64_t k = threadIdx.x; k < K; k += kThreads) {
            const float d = bf16_at(xr, k) - x0;
            s1 += d;
            s2 = fmaf(d, d, s2);
        }
    }
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    const int wave = (int)threadIdx.x / kWave;
    if (lane_id() == 0) {
        red[0][wave] = s1;
        red[1][wave] = s2;
    }
    __syncthreads();
    float q1 = 0.0f, q2 = 0.0f;
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) {
        q1 += red[0][i];
        q2 += red[1][i];
    }
    float rs, mu;
    row_scale<kEpiLayerNorm>(q1, q2, x0, inv_k, eps, rs, mu);
    if constexpr (VEC) {
        for (int64_t k = (int64_t)threadIdx.x * 8; k < K; k += kThreads * 8) {
            float e[8], g[8], be[8];
            load8(xr, k, true, e);
            if (gamma) load8(gamma, k, gb_bf16, g);
            if (beta) load8(beta, k, gb_bf16, be);
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                o[j] = fmaf((e[j] - mu) * rs, gamma ? g[j] : 1.0f, beta ? be[j] : 0.0f);
            const u32x4 out = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                               pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
            *(u32x4*)(y + t * ldy + k) = out;
        }
    } else {
        for (int64_t k = threadIdx.x; k < K; k += kThreads) {
            float g = 1.0f, be = 0.0f;
            if (gamma) g = gb_bf16 ? bf16_at((const uint16_t*)gamma, k) : ((const float*)gamma)[k];
            if (beta) be = gb_bf16 ? bf16_at((const uint16_t*)beta, k) : ((const float*)beta)[k];
            y[t * ldy + k] = to_bf16(fmaf((bf16_at(xr, k) - mu) * rs, g, be));
        }
    }
}

// Row statistics of LayerNorm for the product's epilogue: one wavefront per row, the same
// shifted fp32 sums as the in-product accumulation, (mean, 1/std) per row.
constexpr int kStatsRowsPerBlock = 4;

__global__ __launch_bounds__(kStatsRowsPerBlock * kWave) void layernorm_stats_kernel(
    int64_t T, int64_t K, float eps, float inv_k, const uint16_t* __restrict__ x, int64_t ldx,
    float* __restrict__ rowstats)
{
    const int64_t t = (int64_t)blockIdx.x * kStatsRowsPerBlock + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const uint16_t* xr = x + t * ldx;
    const float x0 = bf16_at(xr, 0);
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll 4
    for (int64_t k = (int64_t)lane * 8; k < K; k += kWave * 8)
        accum_stats<kEpiLayerNorm>(*(const u32x4*)(xr + k), x0, s1, s2);
    s1 = wave_sum(s1);
    s2 = wave_sum(s2);
    if (lane == 0) {
        float rs, mu;
        row_scale<kEpiLayerNorm>(s1, s2, x0, inv_k, eps, rs, mu);
        const f32x2 st = {mu, rs};
        *(f32x2*)(rowstats + 2 * t) = st;
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

template <int BM, int BN, int WM, int WN, int NST, int BK, int EPI, bool RING, bool NTS, int KG>
hipError_t launch_pipe_t(int64_t T, int64_t K, int64_t N, float eps, float inv_k,
                         const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                         uint16_t* y, int64_t ldy, const float* colsum, const float* bias,
                         const float* rowstats, hipStream_t st)
{
    const int64_t nbm = (T + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    if (nbm * nbn > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((normproj_pipe_kernel<BM, BN, WM, WN, NST, BK, EPI, RING, NTS, KG>),
                       dim3((unsigned)(nbm * nbn)), dim3(WM * WN * KG * kWave), 0, st, T, K, N, eps,
                       inv_k, x, ldx, w, ldw, y, ldy, (int)nbm, (int)nbn, colsum, bias, rowstats);
    return hipGetLastError();
}

// Ordinary output stores exist for the epilogues whose output the library reads back itself
// (the pre-norm elimination: plain or RMSNorm).
template <int BM, int BN, int WM, int WN, int NST, int BK, int EPI, bool RING, int KG>
hipError_t launch_pipe(int64_t T, int64_t K, int64_t N, float eps, float inv_k,
                       const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                       uint16_t* y, int64_t ldy, const float* colsum, const float* bias,
                       const float* rowstats, bool nts, hipStream_t st)
{
    if constexpr (EPI == kEpiPlain || EPI == kEpiRms) {
        if (!nts)
            return launch_pipe_t<BM, BN, WM, WN, NST, BK, EPI, RING, false, KG>(
                T, K, N, eps, inv_k, x, ldx, w, ldw, y, ldy, colsum, bias, rowstats, st);
    }
    return launch_pipe_t<BM, BN, WM, WN, NST, BK, EPI, RING, true, KG>(
        T, K, N, eps, inv_k, x, ldx, w, ldw, y, ldy, colsum, bias, rowstats, st);
}

struct MvJob {
    int64_t T, K, N;
    float eps, inv_k;
    const uint16_t* x;
    int64_t ldx;
    const uint16_t* w;
    int64_t ldw;
    uint16_t* y;
    int64_t ldy;
    const float *colsum, *bias;
    hipStream_t st;
};

template <int EPI, int NTILE, int XR, int WAVES, int S>
hipError_t launch_mvl(const MvJob& j)
{
    constexpr int kCols = 16 * NTILE;
    const int64_t nblk = (j.N + kCols - 1) / kCols;
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((normproj_mvl_kernel<EPI, NTILE, XR, WAVES, S>), dim3((unsigned)nblk),
                       dim3(WAVES * kWave), 0, j.st, (int)j.T, j.K, j.N, j.eps, j.inv_k, j.x,
                       j.ldx, j.w, j.ldw, j.y, j.ldy, j.colsum, j.bias);
    return hipGetLastError();
}

// x rows per step: T rounded up to a power of two. Two 16-column tiles (64-byte runs of W'
// rows) per workgroup once that still gives 128 workgroups, else one (32-byte runs); measured
// at T = 16, N = 8192: two tiles 22.8 us, four (whole 128-byte runs, half the workgroups)
// 25.3 us, one 27.7 us. The step count fills the LDS.
template <int EPI>
hipError_t launch_mv(const MvJob& j)
{
    if (j.N >= 32 * 128) {
        if (j.T <= 8) return launch_mvl<EPI, 2, 8, 8, 3>(j);
        return launch_mvl<EPI, 2, 16, 8, 3>(j);
    }
    if (j.T <= 1) return launch_mvl<EPI, 1, 1, 8, 4>(j);
    if (j.T <= 2) return launch_mvl<EPI, 1, 2, 8, 4>(j);
    if (j.T <= 4) return launch_mvl<EPI, 1, 4, 8, 4>(j);
    if (j.T <= 8) return launch_mvl<EPI, 1, 8, 8, 3>(j);
    return launch_mvl<EPI, 1, 16, 8, 2>(j);
}

// Kernel choice for a product shape.
enum Path { kPathMv, kPathBig64, kPathBig32, kPathMid, kPathMidDeep, kPathElem };

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

Path choose_path(int64_t T, int64_t K, int64_t N, const void* x, int64_t ldx, const void* w,
                 int64_t ldw, int64_t ldy, const void* y)
{
    // 16-byte accesses along k of x and along n of W'; anything else takes the element kernel
    const bool vec = K % 8 == 0 && N % 8 == 0 && ldx % 8 == 0 && ldw % 8 == 0 && aligned16(x) &&
                     aligned16(w);
    if (!vec) return kPathElem;
    // the matrix-vector kernel addresses W' and x rows with 32-bit byte offsets from the first
    // of 64 k rows of W' or of x (at most 16 rows)
    if (T <= kGemvMaxT && ldx < (int64_t(1) << 25) && ldw < (int64_t(1) << 25)) return kPathMv;
    // the pipelined kernels address a tile's rows with 32-bit byte offsets from its first row
    const bool pipe_ok = ldy % 8 == 0 && aligned16(y) && ldx < (int64_t(1) << 23) &&
                         ldw < (int64_t(1) << 23);
    const int64_t big_tiles = ((T + 255) / 256) * ((N + 255) / 256);
    // at least one 256 x 256 tile per CU: 8 wavefronts of 64 x 128, k-tiles of 64 through the
    // ring of five parts, or of 32 in 4 whole-tile stages when K needs it
    if (pipe_ok && big_tiles >= 256 && K % 64 == 0) return kPathBig64;
    if (pipe_ok && big_tiles >= 256 && K % 32 == 0) return kPathBig32;
    // 128 x 128 per workgroup of 8 wavefronts, k-tiles of 64: with more tiles than CUs, 2 stages
    // and 2 workgroups per CU, the wavefronts in two k groups of 2 x 2 (64 x 64 each, half the
    // k steps each); with at most one tile per CU, 4 stages (3 k-tiles in flight) in the LDS the
    // second workgroup would have used, wavefronts 4 x 2 (32 x 64 each); two wavefronts per SIMD
    // hide each other's LDS and barrier latency
    const int64_t mid_tiles = ((T + 127) / 128) * ((N + 127) / 128);
    if (pipe_ok && K % 64 == 0) return mid_tiles <= 256 ? kPathMidDeep : kPathMid;
    return kPathElem;
}

template <int EPI>
hipError_t launch_epi(int64_t T, int64_t K, int64_t N, float eps, const uint16_t* xp,
                      int64_t ldx, const uint16_t* wp, int64_t ldw, uint16_t* yp, int64_t ldy,
                      const float* colsum, const float* bias, const float* rowstats,
                      bool nts, hipStream_t st)
{
    const float inv_k = (float)(1.0 / (double)K);
    const Path path = choose_path(T, K, N, xp, ldx, wp, ldw, ldy, yp);
    switch (path) {
    case kPathBig64:
        return launch_pipe<256, 256, 4, 2, 5, 64, EPI, true, 1>(
            T, K, N, eps, inv_k, xp, ldx, wp, ldw, yp, ldy, colsum, bias, rowstats, nts, st);
    case kPathBig32:
        return launch_pipe<256, 256, 4, 2, 4, 32, EPI, false, 1>(
            T, K, N, eps, inv_k, xp, ldx, wp, ldw, yp, ldy, colsum, bias, rowstats, nts, st);
    case kPathMid:
        return launch_pipe<128, 128, 2, 2, 2, 64, EPI, false, 2>(
            T, K, N, eps, inv_k, xp, ldx, wp, ldw, yp, ldy, colsum, bias, rowstats, nts, st);
    case kPathMidDeep:
        return launch_pipe<128, 128, 4, 2, 4, 64, EPI, false, 1>(
            T, K, N, eps, inv_k, xp, ldx, wp, ldw, yp, ldy, colsum, bias, rowstats, nts, st);
    default:
        break;
    }
    if constexpr (EPI == kEpiLayerNormStats) {
        return hipErrorInvalidValue;  // statistics from memory: pipelined kernels only
    } else {
        if (path == kPathMv)
            return launch_mv<EPI>(MvJob{T, K, N, eps, inv_k, xp, ldx, wp, ldw, yp, ldy, colsum,
                                        bias, st});
        const int64_t nbm = (T + kBM - 1) / kBM, nbn = (N + kBN - 1) / kBN;
        if (nbm * nbn > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((normproj_elem_kernel<EPI>), dim3((unsigned)(nbm * nbn)),
                           dim3(kThreads), 0, st, T, K, N, eps, inv_k, xp, ldx, wp, ldw, yp, ldy,
                           (int)nbm, (int)nbn, colsum, bias);
        return hipGetLastError();
    }
}

}  // namespace

bool normproj_pipelined(int64_t T, int64_t K, int64_t N, const void* x, int64_t ldx,
                        const void* w, int64_t ldw, int64_t ldy, const void* y)
{
    const Path p = choose_path(T, K, N, x, ldx, w, ldw, ldy, y);
    return p == kPathBig64 || p == kPathBig32 || p == kPathMid || p == kPathMidDeep;
}

hipError_t launch_normproj(int64_t T, int64_t K, int64_t N, float eps, int epi,
                           const void* x, int64_t ldx, const void* w, int64_t ldw, void* y,
                           int64_t ldy, const float* colsum, const float* bias,
                           const float* rowstats, hipStream_t st)
{
    if (T == 0 || N == 0) return hipSuccess;
    // outputs leave the library: non-temporal stores, unless the caller reads them back next
    const bool nts = (epi & kEpiKeepCached) == 0;
    epi &= ~kEpiKeepCached;
    const uint16_t* xp = (const uint16_t*)x;
    const uint16_t* wp = (const uint16_t*)w;
    uint16_t* yp = (uint16_t*)y;
    switch (epi) {
    case kEpiPlain:
        return launch_epi<kEpiPlain>(T, K, N, eps, xp, ldx, wp, ldw, yp, ldy, colsum, bias,
                                        rowstats, nts, st);
    case kEpiRms:
        return launch_epi<kEpiRms>(T, K, N, eps, xp, ldx, wp, ldw, yp, ldy, colsum, bias,
                                      rowstats, nts, st);
    case kEpiLayerNorm:
        return launch_epi<kEpiLayerNorm>(T, K, N, eps, xp, ldx, wp, ldw, yp, ldy, colsum,
                                            bias, rowstats, nts, st);
    case kEpiLayerNormStats:
        return launch_epi<kEpiLayerNormStats>(T, K, N, eps, xp, ldx, wp, ldw, yp, ldy, colsum,
                                                 bias, rowstats, nts, st);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_layernorm_stats(int64_t T, int64_t K, float eps, const void* x, int64_t ldx,
                                  float* rowstats, hipStream_t st)
{
    if (T == 0) return hipSuccess;
    const int64_t nblk = (T + kStatsRowsPerBlock - 1) / kStatsRowsPerBlock;
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(layernorm_stats_kernel, dim3((unsigned)nblk),
                       dim3(kStatsRowsPerBlock * kWave), 0, st, T, K, eps,
                       (float)(1.0 / (double)K), (const uint16_t*)x, ldx, rowstats);
    return hipGetLastError();
}

hipError_t launch_fold_stats(int64_t K, int64_t N, const void* w, int64_t ldw, const void* gamma,
                             const void* beta, int gb_bf16, float* colsum, float* bias,
                             hipStream_t st)
{
    if (N == 0) return hipSuccess;
    const int64_t nblk = (N + 63) / 64;
    if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fold_stats_kernel, dim3((unsigned)nblk), dim3(kThreads), 0, st, K, N,
                       (const uint16_t*)w, ldw, gamma, beta, gb_bf16, colsum, bias);
    return hipGetLastError();
}

hipError_t launch_layernorm_rows(int64_t T, int64_t K, float eps, const void* x, int64_t ldx,
                                 const void* gamma, const void* beta, int gb_bf16, void* y,
                                 int64_t ldy, hipStream_t st)
{
    if (T == 0) return hipSuccess;
    if (T > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool vec = K % 8 == 0 && ldx % 8 == 0 && ldy % 8 == 0 && aligned16(x) &&
                     aligned16(y) && (gamma == nullptr || aligned16(gamma)) &&
                     (beta == nullptr || aligned16(beta));
    if (vec)
        hipLaunchKernelGGL(layernorm_rows_kernel<true>, dim3((unsigned)T), dim3(kThreads), 0, st,
                           K, eps, (float)(1.0 / (double)K), (const uint16_t*)x, ldx, gamma,
                           beta, gb_bf16, (uint16_t*)y, ldy);
    else
        hipLaunchKernelGGL(layernorm_rows_kernel<false>, dim3((unsigned)T), dim3(kThreads), 0,
                           st, K, eps, (float)(1.0 / (double)K), (const uint16_t*)x, ldx, gamma,
                           beta, gb_bf16, (uint16_t*)y, ldy);
    return hipGetLastError();
}

hipError_t launch_fold(int64_t K, int64_t N, const void* w, int64_t ldw, const void* gamma,
                       int gamma_bf16, void* w_fold, int64_t ldwf, hipStream_t st)
{
    if (K == 0 || N == 0) return hipSuccess;
    int64_t gx = (N + kThreads - 1) / kThreads;
    if (gx > 64) gx = 64;  // wide rows: each thread strides over the rest
    if (K > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(fold_kernel, dim3((unsigned)gx, (unsigned)K), dim3(kThreads), 0, st, K, N,
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
