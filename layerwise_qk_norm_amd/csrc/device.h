// Device-side helpers shared by the gfx950 kernels of libqknorm.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qkn {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 is the upper half of an fp32: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ uint16_t to_bf16(float v)
{
    return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
}

// Cross-lane move through DPP (data-parallel primitives). The controls used here are all
// full-row permutations, so every lane reads a valid source lane.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF,
                                                      false));
}
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8-lane half row
constexpr int kDppRowMirror = 0x140;  // lane i <- lane 15-i within each 16-lane row

// Sum over each group of 8 consecutive lanes; every lane of the group gets the result.
__device__ __forceinline__ float sum8(float v)
{
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    return v;
}

// Sum over all 64 lanes in a fixed order; the result is wave-uniform. Must run with every lane
// of the wave active.
__device__ __forceinline__ float wave_sum(float v)
{
    v = sum8(v);
    v += dpp<kDppRowMirror>(v);  // now: sum of the lane's 16-lane row
    float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

typedef __bf16 bf16x2_dot __attribute__((ext_vector_type(2)));

// s + lo*lo + hi*hi for the two bf16 packed in u (v_dot2_f32_bf16: the products of bf16 values
// are exact in fp32; one instruction per two elements, no widening).
__device__ __forceinline__ float sumsq_bf16x2(uint32_t u, float s)
{
    const bf16x2_dot v = __builtin_bit_cast(bf16x2_dot, u);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
}

__device__ __forceinline__ float lane_read(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Streaming 16-byte accesses that should not displace reusable lines in the caches.
__device__ __forceinline__ u32x4 load_stream(const void* p)
{
    return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ void store_stream(void* p, u32x4 v)
{
    __builtin_nontemporal_store(v, (u32x4*)p);
}

}  // namespace qkn
