// Host-only stand-ins for the kernel launchers of libqknorm.so, used to build the C-ABI layer
// (api.cpp) with the host compiler under AddressSanitizer and UndefinedBehaviorSanitizer. Each
// launcher answers as the real one does on a machine without a GPU: hipErrorNoDevice. Nothing
// here runs device code; only argument validation and dispatch in api.cpp are exercised, and the
// few HIP runtime calls api.cpp makes itself are answered the same way.
#include "../../layerwise_qk_norm_amd/csrc/launch.h"

namespace qkn {

hipError_t launch_rows(const RowJob&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fold(int64_t, int64_t, const void*, int64_t, const void*, int, void*, int64_t,
                       hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_normproj(int64_t, int64_t, int64_t, float, int, const void*, int64_t,
                           const void*, int64_t, void*, int64_t, const float*, const float*,
                           const float*, hipStream_t)
{
    return hipErrorNoDevice;
}
bool normproj_pipelined(int64_t, int64_t, int64_t, const void*, int64_t, const void*, int64_t,
                        int64_t, const void*)
{
    return true;
}
hipError_t launch_layernorm_stats(int64_t, int64_t, float, const void*, int64_t, float*,
                                  hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_fold_stats(int64_t, int64_t, const void*, int64_t, const void*, const void*,
                             int, float*, float*, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_layernorm_rows(int64_t, int64_t, float, const void*, int64_t, const void*,
                                 const void*, int, void*, int64_t, hipStream_t)
{
    return hipErrorNoDevice;
}
hipError_t launch_copy(void*, const void*, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_shard_fused(const ShardArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_shard_publish(int64_t, int64_t, int, const float* const*, const int64_t*,
                                uint64_t* const*, const int64_t*, uint32_t, hipStream_t)
{
    return hipErrorNoDevice;
}

}  // namespace qkn

// The HIP runtime calls api.cpp makes itself (the static workspace's address lookup), answered
// as without a device.
extern "C" {
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipSetDevice(int) { return hipErrorNoDevice; }
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t*) { return hipErrorNoDevice; }
hipError_t hipGetSymbolAddress(void**, const void*) { return hipErrorNoDevice; }
}
