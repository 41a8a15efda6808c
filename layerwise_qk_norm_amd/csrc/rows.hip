// Entry of the row kernels: picks the instantiation for the job's storage types (the kernels
// themselves are in rows_impl.h, instantiated by rows_inst.hip).
#include "rows_impl.h"

namespace qkn {

hipError_t launch_rows(const RowJob& job, hipStream_t stream)
{
    if (job.T == 0) return hipSuccess;
    if (job.mode == kPartial)  // gamma is not read
        return job.bf16 ? dispatch_rows<true, true>(job, stream)
                        : dispatch_rows<false, true>(job, stream);
    if (job.bf16)
        return job.gamma_bf16 ? dispatch_rows<true, true>(job, stream)
                              : dispatch_rows<true, false>(job, stream);
    return job.gamma_bf16 ? dispatch_rows<false, true>(job, stream)
                          : dispatch_rows<false, false>(job, stream);
}

}  // namespace qkn
