// One (x storage, gamma storage) pair of the row kernels, selected at build time with
// QKN_ROWS_BF / QKN_ROWS_GBF so that the instantiations compile in parallel.
#include "rows_impl.h"

#if !defined(QKN_ROWS_BF) || !defined(QKN_ROWS_GBF)
#error "build with -DQKN_ROWS_BF=0|1 -DQKN_ROWS_GBF=0|1"
#endif

namespace qkn {

template <bool BF, bool GBF>
hipError_t dispatch_rows(const RowJob& job, hipStream_t st)
{
    switch (job.mode) {
    case kFused: return dispatch_mode<kFused, BF, GBF>(job, st);
    case kApply: return dispatch_mode<kApply, BF, GBF>(job, st);
    default:
        // the partial sums read no gamma: one instantiation per x storage (gamma "bf16")
        if constexpr (GBF) return dispatch_mode<kPartial, BF, GBF>(job, st);
        else return hipErrorInvalidValue;
    }
}

template hipError_t dispatch_rows<QKN_ROWS_BF != 0, QKN_ROWS_GBF != 0>(const RowJob&, hipStream_t);

}  // namespace qkn
