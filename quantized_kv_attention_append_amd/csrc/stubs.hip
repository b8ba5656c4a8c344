// Entry points whose kernels are not built yet report hipErrorNotSupported.
#include "kvq_internal.h"
namespace kvq {
hipError_t launch_prefill_q2(const PoolView&, int, int, int, int, const uint16_t*, float, int, float*, float*,
                             hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace kvq
