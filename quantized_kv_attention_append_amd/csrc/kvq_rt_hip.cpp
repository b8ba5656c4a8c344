// The host runtime's device-memory calls, with HIP (see kvq_rt.h).
#include "kvq_rt.h"

namespace kvq {
namespace rt {

hipError_t current_device(int* dev) { return hipGetDevice(dev); }
hipError_t alloc(void** p, size_t bytes) { return hipMalloc(p, bytes); }
hipError_t release(void* p) { return hipFree(p); }
hipError_t zero(void* p, size_t bytes) {
    const hipError_t e = hipMemset(p, 0, bytes);
    return e != hipSuccess ? e : hipDeviceSynchronize();
}
hipError_t upload(void* dst, const void* src, size_t bytes) { return hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice); }
const char* error_string(hipError_t e) { return hipGetErrorString(e); }

}  // namespace rt
}  // namespace kvq
