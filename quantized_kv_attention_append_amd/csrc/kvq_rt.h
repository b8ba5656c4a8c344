// The device-memory runtime the host runtime (kvq_host.cpp) goes through:
// allocation, freeing, zeroing and host-to-device copies, all synchronous,
// on the current device.  The library implements it with HIP (kvq_rt_hip.cpp).
// Keeping these few calls behind one interface lets the host runtime's pool,
// reservation, fork, release and argument checks be built and run against
// host memory as well (a test build; it runs no kernels).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace kvq {
namespace rt {

hipError_t current_device(int* dev);
hipError_t alloc(void** p, size_t bytes);  // device memory of the current device
hipError_t release(void* p);
hipError_t zero(void* p, size_t bytes);    // returns once the bytes are zero
hipError_t upload(void* dst, const void* src, size_t bytes);  // host -> device, returns once done
const char* error_string(hipError_t e);

}  // namespace rt
}  // namespace kvq
