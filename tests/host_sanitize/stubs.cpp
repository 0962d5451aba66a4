// Stand-ins for the HIP runtime and the kernel launchers, for sanitizer builds of the
// library's host code (api.cpp, tables.cpp) without a GPU.  In host-table mode no
// code path may reach HIP: every stub counts its calls and fails, and the driver
// checks that the count stays zero.
#include <hip/hip_runtime.h>

#include <atomic>

#include "internal.h"

std::atomic<long> g_hip_calls{0};

namespace {
hipError_t refuse() {
    g_hip_calls.fetch_add(1);
    return hipErrorNotSupported;
}
}  // namespace

extern "C" {
hipError_t hipMalloc(void**, size_t) { return refuse(); }
hipError_t hipFree(void*) { return refuse(); }
hipError_t hipMemcpy(void*, const void*, size_t, hipMemcpyKind) { return refuse(); }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return refuse(); }
hipError_t hipStreamSynchronize(hipStream_t) { return refuse(); }
hipError_t hipDeviceSynchronize() { return refuse(); }
hipError_t hipGetDevice(int*) { return refuse(); }
hipError_t hipSetDevice(int) { return refuse(); }
hipError_t hipGetLastError() { return hipSuccess; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return refuse(); }
hipError_t hipPointerGetAttributes(hipPointerAttribute_t*, const void*) { return refuse(); }
hipError_t hipMemGetAddressRange(hipDeviceptr_t*, size_t*, hipDeviceptr_t) { return refuse(); }
}

namespace ltx3drope {
bool fast_supported(const Problem&) { return g_hip_calls.fetch_add(1), false; }
hipError_t launch_fast(const Problem&, hipStream_t, int) { return refuse(); }
hipError_t launch_plain(const Problem&, hipStream_t, int) { return refuse(); }
hipError_t launch_verify(const Problem&, unsigned*, hipStream_t, int) { return refuse(); }
hipError_t launch_zero_u32(unsigned*, hipStream_t) { return refuse(); }
hipError_t launch_copy(void*, const void*, int64_t, hipStream_t, int) { return refuse(); }
bool neox_fast_supported(const NeoxProblem&) { return g_hip_calls.fetch_add(1), false; }
hipError_t launch_neox_fast(const NeoxProblem&, unsigned*, hipStream_t) { return refuse(); }
hipError_t launch_neox_plain(const NeoxProblem&, unsigned*, hipStream_t, int) { return refuse(); }
bool patch_fast_supported(const PatchProblem&) { return g_hip_calls.fetch_add(1), false; }
hipError_t launch_patch(const PatchProblem&, bool, hipStream_t, int) { return refuse(); }
}  // namespace ltx3drope
