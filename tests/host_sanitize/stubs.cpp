// Stand-ins for the HIP runtime and the kernel launchers, for sanitizer builds of the
// library's host code (api.cpp, tables.cpp) without a GPU.  In host-table mode no
// code path may reach HIP: every stub counts its calls and fails, and the driver
// checks that the count stays zero.  With g_emulate set, the allocation, copy and
// device-selection stand-ins behave like a device 0 backed by host memory, and
// hipMalloc returns g_malloc_fail instead while that is nonzero (failure injection).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>

#include "internal.h"

std::atomic<long> g_hip_calls{0};
std::atomic<int> g_emulate{0};
std::atomic<int> g_malloc_fail{0};
std::atomic<long> g_live_allocs{0};

namespace {
hipError_t refuse() {
    g_hip_calls.fetch_add(1);
    return hipErrorNotSupported;
}
}  // namespace

extern "C" {
hipError_t hipMalloc(void** p, size_t n) {
    if (!g_emulate.load()) return refuse();
    if (const int e = g_malloc_fail.load()) return static_cast<hipError_t>(e);
    *p = std::malloc(n);
    if (*p == nullptr) return hipErrorOutOfMemory;
    g_live_allocs.fetch_add(1);
    return hipSuccess;
}
hipError_t hipFree(void* p) {
    if (!g_emulate.load()) return refuse();
    if (p != nullptr) g_live_allocs.fetch_sub(1);
    std::free(p);
    return hipSuccess;
}
hipError_t hipMemcpy(void*, const void*, size_t, hipMemcpyKind) { return refuse(); }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
    if (!g_emulate.load()) return refuse();
    std::memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return g_emulate.load() ? hipSuccess : refuse(); }
hipError_t hipDeviceSynchronize() { return refuse(); }
hipError_t hipGetDevice(int* d) {
    if (!g_emulate.load()) return refuse();
    *d = 0;
    return hipSuccess;
}
hipError_t hipSetDevice(int d) {
    if (!g_emulate.load()) return refuse();
    return d == 0 ? hipSuccess : hipErrorInvalidDevice;
}
hipError_t hipGetLastError() { return hipSuccess; }
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus*) { return refuse(); }
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
hipError_t launch_dit_freqs(float*, uint32_t, double, bool, hipStream_t) { return refuse(); }
hipError_t scratch_counter(int, unsigned**) { return refuse(); }
}  // namespace ltx3drope
