// The LTX DiT RoPE frequency grid, generated on the device (sglang PR #24660
// page, "Implementation breakdown", step 2: generated directly on the target
// device in the requested precision; "Key source snippets": the grid is
// theta ** linspace(0, 1, dim // num_rope_elems) * pi / 2, cast to float32).
//
// One thread per grid value; the arithmetic is in dit_math.h.  A grid has at
// most 2^24 values and is built once per model, so the launch is bound by its
// own latency, not by memory or arithmetic throughput.
#include <hip/hip_runtime.h>

#include "dit_math.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace ltx3drope {
namespace {

constexpr uint32_t kDitBlock = 256;

__global__ void __launch_bounds__(kDitBlock) dit_freqs(float* __restrict__ out, uint32_t n, double theta,
                                                       int double_precision) {
    const uint32_t i = blockIdx.x * kDitBlock + threadIdx.x;
    if (i >= n) return;
    out[i] = double_precision ? dit::grid_f64(theta, i, n) : dit::grid_f32(static_cast<float>(theta), i, n);
}

}  // namespace

hipError_t launch_dit_freqs(float* out, uint32_t n, double theta, bool double_precision, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const uint32_t blocks = (n + kDitBlock - 1) / kDitBlock;
    hipLaunchKernelGGL(dit_freqs, dim3(blocks), dim3(kDitBlock), 0, stream, out, n, theta, double_precision ? 1 : 0);
    return hipGetLastError();
}

}  // namespace ltx3drope
