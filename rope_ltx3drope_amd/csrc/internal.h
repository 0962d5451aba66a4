// Internal declarations shared by the host side (tables, cache, precheck, gate)
// and the kernel launchers of the ltx3drope library.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "ltx3drope.h"

// A table set: the packed per-axis (cos, sin) pairs of one grid.  Layout, in
// float pairs: t section [T][dim_t/2], then h section [H][dim_h/2], then
// w section [W][dim_w/2].
struct ltx3drope_tables {
    std::atomic<int64_t> refs{1};
    int device = 0;
    int64_t T = 0, H = 0, W = 0;
    int64_t dim_t = 0, dim_h = 0, dim_w = 0;
    double base = 0.0;
    bool host = false;        // built in host-table test mode (malloc, never touched by HIP)
    float* packed = nullptr;  // 2 * pairs floats (device memory unless host)
    int64_t pairs = 0;
};

namespace ltx3drope {

// Everything a kernel needs to know about one launch of an apply_qk call.  All
// sizes fit in 32 bits: the precheck keeps a batch element below 2^32 elements
// and a launch takes as many whole batch elements as stay below 2^32 (pairs
// below 2^31, 16-byte vectors below 2^30).
struct Problem {
    void* q_out;
    void* k_out;
    const void* q;
    const void* k;
    const float* tab;  // packed device tables
    int dtype;         // LTX3DROPE_DTYPE_*
    uint32_t B, T, H, W, heads, D;
    uint32_t PT, PH, PW;  // pairs per head in the t, h and w chunks
    uint32_t tab_pairs;
    uint32_t tabT, tabH;  // the tables' grid frames and rows (section offsets of the packed layout)
    uint32_t t_off, h_off, w_off;  // global coordinate of the tensor's first frame / row / column
};

enum class Kernel { Fast = 1, Plain = 2 };

// Host-side decision whether the vectorised kernel covers this problem
// (16-B aligned pointers, head rows of whole 16-B vectors, chunk boundaries on
// vector boundaries).
bool fast_supported(const Problem& p);

// Launchers (kernels.hip).  They only enqueue; the caller checks hipGetLastError.
hipError_t launch_fast(const Problem& p, hipStream_t stream, int device);
hipError_t launch_plain(const Problem& p, hipStream_t stream, int device);
// Recompute with the plain kernel and count the pairs whose result differs
// from what q_out/k_out already hold (raw bit patterns).
hipError_t launch_verify(const Problem& p, unsigned* mismatches, hipStream_t stream, int device);
hipError_t launch_zero_u32(unsigned* ptr, hipStream_t stream);

// The no-allocation entry point's device scratch (kernels.hip): a static 256-byte array per GPU,
// word 0 the gate's mismatch counter.  scratch_counter() returns its device address on `device`,
// which must be the current device (looked up once per device and kept).
constexpr int kScratchWords = 64;
constexpr int kMaxDevices = 64;
hipError_t scratch_counter(int device, unsigned** out);
hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream, int device);

// The rotate-half RoPE with a gathered cos/sin cache (neox.hip).
struct NeoxProblem {
    void* q_out;
    void* k_out;
    const void* q;
    const void* k;
    const int64_t* positions;
    const void* cache;  // [max_position][D]: cos half, then sin half
    int dtype, cache_dtype;
    uint32_t tokens, q_heads, k_heads, D, max_position;
};
bool neox_fast_supported(const NeoxProblem& p);
hipError_t launch_neox_fast(const NeoxProblem& p, unsigned* errors, hipStream_t stream);
hipError_t launch_neox_plain(const NeoxProblem& p, unsigned* errors, hipStream_t stream, int cu_count);

// Stage-5 space-to-depth and its inverse (patchify.hip).  Dimensions are those of
// the unpatched tensor (B, C, F, H, W); src/dst are the input/output of the call.
struct PatchProblem {
    const void* src;
    void* dst;
    uint32_t elem_bytes, B, C, F, H, W, p;
    bool force_plain;
};
bool patch_fast_supported(const PatchProblem& p);
hipError_t launch_patch(const PatchProblem& p, bool inverse, hipStream_t stream, int cu_count);

// The LTX DiT RoPE frequency grid, n values into device memory (dit_freqs.hip).
hipError_t launch_dit_freqs(float* out, uint32_t n, double theta, bool double_precision, hipStream_t stream);

// Tables and cache (tables.cpp).
int tables_build(int device, int64_t T, int64_t H, int64_t W, int64_t dim_t, int64_t dim_h, int64_t dim_w,
                 double base, hipStream_t stream, ltx3drope_tables_t* out);
int tables_release(ltx3drope_tables_t t);
int cache_clear();
void cache_counters(int64_t* hits, int64_t* misses, int64_t* evictions, int64_t* live, int64_t* alive);
void cache_counters_reset();

// Options (api.cpp).
int64_t option(int which);

}  // namespace ltx3drope
