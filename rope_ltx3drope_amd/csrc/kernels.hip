// HIP kernels of the fused 3D RoPE for gfx950 (MI355X), and their launchers.
//
// Arithmetic (sglang PR #35698 page, "Key source snippets", the CUDA kernel's
// pair-rotation helper; "Implementation breakdown", step 2): each (even, odd)
// pair is widened to fp32 and rotated with four separately rounded products
// followed by one rounded difference and one rounded sum; no fused
// multiply-add.  This file is compiled with -ffp-contract=off and the pragma
// below, and every product/sum goes through __fmul_rn/__fsub_rn/__fadd_rn.
// The result is cast back to the tensor dtype with round-to-nearest-even.  A
// NaN result is written as the canonical quiet NaN (0x7FC00000 in fp32, 0x7FC0
// in bf16) by both kernels, so equal inputs give byte-identical outputs.
//
// Index mapping (same snippet): pair j of a head uses the t table at column j
// for j < dim_t/2, the h table at column j - dim_t/2 for j < (dim_t+dim_h)/2,
// and the w table for the rest; the table row is the token's t, h or w
// coordinate, with token n = (t*H + h)*W + w in each batch element.
//
// Two kernels compute it: rope_plain (plain.hip), the gate's reference path and
// the fallback, and this file's fast kernel:
//  * rope_fast: a one-shot grid in which each thread owns one 16-byte vector
//    (8 bf16 or 4 fp32 values, i.e. 4 or 2 pairs): the first half of the grid
//    covers Q, the second half K.  When a token's heads*head_dim row is a whole
//    number of wavefronts, the token -> (t, h, w) decode runs once per
//    wavefront on scalar values and (head_dim <= 1024) the wavefront assembles
//    the token's (cos, sin) row in LDS.  Otherwise the decode runs once per
//    wavefront plus a step of 0-2 tokens per lane (rows of 32+ vectors) or per
//    lane, and each lane reads its vector's row segment from the packed
//    tables, which stay in the L1/L2 caches (they are tens of KB).  Q and K
//    stream through with non-temporal 16-byte loads and
//    streaming (sc1 | nt) 16-byte stores; bf16 results are packed with the
//    hardware's round-to-nearest-even conversion (v_cvt_pk_bf16_f32).
//    Measured on MI355X, this shape streams faster than a persistent grid with
//    LDS-staged tables and several vectors per lane.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fastdiv.h"
#include "internal.h"
#include "pair_math.h"
#include "stream_store.h"

#pragma clang fp contract(off)

namespace ltx3drope {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kFastBlock = 64;             // one wavefront per workgroup

// ---------------------------------------------------------------------------
// fast kernel: one 16-byte vector of Q and of K per thread, one-shot grid
// ---------------------------------------------------------------------------

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct FastArgs {
    const u32x4* q;
    const u32x4* k;
    u32x4* q_out;
    u32x4* k_out;
    const f32x4* tab;  // packed tables as float4 = two (cos, sin) pairs
    uint32_t total;    // 16-B vectors per tensor
    uint32_t HV;       // 16-B vectors per token (heads * V)
    uint32_t V;        // 16-B vectors per head
    uint32_t N, HW, W;
    uint32_t T, H;     // grid sizes of the tensor (for the span decode's carries)
    uint32_t PT, PH;   // pairs in the t and h chunks
    uint32_t rowT4, rowH4, rowW4;  // float4 per table row of each section (kTabAligned)
    uint32_t offH4, offW4;         // first float4 of the h and w sections (kTabAligned)
    uint32_t PW;                   // pairs in the w chunk
    uint32_t offH2, offW2;         // first (cos, sin) pair of the h and w sections
    uint32_t t_off, h_off, w_off;  // global coordinate of the tensor's first frame / row / column
    FastDiv div_HV, div_V, div_N, div_HW, div_W;  // the token decode's divisors (fastdiv.h)
};

// PPV pairs per 16-B vector: 4 for bf16, 2 for fp32.  How a vector finds its PPV
// (cos, sin) pairs (TAB):
//  * kTabAligned: the t and h chunk widths are multiples of PPV pairs (so is the
//    w chunk, as head_dim is a whole number of vectors), so a vector never
//    straddles two chunks and its pairs are PPV/2 consecutive float4 of one row.
//  * kTabRow (any even split, one token per wavefront, head_dim <= 1024): the
//    wavefront first assembles its token's head_dim/2 pairs -- t row, then h
//    row, then w row -- in LDS, one float2 per lane and step; each lane then
//    reads its PPV pairs as PPV/2 float4.  One 8-byte table load per lane
//    instead of one per pair (or two 16-byte loads): measured on MI355X, any
//    split then streams at the copy kernel's rate, and aligned splits about
//    1 % faster than with kTabAligned's direct loads.
//  * kTabPair (any even split, any token layout): each pair finds its chunk and
//    row on its own and loads its (cos, sin) as one float2.
//
// Grid: 2 * ceil(vectors / 64) workgroups of one wavefront.  The first half of
// the grid rotates Q, the second half K, so that while the grid runs the memory
// system mostly sees one read stream and one write stream rather than four
// (measured on MI355X: 6.6 TB/s against 6.0 TB/s when every thread handles the
// same vector of Q and of K; one-wavefront workgroups beat 128-1024 threads).
// Both halves are one launch.
//
// DEC, how a lane finds its token -> (t, h, w):
//  * kDecodeWave: a token's heads*head_dim row is a whole number of wavefronts,
//    so each wavefront lies inside one token and the decode runs once per
//    wavefront on wave-uniform (scalar) values;
//  * kDecodeSpan: rows of 32 or more vectors that are not whole wavefronts; a
//    wavefront then spans at most three tokens, its first token is decoded once
//    and each lane steps 0, 1 or 2 tokens on from it (measured on one GPU's
//    head share of the largest workload, 4 heads: about 2 % faster than a decode
//    per lane);
//  * kDecodeLane: every lane decodes its own token (rows below 32 vectors).
//
// Q and K are read with non-temporal hints and the results written with the
// streaming store (sc1 | nt): every byte is touched exactly once, so the streams
// should not displace other data from the caches (measured: +3 to +10 % on the
// 0.8-6.8 GB workloads for the hints, about +1 % more for the store policy).
enum : int { kTabAligned = 0, kTabPair = 1, kTabRow = 2 };
enum : int { kDecodeLane = 0, kDecodeWave = 1, kDecodeSpan = 2 };
constexpr uint32_t kTabRowMaxBytes = 4096;  // kTabRow's LDS row: head_dim <= 1024

template <bool BF16, int DEC, int TAB>
__global__ void __launch_bounds__(kFastBlock) rope_fast(FastArgs a) {
    static_assert(TAB != kTabRow || DEC == kDecodeWave, "the LDS row needs one token per wavefront");
    constexpr uint32_t PPV = BF16 ? 4 : 2;
    const uint32_t half = gridDim.x >> 1;
    const bool second = blockIdx.x >= half;  // wave-uniform
    const uint32_t blk = second ? blockIdx.x - half : blockIdx.x;
    const u32x4* __restrict__ src = second ? a.k : a.q;
    u32x4* __restrict__ dst = second ? a.k_out : a.q_out;
    const uint32_t g = blk * kFastBlock + threadIdx.x;
    uint32_t tok, u;
    if constexpr (DEC == kDecodeWave) {
        const uint32_t g0 = blk * kFastBlock;
        if (g0 >= a.total) return;  // whole wavefronts: total is a multiple of 64 here
        tok = fast_div(g0, a.div_HV);
        u = (g0 - tok * a.HV) + threadIdx.x;
    } else if constexpr (DEC == kDecodeSpan) {
        if (g >= a.total) return;
        tok = fast_div(blk * kFastBlock, a.div_HV);  // the wavefront's first token (wave-uniform)
        u = (blk * kFastBlock - tok * a.HV) + threadIdx.x;
    } else {
        if (g >= a.total) return;
        tok = fast_div(g, a.div_HV);
        u = g - tok * a.HV;
    }
    const uint32_t n = fast_mod(tok, a.div_N);
    uint32_t tl = fast_div(n, a.div_HW);  // local coordinates, then global ones
    const uint32_t rem = n - tl * a.HW;
    uint32_t hl = fast_div(rem, a.div_W);
    uint32_t wl = rem - hl * a.W;
    if constexpr (DEC == kDecodeSpan) {
        // step 0, 1 or 2 tokens on from the wavefront's first (a row holds 32 or more vectors)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (u >= a.HV) {
                u -= a.HV;
                if (++wl == a.W) {
                    wl = 0;
                    if (++hl == a.H) {
                        hl = 0;
                        if (++tl == a.T) tl = 0;  // the next batch element starts at the grid's origin
                    }
                }
            }
        }
    }
    const uint32_t t = tl + a.t_off;
    const uint32_t h = hl + a.h_off;
    const uint32_t w = wl + a.w_off;
    const uint32_t j0 = fast_mod(u, a.div_V) * PPV;  // first pair of this vector inside its head
    const u32x4 x = __builtin_nontemporal_load(src + g);
    float c[PPV], s[PPV];
    if constexpr (TAB == kTabAligned) {
        uint32_t idx;
        if (j0 < a.PT) {
            idx = t * a.rowT4 + j0 / 2;
        } else if (j0 < a.PT + a.PH) {
            idx = a.offH4 + h * a.rowH4 + (j0 - a.PT) / 2;
        } else {
            idx = a.offW4 + w * a.rowW4 + (j0 - a.PT - a.PH) / 2;
        }
#pragma unroll
        for (uint32_t r = 0; r < PPV / 2; ++r) {
            const f32x4 cs = a.tab[idx + r];  // (c, s) of two consecutive pairs
            c[2 * r] = cs.x;
            s[2 * r] = cs.y;
            c[2 * r + 1] = cs.z;
            s[2 * r + 1] = cs.w;
        }
    } else if constexpr (TAB == kTabRow) {
        extern __shared__ __align__(16) f32x2 tab_row[];  // head_dim/2 pairs of this token
        const f32x2* tab2 = reinterpret_cast<const f32x2*>(a.tab);
        const uint32_t pairs = a.V * PPV;  // head_dim / 2
        for (uint32_t j = threadIdx.x; j < pairs; j += kFastBlock) {
            uint32_t idx;
            if (j < a.PT) {
                idx = t * a.PT + j;
            } else if (j < a.PT + a.PH) {
                idx = a.offH2 + h * a.PH + (j - a.PT);
            } else {
                idx = a.offW2 + w * a.PW + (j - a.PT - a.PH);
            }
            tab_row[j] = tab2[idx];
        }
        __syncthreads();  // one wavefront: waits for its own LDS writes
        const f32x4* row4 = reinterpret_cast<const f32x4*>(tab_row) + j0 / 2;
#pragma unroll
        for (uint32_t r = 0; r < PPV / 2; ++r) {
            const f32x4 cs = row4[r];
            c[2 * r] = cs.x;
            s[2 * r] = cs.y;
            c[2 * r + 1] = cs.z;
            s[2 * r + 1] = cs.w;
        }
    } else {
        const f32x2* tab2 = reinterpret_cast<const f32x2*>(a.tab);
#pragma unroll
        for (uint32_t r = 0; r < PPV; ++r) {
            const uint32_t j = j0 + r;
            uint32_t idx;
            if (j < a.PT) {
                idx = t * a.PT + j;
            } else if (j < a.PT + a.PH) {
                idx = a.offH2 + h * a.PH + (j - a.PT);
            } else {
                idx = a.offW2 + w * a.PW + (j - a.PT - a.PH);
            }
            const f32x2 cs = tab2[idx];
            c[r] = cs.x;
            s[r] = cs.y;
        }
    }
    u32x4 y;
    if constexpr (BF16) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float ye, yo;
            rotate(bf16_lo(x[r]), bf16_hi(x[r]), c[r], s[r], ye, yo);
            y[r] = bf16_pack_hw(ye, yo);
        }
    } else {
        float y0, y1, y2, y3;
        rotate(__uint_as_float(x.x), __uint_as_float(x.y), c[0], s[0], y0, y1);
        rotate(__uint_as_float(x.z), __uint_as_float(x.w), c[1], s[1], y2, y3);
        y = (u32x4){f32_canon(y0), f32_canon(y1), f32_canon(y2), f32_canon(y3)};
    }
    stream_store16(y, dst + blk * kFastBlock, kFastBlock * 16u, threadIdx.x * 16u);
}

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__global__ void zero_u32(unsigned* p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = 0u;
}

// Bandwidth reference: the same launch shape and cache hints as rope_fast, one
// read stream and one write stream.
__global__ void __launch_bounds__(kFastBlock) copy16(u32x4* __restrict__ dst, const u32x4* __restrict__ src, uint32_t n) {
    const uint32_t i = blockIdx.x * kFastBlock + threadIdx.x;
    if (i < n) stream_store16(__builtin_nontemporal_load(src + i), dst + blockIdx.x * kFastBlock, kFastBlock * 16u, threadIdx.x * 16u);
}

// ---------------------------------------------------------------------------
// launch geometry
// ---------------------------------------------------------------------------

uint32_t elem_size(const Problem& p) { return p.dtype == LTX3DROPE_DTYPE_F32 ? 4u : 2u; }

}  // namespace

// Device scratch of the no-allocation entry point (ltx3drope_apply_qk_noalloc): word 0 is the gate
// verification's mismatch counter.  Each GPU the library runs on holds its own copy until the
// process ends.  Host code must not pass this name to a kernel (on the host it is only a stand-in
// for the symbol): scratch_counter() returns the device address, looked up once per device.
static __device__ __align__(256) unsigned scratch[kScratchWords];

namespace {
std::mutex g_scratch_mu;
unsigned* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_counter(int device, unsigned** out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[device] == nullptr) {
        int current = -1;
        if (hipGetDevice(&current) != hipSuccess || current != device) return hipErrorInvalidDevice;
        void* addr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));  // this device's copy
        if (e != hipSuccess || addr == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
        g_scratch_addr[device] = static_cast<unsigned*>(addr);
    }
    *out = g_scratch_addr[device];
    return hipSuccess;
}

bool fast_supported(const Problem& p) {
    const uint32_t es = elem_size(p);
    for (const void* ptr : {static_cast<const void*>(p.q), static_cast<const void*>(p.k),
                            static_cast<const void*>(p.q_out), static_cast<const void*>(p.k_out)})
        if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return false;
    return (p.D * es) % 16 == 0;  // head rows are whole 16-byte vectors; any even split
}

template <int DEC, int TAB>
hipError_t launch_fast_dt(const FastArgs& a, bool bf16, uint32_t blocks, size_t lds, hipStream_t stream) {
    if (bf16)
        hipLaunchKernelGGL((rope_fast<true, DEC, TAB>), dim3(blocks), dim3(kFastBlock), lds, stream, a);
    else
        hipLaunchKernelGGL((rope_fast<false, DEC, TAB>), dim3(blocks), dim3(kFastBlock), lds, stream, a);
    return hipGetLastError();
}

template <int TAB>
hipError_t launch_fast_tab(const FastArgs& a, bool bf16, int dec, uint32_t blocks, hipStream_t stream) {
    switch (dec) {
        case kDecodeWave: return launch_fast_dt<kDecodeWave, TAB>(a, bf16, blocks, 0, stream);
        case kDecodeSpan: return launch_fast_dt<kDecodeSpan, TAB>(a, bf16, blocks, 0, stream);
        default: return launch_fast_dt<kDecodeLane, TAB>(a, bf16, blocks, 0, stream);
    }
}

hipError_t launch_fast(const Problem& p, hipStream_t stream, int device) {
    if (!fast_supported(p)) return hipErrorInvalidValue;
    const uint32_t es = elem_size(p);
    FastArgs a;
    a.q = static_cast<const u32x4*>(p.q);
    a.k = static_cast<const u32x4*>(p.k);
    a.q_out = static_cast<u32x4*>(p.q_out);
    a.k_out = static_cast<u32x4*>(p.k_out);
    a.tab = reinterpret_cast<const f32x4*>(p.tab);
    a.V = p.D * es / 16;
    a.HV = p.heads * a.V;
    a.total = p.B * p.T * p.H * p.W * a.HV;
    a.N = p.T * p.H * p.W;
    a.HW = p.H * p.W;
    a.W = p.W;
    a.T = p.T;
    a.H = p.H;
    a.PT = p.PT;
    a.PH = p.PH;
    a.rowT4 = p.PT / 2;
    a.rowH4 = p.PH / 2;
    a.rowW4 = p.PW / 2;
    a.offH4 = p.tabT * p.PT / 2;
    a.offW4 = (p.tabT * p.PT + p.tabH * p.PH) / 2;
    a.t_off = p.t_off;
    a.h_off = p.h_off;
    a.w_off = p.w_off;
    a.div_HV = make_fastdiv(a.HV);
    a.div_V = make_fastdiv(a.V);
    a.div_N = make_fastdiv(a.N);
    a.div_HW = make_fastdiv(a.HW);
    a.div_W = make_fastdiv(a.W);
    a.PW = p.PW;
    a.offH2 = p.tabT * p.PT;
    a.offW2 = p.tabT * p.PT + p.tabH * p.PH;
    const uint32_t per_tensor = (a.total + kFastBlock - 1) / kFastBlock;
    if (per_tensor == 0) return hipSuccess;
    const uint32_t blocks = 2 * per_tensor;  // first half Q, second half K
    const bool wave_token = a.HV % 64 == 0;
    const bool bf16 = p.dtype == LTX3DROPE_DTYPE_BF16;
    const uint32_t ppv = 8u / es;
    const bool aligned = p.PT % ppv == 0 && p.PH % ppv == 0;
    const size_t row_bytes = size_t(p.D / 2) * 8;  // kTabRow's LDS: (cos, sin) of every pair of a head
    (void)device;
    if (wave_token && row_bytes <= kTabRowMaxBytes)
        return launch_fast_dt<kDecodeWave, kTabRow>(a, bf16, blocks, row_bytes, stream);
    const int dec = wave_token ? kDecodeWave : a.HV >= 32 ? kDecodeSpan : kDecodeLane;
    if (aligned) return launch_fast_tab<kTabAligned>(a, bf16, dec, blocks, stream);
    return launch_fast_tab<kTabPair>(a, bf16, dec, blocks, stream);
}

hipError_t launch_zero_u32(unsigned* ptr, hipStream_t stream) {
    hipLaunchKernelGGL(zero_u32, dim3(1), dim3(64), 0, stream, ptr);
    return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream, int device) {
    (void)device;
    const uint64_t n = static_cast<uint64_t>(bytes) / 16;
    if (n == 0) return hipSuccess;
    if (n > 0xffffffffull - kFastBlock) return hipErrorInvalidValue;
    const uint32_t blocks = static_cast<uint32_t>((n + kFastBlock - 1) / kFastBlock);
    hipLaunchKernelGGL(copy16, dim3(blocks), dim3(kFastBlock), 0, stream, static_cast<u32x4*>(dst),
                       static_cast<const u32x4*>(src), static_cast<uint32_t>(n));
    return hipGetLastError();
}

}  // namespace ltx3drope
