// HIP kernels of the stage-5 space-to-depth (patchify) and its inverse, for gfx950.
//
// Operation (sglang PR #34471 page, "Key source snippets", the decoder's
// _patchify; _unpatchify is its named counterpart):
//     (B, C, F, H, W) -> (B, C*p*p, F, H/p, W/p)
//     out[b, (c*p + pw)*p + ph, f, hh, ww] = x[b, c, f, hh*p + ph, ww*p + pw]
// (channels packed as channel, width offset, height offset).  Pure data
// movement, so the result is bit-exact for any element type; the kernels move
// elements of 1, 2, 4 or 8 bytes.
//
//  * patch_lds<T, P>: a workgroup of P wavefronts owns P*64 consecutive 16-byte
//    vectors of the unpatched tensor, taken in (b, c, height offset, f, patch
//    row, vector) order, which are exactly 64 consecutive packed vectors of each
//    of the P width-offset planes that share (b, c, height offset).  Each thread
//    loads one vector, the elements are regrouped by width offset through P KB
//    of LDS, and each wavefront stores one plane's contiguous 1 KB.
//  * unpatch_lds<T, P>: the inverse, on 128 unpatched vectors per wavefront in
//    (b, c, f, height offset, patch row, vector) order: two loads per lane that
//    each cover whole runs of 128/P packed vectors, two contiguous 1 KB stores.
//  Both take elements of 1, 2, 4 or 8 bytes and p = 2, 4, 8 or 16, 16-byte
//  aligned tensors and W a multiple of p * 16/sizeof(T).
//  * patch_plain<T, INVERSE>: one element per thread, any shape, any p and
//    element size (1, 2, 4 or 8 bytes).
//
// Measured on MI355X on a 121-frame 544 x 960 bf16 clip, p = 4 (758 MB moved):
// threads in unpatched-row order wrote each 480-byte packed row piecemeal
// (4.1 TB/s); the (b, c, f, height offset, patch row) order with a register
// transpose reached 5.5 TB/s (patchify) and a per-lane gather 6.0 TB/s
// (unpatchify); the LDS-staged kernels reach 6.4 (patchify) and 6.5 TB/s
// (unpatchify) with non-temporal loads and streaming (sc1 | nt) stores.  (The
// register transpose, kept for a while for fp32 with p = 8, took 5.4 and
// 3.3 TB/s there.)
#include <hip/hip_runtime.h>

#include "fastdiv.h"
#include "internal.h"
#include "stream_store.h"

namespace ltx3drope {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kBlock = 64;

template <typename T>
struct Vec {
    T e[16 / sizeof(T)];
};

struct PatchArgs {
    const void* src;
    void* dst;
    uint32_t B, C, F, H, W, p;
    uint32_t groups;          // LDS kernels: 16-byte vectors of the unpatched tensor
    uint64_t numel;           // plain kernel
    uint32_t dst_bytes;       // LDS kernels: output size in bytes when below 2^31 (streaming stores), else 0
    FastDiv div_WE, div_WpE, div_Hp, div_F;  // LDS kernels: W/E, (W/p)/E, H/p and F (fastdiv.h)
};

// LDS kernels' 16-byte store at element offset `off` of the output: a streaming store (sc1 | nt)
// relative to the output's base when its size fits the 32-bit offset, else a global store with
// the non-temporal hint.  dst_bytes is uniform, so the branch is too.
template <typename T>
__device__ __forceinline__ void store_out(const PatchArgs& a, uint64_t off, u32x4 v) {
    if (a.dst_bytes != 0)
        stream_store16(v, a.dst, a.dst_bytes, static_cast<uint32_t>(off * sizeof(T)));
    else
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<T*>(a.dst) + off));
}

// Element offset of output channel (c*p + pw)*p + ph, frame f, patch row hh, column ww.
__device__ __forceinline__ uint64_t packed_offset(const PatchArgs& a, uint32_t b, uint32_t c, uint32_t pw,
                                                  uint32_t ph, uint32_t f, uint32_t hh, uint32_t ww) {
    const uint32_t Hp = a.H / a.p, Wp = a.W / a.p;
    const uint64_t co = (static_cast<uint64_t>(b) * a.C + c) * a.p * a.p + static_cast<uint64_t>(pw) * a.p + ph;
    return ((co * a.F + f) * Hp + hh) * Wp + ww;
}

// (b*C + c, f, height offset, patch row) of row `rowid`.  PH_OUTER: rows in (b, c, height
// offset, f, patch row) order, so that consecutive work walks whole frames of one packed plane
// (patchify: every width-offset plane is then written as one long run); otherwise in (b, c, f,
// height offset, patch row) order (unpatchify: every unpatched frame is then written row group
// by row group).  Measured on a 121-frame 544 x 960 bf16 clip, p = 4: patchify 126.7 against
// 129.1 us, unpatchify 121.7 against 133.5 us for the other order.
struct RowId {
    uint32_t bc, f, ph, hh;
};

template <int P, bool PH_OUTER>
__device__ __forceinline__ RowId decode_row(uint32_t rowid, const PatchArgs& a) {
    RowId d;
    const uint32_t t = fast_div(rowid, a.div_Hp);
    d.hh = rowid - t * a.div_Hp.d;
    if constexpr (PH_OUTER) {
        const uint32_t t2 = fast_div(t, a.div_F);
        d.f = t - t2 * a.F;
        d.ph = t2 % P;
        d.bc = t2 / P;
    } else {
        d.ph = t % P;
        const uint32_t bcf = t / P;
        d.bc = fast_div(bcf, a.div_F);
        d.f = bcf - d.bc * a.F;
    }
    return d;
}

// Element offset of unpatched vector I (16-byte vectors in row order, then x).
template <int P, int E, bool PH_OUTER>
__device__ __forceinline__ uint64_t unpatched_offset(const PatchArgs& a, uint32_t I) {
    const uint32_t rowid = fast_div(I, a.div_WE);
    const uint32_t x = I - rowid * a.div_WE.d;
    const RowId d = decode_row<P, PH_OUTER>(rowid, a);
    const uint64_t row = (static_cast<uint64_t>(d.bc) * a.F + d.f) * a.H + d.hh * P + d.ph;
    return row * a.W + static_cast<uint64_t>(x) * E;
}

// Element offset of packed vector O of the width-offset-0 plane (packed vectors in the same
// order); the plane of width offset pw lies pw * P * F * (H/P) * (W/P) elements further.
template <int P, int E, bool PH_OUTER>
__device__ __forceinline__ uint64_t packed_offset0(const PatchArgs& a, uint32_t O) {
    const uint32_t Hp = a.H / P, Wp = a.W / P;
    const uint32_t rowid = fast_div(O, a.div_WpE);
    const uint32_t wv = O - rowid * a.div_WpE.d;
    const RowId d = decode_row<P, PH_OUTER>(rowid, a);
    const uint64_t co = static_cast<uint64_t>(d.bc) * P * P + d.ph;  // output channel of width offset 0
    return ((co * a.F + d.f) * Hp + d.hh) * Wp + static_cast<uint64_t>(wv) * E;
}

// One chunk of K = E/P elements: the elements of one 16-byte vector that share a width offset.
template <int NB>
struct Chunk;
template <>
struct Chunk<1> { typedef uint8_t type; };
template <>
struct Chunk<2> { typedef uint16_t type; };
template <>
struct Chunk<4> { typedef uint32_t type; };
template <>
struct Chunk<8> { typedef unsigned type __attribute__((ext_vector_type(2))); };

// Regrouping through LDS.  Element g of a run of unpatched elements that starts on a multiple of P
// belongs to width-offset plane g % P, at element g / P of that plane's run (rows hold a whole
// number of P-element groups).  For local 16-byte vector li, elements li*E .. li*E + E - 1:
//  * E a multiple of P: each plane gets K = E/P consecutive elements, one K-element chunk at
//    position li*K of lds[pw];
//  * P a multiple of E: R = P/E consecutive vectors share a position, and element e goes to its
//    own plane (li % R)*E + e, at position li / R.
template <typename T, int P, int N>
__device__ __forceinline__ void scatter_vector(T (&lds)[P][N], uint32_t li, const Vec<T>& v) {
    constexpr int E = 16 / sizeof(T);
    if constexpr (E % P == 0) {
        constexpr int K = E / P;
        typedef typename Chunk<K * sizeof(T)>::type Ch;
#pragma unroll
        for (int pw = 0; pw < P; ++pw) {
            T ch[K];
#pragma unroll
            for (int k = 0; k < K; ++k) ch[k] = v.e[k * P + pw];
            Ch c;
            __builtin_memcpy(&c, ch, sizeof(Ch));
            reinterpret_cast<Ch*>(&lds[pw][0])[li] = c;
        }
    } else {
        static_assert(P % E == 0, "P and the vector's element count must divide one another");
        constexpr uint32_t R = P / E;
        const uint32_t pos = li / R, pw0 = (li % R) * E;
#pragma unroll
        for (int e = 0; e < E; ++e) lds[pw0 + e][pos] = v.e[e];
    }
}

template <typename T, int P, int N>
__device__ __forceinline__ Vec<T> gather_vector(const T (&lds)[P][N], uint32_t li) {
    constexpr int E = 16 / sizeof(T);
    Vec<T> v;
    if constexpr (E % P == 0) {
        constexpr int K = E / P;
        typedef typename Chunk<K * sizeof(T)>::type Ch;
#pragma unroll
        for (int pw = 0; pw < P; ++pw) {
            const Ch c = reinterpret_cast<const Ch*>(&lds[pw][0])[li];
            T ch[K];
            __builtin_memcpy(ch, &c, sizeof(Ch));
#pragma unroll
            for (int k = 0; k < K; ++k) v.e[k * P + pw] = ch[k];
        }
    } else {
        static_assert(P % E == 0, "P and the vector's element count must divide one another");
        constexpr uint32_t R = P / E;
        const uint32_t pos = li / R, pw0 = (li % R) * E;
#pragma unroll
        for (int e = 0; e < E; ++e) v.e[e] = lds[pw0 + e][pos];
    }
    return v;
}

// A workgroup of P wavefronts owns unpatched vectors [w*P*64, (w+1)*P*64) and packed vectors
// [w*64, (w+1)*64) of every width-offset plane.  Thread t loads unpatched vector w*P*64 + t,
// which holds, for each width offset pw, K elements at consecutive packed positions: element
// k*P + pw goes to lds[pw][t*K + k].  After the barrier wavefront pw stores plane pw's 64 packed
// vectors, lds[pw][j*E .. j*E + E - 1] for lane j: one contiguous 1 KB per wavefront.  Measured
// on a 121-frame 544 x 960 bf16 clip, p = 4: 118.6 us, against 127.2 us when one wavefront did
// all of it with P loads and P stores per lane.
template <typename T, int P>
__global__ void __launch_bounds__(P * kBlock) patch_lds(PatchArgs a) {
    constexpr int E = 16 / sizeof(T);
    constexpr uint32_t U = P * kBlock;  // unpatched vectors per workgroup
    __shared__ __align__(16) T lds[P][kBlock * E];
    const uint32_t t = threadIdx.x;
    const uint32_t first = blockIdx.x * U;
    const uint32_t left = a.groups - first;
    const uint32_t valid = left < U ? left : U;  // a multiple of P: rows are whole groups of P vectors
    if (t < valid) {
        const T* src = static_cast<const T*>(a.src);
        scatter_vector<T, P>(lds, t, __builtin_bit_cast(Vec<T>, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                                              src + unpatched_offset<P, E, true>(a, first + t)))));
    }
    __syncthreads();
    const uint32_t pw = t / kBlock, j = t % kBlock;  // wavefront pw stores plane pw
    if (j >= valid / P) return;
    const uint64_t plane_stride = static_cast<uint64_t>(P) * a.F * (a.H / P) * (a.W / P);
    const uint64_t off = packed_offset0<P, E, true>(a, blockIdx.x * kBlock + j) + pw * plane_stride;
    store_out<T>(a, off, reinterpret_cast<const u32x4*>(&lds[pw][0])[j]);
}

// The inverse works on half as much per wavefront: wavefront w owns unpatched vectors
// [w*128, (w+1)*128) and packed vectors [w*128/P, (w+1)*128/P) of every width-offset plane.
// Lane l reads the wavefront's packed vectors l and l + 64 (plane-major: plane (l + 64r) /
// (128/P)) into LDS, then assembles unpatched vectors l and l + 64.  Each load instruction then
// covers whole 128/P-vector runs of 64*P/128 planes, each store instruction a contiguous 1 KB.
// Measured on a 121-frame 544 x 960 bf16 clip, p = 4: 117.1 us against 122.0 us for the
// P*64-vector wavefronts of patch_lds (and 117.8 us with 64 vectors per wavefront).
constexpr uint32_t kUnpatchVectors = 2 * kBlock;  // unpatched 16-byte vectors per wavefront

template <typename T, int P>
__global__ void __launch_bounds__(kBlock) unpatch_lds(PatchArgs a) {
    constexpr int E = 16 / sizeof(T);
    constexpr uint32_t U = kUnpatchVectors;
    constexpr uint32_t PV = U / P;  // packed vectors of each plane per wavefront
    __shared__ __align__(16) T lds[P][PV * E];
    const uint32_t lane = threadIdx.x;
    const uint32_t first = blockIdx.x * U;
    const uint32_t left = a.groups - first;
    const uint32_t valid = left < U ? left : U;  // a multiple of P: rows are whole groups of P vectors
    const T* src = static_cast<const T*>(a.src);
    const uint64_t plane_stride = static_cast<uint64_t>(P) * a.F * (a.H / P) * (a.W / P);
#pragma unroll
    for (uint32_t r = 0; r < U / kBlock; ++r) {
        const uint32_t idx = r * kBlock + lane;
        const uint32_t pw = idx / PV, j = idx % PV;
        if (j < valid / P) {
            const uint64_t off = packed_offset0<P, E, false>(a, blockIdx.x * PV + j) + pw * plane_stride;
            reinterpret_cast<u32x4*>(&lds[pw][0])[j] =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off));
        }
    }
    __syncthreads();
#pragma unroll
    for (uint32_t r = 0; r < U / kBlock; ++r) {
        const uint32_t li = r * kBlock + lane;
        if (li >= valid) break;
        store_out<T>(a, unpatched_offset<P, E, false>(a, first + li),
                     __builtin_bit_cast(u32x4, gather_vector<T, P>(lds, li)));
    }
}

template <typename T, bool INVERSE>
__global__ void __launch_bounds__(256) patch_plain(PatchArgs a) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    const T* src = static_cast<const T*>(a.src);
    T* dst = static_cast<T*>(a.dst);
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < a.numel; i += stride) {
        // i indexes the unpatched tensor (B, C, F, H, W)
        uint64_t r = i;
        const uint32_t x = static_cast<uint32_t>(r % a.W);
        r /= a.W;
        const uint32_t y = static_cast<uint32_t>(r % a.H);
        r /= a.H;
        const uint32_t f = static_cast<uint32_t>(r % a.F);
        r /= a.F;
        const uint32_t c = static_cast<uint32_t>(r % a.C);
        const uint32_t b = static_cast<uint32_t>(r / a.C);
        const uint64_t o = packed_offset(a, b, c, x % a.p, y % a.p, f, y / a.p, x / a.p);
        if constexpr (!INVERSE) {
            dst[o] = src[i];
        } else {
            dst[i] = src[o];
        }
    }
}

template <bool INV>
hipError_t launch_plain_t(PatchArgs a, uint32_t elem_bytes, hipStream_t stream, int cu_count) {
    const uint64_t want = (a.numel + 255) / 256;
    const uint64_t cap = static_cast<uint64_t>(cu_count > 0 ? cu_count : 256) * 32;
    const uint32_t blocks = static_cast<uint32_t>(want < cap ? want : cap);
    switch (elem_bytes) {
        case 1: hipLaunchKernelGGL((patch_plain<uint8_t, INV>), dim3(blocks), dim3(256), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((patch_plain<uint16_t, INV>), dim3(blocks), dim3(256), 0, stream, a); break;
        case 4: hipLaunchKernelGGL((patch_plain<uint32_t, INV>), dim3(blocks), dim3(256), 0, stream, a); break;
        case 8: hipLaunchKernelGGL((patch_plain<uint64_t, INV>), dim3(blocks), dim3(256), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int P>
hipError_t launch_lds_tp(const PatchArgs& a, bool inverse, hipStream_t stream) {
    const uint32_t per_block = inverse ? kUnpatchVectors : P * kBlock;  // unpatched vectors per workgroup
    const uint32_t blocks = (a.groups + per_block - 1) / per_block;
    if (inverse)
        hipLaunchKernelGGL((unpatch_lds<T, P>), dim3(blocks), dim3(kBlock), 0, stream, a);
    else
        hipLaunchKernelGGL((patch_lds<T, P>), dim3(blocks), dim3(P * kBlock), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_lds_t(const PatchArgs& a, uint32_t P, bool inverse, hipStream_t stream) {
    switch (P) {
        case 2: return launch_lds_tp<T, 2>(a, inverse, stream);
        case 4: return launch_lds_tp<T, 4>(a, inverse, stream);
        case 8: return launch_lds_tp<T, 8>(a, inverse, stream);
        case 16: return launch_lds_tp<T, 16>(a, inverse, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// The LDS kernels: 1, 2, 4 or 8-byte elements, p = 2, 4, 8 or 16 (so p and the 16/elem_bytes
// elements of a vector divide one another), 16-byte aligned tensors and W a multiple of
// p * 16/elem_bytes (then W/p is a multiple of 16/elem_bytes too: packed vectors stay aligned).
bool patch_fast_supported(const PatchProblem& p) {
    if (p.elem_bytes != 1 && p.elem_bytes != 2 && p.elem_bytes != 4 && p.elem_bytes != 8) return false;
    if (p.p != 2 && p.p != 4 && p.p != 8 && p.p != 16) return false;
    if (reinterpret_cast<uintptr_t>(p.src) % 16 || reinterpret_cast<uintptr_t>(p.dst) % 16) return false;
    const uint32_t E = 16 / p.elem_bytes;
    return p.W % (p.p * E) == 0;
}

hipError_t launch_patch(const PatchProblem& p, bool inverse, hipStream_t stream, int cu_count) {
    PatchArgs a{};
    a.src = p.src;
    a.dst = p.dst;
    a.B = p.B;
    a.C = p.C;
    a.F = p.F;
    a.H = p.H;
    a.W = p.W;
    a.p = p.p;
    a.numel = static_cast<uint64_t>(p.B) * p.C * p.F * p.H * p.W;
    a.groups = 0;
    const uint64_t bytes = a.numel * p.elem_bytes;
    a.dst_bytes = bytes < (uint64_t(1) << 31) ? static_cast<uint32_t>(bytes) : 0u;
    if (a.numel == 0) return hipSuccess;
    if (patch_fast_supported(p) && !p.force_plain) {
        const uint32_t E = 16 / p.elem_bytes;
        a.groups = static_cast<uint32_t>(a.numel / E);  // 16-byte vectors of the unpatched tensor
        a.div_WE = make_fastdiv(p.W / E);
        a.div_WpE = make_fastdiv(p.W / p.p / E);
        a.div_Hp = make_fastdiv(p.H / p.p);
        a.div_F = make_fastdiv(p.F);
        switch (p.elem_bytes) {
            case 1: return launch_lds_t<uint8_t>(a, p.p, inverse, stream);
            case 2: return launch_lds_t<uint16_t>(a, p.p, inverse, stream);
            case 4: return launch_lds_t<uint32_t>(a, p.p, inverse, stream);
            default: return launch_lds_t<uint64_t>(a, p.p, inverse, stream);
        }
    }
    return inverse ? launch_plain_t<true>(a, p.elem_bytes, stream, cu_count)
                   : launch_plain_t<false>(a, p.elem_bytes, stream, cu_count);
}

}  // namespace ltx3drope
