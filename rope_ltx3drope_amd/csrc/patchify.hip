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
//  * patch_fast<T, P>: one thread per group of P consecutive 16-byte vectors of
//    an input row (P * E elements, E = 16 / sizeof(T)).  Those elements feed P
//    output rows (one per width offset) with E consecutive elements each, so
//    the thread transposes P x E elements in registers and writes P 16-byte
//    vectors.  Used for patchify, and for the inverse when a vector does not
//    split evenly across the P width offsets.  Needs W to be a multiple of
//    P * E and 16-byte aligned tensors.
//  * unpatch_gather<T, P>: the inverse with one unpatched 16-byte vector per
//    thread and P loads of E/P packed elements.
//  * patch_plain<T, INVERSE>: one element per thread, any shape.
// Threads are ordered (b, c, f, height offset, patch row, vector) rather than
// by input row: a wavefront then writes (patchify) or reads (unpatchify)
// consecutive rows of one packed plane, whose rows of W/p elements are not
// whole cache lines.  Measured on a 121-frame 544 x 960 bf16 clip, p = 4:
// patchify 5.5 TB/s against 4.1 TB/s in input-row order; unpatchify 5.9 TB/s
// (with non-temporal hints, which help only once every instruction is
// contiguous).  The register-transpose kernel keeps plain loads and stores:
// with non-temporal hints it measured slower.
#include <hip/hip_runtime.h>

#include "internal.h"

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
    uint32_t groups_per_row;  // fast kernel: W / (P * E)
    uint32_t groups;          // fast kernel: B*C*F*H*groups_per_row
    uint64_t numel;           // plain kernel
};

// Element offset of output channel (c*p + pw)*p + ph, frame f, patch row hh, column ww.
__device__ __forceinline__ uint64_t packed_offset(const PatchArgs& a, uint32_t b, uint32_t c, uint32_t pw,
                                                  uint32_t ph, uint32_t f, uint32_t hh, uint32_t ww) {
    const uint32_t Hp = a.H / a.p, Wp = a.W / a.p;
    const uint64_t co = (static_cast<uint64_t>(b) * a.C + c) * a.p * a.p + static_cast<uint64_t>(pw) * a.p + ph;
    return ((co * a.F + f) * Hp + hh) * Wp + ww;
}

template <typename T, int P, bool INVERSE>
__global__ void __launch_bounds__(kBlock) patch_fast(PatchArgs a) {
    constexpr int E = 16 / sizeof(T);
    const uint32_t g = blockIdx.x * kBlock + threadIdx.x;
    if (g >= a.groups) return;
    // thread order (b, c, f, ph, hh, gi): consecutive threads walk the patch rows of one
    // height offset, so a wavefront's stores for one width offset fill consecutive rows of
    // one output plane, and each input row is read whole by one wavefront
    uint32_t t = g / a.groups_per_row;
    const uint32_t gi = g - t * a.groups_per_row;
    const uint32_t Hp = a.H / P;
    const uint32_t hh = t % Hp;
    t /= Hp;
    const uint32_t ph = t % P;
    t /= P;
    const uint32_t f = t % a.F;
    t /= a.F;
    const uint32_t c = t % a.C;
    const uint32_t b = t / a.C;
    const uint64_t row = ((static_cast<uint64_t>(b) * a.C + c) * a.F + f) * a.H + hh * P + ph;
    const uint64_t row_off = row * a.W + static_cast<uint64_t>(gi) * (P * E);
    const T* src = static_cast<const T*>(a.src);
    T* dst = static_cast<T*>(a.dst);
    if constexpr (!INVERSE) {
        Vec<T> in[P];
#pragma unroll
        for (int r = 0; r < P; ++r)
            in[r] = __builtin_bit_cast(Vec<T>, reinterpret_cast<const u32x4*>(src + row_off)[r]);
#pragma unroll
        for (int pw = 0; pw < P; ++pw) {
            Vec<T> o;
#pragma unroll
            for (int w = 0; w < E; ++w) o.e[w] = in[(w * P + pw) / E].e[(w * P + pw) % E];
            const uint64_t off = packed_offset(a, b, c, pw, ph, f, hh, gi * E);
            *reinterpret_cast<u32x4*>(dst + off) = __builtin_bit_cast(u32x4, o);
        }
    } else {
        Vec<T> in[P];
#pragma unroll
        for (int pw = 0; pw < P; ++pw) {
            const uint64_t off = packed_offset(a, b, c, pw, ph, f, hh, gi * E);
            in[pw] = __builtin_bit_cast(Vec<T>, *reinterpret_cast<const u32x4*>(src + off));
        }
#pragma unroll
        for (int r = 0; r < P; ++r) {
            Vec<T> o;
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const int col = r * E + j;  // column inside the group: w * P + pw
                o.e[j] = in[col % P].e[col / P];
            }
            reinterpret_cast<u32x4*>(dst + row_off)[r] = __builtin_bit_cast(u32x4, o);
        }
    }
}

// Inverse with one 16-byte vector of the unpatched tensor per thread (E elements,
// columns E*vi .. E*vi + E - 1 of one row): for each width offset pw it loads the
// K = E / P consecutive packed elements at patch columns K*vi .. K*vi + K - 1,
// then interleaves them.  Consecutive lanes touch consecutive addresses in every
// load (K elements each) and store (16 bytes each), so every instruction is
// contiguous across the wavefront.
template <int NB>
struct Chunk;  // a naturally aligned chunk of NB bytes
template <>
struct Chunk<2> { typedef uint16_t type; };
template <>
struct Chunk<4> { typedef uint32_t type; };
template <>
struct Chunk<8> { typedef unsigned type __attribute__((ext_vector_type(2))); };

template <typename T, int P>
__global__ void __launch_bounds__(kBlock) unpatch_gather(PatchArgs a) {
    constexpr int E = 16 / sizeof(T);
    constexpr int K = E / P;  // packed elements per width offset
    static_assert(K * P == E && K >= 1, "a vector must split evenly across the width offsets");
    typedef typename Chunk<K * sizeof(T)>::type C;
    const uint32_t g = blockIdx.x * kBlock + threadIdx.x;
    if (g >= a.groups) return;  // here: 16-byte vectors of the unpatched tensor
    // thread order (b, c, f, ph, hh, vi): consecutive threads read consecutive packed
    // elements of one plane, across its rows
    const uint32_t vpr = a.W / E;
    uint32_t t = g / vpr;
    const uint32_t vi = g - t * vpr;
    const uint32_t Hp = a.H / P;
    const uint32_t hh = t % Hp;
    t /= Hp;
    const uint32_t ph = t % P;
    t /= P;
    const uint32_t f = t % a.F;
    t /= a.F;
    const uint32_t c = t % a.C;
    const uint32_t b = t / a.C;
    const uint64_t row = ((static_cast<uint64_t>(b) * a.C + c) * a.F + f) * a.H + hh * P + ph;
    const T* src = static_cast<const T*>(a.src);
    Vec<T> seg[P];
#pragma unroll
    for (int pw = 0; pw < P; ++pw) {
        const C v = __builtin_nontemporal_load(
            reinterpret_cast<const C*>(src + packed_offset(a, b, c, pw, ph, f, hh, vi * K)));
        Vec<T> piece{};
        __builtin_memcpy(&piece.e[0], &v, sizeof(C));  // the first K elements
        seg[pw] = piece;
    }
    Vec<T> o;
#pragma unroll
    for (int j = 0; j < E; ++j) o.e[j] = seg[j % P].e[j / P];
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o),
                                reinterpret_cast<u32x4*>(static_cast<T*>(a.dst) + row * a.W) + vi);
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

template <typename T, bool INV>
hipError_t launch_fast_t(PatchArgs a, uint32_t P, hipStream_t stream) {
    const uint32_t blocks = (a.groups + kBlock - 1) / kBlock;
    switch (P) {
        case 2: hipLaunchKernelGGL((patch_fast<T, 2, INV>), dim3(blocks), dim3(kBlock), 0, stream, a); break;
        case 4: hipLaunchKernelGGL((patch_fast<T, 4, INV>), dim3(blocks), dim3(kBlock), 0, stream, a); break;
        case 8: hipLaunchKernelGGL((patch_fast<T, 8, INV>), dim3(blocks), dim3(kBlock), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
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

}  // namespace

bool patch_fast_supported(const PatchProblem& p) {
    if (p.elem_bytes != 2 && p.elem_bytes != 4) return false;
    if (p.p != 2 && p.p != 4 && p.p != 8) return false;
    if (reinterpret_cast<uintptr_t>(p.src) % 16 || reinterpret_cast<uintptr_t>(p.dst) % 16) return false;
    const uint32_t E = 16 / p.elem_bytes;
    return p.W % (p.p * E) == 0;  // then W/p is a multiple of E too: output vectors stay aligned
}

hipError_t launch_patch(const PatchProblem& p, bool inverse, hipStream_t stream, int cu_count) {
    PatchArgs a;
    a.src = p.src;
    a.dst = p.dst;
    a.B = p.B;
    a.C = p.C;
    a.F = p.F;
    a.H = p.H;
    a.W = p.W;
    a.p = p.p;
    a.numel = static_cast<uint64_t>(p.B) * p.C * p.F * p.H * p.W;
    a.groups_per_row = 0;
    a.groups = 0;
    if (a.numel == 0) return hipSuccess;
    if (patch_fast_supported(p) && !p.force_plain) {
        const uint32_t E = 16 / p.elem_bytes;
        if (inverse && E % p.p == 0) {
            a.groups = static_cast<uint32_t>(a.numel / E);  // one unpatched 16-byte vector per thread
            const uint32_t blocks = (a.groups + kBlock - 1) / kBlock;
            if (p.elem_bytes == 2) {
                if (p.p == 2) hipLaunchKernelGGL((unpatch_gather<uint16_t, 2>), dim3(blocks), dim3(kBlock), 0, stream, a);
                else if (p.p == 4) hipLaunchKernelGGL((unpatch_gather<uint16_t, 4>), dim3(blocks), dim3(kBlock), 0, stream, a);
                else hipLaunchKernelGGL((unpatch_gather<uint16_t, 8>), dim3(blocks), dim3(kBlock), 0, stream, a);
            } else {
                if (p.p == 2) hipLaunchKernelGGL((unpatch_gather<uint32_t, 2>), dim3(blocks), dim3(kBlock), 0, stream, a);
                else hipLaunchKernelGGL((unpatch_gather<uint32_t, 4>), dim3(blocks), dim3(kBlock), 0, stream, a);
            }
            return hipGetLastError();
        }
        a.groups_per_row = p.W / (p.p * E);
        a.groups = static_cast<uint32_t>(a.numel / (p.p * E));
        if (p.elem_bytes == 2)
            return inverse ? launch_fast_t<uint16_t, true>(a, p.p, stream) : launch_fast_t<uint16_t, false>(a, p.p, stream);
        return inverse ? launch_fast_t<uint32_t, true>(a, p.p, stream) : launch_fast_t<uint32_t, false>(a, p.p, stream);
    }
    return inverse ? launch_plain_t<true>(a, p.elem_bytes, stream, cu_count)
                   : launch_plain_t<false>(a, p.elem_bytes, stream, cu_count);
}

}  // namespace ltx3drope
