// HIP kernels of the rotate-half ("NeoX") RoPE with a position-gathered cos/sin
// cache, for gfx950, and their launchers.
//
// Operation (sglang PR #24660 page, "Key source snippets", the Gemma3 text
// encoder's rotary application; "Implementation breakdown", step 2): for each
// token the cache row at its position holds cos[0:D/2] | sin[0:D/2]; both are
// duplicated to the full head and cast to q's dtype, and
//     q' = q * cos + rotate_half(q) * sin,   rotate_half(x) = (-x[D/2:], x[:D/2])
// i.e. for i < D/2, with c = cos[i], s = sin[i]:
//     q'[i]       = R( R(q[i] * c)       + R(-q[i + D/2] * s) )
//     q'[i + D/2] = R( R(q[i + D/2] * c) + R(q[i] * s) )
// where R rounds an fp32 result to q's dtype (each tensor op of the expression
// yields a tensor of q's dtype; fp32 inputs make R the fp32 rounding itself).
// No fused multiply-add (contraction is off in this file).  Same for k.
//
// Kernels:
//  * neox_fast: one wavefront per token of Q, then one per token of K.  Each
//    lane owns one 16-byte vector of the first half of a head row and the
//    matching vector of the second half, for a set of heads: it loads its
//    cos/sin segment once, reads both vectors of a head, writes both, so
//    in-place calls are safe.  bf16 rounding uses the hardware's
//    round-to-nearest-even conversion.
//  * neox_plain: one (i, i + D/2) element pair per thread, scalar accesses,
//    integer round-to-nearest-even; any even head_dim, any 2-element alignment.
// A position outside [0, max_position) is never dereferenced: the token's
// outputs become NaN and the (token, tensor) is counted in `errors`.  Every NaN
// output is the canonical quiet NaN (0x7FC00000 fp32, 0x7FC0 bf16).
#include <hip/hip_runtime.h>

#include "internal.h"
#include "stream_store.h"

#pragma clang fp contract(off)

namespace ltx3drope {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kBlock = 64;  // one wavefront per workgroup

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_hw(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint32_t rne_int(float y) {
    const uint32_t u = __float_as_uint(y);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// fp32 bits with any NaN replaced by the canonical quiet NaN.
__device__ __forceinline__ uint32_t canon_f32(float y) { return y != y ? 0x7fc00000u : __float_as_uint(y); }

// Two fp32 results packed to bf16 (hardware conversion), any NaN written as the canonical 0x7FC0.
__device__ __forceinline__ uint32_t pack_out(float lo, float hi) {
    uint32_t w = pack_hw(lo, hi);
    if (lo != lo) w = (w & 0xffff0000u) | 0x7fc0u;
    if (hi != hi) w = (w & 0x0000ffffu) | 0x7fc00000u;
    return w;
}

// Rounds two fp32 values to bf16 and back (hardware conversion).
__device__ __forceinline__ void round2_bf16(float& a, float& b) {
    const uint32_t p = pack_hw(a, b);
    a = bf16_lo(p);
    b = bf16_hi(p);
}

struct NeoxArgs {
    const void* q;
    const void* k;
    void* q_out;
    void* k_out;
    const int64_t* pos;
    const void* cache;
    unsigned* errors;
    uint32_t tokens, q_heads, k_heads, D;
    uint32_t max_pos;
    uint32_t vh;         // 16-B vectors per half head row (fast kernel)
    uint32_t q_items, k_items;  // element pairs of Q and of K (plain kernel)
};

// Cache values of one 16-B vector of q: 8 (bf16 q) or 4 (fp32 q) consecutive cos, the same sin.
template <bool QBF16, bool CBF16>
__device__ __forceinline__ void load_cs(const void* cache, size_t row_elem, uint32_t half, uint32_t col,
                                        float* c, float* s) {
    constexpr int E = QBF16 ? 8 : 4;
    if constexpr (CBF16) {
        const uint16_t* base = static_cast<const uint16_t*>(cache) + row_elem;
        if constexpr (E == 8) {
            const u32x4 cv = *reinterpret_cast<const u32x4*>(base + col);
            const u32x4 sv = *reinterpret_cast<const u32x4*>(base + half + col);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                c[2 * r] = bf16_lo(cv[r]);
                c[2 * r + 1] = bf16_hi(cv[r]);
                s[2 * r] = bf16_lo(sv[r]);
                s[2 * r + 1] = bf16_hi(sv[r]);
            }
        } else {
            const uint2 cv = *reinterpret_cast<const uint2*>(base + col);
            const uint2 sv = *reinterpret_cast<const uint2*>(base + half + col);
            c[0] = bf16_lo(cv.x); c[1] = bf16_hi(cv.x); c[2] = bf16_lo(cv.y); c[3] = bf16_hi(cv.y);
            s[0] = bf16_lo(sv.x); s[1] = bf16_hi(sv.x); s[2] = bf16_lo(sv.y); s[3] = bf16_hi(sv.y);
        }
    } else {
        const float* base = static_cast<const float*>(cache) + row_elem;
#pragma unroll
        for (int r = 0; r < E / 4; ++r) {
            const f32x4 cv = *reinterpret_cast<const f32x4*>(base + col + 4 * r);
            const f32x4 sv = *reinterpret_cast<const f32x4*>(base + half + col + 4 * r);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[4 * r + j] = cv[j];
                s[4 * r + j] = sv[j];
            }
        }
    }
}

// One wavefront per token (Q tokens in the first part of the grid, K tokens in the
// second).  Lane = (head slot hs, vector v): v < vh indexes the 16-B vectors of a
// half head row, hs < 64 / vh; the lane loads its cos/sin segment once and
// applies it to heads hs, hs + 64/vh, ...  (loading the segment per head cost
// 12 % on a 32k-token bf16 workload: measured 6.4 against 5.9 TB/s).
template <bool QBF16, bool CBF16>
__global__ void __launch_bounds__(kBlock) neox_fast(NeoxArgs a) {
    constexpr int E = QBF16 ? 8 : 4;  // elements per 16-B vector
    constexpr uint32_t es = QBF16 ? 2 : 4;
    const bool second = blockIdx.x >= a.tokens;  // wave-uniform: Q part, then K part
    const uint32_t tok = second ? blockIdx.x - a.tokens : blockIdx.x;
    const uint32_t heads = second ? a.k_heads : a.q_heads;
    const uint32_t hpw = 64u / a.vh;  // head slots per wavefront (vh <= 64 on this path)
    const uint32_t v = threadIdx.x % a.vh;
    const uint32_t hs = threadIdx.x / a.vh;
    if (hs >= hpw) return;
    const char* src = static_cast<const char*>(second ? a.k : a.q);
    char* dst = static_cast<char*>(second ? a.k_out : a.q_out);
    const int64_t p = a.pos[tok];
    const bool bad = p < 0 || p >= static_cast<int64_t>(a.max_pos);
    float c[E], s[E];
    if (!bad) {
        load_cs<QBF16, CBF16>(a.cache, static_cast<size_t>(p) * a.D, a.D / 2, v * E, c, s);
        if constexpr (QBF16 && !CBF16) {  // cast the cache values to q's dtype
#pragma unroll
            for (int j = 0; j < E; j += 2) {
                round2_bf16(c[j], c[j + 1]);
                round2_bf16(s[j], s[j + 1]);
            }
        }
    } else if (hs == 0 && v == 0) {
        atomicAdd(a.errors, 1u);
    }
    const uint32_t token_bytes = heads * a.D * es;  // below 2^31: checked on the host
    char* const dst_tok = dst + static_cast<size_t>(tok) * token_bytes;  // wave-uniform
    for (uint32_t head = hs; head < heads; head += hpw) {
        const size_t row = (static_cast<size_t>(tok) * heads + head) * a.D;  // element offset of the head row
        const size_t off1 = (row + static_cast<size_t>(v) * E) * es;
        const size_t off2 = off1 + static_cast<size_t>(a.D / 2) * es;
        const uint32_t in_tok1 = (head * a.D + v * E) * es;  // off1 - tok * token_bytes
        const uint32_t in_tok2 = in_tok1 + (a.D / 2) * es;
        const u32x4 x1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off1));
        const u32x4 x2 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off2));
        u32x4 y1, y2;
        if (bad) {
            const uint32_t nan = QBF16 ? 0x7fc07fc0u : 0x7fc00000u;
            y1 = (u32x4){nan, nan, nan, nan};
            y2 = y1;
        } else if constexpr (QBF16) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {  // one 32-bit word = two elements
                float a1[2], b1[2], a2[2], b2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float e1 = h ? bf16_hi(x1[w]) : bf16_lo(x1[w]);
                    const float e2 = h ? bf16_hi(x2[w]) : bf16_lo(x2[w]);
                    const int j = 2 * w + h;
                    a1[h] = __fmul_rn(e1, c[j]);
                    b1[h] = __fmul_rn(-e2, s[j]);
                    a2[h] = __fmul_rn(e2, c[j]);
                    b2[h] = __fmul_rn(e1, s[j]);
                }
                round2_bf16(a1[0], a1[1]);
                round2_bf16(b1[0], b1[1]);
                round2_bf16(a2[0], a2[1]);
                round2_bf16(b2[0], b2[1]);
                y1[w] = pack_out(__fadd_rn(a1[0], b1[0]), __fadd_rn(a1[1], b1[1]));
                y2[w] = pack_out(__fadd_rn(a2[0], b2[0]), __fadd_rn(a2[1], b2[1]));
            }
        } else {
#pragma unroll
            for (int j = 0; j < E; ++j) {
                const float e1 = __uint_as_float(x1[j]);
                const float e2 = __uint_as_float(x2[j]);
                y1[j] = canon_f32(__fadd_rn(__fmul_rn(e1, c[j]), __fmul_rn(-e2, s[j])));
                y2[j] = canon_f32(__fadd_rn(__fmul_rn(e2, c[j]), __fmul_rn(e1, s[j])));
            }
        }
        stream_store16(y1, dst_tok, token_bytes, in_tok1);
        stream_store16(y2, dst_tok, token_bytes, in_tok2);
    }
}

template <bool QBF16, bool CBF16>
__global__ void __launch_bounds__(256) neox_plain(NeoxArgs a) {
    const uint32_t half = a.D / 2;
    const uint64_t total = uint64_t(a.q_items) + a.k_items;  // element pairs of Q, then of K
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint64_t g = blockIdx.x * blockDim.x + threadIdx.x; g < total; g += stride) {
        const bool second = g >= a.q_items;
        const uint32_t i = static_cast<uint32_t>(second ? g - a.q_items : g);
        const uint32_t heads = second ? a.k_heads : a.q_heads;
        const uint32_t col = i % half;
        const uint32_t row = i / half;  // (token, head)
        const uint32_t tok = row / heads;
        const uint32_t head = row - tok * heads;
        const size_t e1i = static_cast<size_t>(row) * a.D + col;
        const size_t e2i = e1i + half;
        const int64_t p = a.pos[tok];
        if (p < 0 || p >= static_cast<int64_t>(a.max_pos)) {
            if (QBF16) {
                uint16_t* d = static_cast<uint16_t*>(second ? a.k_out : a.q_out);
                d[e1i] = 0x7fc0u;
                d[e2i] = 0x7fc0u;
            } else {
                float* d = static_cast<float*>(second ? a.k_out : a.q_out);
                d[e1i] = __uint_as_float(0x7fc00000u);
                d[e2i] = __uint_as_float(0x7fc00000u);
            }
            if (head == 0 && col == 0) atomicAdd(a.errors, 1u);
            continue;
        }
        const size_t ci = static_cast<size_t>(p) * a.D + col;
        float c, s;
        if (CBF16) {
            const uint16_t* cc = static_cast<const uint16_t*>(a.cache);
            c = __uint_as_float(static_cast<uint32_t>(cc[ci]) << 16);
            s = __uint_as_float(static_cast<uint32_t>(cc[ci + half]) << 16);
        } else {
            const float* cc = static_cast<const float*>(a.cache);
            c = cc[ci];
            s = cc[ci + half];
        }
        if (QBF16) {
            const uint16_t* x = static_cast<const uint16_t*>(second ? a.k : a.q);
            uint16_t* d = static_cast<uint16_t*>(second ? a.k_out : a.q_out);
            auto R = [](float y) { return __uint_as_float(rne_int(y) << 16); };
            c = R(c);
            s = R(s);
            const float e1 = __uint_as_float(static_cast<uint32_t>(x[e1i]) << 16);
            const float e2 = __uint_as_float(static_cast<uint32_t>(x[e2i]) << 16);
            const float y1 = __fadd_rn(R(__fmul_rn(e1, c)), R(__fmul_rn(-e2, s)));
            const float y2 = __fadd_rn(R(__fmul_rn(e2, c)), R(__fmul_rn(e1, s)));
            d[e1i] = static_cast<uint16_t>(rne_int(y1));
            d[e2i] = static_cast<uint16_t>(rne_int(y2));
        } else {
            const float* x = static_cast<const float*>(second ? a.k : a.q);
            float* d = static_cast<float*>(second ? a.k_out : a.q_out);
            const float e1 = x[e1i], e2 = x[e2i];
            d[e1i] = __uint_as_float(canon_f32(__fadd_rn(__fmul_rn(e1, c), __fmul_rn(-e2, s))));
            d[e2i] = __uint_as_float(canon_f32(__fadd_rn(__fmul_rn(e2, c), __fmul_rn(e1, s))));
        }
    }
}

NeoxArgs make_args(const NeoxProblem& p, unsigned* errors) {
    NeoxArgs a;
    a.q = p.q;
    a.k = p.k;
    a.q_out = p.q_out;
    a.k_out = p.k_out;
    a.pos = p.positions;
    a.cache = p.cache;
    a.errors = errors;
    a.tokens = p.tokens;
    a.q_heads = p.q_heads;
    a.k_heads = p.k_heads;
    a.D = p.D;
    a.max_pos = p.max_position;
    a.vh = 0;
    a.q_items = 0;
    a.k_items = 0;
    return a;
}

}  // namespace

// Half head rows of whole 16-B vectors (at most 64 of them), 16-B aligned
// tensors and at most 2^25 - 1 tokens (two 64-lane workgroups per token, and a
// grid holds fewer than 2^32 work-items).  Then every cache segment a vector
// needs (8 or 4 values, of 2 or 4 bytes) is naturally aligned: the row offset
// p*D and the half offset D/2 are multiples of the segment length.
bool neox_fast_supported(const NeoxProblem& p) {
    const uint32_t es = p.dtype == LTX3DROPE_DTYPE_F32 ? 4u : 2u;
    for (const void* ptr : {p.q, p.k, static_cast<const void*>(p.q_out), static_cast<const void*>(p.k_out), p.cache})
        if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return false;
    const uint64_t heads = p.q_heads > p.k_heads ? p.q_heads : p.k_heads;
    if (heads * p.D * es >= (uint64_t(1) << 31)) return false;  // a token's row is addressed with 32-bit offsets
    if (uint64_t(p.tokens) * 2 * kBlock > 0xffffffffull) return false;  // the grid's work-items must fit in 32 bits
    return (p.D / 2 * es) % 16 == 0 && p.D / 2 * es / 16 <= 64;
}

hipError_t launch_neox_fast(const NeoxProblem& p, unsigned* errors, hipStream_t stream) {
    if (!neox_fast_supported(p)) return hipErrorInvalidValue;
    NeoxArgs a = make_args(p, errors);
    const uint32_t es = p.dtype == LTX3DROPE_DTYPE_F32 ? 4u : 2u;
    a.vh = p.D / 2 * es / 16;
    const uint32_t blocks = 2 * p.tokens;  // one wavefront per token of Q, then of K
    if (blocks == 0) return hipSuccess;
    const bool qb = p.dtype == LTX3DROPE_DTYPE_BF16, cb = p.cache_dtype == LTX3DROPE_DTYPE_BF16;
    if (qb && cb)
        hipLaunchKernelGGL((neox_fast<true, true>), dim3(blocks), dim3(kBlock), 0, stream, a);
    else if (qb)
        hipLaunchKernelGGL((neox_fast<true, false>), dim3(blocks), dim3(kBlock), 0, stream, a);
    else if (cb)
        hipLaunchKernelGGL((neox_fast<false, true>), dim3(blocks), dim3(kBlock), 0, stream, a);
    else
        hipLaunchKernelGGL((neox_fast<false, false>), dim3(blocks), dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_neox_plain(const NeoxProblem& p, unsigned* errors, hipStream_t stream, int cu_count) {
    NeoxArgs a = make_args(p, errors);
    a.q_items = p.tokens * p.q_heads * (p.D / 2);  // each below 2^31: tensors have fewer than 2^32 elements
    a.k_items = p.tokens * p.k_heads * (p.D / 2);
    const uint64_t total = uint64_t(a.q_items) + a.k_items;
    const uint32_t want = static_cast<uint32_t>((total + 255) / 256);
    const uint32_t cap = static_cast<uint32_t>(cu_count > 0 ? cu_count : 256) * 32u;
    const uint32_t blocks = want < cap ? want : cap;
    if (blocks == 0) return hipSuccess;
    const bool qb = p.dtype == LTX3DROPE_DTYPE_BF16, cb = p.cache_dtype == LTX3DROPE_DTYPE_BF16;
    if (qb && cb)
        hipLaunchKernelGGL((neox_plain<true, true>), dim3(blocks), dim3(256), 0, stream, a);
    else if (qb)
        hipLaunchKernelGGL((neox_plain<true, false>), dim3(blocks), dim3(256), 0, stream, a);
    else if (cb)
        hipLaunchKernelGGL((neox_plain<false, true>), dim3(blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((neox_plain<false, false>), dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ltx3drope
