// The plain kernel of the fused 3D RoPE for gfx950: the bit-exact gate's
// reference path and the fallback for shapes the fast kernel does not cover.
//
// One wavefront per token of Q or of K, written from the eager definition
// (sglang PR #35698 page, "Implementation breakdown", step 2): the token's
// (t, h, w) is peeled from its place in the contiguous
// [B, T, H, W, heads, head_dim] layout; the lanes spread over the pairs of a
// head row, each finding its chunk (time, height, width) by walking the chunk
// widths and reading that axis's table row at the token's coordinate once,
// then rotating that pair in every head of the token, eight head rows loaded
// at a time; scalar loads and stores, integer round-to-nearest-even.  With
// VERIFY it recomputes the result and counts pairs whose bits differ from what
// the outputs already hold.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <type_traits>

#include "internal.h"
#include "pair_math.h"

#pragma clang fp contract(off)

namespace ltx3drope {
namespace {

constexpr int kPlainBlock = 256;

// ---------------------------------------------------------------------------
// plain kernel: one token per wavefront
// ---------------------------------------------------------------------------

struct PlainArgs {
    const void* src[2];  // Q, K
    void* dst[2];        // Q_out, K_out
    const float2* tab;   // packed (cos, sin) pairs: the t section, then h, then w
    unsigned* mismatches;
    uint32_t tokens;            // tokens per tensor, B*T*H*W; the grid covers both tensors
    uint32_t heads, half_dim;   // heads per token, pairs per head row (head_dim / 2)
    uint32_t T, H, W;           // the tensor's grid
    uint32_t origin[3];         // coordinate of the tensor's first frame / row / column in the tables' grid
    uint32_t width[3];          // pairs of the t, h and w chunks of a head row
    uint32_t section[3];        // first pair of the t, h and w sections of the packed tables
};

constexpr uint32_t kPlainHeads = 8;  // head rows whose pairs a lane loads before it rotates them

template <bool BF16, bool VERIFY>
__global__ void __launch_bounds__(kPlainBlock) rope_plain(PlainArgs a) {
    constexpr uint32_t kWaves = kPlainBlock / 64;
    using Pair = typename std::conditional<BF16, uint32_t, uint2>::type;  // one (even, odd) pair
    uint32_t bad = 0;
    const uint32_t lane = threadIdx.x % 64;
    // 2 * tokens < 2^32 (a launch holds fewer than 2^32 elements, a token at least 2); the index is
    // 64-bit so that adding the grid's stride cannot wrap
    const uint64_t items = 2ull * a.tokens;
    const uint64_t stride = uint64_t(gridDim.x) * kWaves;
    for (uint64_t item = uint64_t(blockIdx.x) * kWaves + threadIdx.x / 64; item < items; item += stride) {
        const uint32_t x = item < a.tokens ? 0 : 1;  // 0: Q, 1: K
        const uint32_t token = static_cast<uint32_t>(item - x * uint64_t(a.tokens));
        // token = ((b*T + t)*H + h)*W + w: peel the layout from the innermost axis out
        uint32_t coord[3];
        coord[2] = token % a.W;
        uint32_t rest = token / a.W;
        coord[1] = rest % a.H;
        rest /= a.H;
        coord[0] = rest % a.T;
        const Pair* src = static_cast<const Pair*>(a.src[x]);
        Pair* dst = static_cast<Pair*>(a.dst[x]);
        const uint32_t first = token * a.heads * a.half_dim;  // the token's first (even, odd) pair; < 2^31
        for (uint32_t j = lane; j < a.half_dim; j += 64) {
            // pair j of a head row: walk the t, h and w chunk widths to its table; the same
            // (cos, sin) serves every head of the token
            int axis = 0;
            uint32_t col = j;
            while (axis < 2 && col >= a.width[axis]) col -= a.width[axis++];
            const float2 cs = a.tab[a.section[axis] + (coord[axis] + a.origin[axis]) * a.width[axis] + col];
            for (uint32_t h0 = 0; h0 < a.heads; h0 += kPlainHeads) {
                const uint32_t n = a.heads - h0 < kPlainHeads ? a.heads - h0 : kPlainHeads;
                Pair in[kPlainHeads];
#pragma unroll
                for (uint32_t i = 0; i < kPlainHeads; ++i)
                    if (i < n) in[i] = src[first + (h0 + i) * a.half_dim + j];
#pragma unroll
                for (uint32_t i = 0; i < kPlainHeads; ++i) {
                    if (i >= n) break;
                    float ye, yo;
                    Pair out;
                    if constexpr (BF16) {
                        rotate(bf16_lo(in[i]), bf16_hi(in[i]), cs.x, cs.y, ye, yo);
                        out = bf16_rne_int(ye) | (bf16_rne_int(yo) << 16);
                    } else {
                        rotate(__uint_as_float(in[i].x), __uint_as_float(in[i].y), cs.x, cs.y, ye, yo);
                        out = make_uint2(f32_canon(ye), f32_canon(yo));
                    }
                    Pair* at = dst + first + (h0 + i) * a.half_dim + j;
                    if constexpr (VERIFY) {
                        const Pair have = *at;
                        if constexpr (BF16)
                            bad += have != out ? 1u : 0u;
                        else
                            bad += (have.x != out.x || have.y != out.y) ? 1u : 0u;
                    } else {
                        *at = out;
                    }
                }
            }
        }
    }
    if constexpr (VERIFY) {
        if (bad != 0) atomicAdd(a.mismatches, bad);
    }
}

std::mutex g_cu_mu;
std::map<int, int> g_cu;

int plain_cu_count(int device) {
    std::lock_guard<std::mutex> lock(g_cu_mu);
    auto it = g_cu.find(device);
    if (it != g_cu.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    g_cu[device] = n;
    return n;
}

PlainArgs plain_args(const Problem& p, unsigned* mismatches) {
    PlainArgs a;
    a.src[0] = p.q;
    a.src[1] = p.k;
    a.dst[0] = p.q_out;
    a.dst[1] = p.k_out;
    a.tab = reinterpret_cast<const float2*>(p.tab);
    a.mismatches = mismatches;
    a.tokens = p.B * p.T * p.H * p.W;  // < 2^31 (a launch holds fewer than 2^32 elements, a token at least 2)
    a.heads = p.heads;
    a.half_dim = p.D / 2;
    a.T = p.T;
    a.H = p.H;
    a.W = p.W;
    a.origin[0] = p.t_off;
    a.origin[1] = p.h_off;
    a.origin[2] = p.w_off;
    a.width[0] = p.PT;
    a.width[1] = p.PH;
    a.width[2] = p.PW;
    a.section[0] = 0;
    a.section[1] = p.tabT * p.PT;
    a.section[2] = p.tabT * p.PT + p.tabH * p.PH;
    return a;
}

template <bool VERIFY>
hipError_t launch_plain_impl(const Problem& p, unsigned* mismatches, hipStream_t stream, int device) {
    const PlainArgs a = plain_args(p, mismatches);
    const uint64_t want = (2ull * a.tokens + kPlainBlock / 64 - 1) / (kPlainBlock / 64);  // one token per wavefront
    const uint64_t cap = static_cast<uint64_t>(plain_cu_count(device)) * 32u;
    const uint32_t blocks = static_cast<uint32_t>(want < cap ? want : cap);
    if (blocks == 0) return hipSuccess;
    if (p.dtype == LTX3DROPE_DTYPE_BF16)
        hipLaunchKernelGGL((rope_plain<true, VERIFY>), dim3(blocks), dim3(kPlainBlock), 0, stream, a);
    else
        hipLaunchKernelGGL((rope_plain<false, VERIFY>), dim3(blocks), dim3(kPlainBlock), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_plain(const Problem& p, hipStream_t stream, int device) {
    return launch_plain_impl<false>(p, nullptr, stream, device);
}

hipError_t launch_verify(const Problem& p, unsigned* mismatches, hipStream_t stream, int device) {
    return launch_plain_impl<true>(p, mismatches, stream, device);
}

}  // namespace ltx3drope
