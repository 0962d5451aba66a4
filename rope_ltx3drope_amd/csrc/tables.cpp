// Per-axis cos/sin tables and their FIFO cache.
//
// sglang PR #35698 page, "Implementation breakdown", step 1: the per-axis
// (cos, sin) tables of a (num_frames, height, width) grid are a pure function
// of (grid, rope_dim_split, base, device), small, and shared by every decoder
// block on that grid; they are cached under that key, at most 16 entries, with
// simple first-in first-out eviction.
//
// This file is compiled without floating-point contraction or fast-math: the
// table values are float64 libm results rounded once to fp32.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <mutex>
#include <vector>

#include "internal.h"

#pragma STDC FP_CONTRACT OFF

namespace ltx3drope {
namespace {

constexpr size_t kCacheMax = 16;

struct Cache {
    std::mutex mu;
    std::deque<ltx3drope_tables*> fifo;  // oldest first; each entry holds one reference
    int64_t hits = 0, misses = 0, evictions = 0;
};

Cache& cache() {
    static Cache* c = new Cache();  // never destroyed: handles may outlive static destruction order
    return *c;
}

std::atomic<int64_t> g_alive{0};

// Fill one axis: pair (p, i) -> (cos, sin) of p * base^(-2i/d), float64 then fp32.
void fill_axis(float* dst, int64_t length, int64_t dim, double base) {
    const int64_t half = dim / 2;
    std::vector<double> omega(static_cast<size_t>(half));
    for (int64_t i = 0; i < half; ++i) {
        const double expo = -(2.0 * static_cast<double>(i)) / static_cast<double>(dim);
        omega[static_cast<size_t>(i)] = std::pow(base, expo);
    }
    for (int64_t p = 0; p < length; ++p) {
        for (int64_t i = 0; i < half; ++i) {
            const double theta = static_cast<double>(p) * omega[static_cast<size_t>(i)];
            const double c = std::cos(theta);
            const double s = std::sin(theta);
            dst[2 * (p * half + i)] = static_cast<float>(c);
            dst[2 * (p * half + i) + 1] = static_cast<float>(s);
        }
    }
}

bool same_key(const ltx3drope_tables* t, int device, int64_t T, int64_t H, int64_t W, int64_t dt, int64_t dh,
              int64_t dw, double base, bool host) {
    return t->device == device && t->T == T && t->H == H && t->W == W && t->dim_t == dt && t->dim_h == dh &&
           t->dim_w == dw && std::memcmp(&t->base, &base, sizeof(double)) == 0 && t->host == host;
}

void destroy(ltx3drope_tables* t) {
    if (t->packed != nullptr) {
        if (t->host) {
            std::free(t->packed);
        } else {
            int prev = 0;
            const bool have_prev = hipGetDevice(&prev) == hipSuccess;
            (void)hipSetDevice(t->device);
            (void)hipFree(t->packed);
            if (have_prev) (void)hipSetDevice(prev);
        }
    }
    delete t;
    g_alive.fetch_sub(1);
}

void unref(ltx3drope_tables* t) {
    if (t->refs.fetch_sub(1) == 1) destroy(t);
}

// Build a new table set (not yet in the cache).  Returns a status code.
int build_new(int device, int64_t T, int64_t H, int64_t W, int64_t dt, int64_t dh, int64_t dw, double base,
              bool host, hipStream_t stream, ltx3drope_tables** out) {
    const int64_t pairs = T * (dt / 2) + H * (dh / 2) + W * (dw / 2);
    std::vector<float> staging;
    try {
        staging.resize(static_cast<size_t>(2 * pairs));
    } catch (...) {
        return LTX3DROPE_E_NOMEM;
    }
    fill_axis(staging.data(), T, dt, base);
    fill_axis(staging.data() + 2 * T * (dt / 2), H, dh, base);
    fill_axis(staging.data() + 2 * (T * (dt / 2) + H * (dh / 2)), W, dw, base);

    auto* t = new (std::nothrow) ltx3drope_tables();
    if (t == nullptr) return LTX3DROPE_E_NOMEM;
    t->device = device;
    t->T = T;
    t->H = H;
    t->W = W;
    t->dim_t = dt;
    t->dim_h = dh;
    t->dim_w = dw;
    t->base = base;
    t->host = host;
    t->pairs = pairs;
    const size_t bytes = static_cast<size_t>(2 * pairs) * sizeof(float);
    g_alive.fetch_add(1);
    if (host) {
        t->packed = static_cast<float*>(std::malloc(bytes));
        if (t->packed == nullptr) {
            destroy(t);
            return LTX3DROPE_E_NOMEM;
        }
        std::memcpy(t->packed, staging.data(), bytes);
    } else {
        int prev = 0;
        if (hipGetDevice(&prev) != hipSuccess) {
            destroy(t);
            return LTX3DROPE_E_HIP;
        }
        int status = LTX3DROPE_OK;
        if (hipSetDevice(device) != hipSuccess) {
            status = LTX3DROPE_E_HIP;
        } else {
            void* mem = nullptr;
            const hipError_t e = hipMalloc(&mem, bytes);
            if (e == hipErrorOutOfMemory) {
                status = LTX3DROPE_E_NOMEM;
            } else if (e != hipSuccess) {
                status = LTX3DROPE_E_HIP;
            } else {
                t->packed = static_cast<float*>(mem);
                if (hipMemcpyAsync(mem, staging.data(), bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
                    hipStreamSynchronize(stream) != hipSuccess) {
                    status = LTX3DROPE_E_HIP;
                }
            }
        }
        (void)hipSetDevice(prev);
        if (status != LTX3DROPE_OK) {
            (void)hipGetLastError();
            destroy(t);
            return status;
        }
    }
    *out = t;
    return LTX3DROPE_OK;
}

}  // namespace

int tables_build(int device, int64_t T, int64_t H, int64_t W, int64_t dt, int64_t dh, int64_t dw, double base,
                 hipStream_t stream, ltx3drope_tables_t* out) {
    if (out == nullptr) return LTX3DROPE_E_INVALID;
    *out = nullptr;
    if (device < 0 || T <= 0 || H <= 0 || W <= 0) return LTX3DROPE_E_INVALID;
    if (dt <= 0 || dh <= 0 || dw <= 0 || (dt % 2) != 0 || (dh % 2) != 0 || (dw % 2) != 0) return LTX3DROPE_E_INVALID;
    if (!std::isfinite(base) || base <= 0.0) return LTX3DROPE_E_INVALID;
    // keep every table index and the packed size comfortably inside 32 bits
    const int64_t limit = int64_t(1) << 26;
    if (T > limit || H > limit || W > limit || dt > 65536 || dh > 65536 || dw > 65536) return LTX3DROPE_E_INVALID;
    if (T * (dt / 2) + H * (dh / 2) + W * (dw / 2) > limit) return LTX3DROPE_E_INVALID;
    const bool host = option(LTX3DROPE_OPT_HOST_TABLES) != 0;

    Cache& c = cache();
    {
        std::lock_guard<std::mutex> lock(c.mu);
        for (ltx3drope_tables* t : c.fifo) {
            if (same_key(t, device, T, H, W, dt, dh, dw, base, host)) {
                ++c.hits;
                t->refs.fetch_add(1);
                *out = t;
                return LTX3DROPE_OK;
            }
        }
    }
    // Miss: build outside the lock (host math + upload), then insert unless another
    // thread inserted the same key meanwhile.
    ltx3drope_tables* fresh = nullptr;
    const int status = build_new(device, T, H, W, dt, dh, dw, base, host, stream, &fresh);
    if (status != LTX3DROPE_OK) return status;

    ltx3drope_tables* evicted = nullptr;
    ltx3drope_tables* result = fresh;
    {
        std::lock_guard<std::mutex> lock(c.mu);
        ++c.misses;
        for (ltx3drope_tables* t : c.fifo) {
            if (same_key(t, device, T, H, W, dt, dh, dw, base, host)) {
                result = t;
                break;
            }
        }
        if (result == fresh) {
            if (c.fifo.size() >= kCacheMax) {
                evicted = c.fifo.front();
                c.fifo.pop_front();
                ++c.evictions;
            }
            fresh->refs.fetch_add(1);  // the cache's reference
            c.fifo.push_back(fresh);
        } else {
            result->refs.fetch_add(1);
        }
    }
    if (result != fresh) unref(fresh);
    if (evicted != nullptr) unref(evicted);
    *out = result;
    return LTX3DROPE_OK;
}

int tables_release(ltx3drope_tables_t t) {
    if (t == nullptr) return LTX3DROPE_E_INVALID;
    unref(t);
    return LTX3DROPE_OK;
}

int cache_clear() {
    std::deque<ltx3drope_tables*> drop;
    {
        std::lock_guard<std::mutex> lock(cache().mu);
        drop.swap(cache().fifo);
    }
    for (ltx3drope_tables* t : drop) unref(t);
    return LTX3DROPE_OK;
}

void cache_counters(int64_t* hits, int64_t* misses, int64_t* evictions, int64_t* live, int64_t* alive) {
    std::lock_guard<std::mutex> lock(cache().mu);
    *hits = cache().hits;
    *misses = cache().misses;
    *evictions = cache().evictions;
    *live = static_cast<int64_t>(cache().fifo.size());
    *alive = g_alive.load();
}

void cache_counters_reset() {
    std::lock_guard<std::mutex> lock(cache().mu);
    cache().hits = cache().misses = cache().evictions = 0;
}

}  // namespace ltx3drope
