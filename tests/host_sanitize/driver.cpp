// Sanitizer driver for the library's host code (cache, reference counts, precheck,
// options, statistics, the DiT frequency grid), run in host-table mode from several
// threads, then allocation-failure injection against an emulated device.  Exit status 0
// and no sanitizer report mean success.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "ltx3drope.h"

extern std::atomic<long> g_hip_calls;
extern std::atomic<int> g_emulate;
extern std::atomic<int> g_malloc_fail;
extern std::atomic<long> g_live_allocs;

#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            std::exit(1);                                                 \
        }                                                                 \
    } while (0)

namespace {

struct Key {
    int64_t T, H, W, dt, dh, dw;
    double base;
};

// 24 grid keys: more than the cache's 16 entries, so evictions happen while handles are held
std::vector<Key> keys() {
    std::vector<Key> k;
    for (int i = 0; i < 24; ++i)
        k.push_back({1 + i % 5, 2 + i % 7, 3 + i % 4, 8, 8 + 2 * (i % 3), 8, i % 2 ? 10000.0 : 500.0 + i});
    return k;
}

void worker(int id, int iters, std::atomic<int>* failures) {
    std::mt19937 rng(1234u + static_cast<unsigned>(id));
    const std::vector<Key> ks = keys();
    std::vector<ltx3drope_tables_t> held;
    std::vector<float> buf;
    for (int it = 0; it < iters; ++it) {
        const Key& k = ks[rng() % ks.size()];
        ltx3drope_tables_t t = nullptr;
        if (ltx3drope_tables_build(0, k.T, k.H, k.W, k.dt, k.dh, k.dw, k.base, nullptr, &t) != LTX3DROPE_OK ||
            t == nullptr) {
            failures->fetch_add(1);
            continue;
        }
        ltx3drope_tables_desc d;
        CHECK(ltx3drope_tables_describe(t, &d) == LTX3DROPE_OK);
        CHECK(d.T == k.T && d.H == k.H && d.W == k.W && d.dim_h == k.dh);
        // read every table back and check the identity row and the unit circle
        const size_t nt = static_cast<size_t>(k.T * k.dt / 2), nh = static_cast<size_t>(k.H * k.dh / 2),
                     nw = static_cast<size_t>(k.W * k.dw / 2);
        buf.assign(2 * (nt + nh + nw), -7.0f);
        float* ct = buf.data();
        float* st = ct + nt;
        float* ch = st + nt;
        float* sh = ch + nh;
        float* cw = sh + nh;
        float* sw = cw + nw;
        CHECK(ltx3drope_tables_read(t, ct, st, ch, sh, cw, sw) == LTX3DROPE_OK);
        CHECK(ct[0] == 1.0f && st[0] == 0.0f);
        for (size_t i = 0; i < nh; ++i) CHECK(std::fabs(ch[i] * ch[i] + sh[i] * sh[i] - 1.0f) < 1e-6f);
        // the precheck in host mode: a valid call, then refusals (no memory checks, no launch)
        const int64_t D = k.dt + k.dh + k.dw;
        alignas(16) static thread_local char fake[64];
        int reason = -1;
        const int ok = ltx3drope_can_use(nullptr, nullptr, fake, fake + 16, LTX3DROPE_DTYPE_BF16, 1, k.T, k.H, k.W,
                                         2, D, t, &reason);
        CHECK(ok == 1 && reason == LTX3DROPE_REASON_OK);
        CHECK(ltx3drope_can_use(nullptr, nullptr, fake, fake, LTX3DROPE_DTYPE_BF16, 1, k.T, k.H, k.W, 2, D + 2, t,
                                &reason) == 0 && reason == LTX3DROPE_REASON_SPLIT_SUM);
        CHECK(ltx3drope_can_use(nullptr, nullptr, fake + 2, fake, LTX3DROPE_DTYPE_F32, 1, k.T, k.H, k.W, 2, D, t,
                                &reason) == 0 && reason == LTX3DROPE_REASON_ALIGN);
        CHECK(ltx3drope_apply_qk(fake + 32, fake + 48, fake, fake + 16, LTX3DROPE_DTYPE_BF16, 1, k.T, k.H, k.W, 2, D,
                                 t, nullptr) == LTX3DROPE_E_UNSUPPORTED);
        // keep some handles across iterations (evicted entries must stay valid while held)
        held.push_back(t);
        if (held.size() > 6 || (rng() % 4) == 0) {
            const size_t j = rng() % held.size();
            CHECK(ltx3drope_tables_release(held[j]) == LTX3DROPE_OK);
            held.erase(held.begin() + static_cast<long>(j));
        }
        if (rng() % 97 == 0) CHECK(ltx3drope_cache_clear() == LTX3DROPE_OK);
        if (rng() % 13 == 0) {
            ltx3drope_stats_t s;
            CHECK(ltx3drope_stats(&s) == LTX3DROPE_OK);
            CHECK(s.cache_live >= 0 && s.cache_live <= 16 && s.tables_alive >= 0);
        }
        if (rng() % 17 == 0) {
            // the DiT grid's argument checks: an empty grid (dim < num_rope_elems) and refused
            // arguments return before any HIP call
            const int64_t ne = 1 + static_cast<int64_t>(rng() % 8);
            const int64_t dim = static_cast<int64_t>(rng() % static_cast<uint64_t>(ne));
            int64_t n = -1;
            CHECK(ltx3drope_dit_freq_grid(10000.0, dim, ne, static_cast<int>(rng() % 2), nullptr, nullptr, &n) ==
                  LTX3DROPE_OK);
            CHECK(n == 0);
            CHECK(ltx3drope_dit_freq_grid(-1.0, 64, ne, 1, nullptr, nullptr, &n) == LTX3DROPE_E_INVALID);
            CHECK(ltx3drope_dit_freq_grid(10000.0, 64, 2, 0, nullptr, nullptr, &n) == LTX3DROPE_E_INVALID);
        }
    }
    for (ltx3drope_tables_t t : held) CHECK(ltx3drope_tables_release(t) == LTX3DROPE_OK);
}

}  // namespace

int main(int argc, char** argv) {
    const int threads = argc > 1 ? std::atoi(argv[1]) : 8;
    const int iters = argc > 2 ? std::atoi(argv[2]) : 3000;
    CHECK(ltx3drope_set_option(LTX3DROPE_OPT_HOST_TABLES, 1) == LTX3DROPE_OK);
    CHECK(ltx3drope_stats_reset() == LTX3DROPE_OK);
    // argument errors
    ltx3drope_tables_t t = nullptr;
    CHECK(ltx3drope_tables_build(0, 0, 1, 1, 2, 2, 2, 10000.0, nullptr, &t) == LTX3DROPE_E_INVALID);
    CHECK(ltx3drope_tables_build(0, 1, 1, 1, 3, 2, 2, 10000.0, nullptr, &t) == LTX3DROPE_E_INVALID);
    CHECK(ltx3drope_tables_build(0, 1, 1, 1, 2, 2, 2, NAN, nullptr, &t) == LTX3DROPE_E_INVALID);
    CHECK(ltx3drope_tables_release(nullptr) == LTX3DROPE_E_INVALID);
    for (int s = -6; s <= 1; ++s) CHECK(ltx3drope_status_string(s) != nullptr);
    for (int r = -1; r <= 14; ++r) CHECK(ltx3drope_reason_string(r) != nullptr);

    std::atomic<int> failures{0};
    std::vector<std::thread> pool;
    for (int i = 0; i < threads; ++i) pool.emplace_back(worker, i, iters, &failures);
    for (std::thread& th : pool) th.join();
    CHECK(failures.load() == 0);

    CHECK(ltx3drope_cache_clear() == LTX3DROPE_OK);
    ltx3drope_stats_t s;
    CHECK(ltx3drope_stats(&s) == LTX3DROPE_OK);
    CHECK(s.cache_live == 0);
    CHECK(s.tables_alive == 0);  // every table freed once the cache and all holders let go
    CHECK(s.fast_launches == 0 && s.plain_launches == 0);
    CHECK(g_hip_calls.load() == 0);  // host-table mode never reaches HIP

    // Device mode against an emulated device 0, with hipMalloc failures injected: a failed table
    // upload or counter allocation returns E_NOMEM (out of memory) or E_HIP (any other error),
    // leaves nothing behind, and the next successful build is cached as usual.
    CHECK(ltx3drope_set_option(LTX3DROPE_OPT_HOST_TABLES, 0) == LTX3DROPE_OK);
    CHECK(ltx3drope_stats_reset() == LTX3DROPE_OK);
    g_emulate = 1;
    int64_t count = -1;
    g_malloc_fail = hipErrorOutOfMemory;
    t = reinterpret_cast<ltx3drope_tables_t>(&count);
    CHECK(ltx3drope_tables_build(0, 2, 3, 4, 8, 8, 8, 10000.0, nullptr, &t) == LTX3DROPE_E_NOMEM && t == nullptr);
    CHECK(ltx3drope_neox_position_errors(0, 0, &count) == LTX3DROPE_E_NOMEM && count == -1);
    g_malloc_fail = hipErrorInvalidValue;
    CHECK(ltx3drope_tables_build(0, 2, 3, 4, 8, 8, 8, 10000.0, nullptr, &t) == LTX3DROPE_E_HIP && t == nullptr);
    CHECK(ltx3drope_neox_position_errors(0, 0, &count) == LTX3DROPE_E_HIP && count == -1);
    CHECK(ltx3drope_stats(&s) == LTX3DROPE_OK);
    CHECK(s.tables_alive == 0 && s.cache_live == 0 && s.cache_misses == 0 && g_live_allocs.load() == 0);
    g_malloc_fail = 0;
    ltx3drope_tables_t t2 = nullptr;
    CHECK(ltx3drope_tables_build(0, 2, 3, 4, 8, 8, 8, 10000.0, nullptr, &t) == LTX3DROPE_OK && t != nullptr);
    CHECK(ltx3drope_tables_build(0, 2, 3, 4, 8, 8, 8, 10000.0, nullptr, &t2) == LTX3DROPE_OK && t2 == t);
    std::vector<float> c(4), sn(4);
    CHECK(ltx3drope_tables_read(t, c.data(), sn.data(), nullptr, nullptr, nullptr, nullptr) == LTX3DROPE_E_HIP);
    CHECK(ltx3drope_stats(&s) == LTX3DROPE_OK);
    CHECK(s.tables_alive == 1 && s.cache_live == 1 && s.cache_misses == 1 && s.cache_hits == 1);
    CHECK(g_live_allocs.load() == 1);
    CHECK(ltx3drope_tables_release(t) == LTX3DROPE_OK && ltx3drope_tables_release(t2) == LTX3DROPE_OK);
    CHECK(ltx3drope_cache_clear() == LTX3DROPE_OK);
    CHECK(ltx3drope_stats(&s) == LTX3DROPE_OK);
    CHECK(s.tables_alive == 0 && g_live_allocs.load() == 0);
    g_emulate = 0;

    std::printf("host sanitizer driver: %d threads x %d iterations, %lld hits, %lld misses, %lld evictions\n",
                threads, iters, static_cast<long long>(s.cache_hits), static_cast<long long>(s.cache_misses),
                static_cast<long long>(s.cache_evictions));
    return 0;
}
