// C ABI of the ltx3drope library: precheck, bit-exact gate, dispatch, options,
// statistics.
//
// Precheck: sglang PR #35698 page, "Key source snippets", the JIT wrapper's
// can_use predicate (6-D shapes, dtype, same device, positive sizes, head_dim
// equal to the split sum, even positive chunk widths, contiguity, pointer
// alignment, per-axis table shapes and device).  Contiguity is implied by the
// C ABI (plain pointers to contiguous tensors); this library adds the overlap,
// index-width and allocation-extent rules.
//
// Gate: same page, "Implementation breakdown", step 4: the first time a
// configuration is seen, the fast result is compared bit for bit with the
// reference path; equal -> trusted from then on, unequal -> that configuration
// permanently falls back to the reference path.  Here the reference path is
// the plain HIP kernel and the comparison runs on the device.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "internal.h"

namespace ltx3drope {
namespace {

// ---- options ---------------------------------------------------------------

struct Options {
    std::atomic<int64_t> path{0};
    std::atomic<int64_t> gate{1};
    std::atomic<int64_t> force_mismatch{0};
    std::atomic<int64_t> host_tables{0};
    std::atomic<int64_t> log{0};
    Options() {
        if (const char* s = std::getenv("LTX3DROPE_PATH")) {
            if (!std::strcmp(s, "fast")) path = 1;
            if (!std::strcmp(s, "plain")) path = 2;
        }
        if (const char* s = std::getenv("LTX3DROPE_GATE")) {
            if (!std::strcmp(s, "off")) gate = 0;
            if (!std::strcmp(s, "always")) gate = 2;
        }
        if (const char* s = std::getenv("LTX3DROPE_LOG")) log = std::atoi(s) != 0;
    }
};

Options& opts() {
    static Options* o = new Options();
    return *o;
}

// ---- statistics ------------------------------------------------------------

struct Stats {
    std::atomic<int64_t> verifications{0}, trusted{0}, disabled{0}, fast{0}, plain{0}, rejected{0};
};

Stats& stats() {
    static Stats* s = new Stats();
    return *s;
}

// ---- gate ------------------------------------------------------------------

// (device, dtype, B, T, H, W, heads, head_dim, dim_t, dim_h, dim_w, the tables' T, H, W, and the
// tensor's t, h, w offsets in them): a shard placement is a configuration of its own.
using GateKey = std::tuple<int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                           int64_t, int64_t, int64_t, int64_t, int64_t, int64_t>;

struct Gate {
    std::mutex mu;
    std::map<GateKey, int> state;
};

Gate& gate() {
    static Gate* g = new Gate();
    return *g;
}

int gate_get(const GateKey& key) {
    std::lock_guard<std::mutex> lock(gate().mu);
    auto it = gate().state.find(key);
    return it == gate().state.end() ? LTX3DROPE_GATE_UNSEEN : it->second;
}

void gate_set(const GateKey& key, int s) {
    std::lock_guard<std::mutex> lock(gate().mu);
    gate().state[key] = s;
}

// ---- per-device resources ---------------------------------------------------

struct DeviceRes {
    unsigned* counter = nullptr;  // [0]: mismatches of the gate's verification, [1]: out-of-cache positions
    int cu_count = 0;
    std::mutex verify_mu;  // one gate verification at a time per device: they share counter[0]
};

std::mutex g_dev_mu;
std::map<int, DeviceRes> g_dev;

int device_res(int device, DeviceRes** out) {
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DeviceRes& r = g_dev[device];
    if (r.counter == nullptr) {
        void* mem = nullptr;
        const hipError_t e = hipMalloc(&mem, 256);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return e == hipErrorOutOfMemory ? LTX3DROPE_E_NOMEM : LTX3DROPE_E_HIP;
        }
        // both counters start at zero (cleared by a kernel, then waited for once)
        if (launch_zero_u32(static_cast<unsigned*>(mem), nullptr) != hipSuccess ||
            launch_zero_u32(static_cast<unsigned*>(mem) + 1, nullptr) != hipSuccess ||
            hipStreamSynchronize(nullptr) != hipSuccess) {
            (void)hipGetLastError();
            (void)hipFree(mem);
            return LTX3DROPE_E_HIP;
        }
        r.counter = static_cast<unsigned*>(mem);
        if (hipDeviceGetAttribute(&r.cu_count, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
            (void)hipGetLastError();
            r.cu_count = 256;
        }
    }
    *out = &r;
    return LTX3DROPE_OK;
}

// ---- precheck --------------------------------------------------------------

bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bn && b0 < a0 + an;
}

// Is p device memory of `device` inside an allocation that holds [p, p + bytes)?
// Returns NOT_DEVICE_PTR, TABLE_DEVICE (memory of another device), EXTENT or OK.
int check_device_ptr(const void* p, size_t bytes, int device) {
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return LTX3DROPE_REASON_NOT_DEVICE_PTR;
    }
    if (attr.type != hipMemoryTypeDevice) return LTX3DROPE_REASON_NOT_DEVICE_PTR;
    if (attr.device != device) return LTX3DROPE_REASON_TABLE_DEVICE;
    void* base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();
        return LTX3DROPE_REASON_NOT_DEVICE_PTR;
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    if (q < b || q + bytes > b + size) return LTX3DROPE_REASON_EXTENT;
    return LTX3DROPE_REASON_OK;
}

// Where the tensor sits in the tables' grid.  exact_grid: the unsharded rule of
// the page's predicate (the tables' grid equals the tensor's); otherwise the
// tensor may be any slab [offset, offset + size) of the tables' grid.
struct Placement {
    int64_t t0 = 0, h0 = 0, w0 = 0;
    bool inplace = false;
    bool exact_grid = true;
};

// Reads a shard descriptor; false if it is malformed.
bool placement_from(const ltx3drope_shard_t* shard, Placement* out) {
    *out = Placement();
    out->exact_grid = false;
    if (shard == nullptr) return true;
    if (shard->reserved != 0 || (shard->inplace != 0 && shard->inplace != 1)) return false;
    if (shard->t_offset < 0 || shard->h_offset < 0 || shard->w_offset < 0) return false;
    out->t0 = shard->t_offset;
    out->h0 = shard->h_offset;
    out->w0 = shard->w_offset;
    out->inplace = shard->inplace == 1;
    return true;
}

// The precheck.  With check_outputs false, q_out and k_out are ignored (the caller
// will allocate fresh outputs, which cannot overlap anything).
int precheck(const void* q_out, const void* k_out, const void* q, const void* k, int dtype, int64_t B, int64_t T,
             int64_t H, int64_t W, int64_t heads, int64_t D, const ltx3drope_tables* tab, bool check_memory,
             bool check_outputs, const Placement& pl) {
    if ((check_outputs && (!q_out || !k_out)) || !q || !k || !tab) return LTX3DROPE_REASON_NULLPTR;
    if (dtype != LTX3DROPE_DTYPE_F32 && dtype != LTX3DROPE_DTYPE_BF16) return LTX3DROPE_REASON_DTYPE;
    if (B <= 0 || T <= 0 || H <= 0 || W <= 0 || heads <= 0 || D <= 0) return LTX3DROPE_REASON_NONPOSITIVE_DIM;
    if (tab->dim_t <= 0 || tab->dim_h <= 0 || tab->dim_w <= 0 || tab->dim_t % 2 || tab->dim_h % 2 || tab->dim_w % 2)
        return LTX3DROPE_REASON_SPLIT_ODD;
    if (D != tab->dim_t + tab->dim_h + tab->dim_w) return LTX3DROPE_REASON_SPLIT_SUM;
    if (pl.exact_grid) {
        if (tab->T != T || tab->H != H || tab->W != W) return LTX3DROPE_REASON_TABLE_GRID;
    } else {
        if (pl.t0 < 0 || pl.h0 < 0 || pl.w0 < 0 || pl.t0 > tab->T - T || pl.h0 > tab->H - H || pl.w0 > tab->W - W)
            return LTX3DROPE_REASON_TABLE_GRID;
    }
    const size_t es = dtype == LTX3DROPE_DTYPE_F32 ? 4 : 2;
    const uintptr_t pair = 2 * es;
    const void* ptrs[4] = {q, k, q_out, k_out};
    const int nptr = check_outputs ? 4 : 2;
    for (int i = 0; i < nptr; ++i)
        if (reinterpret_cast<uintptr_t>(ptrs[i]) % pair) return LTX3DROPE_REASON_ALIGN;
    // Index width: fewer than 2^32 elements per batch element, so the kernels' 32-bit indices hold
    // every pair (< 2^31) and every 16-byte vector (< 2^30) of a launch; a tensor of 2^32 elements
    // or more runs as several launches of whole batch elements (apply_impl).  Each size < 2^31,
    // the products checked before they can overflow; at most 2^48 elements in all.
    const int64_t lim = int64_t(1) << 32;
    int64_t per_batch = 1;
    for (int64_t f : {T, H, W, heads, D}) {
        if (f >= (int64_t(1) << 31) || per_batch > lim / f) return LTX3DROPE_REASON_TOO_LARGE;
        per_batch *= f;
    }
    if (per_batch >= lim || B >= (int64_t(1) << 31) || B > (int64_t(1) << 48) / per_batch)
        return LTX3DROPE_REASON_TOO_LARGE;
    const size_t bytes = static_cast<size_t>(B * per_batch) * es;
    if (check_outputs) {
        // every output/input and output/output overlap is refused, except exact in-place aliasing
        const bool q_inplace = pl.inplace && q_out == q;
        const bool k_inplace = pl.inplace && k_out == k;
        if ((!q_inplace && ranges_overlap(q_out, bytes, q, bytes)) || ranges_overlap(q_out, bytes, k, bytes) ||
            ranges_overlap(k_out, bytes, q, bytes) || (!k_inplace && ranges_overlap(k_out, bytes, k, bytes)) ||
            ranges_overlap(q_out, bytes, k_out, bytes))
            return LTX3DROPE_REASON_OVERLAP;
    }
    if (check_memory && !tab->host) {
        for (int i = 0; i < nptr; ++i) {
            const int r = check_device_ptr(ptrs[i], bytes, tab->device);
            if (r != LTX3DROPE_REASON_OK) return r;
        }
    }
    return LTX3DROPE_REASON_OK;
}

Problem make_problem(void* q_out, void* k_out, const void* q, const void* k, int dtype, int64_t B, int64_t T,
                     int64_t H, int64_t W, int64_t heads, int64_t D, const ltx3drope_tables* tab,
                     const Placement& pl) {
    Problem p;
    p.q_out = q_out;
    p.k_out = k_out;
    p.q = q;
    p.k = k;
    p.tab = tab->packed;
    p.dtype = dtype;
    p.B = static_cast<uint32_t>(B);
    p.T = static_cast<uint32_t>(T);
    p.H = static_cast<uint32_t>(H);
    p.W = static_cast<uint32_t>(W);
    p.heads = static_cast<uint32_t>(heads);
    p.D = static_cast<uint32_t>(D);
    p.PT = static_cast<uint32_t>(tab->dim_t / 2);
    p.PH = static_cast<uint32_t>(tab->dim_h / 2);
    p.PW = static_cast<uint32_t>(tab->dim_w / 2);
    p.tab_pairs = static_cast<uint32_t>(tab->pairs);
    p.tabT = static_cast<uint32_t>(tab->T);
    p.tabH = static_cast<uint32_t>(tab->H);
    p.t_off = static_cast<uint32_t>(pl.t0);
    p.h_off = static_cast<uint32_t>(pl.h0);
    p.w_off = static_cast<uint32_t>(pl.w0);
    return p;
}

int status_for_reason(int reason) {
    if (reason == LTX3DROPE_REASON_TABLE_GRID || reason == LTX3DROPE_REASON_TABLE_DEVICE)
        return LTX3DROPE_E_TABLE_MISMATCH;
    return LTX3DROPE_E_UNSUPPORTED;
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int device) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != device) (void)hipSetDevice(device);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// Batch elements per launch: all of them when the tensor holds fewer than 2^32 elements, else as
// many whole batch elements as stay below 2^32 (the precheck keeps one below it).
uint32_t batch_per_launch(const Problem& p) {
    const uint64_t per_batch = uint64_t(p.T) * p.H * p.W * p.heads * p.D;
    const uint64_t fit = ((uint64_t(1) << 32) - 1) / per_batch;
    return static_cast<uint32_t>(fit >= p.B ? p.B : fit);
}

// The part of a problem made of batch elements [b0, b0 + count).
Problem batch_slice(const Problem& p, uint32_t b0, uint32_t count) {
    const size_t es = p.dtype == LTX3DROPE_DTYPE_F32 ? 4 : 2;
    const size_t off = size_t(b0) * p.T * p.H * p.W * p.heads * p.D * es;
    Problem c = p;
    c.B = count;
    c.q = static_cast<const char*>(p.q) + off;
    c.k = static_cast<const char*>(p.k) + off;
    c.q_out = static_cast<char*>(p.q_out) + off;
    c.k_out = static_cast<char*>(p.k_out) + off;
    return c;
}

int run_kernel(Kernel which, const Problem& p, hipStream_t stream, int device) {
    const uint32_t step = batch_per_launch(p);
    for (uint32_t b0 = 0; b0 < p.B; b0 += step) {
        const Problem c = batch_slice(p, b0, p.B - b0 < step ? p.B - b0 : step);
        const hipError_t e = which == Kernel::Fast ? launch_fast(c, stream, device) : launch_plain(c, stream, device);
        if (e != hipSuccess || hipGetLastError() != hipSuccess) return LTX3DROPE_E_HIP;
        (which == Kernel::Fast ? stats().fast : stats().plain).fetch_add(1);
    }
    return LTX3DROPE_OK;
}

hipError_t run_verify(const Problem& p, unsigned* counter, hipStream_t stream, int device) {
    const uint32_t step = batch_per_launch(p);
    for (uint32_t b0 = 0; b0 < p.B; b0 += step) {
        const hipError_t e =
            launch_verify(batch_slice(p, b0, p.B - b0 < step ? p.B - b0 : step), counter, stream, device);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Verifications of the no-allocation entry point, one at a time per device: they share that
// device's static scratch counter.
std::mutex g_noalloc_verify_mu[kMaxDevices];

// Fast kernel into the outputs, then the plain kernel re-derives every pair on the
// device and counts disagreements.  Returns a status; *equal receives the verdict.
// The counter is the device's allocated counter block, or (noalloc) the library's
// static device scratch; either way one verification at a time per device uses it,
// from its clearing to its read-back.
int verify_fast(const Problem& p, hipStream_t stream, int device, bool noalloc, bool* equal) {
    unsigned* counter = nullptr;
    std::mutex* mu = nullptr;
    if (noalloc) {
        if (device < 0 || device >= kMaxDevices) return LTX3DROPE_E_INVALID;
        if (scratch_counter(device, &counter) != hipSuccess) {
            (void)hipGetLastError();
            return LTX3DROPE_E_HIP;
        }
        mu = &g_noalloc_verify_mu[device];
    } else {
        DeviceRes* res = nullptr;
        const int st = device_res(device, &res);
        if (st != LTX3DROPE_OK) return st;
        counter = res->counter;
        mu = &res->verify_mu;
    }
    std::lock_guard<std::mutex> lock(*mu);
    int st = run_kernel(Kernel::Fast, p, stream, device);
    if (st != LTX3DROPE_OK) return st;
    if (launch_zero_u32(counter, stream) != hipSuccess) return LTX3DROPE_E_HIP;
    if (run_verify(p, counter, stream, device) != hipSuccess || hipGetLastError() != hipSuccess)
        return LTX3DROPE_E_HIP;
    unsigned host_count = 0;
    if (hipMemcpyAsync(&host_count, counter, sizeof(unsigned), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        return LTX3DROPE_E_HIP;
    }
    stats().verifications.fetch_add(1);
    if (opts().force_mismatch.load() != 0 && host_count == 0) host_count = 1;
    *equal = host_count == 0;
    if (opts().log.load() != 0)
        std::fprintf(stderr, "[ltx3drope] gate: fast kernel %s the plain kernel (%u differing pairs)\n",
                     *equal ? "matches" : "DIFFERS from", host_count);
    return LTX3DROPE_OK;
}

}  // namespace

int64_t option(int which) {
    switch (which) {
        case LTX3DROPE_OPT_PATH: return opts().path.load();
        case LTX3DROPE_OPT_GATE: return opts().gate.load();
        case LTX3DROPE_OPT_FORCE_GATE_MISMATCH: return opts().force_mismatch.load();
        case LTX3DROPE_OPT_HOST_TABLES: return opts().host_tables.load();
        case LTX3DROPE_OPT_LOG: return opts().log.load();
        default: return LTX3DROPE_E_INVALID;
    }
}

}  // namespace ltx3drope

namespace ltx3drope {
namespace {

int apply_impl(void* q_out, void* k_out, const void* q, const void* k, int dtype, int64_t B, int64_t T, int64_t H,
               int64_t W, int64_t heads, int64_t head_dim, ltx3drope_tables_t tables, void* stream_ptr,
               const Placement& pl, bool noalloc) {
    if (tables != nullptr && tables->host) {
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_UNSUPPORTED;
    }
    const int r = precheck(q_out, k_out, q, k, dtype, B, T, H, W, heads, head_dim, tables, true, true, pl);
    if (r != LTX3DROPE_REASON_OK) {
        stats().rejected.fetch_add(1);
        return status_for_reason(r);
    }
    const Problem p = make_problem(q_out, k_out, q, k, dtype, B, T, H, W, heads, head_dim, tables, pl);
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    const int device = tables->device;
    DeviceGuard guard(device);

    const int64_t path = opts().path.load();
    if (path == 2 || !fast_supported(p)) return run_kernel(Kernel::Plain, p, stream, device);
    if (path == 1) return run_kernel(Kernel::Fast, p, stream, device);

    const int64_t gate_mode = opts().gate.load();
    if (gate_mode == 0) return run_kernel(Kernel::Fast, p, stream, device);
    const GateKey key{device, dtype, B, T, H, W, heads, head_dim, tables->dim_t, tables->dim_h, tables->dim_w,
                      tables->T, tables->H, tables->W, pl.t0, pl.h0, pl.w0};
    const int state = gate_get(key);
    if (state == LTX3DROPE_GATE_DISABLED) return run_kernel(Kernel::Plain, p, stream, device);
    const bool inplace = q_out == q || k_out == k;
    if (inplace) {
        // the inputs are overwritten, so this call cannot be verified: trust only an earlier verdict
        return run_kernel(state == LTX3DROPE_GATE_TRUSTED && gate_mode == 1 ? Kernel::Fast : Kernel::Plain, p, stream,
                          device);
    }
    if (state == LTX3DROPE_GATE_TRUSTED && gate_mode == 1) return run_kernel(Kernel::Fast, p, stream, device);
    // The verification waits for its count on the host, which a stream under graph capture cannot
    // do: such a call runs the plain kernel and leaves the configuration unverified.
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &capture) != hipSuccess) {
        (void)hipGetLastError();
        capture = hipStreamCaptureStatusNone;
    }
    if (capture != hipStreamCaptureStatusNone) return run_kernel(Kernel::Plain, p, stream, device);

    bool equal = false;
    const int st = verify_fast(p, stream, device, noalloc, &equal);
    if (st != LTX3DROPE_OK) return st;
    if (equal) {
        if (state != LTX3DROPE_GATE_TRUSTED) stats().trusted.fetch_add(1);
        gate_set(key, LTX3DROPE_GATE_TRUSTED);
        return LTX3DROPE_OK;
    }
    stats().disabled.fetch_add(1);
    gate_set(key, LTX3DROPE_GATE_DISABLED);
    std::fprintf(stderr,
                 "[ltx3drope] fast kernel differs from the plain kernel for dtype=%d B=%lld T=%lld H=%lld W=%lld "
                 "heads=%lld D=%lld; this configuration now uses the plain kernel\n",
                 dtype, static_cast<long long>(B), static_cast<long long>(T), static_cast<long long>(H),
                 static_cast<long long>(W), static_cast<long long>(heads), static_cast<long long>(head_dim));
    return run_kernel(Kernel::Plain, p, stream, device);  // overwrite with the reference result
}

// ---- rotate-half RoPE with a gathered cache -------------------------------

// With check_outputs false, q_out and k_out are ignored (fresh outputs, which cannot overlap anything).
int neox_precheck(const void* q_out, const void* k_out, const void* q, const void* k, int dtype, int64_t tokens,
                  int64_t q_heads, int64_t k_heads, int64_t D, const int64_t* positions, const void* cache,
                  int cache_dtype, int64_t max_position, bool check_memory, bool check_outputs, int* device_out) {
    if (tokens == 0) {
        // nothing to rotate: the sizes and dtypes must still be valid, no pointer is looked at
        // (an empty tensor may have a null data pointer)
        for (int d : {dtype, cache_dtype})
            if (d != LTX3DROPE_DTYPE_F32 && d != LTX3DROPE_DTYPE_BF16) return LTX3DROPE_REASON_DTYPE;
        if (q_heads <= 0 || k_heads <= 0 || D <= 0 || max_position <= 0) return LTX3DROPE_REASON_NONPOSITIVE_DIM;
        if (D % 2) return LTX3DROPE_REASON_SPLIT_ODD;
        if (q_heads >= (int64_t(1) << 31) || k_heads >= (int64_t(1) << 31) || D >= (int64_t(1) << 31) ||
            max_position >= (int64_t(1) << 31) || max_position * D >= (int64_t(1) << 32))
            return LTX3DROPE_REASON_TOO_LARGE;
        return LTX3DROPE_REASON_OK;
    }
    if ((check_outputs && (!q_out || !k_out)) || !q || !k || !positions || !cache) return LTX3DROPE_REASON_NULLPTR;
    for (int d : {dtype, cache_dtype})
        if (d != LTX3DROPE_DTYPE_F32 && d != LTX3DROPE_DTYPE_BF16) return LTX3DROPE_REASON_DTYPE;
    if (tokens <= 0 || q_heads <= 0 || k_heads <= 0 || D <= 0 || max_position <= 0)
        return LTX3DROPE_REASON_NONPOSITIVE_DIM;
    if (D % 2) return LTX3DROPE_REASON_SPLIT_ODD;
    const size_t es = dtype == LTX3DROPE_DTYPE_F32 ? 4 : 2;
    const size_t cs = cache_dtype == LTX3DROPE_DTYPE_F32 ? 4 : 2;
    for (const void* p : {q_out, k_out, q, k})
        if (reinterpret_cast<uintptr_t>(p) % es) return LTX3DROPE_REASON_ALIGN;  // NULL outputs pass
    if (reinterpret_cast<uintptr_t>(cache) % cs || reinterpret_cast<uintptr_t>(positions) % 8)
        return LTX3DROPE_REASON_ALIGN;
    // fewer than 2^32 elements per tensor (and per cache), each size below 2^31
    const int64_t lim = int64_t(1) << 32, size_lim = int64_t(1) << 31;
    auto product_ok = [&](std::initializer_list<int64_t> fs) {
        int64_t n = 1;
        for (int64_t f : fs) {
            if (f >= size_lim || n > lim / f) return false;
            n *= f;
        }
        return n < lim;
    };
    if (!product_ok({tokens, q_heads, D}) || !product_ok({tokens, k_heads, D}) || !product_ok({max_position, D}))
        return LTX3DROPE_REASON_TOO_LARGE;
    const size_t qb = static_cast<size_t>(tokens * q_heads * D) * es;
    const size_t kb = static_cast<size_t>(tokens * k_heads * D) * es;
    const size_t pb = static_cast<size_t>(tokens) * 8;
    const size_t cb = static_cast<size_t>(max_position * D) * cs;
    // outputs: exact aliasing with their own input is allowed; nothing else may overlap an output
    if (check_outputs) {
        if ((q_out != q && ranges_overlap(q_out, qb, q, qb)) || ranges_overlap(q_out, qb, k, kb) ||
            ranges_overlap(k_out, kb, q, qb) || (k_out != k && ranges_overlap(k_out, kb, k, kb)) ||
            ranges_overlap(q_out, qb, k_out, kb))
            return LTX3DROPE_REASON_OVERLAP;
        for (const void* o : {q_out, k_out}) {
            const size_t ob = o == q_out ? qb : kb;
            if (ranges_overlap(o, ob, positions, pb) || ranges_overlap(o, ob, cache, cb))
                return LTX3DROPE_REASON_OVERLAP;
        }
    }
    if (check_memory) {
        hipPointerAttribute_t a;
        std::memset(&a, 0, sizeof(a));
        if (hipPointerGetAttributes(&a, q) != hipSuccess) {
            (void)hipGetLastError();
            return LTX3DROPE_REASON_NOT_DEVICE_PTR;
        }
        if (a.type != hipMemoryTypeDevice) return LTX3DROPE_REASON_NOT_DEVICE_PTR;
        const int device = a.device;
        const std::pair<const void*, size_t> spans[6] = {{q, qb}, {k, kb}, {q_out, qb}, {k_out, kb},
                                                         {positions, pb}, {cache, cb}};
        for (int i = 0; i < 6; ++i) {
            if (!check_outputs && (i == 2 || i == 3)) continue;  // the outputs
            const int r = check_device_ptr(spans[i].first, spans[i].second, device);
            if (r != LTX3DROPE_REASON_OK) return r;
        }
        if (device_out) *device_out = device;
    }
    return LTX3DROPE_REASON_OK;
}

}  // namespace
}  // namespace ltx3drope

using namespace ltx3drope;

extern "C" {

int ltx3drope_tables_build(int device, int64_t T, int64_t H, int64_t W, int64_t dim_t, int64_t dim_h, int64_t dim_w,
                           double base, void* stream, ltx3drope_tables_t* out) {
    return tables_build(device, T, H, W, dim_t, dim_h, dim_w, base, static_cast<hipStream_t>(stream), out);
}

int ltx3drope_tables_release(ltx3drope_tables_t tables) { return tables_release(tables); }

int ltx3drope_tables_describe(ltx3drope_tables_t t, ltx3drope_tables_desc* out) {
    if (t == nullptr || out == nullptr) return LTX3DROPE_E_INVALID;
    out->device = t->device;
    out->T = t->T;
    out->H = t->H;
    out->W = t->W;
    out->dim_t = t->dim_t;
    out->dim_h = t->dim_h;
    out->dim_w = t->dim_w;
    out->base = t->base;
    out->packed = t->packed;
    out->packed_pairs = t->pairs;
    return LTX3DROPE_OK;
}

int ltx3drope_tables_read(ltx3drope_tables_t t, float* cos_t, float* sin_t, float* cos_h, float* sin_h, float* cos_w,
                          float* sin_w) {
    if (t == nullptr) return LTX3DROPE_E_INVALID;
    const size_t n = static_cast<size_t>(2 * t->pairs);
    float* host = static_cast<float*>(std::malloc(n * sizeof(float)));
    if (host == nullptr) return LTX3DROPE_E_NOMEM;
    if (t->host) {
        std::memcpy(host, t->packed, n * sizeof(float));
    } else {
        DeviceGuard guard(t->device);
        if (hipMemcpy(host, t->packed, n * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess) {
            (void)hipGetLastError();
            std::free(host);
            return LTX3DROPE_E_HIP;
        }
    }
    const int64_t sections[3][2] = {{t->T, t->dim_t / 2}, {t->H, t->dim_h / 2}, {t->W, t->dim_w / 2}};
    float* outs[3][2] = {{cos_t, sin_t}, {cos_h, sin_h}, {cos_w, sin_w}};
    size_t off = 0;
    for (int a = 0; a < 3; ++a) {
        const int64_t cnt = sections[a][0] * sections[a][1];
        for (int64_t i = 0; i < cnt; ++i) {
            if (outs[a][0]) outs[a][0][i] = host[off + 2 * i];
            if (outs[a][1]) outs[a][1][i] = host[off + 2 * i + 1];
        }
        off += static_cast<size_t>(2 * cnt);
    }
    std::free(host);
    return LTX3DROPE_OK;
}

int ltx3drope_cache_clear(void) { return cache_clear(); }

int ltx3drope_can_use(const void* q_out, const void* k_out, const void* q, const void* k, int dtype, int64_t B,
                      int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim, ltx3drope_tables_t tables,
                      int* reason) {
    const bool outputs = q_out != nullptr || k_out != nullptr;
    const int r = precheck(q_out, k_out, q, k, dtype, B, T, H, W, heads, head_dim, tables, true, outputs, Placement());
    if (reason) *reason = r;
    return r == LTX3DROPE_REASON_OK ? 1 : 0;
}

int ltx3drope_can_use_shard(const void* q_out, const void* k_out, const void* q, const void* k, int dtype, int64_t B,
                            int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim,
                            const ltx3drope_shard_t* shard, ltx3drope_tables_t tables, int* reason) {
    Placement pl;
    int r = LTX3DROPE_REASON_TABLE_GRID;
    if (placement_from(shard, &pl)) {
        const bool outputs = q_out != nullptr || k_out != nullptr;
        r = precheck(q_out, k_out, q, k, dtype, B, T, H, W, heads, head_dim, tables, true, outputs, pl);
    }
    if (reason) *reason = r;
    return r == LTX3DROPE_REASON_OK ? 1 : 0;
}

int ltx3drope_kernel_choice(const void* q_out, const void* k_out, const void* q, const void* k, int dtype, int64_t B,
                            int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim,
                            ltx3drope_tables_t tables) {
    const bool outputs = q_out != nullptr || k_out != nullptr;
    const int r = precheck(q_out, k_out, q, k, dtype, B, T, H, W, heads, head_dim, tables, false, outputs, Placement());
    if (r != LTX3DROPE_REASON_OK) return status_for_reason(r);
    const Problem p = make_problem(const_cast<void*>(q_out), const_cast<void*>(k_out), q, k, dtype, B, T, H, W, heads,
                                   head_dim, tables, Placement());
    return fast_supported(p) ? static_cast<int>(Kernel::Fast) : static_cast<int>(Kernel::Plain);
}

int ltx3drope_apply_qk(void* q_out, void* k_out, const void* q, const void* k, int dtype, int64_t B, int64_t T,
                       int64_t H, int64_t W, int64_t heads, int64_t head_dim, ltx3drope_tables_t tables,
                       void* stream_ptr) {
    return apply_impl(q_out, k_out, q, k, dtype, B, T, H, W, heads, head_dim, tables, stream_ptr, Placement(), false);
}

int ltx3drope_apply_qk_noalloc(void* q_out, void* k_out, const void* q, const void* k, int dtype, int64_t B,
                               int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim,
                               ltx3drope_tables_t tables, void* stream_ptr) {
    if (tables != nullptr && (tables->device < 0 || tables->device >= kMaxDevices)) {
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_UNSUPPORTED;
    }
    return apply_impl(q_out, k_out, q, k, dtype, B, T, H, W, heads, head_dim, tables, stream_ptr, Placement(), true);
}

int ltx3drope_apply_qk_shard(void* q_out, void* k_out, const void* q, const void* k, int dtype, int64_t B, int64_t T,
                             int64_t H, int64_t W, int64_t heads, int64_t head_dim, const ltx3drope_shard_t* shard,
                             ltx3drope_tables_t tables, void* stream_ptr) {
    Placement pl;
    if (!placement_from(shard, &pl)) {
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_TABLE_MISMATCH;
    }
    return apply_impl(q_out, k_out, q, k, dtype, B, T, H, W, heads, head_dim, tables, stream_ptr, pl, false);
}

int ltx3drope_neox_can_use(const void* q_out, const void* k_out, const void* q, const void* k, int dtype,
                           int64_t tokens, int64_t q_heads, int64_t k_heads, int64_t head_dim,
                           const int64_t* positions, const void* cache, int cache_dtype, int64_t max_position,
                           int* reason) {
    const bool outputs = q_out != nullptr || k_out != nullptr;
    const int r = neox_precheck(q_out, k_out, q, k, dtype, tokens, q_heads, k_heads, head_dim, positions, cache,
                                cache_dtype, max_position, true, outputs, nullptr);
    if (reason) *reason = r;
    return r == LTX3DROPE_REASON_OK ? 1 : 0;
}

int ltx3drope_neox_apply_qk(void* q_out, void* k_out, const void* q, const void* k, int dtype, int64_t tokens,
                            int64_t q_heads, int64_t k_heads, int64_t head_dim, const int64_t* positions,
                            const void* cache, int cache_dtype, int64_t max_position, void* stream_ptr) {
    int device = -1;
    const int r = neox_precheck(q_out, k_out, q, k, dtype, tokens, q_heads, k_heads, head_dim, positions, cache,
                                cache_dtype, max_position, true, true, &device);
    if (r != LTX3DROPE_REASON_OK) {
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_UNSUPPORTED;
    }
    if (tokens == 0) return LTX3DROPE_OK;  // nothing launched
    DeviceGuard guard(device);
    DeviceRes* res = nullptr;
    const int st = device_res(device, &res);
    if (st != LTX3DROPE_OK) return st;
    NeoxProblem p;
    p.q_out = q_out;
    p.k_out = k_out;
    p.q = q;
    p.k = k;
    p.positions = positions;
    p.cache = cache;
    p.dtype = dtype;
    p.cache_dtype = cache_dtype;
    p.tokens = static_cast<uint32_t>(tokens);
    p.q_heads = static_cast<uint32_t>(q_heads);
    p.k_heads = static_cast<uint32_t>(k_heads);
    p.D = static_cast<uint32_t>(head_dim);
    p.max_position = static_cast<uint32_t>(max_position > 0xffffffffll ? 0xffffffffll : max_position);
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    const bool fast = opts().path.load() != 2 && neox_fast_supported(p);
    const hipError_t e = fast ? launch_neox_fast(p, res->counter + 1, stream)
                              : launch_neox_plain(p, res->counter + 1, stream, res->cu_count);
    if (e != hipSuccess || hipGetLastError() != hipSuccess) return LTX3DROPE_E_HIP;
    (fast ? stats().fast : stats().plain).fetch_add(1);
    return LTX3DROPE_OK;
}

int ltx3drope_neox_position_errors(int device, int reset, int64_t* count) {
    if (count == nullptr || device < 0) return LTX3DROPE_E_INVALID;
    DeviceGuard guard(device);
    DeviceRes* res = nullptr;
    const int st = device_res(device, &res);
    if (st != LTX3DROPE_OK) return st;
    unsigned host = 0;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(&host, res->counter + 1, sizeof(unsigned), hipMemcpyDeviceToHost) != hipSuccess) {
        (void)hipGetLastError();
        return LTX3DROPE_E_HIP;
    }
    *count = host;
    if (reset) {
        if (launch_zero_u32(res->counter + 1, nullptr) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
            (void)hipGetLastError();
            return LTX3DROPE_E_HIP;
        }
    }
    return LTX3DROPE_OK;
}

}  // extern "C"

namespace ltx3drope {
namespace {

int patch_call(void* dst, const void* src, int elem_bytes, int64_t B, int64_t C, int64_t F, int64_t H, int64_t W,
               int64_t p, void* stream_ptr, bool inverse) {
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return LTX3DROPE_E_INVALID;
    if (B < 0 || C < 0 || F < 0 || H < 0 || W < 0 || p <= 0 || H % p || W % p) return LTX3DROPE_E_INVALID;
    // an empty tensor: nothing to move, no pointer is looked at (it may be null)
    if (B == 0 || C == 0 || F == 0 || H == 0 || W == 0) return LTX3DROPE_OK;
    if (!dst || !src) return LTX3DROPE_E_INVALID;
    // fewer than 2^32 elements (the LDS kernels index 16-byte vectors with 32 bits), each size and
    // the packed channel count C*p*p below 2^31
    const int64_t lim = int64_t(1) << 32, size_lim = int64_t(1) << 31;
    int64_t numel = 1;
    for (int64_t f : {B, C, F, H, W}) {
        if (f >= size_lim || numel > lim / f) {
            stats().rejected.fetch_add(1);
            return LTX3DROPE_E_UNSUPPORTED;
        }
        numel *= f;
    }
    if (numel >= lim || p >= size_lim || p * p > size_lim / C) {
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_UNSUPPORTED;
    }
    const size_t bytes = static_cast<size_t>(numel) * static_cast<size_t>(elem_bytes);
    if (reinterpret_cast<uintptr_t>(dst) % elem_bytes || reinterpret_cast<uintptr_t>(src) % elem_bytes ||
        ranges_overlap(dst, bytes, src, bytes)) {
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_UNSUPPORTED;
    }
    hipPointerAttribute_t a;
    std::memset(&a, 0, sizeof(a));
    if (hipPointerGetAttributes(&a, src) != hipSuccess || a.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_UNSUPPORTED;
    }
    const int device = a.device;
    if (check_device_ptr(src, bytes, device) != LTX3DROPE_REASON_OK ||
        check_device_ptr(dst, bytes, device) != LTX3DROPE_REASON_OK) {
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_UNSUPPORTED;
    }
    DeviceGuard guard(device);
    DeviceRes* res = nullptr;
    const int st = device_res(device, &res);
    if (st != LTX3DROPE_OK) return st;
    PatchProblem pp;
    pp.src = src;
    pp.dst = dst;
    pp.elem_bytes = static_cast<uint32_t>(elem_bytes);
    pp.B = static_cast<uint32_t>(B);
    pp.C = static_cast<uint32_t>(C);
    pp.F = static_cast<uint32_t>(F);
    pp.H = static_cast<uint32_t>(H);
    pp.W = static_cast<uint32_t>(W);
    pp.p = static_cast<uint32_t>(p);
    pp.force_plain = opts().path.load() == 2;
    const bool fast = !pp.force_plain && patch_fast_supported(pp);
    if (launch_patch(pp, inverse, static_cast<hipStream_t>(stream_ptr), res->cu_count) != hipSuccess ||
        hipGetLastError() != hipSuccess)
        return LTX3DROPE_E_HIP;
    (fast ? stats().fast : stats().plain).fetch_add(1);
    return LTX3DROPE_OK;
}

}  // namespace
}  // namespace ltx3drope

extern "C" {

int ltx3drope_patchify(void* y, const void* x, int elem_bytes, int64_t B, int64_t C, int64_t F, int64_t H, int64_t W,
                       int64_t p, void* stream) {
    return patch_call(y, x, elem_bytes, B, C, F, H, W, p, stream, false);
}

int ltx3drope_unpatchify(void* x, const void* y, int elem_bytes, int64_t B, int64_t C, int64_t F, int64_t H,
                         int64_t W, int64_t p, void* stream) {
    return patch_call(x, y, elem_bytes, B, C, F, H, W, p, stream, true);
}

int ltx3drope_dit_freq_grid(double theta, int64_t dim, int64_t num_rope_elems, int double_precision, float* out,
                            void* stream, int64_t* count) {
    // theta must be a normal float32 (the float32 recipe rounds it to one; a smaller or larger
    // base would leave the power's domain this library covers)
    if (!std::isfinite(theta) || theta < 0x1p-126 || theta > 0x1.fffffep+127 || dim < 0 || num_rope_elems <= 0)
        return LTX3DROPE_E_INVALID;
    const int64_t n = dim / num_rope_elems;
    if (n > (int64_t(1) << 24)) return LTX3DROPE_E_INVALID;
    if (count != nullptr) *count = n;
    if (n == 0) return LTX3DROPE_OK;
    if (out == nullptr) return LTX3DROPE_E_INVALID;
    hipPointerAttribute_t a;
    std::memset(&a, 0, sizeof(a));
    if (hipPointerGetAttributes(&a, out) != hipSuccess || a.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_UNSUPPORTED;
    }
    if (check_device_ptr(out, static_cast<size_t>(n) * sizeof(float), a.device) != LTX3DROPE_REASON_OK) {
        stats().rejected.fetch_add(1);
        return LTX3DROPE_E_UNSUPPORTED;
    }
    DeviceGuard guard(a.device);
    if (launch_dit_freqs(out, static_cast<uint32_t>(n), theta, double_precision != 0, static_cast<hipStream_t>(stream)) !=
            hipSuccess ||
        hipGetLastError() != hipSuccess)
        return LTX3DROPE_E_HIP;
    stats().fast.fetch_add(1);
    return LTX3DROPE_OK;
}

int ltx3drope_gate_state(int device, int dtype, int64_t B, int64_t T, int64_t H, int64_t W, int64_t heads,
                         int64_t head_dim, int64_t dim_t, int64_t dim_h, int64_t dim_w) {
    // the unsharded configuration: tables built for the tensor's own grid, no offsets
    return gate_get(GateKey{device, dtype, B, T, H, W, heads, head_dim, dim_t, dim_h, dim_w, T, H, W, 0, 0, 0});
}

int ltx3drope_gate_reset(void) {
    std::lock_guard<std::mutex> lock(gate().mu);
    gate().state.clear();
    return LTX3DROPE_OK;
}

int ltx3drope_set_option(int option, int64_t value) {
    switch (option) {
        case LTX3DROPE_OPT_PATH:
            if (value < 0 || value > 2) return LTX3DROPE_E_INVALID;
            opts().path = value;
            return LTX3DROPE_OK;
        case LTX3DROPE_OPT_GATE:
            if (value < 0 || value > 2) return LTX3DROPE_E_INVALID;
            opts().gate = value;
            return LTX3DROPE_OK;
        case LTX3DROPE_OPT_FORCE_GATE_MISMATCH: opts().force_mismatch = value != 0; return LTX3DROPE_OK;
        case LTX3DROPE_OPT_HOST_TABLES: opts().host_tables = value != 0; return LTX3DROPE_OK;
        case LTX3DROPE_OPT_LOG: opts().log = value != 0; return LTX3DROPE_OK;
        default: return LTX3DROPE_E_INVALID;
    }
}

int64_t ltx3drope_get_option(int which) { return option(which); }

int ltx3drope_stats(ltx3drope_stats_t* out) {
    if (out == nullptr) return LTX3DROPE_E_INVALID;
    cache_counters(&out->cache_hits, &out->cache_misses, &out->cache_evictions, &out->cache_live, &out->tables_alive);
    out->gate_verifications = stats().verifications.load();
    out->gate_trusted = stats().trusted.load();
    out->gate_disabled = stats().disabled.load();
    out->fast_launches = stats().fast.load();
    out->plain_launches = stats().plain.load();
    out->rejected = stats().rejected.load();
    return LTX3DROPE_OK;
}

int ltx3drope_stats_reset(void) {
    cache_counters_reset();
    stats().verifications = 0;
    stats().trusted = 0;
    stats().disabled = 0;
    stats().fast = 0;
    stats().plain = 0;
    stats().rejected = 0;
    return LTX3DROPE_OK;
}

int ltx3drope_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    if (dst == nullptr || src == nullptr || bytes < 0 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(dst) % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
        return LTX3DROPE_E_INVALID;
    if (ranges_overlap(dst, static_cast<size_t>(bytes), src, static_cast<size_t>(bytes))) return LTX3DROPE_E_INVALID;
    if (bytes / 16 >= (int64_t(1) << 32) - 64) return LTX3DROPE_E_INVALID;
    int device = -1;
    for (const void* p : {static_cast<const void*>(dst), src}) {
        hipPointerAttribute_t a;
        std::memset(&a, 0, sizeof(a));
        if (hipPointerGetAttributes(&a, p) != hipSuccess || a.type != hipMemoryTypeDevice) {
            (void)hipGetLastError();
            return LTX3DROPE_E_INVALID;
        }
        if (device >= 0 && a.device != device) return LTX3DROPE_E_INVALID;  // both on one device
        device = a.device;
        void* base = nullptr;
        size_t size = 0;
        if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
            (void)hipGetLastError();
            return LTX3DROPE_E_INVALID;
        }
        if (reinterpret_cast<uintptr_t>(p) + static_cast<uintptr_t>(bytes) >
            reinterpret_cast<uintptr_t>(base) + size)
            return LTX3DROPE_E_INVALID;
    }
    if (bytes == 0) return LTX3DROPE_OK;
    DeviceGuard guard(device);
    if (launch_copy(dst, src, bytes, static_cast<hipStream_t>(stream), device) != hipSuccess ||
        hipGetLastError() != hipSuccess)
        return LTX3DROPE_E_HIP;
    return LTX3DROPE_OK;
}

const char* ltx3drope_status_string(int status) {
    switch (status) {
        case LTX3DROPE_OK: return "ok";
        case LTX3DROPE_E_INVALID: return "invalid argument";
        case LTX3DROPE_E_UNSUPPORTED: return "unsupported input (precheck failed, nothing launched)";
        case LTX3DROPE_E_TABLE_MISMATCH: return "tables do not match the tensors' grid or device";
        case LTX3DROPE_E_HIP: return "HIP runtime error";
        case LTX3DROPE_E_NOMEM: return "out of memory";
        default: return "unknown status";
    }
}

const char* ltx3drope_reason_string(int reason) {
    switch (reason) {
        case LTX3DROPE_REASON_OK: return "ok";
        case LTX3DROPE_REASON_NULLPTR: return "null pointer or table handle";
        case LTX3DROPE_REASON_DTYPE: return "dtype must be F32 or BF16";
        case LTX3DROPE_REASON_NONPOSITIVE_DIM: return "every size must be positive";
        case LTX3DROPE_REASON_SPLIT_ODD: return "each rope_dim_split entry must be even and positive";
        case LTX3DROPE_REASON_SPLIT_SUM: return "head_dim must equal dim_t + dim_h + dim_w";
        case LTX3DROPE_REASON_TABLE_GRID: return "tables were built for another (T, H, W) grid";
        case LTX3DROPE_REASON_TABLE_DEVICE: return "tables live on another device";
        case LTX3DROPE_REASON_ALIGN: return "pointers must be aligned to one (even, odd) pair";
        case LTX3DROPE_REASON_OVERLAP: return "outputs must not overlap the inputs or each other";
        case LTX3DROPE_REASON_TOO_LARGE: return "a batch element must have fewer than 2^32 elements";
        case LTX3DROPE_REASON_NOT_DEVICE_PTR: return "pointer is not device memory";
        case LTX3DROPE_REASON_HOST_MODE: return "host-table test mode: nothing is launched";
        case LTX3DROPE_REASON_EXTENT: return "a device allocation ends before the tensor does";
        default: return "unknown reason";
    }
}

int ltx3drope_version(void) { return LTX3DROPE_VERSION; }

}  // extern "C"
