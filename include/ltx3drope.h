/*
 * ltx3drope.h - fused 3D rotary position embedding (RoPE) of the LTX-2.5
 * diffusion video decoder, for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one described on the sglang PR #35698 page
 * ("fused LTX-2.5 decoder 3D RoPE", prhub.com.cn): sections "Implementation
 * breakdown" (steps 1-4) and "Key source snippets" (the JIT wrapper and the
 * CUDA kernel).  Every decoder attention block rotates its Q and K over the
 * latent (T, H, W) token grid with per-axis cos/sin tables that all blocks
 * on one grid share.
 *
 * Tensor layout (all four tensors): contiguous [B, T, H, W, heads, head_dim]
 * of one dtype; token n = (t*H + h)*W + w inside each batch element.  The
 * head dimension is cut into a t chunk of dim_t channels, an h chunk of
 * dim_h channels and a w chunk of dim_w channels, in that order
 * (head_dim == dim_t + dim_h + dim_w, each even and > 0).  Inside a chunk the
 * channels form interleaved pairs (x[2j], x[2j+1]).
 *
 * Tables: for an axis of length L and width d, entry (p, i), p in [0, L),
 * i in [0, d/2), holds cos and sin of p * base^(-2i/d), evaluated in float64
 * on the host and rounded once to fp32.  (The page names the builder but not
 * its formula; this is the textbook inverse-frequency reading with integer,
 * tile-local positions, since the cache key has no offset.)
 *
 * Rotation of one pair (e, o) with (c, s) from the token's table row, every
 * operation an fp32 IEEE round-to-nearest-even step and no fused
 * multiply-add ("Key source snippets", the kernel's pair-rotation helper):
 *     e' = (e*c) - (o*s),   o' = (e*s) + (o*c)
 * then cast back to the tensor dtype (bf16: round to nearest, ties to even;
 * fp32: identity).  Q and K use the same (c, s).  ltx3drope_apply_qk writes
 * out of place and never modifies its inputs; the shard entry point can also
 * rotate in place (see ltx3drope_shard_t).
 *
 * All functions are thread-safe, never throw, and return a status code
 * (LTX3DROPE_OK == 0, negative on error) unless stated otherwise.  Pointers
 * named q, k, q_out, k_out are device pointers owned by the caller.  Table
 * handles are owned by the library and reference counted.  A "stream" is a
 * hipStream_t passed as void* (NULL = the device's null stream).
 */
#ifndef LTX3DROPE_H
#define LTX3DROPE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LTX3DROPE_VERSION 1

/* ---- status codes ------------------------------------------------------ */
enum {
    LTX3DROPE_OK = 0,
    LTX3DROPE_E_INVALID = -1,        /* an argument is malformed (null handle, bad size, bad base) */
    LTX3DROPE_E_UNSUPPORTED = -2,    /* the precheck rejects the tensors; nothing was launched */
    LTX3DROPE_E_TABLE_MISMATCH = -3, /* the tables do not belong to this grid / split / device */
    LTX3DROPE_E_HIP = -4,            /* a HIP runtime call failed */
    LTX3DROPE_E_NOMEM = -5           /* a host or device allocation failed */
};

/* ---- element types ----------------------------------------------------- */
enum { LTX3DROPE_DTYPE_F32 = 0, LTX3DROPE_DTYPE_BF16 = 1 };

/* ---- precheck reason codes (ltx3drope_can_use) ------------------------- */
enum {
    LTX3DROPE_REASON_OK = 0,
    LTX3DROPE_REASON_NULLPTR = 1,        /* a tensor pointer or the table handle is NULL */
    LTX3DROPE_REASON_DTYPE = 2,          /* dtype is neither F32 nor BF16 */
    LTX3DROPE_REASON_NONPOSITIVE_DIM = 3,/* B, T, H, W, heads or head_dim <= 0 */
    LTX3DROPE_REASON_SPLIT_ODD = 4,      /* a table chunk width is odd or <= 0 (tables carry the split) */
    LTX3DROPE_REASON_SPLIT_SUM = 5,      /* head_dim != dim_t + dim_h + dim_w */
    LTX3DROPE_REASON_TABLE_GRID = 6,     /* the tables were built for another (T, H, W) */
    LTX3DROPE_REASON_TABLE_DEVICE = 7,   /* the tables live on another device than the tensors */
    LTX3DROPE_REASON_ALIGN = 8,          /* a pointer is not aligned to one pair (2 elements) */
    LTX3DROPE_REASON_OVERLAP = 9,        /* an output overlaps an input or the other output */
    LTX3DROPE_REASON_TOO_LARGE = 10,     /* a batch element of 2^32 elements or more, a size of 2^31 or more,
                                            or more than 2^48 elements in all */
    LTX3DROPE_REASON_NOT_DEVICE_PTR = 11,/* a pointer is not device memory of the tables' device */
    LTX3DROPE_REASON_HOST_MODE = 12,     /* host-table test mode: apply calls refused, nothing launched (a name
                                            for that refusal; the precheck itself never returns it) */
    LTX3DROPE_REASON_EXTENT = 13         /* a pointer's device allocation ends before the tensor does */
};

/* ---- options (ltx3drope_set_option / ltx3drope_get_option) ------------- */
enum {
    LTX3DROPE_OPT_PATH = 1,        /* 0 auto (gate decides), 1 force fast kernel, 2 force plain kernel */
    LTX3DROPE_OPT_GATE = 2,        /* 0 off (trust fast), 1 verify the first call per key (default), 2 verify every call */
    LTX3DROPE_OPT_FORCE_GATE_MISMATCH = 3, /* 1: every verification reports a mismatch (tests the fallback) */
    LTX3DROPE_OPT_HOST_TABLES = 4, /* 1: tables are built in host memory and nothing touches HIP (CPU tests of the
                                      cache and the precheck); can_use still reports the precheck's verdict
                                      (memory checks skipped), and every apply call with such tables returns
                                      E_UNSUPPORTED without launching */
    LTX3DROPE_OPT_LOG = 5          /* 1: one stderr line per gate decision */
};

/* ---- gate states (ltx3drope_gate_state) -------------------------------- */
enum { LTX3DROPE_GATE_UNSEEN = 0, LTX3DROPE_GATE_TRUSTED = 1, LTX3DROPE_GATE_DISABLED = 2 };

typedef struct ltx3drope_tables* ltx3drope_tables_t;

typedef struct {
    int device;
    int64_t T, H, W;
    int64_t dim_t, dim_h, dim_w;
    double base;
    /* device (or, in host-table mode, host) address of the packed tables: float pairs (cos, sin),
       t section [T][dim_t/2], then h section [H][dim_h/2], then w section [W][dim_w/2] */
    const void* packed;
    int64_t packed_pairs;
} ltx3drope_tables_desc;

typedef struct {
    int64_t cache_hits, cache_misses, cache_evictions, cache_live;
    int64_t tables_alive;               /* table objects not yet freed (cache- or caller-held) */
    int64_t gate_verifications, gate_trusted, gate_disabled;
    int64_t fast_launches, plain_launches;
    int64_t rejected;                   /* apply_qk calls refused by the precheck */
} ltx3drope_stats_t;

/*
 * ltx3drope_tables_build - find or build the per-axis tables of one grid.
 *
 * The page's cached table lookup ("Implementation breakdown", step 1): the key
 * is (device, T, H, W, dim_t, dim_h, dim_w, base); a hit returns the cached
 * tables; a miss builds them (float64 on the host, rounded once to fp32),
 * uploads them with hipMemcpyAsync on `stream` followed by a synchronization of
 * that stream, and inserts them.  The cache holds at most 16 entries and
 * evicts first-in first-out (a hit does not refresh an entry).
 *
 * On success *out receives a handle holding one reference for the caller;
 * release it with ltx3drope_tables_release.  Eviction only drops the cache's
 * own reference, so a handle held by a caller stays valid after eviction.
 * Errors: E_INVALID (null out, T/H/W <= 0, a dim odd or <= 0, base not finite
 * or <= 0, device < 0), E_NOMEM, E_HIP.
 */
int ltx3drope_tables_build(int device, int64_t T, int64_t H, int64_t W,
                           int64_t dim_t, int64_t dim_h, int64_t dim_w, double base,
                           void* stream, ltx3drope_tables_t* out);

/* Drop one reference; the table memory is freed when the last one goes (hipFree waits for the
   device's outstanding work).  E_INVALID on NULL. */
int ltx3drope_tables_release(ltx3drope_tables_t tables);

/* Describe a table set (grid, split, base, device, packed address).  E_INVALID on NULL arguments. */
int ltx3drope_tables_describe(ltx3drope_tables_t tables, ltx3drope_tables_desc* out);

/* Copy the six tables to caller-owned host arrays of fp32, row-major [L][d/2] each (any pointer may
   be NULL to skip it).  Synchronous (device-wide copy).  E_INVALID, E_HIP. */
int ltx3drope_tables_read(ltx3drope_tables_t tables, float* cos_t, float* sin_t, float* cos_h,
                          float* sin_h, float* cos_w, float* sin_w);

/* Drop the cache's references to every entry (tables still held by callers stay valid). */
int ltx3drope_cache_clear(void);

/*
 * ltx3drope_can_use - the precheck ("Key source snippets", the JIT wrapper's
 * can_use predicate, plus rules of this library).
 *
 * Returns 1 if ltx3drope_apply_qk would launch for these arguments, 0 if it
 * would refuse.  q_out and k_out may both be NULL: then only the inputs are
 * checked (for a caller that allocates fresh outputs afterwards).  When
 * `reason` is not NULL it receives an LTX3DROPE_REASON_* code (the first
 * failing rule in the order of the enum).  Rules: no NULL
 * pointer or handle; dtype F32 or BF16; B, T, H, W, heads, head_dim > 0;
 * table split widths even and > 0 and summing to head_dim; tables built for
 * (T, H, W); every pointer aligned to one pair (8 B for F32, 4 B for BF16);
 * neither output overlapping an input or the other output; each size below
 * 2^31, fewer than 2^32 elements per batch element (8 GiB of bf16, 16 GiB of
 * fp32) and at most 2^48 in all (a tensor of 2^32 elements or more runs as
 * several launches of whole batch elements); all four pointers
 * device memory of the tables'
 * device, each inside an allocation large enough for the whole tensor
 * (checked last, REASON_NOT_DEVICE_PTR then REASON_EXTENT; skipped in
 * host-table mode).  Pure host logic: no launch, no allocation, no synchronization
 * (pointer attributes are queried from the HIP runtime).
 */
int ltx3drope_can_use(const void* q_out, const void* k_out, const void* q, const void* k, int dtype,
                      int64_t B, int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim,
                      ltx3drope_tables_t tables, int* reason);

/*
 * ltx3drope_apply_qk - rotate Q and K in one launch ("Key source snippets":
 * the wrapper writes fresh q_out and k_out with one kernel launch).
 *
 * q, k: inputs [B, T, H, W, heads, head_dim]; q_out, k_out: caller-allocated
 * outputs of the same shape and dtype (the caller allocates them fresh; they
 * must not overlap the inputs).  The precheck runs first; on failure nothing
 * is launched and E_UNSUPPORTED (or E_TABLE_MISMATCH for REASON_TABLE_GRID /
 * REASON_TABLE_DEVICE) is returned.  Otherwise the work is enqueued on
 * `stream` and the call returns without waiting, except on the first call of
 * a configuration while the bit-exact gate is on: then the fast kernel's
 * output is checked bit for bit against the plain kernel on the device and
 * the stream is synchronized once ("Implementation breakdown", step 4: first
 * call verified; equal -> the fast path is trusted, unequal -> permanent
 * fallback to the plain path for that configuration).  The gate's
 * configuration key is (device, dtype, B, T, H, W, heads, head_dim, dim_t,
 * dim_h, dim_w, the tables' T, H, W and the shard offsets): each shard
 * placement is verified on its own first call.  The comparison is of raw bits: both kernels write a NaN
 * result as the canonical quiet NaN (0x7FC00000 fp32, 0x7FC0 bf16).  On a
 * stream under graph capture an unverified configuration runs the plain
 * kernel and stays unverified (the check cannot wait for its count there).
 * The first verification on a device allocates that device's 256-byte
 * counter, kept until the process ends: E_NOMEM if the device is out of
 * memory, E_HIP for any other failed HIP call or launch.
 */
int ltx3drope_apply_qk(void* q_out, void* k_out, const void* q, const void* k, int dtype,
                       int64_t B, int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim,
                       ltx3drope_tables_t tables, void* stream);

/*
 * ltx3drope_apply_qk_noalloc - ltx3drope_apply_qk for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, precheck, kernels, gate and results as ltx3drope_apply_qk (the caller passes
 * the inputs and the outputs), but it calls no hipMalloc, hipFree or other allocating routine:
 * the gate's verification counts its mismatches in a static 256-byte device array of the
 * library (one copy per GPU, held until the process ends) instead of the counter block
 * ltx3drope_apply_qk allocates on a device's first verification.  The counter is cleared by a
 * kernel before each use; its size does not depend on the input, so every input the precheck
 * accepts fits.  Every call on one GPU shares that array,
 * which keeps the last call's contents: verifications on one GPU are serialized by a host mutex
 * of the library from the counter's clearing to its read-back, and calls that overlap on one GPU
 * without it (from outside the library) would race.  The tables come from
 * ltx3drope_tables_build beforehand (which does allocate, once per grid).  E_UNSUPPORTED also for
 * tables of device index 64 or above.
 */
int ltx3drope_apply_qk_noalloc(void* q_out, void* k_out, const void* q, const void* k, int dtype,
                               int64_t B, int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim,
                               ltx3drope_tables_t tables, void* stream);

/*
 * Shards.  A sequence- or tile-parallel rank holds a slab of a larger token
 * grid; its tokens must take the table rows of their global coordinates.
 * (Positions on the page are tile-local because the table cache key carries
 * no offset: "Implementation breakdown", step 1.  The descriptor below is the
 * offset that splitting one grid over several devices needs.)
 *
 * t_offset, h_offset, w_offset: global frame / row / column of the tensor's
 * first frame / row / column.  The tables passed with a shard describe the
 * whole grid: for each axis offset + local size <= the tables' size, else
 * REASON_TABLE_GRID.  A token at local (t, h, w) is rotated with table rows
 * (t + t_offset, h + h_offset, w + w_offset).
 * inplace: 1 allows q_out == q and k_out == k exactly (partial overlaps stay
 * refused).  In-place calls cannot be checked by the bit-exact gate (the
 * inputs are overwritten); they use the fast kernel only once the
 * configuration is TRUSTED (or the gate is off, or the fast path is forced),
 * and the plain kernel otherwise.  A NULL descriptor means zero offsets,
 * out of place.
 */
typedef struct {
    int64_t t_offset, h_offset, w_offset;
    int32_t inplace;
    int32_t reserved;  /* must be 0 */
} ltx3drope_shard_t;

/* The precheck of a shard call: as ltx3drope_can_use, with the grid rule replaced by the shard's
   containment rule and the in-place exception to the overlap rule.  A malformed descriptor (a
   negative offset, an inplace value other than 0 or 1, or a non-zero reserved field) fails with
   REASON_TABLE_GRID before any other rule is looked at. */
int ltx3drope_can_use_shard(const void* q_out, const void* k_out, const void* q, const void* k, int dtype,
                            int64_t B, int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim,
                            const ltx3drope_shard_t* shard, ltx3drope_tables_t tables, int* reason);

/* ltx3drope_apply_qk on a shard of the tables' grid (see above); B, T, H, W are the tensor's local
   sizes.  Same statuses as ltx3drope_apply_qk; the gate key is the same as for an unsharded call of
   the same local shape (offsets do not change which code runs). */
int ltx3drope_apply_qk_shard(void* q_out, void* k_out, const void* q, const void* k, int dtype,
                             int64_t B, int64_t T, int64_t H, int64_t W, int64_t heads, int64_t head_dim,
                             const ltx3drope_shard_t* shard, ltx3drope_tables_t tables, void* stream);

/*
 * Rotate-half ("NeoX") RoPE with a position-gathered cos/sin cache: the text
 * encoder's rotary (sglang PR #24660 page, "Key source snippets", the Gemma3
 * rotary application; "Implementation breakdown", step 2).
 *
 * q [tokens, q_heads, head_dim], k [tokens, k_heads, head_dim] (the head
 * counts may differ), contiguous, dtype F32 or BF16; positions [tokens] int64
 * device array; cache [max_position, head_dim] of cache_dtype (F32 or BF16)
 * holding cos in columns [0, head_dim/2) and sin in [head_dim/2, head_dim).
 * For i < head_dim/2 with (c, s) = the token's cache row at i, converted to
 * q's dtype:
 *     out[i]            = R( R(x[i] * c)            + R(-x[i + head_dim/2] * s) )
 *     out[i + head_dim/2] = R( R(x[i + head_dim/2] * c) + R(x[i] * s) )
 * where R rounds an fp32 result to q's dtype (bf16: nearest even).  The
 * outputs may alias their own input exactly (q_out == q, k_out == k); every
 * other overlap is refused.  A position outside [0, max_position) is never
 * read: that token's outputs are set to NaN and counted (see
 * ltx3drope_neox_position_errors).  One launch for Q and K, on `stream`.
 * Reasons: NULLPTR, DTYPE (q or cache dtype), NONPOSITIVE_DIM, SPLIT_ODD
 * (odd head_dim), ALIGN (element alignment; positions 8 B), OVERLAP,
 * TOO_LARGE (a tensor or the cache of 2^32 elements or more, or a size of
 * 2^31 or more), NOT_DEVICE_PTR,
 * TABLE_DEVICE (pointers on different devices), EXTENT.  can_use accepts
 * q_out and k_out both NULL (fresh outputs: only the inputs are checked);
 * apply_qk needs both.  tokens = 0 is an empty call: the other sizes and the
 * dtypes are checked, no pointer is looked at (an empty tensor's may be NULL),
 * can_use returns 1 and apply_qk returns OK without launching.  The rules are
 * checked in this order and the first that fails names the reason: with
 * tokens = 0, DTYPE, NONPOSITIVE_DIM (q_heads, k_heads, head_dim or
 * max_position <= 0), SPLIT_ODD, TOO_LARGE (a size of 2^31 or more, or a cache
 * of 2^32 elements or more); otherwise NULLPTR, DTYPE, NONPOSITIVE_DIM,
 * SPLIT_ODD, ALIGN (q_out, k_out, q, k to their element size, the cache to
 * its own, positions to 8 B), TOO_LARGE, OVERLAP (an output over an input
 * other than its own exactly, over the other output, the positions or the
 * cache), then the device-memory rules.  apply_qk returns
 * E_UNSUPPORTED for any of these; the first call on a device allocates the
 * device's 256-byte counter (E_NOMEM when out of memory, E_HIP for another
 * HIP failure), and a failed launch gives E_HIP.
 */
int ltx3drope_neox_can_use(const void* q_out, const void* k_out, const void* q, const void* k, int dtype,
                           int64_t tokens, int64_t q_heads, int64_t k_heads, int64_t head_dim,
                           const int64_t* positions, const void* cache, int cache_dtype, int64_t max_position,
                           int* reason);
int ltx3drope_neox_apply_qk(void* q_out, void* k_out, const void* q, const void* k, int dtype,
                            int64_t tokens, int64_t q_heads, int64_t k_heads, int64_t head_dim,
                            const int64_t* positions, const void* cache, int cache_dtype, int64_t max_position,
                            void* stream);
/* Number of (token, tensor) pairs whose position was outside the cache since the last reset, on
   `device`.  Synchronizes the device.  reset = 1 clears the count afterwards. */
int ltx3drope_neox_position_errors(int device, int reset, int64_t* count);

/*
 * Stage-5 space-to-depth of the diffusion decoder (sglang PR #34471 page,
 * "Key source snippets", _patchify) and its inverse (_unpatchify):
 *     x (B, C, F, H, W) <-> y (B, C*p*p, F, H/p, W/p)
 *     y[b, (c*p + pw)*p + ph, f, hh, ww] = x[b, c, f, hh*p + ph, ww*p + pw]
 * i.e. channels packed as (channel, width offset, height offset).  Both tensors
 * contiguous, elements of elem_bytes = 1, 2, 4 or 8 bytes (the op moves data
 * and never looks at values, so it is exact for every dtype).  B, C, F, H, W
 * are always the unpatched sizes.  A size of 0 is an empty call: OK, nothing
 * launched, no pointer looked at (an empty tensor's may be NULL).  E_INVALID:
 * a size < 0, p <= 0, H or W not a multiple of p, elem_bytes not 1/2/4/8,
 * NULL pointers of a non-empty call.  E_UNSUPPORTED: 2^32
 * elements or more (or C*p*p of 2^31 or more), pointers not aligned to one
 * element, overlapping tensors,
 * not device memory of one device, or allocations smaller than the tensors.
 * Asynchronous on `stream`.  E_NOMEM / E_HIP: the device's first call could not
 * allocate the library's 256-byte per-device counter block; E_HIP: a failed
 * launch.
 */
int ltx3drope_patchify(void* y, const void* x, int elem_bytes, int64_t B, int64_t C, int64_t F, int64_t H,
                       int64_t W, int64_t p, void* stream);
int ltx3drope_unpatchify(void* x, const void* y, int elem_bytes, int64_t B, int64_t C, int64_t F, int64_t H,
                         int64_t W, int64_t p, void* stream);

/*
 * LTX DiT RoPE frequency grid, generated on the device (sglang PR #24660 page,
 * "Key source snippets", the DiT's frequency generation; "Implementation
 * breakdown", step 2: generated on the target device in the requested
 * precision, keeping the official rounding trajectory):
 *     n = dim / num_rope_elems (integer division)
 *     out[i] = float32( theta ** linspace(0, 1, n)[i] * pi / 2 )
 * in float64 (double_precision = 1) or float32 (0), every step rounded to
 * nearest even in that precision: linspace as torch.linspace computes it (a
 * rounded step s = 1/(n-1); s*i for i < n/2, else 1 - s*(n-1-i) rounded once),
 * the correctly rounded power (theta first rounded to float32 in the float32
 * recipe), pi rounded to the working precision, an exact halving, and in the
 * float64 recipe one rounding to float32 at the end.
 * `out`: device memory of n floats (written by one kernel launch on `stream`,
 * asynchronous; its device is the current one).  *count (if not NULL) receives
 * n; n = 0 launches nothing and `out` may be NULL.
 * E_INVALID: theta not in [2^-126, FLT_MAX] (a normal float32), dim < 0,
 * num_rope_elems <= 0, n > 2^24, out NULL while n > 0.  E_UNSUPPORTED: `out`
 * is not device memory holding n floats.  E_HIP: the launch failed.
 */
int ltx3drope_dit_freq_grid(double theta, int64_t dim, int64_t num_rope_elems, int double_precision, float* out,
                            void* stream, int64_t* count);

/* Gate state of one unsharded configuration (tables built for the tensor's own grid, no offsets):
 * LTX3DROPE_GATE_*, or a negative status. */
int ltx3drope_gate_state(int device, int dtype, int64_t B, int64_t T, int64_t H, int64_t W,
                         int64_t heads, int64_t head_dim, int64_t dim_t, int64_t dim_h, int64_t dim_w);

/* Forget every gate decision (all configurations become UNSEEN). */
int ltx3drope_gate_reset(void);

int ltx3drope_set_option(int option, int64_t value);
int64_t ltx3drope_get_option(int option);

int ltx3drope_stats(ltx3drope_stats_t* out);
int ltx3drope_stats_reset(void);

/* Which kernel apply_qk would use for these arguments when the gate trusts the fast path:
   1 fast, 2 plain, or a negative status if the precheck fails (host rules only: device memory is
   not queried).  q_out and k_out may both be NULL: fresh outputs, which are 16-byte aligned. */
int ltx3drope_kernel_choice(const void* q_out, const void* k_out, const void* q, const void* k,
                            int dtype, int64_t B, int64_t T, int64_t H, int64_t W, int64_t heads,
                            int64_t head_dim, ltx3drope_tables_t tables);

/* Measurement helper: copy `bytes` (a multiple of 16, fewer than 2^32 - 64 vectors of 16 B, both
   pointers 16-B aligned, non-overlapping memory of one device) from src to dst with a plain streaming kernel
   on `stream` (the fast kernel's launch shape and cache hints, one read and one write stream); used
   as the bandwidth ceiling and to calibrate traffic counters.  E_INVALID on bad arguments, E_HIP. */
int ltx3drope_copy(void* dst, const void* src, int64_t bytes, void* stream);

const char* ltx3drope_status_string(int status);
const char* ltx3drope_reason_string(int reason);
int ltx3drope_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LTX3DROPE_H */
