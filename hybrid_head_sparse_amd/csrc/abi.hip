// C ABI of the hybrid-head decode-attention step: argument validation (pure
// host code), workspace carve-up, and the per-layer launch (one kernel: pooled
// attention over all heads with the retrieval heads' top-k fused in).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <string>

#include "../../include/lychee.h"
#include "common.hpp"
#include "correction.hpp"

using namespace lychee;

struct lychee_handle {
    lychee_dims dims;
    void* ws_base;
    size_t ws_bytes;
    Workspace ws;
    hipStream_t stream;
    int device;
    int cus;             // compute units of the device
    int per_cu;          // persistent workgroups per compute unit
    uint32_t cost_sparse; // pool cost of a gathered row
    hipEvent_t ev_start;
    hipEvent_t ev_stop;
    unsigned long long* trace;   // phase timestamps (LYCHEE_TRACE build), or null
    uint32_t trace_launch;
};

// Scratch of the allocation-free entry point (lychee_decode_layer_static):
// one copy per GPU, held until the process ends.  In host code the name is a
// host-side stand-in, never a device address: the device address comes from
// hipGetSymbolAddress, once per device (g_static below).
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Clears `words` 32-bit words (the workspace's zero region) with plain vector
// stores: a kernel rather than a memset node, so the call can be captured.
__global__ void __launch_bounds__(256) zero_fill_kernel(uint32_t* p, size_t words) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

namespace {

thread_local std::string g_last_error;

// Per-device state of the allocation-free entry point.  `zero_prefix`: bytes
// at the start of the device's scratch known to be zero once the work already
// enqueued completes (every call restores its zero region, which starts at
// offset 0; a call whose zero region is longer clears the difference first).
constexpr int kMaxDevices = 64;
struct StaticScratch {
    bool ready;
    void* ptr;
    size_t zero_prefix;
    int cus;
};
StaticScratch g_static[kMaxDevices];
std::mutex g_static_mutex;

lychee_status fail(lychee_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

lychee_status ok() {
    g_last_error.clear();
    return LYCHEE_OK;
}

lychee_status check_dims(const lychee_dims* d) {
    if (!d) return fail(LYCHEE_ERR_INVALID_ARG, "dims is NULL");
    if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 || d->max_ctx < 1 ||
        d->k_max < 1)
        return fail(LYCHEE_ERR_INVALID_ARG, "dims must be positive (batch=%d Hq=%d Hkv=%d d=%d max_ctx=%d k_max=%d)",
                    d->batch, d->n_q_heads, d->n_kv_heads, d->head_dim, d->max_ctx, d->k_max);
    if (d->n_q_heads % d->n_kv_heads != 0)
        return fail(LYCHEE_ERR_INVALID_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", d->n_q_heads,
                    d->n_kv_heads);
    if (d->dtype != LYCHEE_F32 && d->dtype != LYCHEE_BF16)
        return fail(LYCHEE_ERR_INVALID_ARG, "dtype %d is not LYCHEE_F32 or LYCHEE_BF16", d->dtype);
    const int G = d->n_q_heads / d->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(LYCHEE_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", G);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(LYCHEE_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
    if (d->n_kv_heads > kMaxKvHeads)
        return fail(LYCHEE_ERR_UNSUPPORTED, "n_kv_heads must be <= %d (got %d)", kMaxKvHeads, d->n_kv_heads);
    if ((long long)d->batch * d->n_kv_heads > kMaxBH)
        return fail(LYCHEE_ERR_UNSUPPORTED, "batch * n_kv_heads must be <= %d (got %lld)", kMaxBH,
                    (long long)d->batch * d->n_kv_heads);
    if (d->max_ctx > kMaxCtx)
        return fail(LYCHEE_ERR_UNSUPPORTED, "max_ctx must be <= %d (got %d)", kMaxCtx, d->max_ctx);
    if (d->k_max > d->max_ctx)
        return fail(LYCHEE_ERR_INVALID_ARG, "k_max (%d) must be <= max_ctx (%d)", d->k_max, d->max_ctx);
    return ok();
}

struct Range {
    uintptr_t lo, hi;
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range span(const void* p, size_t bytes) {
    const uintptr_t a = (uintptr_t)p;
    return Range{a, a + bytes};
}

size_t elem_bytes(const lychee_dims* d) { return d->dtype == LYCHEE_BF16 ? 2u : 4u; }

// Checks shared by the hybrid and dense entry points.
lychee_status check_common(const lychee_dims* d, const void* q, const void* kc, const void* vc, const float* out,
                           const int32_t* n_ctx) {
    lychee_status s = check_dims(d);
    if (s != LYCHEE_OK) return s;
    if (!q || !kc || !vc || !out || !n_ctx) return fail(LYCHEE_ERR_INVALID_ARG, "a tensor pointer is NULL");
    if (((uintptr_t)q | (uintptr_t)kc | (uintptr_t)vc) & 15u)
        return fail(LYCHEE_ERR_INVALID_ARG, "q, k_cache and v_cache must be 16-byte aligned");
    if (((uintptr_t)out | (uintptr_t)n_ctx) & 3u)
        return fail(LYCHEE_ERR_INVALID_ARG, "out and n_ctx must be 4-byte aligned");
    const size_t es = elem_bytes(d);
    const size_t nq = (size_t)d->batch * d->n_q_heads * d->head_dim;
    const size_t nkv = (size_t)d->batch * d->n_kv_heads * d->max_ctx * d->head_dim;
    const Range r_out = span(out, nq * 4);
    if (overlap(r_out, span(q, nq * es)) || overlap(r_out, span(kc, nkv * es)) || overlap(r_out, span(vc, nkv * es)) ||
        overlap(r_out, span(n_ctx, (size_t)d->batch * 4)))
        return fail(LYCHEE_ERR_INVALID_ARG, "out overlaps an input");
    return ok();
}

}  // namespace

extern "C" {

const char* lychee_status_str(lychee_status s) {
    switch (s) {
        case LYCHEE_OK: return "ok";
        case LYCHEE_ERR_INVALID_ARG: return "invalid argument";
        case LYCHEE_ERR_UNSUPPORTED: return "unsupported configuration";
        case LYCHEE_ERR_HIP: return "HIP runtime error";
        case LYCHEE_ERR_WORKSPACE: return "workspace too small or misaligned";
        case LYCHEE_ERR_DEVICE_CHECK: return "device-side contract violation";
    }
    return "unknown status";
}

const char* lychee_last_error(void) { return g_last_error.c_str(); }

size_t lychee_workspace_bytes(const lychee_dims* dims) {
    if (check_dims(dims) != LYCHEE_OK) return 0;
    return carve_workspace(nullptr, dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim, dims->max_ctx,
                           dims->k_max)
        .total_bytes;
}

lychee_status lychee_validate_layer(const lychee_dims* d, const void* q, const void* kc, const void* vc,
                                    const uint8_t* role_mask, const int32_t* S_in, const int32_t* S_out,
                                    const float* out, const int32_t* n_ctx, int32_t k) {
    lychee_status s = check_common(d, q, kc, vc, out, n_ctx);
    if (s != LYCHEE_OK) return s;
    if (!role_mask) return fail(LYCHEE_ERR_INVALID_ARG, "role_mask is NULL");
    if (!S_out) return fail(LYCHEE_ERR_INVALID_ARG, "S_out is NULL");
    if (k < 1 || k > d->k_max) return fail(LYCHEE_ERR_INVALID_ARG, "k must be in [1, k_max=%d] (got %d)", d->k_max, k);
    bool any_sparse = false;
    for (int g = 0; g < d->n_kv_heads; ++g) any_sparse |= (role_mask[g] == 0);
    if (any_sparse && !S_in)
        return fail(LYCHEE_ERR_INVALID_ARG, "S_in is NULL but role_mask has sparse heads (only layer 0 may omit S)");
    if (((uintptr_t)S_out | (uintptr_t)S_in) & 3u)
        return fail(LYCHEE_ERR_INVALID_ARG, "S_in and S_out must be 4-byte aligned");
    const size_t sbytes = (size_t)d->batch * d->n_kv_heads * k * 4;
    const Range r_so = span(S_out, sbytes);
    if (S_in && S_in != S_out && overlap(r_so, span(S_in, sbytes)))
        return fail(LYCHEE_ERR_INVALID_ARG, "S_out partially overlaps S_in (must be equal or disjoint)");
    const size_t es = elem_bytes(d);
    const size_t nq = (size_t)d->batch * d->n_q_heads * d->head_dim;
    const size_t nkv = (size_t)d->batch * d->n_kv_heads * d->max_ctx * d->head_dim;
    if (overlap(r_so, span(q, nq * es)) || overlap(r_so, span(kc, nkv * es)) || overlap(r_so, span(vc, nkv * es)) ||
        overlap(r_so, span(out, nq * 4)) || overlap(r_so, span(n_ctx, (size_t)d->batch * 4)))
        return fail(LYCHEE_ERR_INVALID_ARG, "S_out overlaps another argument");
    if (S_in && overlap(span(S_in, sbytes), span(out, nq * 4)))
        return fail(LYCHEE_ERR_INVALID_ARG, "out overlaps S_in");
    return ok();
}

lychee_status lychee_create(const lychee_dims* dims, void* workspace, size_t workspace_bytes, void* stream,
                            lychee_handle** out_handle) {
    if (!out_handle) return fail(LYCHEE_ERR_INVALID_ARG, "out_handle is NULL");
    *out_handle = nullptr;
    lychee_status s = check_dims(dims);
    if (s != LYCHEE_OK) return s;
    const size_t need = lychee_workspace_bytes(dims);
    if (!workspace || ((uintptr_t)workspace & 255u))
        return fail(LYCHEE_ERR_WORKSPACE, "workspace must be non-NULL and 256-byte aligned");
    if (workspace_bytes < need)
        return fail(LYCHEE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                hipSuccess)
        return fail(LYCHEE_ERR_HIP, "cannot query the current HIP device");
    lychee_handle* h = new lychee_handle();
    h->dims = *dims;
    h->ws_base = workspace;
    h->ws_bytes = workspace_bytes;
    h->ws = carve_workspace(workspace, dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim, dims->max_ctx,
                            dims->k_max);
    h->stream = (hipStream_t)stream;
    h->device = dev;
    // persistent attention workgroups per compute unit: one (the hybrid
    // variants hold more than 256 VGPRs, so a second would only queue behind
    // the first; the dense variants stream fastest with one as well), or
    // LYCHEE_ATTEND_WG_PER_CU (1..8) when set
    int per_cu = 1;
    if (const char* env = getenv("LYCHEE_ATTEND_WG_PER_CU")) {
        const int v = atoi(env);
        if (v >= 1 && v <= 8) per_cu = v;
    }
    h->cus = cus;
    h->per_cu = per_cu;
    // pool cost of a gathered S row against a streamed row's kCostRetrieval:
    // kCostSparse, or LYCHEE_POOL_COST_SPARSE (4..12) when set
    h->cost_sparse = kCostSparse;
    if (const char* env = getenv("LYCHEE_POOL_COST_SPARSE")) {
        const int v = atoi(env);
        if (v >= 4 && v <= 12) h->cost_sparse = (uint32_t)v;
    }
    h->ev_start = nullptr;
    h->ev_stop = nullptr;
    h->trace = nullptr;
    h->trace_launch = 0;
    if (hipMemsetAsync(h->ws.zero_begin, 0, h->ws.zero_bytes, h->stream) != hipSuccess) {
        delete h;
        return fail(LYCHEE_ERR_HIP, "clearing the workspace counters failed");
    }
    *out_handle = h;
    return ok();
}

lychee_status lychee_set_stream(lychee_handle* h, void* stream) {
    if (!h) return fail(LYCHEE_ERR_INVALID_ARG, "handle is NULL");
    h->stream = (hipStream_t)stream;
    return ok();
}

lychee_status lychee_set_profile_events(lychee_handle* h, void* start, void* stop) {
    if (!h) return fail(LYCHEE_ERR_INVALID_ARG, "handle is NULL");
    if ((start == nullptr) != (stop == nullptr))
        return fail(LYCHEE_ERR_INVALID_ARG, "pass both events or neither");
    h->ev_start = (hipEvent_t)start;
    h->ev_stop = (hipEvent_t)stop;
    return ok();
}

static lychee_status run_layer(lychee_handle* h, const void* q, const void* kc, const void* vc,
                               const uint8_t* role_mask, const int32_t* S_in, int32_t* S_out, float* out,
                               const int32_t* n_ctx, int32_t k, bool hybrid, int32_t rule = LYCHEE_SELECT_TOPK,
                               double param = 0.0) {
    const lychee_dims& d = h->dims;
    uint64_t bits = 0;
    for (int g = 0; g < d.n_kv_heads; ++g)
        if (!hybrid || role_mask[g]) bits |= 1ull << g;
    AttendParams ap{};
    ap.q = q;
    ap.kc = kc;
    ap.vc = vc;
    ap.S_in = S_in;
    ap.S_out = S_out;
    ap.out = out;
    ap.n_ctx = n_ctx;
    ap.ws = h->ws;
    ap.role_bits = bits;
    ap.B = d.batch;
    ap.Hkv = d.n_kv_heads;
    ap.max_ctx = d.max_ctx;
    ap.k = hybrid ? k : 1;
    ap.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d.head_dim));
    const int G = d.n_q_heads / d.n_kv_heads;
    ap.sel_ratio = rule == LYCHEE_SELECT_RATIO ? param : 1.0;
    ap.sel_block = 0u;
    if (hybrid && rule == LYCHEE_SELECT_BLOCK)
        while ((1 << ap.sel_block) < (int)param) ++ap.sel_block;          // param: 16 .. 256, a power of two
    ap.sel_zpart = hybrid && rule == LYCHEE_SELECT_TOPP ? 1u : 0u;
    ap.topp_P = rule == LYCHEE_SELECT_TOPP ? (unsigned long long)(param * 0x1p52) : 0ull;
    ap.bkey_stride = block_key_stride(d.max_ctx);
    // The kernel's selection key is the fp32 sum of the G query heads' raw
    // dot products, i.e. G sqrt(d) times the pooled score: tau maps there.
    ap.trace = h->trace;
    ap.trace_launch = h->trace_launch;
    ap.cost_sparse = h->cost_sparse;
    ap.sel_tkey = rule == LYCHEE_SELECT_THRESHOLD
                      ? float_key((float)(param * (double)G * std::sqrt((double)d.head_dim)))
                      : 0u;
    if (h->ev_start && hipEventRecord(h->ev_start, h->stream) != hipSuccess)
        return fail(LYCHEE_ERR_HIP, "hipEventRecord failed");
    hipError_t e = launch_attend(ap, d.dtype, d.head_dim, G, hybrid, h->cus, h->per_cu, h->stream);
    if (e != hipSuccess) return fail(LYCHEE_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
    if (h->ev_stop && hipEventRecord(h->ev_stop, h->stream) != hipSuccess)
        return fail(LYCHEE_ERR_HIP, "hipEventRecord failed");
    return ok();
}

lychee_status lychee_decode_layer(lychee_handle* h, const void* q, const void* k_cache, const void* v_cache,
                                  const uint8_t* role_mask, const int32_t* S_in, int32_t* S_out, float* out,
                                  const int32_t* n_ctx, int32_t k) {
    if (!h) return fail(LYCHEE_ERR_INVALID_ARG, "handle is NULL");
    lychee_status s = lychee_validate_layer(&h->dims, q, k_cache, v_cache, role_mask, S_in, S_out, out, n_ctx, k);
    if (s != LYCHEE_OK) return s;
    return run_layer(h, q, k_cache, v_cache, role_mask, S_in, S_out, out, n_ctx, k, true);
}

lychee_status lychee_decode_layer_select(lychee_handle* h, const void* q, const void* k_cache,
                                         const void* v_cache, const uint8_t* role_mask, const int32_t* S_in,
                                         int32_t* S_out, float* out, const int32_t* n_ctx, int32_t k, int32_t rule,
                                         double param) {
    // the rule is checked first (host-only, so it can be checked without a device)
    if (rule != LYCHEE_SELECT_TOPK && rule != LYCHEE_SELECT_RATIO && rule != LYCHEE_SELECT_THRESHOLD &&
        rule != LYCHEE_SELECT_TOPP && rule != LYCHEE_SELECT_BLOCK)
        return fail(LYCHEE_ERR_INVALID_ARG,
                    "rule must be LYCHEE_SELECT_TOPK, _RATIO, _THRESHOLD, _TOPP or _BLOCK (got %d)", rule);
    if (rule == LYCHEE_SELECT_RATIO && !(param > 0.0 && param <= 1.0))
        return fail(LYCHEE_ERR_INVALID_ARG, "the ratio rule's theta must be in (0, 1] (got %g)", param);
    if (rule == LYCHEE_SELECT_TOPP && !(param > 0.0 && param <= 1.0))
        return fail(LYCHEE_ERR_INVALID_ARG, "the Top-p rule's p must be in (0, 1] (got %g)", param);
    if (rule == LYCHEE_SELECT_BLOCK) {
        const bool pow2 = param == 16.0 || param == 32.0 || param == 64.0 || param == 128.0 || param == 256.0;
        if (!pow2) return fail(LYCHEE_ERR_INVALID_ARG, "the block size must be 16, 32, 64, 128 or 256 (got %g)", param);
        if (k < (int32_t)param || k / (int32_t)param > kMaxSelBlocks)
            return fail(LYCHEE_ERR_INVALID_ARG, "the block rule needs block size <= k <= %d blocks (k = %d, block %g)",
                        kMaxSelBlocks, k, param);
    }
    if (rule == LYCHEE_SELECT_THRESHOLD && std::isnan(param))
        return fail(LYCHEE_ERR_INVALID_ARG, "the threshold rule's tau is NaN");
    if (!h) return fail(LYCHEE_ERR_INVALID_ARG, "handle is NULL");
    lychee_status s = lychee_validate_layer(&h->dims, q, k_cache, v_cache, role_mask, S_in, S_out, out, n_ctx, k);
    if (s != LYCHEE_OK) return s;
    return run_layer(h, q, k_cache, v_cache, role_mask, S_in, S_out, out, n_ctx, k, true, rule, param);
}

lychee_status lychee_decode_layer_static(const lychee_dims* dims, void* stream, const void* q, const void* k_cache,
                                         const void* v_cache, const uint8_t* role_mask, const int32_t* S_in,
                                         int32_t* S_out, float* out, const int32_t* n_ctx, int32_t k) {
    lychee_status s = lychee_validate_layer(dims, q, k_cache, v_cache, role_mask, S_in, S_out, out, n_ctx, k);
    if (s != LYCHEE_OK) return s;
    const Workspace need = carve_workspace(nullptr, dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                                           dims->max_ctx, dims->k_max, false);
    if (need.total_bytes > kScratchBytes)
        return fail(LYCHEE_ERR_WORKSPACE,
                    "these dims need %zu bytes of scratch; the allocation-free entry point has %zu (use "
                    "lychee_decode_layer with a workspace)", need.total_bytes, kScratchBytes);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(LYCHEE_ERR_HIP, "cannot query the current HIP device");
    if (dev < 0 || dev >= kMaxDevices) return fail(LYCHEE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    hipStream_t st = (hipStream_t)stream;
    lychee_handle h{};
    {
        std::lock_guard<std::mutex> lock(g_static_mutex);
        StaticScratch& ss = g_static[dev];
        if (!ss.ready) {
            void* ptr = nullptr;
            hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !ptr)
                return fail(LYCHEE_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
            int cus = 0;
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
                return fail(LYCHEE_ERR_HIP, "cannot query the compute units of device %d", dev);
            ss.ptr = ptr;
            ss.cus = cus;
            ss.zero_prefix = 0;
            ss.ready = true;
        }
        h.dims = *dims;
        h.ws_base = ss.ptr;
        h.ws_bytes = kScratchBytes;
        h.ws = carve_workspace(ss.ptr, dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim, dims->max_ctx,
                               dims->k_max, false);
        h.stream = st;
        h.device = dev;
        h.cus = ss.cus;
        h.per_cu = 1;
        h.cost_sparse = kCostSparse;
        // The zero region starts at offset 0 in every layout and ends with the
        // error-flag words, which calls latch rather than restore (and which
        // need not start at zero here: nothing reads them): the calls keep
        // [0, err) at zero.  Clear what earlier calls have not left at zero.
        const size_t keep_zero = (size_t)((char*)h.ws.err - (char*)ss.ptr);
        if (keep_zero > ss.zero_prefix) {
            const size_t from = ss.zero_prefix, words = (keep_zero - from) / 4;
            hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                               dim3(256), 0, st, (uint32_t*)((char*)ss.ptr + from), words);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return fail(LYCHEE_ERR_HIP, "clearing the scratch failed: %s", hipGetErrorString(e));
        }
        ss.zero_prefix = keep_zero;
    }
    return run_layer(&h, q, k_cache, v_cache, role_mask, S_in, S_out, out, n_ctx, k, true);
}

lychee_status lychee_dense_decode_layer(lychee_handle* h, const void* q, const void* k_cache, const void* v_cache,
                                        float* out, const int32_t* n_ctx) {
    if (!h) return fail(LYCHEE_ERR_INVALID_ARG, "handle is NULL");
    lychee_status s = check_common(&h->dims, q, k_cache, v_cache, out, n_ctx);
    if (s != LYCHEE_OK) return s;
    return run_layer(h, q, k_cache, v_cache, nullptr, nullptr, nullptr, out, n_ctx, 1, false);
}

lychee_status lychee_kv_append(lychee_handle* h, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               int32_t* n_ctx) {
    if (!h) return fail(LYCHEE_ERR_INVALID_ARG, "handle is NULL");
    const lychee_dims& d = h->dims;
    if (!k_new || !v_new || !k_cache || !v_cache || !n_ctx) return fail(LYCHEE_ERR_INVALID_ARG, "a tensor pointer is NULL");
    if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)n_ctx) & 3u)
        return fail(LYCHEE_ERR_INVALID_ARG, "tensors must be 4-byte aligned");
    const size_t es = elem_bytes(&d);
    const size_t nnew = (size_t)d.batch * d.n_kv_heads * d.head_dim * es;
    const size_t nkv = (size_t)d.batch * d.n_kv_heads * d.max_ctx * d.head_dim * es;
    const Range rk = span(k_cache, nkv), rv = span(v_cache, nkv), rn = span(n_ctx, (size_t)d.batch * 4);
    if (overlap(rk, rv) || overlap(rk, rn) || overlap(rv, rn) || overlap(rk, span(k_new, nnew)) ||
        overlap(rk, span(v_new, nnew)) || overlap(rv, span(k_new, nnew)) || overlap(rv, span(v_new, nnew)))
        return fail(LYCHEE_ERR_INVALID_ARG, "the caches, the new rows and n_ctx must not overlap");
    AppendParams ap{};
    ap.k_new = k_new;
    ap.v_new = v_new;
    ap.kc = k_cache;
    ap.vc = v_cache;
    ap.n_ctx = n_ctx;
    ap.err = h->ws.err;
    ap.B = d.batch;
    ap.Hkv = d.n_kv_heads;
    ap.d = d.head_dim;
    ap.max_ctx = d.max_ctx;
    ap.elem_bytes = (int32_t)es;
    hipError_t e = launch_kv_append(ap, h->stream);
    if (e != hipSuccess) return fail(LYCHEE_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
    return ok();
}

lychee_status lychee_correction_attention(lychee_handle* h, const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* n_ctx, int32_t T, float* out) {
    if (!h) return fail(LYCHEE_ERR_INVALID_ARG, "handle is NULL");
    const lychee_dims& d = h->dims;
    if (T < 1 || T > kCorrMaxT) return fail(LYCHEE_ERR_INVALID_ARG, "T must be in [1, %d] (got %d)", kCorrMaxT, T);
    if (d.dtype != LYCHEE_BF16 || d.head_dim != 128)
        return fail(LYCHEE_ERR_UNSUPPORTED, "the correction attention runs on bf16 caches with head_dim 128");
    const int G = d.n_q_heads / d.n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(LYCHEE_ERR_UNSUPPORTED, "the correction attention needs n_q_heads / n_kv_heads in {1, 2, 4, 8}");
    if (!q || !k_cache || !v_cache || !n_ctx || !out) return fail(LYCHEE_ERR_INVALID_ARG, "a tensor pointer is NULL");
    if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15u)
        return fail(LYCHEE_ERR_INVALID_ARG, "q, the caches and out must be 16-byte aligned");
    if ((uintptr_t)n_ctx & 3u) return fail(LYCHEE_ERR_INVALID_ARG, "n_ctx must be 4-byte aligned");
    const size_t nq = (size_t)d.batch * T * d.n_q_heads * d.head_dim;
    const size_t nkv = (size_t)d.batch * d.n_kv_heads * d.max_ctx * d.head_dim * 2;
    const Range ro = span(out, nq * 4);
    if (overlap(ro, span(q, nq * 2)) || overlap(ro, span(k_cache, nkv)) || overlap(ro, span(v_cache, nkv)) ||
        overlap(ro, span(n_ctx, (size_t)d.batch * 4)))
        return fail(LYCHEE_ERR_INVALID_ARG, "out overlaps an input");
    const int BH = d.batch * d.n_kv_heads;
    int nchunks = kCorrTargetWG / BH;
    nchunks = nchunks < 1 ? 1 : nchunks;
    const int by_len = d.max_ctx / 256;             // chunks of at least 256 keys
    nchunks = nchunks > by_len ? (by_len < 1 ? 1 : by_len) : nchunks;
    CorrParams cp{};
    cp.q = q;
    cp.kc = k_cache;
    cp.vc = v_cache;
    cp.n_ctx = n_ctx;
    cp.out = out;
    cp.rec_ml = h->ws.crec_ml;
    cp.rec_o = h->ws.crec_o;
    cp.err = h->ws.err;
    cp.B = d.batch;
    cp.Hkv = d.n_kv_heads;
    cp.max_ctx = d.max_ctx;
    cp.T = T;
    cp.nchunks = nchunks;
    cp.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d.head_dim));
    if (h->ev_start && hipEventRecord(h->ev_start, h->stream) != hipSuccess)
        return fail(LYCHEE_ERR_HIP, "hipEventRecord failed");
    hipError_t e = launch_correction(cp, G, h->stream);
    if (e != hipSuccess) return fail(LYCHEE_ERR_HIP, "correction launch failed: %s", hipGetErrorString(e));
    if (h->ev_stop && hipEventRecord(h->ev_stop, h->stream) != hipSuccess)
        return fail(LYCHEE_ERR_HIP, "hipEventRecord failed");
    return ok();
}

lychee_status lychee_check_device_errors(lychee_handle* h) {
    if (!h) return fail(LYCHEE_ERR_INVALID_ARG, "handle is NULL");
    uint32_t flag = 0;
    if (hipStreamSynchronize(h->stream) != hipSuccess) return fail(LYCHEE_ERR_HIP, "stream synchronize failed");
    if (hipMemcpy(&flag, h->ws.err, sizeof flag, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(LYCHEE_ERR_HIP, "reading the device error flag failed");
    if (flag) {
        if (hipMemset(h->ws.err, 0, sizeof flag) != hipSuccess)
            return fail(LYCHEE_ERR_HIP, "clearing the device error flag failed");
        return fail(LYCHEE_ERR_DEVICE_CHECK, "device error flag 0x%x (1: S_in entry outside [0, n_ctx) and not -1; 2: select count mismatch; "
                    "4: n_ctx < T in a correction; 8: append to a full cache; 16: n_ctx outside [1, max_ctx]; "
                    "32: S_in entries not strictly ascending (a duplicate))",
                    flag);
    }
    return ok();
}

void lychee_destroy(lychee_handle* h) { delete h; }

#ifdef LYCHEE_TRACE
lychee_status lychee_set_trace(lychee_handle* h, void* buffer, uint32_t launch) {
    if (!h) return fail(LYCHEE_ERR_INVALID_ARG, "handle is NULL");
    h->trace = (unsigned long long*)buffer;
    h->trace_launch = launch;
    return ok();
}
#endif

}  // extern "C"
