// Internal definitions shared by the gfx950 kernels and the host launcher of
// the hybrid-head decode-attention step.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lychee {

// ---------------------------------------------------------------- limits
constexpr int kMaxWG = 2048;          // persistent attention workgroups per launch
constexpr int kMaxSelBlocks = 4096;   // floor(k / bs) limit of the block rule (blocks listed in LDS)
constexpr int kMaxBH = 1024;          // batch * n_kv_heads
constexpr int kMaxKvHeads = 64;       // role mask travels as one 64-bit word
constexpr int kMaxCtx = 1 << 18;      // token index fits 18 bits (select bitmap in LDS)
constexpr int kIdxBits = 18;

// ---------------------------------------------------------------- attention kernel
constexpr int kAttendThreads = 256;   // 4 wavefronts of 64
constexpr int kWaves = kAttendThreads / 64;
constexpr int kCombineFanIn = 32;     // level-1 combine groups of consecutive workgroups
constexpr int kLevel2Max = kMaxWG / kCombineFanIn + 2;
// Pool cost of one unit of work: a streamed key row (retrieval head) costs 4,
// a gathered S row (sparse head) 8 -- gathers of scattered 256-byte rows run
// at about half the streaming rate.  8 measured best on the 128K step against
// 7 and 9 (and against retrieval costs 3, 5, 6 and 8): a dearer sparse row
// gives the sparse workgroups fewer rows and the retrieval workgroups more.
constexpr uint32_t kCostRetrieval = 4;
constexpr uint32_t kCostSparse = 6;
constexpr int kIdxChunk = 2048;       // sparse S positions staged in LDS per pass
constexpr int kKeyCap = 4096;         // retrieval selection keys kept in LDS per pass

// ---------------------------------------------------------------- selection
constexpr int kHistBits = 12;                 // first radix digit, histogrammed while streaming
constexpr int kHistBins = 1 << kHistBits;
constexpr int kCandLds = 4096;                // threshold-digit candidates resolved in LDS
// A workgroup appends the keys of a pass whose first digit reaches its own
// crossing at its proportional share s of the budget, k_eff * rows / n, plus
// a margin: the smaller of kSelMargin - 1 shares and 4 Poisson standard
// deviations of s plus 2, raised to at least 3 deviations plus 4 (for passes
// of a few rows, whose share is tiny).  That is a lower bound of the head's
// threshold digit unless the pass holds more than that many of the head's
// top-k_eff keys; the selector checks it and otherwise reads every key.
// Measured on the 128K step against 5 deviations (floor 4): 4 takes fewer
// candidates and wins (1102 -> 1076 us); 3.5 and 3 fall back often enough to
// lose (1185 and 1295 us).
constexpr uint32_t kSelMargin = 2;
// Slices of the context bitmap of the full-scan resolver (the fallback of the
// candidate resolver: every key of the head re-read).
constexpr int kResolveSlices = 8;
// The candidate resolver stages a head's candidates in LDS kFastBatch at a
// time and resolves threshold-digit groups of at most kFastGroup keys.
constexpr int kFastBatch = 8192;
// A helper waits at most this long (s_memrealtime ticks, 100 MHz) for its
// head's arrivals before it withdraws and leaves the resolve to the last one.
constexpr unsigned long long kHelperWaitTicks = 10000;
constexpr int kFastPer = kFastBatch / kAttendThreads;   // entries per thread of a batch
static_assert((kFastBatch / (kAttendThreads / 64)) % 512 == 0, "a wavefront's quarter of a batch is whole 8-step reads");
constexpr int kFastGroup = 1024;
static_assert(kMaxCtx <= (1 << 20), "a workgroup's candidate count fits 20 bits of its word");
static_assert((unsigned long long)kMaxWG * kMaxCtx < (1ull << 32), "workgroup boundaries in 32-bit arithmetic");
// Top-p normaliser partials of one attention launch: one slot per (workgroup
// w, head bg) pair at w + bg.
constexpr int kZSlots = kMaxWG + kMaxBH;

// Cross-workgroup hand-off without cache-wide maintenance.  Data one
// workgroup leaves for another inside the same launch is written with
// device-coherent stores (agent-scope relaxed atomic stores: "sc1" stores that
// reach the device coherence point instead of staying dirty in one XCD's L2)
// and read back with device-coherent loads.  The producer waits for its stores
// to complete (vmcnt(0)) before the barrier that precedes its counter atomic,
// so whoever observes the counter can read the data.  This replaces release /
// acquire fences, whose buffer_wbl2 / buffer_inv are L2-wide and were measured
// to dominate the launch when every workgroup executes them.
//
// Why it is ordered, and the invariant every edit must keep:
//   1. every datum one workgroup hands to another within a launch is written
//      with coherent_store (or an agent-scope atomic) and read with
//      coherent_load (or an atomic) -- a plain store may sit dirty in the
//      producer's XCD-local L2 and a plain load may hit a stale line in the
//      consumer's, and relaxed agent-scope accesses are coherent per
//      location but order nothing between locations;
//   2. the producer executes wait_stores_complete() after its last such store
//      and then __syncthreads() before the counter RMW.  On gfx9 vmcnt counts
//      stores as well as loads, and an sc1 store leaves vmcnt only once the
//      agent coherence point has acknowledged it, so the data is visible
//      device-wide before any wave of the workgroup can pass the barrier
//      and issue the counter RMW.  The asm statement's "memory" clobber keeps
//      the compiler from sinking stores below it;
//   3. the consumer reads the handed-off data only after the RMW's returned
//      value (or a coherent_load of the counter) has been compared and the
//      outcome passed through __syncthreads().  The barrier's workgroup
//      fences stop the compiler hoisting the data loads above it, and a wave
//      issues in order without speculating loads, so the loads leave after
//      the counter was seen.
// Data handed to the next launch (S_out, out) needs none of this: the
// end-of-kernel release and the next kernel's acquire order it.
template <typename V>
__device__ __forceinline__ void coherent_store(V* p, V v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V coherent_load(const V* p) {
    return __hip_atomic_load(const_cast<V*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_complete() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t counter_add(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void counter_reset(uint32_t* p) {
    __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long counter_add64(unsigned long long* p, unsigned long long v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void counter_reset64(unsigned long long* p) {
    __hip_atomic_store(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Compare-and-swap at agent scope; returns the value found.
__device__ __forceinline__ uint32_t counter_cas(uint32_t* p, uint32_t expect, uint32_t desired) {
    __hip_atomic_compare_exchange_strong(p, &expect, desired, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return expect;
}

// Order-preserving map fp32 -> uint32 (larger float -> larger key); -0 maps as +0.
__host__ __device__ inline uint32_t float_key(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Inverse of float_key.
__host__ __device__ inline float key_float(uint32_t key) {
    const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return __builtin_bit_cast(float, u);
}

// ---------------------------------------------------------------- workspace
struct Workspace {
    float* rec1;                 // [(kMaxWG + BH) * RS]      level-1 partial records
    float* rec2;                 // [BH * kLevel2Max * RS]    level-2 partial records
    unsigned long long* cand;    // [BH * max_ctx]            selection candidates (key | index << 32)
    uint32_t* wmeta;             // [kMaxWG + BH]             per (workgroup w, head bg) at w + bg: the
                                 //                           candidates it appended | its largest pass
                                 //                           bound << 20 (retrieval heads)
    uint32_t* score;             // [BH * max_ctx]            every selection key of a retrieval head
                                 //                           (read when a head's bounds fail, and by
                                 //                           the Top-p cut)
    float* crec_ml;              // [CW * 32 G * 2]           correction attention: chunk partials
    float* crec_o;               // [CW * 32 G * D]           (CW = max(512, BH) workgroups)
    // ---- zero-initialised region (restored to zero by every call) ----
    uint32_t* cnt1;              // [BH * kLevel2Max]         level-1 arrival counters
    uint32_t* cnt2;              // [BH]                      level-2 arrival counters
    unsigned long long* selctr;  // [BH]                      workgroups done appending their candidates
    uint32_t* bmax;              // [BH]                      (full-scan resolver) largest bound used
    uint32_t* rdone;             // [BH]                      slices whose resolver has read the head's
                                 //                           histogram and counters
    uint32_t* hist;              // [BH * kHistBins]          first-digit counts from each pass's bound up
    uint32_t* bkey;              // [BH * ceil(max_ctx / 16)] block rule: the largest selection key of
                                 //                           each block (atomic max; read and restored to
                                 //                           zero by the head's block resolve)
    uint32_t* zpart;             // [(kMaxWG + BH) * 4]       Top-p: per (workgroup w, head bg) at w + bg:
                                 //                           bg + 1 (0 = empty), the largest pooled sum m
                                 //                           and the sum of 2^((f - m) c) as a double
                                 //                           (tags restored to 0 by the Top-p cut)
    uint32_t* hready;            // [BH]                      helper hand-off of a retrieval head's
                                 //                           resolve: 0 idle, 3 helper waiting, 6
                                 //                           offered, 1 the helper's, 4 the last
                                 //                           arrival's, 5 the helper withdrew
    uint32_t* err;               // [4]
    void* zero_begin;
    size_t zero_bytes;
    size_t total_bytes;
};

// Block words per head of the block rule: one per 16 tokens (the smallest block).
inline int block_key_stride(int max_ctx) { return (max_ctx + 15) / 16; }

// Record = m[G], l[G], o[G][D] (floats): running max (log2 domain), sum of
// weights, unnormalised weighted value sum.
inline int record_floats(int G, int D) { return G * (D + 2); }

// Carve a workspace for the given dims from `base` (nullptr -> sizes only).
// The zero-initialised region comes first, so the layouts of different dims
// agree on where it starts (the allocation-free entry point relies on it).
// Without `with_correction` the correction attention's chunk records are left
// out (crec_ml / crec_o null): enough for the decode layer alone.
inline Workspace carve_workspace(void* base, int B, int Hq, int Hkv, int D, int max_ctx, int k_max,
                                 bool with_correction = true) {
    (void)k_max;
    const int BH = B * Hkv;
    const int G = Hq / Hkv;
    const size_t RS = (size_t)record_floats(G, D);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    size_t z0 = off;
    size_t o_cnt1 = take(sizeof(uint32_t) * (size_t)BH * kLevel2Max);
    size_t o_cnt2 = take(sizeof(uint32_t) * (size_t)BH);
    size_t o_sc = take(sizeof(unsigned long long) * (size_t)BH);
    size_t o_bmax = take(sizeof(uint32_t) * (size_t)BH);
    size_t o_rdone = take(sizeof(uint32_t) * (size_t)BH);
    size_t o_hist = take(sizeof(uint32_t) * (size_t)BH * kHistBins);
    size_t o_bkey = take(sizeof(uint32_t) * (size_t)BH * (size_t)block_key_stride(max_ctx));
    size_t o_zpart = take(sizeof(uint32_t) * 4 * (size_t)(kMaxWG + BH));
    size_t o_hready = take(sizeof(uint32_t) * (size_t)BH);
    size_t o_err = take(sizeof(uint32_t) * 4);
    const size_t z1 = off;
    size_t o_rec1 = take(sizeof(float) * (size_t)(kMaxWG + BH) * RS);
    size_t o_rec2 = take(sizeof(float) * (size_t)BH * kLevel2Max * RS);
    size_t o_cand = take(sizeof(unsigned long long) * (size_t)BH * max_ctx);
    size_t o_wmeta = take(sizeof(uint32_t) * (size_t)(kMaxWG + BH));
    size_t o_score = take(sizeof(uint32_t) * (size_t)BH * max_ctx);
    const size_t CW = (size_t)(BH > 512 ? BH : 512);
    size_t o_crml = with_correction ? take(sizeof(float) * CW * 32 * G * 2) : 0;
    size_t o_cro = with_correction ? take(sizeof(float) * CW * 32 * G * D) : 0;
    Workspace w{};
    char* p = (char*)base;
    w.total_bytes = off;
    w.zero_bytes = z1 - z0;
    if (p) {
        w.rec1 = (float*)(p + o_rec1);
        w.rec2 = (float*)(p + o_rec2);
        w.cand = (unsigned long long*)(p + o_cand);
        w.wmeta = (uint32_t*)(p + o_wmeta);
        w.score = (uint32_t*)(p + o_score);
        w.crec_ml = with_correction ? (float*)(p + o_crml) : nullptr;
        w.crec_o = with_correction ? (float*)(p + o_cro) : nullptr;
        w.cnt1 = (uint32_t*)(p + o_cnt1);
        w.cnt2 = (uint32_t*)(p + o_cnt2);
        w.selctr = (unsigned long long*)(p + o_sc);
        w.bmax = (uint32_t*)(p + o_bmax);
        w.rdone = (uint32_t*)(p + o_rdone);
        w.hist = (uint32_t*)(p + o_hist);
        w.bkey = (uint32_t*)(p + o_bkey);
        w.zpart = (uint32_t*)(p + o_zpart);
        w.hready = (uint32_t*)(p + o_hready);
        w.err = (uint32_t*)(p + o_err);
        w.zero_begin = p + z0;
    }
    return w;
}

// ---------------------------------------------------------------- launch parameters
struct AttendParams {
    const void* q;
    const void* kc;
    const void* vc;
    const int32_t* S_in;
    int32_t* S_out;
    float* out;
    const int32_t* n_ctx;
    Workspace ws;
    uint64_t role_bits;     // bit g set = KV head g is a retrieval head
    int32_t B, Hkv, max_ctx, k;
    float scale_log2;       // log2(e) / sqrt(d)
    // Selection rule of the retrieval heads: the top min(k, ceil(sel_ratio n))
    // tokens (at least one; sel_ratio = 1 for top-k), of which those whose
    // selection key is >= sel_tkey (0 = no floor: every key is >= 0) are
    // kept.  S is padded with -1.
    double sel_ratio;
    uint32_t sel_tkey;
    // Block rule (sel_block = log2 of the block size, 0 otherwise; the
    // kernel's BLOCK build): retrieval heads fold each block's largest
    // selection key into ws.bkey (no token top-k, no score buffer), and the
    // head's last selection arrival or its helper cuts the blocks.
    uint32_t sel_block;
    // Top-p rule (the kernel's TOPP build): retrieval heads also publish their
    // part of the normaliser (ws.zpart), and the head's last selection arrival
    // or its helper cuts the top-k set to its Top-p prefix; topp_P is p as
    // 52-bit fixed point.
    uint32_t sel_zpart;
    unsigned long long topp_P;
    int32_t bkey_stride;    // block words per head in ws.bkey
    // Phase timestamps (the LYCHEE_TRACE build only; null otherwise):
    // kTraceSlots 64-bit words per workgroup and launch, at
    // (trace_launch * gridDim.x + blockIdx.x) * kTraceSlots.
    unsigned long long* trace;
    uint32_t trace_launch;
    uint32_t cost_sparse;   // pool cost of a gathered S row (a streamed row costs kCostRetrieval)
};

// Slots of a workgroup's phase-timestamp record (s_memrealtime, 100 MHz).
enum TraceSlot {
    kTrEntry = 0,        // first instruction
    kTrPrologue,         // cost prefix and range boundaries ready
    kTrHeadStart,        // first head of the range: before its query loads
    kTrStreamEnd,        // last head's streaming (or gathering) done
    kTrSelArrive,        // last retrieval head: selection arrival counted
    kTrRecordDone,       // last head: partial record stored and complete
    kTrArrive,           // last head: record arrival counted
    kTrMergeDone,        // last merge this workgroup ran
    kTrResolveStart,     // top-k resolve begun (last arrival or helper)
    kTrResolveEnd,       // top-k resolve done
    kTrExit,             // last instruction
    kTrFlags,            // bit 0 retrieval head, 1 sparse head, 2 merger, 3 resolver, 4 helper
    kTrHeads,            // heads the range touched
    kTrResolve0 = 16,    // 16..26: phases inside the candidate resolver
    kTrSStaged = 27,     // a sparse head's S entries staged (the gather starts)
    kTrPro0 = 28,        // 28..31: phases inside the prologue
    kTraceSlots = 32
};

// Persistent grid of the attention kernel: `cus` times `per_cu` workgroups,
// at most kMaxWG.
inline int attend_grid(int cus, int per_cu) {
    const int g = cus * per_cu;
    return g > kMaxWG ? kMaxWG : (g < 1 ? 1 : g);
}

// Host launcher (defined next to the kernel).  dtype: 0 fp32, 1 bf16.  The
// persistent grid is `cus` times `per_cu` workgroups (at most kMaxWG).
hipError_t launch_attend(const AttendParams& p, int dtype, int D, int G, bool hybrid, int cus, int per_cu,
                         hipStream_t stream);

}  // namespace lychee
