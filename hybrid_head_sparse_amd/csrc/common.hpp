// Internal definitions shared by the gfx950 kernels and the host launcher of
// the hybrid-head decode-attention step.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lychee {

// ---------------------------------------------------------------- limits
constexpr int kMaxWG = 2048;          // persistent attention workgroups per launch
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
constexpr uint32_t kCostSparse = 8;
constexpr uint32_t kMinCostPerWG = 64 * kCostSparse;   // never split the pool finer than this
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
// Polls (about 1 us each) a helper spends waiting for the head's last arrival
// before leaving its slice of the top-k to it.
constexpr int kResolveWaitPolls = 64;
// Slices of a retrieval head's context whose top-k winners are resolved by
// separate workgroups (each reads every candidate, marks and writes its slice).
constexpr int kResolveSlices = 8;
// Increments of a head's selection counter: candidates in bits 0..31,
// arrivals in bits 32..47, arrivals whose range ends in the head in 48..63.
constexpr unsigned long long kSelArrival = 1ull << 32;
constexpr unsigned long long kSelFreeArrival = 1ull << 48;
static_assert(kMaxWG < (1 << 16) && kMaxCtx <= (1ll << 32), "selection counter fields");
// Workgroups per retrieval head of the rule-selection kernel (Top-p and block
// rules: each works on a slice of the head; the last to arrive cuts the set).
constexpr int kRuleSplit = 16;

// Cross-workgroup hand-off without cache-wide maintenance.  Data one
// workgroup leaves for another inside the same launch is written with
// device-coherent stores (agent-scope relaxed atomic stores: "sc1" stores that
// reach the device coherence point instead of staying dirty in one XCD's L2)
// and read back with device-coherent loads.  The producer waits for its stores
// to complete (vmcnt(0)) before the barrier that precedes its counter atomic,
// so whoever observes the counter can read the data.  This replaces release /
// acquire fences, whose buffer_wbl2 / buffer_inv are L2-wide and were measured
// to dominate the launch when every workgroup executes them.
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

// Order-preserving map fp32 -> uint32 (larger float -> larger key); -0 maps as +0.
__host__ __device__ inline uint32_t float_key(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- workspace
struct Workspace {
    float* rec1;                 // [(kMaxWG + BH) * RS]      level-1 partial records
    float* rec2;                 // [BH * kLevel2Max * RS]    level-2 partial records
    unsigned long long* cand;    // [BH * max_ctx]            selection candidates (key | index << 32)
    uint32_t* score;             // [BH * max_ctx]            every selection key of a retrieval head
                                 //                           (read when a head's bounds fail, and by
                                 //                           the rule-selection kernel)
    unsigned long long* prec;    // [BH * kRuleSplit * 4]     rule selection: per-slice partials
    float* crec_ml;              // [CW * 32 G * 2]           correction attention: chunk partials
    float* crec_o;               // [CW * 32 G * D]           (CW = max(512, BH) workgroups)
    // ---- zero-initialised region (restored to zero by every call) ----
    uint32_t* cnt1;              // [BH * kLevel2Max]         level-1 arrival counters
    uint32_t* cnt2;              // [BH]                      level-2 arrival counters
    unsigned long long* selctr;  // [BH]                      candidates appended (bits 0..31) |
                                 //                           workgroups done appending (32..47) |
                                 //                           those whose range ends in the head (48..63)
    uint32_t* bmax;              // [BH]                      largest candidate bound used for the head
    uint32_t* rclaim;            // [BH * kResolveSlices]     votes of a helper and the last arrival on
                                 //                           who resolves a slice of a head's top-k
    uint32_t* rdone;             // [BH]                      slices whose resolver has read the head's
                                 //                           histogram and counters
    uint32_t* hist;              // [BH * kHistBins]          first-digit counts from each pass's bound up
    uint32_t* pctr;              // [BH]                      rule selection: slices done
    uint32_t* err;               // [4]
    void* zero_begin;
    size_t zero_bytes;
    size_t total_bytes;
};

// Record = m[G], l[G], o[G][D] (floats): running max (log2 domain), sum of
// weights, unnormalised weighted value sum.
inline int record_floats(int G, int D) { return G * (D + 2); }

// Carve a workspace for the given dims from `base` (nullptr -> sizes only).
inline Workspace carve_workspace(void* base, int B, int Hq, int Hkv, int D, int max_ctx, int k_max) {
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
    size_t o_rec1 = take(sizeof(float) * (size_t)(kMaxWG + BH) * RS);
    size_t o_rec2 = take(sizeof(float) * (size_t)BH * kLevel2Max * RS);
    size_t o_cand = take(sizeof(unsigned long long) * (size_t)BH * max_ctx);
    size_t o_score = take(sizeof(uint32_t) * (size_t)BH * max_ctx);
    size_t o_prec = take(sizeof(unsigned long long) * (size_t)BH * kRuleSplit * 4);
    const size_t CW = (size_t)(BH > 512 ? BH : 512);
    size_t o_crml = take(sizeof(float) * CW * 32 * G * 2);
    size_t o_cro = take(sizeof(float) * CW * 32 * G * D);
    size_t z0 = off;
    size_t o_cnt1 = take(sizeof(uint32_t) * (size_t)BH * kLevel2Max);
    size_t o_cnt2 = take(sizeof(uint32_t) * (size_t)BH);
    size_t o_sc = take(sizeof(unsigned long long) * (size_t)BH);
    size_t o_bmax = take(sizeof(uint32_t) * (size_t)BH);
    size_t o_rclaim = take(sizeof(uint32_t) * (size_t)BH * kResolveSlices);
    size_t o_rdone = take(sizeof(uint32_t) * (size_t)BH);
    size_t o_hist = take(sizeof(uint32_t) * (size_t)BH * kHistBins);
    size_t o_pctr = take(sizeof(uint32_t) * (size_t)BH);
    size_t o_err = take(sizeof(uint32_t) * 4);
    Workspace w{};
    char* p = (char*)base;
    w.total_bytes = off;
    w.zero_bytes = off - z0;
    if (p) {
        w.rec1 = (float*)(p + o_rec1);
        w.rec2 = (float*)(p + o_rec2);
        w.cand = (unsigned long long*)(p + o_cand);
        w.score = (uint32_t*)(p + o_score);
        w.prec = (unsigned long long*)(p + o_prec);
        w.crec_ml = (float*)(p + o_crml);
        w.crec_o = (float*)(p + o_cro);
        w.cnt1 = (uint32_t*)(p + o_cnt1);
        w.cnt2 = (uint32_t*)(p + o_cnt2);
        w.selctr = (unsigned long long*)(p + o_sc);
        w.bmax = (uint32_t*)(p + o_bmax);
        w.rclaim = (uint32_t*)(p + o_rclaim);
        w.rdone = (uint32_t*)(p + o_rdone);
        w.hist = (uint32_t*)(p + o_hist);
        w.pctr = (uint32_t*)(p + o_pctr);
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
    // Retrieval heads only write every token's key to the score buffer and
    // leave S to a later kernel (the block rule): no top-k.
    uint32_t sel_keys_only;
};

// Host launcher (defined next to the kernel).  dtype: 0 fp32, 1 bf16.  The
// persistent grid is `cus` times `per_cu` workgroups (at most kMaxWG).
hipError_t launch_attend(const AttendParams& p, int dtype, int D, int G, bool hybrid, int cus, int per_cu,
                         hipStream_t stream);

}  // namespace lychee
