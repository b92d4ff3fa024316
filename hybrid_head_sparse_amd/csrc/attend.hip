// One layer of the hybrid-head decode step in one launch (gfx950).
//
// For every (sequence b, KV head g) of the layer this kernel computes the
// single-query attention of the G query heads that share the KV head:
//   retrieval head: over all n_b cached tokens (Eq. 1 of section 3.4 of the
//     LycheeDecode long-form digest), and S^(l+1) = argsTopK(A, k) (Eq. 2) on
//     the GQA-pooled logit (the hyper-parameter summary's pooling rule);
//   sparse head: over the min(k, n_b) rows named by S_in (Eq. 3), forwarding S
//     unchanged.
//
// Work pooling.  All (head, row) work -- a row is one streamed key of a
// retrieval head or one gathered S row of a sparse head -- is laid on one cost
// axis (a gathered row weighs 1.5 streamed ones by default) and dealt to the
// persistent workgroups head by head, in proportion to cost, as the digest's
// kernel description asks (the work spread evenly over all thread blocks); a
// head's rows are split evenly among its workgroups.  Each range yields one
// partial (m, l, o) record per head it touches; the last workgroup of each
// group of 32 merges the group's records by the log-sum-exp rule and the last
// group merger writes the output (partials + LSE combine, fused into the same
// launch).
//
// Selection without a second pass over the scores.  While streaming, every
// retrieval workgroup keeps the order-preserving 32-bit keys of its pooled
// logits in LDS and counts their first digit (4096 bins, fine where logits
// live).  When a pass is done it takes its own bound: the digit where its
// histogram reaches its share of k plus a margin.  It adds its counts from
// that bound up to the head's global histogram and appends its keys from the
// bound up, in position order, to its own region of the head's candidate
// list.  The head's last selection arrival hands the resolve to a paired idle
// workgroup (a gathered-rows one, else the head's own first workgroup) or
// does it itself: from the final histogram it takes the
// threshold digit T; if a workgroup's bound lies above T its rows are
// recounted and its candidates replaced (every key re-read as a last
// resort); the candidates above T win, and those in digit T are ranked by
// the rest of the key and then the token index (larger key first, lower index
// first: a strict total order, so the result is exact and unique); the
// winners are written to S in ascending order.  The Ratio and Threshold rules
// change the count and the floor of this cut; the block and Top-p rules have
// builds of their own (block maxima instead of the token top-k; the top-k set
// cut to its Top-p prefix after the resolve).
//
// CDNA4 mapping of the streaming loop: a key row is spread over 16 lanes (one
// DPP row), each lane issuing one 8-32 byte load per row; the G query heads of
// the group share each loaded row.  Each lane forms 16 partial dot products
// (16/G keys x G heads) and a 4-step DPP reduce-scatter leaves lane x with the
// full dot product of (key x/G, head x%G); the per-lane key and head orders
// are permuted (key i^(x/G), head h^(x%G)) so the reduce-scatter needs no
// selects.  The running max is kept per DPP row and only moved when a tile
// exceeds it by 2^8 (lazy rescaling).  Loads are unconditional (clamped and
// masked) so a two-deep software pipeline keeps the next tile in flight.
//
// Cross-workgroup hand-off uses device-coherent stores/loads and relaxed
// counters (see common.hpp): no L2-wide write-back or invalidate.
#include "common.hpp"

namespace lychee {
namespace {

// Phase timestamps of the LYCHEE_TRACE build (thread 0 of each workgroup);
// compiled out otherwise.
#ifdef LYCHEE_TRACE
// tr_row: this workgroup's words, set once at kernel entry
#define LYCHEE_STAMP(slot)                                                                                 \
    do {                                                                                                   \
        if (tr_row && threadIdx.x == 0) tr_row[(slot)] = __builtin_amdgcn_s_memrealtime();                \
    } while (0)
#define LYCHEE_TRACE_SET(slot, v)                                                                          \
    do {                                                                                                   \
        if (tr_row && threadIdx.x == 0) tr_row[(slot)] = (v);                                              \
    } while (0)
#else
#define LYCHEE_STAMP(slot) \
    do {                   \
    } while (0)
#define LYCHEE_TRACE_SET(slot, v) \
    do {                          \
    } while (0)
#endif

constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor2 = 0x122;
constexpr int kDppRowRor1 = 0x121;
constexpr int kDppRowHalfMirror = 0x141;   // lane x <-> x ^ 7 inside each half row
constexpr int kDppQuadXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr float kLazyThresh = 8.0f;        // log2 units: rescale only when the max grows by > 2^8

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Lane h of each row of 16, broadcast to the whole row (DPP row_newbcast).
template <int H>
__device__ __forceinline__ float row_bcast(float v) {
    static_assert(H >= 0 && H < 16, "lane within a row");
    return dpp<0x150 + H>(v);
}

// row_bcast with the lane given at run time (a constant once the caller's
// loop over h < G is unrolled, so the switch folds away).
__device__ __forceinline__ float row_bcast_dyn(float v, int h) {
    switch (h) {
        case 0: return row_bcast<0>(v);
        case 1: return row_bcast<1>(v);
        case 2: return row_bcast<2>(v);
        case 3: return row_bcast<3>(v);
        case 4: return row_bcast<4>(v);
        case 5: return row_bcast<5>(v);
        case 6: return row_bcast<6>(v);
        default: return row_bcast<7>(v);
    }
}

// Value of lane ^ 16 / lane ^ 32 through the VALU lane swaps.  With both
// operands equal to v, permlane16_swap returns (v of lane - 16, v of lane + 16)
// in (first, second) for the lanes of odd / even rows, and permlane32_swap the
// same for the upper / lower 32 lanes.
__device__ __forceinline__ float lane_xor16(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor32(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Element type traits: fp32, or bf16 stored as its 16-bit pattern.
struct F32 {
    static constexpr int kBytes = 4;
};
struct BF16 {
    static constexpr int kBytes = 2;
};

template <typename T, int D, int G>
struct Geo {
    static constexpr int EPL = D / 16;                 // elements of a row held by one lane
    static constexpr int NDW = EPL * T::kBytes / 4;    // dwords of a row held by one lane
    static constexpr int NK = 16 / G;                  // keys per DPP row per tile
    static constexpr int KPW = 4 * NK;                 // keys per wavefront per tile
    static constexpr int LOG2G = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
    static constexpr int RS = G * (D + 2);             // record floats
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
};

template <int NDW>
struct Frag {
    uint32_t w[NDW];
};

// K/V rows are read once per launch: non-temporal loads keep them from
// evicting what is reused (the kernel's code, records, candidates) from L2.
// Measured on the 128K Llama3-shaped step: the all-retrieval layer streams at
// about 7.4 TB/s instead of 6.4, and the whole step runs about 5% faster.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int NDW>
__device__ __forceinline__ void load_frag_once(Frag<NDW>& f, const uint32_t* p) {
    if constexpr (NDW == 2) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        f.w[0] = v.x; f.w[1] = v.y;
    } else if constexpr (NDW == 4) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        f.w[0] = v.x; f.w[1] = v.y; f.w[2] = v.z; f.w[3] = v.w;
    } else {
        static_assert(NDW == 8, "fragment size");
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4));
        f.w[0] = a.x; f.w[1] = a.y; f.w[2] = a.z; f.w[3] = a.w;
        f.w[4] = b.x; f.w[5] = b.y; f.w[6] = b.z; f.w[7] = b.w;
    }
}

template <int NDW>
__device__ __forceinline__ void load_frag(Frag<NDW>& f, const uint32_t* p) {
    if constexpr (NDW == 2) {
        uint2 v = *reinterpret_cast<const uint2*>(p);
        f.w[0] = v.x; f.w[1] = v.y;
    } else if constexpr (NDW == 4) {
        uint4 v = *reinterpret_cast<const uint4*>(p);
        f.w[0] = v.x; f.w[1] = v.y; f.w[2] = v.z; f.w[3] = v.w;
    } else {
        static_assert(NDW == 8, "fragment size");
        uint4 a = *reinterpret_cast<const uint4*>(p);
        uint4 b = *reinterpret_cast<const uint4*>(p + 4);
        f.w[0] = a.x; f.w[1] = a.y; f.w[2] = a.z; f.w[3] = a.w;
        f.w[4] = b.x; f.w[5] = b.y; f.w[6] = b.z; f.w[7] = b.w;
    }
}

template <int NDW>
__device__ __forceinline__ void zero_frag(Frag<NDW>& f) {
#pragma unroll
    for (int i = 0; i < NDW; ++i) f.w[i] = 0u;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Partial dot product of one lane's slice of a query row and a key row, in a
// fixed order (so bit-identical rows give bit-identical results).
template <typename T, int NDW>
__device__ __forceinline__ float dot_frag(const Frag<NDW>& a, const Frag<NDW>& b) {
    float acc = 0.0f;
    if constexpr (T::kBytes == 2) {
#pragma unroll
        for (int i = 0; i < NDW; ++i)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w[i]),
                                                  __builtin_bit_cast(bf16x2, b.w[i]), acc, false);
    } else {
#pragma unroll
        for (int i = 0; i < NDW; ++i)
            acc = __builtin_fmaf(__builtin_bit_cast(float, a.w[i]), __builtin_bit_cast(float, b.w[i]), acc);
    }
    return acc;
}

// Element e of a lane's slice as fp32.
template <typename T, int NDW>
__device__ __forceinline__ float frag_elem(const Frag<NDW>& f, int e) {
    if constexpr (T::kBytes == 2) {
        uint32_t w = f.w[e >> 1];
        return __builtin_bit_cast(float, (e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else {
        return __builtin_bit_cast(float, f.w[e]);
    }
}

// Sum over the 2^s lanes of a row that share x % G... (rotation allreduce by
// 8, 4, 2, 1 restricted to offsets that are multiples of G).
template <int G>
__device__ __forceinline__ float row_sum_same_head(float v) {
    if constexpr (G <= 8) v += dpp<kDppRowRor8>(v);
    if constexpr (G <= 4) v += dpp<kDppRowRor4>(v);
    if constexpr (G <= 2) v += dpp<kDppRowRor2>(v);
    if constexpr (G <= 1) v += dpp<kDppRowRor1>(v);
    return v;
}
template <int G>
__device__ __forceinline__ float row_max_same_head(float v) {
    if constexpr (G <= 8) v = fmaxf(v, dpp<kDppRowRor8>(v));
    if constexpr (G <= 4) v = fmaxf(v, dpp<kDppRowRor4>(v));
    if constexpr (G <= 2) v = fmaxf(v, dpp<kDppRowRor2>(v));
    if constexpr (G <= 1) v = fmaxf(v, dpp<kDppRowRor1>(v));
    return v;
}

__device__ __forceinline__ float safe_scale(float m, float M) {
    return (m == -INFINITY) ? 0.0f : fast_exp2(m - M);
}

// Reductions over the 64 lanes: rotations by 8, 4, 2, 1 inside each row,
// then across rows by the lane swaps.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<kDppRowRor8>(v));
    v = fmaxf(v, dpp<kDppRowRor4>(v));
    v = fmaxf(v, dpp<kDppRowRor2>(v));
    v = fmaxf(v, dpp<kDppRowRor1>(v));
    v = fmaxf(v, lane_xor16(v));
    return fmaxf(v, lane_xor32(v));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<kDppRowRor8>(v);
    v += dpp<kDppRowRor4>(v);
    v += dpp<kDppRowRor2>(v);
    v += dpp<kDppRowRor1>(v);
    v += lane_xor16(v);
    return v + lane_xor32(v);
}

// Records merged by one call: one or two per lane of a wavefront.
constexpr int kMergeMax = 128;
static_assert(kLevel2Max <= kMergeMax && kCombineFanIn <= kMergeMax, "merge fan-in exceeds two records per lane");

// LDS floats merge_records needs: per head a scale per record, then M and L.
template <int G>
constexpr int merge_lds_floats() { return G * kMergeMax + 2 * G; }

// Merge `count` (<= kMergeMax) records (RS floats apart, written by other
// workgroups with device-coherent stores) into one (m, l, o) per head.
// Wavefront w owns heads w, w+4, ..: its lanes load (m, l) of one or two
// records each, reduce M = max m and L = sum l 2^(m - M) across the wavefront,
// and leave the per-record scales 2^(m - M) in LDS.  The o loads of the first
// CH records (a whole level-1 group of 32 when G D <= 512) are issued before that and land while it runs; the output
// pass then reads the scales as wavefront-uniform (broadcast) LDS words.  If
// `out` is non-null the normalised output o / l is written there (query heads
// contiguous, D floats each); otherwise the merged record goes to `dst` with
// device-coherent stores.
template <int D, int G>
__device__ void merge_records(const float* recs, int count, float* dst, float* out, float* s_ml) {
    constexpr int RS = G * (D + 2);
    constexpr int OPT = (G * D + kAttendThreads - 1) / kAttendThreads;   // outputs per thread
    constexpr int CH = 32 / OPT;                                        // records per load batch (a level-1
                                                                        // group of 32 in one round trip)
    constexpr int HPW = (G + kWaves - 1) / kWaves;                      // heads per wavefront
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float* s_sc = s_ml;                     // [G][kMergeMax]
    float* s_M = s_ml + G * kMergeMax;      // [G]
    float* s_L = s_M + G;                   // [G]
    const int r0i = min(lane, count - 1), r1i = min(lane + 64, count - 1);
    float mv[HPW][2], lv[HPW][2];
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int h = min(wave + kWaves * i, G - 1);
        mv[i][0] = coherent_load(&recs[(size_t)r0i * RS + h]);
        lv[i][0] = coherent_load(&recs[(size_t)r0i * RS + G + h]);
        mv[i][1] = coherent_load(&recs[(size_t)r1i * RS + h]);
        lv[i][1] = coherent_load(&recs[(size_t)r1i * RS + G + h]);
    }
    float ov[OPT][CH];
#pragma unroll
    for (int q = 0; q < OPT; ++q) {
        const int idx = min(tid + kAttendThreads * q, G * D - 1);
        const int h = idx / D, t = idx - h * D;
#pragma unroll
        for (int j = 0; j < CH; ++j) ov[q][j] = coherent_load(&recs[(size_t)min(j, count - 1) * RS + 2 * G + h * D + t]);
    }
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
        const int h = wave + kWaves * i;
        if (h < G) {
            const float m0 = lane < count ? mv[i][0] : -INFINITY;
            const float m1 = lane + 64 < count ? mv[i][1] : -INFINITY;
            const float M = wave_max(fmaxf(m0, m1));
            const float c0 = safe_scale(m0, M), c1 = safe_scale(m1, M);
            const float L = wave_sum((lane < count ? lv[i][0] * c0 : 0.0f) + (lane + 64 < count ? lv[i][1] * c1 : 0.0f));
            s_sc[h * kMergeMax + lane] = c0;
            s_sc[h * kMergeMax + 64 + lane] = c1;
            if (lane == 0) {
                s_M[h] = M;
                s_L[h] = L;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < OPT; ++q) {
        const int idx = tid + kAttendThreads * q;
        if (idx >= G * D) break;
        const int h = idx / D, t = idx - h * D;
        const float* sc = s_sc + h * kMergeMax;
        float O = 0.0f;
        for (int r0 = 0; r0 < count; r0 += CH) {
            if (r0 > 0) {   // more records than one batch: load the next batch
#pragma unroll
                for (int j = 0; j < CH; ++j)
                    ov[q][j] = coherent_load(&recs[(size_t)min(r0 + j, count - 1) * RS + 2 * G + h * D + t]);
            }
#pragma unroll
            for (int j = 0; j < CH; ++j)     // scales of records past count are zero
                O += ov[q][j] * sc[r0 + j];
        }
        const float L = s_L[h];
        if (out) {
            out[(size_t)h * D + t] = (L > 0.0f) ? O / L : 0.0f;
        } else {
            coherent_store(&dst[2 * G + h * D + t], O);
            if (t == 0) {
                coherent_store(&dst[h], s_M[h]);
                coherent_store(&dst[G + h], L);
            }
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------- selection helpers

// First digit of a key: a monotone map of the 32-bit key onto the histogram
// bins.  Positive logits of magnitude in [2^-12, 2^12), where attention logits
// live, get one bin per step of their top 7 mantissa bits (128 bins per
// octave); every other key (negative, zero, tiny or huge logits) falls in a
// bin of 64 such steps (2 per octave).  The keys of one bin always agree on
// their top 10 bits, so the low 22 bits and the token index order a bin's
// keys exactly (the composite below).
constexpr uint32_t kFineLo = 0x8000u + (127u - 12u) * 128u;      // key >> 16 of +2^-12
constexpr uint32_t kFineBins = 24u * 128u;                        // up to +2^12
constexpr int kCoarseShift = 6;
constexpr uint32_t kFineBase = kFineLo >> kCoarseShift;           // digits below the fine range
constexpr uint32_t kFineEnd = kFineLo + kFineBins;
constexpr uint32_t kTopDigit = kFineBase + kFineBins + ((0xFFFFu - kFineEnd) >> kCoarseShift);
static_assert(kFineLo % (1u << kCoarseShift) == 0 && kFineEnd % (1u << kCoarseShift) == 0,
              "coarse bins line up with the fine range");
static_assert(kTopDigit < (uint32_t)kHistBins, "every digit has a bin");
constexpr int kLowBits = 22;                             // key bits a bin's keys may differ in
constexpr uint32_t kIdxMask = (1u << kIdxBits) - 1u;
constexpr int kCompBits = kLowBits + kIdxBits;           // composite: low key bits, then inverted index

__device__ __forceinline__ uint32_t key_digit(uint32_t key) {
    const uint32_t k16 = key >> 16;
    const uint32_t lo = k16 >> kCoarseShift;
    const uint32_t mid = kFineBase + (k16 - kFineLo);
    const uint32_t hi = kFineBase + kFineBins + ((k16 - kFineEnd) >> kCoarseShift);
    return k16 < kFineLo ? lo : (k16 < kFineEnd ? mid : hi);
}
// Smallest key of digit d (d <= kTopDigit + 1; kTopDigit + 1 maps past every key).
__device__ __forceinline__ unsigned long long digit_first_key(uint32_t d) {
    const uint32_t k16 = d < kFineBase ? (d << kCoarseShift)
                         : d < kFineBase + kFineBins ? kFineLo + (d - kFineBase)
                                                     : kFineEnd + ((d - kFineBase - kFineBins) << kCoarseShift);
    return (unsigned long long)k16 << 16;
}
constexpr int kWords = kMaxCtx / 32;                     // context bitmap words
constexpr int kHistPerThread = kHistBins / kAttendThreads;
constexpr int kToppBins = 256;                           // Top-p cut: 8-bit radix digits
constexpr int kToppCopies = 4;                           // Top-p cut: interleaved histogram copies (lane & 3)
constexpr int kToppSlots = 16;                           // Top-p cut: set entries a thread holds in registers
constexpr int kCandPerThread = kCandLds / kAttendThreads;

__device__ __forceinline__ unsigned long long pack_cand(uint32_t key, uint32_t idx) {
    return ((unsigned long long)idx << 32) | key;
}
__device__ __forceinline__ unsigned long long composite(uint32_t key, uint32_t idx) {
    return ((unsigned long long)(key & ((1u << kLowBits) - 1u)) << kIdxBits) | (unsigned long long)(kIdxMask - idx);
}
__device__ __forceinline__ uint32_t comp_index(unsigned long long c) { return kIdxMask - (uint32_t)(c & kIdxMask); }
// The whole selection order as one 64-bit value: the key, then the smaller
// index first (kIdxMask - idx): a key wins iff this value is at least the
// k-th largest one.
__device__ __forceinline__ unsigned long long full_order(uint32_t key, uint32_t idx) {
    return ((unsigned long long)key << 32) | (unsigned long long)(kIdxMask - idx);
}
__device__ __forceinline__ uint32_t comp_digit(unsigned long long c, int shift, int bits) {
    return (uint32_t)(c >> shift) & ((1u << bits) - 1u);
}

// Inclusive prefix sum across the 64 lanes of a wavefront: shifts within
// each row of 16 lanes (1, 2, 4, 8), then the row broadcasts of lane 15 into
// rows 1 and 3 and of lane 31 into rows 2 and 3.  Lanes whose DPP source is
// outside the row or whose row is masked off add the `old` operand, 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return x;
}

// Block-wide exclusive prefix sum of one value per thread.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_inclusive_scan(v);
    __syncthreads();
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
        const uint32_t c = s_wave[wv];
        base += (wv < wave) ? c : 0u;
        tot += c;
    }
    *total = tot;
    return base + inc - v;
}

// Inclusive max-scan of signed values across the 64 lanes (the pattern of
// wave_inclusive_scan; lanes without a DPP source take INT32_MIN).
__device__ __forceinline__ int32_t wave_inclusive_max(int32_t x) {
    constexpr int32_t lo = -2147483647 - 1;
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, 0x111, 0xF, 0xF, false));   // row_shr:1
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, 0x112, 0xF, 0xF, false));   // row_shr:2
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, 0x114, 0xF, 0xF, false));   // row_shr:4
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, 0x118, 0xF, 0xF, false));   // row_shr:8
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, 0x142, 0xA, 0xF, false));   // row_bcast:15
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, 0x143, 0xC, 0xF, false));   // row_bcast:31
    return x;
}

// Block-wide exclusive max-scan of one value per thread (INT32_MIN for the
// first thread); *total gets the block's maximum.
__device__ __forceinline__ int32_t block_exclusive_max(int32_t v, uint32_t* s_wave, int32_t* total) {
    constexpr int32_t lo = -2147483647 - 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t inc = wave_inclusive_max(v);
    const int32_t up = __shfl_up(inc, 1);
    const int32_t exc = lane ? up : lo;
    __syncthreads();
    if (lane == 63) s_wave[wave] = (uint32_t)inc;
    __syncthreads();
    int32_t base = lo, tot = lo;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
        const int32_t c = (int32_t)s_wave[wv];
        base = (wv < wave) ? max(base, c) : base;
        tot = max(tot, c);
    }
    *total = tot;
    return max(base, exc);
}

// Crossing of a histogram spread over the block, PER bins per thread held in
// `cnt` (thread t holds the bins of descending rank t*PER .. t*PER+PER-1, i.e.
// bin nbins-1-rank): finds D with (count above D) < need <= (count >= D).
// Result in s_res[0] (digit), s_res[1] (count above D), s_res[3] (count at
// or above D); if the whole histogram holds fewer than `need`, D = 0 and the
// counts above it and in all are returned.
template <int PER>
__device__ __forceinline__ void block_crossing(const uint32_t (&cnt)[PER], int nbins, uint32_t need, uint32_t* s_wave,
                               uint32_t* s_res) {
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) sum += cnt[i];
    uint32_t tot;
    const uint32_t before = block_exclusive_scan(sum, s_wave, &tot);
    const int r0 = (int)threadIdx.x * PER;
    if (tot < need) {
        // fewer than `need` counted: every digit qualifies (D = 0); the owner of
        // bin 0 (descending rank nbins-1) reports the count above it
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (r0 + i == nbins - 1) {
                s_res[0] = 0u;
                s_res[1] = tot - cnt[i];
                s_res[3] = tot;
            }
        }
    } else if (before < need && need <= before + sum) {
        uint32_t acc = before;
        bool found = false;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (!found && acc + cnt[i] >= need) {
                s_res[0] = (uint32_t)(nbins - 1 - (r0 + i));
                s_res[1] = acc;
                s_res[3] = acc + cnt[i];
                found = true;
            }
            acc += cnt[i];
        }
    }
    __syncthreads();
}

template <typename T, int D, int G, bool HYBRID, bool BLOCK, bool TOPP>
__global__ void __launch_bounds__(kAttendThreads) attend_kernel(const AttendParams p) {
    using Ge = Geo<T, D, G>;
    constexpr int EPL = Ge::EPL, NDW = Ge::NDW, NK = Ge::NK, KPW = Ge::KPW, RS = Ge::RS;
    constexpr int LOG2G = Ge::LOG2G;
    constexpr uint32_t STRIDE = kWaves * KPW;          // positions per workgroup tile round

    struct StreamLds {
        uint32_t hist[HYBRID ? kHistBins : 1];
        uint32_t gbuf[HYBRID ? kKeyCap : 1];        // a pass's kept positions, staged for the append
        uint32_t keys[HYBRID ? kKeyCap : 1];
        int32_t idx[HYBRID ? kIdxChunk : 1];
        float pw[kWaves][4][16];
        float wo[kWaves][G][D];
        float wm[kWaves][G];
        float wl[kWaves][G];
        float ml[merge_lds_floats<G>()];
    };
    struct SelectLds {
        uint32_t bits[HYBRID ? kWords : 4];   // selected-position bitmap (16-byte aligned: read 4 words per lane)
        union {
            unsigned long long comp[HYBRID ? kCandLds + kAttendThreads : 1];   // threshold-digit candidates
                                                                               // (+ one spare slot per thread)
            uint32_t h12[HYBRID ? kHistBins : 1];              // the head's final first-digit histogram
        };
        uint32_t h[256];
    };
    struct FastLds {                          // the candidate resolver (fast_resolve)
        union {
            uint32_t h12[HYBRID ? kHistBins : 1];     // the head's first-digit histogram (up to the crossing)
            uint32_t map[HYBRID ? kFastBatch : 1];    // then: the candidate row of each entry of a batch
        };
        uint32_t wm[HYBRID ? kMaxWG : 1];         // workgroup words: candidates | bound << 20
        uint32_t coff[HYBRID ? kMaxWG + 1 : 1];   // flat offset of each workgroup's candidates
        uint32_t key[HYBRID ? kFastBatch : 1];    // a batch of candidates, entry f at [f]
        uint32_t idx[HYBRID ? kFastBatch : 1];
        alignas(16) unsigned long long comp[HYBRID ? kFastGroup : 1];   // the threshold digit's composites
        uint32_t jc[HYBRID ? kFastPer * kWaves : 1];   // winners per (step, wavefront), then their prefix
    };
    struct BlockLds {                         // the block rule's resolve (block_resolve)
        uint32_t h12[HYBRID ? kHistBins : 1];     // first-digit histogram of the block words
        uint32_t w[HYBRID ? kMaxCtx / 16 : 1];    // the head's block words (blocks of >= 16 tokens)
        uint32_t list[HYBRID ? kMaxSelBlocks : 1];   // the kept blocks, ascending (at most floor(k / bs))
        alignas(16) unsigned long long comp[HYBRID ? kFastGroup : 1];   // the threshold digit's composites
    };
    struct ToppLds {                          // the Top-p cut (topp_cut)
        unsigned long long hist[HYBRID ? kToppBins * kToppCopies : 1];   // a digit's share-weighted counts
        unsigned long long lo[kWaves], hi[kWaves], tot[kWaves];
        uint32_t cnt[kWaves];
        unsigned long long above, cutv;
        uint32_t digit, found;
    };
    union Lds {
        StreamLds st;
        SelectLds se;
        FastLds fr;
        BlockLds bl;
        ToppLds tp;
    };
    __shared__ __attribute__((aligned(16))) Lds u;
    __shared__ uint32_t s_pref[kMaxBH + 1];
    __shared__ uint32_t s_bound[kMaxWG + 1];   // cost position where each workgroup's range starts
    __shared__ uint32_t s_first[kMaxBH + 1];   // first workgroup of each head
    __shared__ int32_t s_nctx[kMaxBH];
    __shared__ uint32_t s_ke[kMaxBH];          // tokens a retrieval head of sequence b selects
    __shared__ uint32_t s_wave[kWaves];
    __shared__ uint32_t s_res[4];
    __shared__ int s_flag[2];
    __shared__ uint32_t s_sel[4];     // selection arrival: 1 if this workgroup resolves the head's top-k
    __shared__ int s_rel;
    __shared__ uint32_t s_ceq;        // resolver: threshold-digit composites appended so far
    __shared__ unsigned long long s_cut;   // resolver: the smallest winning full_order of the threshold digit
    __shared__ uint32_t s_lds_set;         // Top-p build: the resolved set is in LDS (one batch; see topp_cut)
    __shared__ uint32_t s_zk[kWaves];      // Top-p normaliser: per-wavefront largest key, then sum
    __shared__ double s_zd[kWaves];

#ifdef LYCHEE_TRACE
    unsigned long long* const tr_row =
        p.trace ? p.trace + ((size_t)p.trace_launch * gridDim.x + blockIdx.x) * kTraceSlots : nullptr;
#endif
    LYCHEE_STAMP(kTrEntry);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wavefront
    const int row = lane >> 4, x = lane & 15;
    const int xh = x >> LOG2G, xl = x & (G - 1);
    const int BH = p.B * p.Hkv;
    const int Hq = p.Hkv * G;

    // ---- prologue: contexts, pool cost per (b, g) and its exclusive prefix ----
    // (thread t takes sequences and heads t, t + 256, ..: one pass when there
    // are at most 256 of them)
    {
        bool bad_n = false;
        for (int b = tid; b < p.B; b += kAttendThreads) {
            // a context outside [1, max_ctx] breaks the contract: it is
            // clamped to [0, max_ctx] (a sequence of 0 rows gets zeros and an
            // empty set, written below) and latches error bit 16
            int n = p.n_ctx[b];
            if (n < 1 || n > p.max_ctx) {
                bad_n = true;
                n = n < 0 ? 0 : (n > p.max_ctx ? p.max_ctx : n);
            }
            // min(k, n), or under the ratio rule min(k, ceil(theta n)) (at least one)
            const double t = ceil(p.sel_ratio * (double)n);
            const uint32_t kr = t < 1.0 ? 1u : (t > (double)n ? (uint32_t)n : (uint32_t)t);
            s_nctx[b] = n;
            s_ke[b] = min((uint32_t)min(p.k, n), kr);
        }
        if (bad_n && blockIdx.x == 0) atomicOr(p.ws.err, 16u);
        __syncthreads();
        LYCHEE_STAMP(kTrPro0 + 0);
        uint32_t run = 0;
        for (int c0 = 0; c0 < BH; c0 += kAttendThreads) {   // (uniform loop)
            const int bg = c0 + tid;
            uint32_t cost = 0;
            if (bg < BH) {
                const int b = bg / p.Hkv, g = bg - b * p.Hkv;
                const int n = s_nctx[b];
                const bool retr = !HYBRID || ((p.role_bits >> g) & 1ull);
                cost = retr ? kCostRetrieval * (uint32_t)n : p.cost_sparse * (uint32_t)min(p.k, n);
            }
            uint32_t tot;
            const uint32_t ex = block_exclusive_scan(cost, s_wave, &tot);
            if (bg < BH) s_pref[bg] = run + ex;
            run += tot;
        }
        if (tid == 0) s_pref[BH] = run;
        __syncthreads();
        LYCHEE_STAMP(kTrPro0 + 1);
    }

    const uint32_t U = s_pref[BH];
    int P = (int)gridDim.x;
    {
        const uint32_t pmax = U / (64u * p.cost_sparse);   // never split the pool finer than 64 gathered rows
        if ((uint32_t)P > pmax) P = (int)(pmax < 1 ? 1 : pmax);
    }
    const int w = blockIdx.x;
    if (w >= P) {
        LYCHEE_STAMP(kTrExit);
        return;
    }

    // A resolver's S entry: device-coherent in the Top-p build, whose cut
    // reads the row back from its coherence point.
    auto put_s = [&](int32_t* row, uint32_t i, int32_t v) {
        if constexpr (TOPP) coherent_store(&row[i], v);
        else row[i] = v;
    };
    auto is_retr = [&](int hb) -> bool { return !HYBRID || ((p.role_bits >> (hb % p.Hkv)) & 1ull); };
    // Heads of a sequence with no context (out of contract, flagged in the
    // prologue) own no rows: workgroup bg % P writes their zero output and
    // their S_out row (-1 for a retrieval head, a copy of S_in for a sparse
    // one).
    for (int bg = w; bg < BH; bg += P) {
        const int b = bg / p.Hkv, g = bg - b * p.Hkv;
        if (s_nctx[b] != 0) continue;
        float* ob = p.out + ((size_t)b * Hq + (size_t)g * G) * D;
        for (int i = tid; i < G * D; i += kAttendThreads) ob[i] = 0.0f;
        if (HYBRID) {
            int32_t* so = p.S_out + (size_t)bg * p.k;
            const int32_t* si = p.S_in ? p.S_in + (size_t)bg * p.k : nullptr;
            if (is_retr(bg)) {
                for (int i = tid; i < p.k; i += kAttendThreads) so[i] = -1;
            } else if (si && si != so) {
                for (int i = tid; i < p.k; i += kAttendThreads) so[i] = si[i];
            }
        }
    }
    auto head_of = [&](uint32_t c) -> int {     // last (b, g) whose cost range starts at or before c
        int cnt = 0;                              // (wave-parallel: the starts are increasing)
        for (int base = 0; base < BH; base += 64) {
            const int i = base + lane;
            cnt += __popcll(__ballot(i < BH && s_pref[i] <= c));
        }
        return cnt - 1;
    };
    // Workgroup boundaries, head-aligned: head h gets the workgroups
    // [first(h), first(h+1)) with first(h) = round(P pref(h) / U) (cumulative
    // rounding: the counts sum to P and follow the heads' costs), and its
    // rows are split evenly among them, so a workgroup pays one head's fixed
    // costs (query loads, S staging, record, selection hand-off) once.  A
    // head whose share rounds to no workgroup falls into the range of the
    // workgroup before it, which then spans heads (many small heads).  Every
    // workgroup tabulates all P+1 boundaries once, in parallel.
    for (int h = tid; h <= BH; h += kAttendThreads)
        // floor((P pref + floor(U/2)) / U) in fp64: the numerator (< 2^42) is
        // exact and a quotient within 1/U of an integer stays apart from it
        // after rounding, so the floor is exact (no 64-bit integer division)
        s_first[h] = U ? (uint32_t)(((double)P * (double)s_pref[h] + (double)(U / 2u)) / (double)U) : 0u;
    __syncthreads();
    for (int ww = tid; ww <= P; ww += kAttendThreads) {
        uint32_t bnd;
        if (ww == 0) {
            bnd = 0u;
        } else if (ww >= P) {
            bnd = U;
        } else {
            int a = 0, z = BH - 1;                 // last head with first(h) <= ww
            while (a < z) {
                const int mid = (a + z + 1) >> 1;
                if (s_first[mid] <= (uint32_t)ww) a = mid; else z = mid - 1;
            }
            const uint32_t h0 = s_pref[a], h1 = s_pref[a + 1];
            const uint32_t cwa = is_retr(a) ? kCostRetrieval : p.cost_sparse;
            const uint32_t rows = (h1 - h0) / cwa;
            const uint32_t i = (uint32_t)ww - s_first[a], nwh = s_first[a + 1] - s_first[a];   // nwh >= 1
            bnd = h0 + cwa * ((i * rows) / nwh);   // i * rows <= kMaxWG * kMaxCtx: 32-bit
        }
        s_bound[ww] = bnd;
    }
    __syncthreads();
    LYCHEE_STAMP(kTrPro0 + 2);
    // Workgroups whose ranges hold cost positions c0 and c1: the number of
    // range starts s_bound[1..P-1] at or before each (the starts are
    // non-decreasing; an empty range shares its start with the next one, so
    // the count lands on the non-empty range).  Wavefront-parallel.
    auto wg_pair = [&](uint32_t c0, uint32_t c1, int& w0, int& w1) {
        int n0 = 0, n1 = 0;
        for (int base = 1; base < P; base += 64) {
            const int i = base + lane;
            const uint32_t v = i < P ? s_bound[i] : 0xFFFFFFFFu;
            n0 += __popcll(__ballot(v <= c0));
            n1 += __popcll(__ballot(v <= c1));
        }
        w0 = n0;
        w1 = n1;
    };
    const uint32_t lo = s_bound[w], hi = s_bound[w + 1];
    // Resolve helpers.  A workgroup that holds gathered rows only is idle
    // once its own work is done; the r-th retrieval head (head order, heads
    // with rows) is paired with the r-th such workgroup, taken as the first
    // workgroup of a sparse head that has at least two (so its range lies
    // inside that head).  A retrieval head left without one (more retrieval
    // heads than such workgroups, as in a layer of retrieval heads only) is
    // helped by its own first workgroup when it spans at least two: that
    // workgroup is idle once its range is recorded, and it takes the resolve
    // while the head's last selection arrival records and merges (if it is
    // that arrival itself, it offers the resolve to itself and takes it
    // back, as when no helper comes).  The pairing follows from the
    // boundaries alone, so every workgroup derives the same one
    // (wavefront-parallel ballots).
    auto helper_cand = [&](int a) -> bool { return a < BH && !is_retr(a) && s_first[a + 1] >= s_first[a] + 2u; };
    auto has_rows = [&](int a) -> bool { return a < BH && s_pref[a + 1] > s_pref[a]; };
    auto needs_help = [&](int a) -> bool { return has_rows(a) && is_retr(a); };
    auto own_helper = [&](int a) -> bool { return s_first[a + 1] >= s_first[a] + 2u; };   // a < BH
    auto kth_bit = [](unsigned long long m, int k) -> int {   // position of the k-th set bit (k from 0)
        for (int t = 0; t < k; ++t) m &= m - 1ull;
        return __ffsll((long long)m) - 1;
    };
    auto helper_of = [&](int X) -> int {       // X's helper workgroup, or -1
        int r = 0;
        for (int base = 0; base < X; base += 64) {
            const int i = base + lane;
            r += __popcll(__ballot(i < X && needs_help(i)));
        }
        int seen = 0;
        for (int base = 0; base < BH; base += 64) {
            const unsigned long long m = __ballot(helper_cand(base + lane));
            const int c = __popcll(m);
            if (seen + c > r) return (int)s_first[base + kth_bit(m, r - seen)];
            seen += c;
        }
        return own_helper(X) ? (int)s_first[X] : -1;
    };
    auto helped_by = [&](int ww) -> int {      // the head workgroup ww helps, or -1
        int r = -1, seen = 0;
        for (int base = 0; base < BH; base += 64) {
            const int i = base + lane;
            const bool c = helper_cand(i);
            const unsigned long long m = __ballot(c);
            const unsigned long long me = __ballot(c && s_first[i] == (uint32_t)ww);
            if (me) {
                r = seen + __popcll(m & ((1ull << (__ffsll((long long)me) - 1)) - 1ull));
                break;
            }
            seen += __popcll(m);
        }
        if (r < 0) {
            // the first workgroup of a retrieval head that no gathered-rows
            // workgroup helps: its rank among those heads is at least the
            // number of gathered-rows helpers
            int ncand = 0;
            for (int base = 0; base < BH; base += 64) ncand += __popcll(__ballot(helper_cand(base + lane)));
            for (int base = 0, seen = 0; base < BH; base += 64) {
                const int i = base + lane;
                const bool nh = needs_help(i);
                const unsigned long long m = __ballot(nh);
                const unsigned long long me = __ballot(nh && s_first[i] == (uint32_t)ww && own_helper(i));
                if (me) {
                    const int bit = __ffsll((long long)me) - 1;
                    return seen + __popcll(m & ((1ull << bit) - 1ull)) >= ncand ? base + bit : -1;
                }
                seen += __popcll(m);
            }
            return -1;
        }
        for (int base = 0, seen = 0; base < BH; base += 64) {
            const unsigned long long m = __ballot(needs_help(base + lane));
            const int c = __popcll(m);
            if (seen + c > r) return base + kth_bit(m, r - seen);
            seen += c;
        }
        return -1;
    };
    LYCHEE_STAMP(kTrPrologue);
#ifdef LYCHEE_TRACE
    uint32_t tr_flags = 0, tr_heads = 0;
#endif

    // Classify the candidates this thread holds (slot e is candidate
    // base + tid + 256 e; slots from nslots on, or past C, hold none): key above
    // kab (the top of the threshold digit's range, raised to just under the
    // threshold rule's key floor) -> the bitmap bit if its index lies in the
    // slice [rlo, rlo + rlen), else counted in `below` if it lies under the slice; inside the digit's range -> the composite is appended to u.se.comp
    // at the position an LDS counter (s_ceq) hands out (the group is ranked by
    // value, so its order does not matter).  LDS operations cost per active
    // lane, so only the lanes with something to write issue them.
    auto classify_batch = [&](auto& vals, uint32_t nslots, uint32_t base, uint32_t C, uint32_t klo, uint32_t khi,
                              uint32_t kab, uint32_t rlo, uint32_t rlen, uint32_t& below) {
        constexpr int NB = (int)(sizeof(vals) / sizeof(vals[0]));
        static_assert(NB % 8 == 0 && NB <= 64, "slots come in groups of 8, at most 64");
        const uint32_t lim = C - base;
#pragma unroll
        for (int g8 = 0; g8 < NB; g8 += 8) {
            if ((uint32_t)g8 < nslots) {
#pragma unroll
                for (int e = g8; e < g8 + 8; ++e) {
                    const uint32_t key = (uint32_t)vals[e];
                    const uint32_t j = (uint32_t)(vals[e] >> 32) & kIdxMask;
                    const bool valid = tid + (uint32_t)(kAttendThreads * e) < lim;
                    const bool above = valid && key > kab;
                    const bool eq = valid && key - klo <= khi - klo;
                    if (above && j - rlo < rlen) atomicOr(&u.se.bits[(j - rlo) >> 5], 1u << (j & 31));
                    below += (above && j < rlo) ? 1u : 0u;
                    if (eq) {
                        const uint32_t at = atomicAdd(&s_ceq, 1u);
                        if (at < (uint32_t)kCandLds) u.se.comp[at] = composite(key, j);
                    }
                }
            }
        }
    };

    // Exact top-k of one retrieval head, for the slices [j0, j1) of its
    // context, by the full-scan path (force_fb: every key of the head re-read
    // from the score buffer; the fallback of fast_resolve below, for heads
    // whose candidates or threshold group exceed its LDS).  Slice j starts at
    // bitmap word j W / kResolveSlices, rounded down to 4 words.  Without
    // force_fb (not used by this kernel) the final first-digit histogram gives the threshold
    // digit T and the count above it; every key with digit >= T is in the
    // candidate list.  Every slice's resolver reads all of them and reaches the
    // same T and the same winners among the keys of digit T; it marks only the
    // winners inside its slice in the LDS bitmap, counts those below it (its
    // first position in S) and writes its part of S_out.  The resolver that
    // finishes reading the head's histogram and counters last, over all
    // slices, restores them to zero.
    auto resolve_topk = [&](int hb, int n, uint32_t ke, uint32_t C, uint32_t j0, uint32_t j1, bool force_fb) {
        int32_t* srow = p.S_out + (size_t)hb * p.k;
        const unsigned long long* cand = p.ws.cand + (size_t)hb * p.max_ctx;
        const uint32_t* sc = p.ws.score + (size_t)hb * p.max_ctx;
        uint32_t* gh = p.ws.hist + (size_t)hb * kHistBins;
        bool fb = false;           // reading every key instead of the candidates
        // candidate i of the list in use: (key, index) packed like the appends
        auto fetch = [&](uint32_t i) -> unsigned long long {
            return fb ? pack_cand(coherent_load(&sc[i]), i) : coherent_load(&cand[i]);
        };
        const uint32_t Wn = ((uint32_t)n + 31u) >> 5;       // bitmap words of the whole context
        auto slice_word = [&](uint32_t j) -> uint32_t {
            return j >= (uint32_t)kResolveSlices ? Wn : ((j * Wn) / (uint32_t)kResolveSlices) & ~3u;
        };
        const uint32_t wlo = slice_word(j0), whi = slice_word(j1);
        const uint32_t rlo = wlo * 32u, rlen = (whi - wlo) * 32u;
        const int W = (int)(whi - wlo);                      // bitmap words of the slices
        uint32_t below = 0;                                  // this thread's winners under the slices
        auto mark = [&](uint32_t j, uint32_t key) {          // winner j with selection key `key`
            if (key < p.sel_tkey) return;                    // under the threshold rule's floor
            if (j - rlo < rlen) atomicOr(&u.se.bits[(j - rlo) >> 5], 1u << (j & 31));
            below += j < rlo ? 1u : 0u;
        };
        // this resolver is done reading the head's histogram and counters
        auto release_head = [&]() {
            if (tid == 0) {
                const uint32_t cnt = j1 - j0;
                const uint32_t old = counter_add(&p.ws.rdone[hb], cnt);
                s_rel = old + cnt == (uint32_t)kResolveSlices;
                if (s_rel) {
                    counter_reset(&p.ws.rdone[hb]);
                    counter_reset64(&p.ws.selctr[hb]);
                    counter_reset(&p.ws.bmax[hb]);
                }
            }
            __syncthreads();
            if (s_rel)
                for (int i = tid; i < kHistBins; i += kAttendThreads) coherent_store(&gh[i], 0u);
        };
        __syncthreads();
        if (ke == (uint32_t)n && p.sel_tkey == 0u) {      // every token (the threshold rule still filters)
            release_head();
            for (uint32_t i = rlo + tid; i < min(rlo + rlen, (uint32_t)n); i += kAttendThreads) put_s(srow, i, (int32_t)i);
            if (whi == Wn)
                for (int i = n + tid; i < p.k; i += kAttendThreads) put_s(srow, i, -1);
        } else {
            constexpr int RC = 32;     // candidate slots per thread in the first load (8192 per head; fewer registers)
            constexpr int kB = 16;     // batch of later candidates
            // one round of loads: the head's histogram, the candidates (C came
            // with the arrival that made this workgroup the last one) and the
            // largest bound used
            C = max(1u, min(C, (uint32_t)p.max_ctx));
            if (tid == 0) s_ceq = 0u;        // (ordered before the classification by the crossing's barriers)
            const uint32_t nslots = min((C + kAttendThreads - 1) / kAttendThreads, (uint32_t)RC);
            const uint32_t bmaxv = coherent_load(&p.ws.bmax[hb]);
            uint32_t gv[kHistPerThread];
#pragma unroll
            for (int j = 0; j < kHistPerThread; ++j) gv[j] = coherent_load(&gh[tid + kAttendThreads * j]);
            unsigned long long cv[RC];
#pragma unroll
            for (int e = 0; e < RC; ++e) {
                cv[e] = 0ull;
                if ((uint32_t)e < nslots) cv[e] = coherent_load(&cand[min(tid + (uint32_t)(kAttendThreads * e), C - 1u)]);
            }
#pragma unroll
            for (int j = 0; j < kHistPerThread; ++j) u.se.h12[tid + kAttendThreads * j] = gv[j];
            {
                const int W4 = (W + 3) >> 2;
                uint4* b4 = reinterpret_cast<uint4*>(u.se.bits);
                for (int i = tid; i < W4; i += kAttendThreads) b4[i] = make_uint4(0u, 0u, 0u, 0u);
            }
            auto hist_rest = [&](uint32_t from, uint32_t cnt) {    // candidates [from, cnt) from memory
                for (uint32_t base = from; base < cnt; base += kAttendThreads * kB) {
                    unsigned long long bv[kB];
#pragma unroll
                    for (int e = 0; e < kB; ++e) bv[e] = fetch(min(base + tid + (uint32_t)(kAttendThreads * e), cnt - 1u));
#pragma unroll
                    for (int e = 0; e < kB; ++e) {
                        const bool valid = base + tid + (uint32_t)(kAttendThreads * e) < cnt;
                        atomicAdd(&u.se.h12[valid ? key_digit((uint32_t)bv[e]) : 0u], valid ? 1u : 0u);
                    }
                }
            };
            __syncthreads();
            auto crossing12 = [&]() {
                uint32_t hc[kHistPerThread];
                // thread t takes descending ranks 16t.. = bins 4095-16t down to 4080-16t
                const uint4* hv = reinterpret_cast<const uint4*>(u.se.h12 + kHistBins - kHistPerThread * (tid + 1));
#pragma unroll
                for (int c = 0; c < kHistPerThread / 4; ++c) {
                    const uint4 v4 = hv[c];
                    hc[kHistPerThread - 1 - 4 * c] = v4.x;
                    hc[kHistPerThread - 2 - 4 * c] = v4.y;
                    hc[kHistPerThread - 3 - 4 * c] = v4.z;
                    hc[kHistPerThread - 4 - 4 * c] = v4.w;
                }
                block_crossing<kHistPerThread>(hc, kHistBins, ke, s_wave, s_res);
            };
            crossing12();
            uint32_t T_ = s_res[0];
            uint32_t c_above = s_res[1];
            // Every pass added its counts and appended its keys from its bound
            // up, and every bound is <= bmax.  If bmax <= T, the histogram is
            // exact from T up and the candidates hold every key from T up, so T
            // is the head's threshold digit.  Otherwise a pass held more than its
            // margin of the head's top keys: count and use every key instead.
            fb = force_fb || bmaxv > T_;
            release_head();
            uint32_t Cs = C;
            if (fb) {
                Cs = (uint32_t)n;
                __syncthreads();
                for (int i = tid; i < kHistBins; i += kAttendThreads) u.se.h12[i] = 0u;
                __syncthreads();
                hist_rest(0u, Cs);
                __syncthreads();
                crossing12();
                T_ = s_res[0];
                c_above = s_res[1];
            }
            const uint32_t klo = (uint32_t)digit_first_key(T_);              // key range of digit T
            const uint32_t khi = (uint32_t)(digit_first_key(T_ + 1u) - 1ull);
            // key of a composite of digit T (the digit's keys share their bits above kLowBits)
            auto comp_key = [&](unsigned long long cp) -> uint32_t {
                return (klo & ~((1u << kLowBits) - 1u)) | (uint32_t)(cp >> kIdxBits);
            };
            const uint32_t kab = p.sel_tkey ? max(khi, p.sel_tkey - 1u) : khi;   // winners above the digit
            if (!fb) classify_batch(cv, nslots, 0u, C, klo, khi, kab, rlo, rlen, below);
            for (uint32_t base = fb ? 0u : kAttendThreads * RC; base < Cs; base += kAttendThreads * kB) {
                unsigned long long bv[kB];
#pragma unroll
                for (int e = 0; e < kB; ++e) bv[e] = fetch(min(base + tid + (uint32_t)(kAttendThreads * e), Cs - 1u));
                classify_batch(bv, (uint32_t)kB, base, Cs, klo, khi, kab, rlo, rlen, below);
            }
            __syncthreads();
            uint32_t c_left = s_ceq;          // keys of digit T appended
            uint32_t r_left = ke - c_above;
            int shift = kCompBits;
            bool done = (r_left == 0u);
            if (!done && c_left > (uint32_t)kCandLds) {
                // Too many ties with the threshold digit for LDS: narrow by passes
                // over the candidate list, each fixing the next 8 bits (prefix) of
                // the composite of the k-th element.
                unsigned long long prefix = 0;
                while (!done && c_left > (uint32_t)kCandLds && shift > 0) {
                    const int bits = shift >= 8 ? 8 : shift;
                    const int nshift = shift - bits;
                    for (int i = tid; i < 256; i += kAttendThreads) u.se.h[i] = 0u;
                    __syncthreads();
                    for (uint32_t base = 0; base < Cs; base += kAttendThreads * kB) {
                        unsigned long long bv[kB];
#pragma unroll
                        for (int e = 0; e < kB; ++e) bv[e] = fetch(min(base + tid + (uint32_t)(kAttendThreads * e), Cs - 1u));
#pragma unroll
                        for (int e = 0; e < kB; ++e) {
                            if (base + tid + (uint32_t)(kAttendThreads * e) >= Cs) continue;
                            const uint32_t key = (uint32_t)bv[e], j = (uint32_t)(bv[e] >> 32);
                            if (key - klo > khi - klo) continue;
                            const unsigned long long cp = composite(key, j);
                            if (shift < kCompBits && (cp >> shift) != prefix) continue;
                            atomicAdd(&u.se.h[comp_digit(cp, nshift, bits)], 1u);
                        }
                    }
                    __syncthreads();
                    uint32_t hb1[1] = {tid < (1 << bits) ? u.se.h[(1 << bits) - 1 - tid] : 0u};
                    block_crossing<1>(hb1, 1 << bits, r_left, s_wave, s_res);
                    const uint32_t Dg = min(s_res[0], (1u << bits) - 1u), gt = s_res[1];
                    const uint32_t keep = u.se.h[Dg];
                    for (uint32_t base = 0; base < Cs; base += kAttendThreads * kB) {
                        unsigned long long bv[kB];
#pragma unroll
                        for (int e = 0; e < kB; ++e) bv[e] = fetch(min(base + tid + (uint32_t)(kAttendThreads * e), Cs - 1u));
#pragma unroll
                        for (int e = 0; e < kB; ++e) {
                            if (base + tid + (uint32_t)(kAttendThreads * e) >= Cs) continue;
                            const uint32_t key = (uint32_t)bv[e], j = (uint32_t)(bv[e] >> 32);
                            if (key - klo > khi - klo) continue;
                            const unsigned long long cp = composite(key, j);
                            if (shift < kCompBits && (cp >> shift) != prefix) continue;
                            const uint32_t dg = comp_digit(cp, nshift, bits);
                            if (dg > Dg || (r_left - gt == keep && dg == Dg)) mark(j, key);
                        }
                    }
                    __syncthreads();
                    r_left -= gt;
                    c_left = keep;
                    prefix = (prefix << bits) | Dg;
                    shift = nshift;
                    if (r_left == 0u || r_left == c_left) done = true;
                }
                if (!done) {
                    // the k-th element's prefix group now fits in LDS: gather it
                    uint32_t c_pre = 0;
                    for (uint32_t base = 0; base < Cs; base += kAttendThreads * kB) {
                        unsigned long long bv[kB];
                        unsigned long long cpv[kB];
#pragma unroll
                        for (int e = 0; e < kB; ++e) bv[e] = fetch(min(base + tid + (uint32_t)(kAttendThreads * e), Cs - 1u));
                        unsigned long long m = 0;
#pragma unroll
                        for (int e = 0; e < kB; ++e) {
                            const uint32_t key = (uint32_t)bv[e], j = (uint32_t)(bv[e] >> 32);
                            cpv[e] = composite(key, j);
                            if (base + tid + (uint32_t)(kAttendThreads * e) < Cs && key - klo <= khi - klo &&
                                (cpv[e] >> shift) == prefix)
                                m |= 1ull << e;
                        }
                        uint32_t tot;
                        uint32_t pos = c_pre + block_exclusive_scan((uint32_t)__popcll(m), s_wave, &tot);
#pragma unroll
                        for (int e = 0; e < kB; ++e) {
                            if ((m >> e) & 1ull) {
                                if (pos < (uint32_t)kCandLds) u.se.comp[pos] = cpv[e];
                                ++pos;
                            }
                        }
                        c_pre += tot;
                    }
                    __syncthreads();
                    c_left = min(c_pre, (uint32_t)kCandLds);
                }
            }
            if (!done && r_left == c_left) {   // the whole threshold group is selected
                for (uint32_t i = tid; i < c_left; i += kAttendThreads) {
                    const unsigned long long cp = u.se.comp[i];
                    mark(comp_index(cp), comp_key(cp));
                }
                done = true;
            }
            // radix select in LDS over the remaining composite bits; a group of
            // at most 256 is finished by direct rank, one composite per thread
            // counted against all of them (wavefront-uniform LDS reads)
            while (!done) {
                if (c_left <= (uint32_t)kAttendThreads) {
                    const unsigned long long mine = u.se.comp[min((uint32_t)tid, c_left - 1u)];
                    uint32_t above = 0;
                    for (uint32_t r = 0; r < c_left; ++r) above += u.se.comp[r] > mine;
                    if ((uint32_t)tid < c_left && above < r_left) mark(comp_index(mine), comp_key(mine));
                    done = true;
                    break;
                }
                if (shift == 0) {             // unreachable: composites are distinct
                    if (tid == 0) atomicOr(p.ws.err, 2u);
                    break;
                }
                const int bits = shift >= 8 ? 8 : shift;
                shift -= bits;
                for (int i = tid; i < 256; i += kAttendThreads) u.se.h[i] = 0u;
                __syncthreads();
                unsigned long long mine[kCandPerThread];
                uint32_t dg[kCandPerThread];
                const uint32_t nsl = (c_left + kAttendThreads - 1) / kAttendThreads;
#pragma unroll
                for (int e = 0; e < kCandPerThread; ++e) {
                    const uint32_t i = tid + (uint32_t)(kAttendThreads * e);
                    mine[e] = 0ull;
                    dg[e] = 0xFFFFFFFFu;
                    if ((uint32_t)e < nsl) {
                        mine[e] = u.se.comp[min(i, (uint32_t)kCandLds - 1u)];
                        const bool valid = i < c_left;
                        dg[e] = valid ? comp_digit(mine[e], shift, bits) : 0xFFFFFFFFu;
                        atomicAdd(&u.se.h[valid ? dg[e] : 0u], valid ? 1u : 0u);
                    }
                }
                __syncthreads();
                uint32_t hb1[1] = {tid < (1 << bits) ? u.se.h[(1 << bits) - 1 - tid] : 0u};
                block_crossing<1>(hb1, 1 << bits, r_left, s_wave, s_res);
                const uint32_t Dg = min(s_res[0], (1u << bits) - 1u), gt = s_res[1];
                const uint32_t keep = u.se.h[Dg];
                uint32_t m = 0;
#pragma unroll
                for (int e = 0; e < kCandPerThread; ++e) {
                    if ((uint32_t)e < nsl) {
                        const bool sel = dg[e] != 0xFFFFFFFFu && dg[e] > Dg;
                        if (sel) mark(comp_index(mine[e]) & kIdxMask, comp_key(mine[e]));
                        m |= (uint32_t)(dg[e] == Dg) << e;
                    }
                }
                uint32_t tot;
                uint32_t pos = block_exclusive_scan((uint32_t)__popc(m), s_wave, &tot);
#pragma unroll
                for (int e = 0; e < kCandPerThread; ++e) {
                    if ((uint32_t)e < nsl) {
                        const bool is = (m >> e) & 1u;
                        u.se.comp[is ? pos : (uint32_t)(kCandLds + tid)] = mine[e];
                        pos += is;
                    }
                }
                __syncthreads();
                r_left -= gt;
                c_left = keep;
                if (r_left == 0u) {
                    done = true;
                } else if (r_left == c_left) {
                    for (uint32_t i = tid; i < c_left; i += kAttendThreads) {
                        const unsigned long long cp = u.se.comp[i];
                        mark(comp_index(cp), comp_key(cp));
                    }
                    done = true;
                }
                __syncthreads();
            }
            __syncthreads();
            // Emit S in ascending order.  Wavefront v owns the bitmap words
            // [v WPW, (v+1) WPW): it counts them, takes its base from the counts
            // of the wavefronts before it (block scan), then walks them 256 at a
            // time, four consecutive words per lane (16-byte LDS reads); a
            // wavefront scan of the lanes' bit counts gives each lane its first
            // position, so a wavefront's stores are nearly consecutive.
            constexpr int kMaxSteps = kWords / (kWaves * 256);
            const int WPW = ((W + kWaves * 256 - 1) / (kWaves * 256)) * 256;
            const int wb = wave * WPW, we = min(W, wb + WPW);
            const uint4* b4 = reinterpret_cast<const uint4*>(u.se.bits);
            uint32_t cnt = 0;
#pragma unroll
            for (int st = 0; st < kMaxSteps; ++st) {
                const int i = wb + st * 256 + lane * 4;
                if (st * 256 < WPW && i < we) {
                    const uint4 v = b4[i >> 2];
                    cnt += __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
                }
            }
            uint32_t below_total;
            (void)block_exclusive_scan(below, s_wave, &below_total);   // winners under the slices
            uint32_t total;
            uint32_t pos = block_exclusive_scan(cnt, s_wave, &total);   // this lane's words come first...
            pos = below_total + __builtin_amdgcn_readfirstlane(pos);    // ...lane 0's base is the wavefront's
            const uint32_t last = (uint32_t)p.k - 1u;
            for (int i0 = wb; i0 < we; i0 += 256) {
                const int i = i0 + lane * 4;
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (i < we) v = b4[i >> 2];
                const uint32_t c = __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
                const uint32_t incl = wave_inclusive_scan(c);
                uint32_t at = pos + incl - c;
                pos += __builtin_amdgcn_readlane(incl, 63);
                uint32_t wq[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t bw = wq[q];
                    while (bw) {
                        const int bit = __ffs(bw) - 1;
                        bw &= bw - 1u;
                        put_s(srow, min(at, last), (int32_t)(rlo + (uint32_t)((i + q) * 32 + bit)));   // at < ke unless the counts disagree (flagged below)
                        ++at;
                    }
                }
            }
            if (whi == Wn) {           // the slice holding the end of the context
                // (the threshold rule keeps the winners at or above its floor)
                const uint32_t kept = p.sel_tkey ? min(below_total + total, ke) : ke;
                for (int i = (int)kept + tid; i < p.k; i += kAttendThreads) put_s(srow, i, -1);
                if (tid == 0 && (p.sel_tkey ? below_total + total > ke : below_total + total != ke))
                    atomicOr(p.ws.err, 2u);
            }
        }
        __syncthreads();
    };

    // Crossing of the LDS histogram u.se.h12 at `need` (see block_crossing).
    auto crossing_h12 = [&](uint32_t need) {
        uint32_t hc[kHistPerThread];
        // thread t takes descending ranks 16t.. = bins 4095-16t down to 4080-16t
        const uint4* hv = reinterpret_cast<const uint4*>(u.se.h12 + kHistBins - kHistPerThread * (tid + 1));
#pragma unroll
        for (int c = 0; c < kHistPerThread / 4; ++c) {
            const uint4 v4 = hv[c];
            hc[kHistPerThread - 1 - 4 * c] = v4.x;
            hc[kHistPerThread - 2 - 4 * c] = v4.y;
            hc[kHistPerThread - 3 - 4 * c] = v4.z;
            hc[kHistPerThread - 4 - 4 * c] = v4.w;
        }
        block_crossing<kHistPerThread>(hc, kHistBins, need, s_wave, s_res);
    };

    // Exact top-k of one retrieval head (Eq. 2: the k_eff largest pooled
    // scores, ties to the lower token index), resolved by the head's last
    // selection arrival from the candidates the head's workgroups appended
    // (each in its own region, in position order, with its candidate count
    // and largest pass bound in its word):
    //  1. the head's histogram and the words in one round of loads; the
    //     crossing at k_eff gives the threshold digit T.  A workgroup whose
    //     bound lies above T kept too few keys and left its counts in
    //     [T, bound) out of the histogram: its rows are re-read from the
    //     score buffer and counted, and the crossing is taken again -- exact
    //     now, since every key of digit >= T is counted -- and its keys from
    //     the final T up replace its candidates;
    //  2. the candidates, workgroup after workgroup (so in position order),
    //     are gathered kFastBatch at a time: a map gives each flat entry its
    //     row, every thread loads its kFastPer entries at once and writes
    //     them to LDS lane-consecutively, and the keys of digit T are
    //     collected as composites (rest of the key, then the inverted index);
    //  3. the cut: the (k_eff - count above T)-th largest composite;
    //  4. an ordered compaction of each batch: ballots count the winners of
    //     every (step, wavefront), one block scan gives each its first
    //     position, and the winners are written in flat order.
    // The code runs once per head and launch: loads are issued in batches
    // (one round trip each) and the loops stay rolled elsewhere.  Heads whose
    // threshold-digit keys overflow kFastGroup return true and take
    // resolve_topk's full scan instead (from the caller's single call site,
    // so that both stay inlined and the kernel's parameters stay in
    // registers).
    auto fast_resolve = [&](int hb, int n, uint32_t ke, uint32_t h0, int wf, int nw) -> bool {
        int32_t* srow = p.S_out + (size_t)hb * p.k;
        const unsigned long long* cand = p.ws.cand + (size_t)hb * p.max_ctx;
        const uint32_t* sc = p.ws.score + (size_t)hb * p.max_ctx;
        uint32_t* gh = p.ws.hist + (size_t)hb * kHistBins;
        const uint32_t hh1 = h0 + kCostRetrieval * (uint32_t)n;   // the head's end on the cost axis
        uint32_t* s_wm = u.fr.wm;
        uint32_t* s_coff = u.fr.coff;
        auto rows_of = [&](int i, uint32_t& r0, uint32_t& r1) {   // rows of the head's i-th workgroup
            r0 = (max(s_bound[wf + i], h0) - h0) / kCostRetrieval;
            r1 = (min(s_bound[wf + i + 1], hh1) - h0) / kCostRetrieval;
        };
        if (TOPP && tid == 0) s_lds_set = 0u;
        __syncthreads();
        // 1. histogram (restored to zero once read) and words
        {
            uint32_t gv[kHistPerThread];                         // every load in flight at once
#pragma unroll
            for (int j = 0; j < kHistPerThread; ++j) gv[j] = coherent_load(&gh[tid + kAttendThreads * j]);
            constexpr int WPT = kMaxWG / kAttendThreads;
            uint32_t wv[WPT];
#pragma unroll
            for (int e = 0; e < WPT; ++e) {
                const int i = tid + kAttendThreads * e;
                wv[e] = i < nw ? coherent_load(&p.ws.wmeta[wf + i + hb]) : 0u;
            }
#pragma unroll
            for (int j = 0; j < kHistPerThread; ++j) {
                u.fr.h12[tid + kAttendThreads * j] = gv[j];
                coherent_store(&gh[tid + kAttendThreads * j], 0u);
            }
#pragma unroll
            for (int e = 0; e < WPT; ++e) {
                const int i = tid + kAttendThreads * e;
                if (i < nw) s_wm[i] = wv[e];
            }
        }
        if (ke == (uint32_t)n && p.sel_tkey == 0u) {          // every token
            for (uint32_t i = tid; i < (uint32_t)n; i += kAttendThreads) put_s(srow, i, (int32_t)i);
            for (int i = n + tid; i < p.k; i += kAttendThreads) put_s(srow, i, -1);
            __syncthreads();
            return false;
        }
        __syncthreads();
        LYCHEE_STAMP(kTrResolve0 + 0);
        auto crossing = [&]() {
            uint32_t hc[kHistPerThread];
            // thread t takes descending ranks 16t.. = bins 4095-16t down to 4080-16t
            const uint4* hv = reinterpret_cast<const uint4*>(u.fr.h12 + kHistBins - kHistPerThread * (tid + 1));
#pragma unroll
            for (int c = 0; c < kHistPerThread / 4; ++c) {
                const uint4 v4 = hv[c];
                hc[kHistPerThread - 1 - 4 * c] = v4.x;
                hc[kHistPerThread - 2 - 4 * c] = v4.y;
                hc[kHistPerThread - 3 - 4 * c] = v4.z;
                hc[kHistPerThread - 4 - 4 * c] = v4.w;
            }
            block_crossing<kHistPerThread>(hc, kHistBins, ke, s_wave, s_res);
        };
        // the workgroups whose bound lies above Tc, listed in s_coff (free
        // until the offsets are taken)
        auto list_failing = [&](uint32_t Tc) -> uint32_t {
            uint32_t nf = 0;
            for (int i0 = 0; i0 < nw; i0 += kAttendThreads) {
                const int i = i0 + tid;
                const bool f = i < nw && (s_wm[i] >> 20) > Tc;
                uint32_t tot;
                const uint32_t pos = nf + block_exclusive_scan((uint32_t)f, s_wave, &tot);
                if (f) s_coff[pos] = (uint32_t)i;
                nf += tot;
            }
            __syncthreads();
            return nf;
        };
        crossing();
        uint32_t Td = s_res[0], c_above = s_res[1];
        const uint32_t nfail = list_failing(Td);
        if (__builtin_expect(nfail != 0u, 0)) {
            // counts in [T, bound) of the workgroups whose bound lies above T
            for (uint32_t q = 0; q < nfail; ++q) {               // (uniform loop)
                const int i = (int)s_coff[q];
                const uint32_t bi = s_wm[i] >> 20;
                uint32_t r0, r1;
                rows_of(i, r0, r1);
#pragma unroll 8
                for (uint32_t j = r0 + tid; j < r1; j += kAttendThreads) {
                    const uint32_t d = key_digit(coherent_load(&sc[j]));
                    if (d >= Td && d < bi) atomicAdd(&u.fr.h12[d], 1u);
                }
            }
            __syncthreads();
            crossing();
            Td = s_res[0];
            c_above = s_res[1];
            // their keys from the final T up replace their candidates (the
            // added counts lie at digits >= T, so the final T is at least the
            // first and the list holds every workgroup whose bound is above it)
            const uint32_t kb = (uint32_t)digit_first_key(Td);
            unsigned long long* cw = p.ws.cand + (size_t)hb * p.max_ctx;
            for (uint32_t q = 0; q < nfail; ++q) {               // (uniform loop)
                const int i = (int)s_coff[q];
                if ((s_wm[i] >> 20) <= Td) continue;
                uint32_t r0, r1;
                rows_of(i, r0, r1);
                uint32_t written = 0;
                for (uint32_t base = r0; base < r1; base += kAttendThreads * 8) {
                    uint32_t m8 = 0, kv[8];
                    for (int e = 0; e < 8; ++e) {                // thread t: rows base + 8t .. 8t + 7
                        const uint32_t j = base + 8u * (uint32_t)tid + (uint32_t)e;
                        kv[e] = j < r1 ? coherent_load(&sc[j]) : 0u;
                        m8 |= (uint32_t)(j < r1 && kv[e] >= kb) << e;
                    }
                    uint32_t tot;
                    uint32_t at = written + block_exclusive_scan((uint32_t)__popc(m8), s_wave, &tot);
                    for (int e = 0; e < 8; ++e)
                        if ((m8 >> e) & 1u) coherent_store(&cw[r0 + at++], pack_cand(kv[e], base + 8u * (uint32_t)tid + (uint32_t)e));
                    written += tot;
                }
                if (tid == 0) s_wm[i] = written | (Td << 20);
                __syncthreads();
            }
            wait_stores_complete();
            __syncthreads();
            LYCHEE_STAMP(kTrResolve0 + 2);
        }
        LYCHEE_STAMP(kTrResolve0 + 1);
        // 2. candidates: flat offsets of the workgroups' runs
        uint32_t C;
        {
            uint32_t mine = 0;
            const int per = (nw + kAttendThreads - 1) / kAttendThreads;   // contiguous per thread
            for (int e = 0; e < per; ++e) {
                const int i = tid * per + e;
                mine += i < nw ? (s_wm[i] & 0xFFFFFu) : 0u;
            }
            uint32_t at = block_exclusive_scan(mine, s_wave, &C);
            for (int e = 0; e < per; ++e) {
                const int i = tid * per + e;
                if (i < nw) {
                    s_coff[i] = at;
                    at += s_wm[i] & 0xFFFFFu;
                }
            }
            if (tid == 0) s_coff[nw] = C;
            if (tid == 0) s_ceq = 0u;
        }
        __syncthreads();
        LYCHEE_STAMP(kTrResolve0 + 5);
        LYCHEE_TRACE_SET(13, (unsigned long long)C | ((unsigned long long)Td << 32));
        const uint32_t klo = (uint32_t)digit_first_key(Td);       // key range of digit T
        const uint32_t khi = (uint32_t)(digit_first_key(Td + 1u) - 1ull);
        const uint32_t tkey = p.sel_tkey;
        const uint32_t nbatch = (C + kFastBatch - 1u) / kFastBatch;
        const uint32_t last = (uint32_t)p.k - 1u;
        const unsigned long long lt_mask = (1ull << lane) - 1ull;   // lanes below this one
        unsigned long long cut = 0ull;                            // winners: full_order >= cut
        uint32_t total = 0;
        // Entry f of a batch (flat order) sits at LDS slot f = 256 j + tid:
        // thread t holds entries t, t + 256, .. (kFastPer of them), so every
        // LDS access below is lane-consecutive.  Pass 0 gathers each batch
        // and collects the threshold digit's composites, then takes the cut;
        // pass 1 emits the winners of each batch in flat order (gathering
        // again only when there is more than one batch).
        for (int pass = 0; pass < 2; ++pass) {
            for (uint32_t bb = 0; bb < nbatch; ++bb) {
                const uint32_t b0 = bb * (uint32_t)kFastBatch, len = min((uint32_t)kFastBatch, C - b0);
                if (pass == 0 || nbatch > 1u) {
                    // source row of every entry: tpp threads write each
                    // workgroup's run (more threads per run when there are
                    // fewer runs), four entries a step each
                    {
                        const int tpp = nw >= kAttendThreads / 2 ? 1 : (nw >= kAttendThreads / 4 ? 2 : (nw >= kAttendThreads / 8 ? 4 : 8));
                        const int sub = tid & (tpp - 1);
                        for (int i = tid / tpp; i < nw; i += kAttendThreads / tpp) {
                            const uint32_t ci = s_coff[i];
                            const uint32_t f0 = max(ci, b0), f1 = max(f0, min(s_coff[i + 1], b0 + len));
                            const uint32_t r = (max(s_bound[wf + i], h0) - h0) / kCostRetrieval + (f0 - ci);
                            uint32_t f = f0 + (uint32_t)sub;
                            for (; f + 3u * (uint32_t)tpp < f1; f += 4u * (uint32_t)tpp) {
                                u.fr.map[f - b0] = r + (f - f0);
                                u.fr.map[f + (uint32_t)tpp - b0] = r + (f + (uint32_t)tpp - f0);
                                u.fr.map[f + 2u * (uint32_t)tpp - b0] = r + (f + 2u * (uint32_t)tpp - f0);
                                u.fr.map[f + 3u * (uint32_t)tpp - b0] = r + (f + 3u * (uint32_t)tpp - f0);
                            }
                            for (; f < f1; f += (uint32_t)tpp) u.fr.map[f - b0] = r + (f - f0);
                        }
                    }
                    __syncthreads();
                    // all kFastPer loads in flight at once (straight-line code
                    // kept short: reads, loads, writes; rows past the batch
                    // load the head's first entry, unused)
                    // (the keys of digit T flagged on the way: bit j of mm)
                    uint32_t mm = 0;
                    {
                        uint32_t at[kFastPer];
#pragma unroll
                        for (int j = 0; j < kFastPer; ++j) at[j] = u.fr.map[kAttendThreads * j + tid];
                        unsigned long long e[kFastPer];
#pragma unroll
                        for (int j = 0; j < kFastPer; ++j)
                            e[j] = coherent_load(&cand[kAttendThreads * j + tid < len ? at[j] : 0u]);
#pragma unroll
                        for (int j = 0; j < kFastPer; ++j) {
                            const uint32_t key = (uint32_t)e[j];
                            u.fr.key[kAttendThreads * j + tid] = key;
                            u.fr.idx[kAttendThreads * j + tid] = (uint32_t)(e[j] >> 32);
                            mm |= (uint32_t)(kAttendThreads * j + tid < len && key - klo <= khi - klo) << j;
                        }
                    }
                    LYCHEE_STAMP(kTrResolve0 + 10);
                    if (pass == 0) {
                        // keys of digit T (own entries only: no barrier needed
                        // before reading them back), placed by one block scan
                        uint32_t gtot;
                        uint32_t q = s_ceq + block_exclusive_scan((uint32_t)__popc(mm), s_wave, &gtot);
                        while (mm) {
                            const int j = __builtin_ctz(mm);
                            mm &= mm - 1u;
                            const uint32_t f = kAttendThreads * j + tid;
                            if (q < (uint32_t)kFastGroup) u.fr.comp[q] = full_order(u.fr.key[f], u.fr.idx[f]);
                            ++q;
                        }
                        __syncthreads();
                        if (tid == 0) s_ceq += gtot;
                    }
                    __syncthreads();
                    LYCHEE_STAMP(kTrResolve0 + 8);
                }
                if (pass == 0) continue;
                // One pass: wavefront v compacts the winners of its quarter
                // of the batch (64 consecutive entries per step, ballot ranks,
                // a running count) into its part of u.fr.map; the four counts
                // then place the quarters, copied to S in order.
                {
                    constexpr uint32_t kQ = kFastBatch / kWaves;
                    uint32_t* sbuf = u.fr.map + (uint32_t)wave * kQ;
                    const uint32_t f0 = min((uint32_t)wave * kQ, len), f1 = min(f0 + kQ, len);
                    uint32_t wcnt = 0;
#pragma unroll 1
                    for (uint32_t f = f0; f < f1; f += 64u * 8u) {
                        uint32_t kk[8], ii[8];
#pragma unroll
                        for (int e2 = 0; e2 < 8; ++e2) {
                            const uint32_t fl = f + 64u * e2 + (uint32_t)lane;
                            kk[e2] = u.fr.key[fl];
                            ii[e2] = u.fr.idx[fl];
                        }
#pragma unroll
                        for (int e2 = 0; e2 < 8; ++e2) {
                            const uint32_t fl = f + 64u * e2 + (uint32_t)lane;
                            const bool wv = fl < f1 && full_order(kk[e2], ii[e2]) >= cut;
                            const unsigned long long bw = __ballot(wv);
                            // (the Top-p build keeps the entry, so the set's keys stay at hand)
                            if (wv) sbuf[wcnt + (uint32_t)__popcll(bw & lt_mask)] = TOPP ? fl : ii[e2];
                            wcnt += (uint32_t)__popcll(bw);
                        }
                    }
                    if (lane == 0) u.fr.jc[wave] = wcnt;
                    __syncthreads();
                    LYCHEE_STAMP(kTrResolve0 + 9);
                    uint32_t base = 0, tot = 0;
#pragma unroll
                    for (int v = 0; v < kWaves; ++v) {
                        const uint32_t c = u.fr.jc[v];
                        base += v < wave ? c : 0u;
                        tot += c;
                    }
                    for (uint32_t i = (uint32_t)lane; i < wcnt; i += 64u)
                        put_s(srow, min(total + base + i, last), (int32_t)(TOPP ? u.fr.idx[sbuf[i]] : sbuf[i]));
                    total += tot;
                    __syncthreads();
                }
            }
            if (pass == 1) break;
            LYCHEE_STAMP(kTrResolve0 + 3);
            const uint32_t g = s_ceq;
            LYCHEE_TRACE_SET(14, (unsigned long long)g | ((unsigned long long)c_above << 32));
            LYCHEE_TRACE_SET(15, (unsigned long long)ke | ((unsigned long long)nw << 32));
            if (g > (uint32_t)kFastGroup || c_above > ke || ke - c_above > g) {
                // more keys of digit T than LDS holds (or counts that disagree): full scan
                __syncthreads();
                return true;
            }
            // the cut among digit T: the r_left-th largest composite (winners >= cut)
            const uint32_t r_left = ke - c_above;
            if (r_left == 0u) {                                    // none of digit T
                cut = khi == 0xFFFFFFFFu ? ~0ull : (unsigned long long)(khi + 1u) << 32;
            } else if (r_left == g) {                              // all of digit T
                cut = (unsigned long long)klo << 32;
            } else {
                // rank every value against all: lane l ranks values l, l + 64,
                // .. and wavefront v counts over the v-th quarter of the
                // values (8 read per round trip); the four partial counts
                // meet in u.fr.map (free between the gathers)
                uint32_t* rank = u.fr.map;
                for (uint32_t q0 = tid; q0 < g; q0 += kAttendThreads) rank[q0] = 0u;
                __syncthreads();
                const uint32_t qs = (g + kWaves - 1u) / kWaves;
                const uint32_t qa = min(g, (uint32_t)wave * qs), qb = min(g, qa + qs);
                for (uint32_t q0 = (uint32_t)lane; q0 < g; q0 += 64u) {
                    const unsigned long long mine = u.fr.comp[q0];
                    uint32_t above = 0, q = qa;
                    for (; q + 8u <= qb; q += 8u) {
                        unsigned long long c8[8];
#pragma unroll
                        for (int e2 = 0; e2 < 8; ++e2) c8[e2] = u.fr.comp[q + e2];
#pragma unroll
                        for (int e2 = 0; e2 < 8; ++e2) above += c8[e2] > mine;
                    }
                    for (; q < qb; ++q) above += u.fr.comp[q] > mine;
                    if (above) atomicAdd(&rank[q0], above);
                }
                __syncthreads();
                for (uint32_t q0 = tid; q0 < g; q0 += kAttendThreads)
                    if (rank[q0] == r_left - 1u) s_cut = u.fr.comp[q0];
                __syncthreads();
                cut = s_cut;
            }
            // the threshold rule keeps no key below tkey
            cut = max(cut, (unsigned long long)tkey << 32);
            LYCHEE_STAMP(kTrResolve0 + 4);
        }
        LYCHEE_STAMP(kTrResolve0 + 6);
        // padding after the kept tokens; the count must be k_eff (at most that
        // under the threshold rule)
        const uint32_t kept = min(total, ke);
        for (int i = (int)kept + tid; i < p.k; i += kAttendThreads) put_s(srow, i, -1);
        if (tid == 0 && (tkey ? total > ke : total != ke)) atomicOr(p.ws.err, 2u);
        // one batch: its winners' entries stay in u.fr.map (wavefront v's at
        // v kFastBatch / kWaves, u.fr.jc[v] of them) beside their keys and
        // indices in u.fr.key / u.fr.idx, in the order of S
        if (TOPP && tid == 0) s_lds_set = (nbatch == 1u && total == ke) ? 1u : 0u;
        __syncthreads();
        LYCHEE_STAMP(kTrResolve0 + 7);
        return false;
    };

    // The block rule (blocks of bs = 2^sel_block tokens, a block scored by the
    // largest selection key of its tokens): the floor(k / bs) highest blocks,
    // ties to the lower block, their tokens listed ascending in S (a short last
    // block is the highest kept one, so its missing tokens fall at the end).
    // Every pass folded its blocks' largest keys into the head's block words;
    // the head's last selection arrival (or its helper) reads them here,
    // restores them to zero, and cuts on full_order(word, block):
    // 1. the words to LDS and their first digits to a histogram; the crossing
    //    at floor(k / bs) gives the threshold digit T and the count above it;
    // 2. the cut within digit T: by counting ranks when T holds at most
    //    kFastGroup blocks, else by 12-bit radix passes over the composites of
    //    T (a composite prefix: a digit is an aligned key range);
    // 3. one block scan lists the kept blocks ascending; S is written from
    //    the list.
    auto block_resolve = [&](int hb, int n) __attribute__((always_inline)) {
        int32_t* srow = p.S_out + (size_t)hb * p.k;
        uint32_t* bk = p.ws.bkey + (size_t)hb * (size_t)p.bkey_stride;
        const uint32_t bsh = p.sel_block;
        const uint32_t nb = ((uint32_t)n + (1u << bsh) - 1u) >> bsh;
        const uint32_t m = min((uint32_t)p.k >> bsh, nb);               // blocks kept
        __syncthreads();
        for (int i = tid; i < kHistBins; i += kAttendThreads) u.bl.h12[i] = 0u;
        if (tid == 0) s_ceq = 0u;
        __syncthreads();
        for (uint32_t base = 0; base < nb; base += kAttendThreads * 8u) {
            uint32_t wv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {                                  // every load in flight at once
                const uint32_t i = base + (uint32_t)(kAttendThreads * e + tid);
                wv[e] = i < nb ? coherent_load(&bk[i]) : 0u;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t i = base + (uint32_t)(kAttendThreads * e + tid);
                if (i < nb) {
                    coherent_store(&bk[i], 0u);                            // below every key, for the next call
                    u.bl.w[i] = wv[e];
                    atomicAdd(&u.bl.h12[key_digit(wv[e])], 1u);
                }
            }
        }
        __syncthreads();
        unsigned long long cut = 0ull;                                     // kept: full_order >= cut
        if (m < nb) {
            {
                uint32_t hc[kHistPerThread];
#pragma unroll
                for (int i = 0; i < kHistPerThread; ++i) hc[i] = u.bl.h12[kHistBins - 1 - (kHistPerThread * tid + i)];
                block_crossing<kHistPerThread>(hc, kHistBins, m, s_wave, s_res);
            }
            const uint32_t Td = s_res[0], above = s_res[1], g = s_res[3] - s_res[1];
            const uint32_t klo = (uint32_t)digit_first_key(Td);
            const uint32_t khi = (uint32_t)(digit_first_key(Td + 1u) - 1ull);
            const uint32_t r_left = m - above;                             // blocks of digit T kept (>= 1)
            __syncthreads();                                               // s_res is rewritten below
            if (r_left == g) {
                cut = (unsigned long long)klo << 32;                       // every block of digit T
            } else if (g <= (uint32_t)kFastGroup) {
                for (uint32_t i = tid; i < nb; i += kAttendThreads) {
                    const uint32_t wv = u.bl.w[i];
                    if (wv >= klo && wv <= khi) u.bl.comp[atomicAdd(&s_ceq, 1u)] = full_order(wv, i);
                }
                __syncthreads();
                // the r_left-th largest of the group: r_left - 1 of its
                // composites lie above it (composites are distinct)
                for (uint32_t q = tid; q < g; q += kAttendThreads) {
                    const unsigned long long mine = u.bl.comp[q];
                    uint32_t gt = 0, j = 0;
                    for (; j + 8u <= g; j += 8u) {
                        unsigned long long c8[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) c8[e] = u.bl.comp[j + e];
#pragma unroll
                        for (int e = 0; e < 8; ++e) gt += c8[e] > mine ? 1u : 0u;
                    }
                    for (; j < g; ++j) gt += u.bl.comp[j] > mine ? 1u : 0u;
                    if (gt == r_left - 1u) s_cut = mine;
                }
                __syncthreads();
                cut = s_cut;
            } else {
                // many blocks share digit T (e.g. identical keys): 12-bit radix
                // passes over its composites, which share the bits above `shift`
                const uint32_t x = klo ^ khi;
                int shift = 32 + (x ? 32 - __clz(x) : 0);
                unsigned long long prefix = ((unsigned long long)klo << 32) >> shift;
                uint32_t need = r_left;
                while (shift > 0) {
                    const int bits = shift >= 12 ? 12 : shift;
                    const int nshift = shift - bits;
                    const uint32_t nbin = 1u << bits;
                    for (int i = tid; i < kHistBins; i += kAttendThreads) u.bl.h12[i] = 0u;
                    __syncthreads();
                    for (uint32_t i = tid; i < nb; i += kAttendThreads) {
                        const unsigned long long c = full_order(u.bl.w[i], i);
                        if ((c >> shift) == prefix) atomicAdd(&u.bl.h12[(uint32_t)(c >> nshift) & (nbin - 1u)], 1u);
                    }
                    __syncthreads();
                    uint32_t hc[kHistPerThread];
#pragma unroll
                    for (int i = 0; i < kHistPerThread; ++i) {
                        const uint32_t rank = (uint32_t)(kHistPerThread * tid + i);
                        hc[i] = rank < nbin ? u.bl.h12[nbin - 1u - rank] : 0u;
                    }
                    block_crossing<kHistPerThread>(hc, (int)nbin, need, s_wave, s_res);
                    const uint32_t d = s_res[0], ab = s_res[1], gs = s_res[3] - s_res[1];
                    __syncthreads();
                    prefix = (prefix << bits) | d;
                    need -= ab;
                    shift = nshift;
                    if (gs == 1u && shift > 0) {                           // the bin holds the cut alone
                        for (uint32_t i = tid; i < nb; i += kAttendThreads) {
                            const unsigned long long c = full_order(u.bl.w[i], i);
                            if ((c >> shift) == prefix) s_cut = c;
                        }
                        __syncthreads();
                        prefix = s_cut;
                        shift = 0;
                    }
                }
                cut = prefix;
            }
        }
        // the kept blocks, ascending: thread t takes blocks [per t, per t + per)
        const uint32_t per = (nb + kAttendThreads - 1u) / kAttendThreads;
        const uint32_t e0 = (uint32_t)tid * per;
        uint32_t mine = 0;
        for (uint32_t e = 0; e < per; ++e) {
            const uint32_t i = e0 + e;
            mine += (i < nb && full_order(u.bl.w[i], i) >= cut) ? 1u : 0u;
        }
        uint32_t tot;
        uint32_t at = block_exclusive_scan(mine, s_wave, &tot);
        for (uint32_t e = 0; e < per; ++e) {
            const uint32_t i = e0 + e;
            if (i < nb && full_order(u.bl.w[i], i) >= cut) {
                if (at < (uint32_t)kMaxSelBlocks) u.bl.list[at] = i;
                ++at;
            }
        }
        __syncthreads();
        const uint32_t kept = min(min(tot, m), (uint32_t)kMaxSelBlocks);
        const uint32_t bmask = (1u << bsh) - 1u;
        for (uint32_t i = tid; i < (uint32_t)p.k; i += kAttendThreads) {
            const uint32_t r = i >> bsh;
            int32_t v = -1;
            if (r < kept) {
                const uint32_t tok = (u.bl.list[r] << bsh) + (i & bmask);
                v = tok < (uint32_t)n ? (int32_t)tok : -1;
            }
            srow[i] = v;
        }
        if (tid == 0 && tot != m) atomicOr(p.ws.err, 2u);
        __syncthreads();
    };

    // Top-p (the Top-p reading of the digest's ablation of selection
    // methods): the shortest prefix of the ranking (pooled score descending,
    // index ascending) of the head's top-min(k, n) set whose share of the
    // softmax of the pooled scores over the whole context reaches p.  Run by
    // the workgroup that resolved the set, right after it:
    // 1. the set (read back from S) and its keys (from the score buffer),
    //    composites key << 18 | inverted index (larger = earlier in the
    //    ranking); the normaliser parts of the head's workgroups, merged in
    //    slot order into Z (slot tags restored to zero);
    // 2. shares exp(.)/Z as 52-bit fixed point (integer sums do not depend
    //    on order); a set holding less than p stays as it is (decided from
    //    Z alone, before the set is read, when k_eff shares of the largest
    //    pooled sum stay below p);
    // 3. an MSD radix of 8-bit digits from the highest bit where the
    //    composites differ, share-weighted, until a digit's group holds one
    //    composite: the cut;
    // 4. the kept tokens compacted to the front of the row (ascending) by one
    //    block scan, -1 after them.
    auto topp_cut = [&](int hb, int n, int wf, int nw) __attribute__((always_inline)) {
        int32_t* srow = p.S_out + (size_t)hb * p.k;
        const uint32_t* sc = p.ws.score + (size_t)hb * p.max_ctx;
        unsigned long long* cp = p.ws.cand + (size_t)hb * p.max_ctx;   // free once the set is resolved
        const uint32_t ke = (uint32_t)min(p.k, max(n, 0));
        const float cl = p.scale_log2 * (1.0f / (float)G);             // key units -> log2 of a share
        // The set from the resolver's LDS when it resolved in one batch (no
        // wait for the row's stores, no load rounds for S and its keys), else
        // read back from S and the score buffer.
        const bool lds_set = s_lds_set != 0u && ke <= (uint32_t)(kToppSlots * kAttendThreads);
        // The parts of the head's workgroups first: their loads travel while
        // the row's coherent stores are acknowledged (vmcnt counts both).
        constexpr int kZPer = kMaxWG / kAttendThreads;                 // part slots per thread
        uint32_t zt[kZPer], zm_[kZPer], zlo[kZPer], zhi[kZPer];
#pragma unroll
        for (int e = 0; e < kZPer; ++e) {
            const int i = tid + kAttendThreads * e;
            const uint32_t* zw = p.ws.zpart + 4 * (size_t)(wf + hb + min(i, nw - 1));
            zt[e] = coherent_load(&zw[0]);
            zm_[e] = coherent_load(&zw[1]);
            zlo[e] = coherent_load(&zw[2]);
            zhi[e] = coherent_load(&zw[3]);
            if (i >= nw) zt[e] = 0u;                                   // not this head's part
        }
        if (!lds_set) wait_stores_complete();                         // the row's coherent stores
        __syncthreads();
        const uint32_t per = (ke + kAttendThreads - 1u) / kAttendThreads;
        const uint32_t e0 = (uint32_t)tid * per;
        uint32_t iv[kToppSlots], kk[kToppSlots];
        if (!lds_set) {
            // Every load is issued on every path (indices clamped, results
            // masked): loads under per-slot branches each get a wait of their
            // own, which serialises the rounds.  ke >= 1 and nw >= 1 here.
#pragma unroll
            for (int e = 0; e < kToppSlots; ++e)
                iv[e] = (uint32_t)coherent_load(&srow[min(e0 + (uint32_t)e, ke - 1u)]);
        }
        // (up to the decision below, only the per-wavefront words s_zk and
        // s_zd are written: u.fr, where the set may be, stays as it is)
        // the largest pooled sum over the parts
        float fmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < kZPer; ++e)
            if (zt[e] == (uint32_t)hb + 1u) fmax = fmaxf(fmax, __builtin_bit_cast(float, zm_[e]));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) fmax = fmaxf(fmax, __shfl_xor(fmax, o));
        if (lane == 0) s_zk[wave] = __builtin_bit_cast(uint32_t, fmax);
        __syncthreads();
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) fmax = fmaxf(fmax, __builtin_bit_cast(float, s_zk[wv]));
        // Z = sum of z_w 2^((m_w - fmax) c), the parts in slot order
        double z = 0.0;
        {
            double zs = 0.0;
#pragma unroll
            for (int e = 0; e < kZPer; ++e) {
                if (zt[e] == (uint32_t)hb + 1u) {
                    const double zw = __builtin_bit_cast(double, ((unsigned long long)zhi[e] << 32) | zlo[e]);
                    zs += zw * (double)exp2f((__builtin_bit_cast(float, zm_[e]) - fmax) * cl);
                    coherent_store(&p.ws.zpart[4 * (size_t)(wf + hb + tid + kAttendThreads * e)], 0u);   // free again
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) zs += __shfl_xor(zs, o);
            if (lane == 0) s_zd[wave] = zs;
            __syncthreads();
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) z += s_zd[wv];
        }
        const double inv_z = 1.0 / z;
        // No cut possible: no pooled sum exceeds fmax, so every share is at
        // most 1 / Z (2^-16 of slack covers exp2f's rounding at arguments
        // <= 0), and ke such shares stay below p.  The row stays as the
        // resolver wrote it, exactly as the share sums below would decide.
        // (z, inv_z and the parts are the same in every thread: the
        // decision is uniform.)
        if (cl > 0.0f && (double)ke * ((1.0 + 0x1p-16) * inv_z * 0x1p52) < (double)p.topp_P) {
            __syncthreads();
            return;
        }
        if (lds_set) {
            // entry i of S: wavefront v's part of u.fr.map, after the parts
            // of the wavefronts before it
            constexpr uint32_t kQ = kFastBatch / kWaves;
            const uint32_t b1 = u.fr.jc[0], b2 = b1 + u.fr.jc[1], b3 = b2 + u.fr.jc[2];
#pragma unroll
            for (int e = 0; e < kToppSlots; ++e) {
                const uint32_t i = min(e0 + (uint32_t)e, ke - 1u);
                const uint32_t v = (i >= b1 ? 1u : 0u) + (i >= b2 ? 1u : 0u) + (i >= b3 ? 1u : 0u);
                const uint32_t base = v == 0u ? 0u : (v == 1u ? b1 : (v == 2u ? b2 : b3));
                const uint32_t f = u.fr.map[v * kQ + (i - base)];
                iv[e] = u.fr.idx[f];
                kk[e] = u.fr.key[f];
            }
            __syncthreads();                                           // (the cut's words reuse u.fr.map)
        }
        unsigned long long cr[kToppSlots];
        unsigned long long clo = ~0ull, chi = 0ull;
        bool bad = false;
        if (!lds_set) {
#pragma unroll
            for (int e = 0; e < kToppSlots; ++e) kk[e] = coherent_load(&sc[iv[e] < (uint32_t)n ? iv[e] : 0u]);
        }
#pragma unroll
        for (int e = 0; e < kToppSlots; ++e) {
            const uint32_t i = e0 + (uint32_t)e;
            cr[e] = 0ull;
            if ((uint32_t)e < per && i < ke) {
                bad |= iv[e] >= (uint32_t)n;
                const uint32_t jj = iv[e] < (uint32_t)n ? iv[e] : 0u;
                cr[e] = ((unsigned long long)kk[e] << kIdxBits) | (unsigned long long)(kIdxMask - jj);
                clo = cr[e] < clo ? cr[e] : clo;
                chi = cr[e] > chi ? cr[e] : chi;
            }
        }
        for (uint32_t e = kToppSlots; e < per; ++e) {                  // (more than kToppSlots per thread)
            const uint32_t i = e0 + e;
            if (i < ke) {
                const uint32_t j = (uint32_t)coherent_load(&srow[i]);
                bad |= j >= (uint32_t)n;
                const uint32_t jj = j < (uint32_t)n ? j : 0u;
                const unsigned long long c = ((unsigned long long)coherent_load(&sc[jj]) << kIdxBits) |
                                             (unsigned long long)(kIdxMask - jj);
                cp[i] = c;                                             // (read back by this thread only)
                clo = c < clo ? c : clo;
                chi = c > chi ? c : chi;
            }
        }
        if (bad) atomicOr(p.ws.err, 2u);
        // the composites' range
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const unsigned long long ylo = __shfl_xor(clo, o), yhi = __shfl_xor(chi, o);
            clo = ylo < clo ? ylo : clo;
            chi = yhi > chi ? yhi : chi;
        }
        if (lane == 0) {
            u.tp.lo[wave] = clo;
            u.tp.hi[wave] = chi;
        }
        __syncthreads();
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) {
            clo = u.tp.lo[wv] < clo ? u.tp.lo[wv] : clo;
            chi = u.tp.hi[wv] > chi ? u.tp.hi[wv] : chi;
        }
        auto weight = [&](unsigned long long c) -> unsigned long long {
            const float f = key_float((uint32_t)(c >> kIdxBits));
            return (unsigned long long)((double)exp2f((f - fmax) * cl) * inv_z * 0x1p52);
        };
        const unsigned long long target = p.topp_P;
        unsigned long long wr[kToppSlots];
#pragma unroll
        for (int e = 0; e < kToppSlots; ++e) wr[e] = ((uint32_t)e < per && e0 + (uint32_t)e < ke) ? weight(cr[e]) : 0ull;
        auto for_each_elem = [&](auto&& f) {
#pragma unroll
            for (int e = 0; e < kToppSlots; ++e)
                if ((uint32_t)e < per && e0 + (uint32_t)e < ke) f(cr[e], wr[e]);
            for (uint32_t e = kToppSlots; e < per; ++e)
                if (e0 + e < ke) {
                    const unsigned long long c = cp[e0 + e];
                    f(c, weight(c));
                }
        };
        // the set's whole share: below p, no prefix reaches p and the row stays
        bool cut = true;
        {
            unsigned long long tot = 0;
            for_each_elem([&](unsigned long long, unsigned long long wt) { tot += wt; });
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
            if (lane == 0) u.tp.tot[wave] = tot;
            __syncthreads();
            tot = 0;
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) tot += u.tp.tot[wv];
            cut = ke > 0u && tot >= target;
        }
        int shift = clo == chi ? 0 : 64 - __clzll((long long)(clo ^ chi));
        unsigned long long prefix = chi >> shift, above = 0;
        while (cut && shift > 0) {
            const int bits = shift >= 8 ? 8 : shift;
            const int nshift = shift - bits;
            const uint32_t nbin = 1u << bits;
            for (int i = tid; i < kToppBins * kToppCopies; i += kAttendThreads) u.tp.hist[i] = 0ull;
            __syncthreads();
            // the set's keys share their leading digits, so most lanes of a
            // wavefront add to one or two bins: lane & 3 picks one of four
            // interleaved copies, so fewer lanes meet on one address
            const uint32_t cpy = (uint32_t)lane & (uint32_t)(kToppCopies - 1);
            for_each_elem([&](unsigned long long c, unsigned long long wt) {
                if ((c >> shift) == prefix) {
                    const uint32_t dg = (uint32_t)(c >> nshift) & (nbin - 1u);
                    atomicAdd(&u.tp.hist[dg * kToppCopies + cpy], wt);
                }
            });
            __syncthreads();
            if (wave == 0) {
                // crossing: lane l holds digits nbin-1-4l .. nbin-4-4l (descending
                // rank 4l .. 4l+3); a wavefront scan gives each its running share
                unsigned long long h[4], ls = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t t = 4u * (uint32_t)lane + (uint32_t)r;
                    h[r] = 0ull;
                    if (t < nbin) {
#pragma unroll
                        for (int q = 0; q < kToppCopies; ++q) h[r] += u.tp.hist[(nbin - 1u - t) * kToppCopies + q];
                    }
                    ls += h[r];
                }
                unsigned long long inc = ls;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const unsigned long long y = __shfl_up(inc, o);
                    if (lane >= o) inc += y;
                }
                unsigned long long run = above + inc - ls, before = 0;
                int found = -1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (found < 0 && run + h[r] >= target) {
                        found = 4 * lane + r;
                        before = run;
                    }
                    run += h[r];
                }
                const unsigned long long m = __ballot(found >= 0);
                if (m == 0ull) {
                    if (lane == 0) u.tp.found = 0u;
                } else if (lane == __ffsll((long long)m) - 1) {
                    const uint32_t dg = nbin - 1u - (uint32_t)found;
                    u.tp.found = 1u;
                    u.tp.digit = dg;
                    u.tp.above = before;
                }
            }
            __syncthreads();
            if (!u.tp.found) {                         // (the whole-share test above rules this out)
                cut = false;
                break;
            }
            prefix = (prefix << bits) | u.tp.digit;
            above = u.tp.above;
            shift = nshift;
            // the composites of the new prefix, counted (one is the cut)
            if (shift > 0) {
                uint32_t mine = 0;
                for_each_elem([&](unsigned long long c, unsigned long long) { mine += (c >> shift) == prefix ? 1u : 0u; });
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) mine += (uint32_t)__shfl_xor((int)mine, o);
                if (lane == 0) u.tp.cnt[wave] = mine;
            }
            __syncthreads();                           // (and the digit's words are rewritten by the next pass)
            uint32_t grp = 0;
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) grp += u.tp.cnt[wv];
            const bool single = shift > 0 && grp == 1u;
            if (single) {
                // the digit's group is one composite: it is the cut
                for_each_elem([&](unsigned long long c, unsigned long long) {
                    if ((c >> shift) == prefix) u.tp.cutv = c;
                });
                __syncthreads();
                prefix = u.tp.cutv;
                shift = 0;
            }
        }
        if (cut) {
            // the kept tokens (composites >= prefix) in their ascending order,
            // compacted to the front of the row (after the resolver's stores
            // to it are complete: the same words are written again)
            if (lds_set) {
                wait_stores_complete();
                __syncthreads();
            }
            uint32_t mine = 0;
            for_each_elem([&](unsigned long long c, unsigned long long) { mine += c >= prefix ? 1u : 0u; });
            uint32_t total;
            uint32_t at = block_exclusive_scan(mine, s_wave, &total);
            for_each_elem([&](unsigned long long c, unsigned long long) {
                if (c >= prefix) srow[at++] = (int32_t)(kIdxMask - (uint32_t)(c & kIdxMask));
            });
            for (uint32_t i = total + (uint32_t)tid; i < ke; i += kAttendThreads) srow[i] = -1;
        }
        __syncthreads();
    };

    // The heads of the range in order; a head whose top-k this workgroup
    // resolves (as its last selection arrival, or as its helper once the
    // range is done) waits in `pending` and is resolved at the top of the
    // next pass, so the resolver has a single call site.
    int pending = -1;
    bool helped = false;
    int next_bg = head_of(lo);
    LYCHEE_STAMP(kTrPro0 + 3);
    for (;;) {
        if (__builtin_expect(pending >= 0, 0)) {   // (out of the way of the streaming path)
            const int X = pending;
            pending = -1;
            const int b = X / p.Hkv;
            const uint32_t h0 = s_pref[X], h1 = s_pref[X + 1];
            int wf, wl;
            wg_pair(h0, h1 - 1, wf, wl);
            LYCHEE_STAMP(kTrResolveStart);
#ifdef LYCHEE_TRACE
            tr_flags |= 8u;
#endif
            if constexpr (BLOCK) {
                block_resolve(X, s_nctx[b]);
            } else if (__builtin_expect(fast_resolve(X, s_nctx[b], s_ke[b], h0, wf, wl - wf + 1), 0)) {
#ifdef LYCHEE_TRACE
                tr_flags |= 32u;
#endif
                resolve_topk(X, s_nctx[b], s_ke[b], 0u, 0u, (uint32_t)kResolveSlices, true);
            }
            if constexpr (TOPP) topp_cut(X, s_nctx[b], wf, wl - wf + 1);
            // the hand-off word back to idle for the next launch where this
            // workgroup is the last party to touch it (1: it is the helper;
            // 5: the helper withdrew; 4 is restored by the helper)
            if (tid == 0) {
                const uint32_t v = coherent_load(&p.ws.hready[X]);
                if (v == 1u || v == 5u) coherent_store(&p.ws.hready[X], 0u);
            }
            LYCHEE_STAMP(kTrResolveEnd);
            __syncthreads();
        }
        if (!(next_bg < BH && s_pref[next_bg] < hi)) {
            // range done: the helper duty, if any (a bounded wait for the
            // head's last arrival; on time-out the helper withdraws and the
            // last arrival resolves)
            if (HYBRID && !helped) {
                helped = true;
                const int X = helped_by(w);
                if (X >= 0) {
                    if (tid == 0) {
                        // waiting (0 -> 3; 1 if already handed over, 6 offered:
                        // take it, 4 taken by the last arrival)
                        uint32_t v = counter_cas(&p.ws.hready[X], 0u, 3u);
                        if (v == 6u) v = counter_cas(&p.ws.hready[X], 6u, 1u) == 6u ? 1u : 4u;
                        if (v == 4u) {
                            coherent_store(&p.ws.hready[X], 0u);               // the last arrival resolves
                        } else if (v != 1u) {
                            const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
                            for (;;) {
                                v = coherent_load(&p.ws.hready[X]);
                                if (v == 1u) break;
                                if (__builtin_amdgcn_s_memrealtime() - t0 > kHelperWaitTicks) {
                                    v = counter_cas(&p.ws.hready[X], 3u, 5u) == 3u ? 5u : 1u;   // withdraw, unless
                                    break;                                                      // handed over meanwhile
                                }
                                __builtin_amdgcn_s_sleep(2);
                            }
                        }
                        s_flag[0] = v == 1u;
                    }
                    __syncthreads();
                    if (s_flag[0]) {
                        pending = X;
#ifdef LYCHEE_TRACE
                        tr_flags |= 64u;
#endif
                        continue;
                    }
                }
            }
            break;
        }
        const int bg = next_bg++;
        const uint32_t h0 = s_pref[bg], h1 = s_pref[bg + 1];
        if (h1 <= lo || h1 == h0) continue;
        const int b = bg / p.Hkv, g = bg - b * p.Hkv;
        const bool retr = is_retr(bg);
        const uint32_t cw = retr ? kCostRetrieval : p.cost_sparse;
        const uint32_t seg_lo = (max(lo, h0) - h0) / cw;     // first row (position) of this head
        const uint32_t seg_hi = (min(hi, h1) - h0) / cw;
        const int n = s_nctx[b];
        const uint32_t ks = (uint32_t)min(p.k, n);         // S entries of the head
        const uint32_t ke = s_ke[b];                          // tokens a retrieval head selects
#ifdef LYCHEE_TRACE
        if (tr_heads == 0) LYCHEE_STAMP(kTrHeadStart);
        ++tr_heads;
        tr_flags |= retr ? 1u : 2u;
#endif

        // query slices: register h' holds query head g*G + (h' ^ xl), elements x*EPL..
        Frag<NDW> qf[G];
        {
            const uint32_t* qbase = reinterpret_cast<const uint32_t*>(p.q);
#pragma unroll
            for (int hp = 0; hp < G; ++hp) {
                const size_t qrow = (size_t)b * Hq + (size_t)g * G + (hp ^ xl);
                load_frag<NDW>(qf[hp], qbase + (qrow * D + (size_t)x * EPL) * T::kBytes / 4);
            }
        }
        const size_t kv_row0 = (size_t)bg * (size_t)p.max_ctx;
        const uint32_t* kbase = reinterpret_cast<const uint32_t*>(p.kc) + (kv_row0 * D + (size_t)x * EPL) * T::kBytes / 4;
        const uint32_t* vbase = reinterpret_cast<const uint32_t*>(p.vc) + (kv_row0 * D + (size_t)x * EPL) * T::kBytes / 4;
        constexpr size_t kRowDw = (size_t)D * T::kBytes / 4;   // dwords per cache row

        float m_run = -INFINITY, l_run = 0.0f;
        float o[G][EPL];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
        bool bad_index = false;
        bool bad_order = false;        // a sparse head's S_in entries not strictly ascending
        uint32_t key_base = 0;         // position of u.st.keys[0] (retrieval selection keys)

        // Load the K/V fragments of the tile starting at position tb of
        // [r_lo, r_hi).  Loads are unconditional: positions past r_hi (and
        // invalid S entries) are clamped to a valid row and masked out of the
        // softmax, so the next tile's loads stay in flight during compute.
        auto load_tile = [&](uint32_t tb, uint32_t r_lo, uint32_t r_hi, const int32_t* sidx, Frag<NDW>* kf,
                             Frag<NDW>* vf, int& tok_mine, bool& vmine) {
            const uint32_t rb = tb + (uint32_t)row * NK;
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const uint32_t pk = min(rb + (uint32_t)(i ^ xh), r_hi - 1);
                const uint32_t pv = min(rb + (uint32_t)i, r_hi - 1);
                int tk, tv;
                if (sidx) {
                    tk = sidx[pk - r_lo];
                    tv = sidx[pv - r_lo];
                    const bool okk = (unsigned)tk < (unsigned)n;
                    if ((unsigned)(tk + 1) > (unsigned)n) bad_index = true;   // -1 (padding of a shorter set) is fine
                    if (i == 0) vmine = okk && (rb + (uint32_t)xh < r_hi);
                    tk = okk ? tk : 0;
                    tv = ((unsigned)tv < (unsigned)n) ? tv : 0;
                } else {
                    tk = (int)pk;
                    tv = (int)pv;
                    if (i == 0) vmine = rb + (uint32_t)xh < r_hi;
                }
                if (i == 0) tok_mine = tk;
                load_frag_once<NDW>(kf[i], kbase + (size_t)tk * kRowDw);
                load_frag_once<NDW>(vf[i], vbase + (size_t)tv * kRowDw);
            }
        };

        auto compute_tile = [&](const Frag<NDW>* kf, const Frag<NDW>* vf, int tok_mine, bool vmine) {
            // 16 partial dots: slot s = i'*G + h' holds (key i'^xh, head h'^xl)
            float a[16];
#pragma unroll
            for (int i = 0; i < NK; ++i)
#pragma unroll
                for (int hp = 0; hp < G; ++hp) a[i * G + hp] = dot_frag<T, NDW>(qf[hp], kf[i]);
            // reduce-scatter over the 16 lanes of the row: lane x ends with value x
            float r8[8], r4[4], r2[2];
#pragma unroll
            for (int s = 0; s < 8; ++s) r8[s] = a[s] + dpp<kDppRowRor8>(a[s + 8]);
#pragma unroll
            for (int s = 0; s < 4; ++s) r4[s] = r8[s] + dpp<kDppRowHalfMirror>(r8[7 - s]);
#pragma unroll
            for (int s = 0; s < 2; ++s) r2[s] = r4[s] + dpp<kDppQuadXor2>(r4[s ^ 2]);
            const float dfull = r2[0] + dpp<kDppQuadXor1>(r2[1]);   // key (row base + xh), head xl

            if constexpr (HYBRID) {
                if (retr) {
                    float pooled = dfull;           // sum over the G heads of this key
                    if constexpr (G >= 2) pooled += dpp<kDppQuadXor1>(pooled);
                    if constexpr (G >= 4) pooled += dpp<kDppQuadXor2>(pooled);
                    if constexpr (G >= 8) pooled += dpp<kDppRowHalfMirror>(pooled);
                    if (xl == 0 && vmine) {
                        const uint32_t key = float_key(pooled);
                        u.st.keys[(uint32_t)tok_mine - key_base] = key;
                        atomicAdd(&u.st.hist[key_digit(key)], 1u);
                    }
                }
            }

            const float z = vmine ? dfull * p.scale_log2 : -INFINITY;
            const float mt = row_max_same_head<G>(z);
            if (__any(mt > m_run + kLazyThresh)) {
                const float mn = fmaxf(m_run, mt);
                const float alpha = (mn == m_run) ? 1.0f : fast_exp2(m_run - mn);
                m_run = mn;
                l_run *= alpha;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float ah = row_bcast_dyn(alpha, h);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[h][e] *= ah;
                }
            }
            const float pr = vmine ? fast_exp2(z - m_run) : 0.0f;
            l_run += pr;

            // broadcast the row's 16 weights to every lane of the row
            u.st.pw[wave][row][x] = pr;
            compiler_fence();
            float pw[16];
            {
                const float4* src = reinterpret_cast<const float4*>(&u.st.pw[wave][row][0]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float4 v4 = src[c];
                    pw[4 * c + 0] = v4.x; pw[4 * c + 1] = v4.y; pw[4 * c + 2] = v4.z; pw[4 * c + 3] = v4.w;
                }
            }
            compiler_fence();
#pragma unroll
            for (int i = 0; i < NK; ++i) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const float ve = frag_elem<T, NDW>(vf[i], e);
#pragma unroll
                    for (int h = 0; h < G; ++h) o[h][e] = __builtin_fmaf(pw[i * G + h], ve, o[h][e]);
                }
            }
        };

        // Two-deep software pipeline over the tiles of [r_lo, r_hi): wave w
        // owns tiles starting at r_lo + w*KPW, stepping by STRIDE.
        // The bounds are wavefront-uniform by construction; saying so keeps the
        // loop's exits scalar, so no path reaches the loop top with lanes off
        // and tile B's loads still in flight (the wait there would have to
        // drain every load, tile A's prefetch included).
        auto stream_range = [&](uint32_t r_lo, uint32_t r_hi, const int32_t* sidx) {
            r_lo = __builtin_amdgcn_readfirstlane(r_lo);
            r_hi = __builtin_amdgcn_readfirstlane(r_hi);
            uint32_t tb = r_lo + (uint32_t)wave * KPW;
            if (tb >= r_hi) return;
            Frag<NDW> kA[NK], vA[NK], kB[NK], vB[NK];
            int tokA = 0, tokB = 0;
            bool vmA = false, vmB = false;
            load_tile(tb, r_lo, r_hi, sidx, kA, vA, tokA, vmA);
            // One exit, at the bottom: an exit between the two halves would
            // reach the loop top (as the structurizer lays it out) with tile
            // B's loads in flight, and the wait there would drain tile A's
            // prefetch on every iteration.  Tile A's loads of the last round
            // may lie past the range (clamped rows, never computed).
            for (;;) {
                const uint32_t t1 = tb + STRIDE;
                load_tile(t1, r_lo, r_hi, sidx, kB, vB, tokB, vmB);
                compute_tile(kA, vA, tokA, vmA);
                const uint32_t t2 = t1 + STRIDE;
                load_tile(t2, r_lo, r_hi, sidx, kA, vA, tokA, vmA);
                if (t1 < r_hi) compute_tile(kB, vB, tokB, vmB);
                if (t2 >= r_hi) break;
                tb = t2;
            }
        };

        int wf, wl;                    // the head's first and last workgroups
        wg_pair(h0, h1 - 1, wf, wl);
        const int nw = wl - wf + 1;
        if (!HYBRID) {
            stream_range(seg_lo, seg_hi, nullptr);
            LYCHEE_STAMP(kTrStreamEnd);
        } else if (retr) {
            uint32_t* sc = p.ws.score + (size_t)bg * p.max_ctx;
            uint32_t* gh = p.ws.hist + (size_t)bg * kHistBins;
            uint32_t w_count = 0, w_bound = 0;   // candidates appended, largest pass bound
            float zm = -INFINITY;                // Top-p: largest pooled sum of the range so far
            double zs = 0.0;                     // and the sum of 2^((f - zm) c) over it
            for (int i = tid; i < kHistBins; i += kAttendThreads) u.st.hist[i] = 0u;
            // equal passes of at most kKeyCap rows (no short tail pass)
            const uint32_t npass = (seg_hi - seg_lo + kKeyCap - 1) / kKeyCap;
            const uint32_t plen = npass ? (seg_hi - seg_lo + npass - 1) / npass : 1u;
            for (uint32_t c_lo = seg_lo; c_lo < seg_hi; c_lo += plen) {
                const uint32_t c_hi = min(seg_hi, c_lo + plen);
                const uint32_t len = c_hi - c_lo;
                key_base = c_lo;
                __syncthreads();
                stream_range(c_lo, c_hi, nullptr);
                __syncthreads();
                LYCHEE_STAMP(kTrStreamEnd);
                if (BLOCK) {
                    // The block rule: the largest key of each block of the pass
                    // (blocks of 2^sel_block >= 16 tokens, numbered from token
                    // 0), folded into the head's block words by atomic max.
                    // Thread t takes positions 16t .. 16t + 15, so at most two
                    // blocks; a block split between threads, passes or
                    // workgroups gets one atomic from each part.  No token
                    // top-k: the head's block resolve reads the block words.
                    const uint32_t i0 = 16u * (uint32_t)tid;
                    if (i0 < len) {
                        uint32_t* bk = p.ws.bkey + (size_t)bg * (size_t)p.bkey_stride;
                        const uint4* k4 = reinterpret_cast<const uint4*>(u.st.keys + i0);
                        uint32_t blk = (c_lo + i0) >> p.sel_block, bmx = 0u;
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const uint4 v = k4[c];
                            const uint32_t kv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const uint32_t i = i0 + 4u * (uint32_t)c + (uint32_t)e;
                                if (i < len) {
                                    const uint32_t bi = (c_lo + i) >> p.sel_block;
                                    if (bi != blk) {
                                        atomicMax(&bk[blk], bmx);
                                        blk = bi;
                                        bmx = 0u;
                                    }
                                    bmx = max(bmx, kv[e]);
                                }
                            }
                        }
                        atomicMax(&bk[blk], bmx);
                    }
                    for (int i = tid; i < kHistBins; i += kAttendThreads) u.st.hist[i] = 0u;
                    __syncthreads();
                    continue;
                }
                // every key to the score buffer (read only if the bound below fails,
                // or by the Top-p cut)
                for (uint32_t i = tid; i < len; i += kAttendThreads) coherent_store(&sc[c_lo + i], u.st.keys[i]);
                if (TOPP) {
                    // The Top-p rule: this pass's part of the normaliser, with
                    // f the pooled sum a key encodes and c = scale_log2 / G:
                    // m = the pass's largest f, z = sum of 2^((f - m) c) (fp32
                    // terms, fp32 per thread, double across threads in a
                    // fixed order), merged into the range's running pair.
                    const uint32_t i0 = 16u * (uint32_t)tid;
                    uint32_t kv[16];
                    uint32_t kmax = 0u;
                    {
                        const uint4* k4 = reinterpret_cast<const uint4*>(u.st.keys + i0);
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const uint4 v = k4[c];
                            kv[4 * c + 0] = v.x; kv[4 * c + 1] = v.y; kv[4 * c + 2] = v.z; kv[4 * c + 3] = v.w;
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        kv[e] = i0 + (uint32_t)e < len ? kv[e] : 0u;      // 0: below every key
                        kmax = max(kmax, kv[e]);
                    }
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
                    if (lane == 0) s_zk[wave] = kmax;
                    __syncthreads();
                    kmax = s_zk[0];
#pragma unroll
                    for (int wv = 1; wv < kWaves; ++wv) kmax = max(kmax, s_zk[wv]);
                    const float c = p.scale_log2 * (1.0f / (float)G);
                    const float mp = key_float(kmax);
                    float zt = 0.0f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) zt += kv[e] ? exp2f((key_float(kv[e]) - mp) * c) : 0.0f;
                    double zd = (double)zt;
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) zd += __shfl_xor(zd, o);
                    if (lane == 0) s_zd[wave] = zd;
                    __syncthreads();
                    double zp = s_zd[0];
#pragma unroll
                    for (int wv = 1; wv < kWaves; ++wv) zp += s_zd[wv];
                    if (zm == -INFINITY) {
                        zm = mp;
                        zs = zp;
                    } else {
                        const float M = fmaxf(zm, mp);
                        zs = zs * (double)exp2f((zm - M) * c) + zp * (double)exp2f((mp - M) * c);
                        zm = M;
                    }
                }
                // this pass's bound: its own crossing at its share s of k_eff plus
                // a margin, the smaller of kSelMargin - 1 shares and 4 standard
                // deviations of a Poisson count with mean s (plus 2), but never
                // under 3 deviations plus 4 (a pass of a few rows keeps them all)
                const float share = (float)ke * (float)len / (float)n;
                const float rs = sqrtf(share);
                const float margin = fmaxf(fminf((float)(kSelMargin - 1u) * share, 4.0f * rs + 2.0f), 3.0f * rs + 4.0f);
                // (a need beyond the pass's rows gives bound 0: every key kept)
                const uint32_t need = (uint32_t)fminf((float)len + 1.0f, ceilf(share + margin));
                // the pass's bound Tw: the crossing of its histogram at `need`
                // (thread t holds bins 4095 - 16t down to 4080 - 16t)
                uint32_t hc[kHistPerThread];
                {
                    uint4* hv = reinterpret_cast<uint4*>(u.st.hist + kHistBins - kHistPerThread * (tid + 1));
#pragma unroll
                    for (int c = 0; c < kHistPerThread / 4; ++c) {
                        const uint4 v4 = hv[c];
                        hc[kHistPerThread - 1 - 4 * c] = v4.x;
                        hc[kHistPerThread - 2 - 4 * c] = v4.y;
                        hc[kHistPerThread - 3 - 4 * c] = v4.z;
                        hc[kHistPerThread - 4 - 4 * c] = v4.w;
                    }
                }
                block_crossing<kHistPerThread>(hc, kHistBins, need, s_wave, s_res);
                const uint32_t Tw = s_res[0];
                // the pass's counts from Tw up to the head's histogram (few bins,
                // so few atomics on any one of them; other workgroups add to the
                // same bins), then zeros for the next pass
#pragma unroll
                for (int c = 0; c < kHistPerThread; ++c) {
                    const int i = tid + kAttendThreads * c;
                    const uint32_t cnt = u.st.hist[i];
                    if (cnt && (uint32_t)i >= Tw) atomicAdd(&gh[i], cnt);
                    u.st.hist[i] = 0u;
                }
                // Keys from Tw up, in position order, appended to this
                // workgroup's region of the head's candidate list (it starts at
                // the range's first row, and a pass keeps at most its rows):
                // thread t flags positions 16t .. 16t + 15, a block scan ranks
                // them, and the kept positions are staged in LDS for consecutive
                // device-coherent stores.
                {
                    const uint32_t kb = (uint32_t)digit_first_key(Tw);  // Tw <= kTopDigit: a real key
                    uint32_t m16 = 0;
                    const uint4* k4 = reinterpret_cast<const uint4*>(u.st.keys + 16 * tid);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint4 v = k4[c];
                        const uint32_t i0 = 16u * (uint32_t)tid + 4u * (uint32_t)c;
                        m16 |= (uint32_t)(i0 + 0u < len && v.x >= kb) << (4 * c + 0);
                        m16 |= (uint32_t)(i0 + 1u < len && v.y >= kb) << (4 * c + 1);
                        m16 |= (uint32_t)(i0 + 2u < len && v.z >= kb) << (4 * c + 2);
                        m16 |= (uint32_t)(i0 + 3u < len && v.w >= kb) << (4 * c + 3);
                    }
                    uint32_t kept;
                    uint32_t at = block_exclusive_scan((uint32_t)__popc(m16), s_wave, &kept);
                    while (m16) {
                        const int e = __ffs(m16) - 1;
                        m16 &= m16 - 1u;
                        u.st.gbuf[at++] = 16u * (uint32_t)tid + (uint32_t)e;
                    }
                    __syncthreads();
                    unsigned long long* cand = p.ws.cand + (size_t)bg * p.max_ctx + seg_lo + w_count;
                    for (uint32_t j = tid; j < kept; j += kAttendThreads) {
                        const uint32_t off = u.st.gbuf[j];
                        coherent_store(&cand[j], pack_cand(u.st.keys[off], c_lo + off));
                    }
                    w_count += kept;
                    w_bound = max(w_bound, Tw);
                }
                __syncthreads();
            }
            // Selection arrival, before the record: this workgroup's word (its
            // candidates and largest bound) and, once every store above is
            // complete, one count on the head's arrival counter.  The last
            // arrival hands the resolve to the head's helper if the helper is
            // already waiting (hready 3 -> 1); otherwise it offers it (0 -> 6)
            // and, after its record and merges, takes it back unless the
            // helper took it meanwhile (6 -> 4 against the helper's 6 -> 1).
            // States of hready: 0 idle, 3 helper waiting, 6 offered, 1 the
            // helper's (it restores 0 after the resolve), 4 the last arrival's
            // (the helper restores 0 when it comes), 5 helper withdrew (the
            // last arrival resolves and restores 0).
            if (TOPP && tid == 0 && zm != -INFINITY) {   // the range's normaliser part (device-coherent:
                const unsigned long long zb = __builtin_bit_cast(unsigned long long, zs);   // the resolver reads it)
                uint32_t* zw = p.ws.zpart + 4 * (size_t)(w + bg);
                coherent_store(&zw[1], __builtin_bit_cast(uint32_t, zm));
                coherent_store(&zw[2], (uint32_t)zb);
                coherent_store(&zw[3], (uint32_t)(zb >> 32));
                coherent_store(&zw[0], (uint32_t)bg + 1u);
            }
            if (tid == 0 && !BLOCK) coherent_store(&p.ws.wmeta[w + bg], w_count | (w_bound << 20));
            const int hw = helper_of(bg);   // (while the stores travel)
            wait_stores_complete();
            __syncthreads();
            if (tid == 0) {
                uint32_t last = 0;
                {
                    const uint32_t before = (uint32_t)counter_add64(&p.ws.selctr[bg], 1ull);
                    last = before + 1u == (uint32_t)nw;
                    if (last) {
                        counter_reset64(&p.ws.selctr[bg]);
                        if (hw >= 0) {
                            // 3 -> 1 if the helper waits, else 0 -> 6; at most three
                            // rounds (the helper moves 0 -> 3 once and 3 -> 5 once)
                            uint32_t expect = 3u;
                            for (int round = 0; round < 4; ++round) {
                                const uint32_t v = counter_cas(&p.ws.hready[bg], expect, expect == 3u ? 1u : 6u);
                                if (v == expect) {
                                    last = expect == 3u ? 0u : 2u;   // handed over / offered
                                    break;
                                }
                                if (v == 5u) break;         // the helper withdrew: resolve here
                                expect = v;                 // 0 or 3: try that
                            }
                        }
                    }
                }
                s_sel[0] = last;
            }
            LYCHEE_STAMP(kTrSelArrive);
        } else {
            // sparse head: stage the S entries of the range in LDS (one batched
            // load per chunk), forward them to S_out, then gather-stream
            const int32_t* Srow = p.S_in + (size_t)bg * p.k;
            int32_t* Sout = (p.S_out != p.S_in) ? p.S_out + (size_t)bg * p.k : nullptr;
            constexpr int PER = kIdxChunk / kAttendThreads;
            // Order check: the entries other than -1 must be strictly
            // ascending (the form S_out has), so a duplicate sits next to its
            // twin once the -1 holes are skipped.  run_max is the largest
            // entry before the chunk: the entry before this range if it is
            // not a hole (a twin across the range boundary with holes between
            // goes unseen), then the chunks before.
            int32_t run_max = -2147483647 - 1;
            if (seg_lo > 0) {
                const int32_t pv = Srow[seg_lo - 1];
                if (pv != -1) run_max = pv;
            }
            for (uint32_t c_lo = seg_lo; c_lo < seg_hi; c_lo += kIdxChunk) {
                const uint32_t c_hi = min(seg_hi, c_lo + (uint32_t)kIdxChunk);
                __syncthreads();
                int32_t v[PER];
#pragma unroll
                for (int j = 0; j < PER; ++j) v[j] = Srow[min(c_lo + tid + (uint32_t)(kAttendThreads * j), c_hi - 1)];
#pragma unroll
                for (int j = 0; j < PER; ++j) {
                    const uint32_t pos = c_lo + tid + (uint32_t)(kAttendThreads * j);
                    if (pos < c_hi) {
                        u.st.idx[pos - c_lo] = v[j];
                        if (Sout) Sout[pos] = v[j];
                    }
                }
                __syncthreads();
                {   // thread t checks the chunk's entries PER t .. PER t + PER - 1
                    int32_t e[PER];
                    int32_t lm = -2147483647 - 1;
#pragma unroll
                    for (int j = 0; j < PER; ++j) {
                        const uint32_t at = (uint32_t)(tid * PER + j);
                        e[j] = c_lo + at < c_hi ? u.st.idx[at] : -1;
                        lm = e[j] != -1 ? max(lm, e[j]) : lm;
                    }
                    int32_t cmax;
                    int32_t m = max(run_max, block_exclusive_max(lm, s_wave, &cmax));
#pragma unroll
                    for (int j = 0; j < PER; ++j) {
                        if (e[j] != -1) {
                            bad_order |= e[j] <= m;
                            m = max(m, e[j]);
                        }
                    }
                    run_max = max(run_max, cmax);
                }
                LYCHEE_STAMP(kTrSStaged);
                stream_range(c_lo, c_hi, u.st.idx);
            }
            LYCHEE_STAMP(kTrStreamEnd);
            // entries past min(k, n) (the -1 padding of a short context) belong
            // to the workgroup that finishes the head
            if (Sout && h1 <= hi) {
                for (uint32_t i = ks + tid; i < (uint32_t)p.k; i += kAttendThreads) Sout[i] = Srow[i];
            }
        }
        if (bad_index) atomicOr(p.ws.err, 1u);
        if (bad_order) atomicOr(p.ws.err, 32u);

        // ---- merge the 4 rows of each wavefront, then the 4 wavefronts ----
        const float lrow = row_sum_same_head<G>(l_run);           // head xl, this row
        float M = m_run;
        M = fmaxf(M, lane_xor16(M));
        M = fmaxf(M, lane_xor32(M));
        const float sc = safe_scale(m_run, M);
        float lw = lrow * sc;
        lw += lane_xor16(lw);
        lw += lane_xor32(lw);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float sch = row_bcast_dyn(sc, h);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float v = o[h][e] * sch;
                v += lane_xor16(v);
                v += lane_xor32(v);
                o[h][e] = v;
            }
        }
        __syncthreads();
        if (row == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < EPL; ++e) u.st.wo[wave][h][x * EPL + e] = o[h][e];
            if (x < G) {
                u.st.wm[wave][x] = M;
                u.st.wl[wave][x] = lw;
            }
        }
        __syncthreads();

        float* rec = p.ws.rec1 + (size_t)(w + bg) * RS;
        for (int idx = tid; idx < G * D; idx += kAttendThreads) {
            const int h = idx / D, t = idx - h * D;
            float Mw = -INFINITY;
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) Mw = fmaxf(Mw, u.st.wm[wv][h]);
            float O = 0.0f, L = 0.0f;
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) {
                const float s = safe_scale(u.st.wm[wv][h], Mw);
                O += u.st.wo[wv][h][t] * s;
                L += u.st.wl[wv][h] * s;
            }
            coherent_store(&rec[2 * G + h * D + t], O);
            if (t == 0) {
                coherent_store(&rec[h], Mw);
                coherent_store(&rec[G + h], L);
            }
        }

        // ---- arrival of the record at its group's merger ----
        const int c = (w - wf) / kCombineFanIn;
        const int nc = (nw + kCombineFanIn - 1) / kCombineFanIn;
        const int csize = min(kCombineFanIn, nw - c * kCombineFanIn);
        wait_stores_complete();
        LYCHEE_STAMP(kTrRecordDone);
        __syncthreads();
        if (tid == 0) {
            uint32_t* ctr = p.ws.cnt1 + (size_t)bg * kLevel2Max + c;
            const uint32_t old = counter_add(ctr, 1u);
            const int last = (int)(old + 1u == (uint32_t)csize);
            if (last) counter_reset(ctr);
            s_flag[0] = last;
        }
        __syncthreads();
        LYCHEE_STAMP(kTrArrive);
        const uint32_t sel_role = (HYBRID && retr) ? s_sel[0] : 0u;
        if (s_flag[0]) {
            const float* grp = p.ws.rec1 + (size_t)(wf + c * kCombineFanIn + bg) * RS;
            float* out_bg = p.out + ((size_t)b * Hq + (size_t)g * G) * D;
            if (nc == 1) {
                merge_records<D, G>(grp, csize, nullptr, out_bg, u.st.ml);
            } else {
                float* r2 = p.ws.rec2 + ((size_t)bg * kLevel2Max + c) * RS;
                merge_records<D, G>(grp, csize, r2, nullptr, u.st.ml);
                wait_stores_complete();
                __syncthreads();
                if (tid == 0) {
                    uint32_t* ctr = p.ws.cnt2 + bg;
                    const uint32_t old = counter_add(ctr, 1u);
                    const int last = (int)(old + 1u == (uint32_t)nc);
                    if (last) counter_reset(ctr);
                    s_flag[0] = last;
                }
                __syncthreads();
                if (s_flag[0]) merge_records<D, G>(p.ws.rec2 + (size_t)bg * kLevel2Max * RS, nc, nullptr, out_bg, u.st.ml);
            }
            LYCHEE_STAMP(kTrMergeDone);
#ifdef LYCHEE_TRACE
            tr_flags |= 4u;
#endif
        }
        if (sel_role == 1u) pending = bg;   // the head's last selection arrival resolves its top-k
        if (sel_role == 2u) {               // offered to the helper: take it back unless taken
            if (tid == 0) s_flag[1] = counter_cas(&p.ws.hready[bg], 6u, 4u) == 6u;
            __syncthreads();
            if (s_flag[1]) pending = bg;
        }

        __syncthreads();
    }

#ifdef LYCHEE_TRACE
    LYCHEE_TRACE_SET(kTrFlags, tr_flags);
    LYCHEE_TRACE_SET(kTrHeads, tr_heads);
#endif
    LYCHEE_STAMP(kTrExit);
}

template <typename T, int D, int G, bool HYBRID, bool BLOCK, bool TOPP>
hipError_t launch_one(const AttendParams& p, int cus, int per_cu, hipStream_t stream) {
    const int grid = attend_grid(cus, per_cu);
    hipLaunchKernelGGL((attend_kernel<T, D, G, HYBRID, BLOCK, TOPP>), dim3(grid), dim3(kAttendThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D, bool HYBRID, bool BLOCK, bool TOPP>
hipError_t launch_g(const AttendParams& p, int G, int cus, int per_cu, hipStream_t stream) {
    switch (G) {
        case 1: return launch_one<T, D, 1, HYBRID, BLOCK, TOPP>(p, cus, per_cu, stream);
        case 2: return launch_one<T, D, 2, HYBRID, BLOCK, TOPP>(p, cus, per_cu, stream);
        case 4: return launch_one<T, D, 4, HYBRID, BLOCK, TOPP>(p, cus, per_cu, stream);
        case 8: return launch_one<T, D, 8, HYBRID, BLOCK, TOPP>(p, cus, per_cu, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, bool HYBRID, bool BLOCK, bool TOPP>
hipError_t launch_d(const AttendParams& p, int D, int G, int cus, int per_cu, hipStream_t stream) {
    if (D == 64) return launch_g<T, 64, HYBRID, BLOCK, TOPP>(p, G, cus, per_cu, stream);
    if (D == 128) return launch_g<T, 128, HYBRID, BLOCK, TOPP>(p, G, cus, per_cu, stream);
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_t(const AttendParams& p, int D, int G, bool hybrid, int cus, int per_cu, hipStream_t stream) {
    if (!hybrid) return launch_d<T, false, false, false>(p, D, G, cus, per_cu, stream);
    // the block and Top-p rules have builds of their own: their cuts stay out of
    // the token top-k build's code and register allocation
    if (p.sel_block) return launch_d<T, true, true, false>(p, D, G, cus, per_cu, stream);
    if (p.sel_zpart) return launch_d<T, true, false, true>(p, D, G, cus, per_cu, stream);
    return launch_d<T, true, false, false>(p, D, G, cus, per_cu, stream);
}

}  // namespace

hipError_t launch_attend(const AttendParams& p, int dtype, int D, int G, bool hybrid, int cus, int per_cu,
                         hipStream_t stream) {
#ifdef LYCHEE_ONE_VARIANT   // compile-time probe of one variant's resources (not a library build)
    return hybrid ? launch_one<BF16, 128, 4, true, false, false>(p, cus, per_cu, stream) : hipErrorInvalidValue;
#endif
    if (dtype == 1) return launch_t<BF16>(p, D, G, hybrid, cus, per_cu, stream);
    if (dtype == 0) return launch_t<F32>(p, D, G, hybrid, cus, per_cu, stream);
    return hipErrorInvalidValue;
}

}  // namespace lychee
