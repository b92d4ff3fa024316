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
// axis (a gathered row weighs twice a streamed one) and cut into equal
// contiguous ranges, one per persistent workgroup, as the digest's kernel
// description asks (equal-size splits spread over all thread blocks).  Each
// range yields one partial (m, l, o) record per head it touches; the last
// workgroup of each group of 32 merges the group's records by the
// log-sum-exp rule and the last group merger writes the output (partials +
// LSE combine, fused into the same launch).
//
// Selection without a second pass over the scores.  While streaming, every
// retrieval workgroup keeps the order-preserving 32-bit keys of its pooled
// logits in LDS and counts their first digit (4096 bins, fine where logits
// live).  When a pass is done it takes its own bound: the digit where its
// histogram reaches its share of k plus a margin.  It adds its counts from
// that bound up to the head's global histogram and appends its keys from the
// bound up to the head's candidate list.  The resolver reads the final
// histogram: if no pass's bound exceeds the head's threshold digit T, the
// histogram is exact from T up and the candidates hold every key from T up
// (otherwise it re-reads every key).  It keeps the candidates above T,
// resolves the ones in digit T by the rest of the key and then the token
// index (larger key first, lower index first: a strict total order, so the
// result is exact and unique), marks the winners in an LDS bitmap of the
// context and writes them in ascending order.  The resolve runs on the head's
// first arrival whose range ends in the head (it waits, bounded, for the last
// one) or on the last arrival, whichever votes first.
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
// 32/OPT records are issued before that and land while it runs; the output
// pass then reads the scales as wavefront-uniform (broadcast) LDS words.  If
// `out` is non-null the normalised output o / l is written there (query heads
// contiguous, D floats each); otherwise the merged record goes to `dst` with
// device-coherent stores.
template <int D, int G>
__device__ void merge_records(const float* recs, int count, float* dst, float* out, float* s_ml) {
    constexpr int RS = G * (D + 2);
    constexpr int OPT = (G * D + kAttendThreads - 1) / kAttendThreads;   // outputs per thread
    constexpr int CH = 32 / OPT;                                        // records per load batch
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
constexpr int kCandPerThread = kCandLds / kAttendThreads;

__device__ __forceinline__ unsigned long long pack_cand(uint32_t key, uint32_t idx) {
    return ((unsigned long long)idx << 32) | key;
}
__device__ __forceinline__ unsigned long long composite(uint32_t key, uint32_t idx) {
    return ((unsigned long long)(key & ((1u << kLowBits) - 1u)) << kIdxBits) | (unsigned long long)(kIdxMask - idx);
}
__device__ __forceinline__ uint32_t comp_index(unsigned long long c) { return kIdxMask - (uint32_t)(c & kIdxMask); }
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
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
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

// Crossing of a histogram spread over the block, PER bins per thread held in
// `cnt` (thread t holds the bins of descending rank t*PER .. t*PER+PER-1, i.e.
// bin nbins-1-rank): finds D with (count above D) < need <= (count >= D).
// Result in s_res[0] (digit), s_res[1] (count above D), s_res[3] (count at
// or above D); if the whole histogram holds fewer than `need`, D = 0 and the
// counts above it and in all are returned.
template <int PER>
__device__ void block_crossing(const uint32_t (&cnt)[PER], int nbins, uint32_t need, uint32_t* s_wave,
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

template <typename T, int D, int G, bool HYBRID>
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
    union Lds {
        StreamLds st;
        SelectLds se;
    };
    __shared__ __attribute__((aligned(16))) Lds u;
    __shared__ uint32_t s_pref[kMaxBH + 1];
    __shared__ uint32_t s_bound[kMaxWG + 1];   // cost position where each workgroup's range starts
    __shared__ int32_t s_nctx[kMaxBH];
    __shared__ uint32_t s_ke[kMaxBH];          // tokens a retrieval head of sequence b selects
    __shared__ uint32_t s_wave[kWaves];
    __shared__ uint32_t s_res[4];
    __shared__ uint32_t s_ctr;
    __shared__ uint32_t s_lcnt;       // a pass's kept keys staged so far
    __shared__ int s_flag[2];
    __shared__ uint32_t s_sel[4];     // selection arrival: role, candidates of the head, slice or helpers, slices taken
    __shared__ int s_rel;
    __shared__ uint32_t s_ceq;        // resolver: threshold-digit composites appended so far

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int row = lane >> 4, x = lane & 15;
    const int xh = x >> LOG2G, xl = x & (G - 1);
    const int BH = p.B * p.Hkv;
    const int Hq = p.Hkv * G;

    // ---- prologue: contexts, pool cost per (b, g) and its exclusive prefix ----
    {
        constexpr int PER = kMaxBH / kAttendThreads;   // 4 entries per thread
        int nb[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) nb[i] = p.n_ctx[min(tid * PER + i, p.B - 1)];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (tid * PER + i < p.B) {
                const int n = nb[i];
                // min(k, n), or under the ratio rule min(k, ceil(theta n)) (at least one)
                const double t = ceil(p.sel_ratio * (double)n);
                const uint32_t kr = t < 1.0 ? 1u : (t > (double)n ? (uint32_t)n : (uint32_t)t);
                s_nctx[tid * PER + i] = n;
                s_ke[tid * PER + i] = min((uint32_t)min(p.k, n), kr);
            }
        }
        __syncthreads();
        uint32_t u_[PER];
        uint32_t tot = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int bg = tid * PER + i;
            uint32_t cost = 0;
            if (bg < BH) {
                const int b = bg / p.Hkv, g = bg - b * p.Hkv;
                const int n = s_nctx[b];
                const bool retr = !HYBRID || ((p.role_bits >> g) & 1ull);
                cost = retr ? kCostRetrieval * (uint32_t)n : kCostSparse * (uint32_t)min(p.k, n);
            }
            u_[i] = cost;
            tot += cost;
        }
        uint32_t total;
        uint32_t run = block_exclusive_scan(tot, s_wave, &total);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int bg = tid * PER + i;
            if (bg <= BH) s_pref[bg] = run;
            run += u_[i];
        }
        if (tid == kAttendThreads - 1 && BH == kMaxBH) s_pref[kMaxBH] = run;
        __syncthreads();
    }

    const uint32_t U = s_pref[BH];
    int P = (int)gridDim.x;
    {
        const uint32_t pmax = U / kMinCostPerWG;
        if ((uint32_t)P > pmax) P = (int)(pmax < 1 ? 1 : pmax);
    }
    const int w = blockIdx.x;
    if (w >= P) return;

    auto is_retr = [&](int hb) -> bool { return !HYBRID || ((p.role_bits >> (hb % p.Hkv)) & 1ull); };
    auto head_of = [&](uint32_t c) -> int {     // last (b, g) whose cost range starts at or before c
        int cnt = 0;                              // (wave-parallel: the starts are increasing)
        for (int base = 0; base < BH; base += 64) {
            const int i = base + lane;
            cnt += __popcll(__ballot(i < BH && s_pref[i] <= c));
        }
        return cnt - 1;
    };
    // Workgroup boundaries: the equal split of the cost axis, moved up to the
    // next row boundary of the head it falls in (so every range holds whole
    // rows).  Every workgroup tabulates all P+1 of them once, in parallel.
    const uint32_t qU = U / (uint32_t)P, rU = U % (uint32_t)P;   // ww * rU < P^2 <= 2^22
    for (int ww = tid; ww <= P; ww += kAttendThreads) {
        uint32_t bnd;
        if (ww == 0) {
            bnd = 0u;
        } else if (ww >= P) {
            bnd = U;
        } else {
            const uint32_t raw = (uint32_t)ww * qU + ((uint32_t)ww * rU) / (uint32_t)P;   // = floor(ww U / P)
            int a = 0, z = BH - 1;                 // head holding raw (serial search per thread)
            while (a < z) {
                const int mid = (a + z + 1) >> 1;
                if (s_pref[mid] <= raw) a = mid; else z = mid - 1;
            }
            const uint32_t h0 = s_pref[a], h1 = s_pref[a + 1], off = raw - h0;
            const uint32_t cwa = is_retr(a) ? kCostRetrieval : kCostSparse;
            const uint32_t up = cwa * ((off + cwa - 1u) / cwa);   // next row start
            bnd = min(h0 + up, h1);
        }
        s_bound[ww] = bnd;
    }
    __syncthreads();
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
    // context (slice j starts at bitmap word j W / kResolveSlices, rounded
    // down to 4 words): the final first-digit histogram gives the threshold
    // digit T and the count above it; every key with digit >= T is in the
    // candidate list.  Every slice's resolver reads all of them and reaches the
    // same T and the same winners among the keys of digit T; it marks only the
    // winners inside its slice in the LDS bitmap, counts those below it (its
    // first position in S) and writes its part of S_out.  The resolver that
    // finishes reading the head's histogram and counters last, over all
    // slices, restores them to zero.
    auto resolve_topk = [&](int hb, int n, uint32_t ke, uint32_t C, uint32_t j0, uint32_t j1) {
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
            for (uint32_t i = rlo + tid; i < min(rlo + rlen, (uint32_t)n); i += kAttendThreads) srow[i] = (int32_t)i;
            if (whi == Wn)
                for (int i = n + tid; i < p.k; i += kAttendThreads) srow[i] = -1;
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
            fb = bmaxv > T_;
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
                        srow[min(at, last)] = (int32_t)(rlo + (uint32_t)((i + q) * 32 + bit));   // at < ke unless the counts disagree (flagged below)
                        ++at;
                    }
                }
            }
            if (whi == Wn) {           // the slice holding the end of the context
                // (the threshold rule keeps the winners at or above its floor)
                const uint32_t kept = p.sel_tkey ? min(below_total + total, ke) : ke;
                for (int i = (int)kept + tid; i < p.k; i += kAttendThreads) srow[i] = -1;
                if (tid == 0 && (p.sel_tkey ? below_total + total > ke : below_total + total != ke))
                    atomicOr(p.ws.err, 2u);
            }
        }
        __syncthreads();
    };

    // A retrieval head's top-k is resolved in kResolveSlices slices of its
    // context.  Slice j goes to the head's free selection arrival number j (one
    // whose range ends in the head), a helper, or to the last arrival: the
    // helper polls, once its own work is done, for the last arrival, which
    // still has its record and merges to do, and takes the slice if it gets
    // there first.  Each of the two adds its vote to the slice's rclaim word
    // once: 1 = helper, ready; 2 = helper, gave up waiting; 4 = last.  The
    // first ready vote resolves; the second vote restores the word to zero.
    // The last arrival takes the slices that have no helper without a vote.
    int pend_bg = -1;              // head this workgroup waits for after its range
    uint32_t pend_nw = 0, pend_ke = 0, pend_slice = 0;
    int pend_n = 0;
    auto vote = [&](int word, uint32_t v) -> uint32_t {   // one lane; returns the earlier votes
        const uint32_t old = counter_add(&p.ws.rclaim[word], v);
        if (old != 0u) counter_reset(&p.ws.rclaim[word]);
        return old;
    };

    for (int bg = head_of(lo); bg < BH && s_pref[bg] < hi; ++bg) {
        const uint32_t h0 = s_pref[bg], h1 = s_pref[bg + 1];
        if (h1 <= lo || h1 == h0) continue;
        const int b = bg / p.Hkv, g = bg - b * p.Hkv;
        const bool retr = is_retr(bg);
        const uint32_t cw = retr ? kCostRetrieval : kCostSparse;
        const uint32_t seg_lo = (max(lo, h0) - h0) / cw;     // first row (position) of this head
        const uint32_t seg_hi = (min(hi, h1) - h0) / cw;
        const int n = s_nctx[b];
        const uint32_t ks = (uint32_t)min(p.k, n);         // S entries of the head
        const uint32_t ke = s_ke[b];                          // tokens a retrieval head selects

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
        auto stream_range = [&](uint32_t r_lo, uint32_t r_hi, const int32_t* sidx) {
            uint32_t tb = r_lo + (uint32_t)wave * KPW;
            if (tb >= r_hi) return;
            Frag<NDW> kA[NK], vA[NK], kB[NK], vB[NK];
            int tokA = 0, tokB = 0;
            bool vmA = false, vmB = false;
            load_tile(tb, r_lo, r_hi, sidx, kA, vA, tokA, vmA);
            for (;;) {
                const uint32_t t1 = tb + STRIDE;
                load_tile(t1, r_lo, r_hi, sidx, kB, vB, tokB, vmB);
                compute_tile(kA, vA, tokA, vmA);
                if (t1 >= r_hi) break;
                const uint32_t t2 = t1 + STRIDE;
                load_tile(t2, r_lo, r_hi, sidx, kA, vA, tokA, vmA);
                compute_tile(kB, vB, tokB, vmB);
                if (t2 >= r_hi) break;
                tb = t2;
            }
        };

        int wf, wl;                    // the head's first and last workgroups
        wg_pair(h0, h1 - 1, wf, wl);
        const int nw = wl - wf + 1;
        if (!HYBRID) {
            stream_range(seg_lo, seg_hi, nullptr);
        } else if (retr) {
            uint32_t* sc = p.ws.score + (size_t)bg * p.max_ctx;
            uint32_t* gh = p.ws.hist + (size_t)bg * kHistBins;
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
                // every key to the score buffer (read only if the bound below fails,
                // or by the rule-selection kernel)
                for (uint32_t i = tid; i < len; i += kAttendThreads) coherent_store(&sc[c_lo + i], u.st.keys[i]);
                if (p.sel_keys_only) {     // a later kernel selects from the keys alone
                    for (int i = tid; i < kHistBins; i += kAttendThreads) u.st.hist[i] = 0u;
                    __syncthreads();
                    continue;
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
                if (tid == 0) s_lcnt = 0u;
                block_crossing<kHistPerThread>(hc, kHistBins, need, s_wave, s_res);
                const uint32_t Tw = s_res[0];
                const uint32_t nkeep = s_res[3];                      // keys with digit >= Tw
                // wavefront 0: the pass's bound to the head's bound word and a
                // range of the candidate list for its keys from Tw up (it waits
                // for that reply alone); wavefronts 1-3: the pass's counts from Tw
                // up to the head's histogram (few bins, so few atomics on any one
                // of them; other workgroups add to the same bins), then zeros
                if (wave == 0) {
                    if (tid == 0) {
                        __hip_atomic_fetch_max(&p.ws.bmax[bg], Tw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        s_ctr = nkeep ? (uint32_t)counter_add64(&p.ws.selctr[bg], nkeep) : 0u;
                    }
                } else {
                    for (int i = tid - 64; i < kHistBins; i += kAttendThreads - 64) {
                        const uint32_t cnt = u.st.hist[i];
                        if (cnt && (uint32_t)i >= Tw) atomicAdd(&gh[i], cnt);
                        u.st.hist[i] = 0u;                           // the next pass starts from zero
                    }
                }
                // while the reservation travels: the kept positions to LDS (any
                // order: the selector's result does not depend on it) ...
                {
                    const uint32_t kb = (uint32_t)digit_first_key(Tw);  // Tw <= kTopDigit: a real key
                    for (uint32_t i = tid; i < len; i += kAttendThreads) {
                        if (u.st.keys[i] >= kb) {
                            const uint32_t at = atomicAdd(&s_lcnt, 1u);
                            if (at < (uint32_t)kKeyCap) u.st.gbuf[at] = i;
                        }
                    }
                }
                __syncthreads();
                // ... then out with consecutive device-coherent stores
                {
                    unsigned long long* cand = p.ws.cand + (size_t)bg * p.max_ctx;
                    const uint32_t base = s_ctr, cnt = min(nkeep, (uint32_t)kKeyCap);
                    for (uint32_t j = tid; j < cnt; j += kAttendThreads) {
                        const uint32_t off = u.st.gbuf[j];
                        if (base + j < (uint32_t)p.max_ctx)
                            coherent_store(&cand[base + j], pack_cand(u.st.keys[off], c_lo + off));
                    }
                }
                __syncthreads();
            }
            // Selection arrival, before the record: once its stores (candidates,
            // scores, histogram and bound atomics) complete, this workgroup's
            // part of the head's selection is in place.  Arrivals whose range
            // ends in this head also count as free ones.  Roles in resolving
            // the top-k (below): 1 the last arrival (with the number of helpers
            // before it); 2 one of the first kResolveSlices free arrivals that
            // is not last, a helper for slice number = free arrivals before it.
            wait_stores_complete();
            __syncthreads();
            if (tid == 0 && p.sel_keys_only) s_sel[0] = 0u;   // no top-k to resolve
            if (tid == 0 && !p.sel_keys_only) {
                const bool ends_here = h1 >= hi;
                const unsigned long long o64 =
                    counter_add64(&p.ws.selctr[bg], kSelArrival | (ends_here ? kSelFreeArrival : 0ull));
                const uint32_t before = (uint32_t)(o64 >> 32) & 0xFFFFu;   // arrivals before this one
                const uint32_t free_before = (uint32_t)(o64 >> 48);
                const bool last = before + 1u == (uint32_t)nw;
                s_sel[0] = last ? 1u : (ends_here && free_before < (uint32_t)kResolveSlices ? 2u : 0u);
                s_sel[1] = (uint32_t)o64;                // candidates of the whole head when last
                s_sel[2] = last ? min(free_before, (uint32_t)kResolveSlices) : free_before;
            }
        } else {
            // sparse head: stage the S entries of the range in LDS (one batched
            // load per chunk), forward them to S_out, then gather-stream
            const int32_t* Srow = p.S_in + (size_t)bg * p.k;
            int32_t* Sout = (p.S_out != p.S_in) ? p.S_out + (size_t)bg * p.k : nullptr;
            constexpr int PER = kIdxChunk / kAttendThreads;
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
                stream_range(c_lo, c_hi, u.st.idx);
            }
            // entries past min(k, n) (the -1 padding of a short context) belong
            // to the workgroup that finishes the head
            if (Sout && h1 <= hi) {
                for (uint32_t i = ks + tid; i < (uint32_t)p.k; i += kAttendThreads) Sout[i] = Srow[i];
            }
        }
        if (bad_index) atomicOr(p.ws.err, 1u);

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
        __syncthreads();
        if (tid == 0) {
            uint32_t* ctr = p.ws.cnt1 + (size_t)bg * kLevel2Max + c;
            const uint32_t old = counter_add(ctr, 1u);
            const int last = (int)(old + 1u == (uint32_t)csize);
            if (last) counter_reset(ctr);
            s_flag[0] = last;
        }
        __syncthreads();
        const uint32_t sel_role = (HYBRID && retr) ? s_sel[0] : 0u;
        const uint32_t C_head = s_sel[1];
        const uint32_t sel_aux = s_sel[2];           // helpers before the last arrival, or a helper's slice
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
        }
        if (sel_role == 1u) {
            // the last arrival votes on each slice that has a helper and takes
            // the slices with none, or whose helper gave up or is still waiting
            if (wave == 0) {
                uint32_t old = 0;
                if (lane < kResolveSlices && (uint32_t)lane < sel_aux)
                    old = vote(bg * kResolveSlices + lane, 4u);
                const unsigned long long take = __ballot(lane < kResolveSlices && (old == 0u || old == 2u));
                if (lane == 0) s_sel[3] = (uint32_t)take;
            }
            __syncthreads();
            const uint32_t take = s_sel[3];
            for (uint32_t j0 = 0; j0 < (uint32_t)kResolveSlices;) {     // each run of taken slices at once
                if (!((take >> j0) & 1u)) {
                    ++j0;
                    continue;
                }
                uint32_t j1 = j0 + 1u;
                while (j1 < (uint32_t)kResolveSlices && ((take >> j1) & 1u)) ++j1;
                resolve_topk(bg, n, ke, C_head, j0, j1);
                j0 = j1;
            }
        } else if (sel_role == 2u) {   // the range ends in this head: wait and vote after the loop
            pend_bg = bg;
            pend_nw = (uint32_t)nw;
            pend_n = n;
            pend_ke = ke;
            pend_slice = sel_aux;
        }

        __syncthreads();
    }

    if (HYBRID && pend_bg >= 0) {
        if (tid == 0) {
            // wait (bounded) for the last arrival, or for its vote
            uint32_t ready = 0, C = 0;
            for (int it = 0; it < kResolveWaitPolls; ++it) {
                const unsigned long long s = coherent_load(&p.ws.selctr[pend_bg]);
                const uint32_t votes = coherent_load(&p.ws.rclaim[pend_bg * kResolveSlices + pend_slice]);
                if (((uint32_t)(s >> 32) & 0xFFFFu) == pend_nw) {
                    ready = 1;
                    C = (uint32_t)s;
                    break;
                }
                if (votes != 0u) break;     // the last arrival voted first
                __builtin_amdgcn_s_sleep(4);
            }
            const uint32_t old = vote(pend_bg * kResolveSlices + pend_slice, ready ? 1u : 2u);
            s_flag[0] = ready && old == 0u;
            s_res[2] = C;
        }
        __syncthreads();
        if (s_flag[0]) resolve_topk(pend_bg, pend_n, pend_ke, s_res[2], pend_slice, pend_slice + 1u);
    }
}

template <typename T, int D, int G, bool HYBRID>
hipError_t launch_one(const AttendParams& p, int cus, int per_cu, hipStream_t stream) {
    int grid = cus * per_cu;
    if (grid > kMaxWG) grid = kMaxWG;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((attend_kernel<T, D, G, HYBRID>), dim3(grid), dim3(kAttendThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D, bool HYBRID>
hipError_t launch_g(const AttendParams& p, int G, int cus, int per_cu, hipStream_t stream) {
    switch (G) {
        case 1: return launch_one<T, D, 1, HYBRID>(p, cus, per_cu, stream);
        case 2: return launch_one<T, D, 2, HYBRID>(p, cus, per_cu, stream);
        case 4: return launch_one<T, D, 4, HYBRID>(p, cus, per_cu, stream);
        case 8: return launch_one<T, D, 8, HYBRID>(p, cus, per_cu, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, bool HYBRID>
hipError_t launch_d(const AttendParams& p, int D, int G, int cus, int per_cu, hipStream_t stream) {
    if (D == 64) return launch_g<T, 64, HYBRID>(p, G, cus, per_cu, stream);
    if (D == 128) return launch_g<T, 128, HYBRID>(p, G, cus, per_cu, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attend(const AttendParams& p, int dtype, int D, int G, bool hybrid, int cus, int per_cu,
                         hipStream_t stream) {
    if (dtype == 1) return hybrid ? launch_d<BF16, true>(p, D, G, cus, per_cu, stream)
                                  : launch_d<BF16, false>(p, D, G, cus, per_cu, stream);
    if (dtype == 0) return hybrid ? launch_d<F32, true>(p, D, G, cus, per_cu, stream)
                                  : launch_d<F32, false>(p, D, G, cus, per_cu, stream);
    return hipErrorInvalidValue;
}

}  // namespace lychee
