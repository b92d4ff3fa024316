// Pooled split-K decode attention for retrieval and sparse heads (gfx950).
//
// Computes, for every (sequence b, KV head g) of one layer, the single-query
// attention of its G query heads:
//   retrieval head: over all n_b cached tokens (Eq. 1 of section 3.4 of the
//     LycheeDecode long-form digest), plus the GQA-pooled selection score of
//     every token (the hyper-parameter summary's pooling rule) written for the
//     top-k pass, and a histogram of its first radix digit;
//   sparse head: over the min(k, n_b) rows named by S_in (Eq. 3); S is
//     forwarded unchanged.
// All (head, unit) work -- a unit is one streamed key row or one gathered S
// row -- is concatenated into one pool and cut into equal contiguous ranges,
// one per persistent workgroup, as the digest's workload-pooling description
// asks (equal-size splits spread homogeneously over thread blocks).  Each
// range yields one partial (m, l, o) record per head it touches; the records
// of a head are merged with the log-sum-exp rule by the last workgroup to
// finish (two-level, so no workgroup ever merges more than 16 records), again
// as the digest's kernel description has it (partials + LSE combine), but
// fused into the same launch instead of a separate reduction kernel.
//
// CDNA4 mapping: a key row (d elements) is spread over 16 lanes (one DPP row)
// so every lane issues one coalesced 8-32 byte load per row; the G query heads
// of the group share each loaded row.  Each lane forms 16 partial dot products
// (NK = 16/G keys x G heads) and a 4-step DPP reduce-scatter leaves lane x of
// the row with the full dot product of (key x/G, head x%G).  The per-lane key
// and query-head orders are permuted (key i^(x/G), head h^(x%G)) so that the
// reduce-scatter needs no per-lane selects.  The online-softmax running max is
// kept per DPP row and only moved when a tile exceeds it by 2^8 (lazy
// rescaling), so the common path has no cross-lane max broadcast.
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

// Merge `count` records spaced RS floats apart into one (m, l, o) per head.
// If `out` is non-null the normalised output o / l is written there (query
// heads contiguous, D floats each); otherwise the merged record goes to `dst`.
// Every global read is batched (independent loads issued together), so a
// merge costs one or two memory round trips rather than one per record.
template <int D, int G>
__device__ void merge_records(const float* recs, int count, float* dst, float* out, float* s_ml) {
    constexpr int RS = G * (D + 2);
    constexpr int NML = 2 * G;
    constexpr int kBatch = 16;
    const int tid = threadIdx.x;
    const int tot = count * NML;
    for (int base = 0; base < tot; base += kAttendThreads * 4) {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = min(base + tid + kAttendThreads * j, tot - 1);
            v[j] = coherent_load(&recs[(size_t)(i / NML) * RS + (i % NML)]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = base + tid + kAttendThreads * j;
            if (i < tot) s_ml[i] = v[j];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kAttendThreads) {
        const int h = idx / D, t = idx - h * D;
        float M = -INFINITY;
        for (int r = 0; r < count; ++r) M = fmaxf(M, s_ml[r * NML + h]);
        float L = 0.0f, O = 0.0f;
        for (int r0 = 0; r0 < count; r0 += kBatch) {
            float ov[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int r = min(r0 + j, count - 1);
                ov[j] = coherent_load(&recs[(size_t)r * RS + 2 * G + h * D + t]);
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int r = r0 + j;
                if (r < count) {
                    const float sc = safe_scale(s_ml[r * NML + h], M);
                    L += s_ml[r * NML + G + h] * sc;
                    O += ov[j] * sc;
                }
            }
        }
        if (out) {
            out[(size_t)h * D + t] = (L > 0.0f) ? O / L : 0.0f;
        } else {
            coherent_store(&dst[2 * G + h * D + t], O);
            if (t == 0) {
                coherent_store(&dst[h], M);
                coherent_store(&dst[G + h], L);
            }
        }
    }
    __syncthreads();
}

constexpr int kIdxChunk = 2048;   // sparse S positions staged in LDS per pass

template <typename T, int D, int G, bool HYBRID>
__global__ void __launch_bounds__(kAttendThreads) attend_kernel(const AttendParams p) {
    using Ge = Geo<T, D, G>;
    constexpr int EPL = Ge::EPL, NDW = Ge::NDW, NK = Ge::NK, KPW = Ge::KPW, RS = Ge::RS;
    constexpr int LOG2G = Ge::LOG2G;
    constexpr uint32_t STRIDE = kWaves * KPW;          // positions per workgroup tile round

    __shared__ uint32_t s_pref[kMaxBH + 1];
    __shared__ uint32_t s_hist[HYBRID ? kHistBins : 1];
    __shared__ int32_t s_idx[HYBRID ? kIdxChunk : 1];
    __shared__ __attribute__((aligned(16))) float s_p[kWaves][4][16];
    __shared__ float s_wo[kWaves][G][D];
    __shared__ float s_wm[kWaves][G];
    __shared__ float s_wl[kWaves][G];
    __shared__ float s_ml[kLevel2Max * 2 * G];
    __shared__ uint32_t s_part[kAttendThreads / 64];
    __shared__ int s_flag;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int row = lane >> 4, x = lane & 15;
    const int xh = x >> LOG2G, xl = x & (G - 1);
    const int BH = p.B * p.Hkv;
    const int Hq = p.Hkv * G;

    // ---- units per (b, g) and their exclusive prefix (every workgroup redoes
    // this; BH <= 1024 so it is one batched load and a block scan) ----
    {
        constexpr int PER = kMaxBH / kAttendThreads;   // 4 entries per thread
        uint32_t u[PER];
        int nv[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int bg = min(tid * PER + i, BH - 1);
            nv[i] = p.n_ctx[bg / p.Hkv];
        }
        uint32_t tot = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int bg = tid * PER + i;
            uint32_t units = 0;
            if (bg < BH) {
                const int g = bg % p.Hkv;
                const bool retr = !HYBRID || ((p.role_bits >> g) & 1ull);
                units = retr ? (uint32_t)nv[i] : (uint32_t)min(p.k, nv[i]);
            }
            u[i] = units;
            tot += units;
        }
        uint32_t inc = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(inc, off);
            if (lane >= off) inc += y;
        }
        if (lane == 63) s_part[wave] = inc;
        __syncthreads();
        uint32_t base = 0;
        for (int wv = 0; wv < wave; ++wv) base += s_part[wv];
        uint32_t run = base + inc - tot;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int bg = tid * PER + i;
            if (bg <= BH) s_pref[bg] = run;
            run += u[i];
        }
        if (tid == kAttendThreads - 1 && BH == kMaxBH) s_pref[kMaxBH] = run;
        if (HYBRID) {
            for (int i = tid; i < kHistBins; i += kAttendThreads) s_hist[i] = 0u;
        }
        __syncthreads();
    }

    const uint32_t U = s_pref[BH];
    int P = (int)gridDim.x;
    {
        const uint32_t pmax = (U + kMinUnitsPerWG - 1) / kMinUnitsPerWG;
        if ((uint32_t)P > pmax) P = (int)(pmax < 1 ? 1 : pmax);
    }
    const int w = blockIdx.x;
    if (w >= P) return;
    auto range_lo = [&](int ww) -> uint32_t {
        if (ww >= P) return U;
        return (uint32_t)(((uint64_t)ww * U / (uint64_t)P) & ~(uint64_t)(kUnitAlign - 1));
    };
    auto wg_of = [&](uint32_t unit) -> int {
        int ww = (int)(((uint64_t)unit * (uint64_t)P) / (uint64_t)U);
        if (ww >= P) ww = P - 1;
        while (ww > 0 && range_lo(ww) > unit) --ww;
        while (ww + 1 < P && range_lo(ww + 1) <= unit) ++ww;
        return ww;
    };
    const uint32_t lo = range_lo(w), hi = range_lo(w + 1);

    // first (b, g) whose unit range contains lo
    int bg = 0;
    {
        int a = 0, z = BH - 1;
        while (a < z) {
            const int mid = (a + z + 1) >> 1;
            if (s_pref[mid] <= lo) a = mid; else z = mid - 1;
        }
        bg = a;
    }

    for (; bg < BH && s_pref[bg] < hi; ++bg) {
        const uint32_t h0 = s_pref[bg], h1 = s_pref[bg + 1];
        if (h1 <= lo || h1 == h0) continue;
        const uint32_t seg_lo = max(lo, h0) - h0;
        const uint32_t seg_hi = min(hi, h1) - h0;
        const int b = bg / p.Hkv, g = bg - b * p.Hkv;
        const bool retr = !HYBRID || ((p.role_bits >> g) & 1ull);
        const int n = p.n_ctx[b];

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
        float* score_row = (HYBRID && retr) ? p.ws.scores + (size_t)bg * p.ws.sstride : nullptr;

        float m_run = -INFINITY, l_run = 0.0f;
        float o[G][EPL];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
        bool bad_index = false;

        // Load the K/V fragments of the tile starting at position tb of [r_lo, r_hi).
        // Loads are unconditional: positions past r_hi (and invalid S entries)
        // are clamped to a valid row and masked out of the softmax, so the
        // compiler can keep the next tile's loads in flight during compute.
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
                    if (!okk) bad_index = true;
                    if (i == 0) vmine = okk && (rb + (uint32_t)xh < r_hi);
                    tk = okk ? tk : 0;
                    tv = ((unsigned)tv < (unsigned)n) ? tv : 0;
                } else {
                    tk = (int)pk;
                    tv = (int)pv;
                    if (i == 0) vmine = rb + (uint32_t)xh < r_hi;
                }
                if (i == 0) tok_mine = tk;
                load_frag<NDW>(kf[i], kbase + (size_t)tk * kRowDw);
                load_frag<NDW>(vf[i], vbase + (size_t)tv * kRowDw);
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
                        score_row[tok_mine] = pooled;
                        atomicAdd(&s_hist[float_key(pooled) >> (32 - kHistBits)], 1u);
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
                    const float ah = __shfl(alpha, (lane & 48) | h);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[h][e] *= ah;
                }
            }
            const float pr = vmine ? fast_exp2(z - m_run) : 0.0f;
            l_run += pr;

            // broadcast the row's 16 weights to every lane of the row
            s_p[wave][row][x] = pr;
            compiler_fence();
            float pw[16];
            {
                const float4* src = reinterpret_cast<const float4*>(&s_p[wave][row][0]);
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

        if (!HYBRID || retr) {
            stream_range(seg_lo, seg_hi, nullptr);
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
                        s_idx[pos - c_lo] = v[j];
                        if (Sout) Sout[pos] = v[j];
                    }
                }
                __syncthreads();
                stream_range(c_lo, c_hi, s_idx);
            }
            // entries past min(k, n) (the -1 padding of a short context) belong
            // to the workgroup that finishes the head
            if (Sout && h1 <= hi) {
                const uint32_t ke = h1 - h0;
                for (uint32_t i = ke + tid; i < (uint32_t)p.k; i += kAttendThreads) Sout[i] = Srow[i];
            }
        }
        if (bad_index) atomicOr(p.ws.err, 1u);

        // ---- merge the 4 rows of each wavefront, then the 4 wavefronts ----
        const float lrow = row_sum_same_head<G>(l_run);           // head xl, this row
        float M = m_run;
        M = fmaxf(M, __shfl_xor(M, 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        const float sc = safe_scale(m_run, M);
        float lw = lrow * sc;
        lw += __shfl_xor(lw, 16);
        lw += __shfl_xor(lw, 32);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float sch = __shfl(sc, (lane & 48) | h);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float v = o[h][e] * sch;
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                o[h][e] = v;
            }
        }
        if (row == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < EPL; ++e) s_wo[wave][h][x * EPL + e] = o[h][e];
            if (x < G) {
                s_wm[wave][x] = M;
                s_wl[wave][x] = lw;
            }
        }
        __syncthreads();

        float* rec = p.ws.rec1 + (size_t)(w + bg) * RS;
        for (int idx = tid; idx < G * D; idx += kAttendThreads) {
            const int h = idx / D, t = idx - h * D;
            float Mw = -INFINITY;
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) Mw = fmaxf(Mw, s_wm[wv][h]);
            float O = 0.0f, L = 0.0f;
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) {
                const float s = safe_scale(s_wm[wv][h], Mw);
                O += s_wo[wv][h][t] * s;
                L += s_wl[wv][h] * s;
            }
            coherent_store(&rec[2 * G + h * D + t], O);
            if (t == 0) {
                coherent_store(&rec[h], Mw);
                coherent_store(&rec[G + h], L);
            }
        }

        if constexpr (HYBRID) {
            if (retr) {
                uint32_t* gh = p.ws.hist + (size_t)bg * kHistBins;
                for (int i = tid; i < kHistBins; i += kAttendThreads) {
                    const uint32_t c = s_hist[i];
                    if (c) {
                        atomicAdd(&gh[i], c);
                        s_hist[i] = 0u;
                    }
                }
            }
        }

        // ---- arrival: the last workgroup of a group of 16 merges their records;
        // the last group merger produces the output ----
        const int wf = wg_of(h0), wl = wg_of(h1 - 1);
        const int nw = wl - wf + 1;
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
            s_flag = last;
        }
        __syncthreads();
        if (s_flag) {
            const float* grp = p.ws.rec1 + (size_t)(wf + c * kCombineFanIn + bg) * RS;
            float* out_bg = p.out + ((size_t)b * Hq + (size_t)g * G) * D;
            if (nc == 1) {
                merge_records<D, G>(grp, csize, nullptr, out_bg, s_ml);
            } else {
                float* r2 = p.ws.rec2 + ((size_t)bg * kLevel2Max + c) * RS;
                merge_records<D, G>(grp, csize, r2, nullptr, s_ml);
                wait_stores_complete();
                __syncthreads();
                if (tid == 0) {
                    uint32_t* ctr = p.ws.cnt2 + bg;
                    const uint32_t old = counter_add(ctr, 1u);
                    const int last = (int)(old + 1u == (uint32_t)nc);
                    if (last) counter_reset(ctr);
                    s_flag = last;
                }
                __syncthreads();
                if (s_flag) {
                    merge_records<D, G>(p.ws.rec2 + (size_t)bg * kLevel2Max * RS, nc, nullptr, out_bg, s_ml);
                }
            }
        }
        __syncthreads();
    }
}

template <typename T, int D, int G, bool HYBRID>
hipError_t launch_one(const AttendParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((attend_kernel<T, D, G, HYBRID>), dim3(grid), dim3(kAttendThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D, bool HYBRID>
hipError_t launch_g(const AttendParams& p, int G, int grid, hipStream_t stream) {
    switch (G) {
        case 1: return launch_one<T, D, 1, HYBRID>(p, grid, stream);
        case 2: return launch_one<T, D, 2, HYBRID>(p, grid, stream);
        case 4: return launch_one<T, D, 4, HYBRID>(p, grid, stream);
        case 8: return launch_one<T, D, 8, HYBRID>(p, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, bool HYBRID>
hipError_t launch_d(const AttendParams& p, int D, int G, int grid, hipStream_t stream) {
    if (D == 64) return launch_g<T, 64, HYBRID>(p, G, grid, stream);
    if (D == 128) return launch_g<T, 128, HYBRID>(p, G, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attend(const AttendParams& p, int dtype, int D, int G, bool hybrid, int grid,
                         hipStream_t stream) {
    if (dtype == 1) return hybrid ? launch_d<BF16, true>(p, D, G, grid, stream)
                                  : launch_d<BF16, false>(p, D, G, grid, stream);
    if (dtype == 0) return hybrid ? launch_d<F32, true>(p, D, G, grid, stream)
                                  : launch_d<F32, false>(p, D, G, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace lychee
