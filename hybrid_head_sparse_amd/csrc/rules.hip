// Rule selection after the attention kernel (gfx950): the Top-p and the
// block-granular selection rules.
//
// The attention kernel writes each retrieval head's top-min(k, n) token set to
// S (ascending) and every token's pooled selection key (the order-preserving
// key of the fp32 sum over the G query heads of q . k_j) to the workspace's
// score buffer.  This kernel, launched right after it on the same stream,
// replaces the retrieval rows of S under one of two rules:
//
//   Top-p (one of the selection methods compared in section 4.4.1 / Figure 6
//   of the LycheeDecode digest): the shortest prefix of the ranking (pooled
//   score descending, index ascending) whose share of the softmax of the
//   pooled scores over the whole context reaches p, at most min(k, n) tokens.
//
//   Block (the digest's kernel works on blocks of 64 tokens; a block's score
//   is read as the largest pooled score of its tokens): the floor(k / bs)
//   highest blocks of bs tokens (ties to the lower block), their tokens listed
//   ascending.
//
// kRuleSplit workgroups of 512 threads per (sequence, KV head); sparse heads
// return at once.  Workgroup q of a retrieval head works on slice q:
//   Top-p: the slice's part of the softmax normaliser, z_q = sum 2^((f_j -
//     m_q) c) with m_q the slice's largest key (f the fp32 pooled sum, c =
//     log2(e) / (G sqrt(d)); fp32 terms added in double in a fixed order),
//     published as a partial, and the composites (key << 18 | inverted index:
//     larger = earlier in the ranking) of the slice of the selected entries;
//   Block: the largest key of each of the slice's blocks (wavefront max over
//     the block's lanes), written as the block's composite (key << 18 |
//     inverted block index).
// Each workgroup then counts itself in; the last of the kRuleSplit to arrive
// resets the counter, merges the partials in slice order and cuts the
// composites with an MSD radix: a 256-bin histogram per 8-bit digit of
// weights (Top-p: shares exp(.)/Z in 52-bit fixed point; block: one per
// block), the highest digit whose cumulative weight from the top reaches the
// target (p; floor(k / bs)) fixing the next bits, until a digit's group holds
// a single composite.  Integer weights make the
// LDS atomics' sums independent of their order, so every run cuts the same.
// The radix starts at the highest bit where the composites differ: the
// leading bits (sign and exponent of the key) are shared by most of them,
// and a digit taken there would pile every atomic onto one or two bins.
// Top-p compacts the kept tokens to the front of the row (still ascending)
// and leaves the row as is when the set's total share stays below p; the
// block rule lists the kept blocks in LDS and expands them into S.

#include "common.hpp"
#include "rules.hpp"

namespace lychee {
namespace {

constexpr int kRuleThreads = 512;
constexpr int kRuleWaves = kRuleThreads / 64;
constexpr int kRuleSlots = 16;        // composites the last workgroup holds in registers per thread
constexpr int kDigitBits = 8;         // radix digit: 256 bins, 4 per lane of one wavefront
constexpr int kZBatch = 16;           // score loads in flight per thread
constexpr int kSliceBlocks = kMaxCtx / 16 / kRuleSplit;   // blocks of one slice (bs >= 16)
constexpr uint32_t kIdxMaskP = (1u << kIdxBits) - 1u;

// Inverse of float_key.
__device__ __forceinline__ float key_to_float(uint32_t key) {
    const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
    return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long y = __shfl_xor(v, o);
        v = y < v ? y : v;
    }
    return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long y = __shfl_xor(v, o);
        v = y > v ? y : v;
    }
    return v;
}

// Inclusive max-scan of unsigned values over groups of `grp` lanes (16, 32
// or 64) with DPP: the last lane of each group ends with the group's max.
// Lanes without a DPP source take 0, below every key.
__device__ __forceinline__ uint32_t group_max_scan(uint32_t v, uint32_t grp) {
    auto mx = [](uint32_t a, int b) { return a > (uint32_t)b ? a : (uint32_t)b; };
    v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));   // row_shr:1
    v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));   // row_shr:2
    v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));   // row_shr:4
    v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));   // row_shr:8
    if (grp >= 32u) v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));   // row_bcast:15
    if (grp >= 64u) v = mx(v, __builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));   // row_bcast:31
    return v;
}

__global__ void __launch_bounds__(kRuleThreads) rule_select_kernel(RuleParams p) {
    const int bg = blockIdx.x / kRuleSplit, q = blockIdx.x - bg * kRuleSplit;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    if (!((p.role_bits >> g) & 1ull)) return;          // sparse head: S was forwarded
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool topp = p.mode == kRuleTopP;
    const int n = max(0, min(p.n_ctx[b], p.max_ctx));   // (1 <= n_ctx <= max_ctx by contract)
    if (n == 0) {                                        // out of contract (the attention kernel
        if (q == 0)                                      // flagged it): an empty set
            for (int i = threadIdx.x; i < p.k; i += kRuleThreads) p.S[(size_t)bg * p.k + i] = -1;
        return;
    }
    const uint32_t ke = (uint32_t)min(p.k, n);
    const uint32_t bs = (uint32_t)p.block;
    const uint32_t nb = topp ? 0u : ((uint32_t)n + bs - 1u) / bs;
    const uint32_t nel = topp ? ke : nb;                // composites the cut ranks
    int32_t* srow = p.S + (size_t)bg * p.k;
    const uint32_t* sc = p.score + (size_t)bg * p.max_ctx;
    unsigned long long* cp = p.comp + (size_t)bg * p.max_ctx;
    unsigned long long* rec = p.rec + (size_t)bg * kRuleSplit * 4;

    __shared__ unsigned long long s_hist[1 << kDigitBits];
    __shared__ uint32_t s_hcnt[1 << kDigitBits];
    __shared__ unsigned long long s_rec[kRuleSplit * 4];
    __shared__ double s_d[kRuleWaves];
    __shared__ float s_f[kRuleWaves];
    __shared__ uint32_t s_cnt[kRuleWaves];
    __shared__ unsigned long long s_lo[kRuleWaves], s_hi[kRuleWaves];
    __shared__ unsigned long long s_above, s_cut;
    __shared__ uint32_t s_digit, s_found, s_last, s_single;
    __shared__ uint32_t s_bmax[kSliceBlocks];
    __shared__ uint32_t s_blk[kMaxSelBlocks];

    // ---- slice q ----
    float mq = -INFINITY;
    double zq = 0.0;
    unsigned long long clo = ~0ull, chi = 0ull;     // range of the slice's composites
    if (topp) {
        // the slice's part of the normaliser, in one pass: each thread keeps a
        // running max and its sum rescaled to it; the block merge is fixed-order
        const uint32_t za = (uint32_t)(((uint64_t)n * (uint32_t)q) / kRuleSplit);
        const uint32_t zb = (uint32_t)(((uint64_t)n * (uint32_t)(q + 1)) / kRuleSplit);
        float m_t = -INFINITY;
        double z_t = 0.0;
        for (uint32_t base = za; base < zb; base += kRuleThreads * kZBatch) {
            uint32_t kv[kZBatch];
#pragma unroll
            for (int e = 0; e < kZBatch; ++e) kv[e] = sc[min(base + (uint32_t)tid + (uint32_t)(kRuleThreads * e), zb - 1u)];
            float bm = -INFINITY;
#pragma unroll
            for (int e = 0; e < kZBatch; ++e) bm = fmaxf(bm, key_to_float(kv[e]));   // clamped repeats change no max
            if (bm > m_t) {
                if (m_t != -INFINITY) z_t *= (double)exp2f((m_t - bm) * p.c_log2);
                m_t = bm;
            }
            float zs = 0.0f;
#pragma unroll
            for (int e = 0; e < kZBatch; ++e) {
                const bool valid = base + (uint32_t)tid + (uint32_t)(kRuleThreads * e) < zb;
                zs += valid ? exp2f((key_to_float(kv[e]) - m_t) * p.c_log2) : 0.0f;
            }
            z_t += (double)zs;
        }
        mq = wave_max_f(m_t);
        if (lane == 0) s_f[wave] = mq;
        __syncthreads();
        mq = s_f[0];
#pragma unroll
        for (int w = 1; w < kRuleWaves; ++w) mq = fmaxf(mq, s_f[w]);
        zq = m_t == -INFINITY ? 0.0 : z_t * (double)exp2f((m_t - mq) * p.c_log2);
        zq = wave_sum_d(zq);
        if (lane == 0) s_d[wave] = zq;

        // the slice of the selected entries: composites to the scratch
        const uint32_t ea = (uint32_t)(((uint64_t)ke * (uint32_t)q) / kRuleSplit);
        const uint32_t eb = (uint32_t)(((uint64_t)ke * (uint32_t)(q + 1)) / kRuleSplit);
        bool bad = false;
        for (uint32_t i = ea + (uint32_t)tid; i < eb; i += kRuleThreads) {
            const int32_t j = srow[i];
            bad |= (uint32_t)j >= (uint32_t)n;
            const uint32_t jj = (uint32_t)j < (uint32_t)n ? (uint32_t)j : 0u;
            const unsigned long long c = ((unsigned long long)sc[jj] << kIdxBits) | (unsigned long long)(kIdxMaskP - jj);
            coherent_store(&cp[i], c);
            clo = c < clo ? c : clo;
            chi = c > chi ? c : chi;
        }
        if (bad) atomicOr(p.err, 2u);
    } else {
        // the slice's blocks: each block's largest key.  Loads are coalesced
        // (consecutive tokens in consecutive lanes); a group of min(bs, 64)
        // lanes holds tokens of one block (slices start on a block, batches on
        // a multiple of 64) and a DPP max-scan leaves the group's max in its
        // last lane, which folds it into the block's LDS word (one writer per
        // word when bs <= 64).
        const uint32_t qa = (uint32_t)(((uint64_t)nb * (uint32_t)q) / kRuleSplit);
        const uint32_t qb = (uint32_t)(((uint64_t)nb * (uint32_t)(q + 1)) / kRuleSplit);
        for (uint32_t i = tid; i < qb - qa; i += kRuleThreads) s_bmax[i] = 0u;   // below every key
        __syncthreads();
        const uint32_t t0 = qa * bs, t1 = min((uint32_t)n, qb * bs);
        const uint32_t grp = bs < 64u ? bs : 64u;
        for (uint32_t base = t0; base < t1; base += kRuleThreads * kZBatch) {
            uint32_t kv[kZBatch];
#pragma unroll
            for (int e = 0; e < kZBatch; ++e) {
                const uint32_t j = base + (uint32_t)tid + (uint32_t)(kRuleThreads * e);
                kv[e] = j < t1 ? sc[j] : 0u;
            }
#pragma unroll
            for (int e = 0; e < kZBatch; ++e) {
                const uint32_t v = group_max_scan(kv[e], grp);
                const uint32_t jfirst = base + (uint32_t)tid + (uint32_t)(kRuleThreads * e) - (grp - 1u);
                if ((lane & (grp - 1u)) == grp - 1u && jfirst < t1) atomicMax(&s_bmax[jfirst / bs - qa], v);
            }
        }
        __syncthreads();
        for (uint32_t i = tid; i < qb - qa; i += kRuleThreads) {
            const unsigned long long c = ((unsigned long long)s_bmax[i] << kIdxBits) | (unsigned long long)(kIdxMaskP - (qa + i));
            coherent_store(&cp[qa + i], c);
            clo = c < clo ? c : clo;
            chi = c > chi ? c : chi;
        }
    }
    clo = wave_min_u64(clo);
    chi = wave_max_u64(chi);
    if (lane == 0) {
        s_lo[wave] = clo;
        s_hi[wave] = chi;
    }
    __syncthreads();
    if (tid == 0) {
        double z = 0.0;
        unsigned long long lo = ~0ull, hi = 0ull;
#pragma unroll
        for (int w = 0; w < kRuleWaves; ++w) {
            if (topp) z += s_d[w];
            lo = s_lo[w] < lo ? s_lo[w] : lo;
            hi = s_hi[w] > hi ? s_hi[w] : hi;
        }
        coherent_store(&rec[q * 4 + 0], (unsigned long long)__builtin_bit_cast(uint32_t, mq));
        coherent_store(&rec[q * 4 + 1], __builtin_bit_cast(unsigned long long, z));
        coherent_store(&rec[q * 4 + 2], lo);
        coherent_store(&rec[q * 4 + 3], hi);
    }

    // count in; the last slice to arrive goes on
    wait_stores_complete();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = counter_add(&p.ctr[bg], 1u);
        s_last = old + 1u == (uint32_t)kRuleSplit;
        if (s_last) counter_reset(&p.ctr[bg]);
    }
    __syncthreads();
    if (!s_last) return;

    // ---- the last slice: merge the partials in slice order (every slice's
    // stores completed before it counted in) ----
    if (tid < kRuleSplit * 4) s_rec[tid] = coherent_load(&rec[tid]);
    __syncthreads();
    float fmax = -INFINITY;
    double z = 0.0;
    clo = ~0ull;
    chi = 0ull;
#pragma unroll
    for (int s = 0; s < kRuleSplit; ++s) {
        const unsigned long long lo = s_rec[s * 4 + 2], hi = s_rec[s * 4 + 3];
        fmax = fmaxf(fmax, __builtin_bit_cast(float, (uint32_t)s_rec[s * 4 + 0]));
        clo = lo < clo ? lo : clo;
        chi = hi > chi ? hi : chi;
    }
#pragma unroll
    for (int s = 0; s < kRuleSplit; ++s) {
        const float m = __builtin_bit_cast(float, (uint32_t)s_rec[s * 4 + 0]);
        if (topp && m != -INFINITY) z += __builtin_bit_cast(double, s_rec[s * 4 + 1]) * (double)exp2f((m - fmax) * p.c_log2);
    }
    const double inv_z = topp ? 1.0 / z : 0.0;
    // weight of a composite in the cut
    auto weight = [&](unsigned long long c) -> unsigned long long {
        if (!topp) return 1ull;
        const float f = key_to_float((uint32_t)(c >> kIdxBits));
        return (unsigned long long)((double)exp2f((f - fmax) * p.c_log2) * inv_z * 0x1p52);
    };
    const uint32_t kb = topp ? 0u : min((uint32_t)p.k / bs, nb);   // blocks kept
    const unsigned long long target = topp ? p.P : (unsigned long long)kb;

    // the composites: thread t holds elements [t per, (t + 1) per) (ascending
    // index order across the block), the first kRuleSlots in registers, the
    // rest read from the scratch when needed
    const uint32_t per = (nel + kRuleThreads - 1u) / kRuleThreads;
    const uint32_t e0 = (uint32_t)tid * per;
    unsigned long long cr[kRuleSlots];
#pragma unroll
    for (int e = 0; e < kRuleSlots; ++e) {
        const uint32_t i = e0 + (uint32_t)e;
        cr[e] = ((uint32_t)e < per && i < nel) ? coherent_load(&cp[i]) : 0ull;
    }
    // f(c) for each of this thread's elements, in order
    auto for_each_elem = [&](auto&& f) {
#pragma unroll
        for (int e = 0; e < kRuleSlots; ++e)
            if ((uint32_t)e < per && e0 + (uint32_t)e < nel) f(cr[e]);
        for (uint32_t e = kRuleSlots; e < per; ++e)
            if (e0 + e < nel) f(coherent_load(&cp[e0 + e]));
    };

    // the cut: MSD radix from the highest bit where the composites differ,
    // kDigitBits per digit.  A digit whose group holds one composite ends it:
    // that composite is the cut.  (A single composite overall is kept
    // whatever its weight: Top-p keeps at least one token, and kb >= 1 blocks
    // are kept.)  The block rule keeps every block when kb = nb.
    int shift = clo == chi ? 0 : 64 - __clzll((long long)(clo ^ chi));
    unsigned long long prefix = chi >> shift, above = 0;
    bool cut = topp || kb < nb;
    while (cut && shift > 0) {
        const int bits = shift >= kDigitBits ? kDigitBits : shift;
        const int nshift = shift - bits;
        const uint32_t nbin = 1u << bits;
        for (int i = tid; i < (1 << kDigitBits); i += kRuleThreads) {
            s_hist[i] = 0ull;
            if (topp) s_hcnt[i] = 0u;
        }
        __syncthreads();
        for_each_elem([&](unsigned long long c) {
            if ((c >> shift) == prefix) {
                const uint32_t dg = (uint32_t)(c >> nshift) & (nbin - 1u);
                atomicAdd(&s_hist[dg], weight(c));
                if (topp) atomicAdd(&s_hcnt[dg], 1u);     // (the block rule's weights are counts)
            }
        });
        __syncthreads();
        if (wave == 0) {
            // crossing: lane l holds digits nbin-1-4l .. nbin-4-4l (descending
            // rank 4l .. 4l+3); a wavefront scan gives each its running weight
            unsigned long long h[4], ls = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t t = 4u * (uint32_t)lane + (uint32_t)r;
                h[r] = t < nbin ? s_hist[nbin - 1u - t] : 0ull;
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
                if (lane == 0) s_found = 0u;
            } else if (lane == __ffsll((long long)m) - 1) {
                const uint32_t dg = nbin - 1u - (uint32_t)found;
                s_found = 1u;
                s_digit = dg;
                s_above = before;
                s_single = topp ? s_hcnt[dg] == 1u : h[found & 3] == 1ull;
            }
        }
        __syncthreads();
        if (!s_found) {           // Top-p: the set's share stays below p, keep it whole
            cut = false;
            break;
        }
        prefix = (prefix << bits) | s_digit;
        above = s_above;
        shift = nshift;
        const bool single = s_single;
        __syncthreads();          // s_found / s_digit / s_single are rewritten by the next digit
        if (single && shift > 0) {
            // the digit's group is one composite: it is the cut
            for_each_elem([&](unsigned long long c) {
                if ((c >> shift) == prefix) s_cut = c;
            });
            __syncthreads();
            prefix = s_cut;
            shift = 0;
        }
    }
    if (topp && !cut) return;
    const unsigned long long cutc = cut ? prefix : 0ull;   // keep the composites >= cutc

    // keep the elements at or above the cut in their (ascending index) order,
    // placed by one block scan.  Top-p compacts the tokens in S, the block
    // rule lists the blocks in LDS.
    uint32_t mine = 0;
    for_each_elem([&](unsigned long long c) { mine += c >= cutc ? 1u : 0u; });
    uint32_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) s_cnt[wave] = incl;
    __syncthreads();
    uint32_t at = incl - mine, total = 0;
#pragma unroll
    for (int w = 0; w < kRuleWaves; ++w) {
        at += w < wave ? s_cnt[w] : 0u;
        total += s_cnt[w];
    }
    for_each_elem([&](unsigned long long c) {
        if (c >= cutc) {
            const uint32_t idx = kIdxMaskP - (uint32_t)(c & kIdxMaskP);
            if (topp) srow[at] = (int32_t)idx;
            else if (at < (uint32_t)kMaxSelBlocks) s_blk[at] = idx;
            ++at;
        }
    });
    if (topp) {
        for (uint32_t i = total + (uint32_t)tid; i < ke; i += kRuleThreads) srow[i] = -1;
        return;
    }
    __syncthreads();
    // the block rule: the kept blocks' tokens, ascending (a short last block
    // is the highest kept one, so its missing tokens fall at the end)
    if (tid == 0 && total != kb) atomicOr(p.err, 2u);
    const uint32_t kept = min(total, kb);
    for (uint32_t i = tid; i < (uint32_t)p.k; i += kRuleThreads) {
        const uint32_t r = i / bs;
        int32_t v = -1;
        if (r < kept) {
            const uint32_t tok = s_blk[r] * bs + (i - r * bs);
            v = tok < (uint32_t)n ? (int32_t)tok : -1;
        }
        srow[i] = v;
    }
}

}  // namespace

hipError_t launch_rule_select(const RuleParams& p, hipStream_t stream) {
    const int blocks = p.B * p.Hkv * kRuleSplit;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(rule_select_kernel, dim3(blocks), dim3(kRuleThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lychee
