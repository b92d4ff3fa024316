// Rule selection after the attention kernel (gfx950): the Top-p and the
// block-granular selection rules.
//
// The attention kernel writes each retrieval head's top-min(k, n) token set to
// S (ascending) and, under Top-p, every token's pooled selection key (the
// order-preserving key of the fp32 sum over the G query heads of q . k_j) to
// the workspace's score buffer.  This kernel, launched right after it on the
// same stream, replaces the retrieval rows of S under one of two rules:
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
// One workgroup of 512 threads per (sequence, KV head); sparse heads return at
// once.  The attention kernel did the passes over the context:
//   Top-p: each of its workgroups published its part of the normaliser
//     (largest pooled sum m_w, sum of 2^((f - m_w) c) with c = log2(e) /
//     (G sqrt(d))); they are merged here in workgroup order (fixed, so every
//     run sums alike) into Z, and the composites (key << 18 | inverted index:
//     larger = earlier in the ranking) of the selected entries are formed;
//   Block: it folded each block's largest key into the block words; the
//     composites are (key << 18 | inverted block index).
// The composites are cut with an MSD radix: a 256-bin histogram per 8-bit
// digit of weights (Top-p: shares exp(.)/Z in 52-bit fixed point; block: one
// per block), the highest digit whose cumulative weight from the top reaches
// the target (p; floor(k / bs)) fixing the next bits, until a digit's group
// holds a single composite.  Integer weights make the LDS atomics' sums
// independent of their order, so every run cuts the same.  The radix starts
// at the highest bit where the composites differ: the leading bits (sign and
// exponent of the key) are shared by most of them, and a digit taken there
// would pile every atomic onto one or two bins.  Top-p compacts the kept
// tokens to the front of the row (still ascending) and leaves the row as is
// when the set's total share stays below p; the block rule lists the kept
// blocks in LDS and expands them into S.  The block words and the partials'
// tags are restored to zero for the next call.

#include "common.hpp"
#include "rules.hpp"

namespace lychee {
namespace {

constexpr int kRuleThreads = 512;
constexpr int kRuleWaves = kRuleThreads / 64;
constexpr int kRuleSlots = 16;        // composites the last workgroup holds in registers per thread
constexpr int kDigitBits = 8;         // radix digit: 256 bins, 4 per lane of one wavefront
constexpr int kZPer = (kZSlots + kRuleThreads - 1) / kRuleThreads;   // partial slots per thread
constexpr uint32_t kIdxMaskP = (1u << kIdxBits) - 1u;

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

__global__ void __launch_bounds__(kRuleThreads) rule_select_kernel(RuleParams p) {
    const int bg = blockIdx.x;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    if (!((p.role_bits >> g) & 1ull)) return;          // sparse head: S was forwarded
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool topp = p.mode == kRuleTopP;
    const int n = max(0, min(p.n_ctx[b], p.max_ctx));   // (1 <= n_ctx <= max_ctx by contract)
    if (n == 0) {                                        // out of contract (the attention kernel
        for (int i = threadIdx.x; i < p.k; i += kRuleThreads) p.S[(size_t)bg * p.k + i] = -1;   // flagged it)
        return;
    }
    const uint32_t ke = (uint32_t)min(p.k, n);
    const uint32_t bs = (uint32_t)p.block;
    const uint32_t nb = topp ? 0u : ((uint32_t)n + bs - 1u) / bs;
    const uint32_t nel = topp ? ke : nb;                // composites the cut ranks
    int32_t* srow = p.S + (size_t)bg * p.k;
    const uint32_t* sc = p.score + (size_t)bg * p.max_ctx;
    unsigned long long* cp = p.comp + (size_t)bg * p.max_ctx;
    uint32_t* bk = p.bkey + (size_t)bg * p.bkey_stride;

    __shared__ unsigned long long s_hist[1 << kDigitBits];
    __shared__ uint32_t s_hcnt[1 << kDigitBits];
    __shared__ double s_d[kRuleWaves];
    __shared__ float s_f[kRuleWaves];
    __shared__ uint32_t s_cnt[kRuleWaves];
    __shared__ unsigned long long s_lo[kRuleWaves], s_hi[kRuleWaves];
    __shared__ unsigned long long s_above, s_cut;
    __shared__ uint32_t s_digit, s_found, s_single;
    __shared__ uint32_t s_blk[kMaxSelBlocks];

    // ---- the composites: thread t holds elements [t per, (t + 1) per)
    // (ascending index order across the block), the first kRuleSlots in
    // registers, the rest in the scratch (written and read by the same
    // thread).  Loads go out in two rounds: this thread's S entries (Top-p)
    // or block words, with the normaliser partials; then (Top-p) the keys of
    // the S entries. ----
    const uint32_t per = (nel + kRuleThreads - 1u) / kRuleThreads;
    const uint32_t e0 = (uint32_t)tid * per;
    unsigned long long cr[kRuleSlots];
    unsigned long long clo = ~0ull, chi = 0ull;     // range of the composites
    bool bad = false;
    uint32_t iv[kRuleSlots];
#pragma unroll
    for (int e = 0; e < kRuleSlots; ++e) {
        const uint32_t i = e0 + (uint32_t)e;
        iv[e] = 0u;
        if ((uint32_t)e < per && i < nel) iv[e] = topp ? (uint32_t)srow[i] : bk[i];
    }
    uint4 zr[kZPer];
    if (topp) {
#pragma unroll
        for (int e = 0; e < kZPer; ++e) {
            const int sl = tid + kRuleThreads * e;
            zr[e] = sl < p.nslots ? reinterpret_cast<const uint4*>(p.zpart)[sl] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
#pragma unroll
    for (int e = 0; e < kRuleSlots; ++e) {
        const uint32_t i = e0 + (uint32_t)e;
        cr[e] = 0ull;
        if ((uint32_t)e < per && i < nel) {
            if (topp) {
                bad |= iv[e] >= (uint32_t)n;
                const uint32_t jj = iv[e] < (uint32_t)n ? iv[e] : 0u;
                cr[e] = ((unsigned long long)sc[jj] << kIdxBits) | (unsigned long long)(kIdxMaskP - jj);
            } else {
                cr[e] = ((unsigned long long)iv[e] << kIdxBits) | (unsigned long long)(kIdxMaskP - i);
                bk[i] = 0u;                          // below every key, for the next call
            }
            clo = cr[e] < clo ? cr[e] : clo;
            chi = cr[e] > chi ? cr[e] : chi;
        }
    }
    for (uint32_t e = kRuleSlots; e < per; ++e) {    // (more than kRuleSlots per thread)
        const uint32_t i = e0 + e;
        if (i < nel) {
            unsigned long long c;
            if (topp) {
                const uint32_t j = (uint32_t)srow[i];
                bad |= j >= (uint32_t)n;
                const uint32_t jj = j < (uint32_t)n ? j : 0u;
                c = ((unsigned long long)sc[jj] << kIdxBits) | (unsigned long long)(kIdxMaskP - jj);
            } else {
                c = ((unsigned long long)bk[i] << kIdxBits) | (unsigned long long)(kIdxMaskP - i);
                bk[i] = 0u;
            }
            coherent_store(&cp[i], c);
            clo = c < clo ? c : clo;
            chi = c > chi ? c : chi;
        }
    }
    if (bad) atomicOr(p.err, 2u);
    // ---- block reductions: the composites' range and (Top-p) the largest
    // pooled sum over the partials of this head; then the normaliser
    // Z = sum of z_w 2^((m_w - fmax) c), the partials in slot order ----
    float fmax = -INFINITY;
    double z = 0.0;
    if (topp) {
#pragma unroll
        for (int e = 0; e < kZPer; ++e)
            if (zr[e].x == (uint32_t)bg + 1u) fmax = fmaxf(fmax, __builtin_bit_cast(float, zr[e].y));
        fmax = wave_max_f(fmax);
    }
    clo = wave_min_u64(clo);
    chi = wave_max_u64(chi);
    if (lane == 0) {
        s_lo[wave] = clo;
        s_hi[wave] = chi;
        s_f[wave] = fmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kRuleWaves; ++w) {
        clo = s_lo[w] < clo ? s_lo[w] : clo;
        chi = s_hi[w] > chi ? s_hi[w] : chi;
        fmax = fmaxf(fmax, s_f[w]);
    }
    if (topp) {
        double zt = 0.0;
#pragma unroll
        for (int e = 0; e < kZPer; ++e) {
            if (zr[e].x == (uint32_t)bg + 1u) {
                const double zw = __builtin_bit_cast(double, ((unsigned long long)zr[e].w << 32) | zr[e].z);
                zt += zw * (double)exp2f((__builtin_bit_cast(float, zr[e].y) - fmax) * p.c_log2);
                p.zpart[4 * (size_t)(tid + kRuleThreads * e)] = 0u;    // the slot is free again
            }
        }
        zt = wave_sum_d(zt);
        if (lane == 0) s_d[wave] = zt;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kRuleWaves; ++w) z += s_d[w];
    }
    const double inv_z = topp ? 1.0 / z : 0.0;
    // weight of a composite in the cut
    auto weight = [&](unsigned long long c) -> unsigned long long {
        if (!topp) return 1ull;
        const float f = key_float((uint32_t)(c >> kIdxBits));
        return (unsigned long long)((double)exp2f((f - fmax) * p.c_log2) * inv_z * 0x1p52);
    };
    const uint32_t kb = topp ? 0u : min((uint32_t)p.k / bs, nb);   // blocks kept
    const unsigned long long target = topp ? p.P : (unsigned long long)kb;

    // f(c, weight) for each of this thread's elements, in order (the weights
    // of the register slots are computed once)
    unsigned long long wr[kRuleSlots];
#pragma unroll
    for (int e = 0; e < kRuleSlots; ++e) wr[e] = ((uint32_t)e < per && e0 + (uint32_t)e < nel) ? weight(cr[e]) : 0ull;
    auto for_each_elem = [&](auto&& f) {
#pragma unroll
        for (int e = 0; e < kRuleSlots; ++e)
            if ((uint32_t)e < per && e0 + (uint32_t)e < nel) f(cr[e], wr[e]);
        for (uint32_t e = kRuleSlots; e < per; ++e)
            if (e0 + e < nel) {
                const unsigned long long c = coherent_load(&cp[e0 + e]);
                f(c, weight(c));
            }
    };

    if (topp) {
        // The set's whole share (integer weights: the sum is the same in any
        // order).  Below p, no prefix of it reaches p: the row stays as is.
        unsigned long long tot = 0;
        for_each_elem([&](unsigned long long, unsigned long long wt) { tot += wt; });
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
        if (lane == 0) s_lo[wave] = tot;
        __syncthreads();
        tot = 0;
#pragma unroll
        for (int w = 0; w < kRuleWaves; ++w) tot += s_lo[w];
        if (tot < target) return;
        __syncthreads();          // s_lo is not reused below, but keep the waves together
    }

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
            if (topp) s_hist[i] = 0ull;
            s_hcnt[i] = 0u;
        }
        __syncthreads();
        for_each_elem([&](unsigned long long c, unsigned long long wt) {
            if ((c >> shift) == prefix) {
                const uint32_t dg = (uint32_t)(c >> nshift) & (nbin - 1u);
                if (topp) atomicAdd(&s_hist[dg], wt);
                atomicAdd(&s_hcnt[dg], 1u);     // (the block rule's weights are these counts)
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
                h[r] = t < nbin ? (topp ? s_hist[nbin - 1u - t] : (unsigned long long)s_hcnt[nbin - 1u - t]) : 0ull;
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
                s_single = s_hcnt[dg] == 1u;
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
            for_each_elem([&](unsigned long long c, unsigned long long) {
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
    for_each_elem([&](unsigned long long c, unsigned long long) { mine += c >= cutc ? 1u : 0u; });
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
    for_each_elem([&](unsigned long long c, unsigned long long) {
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
    const int blocks = p.B * p.Hkv;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(rule_select_kernel, dim3(blocks), dim3(kRuleThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lychee
