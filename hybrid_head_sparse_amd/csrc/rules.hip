// Top-p selection after the attention kernel (gfx950).
//
// The attention kernel writes each retrieval head's top-min(k, n) token set to
// S (ascending) and every token's pooled selection key (the order-preserving
// key of the fp32 sum over the G query heads of q . k_j) to the workspace's
// score buffer.  This kernel, launched right after it on the same stream,
// replaces the retrieval rows of S under the Top-p rule (one of the selection
// methods compared in section 4.4.1 / Figure 6 of the LycheeDecode digest):
// the shortest prefix of the ranking (pooled score descending, index
// ascending) whose share of the softmax of the pooled scores over the whole
// context reaches p, at most min(k, n) tokens.  (The block-granular rule is
// cut inside the attention kernel.)
//
// One workgroup of 512 threads per (sequence, KV head); sparse heads return at
// once.  The attention kernel did the pass over the context: each of its
// workgroups published its part of the normaliser (largest pooled sum m_w,
// sum of 2^((f - m_w) c) with c = log2(e) / (G sqrt(d))); they are merged here
// in workgroup order (fixed, so every run sums alike) into Z, and the
// composites (key << 18 | inverted index: larger = earlier in the ranking) of
// the selected entries are formed.  The composites are cut with an MSD radix:
// a 256-bin histogram per 8-bit digit of their shares exp(.)/Z in 52-bit
// fixed point, the highest digit whose cumulative share from the top reaches
// p fixing the next bits, until a digit's group holds a single composite.
// Integer weights make the LDS atomics' sums independent of their order, so
// every run cuts the same.  The radix starts at the highest bit where the
// composites differ: the leading bits (sign and exponent of the key) are
// shared by most of them, and a digit taken there would pile every atomic
// onto one or two bins.  The kept tokens are compacted to the front of the
// row (still ascending); a row whose whole set holds less than p stays as it
// is.  The partials' tags are restored to zero for the next call.

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
    const int n = max(0, min(p.n_ctx[b], p.max_ctx));   // (1 <= n_ctx <= max_ctx by contract)
    if (n == 0) {                                        // out of contract (the attention kernel
        for (int i = threadIdx.x; i < p.k; i += kRuleThreads) p.S[(size_t)bg * p.k + i] = -1;   // flagged it)
        return;
    }
    const uint32_t ke = (uint32_t)min(p.k, n);
    const uint32_t nel = ke;                            // composites the cut ranks
    int32_t* srow = p.S + (size_t)bg * p.k;
    const uint32_t* sc = p.score + (size_t)bg * p.max_ctx;
    unsigned long long* cp = p.comp + (size_t)bg * p.max_ctx;

    __shared__ unsigned long long s_hist[1 << kDigitBits];
    __shared__ uint32_t s_hcnt[1 << kDigitBits];
    __shared__ double s_d[kRuleWaves];
    __shared__ float s_f[kRuleWaves];
    __shared__ uint32_t s_cnt[kRuleWaves];
    __shared__ unsigned long long s_lo[kRuleWaves], s_hi[kRuleWaves];
    __shared__ unsigned long long s_above, s_cut;
    __shared__ uint32_t s_digit, s_found, s_single;

    // ---- the composites: thread t holds elements [t per, (t + 1) per)
    // (ascending index order across the block), the first kRuleSlots in
    // registers, the rest in the scratch (written and read by the same
    // thread).  Loads go out in two rounds: this thread's S entries with the
    // normaliser partials; then the keys of the S entries. ----
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
        if ((uint32_t)e < per && i < nel) iv[e] = (uint32_t)srow[i];
    }
    uint4 zr[kZPer];
#pragma unroll
    for (int e = 0; e < kZPer; ++e) {
        const int sl = tid + kRuleThreads * e;
        zr[e] = sl < p.nslots ? reinterpret_cast<const uint4*>(p.zpart)[sl] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int e = 0; e < kRuleSlots; ++e) {
        const uint32_t i = e0 + (uint32_t)e;
        cr[e] = 0ull;
        if ((uint32_t)e < per && i < nel) {
            bad |= iv[e] >= (uint32_t)n;
            const uint32_t jj = iv[e] < (uint32_t)n ? iv[e] : 0u;
            cr[e] = ((unsigned long long)sc[jj] << kIdxBits) | (unsigned long long)(kIdxMaskP - jj);
            clo = cr[e] < clo ? cr[e] : clo;
            chi = cr[e] > chi ? cr[e] : chi;
        }
    }
    for (uint32_t e = kRuleSlots; e < per; ++e) {    // (more than kRuleSlots per thread)
        const uint32_t i = e0 + e;
        if (i < nel) {
            const uint32_t j = (uint32_t)srow[i];
            bad |= j >= (uint32_t)n;
            const uint32_t jj = j < (uint32_t)n ? j : 0u;
            const unsigned long long c = ((unsigned long long)sc[jj] << kIdxBits) | (unsigned long long)(kIdxMaskP - jj);
            coherent_store(&cp[i], c);
            clo = c < clo ? c : clo;
            chi = c > chi ? c : chi;
        }
    }
    if (bad) atomicOr(p.err, 2u);
    // ---- block reductions: the composites' range and the largest pooled sum
    // over the partials of this head; then the normaliser
    // Z = sum of z_w 2^((m_w - fmax) c), the partials in slot order ----
    float fmax = -INFINITY;
    double z = 0.0;
#pragma unroll
    for (int e = 0; e < kZPer; ++e)
        if (zr[e].x == (uint32_t)bg + 1u) fmax = fmaxf(fmax, __builtin_bit_cast(float, zr[e].y));
    fmax = wave_max_f(fmax);
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
    {
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
    const double inv_z = 1.0 / z;
    // weight of a composite in the cut: its share of the softmax
    auto weight = [&](unsigned long long c) -> unsigned long long {
        const float f = key_float((uint32_t)(c >> kIdxBits));
        return (unsigned long long)((double)exp2f((f - fmax) * p.c_log2) * inv_z * 0x1p52);
    };
    const unsigned long long target = p.P;

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

    {
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
    // whatever its weight: Top-p keeps at least one token.)
    int shift = clo == chi ? 0 : 64 - __clzll((long long)(clo ^ chi));
    unsigned long long prefix = chi >> shift, above = 0;
    bool cut = true;
    while (cut && shift > 0) {
        const int bits = shift >= kDigitBits ? kDigitBits : shift;
        const int nshift = shift - bits;
        const uint32_t nbin = 1u << bits;
        for (int i = tid; i < (1 << kDigitBits); i += kRuleThreads) {
            s_hist[i] = 0ull;
            s_hcnt[i] = 0u;
        }
        __syncthreads();
        for_each_elem([&](unsigned long long c, unsigned long long wt) {
            if ((c >> shift) == prefix) {
                const uint32_t dg = (uint32_t)(c >> nshift) & (nbin - 1u);
                atomicAdd(&s_hist[dg], wt);
                atomicAdd(&s_hcnt[dg], 1u);     // (the group's size: a single composite ends the cut)
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
                s_single = s_hcnt[dg] == 1u;
            }
        }
        __syncthreads();
        if (!s_found) {           // the set's share stays below p: keep it whole
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
    if (!cut) return;
    const unsigned long long cutc = prefix;   // keep the composites >= cutc

    // keep the elements at or above the cut in their (ascending index) order,
    // compacted to the front of the row by one block scan
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
        if (c >= cutc) srow[at++] = (int32_t)(kIdxMaskP - (uint32_t)(c & kIdxMaskP));
    });
    for (uint32_t i = total + (uint32_t)tid; i < ke; i += kRuleThreads) srow[i] = -1;
}

}  // namespace

hipError_t launch_rule_select(const RuleParams& p, hipStream_t stream) {
    const int blocks = p.B * p.Hkv;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(rule_select_kernel, dim3(blocks), dim3(kRuleThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lychee
