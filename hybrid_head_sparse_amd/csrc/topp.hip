// Top-p trim of the retrieval rows of S (gfx950).
//
// The Top-p selection rule (one of the selection methods compared in section
// 4.4.1 / Figure 6 of the LycheeDecode digest): a retrieval head keeps the
// shortest prefix of its ranking (pooled score descending, index ascending)
// whose share of the softmax of the pooled scores over the whole context
// reaches p, at most min(k, n) tokens.  The attention kernel has already
// written the head's top-min(k, n) set to S (ascending) and every token's
// pooled key to the workspace's score buffer; this kernel, launched right
// after it on the same stream, cuts that set down to the Top-p prefix.
//
// kTopPSplit workgroups of 512 threads per (sequence, KV head); sparse heads
// return at once.  Workgroup q of a retrieval head:
//   1. takes slice q of the context and sums its part of the softmax
//      normaliser, z_q = sum 2^((f_j - m_q) c) with m_q the slice's largest
//      key (f the fp32 pooled sum, c = log2(e) / (G sqrt(d)); fp32 terms
//      added in double in a fixed order);
//   2. takes slice q of the selected entries and writes their composites
//      (key << 18 | inverted index: larger = earlier in the ranking) to the
//      head's part of the candidate scratch;
//   3. publishes (m_q, z_q) with device-coherent stores and counts
//      itself in; the last of the kTopPSplit to arrive resets the counter and
//      merges the partials in slice order, so the merge and the cut are the
//      same on every run.
// The last workgroup then finds the cut with an MSD radix over the
// composites: shares exp(.)/Z as 52-bit fixed point (sums of integers do not
// depend on the order LDS atomics land in), a 256-bin share histogram per
// 8-bit digit, the highest digit whose cumulative share from the top reaches
// p fixing the next bits.  The radix starts at the highest bit where the
// set's composites differ: the leading bits (sign and exponent of the key)
// are shared by most of the set, and a digit taken there would pile every
// atomic onto one or two bins.  The tokens at or above the cut are compacted
// to the front of the row (still ascending), the rest becomes -1.  If the
// selected set's total share stays below p, the row is left as is.

#include "common.hpp"
#include "topp.hpp"

namespace lychee {
namespace {

constexpr int kTopPThreads = 512;
constexpr int kTopPWaves = kTopPThreads / 64;
constexpr int kTopPSlots = 16;        // composites the last workgroup holds in registers per thread
constexpr int kZBatch = 16;           // score loads in flight per thread for the normaliser
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

__global__ void __launch_bounds__(kTopPThreads) topp_trim_kernel(TopPParams p) {
    const int bg = blockIdx.x / kTopPSplit, q = blockIdx.x - bg * kTopPSplit;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    if (!((p.role_bits >> g) & 1ull)) return;          // sparse head: S was forwarded
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = min(p.n_ctx[b], p.max_ctx);           // (1 <= n_ctx <= max_ctx by contract)
    const uint32_t ke = (uint32_t)min(p.k, n);
    int32_t* srow = p.S + (size_t)bg * p.k;
    const uint32_t* sc = p.score + (size_t)bg * p.max_ctx;
    unsigned long long* cp = p.comp + (size_t)bg * p.max_ctx;
    unsigned long long* rec = p.rec + (size_t)bg * kTopPSplit * 2;

    __shared__ unsigned long long s_hist[256];
    __shared__ double s_d[kTopPWaves];
    __shared__ float s_f[kTopPWaves];
    __shared__ uint32_t s_cnt[kTopPWaves];
    __shared__ unsigned long long s_lo[kTopPWaves], s_hi[kTopPWaves];
    __shared__ unsigned long long s_above;
    __shared__ uint32_t s_digit, s_found, s_last;

    // 1. slice q of the normaliser (its largest key first, then the sum)
    const uint32_t za = (uint32_t)(((uint64_t)n * (uint32_t)q) / kTopPSplit);
    const uint32_t zb = (uint32_t)(((uint64_t)n * (uint32_t)(q + 1)) / kTopPSplit);
    float mq = -INFINITY;
    for (uint32_t base = za; base < zb; base += kTopPThreads * kZBatch) {
        uint32_t kv[kZBatch];
#pragma unroll
        for (int e = 0; e < kZBatch; ++e) kv[e] = sc[min(base + (uint32_t)tid + (uint32_t)(kTopPThreads * e), zb - 1u)];
#pragma unroll
        for (int e = 0; e < kZBatch; ++e) mq = fmaxf(mq, key_to_float(kv[e]));   // clamped repeats change no max
    }
    mq = wave_max_f(mq);
    if (lane == 0) s_f[wave] = mq;
    __syncthreads();
    mq = s_f[0];
#pragma unroll
    for (int w = 1; w < kTopPWaves; ++w) mq = fmaxf(mq, s_f[w]);
    double zq = 0.0;
    for (uint32_t base = za; base < zb; base += kTopPThreads * kZBatch) {
        uint32_t kv[kZBatch];
#pragma unroll
        for (int e = 0; e < kZBatch; ++e) kv[e] = sc[min(base + (uint32_t)tid + (uint32_t)(kTopPThreads * e), zb - 1u)];
        float zs = 0.0f;
#pragma unroll
        for (int e = 0; e < kZBatch; ++e) {
            const bool valid = base + (uint32_t)tid + (uint32_t)(kTopPThreads * e) < zb;
            zs += valid ? exp2f((key_to_float(kv[e]) - mq) * p.c_log2) : 0.0f;
        }
        zq += (double)zs;
    }
    zq = wave_sum_d(zq);
    if (lane == 0) s_d[wave] = zq;

    // 2. slice q of the selected entries: composites to the scratch
    const uint32_t ea = (uint32_t)(((uint64_t)ke * (uint32_t)q) / kTopPSplit);
    const uint32_t eb = (uint32_t)(((uint64_t)ke * (uint32_t)(q + 1)) / kTopPSplit);
    bool bad = false;
    for (uint32_t i = ea + (uint32_t)tid; i < eb; i += kTopPThreads) {
        const int32_t j = srow[i];
        bad |= (uint32_t)j >= (uint32_t)n;
        const uint32_t jj = (uint32_t)j < (uint32_t)n ? (uint32_t)j : 0u;
        coherent_store(&cp[i], ((unsigned long long)sc[jj] << kIdxBits) | (unsigned long long)(kIdxMaskP - jj));
    }
    if (bad) atomicOr(p.err, 2u);
    __syncthreads();

    // 3. publish the partials, count in; the last slice to arrive goes on
    if (tid == 0) {
        double z = 0.0;
#pragma unroll
        for (int w = 0; w < kTopPWaves; ++w) z += s_d[w];
        coherent_store(&rec[q * 2 + 0], (unsigned long long)__builtin_bit_cast(uint32_t, mq));
        coherent_store(&rec[q * 2 + 1], __builtin_bit_cast(unsigned long long, z));
    }
    wait_stores_complete();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = counter_add(&p.ctr[bg], 1u);
        s_last = old + 1u == (uint32_t)kTopPSplit;
        if (s_last) counter_reset(&p.ctr[bg]);
    }
    __syncthreads();
    if (!s_last) return;

    // merge the partials in slice order (every slice's stores completed
    // before it counted in)
    float fmax = -INFINITY;
    float mqs[kTopPSplit];
    double zqs[kTopPSplit];
#pragma unroll
    for (int s = 0; s < kTopPSplit; ++s) {
        mqs[s] = __builtin_bit_cast(float, (uint32_t)coherent_load(&rec[s * 2 + 0]));
        zqs[s] = __builtin_bit_cast(double, coherent_load(&rec[s * 2 + 1]));
        fmax = fmaxf(fmax, mqs[s]);
    }
    double z = 0.0;
#pragma unroll
    for (int s = 0; s < kTopPSplit; ++s)
        if (mqs[s] != -INFINITY) z += zqs[s] * (double)exp2f((mqs[s] - fmax) * p.c_log2);
    const double inv_z = 1.0 / z;
    auto share = [&](unsigned long long c) -> unsigned long long {
        const float f = key_to_float((uint32_t)(c >> kIdxBits));
        return (unsigned long long)((double)exp2f((f - fmax) * p.c_log2) * inv_z * 0x1p52);
    };

    // the composites (entry i = tid + 512 e: slot e in registers for
    // e < kTopPSlots, read from the scratch beyond) and their range
    unsigned long long cr[kTopPSlots];
    unsigned long long clo = ~0ull, chi = 0ull;
#pragma unroll
    for (int e = 0; e < kTopPSlots; ++e) {
        const uint32_t i = (uint32_t)tid + (uint32_t)(kTopPThreads * e);
        cr[e] = i < ke ? coherent_load(&cp[i]) : 0ull;
        if (i < ke) {
            clo = cr[e] < clo ? cr[e] : clo;
            chi = cr[e] > chi ? cr[e] : chi;
        }
    }
    for (uint32_t i = (uint32_t)tid + (uint32_t)(kTopPThreads * kTopPSlots); i < ke; i += kTopPThreads) {
        const unsigned long long c = coherent_load(&cp[i]);
        clo = c < clo ? c : clo;
        chi = c > chi ? c : chi;
    }
    clo = wave_min_u64(clo);
    chi = wave_max_u64(chi);
    if (lane == 0) {
        s_lo[wave] = clo;
        s_hi[wave] = chi;
    }
    __syncthreads();
    clo = s_lo[0];
    chi = s_hi[0];
#pragma unroll
    for (int w = 1; w < kTopPWaves; ++w) {
        clo = s_lo[w] < clo ? s_lo[w] : clo;
        chi = s_hi[w] > chi ? s_hi[w] : chi;
    }

    // the cut: MSD radix from the highest bit where the composites differ (a
    // single composite is kept whatever its share: the rule keeps at least one)
    int shift = clo == chi ? 0 : 64 - __clzll((long long)(clo ^ chi));
    unsigned long long prefix = chi >> shift, above = 0;
    bool cut = true;
    while (shift > 0) {
        const int bits = shift >= 8 ? 8 : shift;
        const int nshift = shift - bits;
        const uint32_t nb = 1u << bits;
        for (int i = tid; i < 256; i += kTopPThreads) s_hist[i] = 0ull;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kTopPSlots; ++e) {
            const uint32_t i = (uint32_t)tid + (uint32_t)(kTopPThreads * e);
            const unsigned long long c = cr[e];
            if (i < ke && (c >> shift) == prefix) atomicAdd(&s_hist[(uint32_t)(c >> nshift) & (nb - 1u)], share(c));
        }
        for (uint32_t i = (uint32_t)tid + (uint32_t)(kTopPThreads * kTopPSlots); i < ke; i += kTopPThreads) {
            const unsigned long long c = coherent_load(&cp[i]);
            if ((c >> shift) == prefix) atomicAdd(&s_hist[(uint32_t)(c >> nshift) & (nb - 1u)], share(c));
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds digits nb-1-4l .. nb-4-4l (descending rank 4l .. 4l+3)
            unsigned long long h[4], ls = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t t = 4u * (uint32_t)lane + (uint32_t)r;
                h[r] = t < nb ? s_hist[nb - 1u - t] : 0ull;
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
                if (found < 0 && run + h[r] >= p.P) {
                    found = 4 * lane + r;
                    before = run;
                }
                run += h[r];
            }
            const unsigned long long m = __ballot(found >= 0);
            if (m == 0ull) {
                if (lane == 0) s_found = 0u;
            } else if (lane == __ffsll((long long)m) - 1) {
                s_found = 1u;
                s_digit = nb - 1u - (uint32_t)found;
                s_above = before;
            }
        }
        __syncthreads();
        if (!s_found) {           // the selected set's share stays below p: keep it whole
            cut = false;
            break;
        }
        prefix = (prefix << bits) | s_digit;
        above = s_above;
        shift = nshift;
        __syncthreads();          // s_found / s_digit are rewritten by the next digit
    }

    // keep the composites at or above the cut, in their (ascending index) order
    if (!cut) return;
    uint32_t base = 0;
    auto emit = [&](unsigned long long c, bool valid) {     // one chunk of kTopPThreads entries, block-uniform
        const bool keep = valid && c >= prefix;
        const unsigned long long m = __ballot(keep);
        const uint32_t below_lane = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) s_cnt[wave] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t off = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < kTopPWaves; ++w) {
            off += w < wave ? s_cnt[w] : 0u;
            tot += s_cnt[w];
        }
        if (keep) srow[base + off + below_lane] = (int32_t)(kIdxMaskP - (uint32_t)(c & kIdxMaskP));
        base += tot;
        __syncthreads();          // s_cnt is rewritten by the next chunk
    };
#pragma unroll
    for (int e = 0; e < kTopPSlots; ++e)
        if ((uint32_t)(kTopPThreads * e) < ke) emit(cr[e], (uint32_t)tid + (uint32_t)(kTopPThreads * e) < ke);
    for (uint32_t c0 = (uint32_t)(kTopPThreads * kTopPSlots); c0 < ke; c0 += kTopPThreads) {
        const uint32_t i = c0 + (uint32_t)tid;
        emit(i < ke ? coherent_load(&cp[i]) : 0ull, i < ke);
    }
    for (uint32_t i = base + (uint32_t)tid; i < ke; i += kTopPThreads) srow[i] = -1;
}

}  // namespace

hipError_t launch_topp_trim(const TopPParams& p, hipStream_t stream) {
    const int blocks = p.B * p.Hkv * kTopPSplit;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(topp_trim_kernel, dim3(blocks), dim3(kTopPThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lychee
