// Per-head top-k of the GQA-pooled selection scores (gfx950).
//
// S^(l+1) = argsTopK(A, k) of Eq. 2 (section 3.4 of the LycheeDecode
// long-form digest), with the hyper-parameter summary's pooling rule, for
// every retrieval KV head: the min(k, n) tokens with the largest pooled score,
// ties to the lower token index, written in ascending token order and padded
// with -1 up to k.  Selection is exact: it is a radix select over the
// order-preserving 32-bit key of the fp32 score followed by the token index,
// so (score desc, index asc) is a strict total order and the result is unique.
//
// Pass structure (no workgroup ever waits for another):
//   1. The attention kernel already built a histogram of the first 12-bit
//      digit of every score.  Each select workgroup reads it and finds the
//      digit T holding the k-th largest key.
//   2. Each workgroup scans a 4096-score segment: keys whose first digit is
//      above T are certainly selected (their indices are appended to a list),
//      keys in digit T are candidates ((key, index) appended to another list).
//   3. The last workgroup of the head to arrive resolves the candidates by
//      radix select on the remaining key bits and the index (in LDS; a
//      candidate set larger than the LDS buffer is first narrowed by passes
//      over global memory), marks every selected index in an LDS bitmap of the
//      context, and emits the set bits in ascending order.
//   It then clears the head's histogram and counters for the next call.
#include "common.hpp"

namespace lychee {
namespace {

constexpr int kThr = kSelectThreads;
constexpr int kPerThread = kSelectSeg / kThr;          // 16 scores per thread in a segment
constexpr int kLowBits = 32 - kHistBits;               // key bits left after the first digit
constexpr uint32_t kIdxMask = (1u << kIdxBits) - 1u;
constexpr int kCompBits = kLowBits + kIdxBits;         // 38-bit composite (low key bits, inverted index)
constexpr int kWords = kMaxCtx / 32;                   // bitmap words
constexpr int kWordsPerThread = kWords / kThr;         // 32
constexpr int kCandPerThread = kCandLds / kThr;        // 32

__device__ __forceinline__ unsigned long long pack_cand(uint32_t key, uint32_t idx) {
    return ((unsigned long long)idx << 32) | key;
}
__device__ __forceinline__ uint2 unpack_cand(unsigned long long v) {
    return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
    return ((uint64_t)(key & ((1u << kLowBits) - 1u)) << kIdxBits) | (uint64_t)(kIdxMask - idx);
}
__device__ __forceinline__ uint32_t comp_index(uint64_t c) {
    return kIdxMask - (uint32_t)(c & kIdxMask);
}
__device__ __forceinline__ uint32_t comp_digit(uint64_t c, int shift, int bits) {
    return (uint32_t)(c >> shift) & ((1u << bits) - 1u);
}

// Block-wide exclusive prefix sum of one value per thread.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    __syncthreads();
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int wv = 0; wv < kThr / 64; ++wv) {
        if (wv < wave) base += s_wave[wv];
        tot += s_wave[wv];
    }
    *total = tot;
    return base + inc - v;
}

// Find the digit D of an `nbins` histogram (bins read through `bin(i)`) such
// that (count of bins above D) < need <= (count of bins >= D).  Every thread
// calls; the result lands in s_res[0] (digit) and s_res[1] (count above D).
template <typename BinFn>
__device__ void find_crossing(BinFn bin, int nbins, uint32_t need, uint32_t* s_wave, uint32_t* s_res) {
    const int per = (nbins + kThr - 1) / kThr;
    const int r0 = threadIdx.x * per;                   // descending rank of my first bin
    uint32_t sum = 0;
    for (int i = 0; i < per; ++i) {
        const int rank = r0 + i;
        if (rank < nbins) sum += bin(nbins - 1 - rank);
    }
    uint32_t tot;
    const uint32_t before = block_exclusive_scan(sum, s_wave, &tot);
    if (before < need && need <= before + sum) {
        uint32_t acc = before;
        for (int i = 0; i < per; ++i) {
            const int rank = r0 + i;
            if (rank >= nbins) break;
            const uint32_t c = bin(nbins - 1 - rank);
            if (acc + c >= need) {
                s_res[0] = (uint32_t)(nbins - 1 - rank);
                s_res[1] = acc;
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kThr) select_kernel(const SelectParams p) {
    __shared__ uint32_t s_bits[kWords];
    __shared__ uint64_t s_comp[kCandLds];
    __shared__ uint32_t s_h[256];
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_wave[kThr / 64];
    __shared__ uint32_t s_res[4];
    __shared__ uint32_t s_base[2];
    __shared__ uint32_t s_ctr;
    __shared__ int s_flag;

    const int tid = threadIdx.x;
    const int seg = blockIdx.x;
    const int b = blockIdx.y / p.n_retrieval;
    const int rsel = blockIdx.y - b * p.n_retrieval;
    int g = -1;
    {
        int seen = 0;
        for (int i = 0; i < p.Hkv; ++i) {
            if ((p.role_bits >> i) & 1ull) {
                if (seen == rsel) { g = i; break; }
                ++seen;
            }
        }
    }
    if (g < 0) return;
    const int bg = b * p.Hkv + g;
    const int n = p.n_ctx[b];
    const uint32_t ke = (uint32_t)min(p.k, n);
    const int nseg = (n + kSelectSeg - 1) / kSelectSeg;
    if (seg >= nseg) return;

    uint32_t* hist = p.ws.hist + (size_t)bg * kHistBins;
    uint32_t* selcnt = p.ws.selcnt + (size_t)bg * 4;
    const float* scores = p.ws.scores + (size_t)bg * p.ws.sstride;
    int32_t* above = p.ws.above + (size_t)bg * p.k_max;
    unsigned long long* cand = reinterpret_cast<unsigned long long*>(p.ws.cand) + (size_t)bg * p.max_ctx;

    // ---- 1. threshold digit of the first 12 bits (histogram staged in LDS
    // with one batched load) ----
    {
        constexpr int V4 = kHistBins / 4 / kThr;   // uint4 per thread
        uint4 hv[V4];
#pragma unroll
        for (int j = 0; j < V4; ++j) hv[j] = reinterpret_cast<const uint4*>(hist)[tid + kThr * j];
#pragma unroll
        for (int j = 0; j < V4; ++j) reinterpret_cast<uint4*>(s_hist)[tid + kThr * j] = hv[j];
        __syncthreads();
    }
    find_crossing([&](int i) { return s_hist[i]; }, kHistBins, ke, s_wave, s_res);
    const uint32_t T = s_res[0];
    const uint32_t n_above_digit = s_res[1];

    // ---- 2. scan my segment ----
    uint32_t keys[kPerThread];
    uint32_t cls = 0;          // 2 bits per element: 1 above, 2 candidate
    uint32_t a_cnt = 0, c_cnt = 0;
    const int j0 = seg * kSelectSeg;
#pragma unroll
    for (int c = 0; c < kPerThread / 4; ++c) {
        const int j = j0 + 4 * (tid + kThr * c);
        float4 v4;
        if (j + 3 < n) {
            v4 = *reinterpret_cast<const float4*>(scores + j);
        } else {
            v4.x = (j + 0 < n) ? scores[j + 0] : 0.0f;
            v4.y = (j + 1 < n) ? scores[j + 1] : 0.0f;
            v4.z = (j + 2 < n) ? scores[j + 2] : 0.0f;
            v4.w = (j + 3 < n) ? scores[j + 3] : 0.0f;
        }
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int slot = 4 * c + e;
            const uint32_t key = float_key(vv[e]);
            keys[slot] = key;
            const uint32_t dg = key >> kLowBits;
            const bool valid = (j + e) < n;
            if (valid && dg > T) { cls |= 1u << (2 * slot); ++a_cnt; }
            else if (valid && dg == T) { cls |= 2u << (2 * slot); ++c_cnt; }
        }
    }
    uint32_t tot_packed;
    const uint32_t pref = block_exclusive_scan((a_cnt << 16) | c_cnt, s_wave, &tot_packed);
    if (tid == 0) {
        const uint32_t ta = tot_packed >> 16, tc = tot_packed & 0xFFFFu;
        s_base[0] = ta ? atomicAdd(&selcnt[1], ta) : 0u;
        s_base[1] = tc ? atomicAdd(&selcnt[2], tc) : 0u;
    }
    __syncthreads();
    {
        uint32_t pa = s_base[0] + (pref >> 16);
        uint32_t pc = s_base[1] + (pref & 0xFFFFu);
#pragma unroll
        for (int c = 0; c < kPerThread / 4; ++c) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int slot = 4 * c + e;
                const uint32_t cl = (cls >> (2 * slot)) & 3u;
                const uint32_t j = (uint32_t)(j0 + 4 * (tid + kThr * c) + e);
                if (cl == 1u) {
                    if (pa < (uint32_t)p.k_max) coherent_store(&above[pa], (int32_t)j);
                    ++pa;
                } else if (cl == 2u) {
                    if (pc < (uint32_t)p.max_ctx) coherent_store(&cand[pc], pack_cand(keys[slot], j));
                    ++pc;
                }
            }
        }
    }

    // ---- arrival ----
    wait_stores_complete();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = counter_add(&selcnt[0], 1u);
        const int last = (int)(old + 1u == (uint32_t)nseg);
        if (last) counter_reset(&selcnt[0]);
        s_flag = last;
    }
    __syncthreads();
    if (!s_flag) return;

    // ---- 3. the last workgroup resolves the head ----
    const int W = (n + 31) >> 5;
    for (int i = tid; i < W; i += kThr) s_bits[i] = 0u;
    const uint32_t n_above = min(coherent_load(&selcnt[1]), (uint32_t)p.k_max);
    uint32_t c_left = min(coherent_load(&selcnt[2]), (uint32_t)p.max_ctx);
    uint32_t r_left = ke - n_above_digit;
    __syncthreads();
    for (uint32_t base = 0; base < n_above; base += kThr * kPerThread) {
        int32_t av[kPerThread];
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) av[e] = coherent_load(&above[min(base + tid + (uint32_t)(kThr * e), n_above - 1)]);
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
            if (base + tid + (uint32_t)(kThr * e) < n_above) {
                const uint32_t j = (uint32_t)av[e];
                atomicOr(&s_bits[j >> 5], 1u << (j & 31));
            }
        }
    }

    int shift = kCompBits;         // bits of the composite not yet resolved: [0, shift)
    bool done = false;
    if (r_left == c_left) {
        for (uint32_t base = 0; base < c_left; base += kThr * kPerThread) {
            uint2 cv[kPerThread];
#pragma unroll
            for (int e = 0; e < kPerThread; ++e) cv[e] = unpack_cand(coherent_load(&cand[min(base + tid + (uint32_t)(kThr * e), c_left - 1)]));
#pragma unroll
            for (int e = 0; e < kPerThread; ++e) {
                if (base + tid + (uint32_t)(kThr * e) < c_left) {
                    const uint32_t j = cv[e].y;
                    atomicOr(&s_bits[j >> 5], 1u << (j & 31));
                }
            }
        }
        done = true;
    }

    // narrow an oversized candidate set with passes over global memory
    while (!done && c_left > (uint32_t)kCandLds) {
        if (shift == 0) {          // unreachable: composites are distinct
            if (tid == 0) atomicOr(p.ws.err, 2u);
            done = true;
            break;
        }
        const int bits = shift >= 8 ? 8 : shift;
        shift -= bits;
        for (int i = tid; i < 256; i += kThr) s_h[i] = 0u;
        __syncthreads();
        for (uint32_t base = 0; base < c_left; base += kThr * kPerThread) {
            uint2 cv[kPerThread];
#pragma unroll
            for (int e = 0; e < kPerThread; ++e) cv[e] = unpack_cand(coherent_load(&cand[min(base + tid + (uint32_t)(kThr * e), c_left - 1)]));
#pragma unroll
            for (int e = 0; e < kPerThread; ++e)
                if (base + tid + (uint32_t)(kThr * e) < c_left)
                    atomicAdd(&s_h[comp_digit(composite(cv[e].x, cv[e].y), shift, bits)], 1u);
        }
        __syncthreads();
        find_crossing([&](int i) { return s_h[i]; }, 1 << bits, r_left, s_wave, s_res);
        const uint32_t D = min(s_res[0], (1u << bits) - 1u), gt = s_res[1];
        const uint32_t keep = s_h[D];
        if (tid == 0) s_ctr = 0u;
        __syncthreads();
        for (uint32_t c0 = 0; c0 < c_left; c0 += kThr * kPerThread) {
            uint2 mine[kPerThread];
            uint32_t dg[kPerThread];
#pragma unroll
            for (int e = 0; e < kPerThread; ++e) {
                const uint32_t i = c0 + tid + (uint32_t)(kThr * e);
                mine[e] = unpack_cand(coherent_load(&cand[min(i, c_left - 1)]));
                dg[e] = (i < c_left) ? comp_digit(composite(mine[e].x, mine[e].y), shift, bits) : 0xFFFFFFFFu;
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < kPerThread; ++e) {
                if (dg[e] == 0xFFFFFFFFu) continue;
                if (dg[e] > D) {
                    const uint32_t j = mine[e].y;
                    atomicOr(&s_bits[j >> 5], 1u << (j & 31));
                } else if (dg[e] == D) {
                    coherent_store(&cand[atomicAdd(&s_ctr, 1u)], pack_cand(mine[e].x, mine[e].y));
                }
            }
            wait_stores_complete();
            __syncthreads();
        }
        r_left -= gt;
        c_left = keep;
        if (r_left == 0u) {
            done = true;
        } else if (r_left == c_left) {
            for (uint32_t base = 0; base < c_left; base += kThr * kPerThread) {
                uint2 cv[kPerThread];
#pragma unroll
                for (int e = 0; e < kPerThread; ++e) cv[e] = unpack_cand(coherent_load(&cand[min(base + tid + (uint32_t)(kThr * e), c_left - 1)]));
#pragma unroll
                for (int e = 0; e < kPerThread; ++e) {
                    if (base + tid + (uint32_t)(kThr * e) < c_left) {
                        const uint32_t j = cv[e].y;
                        atomicOr(&s_bits[j >> 5], 1u << (j & 31));
                    }
                }
            }
            done = true;
        }
        __syncthreads();
    }

    if (!done) {
        // resolve in LDS
        for (uint32_t base = 0; base < c_left; base += kThr * kPerThread) {
            uint2 cv[kPerThread];
#pragma unroll
            for (int e = 0; e < kPerThread; ++e) cv[e] = unpack_cand(coherent_load(&cand[min(base + tid + (uint32_t)(kThr * e), c_left - 1)]));
#pragma unroll
            for (int e = 0; e < kPerThread; ++e) {
                const uint32_t i = base + tid + (uint32_t)(kThr * e);
                if (i < c_left) s_comp[i] = composite(cv[e].x, cv[e].y);
            }
        }
        __syncthreads();
        while (!done) {
            const int bits = shift >= 8 ? 8 : shift;
            shift -= bits;
            for (int i = tid; i < 256; i += kThr) s_h[i] = 0u;
            __syncthreads();
            uint64_t mine[kCandPerThread];
            uint32_t dg[kCandPerThread];
#pragma unroll
            for (int e = 0; e < kCandPerThread; ++e) {
                const uint32_t i = tid + (uint32_t)(kThr * e);
                mine[e] = (i < c_left) ? s_comp[i] : 0ull;
                dg[e] = (i < c_left) ? comp_digit(mine[e], shift, bits) : 0xFFFFFFFFu;
                if (i < c_left) atomicAdd(&s_h[dg[e]], 1u);
            }
            __syncthreads();
            find_crossing([&](int i) { return s_h[i]; }, 1 << bits, r_left, s_wave, s_res);
            const uint32_t D = min(s_res[0], (1u << bits) - 1u), gt = s_res[1];
            const uint32_t keep = s_h[D];
            if (tid == 0) s_ctr = 0u;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < kCandPerThread; ++e) {
                if (dg[e] == 0xFFFFFFFFu) continue;
                if (dg[e] > D) {
                    const uint32_t j = comp_index(mine[e]);
                    atomicOr(&s_bits[j >> 5], 1u << (j & 31));
                } else if (dg[e] == D) {
                    s_comp[atomicAdd(&s_ctr, 1u)] = mine[e];
                }
            }
            __syncthreads();
            r_left -= gt;
            c_left = keep;
            if (r_left == 0u) {
                done = true;
            } else if (r_left == c_left) {
                for (uint32_t i = tid; i < c_left; i += kThr) {
                    const uint32_t j = comp_index(s_comp[i]);
                    atomicOr(&s_bits[j >> 5], 1u << (j & 31));
                }
                done = true;
            } else if (shift == 0) {
                done = true;   // unreachable: composites are distinct
                if (tid == 0) atomicOr(p.ws.err, 2u);
            }
            __syncthreads();
        }
    }
    __syncthreads();

    // ---- emit the bitmap in ascending order ----
    int32_t* srow = p.S_out + (size_t)bg * p.k;
    const int w0 = tid * kWordsPerThread;
    uint32_t cnt = 0;
#pragma unroll 4
    for (int i = 0; i < kWordsPerThread; ++i)
        if (w0 + i < W) cnt += __popc(s_bits[w0 + i]);
    uint32_t total;
    uint32_t pos = block_exclusive_scan(cnt, s_wave, &total);
    for (int i = 0; i < kWordsPerThread; ++i) {
        if (w0 + i >= W) break;
        uint32_t bitsw = s_bits[w0 + i];
        while (bitsw) {
            const int bit = __ffs(bitsw) - 1;
            bitsw &= bitsw - 1u;
            if (pos < (uint32_t)p.k) srow[pos] = (w0 + i) * 32 + bit;
            ++pos;
        }
    }
    for (int i = (int)ke + tid; i < p.k; i += kThr) srow[i] = -1;
    if (tid == 0 && total != ke) atomicOr(p.ws.err, 2u);

    // ---- restore the zero invariant of this head's histogram and counters ----
    for (int i = tid; i < kHistBins; i += kThr) hist[i] = 0u;
    if (tid == 0) {
        selcnt[1] = 0u;
        selcnt[2] = 0u;
    }
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
    if (p.n_retrieval <= 0) return hipSuccess;
    const int nseg = (p.max_ctx + kSelectSeg - 1) / kSelectSeg;
    hipLaunchKernelGGL(select_kernel, dim3(nseg, p.B * p.n_retrieval), dim3(kThr), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lychee
