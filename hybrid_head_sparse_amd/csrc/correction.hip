// The multi-step loop around the hybrid step (gfx950): the cache append of
// Algorithm 1 and the attention of the digest's Cache Correction, the dense
// re-prefill over the last T <= 32 decoded tokens every 32 steps (section
// 4.2.2 of the LycheeDecode digest).  Only the attention part is computed:
// each of the last T positions p = n - T + t attends, for every query head,
// densely and causally to cache rows 0..p with its own query.
//
// Correction attention.  Per KV head this is a (T G) x n x d contraction, so
// it runs on the matrix cores: v_mfma_f32_32x32x8_bf16 (bf16 operands, fp32
// accumulation).  A workgroup takes one (sequence, KV head) and one chunk of
// its context; wavefront w is query head g G + w and holds that head's T
// queries (padded to 32) as the 32 columns of its tiles.  Per tile of 32 keys:
//   S^T = K Q^T          (16 MFMAs over d = 128; K straight from memory,
//                         each lane a contiguous 128 bytes of one key row)
//   causal mask, online softmax in the log2 domain (each lane holds 16 keys
//   of one query; one exchange with the other half-wave gives the tile max)
//   O += P V             (16 MFMAs: the 16 probabilities a lane holds are,
//                         converted to bf16, exactly its A operand; V is
//                         staged transposed in LDS, double-buffered, so each
//                         B operand is one 8-byte LDS read)
// The contraction over d uses the order lane half h -> d in [64 h, 64 h + 64)
// for both K and Q (any common order of d gives the same dot products).  A
// chunk's per-query partials (max, sum, unnormalised O) go to the workspace
// and a second kernel merges the chunks by the log-sum-exp rule.
//
// Lane layout of v_mfma_f32_32x32x8_bf16 (checked on the device): lane l
// holds A[l % 32][4 (l / 32) + i], B[4 (l / 32) + i][l % 32] (i < 4) and
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] in accumulator r < 16.

#include "common.hpp"
#include "correction.hpp"

namespace lychee {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kD = 128;               // head dim of the MFMA path
constexpr int kTile = 32;             // keys per tile
constexpr int kVtStride = kTile + 4;  // bf16 per transposed V row in LDS (padded)

__device__ __forceinline__ short f2bf(float f) {       // round to nearest even
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (short)(u >> 16);
}

// row of accumulator register r for lane half h
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int G>
__global__ void __launch_bounds__(64 * G) correction_partial_kernel(CorrParams p) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, c32 = lane & 31;
    const int bg = blockIdx.x / p.nchunks, chunk = blockIdx.x - bg * p.nchunks;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    const int n = min(p.n_ctx[b], p.max_ctx);
    const int T = p.T;
    const int Hq = p.Hkv * G;
    if (n < T) {                       // out of contract: flagged, partials stay empty
        if (threadIdx.x == 0 && chunk == 0) atomicOr(p.err, 4u);
    }
    const int c0 = (int)(((long long)n * chunk) / p.nchunks);
    const int c1 = (int)(((long long)n * (chunk + 1)) / p.nchunks);
    const size_t kv_row0 = (size_t)bg * p.max_ctx;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(p.kc);
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(p.vc);

    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kD * kVtStride];
    __shared__ float s_alpha[G][32];

    // this lane's query: t = c32 (rows t >= T repeat row T - 1, ignored at the end)
    const int tq = min(c32, T - 1);
    const int pos_q = n - T + c32;     // causal limit of query c32 (keys <= pos_q)
    v4s qop[16];
    {
        const uint4* qr = reinterpret_cast<const uint4*>(
            reinterpret_cast<const uint16_t*>(p.q) + (((size_t)b * T + tq) * Hq + (size_t)g * G + w) * kD + 64 * h);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint4 v = qr[c];
            qop[2 * c] = __builtin_bit_cast(v4s, make_uint2(v.x, v.y));
            qop[2 * c + 1] = __builtin_bit_cast(v4s, make_uint2(v.z, v.w));
        }
    }
    v16f acc_o[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) acc_o[t4] = v16f{};
    float m_run = -INFINITY, l_part = 0.0f;

    // stage the V tile starting at key k0 into s_vt[buf], transposed
    auto stage_v = [&](int k0, int buf) {
        constexpr int kChunks = kTile * kD / 8;              // 16-byte pieces of the tile
#pragma unroll
        for (int ci = threadIdx.x; ci < kChunks; ci += 64 * G) {
            const int key = ci >> 4, d0 = (ci & 15) * 8;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (k0 + key < c1) v = *reinterpret_cast<const uint4*>(vc + (kv_row0 + (size_t)(k0 + key)) * kD + d0);
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s_vt[buf][(d0 + 2 * i) * kVtStride + key] = (uint16_t)(wv[i] & 0xFFFFu);
                s_vt[buf][(d0 + 2 * i + 1) * kVtStride + key] = (uint16_t)(wv[i] >> 16);
            }
        }
    };
    auto load_k = [&](int k0, uint4* kr) {
        const int key = min(k0 + c32, c1 - 1);
        const uint4* src = reinterpret_cast<const uint4*>(kc + (kv_row0 + (size_t)key) * kD + 64 * h);
#pragma unroll
        for (int c = 0; c < 8; ++c) kr[c] = src[c];
    };

    const int ntiles = c1 > c0 ? (c1 - c0 + kTile - 1) / kTile : 0;
    uint4 kcur[8], knext[8];
    if (ntiles > 0) {
        load_k(c0, kcur);
        stage_v(c0, 0);
    }
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int k0 = c0 + it * kTile;
        const int buf = it & 1;
        if (it + 1 < ntiles) {           // next tile in flight during this one
            load_k(k0 + kTile, knext);
            stage_v(k0 + kTile, buf ^ 1);
        }
        // S^T = K Q^T
        v16f s = v16f{};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const v4s a0 = __builtin_bit_cast(v4s, make_uint2(kcur[c].x, kcur[c].y));
            const v4s a1 = __builtin_bit_cast(v4s, make_uint2(kcur[c].z, kcur[c].w));
            s = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a0, qop[2 * c], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a1, qop[2 * c + 1], s, 0, 0, 0);
        }
        // causal mask and the tile max of this lane's query
        float z[16];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + acc_row(r, h);
            const bool ok = key < c1 && key <= pos_q;
            z[r] = ok ? s[r] * p.scale_log2 : -INFINITY;
            mt = fmaxf(mt, z[r]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        // lazy rescale (when the max grows by more than 2^8, or from empty)
        const bool grow = m_new > m_run + 8.0f || (m_run == -INFINITY && m_new != -INFINITY);
        if (__any(grow)) {
            const float alpha = (!grow) ? 1.0f : (m_run == -INFINITY ? 0.0f : exp2f(m_run - m_new));
            if (grow) m_run = m_new;
            l_part *= alpha;
            if (h == 0) s_alpha[w][c32] = alpha;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float ar = s_alpha[w][acc_row(r, h)];
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) acc_o[t4][r] *= ar;
            }
        }
        // probabilities (this lane's 16 keys of its query), as the A operand of P V
        v4s pa[4];
        float ls = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = z[r] == -INFINITY ? 0.0f : exp2f(z[r] - m_run);
            ls += pr;
            pa[r >> 2][r & 3] = f2bf(pr);
        }
        l_part += ls;
        // O += P V (B operand: 4 consecutive keys of one d column of V^T)
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const uint2 bv = *reinterpret_cast<const uint2*>(&s_vt[buf][(32 * t4 + c32) * kVtStride + 8 * ks + 4 * h]);
                acc_o[t4] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(pa[ks], __builtin_bit_cast(v4s, bv), acc_o[t4], 0, 0, 0);
            }
        }
        __syncthreads();                 // buf is restaged two tiles on; buf ^ 1 is complete
        if (it + 1 < ntiles) {
#pragma unroll
            for (int c = 0; c < 8; ++c) kcur[c] = knext[c];
        }
    }

    // partials of this chunk: per query row (w, q): m (log2), l, unnormalised O
    const size_t rec = (size_t)blockIdx.x * (32 * G);
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (h == 0) {
        p.rec_ml[(rec + (size_t)w * 32 + c32) * 2 + 0] = m_run;
        p.rec_ml[(rec + (size_t)w * 32 + c32) * 2 + 1] = l_tot;
    }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            p.rec_o[(rec + (size_t)w * 32 + acc_row(r, h)) * kD + 32 * t4 + c32] = acc_o[t4][r];
}

// Merge the chunks of one (sequence, query head): 32 rows x 128 columns, one
// row and 16 columns per thread; chunks in order (log-sum-exp).
template <int G>
__global__ void __launch_bounds__(256) correction_combine_kernel(CorrParams p) {
    const int bg = blockIdx.x / G, w = blockIdx.x - bg * G;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    const int row = threadIdx.x >> 3, d0 = (threadIdx.x & 7) * 16;
    if (row >= p.T) return;
    const int Hq = p.Hkv * G;
    float M = -INFINITY;
    for (int c = 0; c < p.nchunks; ++c) {
        const size_t r = ((size_t)(bg * p.nchunks + c) * (32 * G) + (size_t)w * 32 + row);
        M = fmaxf(M, p.rec_ml[r * 2]);
    }
    float L = 0.0f, o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = 0.0f;
    for (int c = 0; c < p.nchunks; ++c) {
        const size_t r = ((size_t)(bg * p.nchunks + c) * (32 * G) + (size_t)w * 32 + row);
        const float m = p.rec_ml[r * 2];
        if (m == -INFINITY) continue;
        const float sc = exp2f(m - M);
        L += p.rec_ml[r * 2 + 1] * sc;
        const float4* src = reinterpret_cast<const float4*>(p.rec_o + r * kD + d0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 v = src[i];
            o[4 * i + 0] += v.x * sc;
            o[4 * i + 1] += v.y * sc;
            o[4 * i + 2] += v.z * sc;
            o[4 * i + 3] += v.w * sc;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    float4* dst = reinterpret_cast<float4*>(p.out + (((size_t)b * p.T + row) * Hq + (size_t)g * G + w) * kD + d0);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_float4(o[4 * i] * inv, o[4 * i + 1] * inv, o[4 * i + 2] * inv, o[4 * i + 3] * inv);
}

// Algorithm 1's cache append: row n_ctx[b] of every (b, g) gets the new K and
// V rows, then n_ctx[b] grows by one.  One workgroup per sequence; a full cache
// sets the error flag and changes nothing.
__global__ void __launch_bounds__(256) kv_append_kernel(AppendParams p) {
    const int b = blockIdx.x;
    const int n = p.n_ctx[b];
    const bool full = n < 0 || n >= p.max_ctx;
    if (!full) {
        const int row_bytes = p.d * p.elem_bytes;
        const int per_head = row_bytes / 4;                 // dwords (rows are 4-byte multiples)
        const int total = p.Hkv * per_head;
        for (int i = threadIdx.x; i < total; i += blockDim.x) {
            const int g = i / per_head, e = i - g * per_head;
            const size_t src = ((size_t)b * p.Hkv + g) * per_head + e;
            const size_t dst = (((size_t)b * p.Hkv + g) * p.max_ctx + (size_t)n) * per_head + e;
            reinterpret_cast<uint32_t*>(p.kc)[dst] = reinterpret_cast<const uint32_t*>(p.k_new)[src];
            reinterpret_cast<uint32_t*>(p.vc)[dst] = reinterpret_cast<const uint32_t*>(p.v_new)[src];
        }
    }
    __syncthreads();                   // every thread has read n
    if (threadIdx.x == 0) {
        if (full) atomicOr(p.err, 8u);
        else p.n_ctx[b] = n + 1;
    }
}

template <int G>
hipError_t launch_g(const CorrParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(correction_partial_kernel<G>, dim3(p.B * p.Hkv * p.nchunks), dim3(64 * G), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(correction_combine_kernel<G>, dim3(p.B * p.Hkv * G), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_correction(const CorrParams& p, int G, hipStream_t stream) {
    switch (G) {
        case 1: return launch_g<1>(p, stream);
        case 2: return launch_g<2>(p, stream);
        case 4: return launch_g<4>(p, stream);
        case 8: return launch_g<8>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(kv_append_kernel, dim3(p.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace lychee
