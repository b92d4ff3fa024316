// The multi-step loop around the hybrid step (gfx950): the cache append of
// Algorithm 1 and the attention of the digest's Cache Correction, the dense
// re-prefill over the last T <= 32 decoded tokens every 32 steps (section
// 4.2.2 of the LycheeDecode digest).  Only the attention part is computed:
// each of the last T positions p = n - T + t attends, for every query head,
// densely and causally to cache rows 0..p with its own query.
//
// Correction attention.  Per KV head this is a (T G) x n x d contraction, so
// it runs on the matrix cores: v_mfma_f32_32x32x16_bf16 (bf16 operands, fp32
// accumulation; the gfx950 form, twice the work of the 32x32x8 form per
// instruction).  A workgroup takes one (sequence, KV head) and one chunk of
// its context; wavefront w is query head g G + w and holds that head's T
// queries (padded to 32) as the 32 columns of its tiles.  Per tile of 32 keys:
//   S^T = K Q^T          (8 MFMAs over d = 128; the A operands, 16 bytes of
//                         one key row per lane and MFMA, read from the tile's
//                         K in LDS)
//   causal mask, online softmax in the log2 domain (each lane holds 16 keys
//   of one query; one exchange with the other half-wave gives the tile max;
//   a tile that every query sees whole skips the mask, and its exponent is
//   one fma of the raw score); probabilities go to bf16 by the hardware
//   round-to-nearest-even conversion
//   O += P V             (8 MFMAs: the 16 probabilities a lane holds are,
//                         converted to bf16, its A operands for the tile's
//                         two 16-key steps; V is staged transposed in LDS,
//                         so a B operand is two 8-byte reads)
// The workgroup loads each tile's K and V once (16-byte pieces, two tiles
// ahead) and stages them in double-buffered LDS: K row-major with padded rows,
// V transposed.  Every wavefront reads its operands of both MFMA groups at the
// top of the tile.
// A contraction may take its index in any order common to both operands: over
// d, lane half h takes d in [64 h, 64 h + 64); over the keys of a 16-key step
// s, element i of lane half h is key 16 s + 8 (i / 4) + 4 h + i % 4, which is
// where the S^T accumulator already holds it.  A
// chunk's per-query partials (max, sum, unnormalised O) go to the workspace
// and a second kernel merges the chunks by the log-sum-exp rule.
//
// Lane layout of v_mfma_f32_32x32x16_bf16 (checked on the device): lane l
// holds A[l % 32][8 (l / 32) + i], B[8 (l / 32) + i][l % 32] (i < 8) and
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] in accumulator r < 16.

#include "common.hpp"
#include "correction.hpp"

namespace lychee {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;               // head dim of the MFMA path
constexpr int kTile = 32;             // keys per tile
constexpr int kVtStride = kTile + 4;  // bf16 per transposed V row in LDS (padded)
constexpr int kKStride = kD + 8;      // bf16 per K row in LDS (padded by 16 bytes)

// the value of lane l ^ 32 (gfx950 permlane32 swap: no LDS round trip)
__device__ __forceinline__ float lane_xor32(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// row of accumulator register r for lane half h
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

template <int G>
__global__ void __launch_bounds__(64 * G, G >= 4 ? 2 : 1) correction_partial_kernel(CorrParams p) {   // 2 waves per SIMD (G >= 4)
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, c32 = lane & 31;
    const int bg = blockIdx.x / p.nchunks, chunk = blockIdx.x - bg * p.nchunks;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    const int n = max(0, min(p.n_ctx[b], p.max_ctx));
    const int T = p.T;
    const int Hq = p.Hkv * G;
    if (n < T) {                       // out of contract: flagged, the rows are undefined
        if (threadIdx.x == 0 && chunk == 0) atomicOr(p.err, 4u);
    }
    const int c0 = (int)(((long long)n * chunk) / p.nchunks);
    const int c1 = (int)(((long long)n * (chunk + 1)) / p.nchunks);
    const size_t kv_row0 = (size_t)bg * p.max_ctx;
    const int last = max(c1 - 1, 0);   // loads clamp to the chunk's last row (row 0 for an empty chunk)
    // this head's rows (a wavefront-uniform base; per-lane offsets stay 32-bit:
    // a head's slot is max_ctx * 256 bytes)
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(p.kc) + kv_row0 * kD;
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(p.vc) + kv_row0 * kD;

    // K of a tile, row-major with rows padded to kKStride (so the A-operand
    // reads of 8 consecutive lanes, 8 keys at one offset, fall on distinct
    // bank groups); V of a tile transposed (d-major).  Both double-buffered.
    __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kTile * kKStride];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kD * kVtStride];
    __shared__ float s_alpha[G][32];

    // this lane's query: t = c32 (rows t >= T repeat row T - 1, ignored at the end)
    const int tq = min(c32, T - 1);
    const int pos_q = n - T + c32;     // causal limit of query c32 (keys <= pos_q)
    v8bf qop[8];
    {
        const uint4* qr = reinterpret_cast<const uint4*>(
            reinterpret_cast<const uint16_t*>(p.q) + (((size_t)b * T + tq) * Hq + (size_t)g * G + w) * kD + 64 * h);
#pragma unroll
        for (int c = 0; c < 8; ++c) qop[c] = __builtin_bit_cast(v8bf, qr[c]);
    }
    v16f acc_o[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) acc_o[t4] = v16f{};
    float m_run = -INFINITY, l_part = 0.0f;

    // A tile's K and V are loaded cooperatively, once per workgroup, as
    // 16-byte pieces (8 columns of one key): kPieces per thread and operand.
    // K piece j of a thread is key (tid + 64 G j) / 16, columns 8 ((tid + 64 G
    // j) % 16): whole rows per 16 lanes, stored as they come.  V is stored
    // transposed, so consecutive lanes take consecutive keys of one column
    // block (their 32-bit LDS words then fall on distinct banks).  With an
    // even number of pieces per thread, a thread takes a pair of keys (pair
    // index i = tid + 64 G (j / 2): keys 2 (i % 16) and 2 (i % 16) + 1, columns
    // 8 (i / 16)) and writes both keys of a column as one 32-bit word;
    // otherwise piece j (i = tid + 64 G j) is key i % 32, columns 8 (i / 32).
    constexpr int kPieces = kTile * kD / 8 / (64 * G);
    constexpr bool kPairs = kPieces % 2 == 0;
    auto piece_key = [&](int j) -> int {
        if constexpr (kPairs) return 2 * ((threadIdx.x + 64 * G * (j >> 1)) & 15) + (j & 1);
        else return (threadIdx.x + 64 * G * j) & 31;
    };
    auto piece_d0 = [&](int j) -> int {
        if constexpr (kPairs) return ((threadIdx.x + 64 * G * (j >> 1)) >> 4) * 8;
        else return ((threadIdx.x + 64 * G * j) >> 5) * 8;
    };
    // Every load is issued on every path (rows past the chunk are clamped to
    // its last row, V pieces there are zeroed after the load; K there only
    // meets masked scores): the wait counts are then exact.
    auto load_kv = [&](int k0, u32x4 (&kr)[kPieces], uint4 (&vr)[kPieces]) {
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
            const int idx = threadIdx.x + 64 * G * j;
            const int key = min(k0 + (idx >> 4), last);
            kr[j] = *reinterpret_cast<const u32x4*>(kc + ((uint32_t)key * kD + (uint32_t)(idx & 15) * 8u));
        }
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
            const int key = piece_key(j), d0 = piece_d0(j);
            vr[j] = *reinterpret_cast<const uint4*>(vc + ((uint32_t)min(k0 + key, last) * kD + (uint32_t)d0));
        }
    };
    auto store_kv = [&](int k0, const u32x4 (&kr)[kPieces], uint4 (&vr)[kPieces], int buf) {
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
            const int idx = threadIdx.x + 64 * G * j;
            *reinterpret_cast<u32x4*>(&s_k[buf][(idx >> 4) * kKStride + (idx & 15) * 8]) = kr[j];
        }
#pragma unroll
        for (int j = 0; j < kPieces; ++j)       // V rows past the chunk contribute 0
            if (k0 + piece_key(j) >= c1) vr[j] = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (kPairs) {
#pragma unroll
            for (int j = 0; j < kPieces; j += 2) {
                const int key = piece_key(j), d0 = piece_d0(j);      // key even; key + 1 in piece j + 1
                const uint32_t a[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
                const uint32_t c[4] = {vr[j + 1].x, vr[j + 1].y, vr[j + 1].z, vr[j + 1].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    *reinterpret_cast<uint32_t*>(&s_vt[buf][(d0 + 2 * i) * kVtStride + key]) =
                        (a[i] & 0xFFFFu) | (c[i] << 16);
                    *reinterpret_cast<uint32_t*>(&s_vt[buf][(d0 + 2 * i + 1) * kVtStride + key]) =
                        (a[i] >> 16) | (c[i] & 0xFFFF0000u);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kPieces; ++j) {
                const int key = piece_key(j), d0 = piece_d0(j);
                const uint32_t wv[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s_vt[buf][(d0 + 2 * i) * kVtStride + key] = (uint16_t)(wv[i] & 0xFFFFu);
                    s_vt[buf][(d0 + 2 * i + 1) * kVtStride + key] = (uint16_t)(wv[i] >> 16);
                }
            }
        }
    };

    // Two register sets of pieces, alternating: at tile it, tile it's K and V
    // are in LDS buffer it & 1, tile it + 1's pieces are in one set, and tile
    // it + 2's loads go to the other (free since its tile went to LDS at the
    // end of tile it - 1), so each load has about two tiles of work to arrive.
    // The first loads are issued on every path (a chunk without rows reads row
    // 0 and uses nothing): with no branch before the loop, the wait counts at
    // its top need not cover the query loads of a path that skips them.
    const int ntiles = c1 > c0 ? (c1 - c0 + kTile - 1) / kTile : 0;
    u32x4 kA[kPieces], kB[kPieces];
    uint4 vA[kPieces], vB[kPieces];
    load_kv(c0, kA, vA);
    load_kv(c0 + kTile, kB, vB);
    store_kv(c0, kA, vA, 0);
    __syncthreads();
    // tile it: its K and V in LDS, the next tile's pieces in (kn, vn); (kf, vf) free
    auto tile = [&](int it, u32x4 (&kn)[kPieces], uint4 (&vn)[kPieces], u32x4 (&kf)[kPieces],
                    uint4 (&vf)[kPieces]) {
        const int k0 = c0 + it * kTile;
        const int buf = it & 1;
        load_kv(k0 + 2 * kTile, kf, vf);
        // S^T = K Q^T (A operand: key c32, columns 64 h + 8 c .. + 7)
        v8bf ka[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
            ka[c] = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(&s_k[buf][c32 * kKStride + 64 * h + 8 * c]));
        // the B operands of O += P V (keys 16 s + 4 h + 0..3 and 16 s + 8 + 4 h
        // + 0..3 of one d column of V^T), read here so that their latency
        // passes during the S MFMAs and the softmax rather than before each
        // P V MFMA
        v8bf bv[4][2];
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint16_t* col = &s_vt[buf][(32 * t4 + c32) * kVtStride + 16 * ks + 4 * h];
                const uint2 lo = *reinterpret_cast<const uint2*>(col);
                const uint2 hi = *reinterpret_cast<const uint2*>(col + 8);
                bv[t4][ks] = __builtin_bit_cast(v8bf, make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        v16f s = v16f{};
#pragma unroll
        for (int c = 0; c < 8; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qop[c], s, 0, 0, 0);
        // causal mask and the tile max of this lane's query
        float z[16];
        float mt = -INFINITY;
        // every key of the tile visible to every query (wavefront-uniform):
        // no mask, and the scale (positive) applies to the raw maximum
        const bool full = k0 + kTile <= c1 && k0 + kTile - 1 <= n - T;
        if (full) {
            float ms = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) ms = fmaxf(ms, s[r]);
            mt = ms * p.scale_log2;
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + acc_row(r, h);
                const bool ok = key < c1 && key <= pos_q;
                z[r] = ok ? s[r] * p.scale_log2 : -INFINITY;
                mt = fmaxf(mt, z[r]);
            }
        }
        mt = fmaxf(mt, lane_xor32(mt));
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
        // probabilities (this lane's 16 keys of its query): accumulators 8 s ..
        // 8 s + 7 are the A operand of 16-key step s
        v8bf pa[2];
        float ls = 0.0f;
        if (full) {                      // m_run is finite here
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], p.scale_log2, -m_run));
                ls += pr;
                pa[r >> 3][r & 7] = (__bf16)pr;
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float pr = z[r] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(z[r] - m_run);
                ls += pr;
                pa[r >> 3][r & 7] = (__bf16)pr;
            }
        }
        l_part += ls;
        // O += P V
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                acc_o[t4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], bv[t4][ks], acc_o[t4], 0, 0, 0);
        // the next tile to the other buffer (last read before the previous barrier)
        if (it + 1 < ntiles) store_kv(k0 + kTile, kn, vn, buf ^ 1);
        __syncthreads();                 // buf ^ 1 complete; buf is restaged only after the next barrier
    };
    int it = 0;
    for (; it + 1 < ntiles; it += 2) {
        tile(it, kB, vB, kA, vA);
        tile(it + 1, kA, vA, kB, vB);
    }
    if (it < ntiles) tile(it, kB, vB, kA, vA);

    // partials of this chunk: per query row (w, q): m (log2), l, unnormalised O
    const size_t rec = (size_t)blockIdx.x * (32 * G);
    const float l_tot = l_part + lane_xor32(l_part);
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

// Merge the chunks of one query row (sequence, query head, position): 128
// threads, one output column each.  The chunks' scales 2^(m_c - M) and the
// normaliser go through LDS first; then every thread sums its column over the
// chunks in order (coalesced 512-byte rows, independent loads).
template <int G>
__global__ void __launch_bounds__(kD) correction_combine_kernel(CorrParams p) {
    constexpr int kMaxChunksLds = 1024;
    __shared__ float s_scale[kMaxChunksLds];
    __shared__ float s_red[kD / 64];
    const int row = blockIdx.x % 32, qh = blockIdx.x / 32;       // qh = bg * G + w
    const int bg = qh / G, w = qh - bg * G;
    const int b = bg / p.Hkv, g = bg - b * p.Hkv;
    if (row >= p.T) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Hq = p.Hkv * G;
    const int nc = min(p.nchunks, kMaxChunksLds);
    auto rec_row = [&](int c) -> size_t { return (size_t)(bg * p.nchunks + c) * (32 * G) + (size_t)w * 32 + row; };
    float m = -INFINITY;
    for (int c = tid; c < nc; c += kD) m = fmaxf(m, p.rec_ml[rec_row(c) * 2]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) s_red[wave] = m;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int i = 1; i < kD / 64; ++i) M = fmaxf(M, s_red[i]);
    float lsum = 0.0f;
    for (int c = tid; c < nc; c += kD) {
        const float mc = p.rec_ml[rec_row(c) * 2];
        const float sc = mc == -INFINITY ? 0.0f : exp2f(mc - M);
        s_scale[c] = sc;
        lsum += sc * p.rec_ml[rec_row(c) * 2 + 1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lsum += __shfl_xor(lsum, o);
    __syncthreads();                   // s_red is reused; s_scale complete
    if (lane == 0) s_red[wave] = lsum;
    __syncthreads();
    float L = 0.0f;
#pragma unroll
    for (int i = 0; i < kD / 64; ++i) L += s_red[i];
    float acc = 0.0f;
    int c = 0;
    for (; c + 8 <= nc; c += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = p.rec_o[rec_row(c + j) * kD + tid];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += v[j] * s_scale[c + j];
    }
    for (; c < nc; ++c) acc += p.rec_o[rec_row(c) * kD + tid] * s_scale[c];
    p.out[(((size_t)b * p.T + row) * Hq + (size_t)g * G + w) * kD + tid] = L > 0.0f ? acc / L : 0.0f;
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
    hipLaunchKernelGGL(correction_combine_kernel<G>, dim3(p.B * p.Hkv * G * 32), dim3(kD), 0, stream, p);
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
