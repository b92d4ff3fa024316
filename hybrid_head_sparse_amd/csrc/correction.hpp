// Launch parameters of the multi-step loop's kernels: the correction
// attention and the cache append (internal, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lychee {

constexpr int kCorrMaxT = 32;          // positions a correction covers (one MFMA tile of queries)
constexpr int kCorrTargetWG = 512;     // partial workgroups per launch (context chunks x heads)

struct CorrParams {
    const void* q;                     // [B, T, Hq, d] bf16: the last T positions' queries
    const void* kc;                    // [B, Hkv, max_ctx, d] bf16
    const void* vc;
    const int32_t* n_ctx;              // [B]
    float* out;                        // [B, T, Hq, d]
    float* rec_ml;                     // [B Hkv nchunks, 32 G, 2]: chunk partials (max, sum)
    float* rec_o;                      // [B Hkv nchunks, 32 G, d]: unnormalised chunk outputs
    uint32_t* err;                     // device error flag (bit 4: n_ctx < T)
    int32_t B, Hkv, max_ctx, T, nchunks;
    float scale_log2;                  // log2(e) / sqrt(d)
};

struct AppendParams {
    const void* k_new;                 // [B, Hkv, d]
    const void* v_new;
    void* kc;                          // [B, Hkv, max_ctx, d]
    void* vc;
    int32_t* n_ctx;                    // [B], grows by one per append
    uint32_t* err;                     // device error flag (bit 8: a full cache)
    int32_t B, Hkv, d, max_ctx, elem_bytes;
};

hipError_t launch_correction(const CorrParams& p, int G, hipStream_t stream);
hipError_t launch_kv_append(const AppendParams& p, hipStream_t stream);

}  // namespace lychee
