// Launch parameters of the Top-p trim kernel (internal, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lychee {

struct TopPParams {
    int32_t* S;                    // [B, Hkv, k]: retrieval rows hold the top-min(k, n) set, ascending
    const uint32_t* score;         // [B*Hkv, max_ctx]: every token's selection key (the attention
                                   //                   kernel's score buffer)
    unsigned long long* comp;      // [B*Hkv, max_ctx]: scratch (the candidate buffer, free after
                                   //                   the attention kernel)
    unsigned long long* rec;       // [B*Hkv, kTopPSplit, 2]: per-slice partials (largest key,
                                   //                   normaliser)
    uint32_t* ctr;                 // [B*Hkv]: slices done (zero between calls)
    const int32_t* n_ctx;          // [B]
    uint32_t* err;                 // device error flag (bit 2: an S entry outside [0, n))
    uint64_t role_bits;            // bit g set = KV head g is a retrieval head
    int32_t B, Hkv, max_ctx, k;
    float c_log2;                  // log2(e) / (G sqrt(d)): selection key units -> log2 of the share
    unsigned long long P;          // p as 52-bit fixed point
};

hipError_t launch_topp_trim(const TopPParams& p, hipStream_t stream);

}  // namespace lychee
