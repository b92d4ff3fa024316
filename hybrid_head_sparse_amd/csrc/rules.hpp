// Launch parameters of the rule-selection kernel that runs after the
// attention kernel for the Top-p rule (internal, not part of the ABI), and the
// limit of the block rule, which the attention kernel cuts itself.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lychee {

constexpr int kMaxSelBlocks = 4096;   // floor(k / bs) limit of the block rule (blocks listed in LDS)

struct RuleParams {
    int32_t* S;                    // [B, Hkv, k]: retrieval rows hold the top-min(k, n) set, ascending
    const uint32_t* score;         // [B*Hkv, max_ctx]: every token's selection key (the attention
                                   //                   kernel's score buffer)
    unsigned long long* comp;      // [B*Hkv, max_ctx]: scratch (the candidate buffer, free after
                                   //                   the attention kernel)
    uint32_t* zpart;               // [nslots, 4]: the attention kernel's normaliser partials
                                   //                   (tag bg + 1, m, z as double; tags restored to 0)
    const int32_t* n_ctx;          // [B]
    uint32_t* err;                 // device error flag (bit 2: an S entry outside [0, n))
    uint64_t role_bits;            // bit g set = KV head g is a retrieval head
    int32_t B, Hkv, max_ctx, k;
    int32_t nslots;                // partial slots the attention launch may have written
    float c_log2;                  // log2(e) / (G sqrt(d)), key units -> log2 of the share
    unsigned long long P;          // p as 52-bit fixed point
};

hipError_t launch_rule_select(const RuleParams& p, hipStream_t stream);

}  // namespace lychee
