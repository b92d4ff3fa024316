// Launch parameters of the rule-selection kernel that runs after the
// attention kernel for the Top-p and block-granular rules (internal, not part
// of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lychee {

constexpr int kRuleTopP = 0;       // cut the top-min(k, n) set to its Top-p prefix
constexpr int kRuleBlock = 1;      // replace it with the top floor(k / bs) blocks of bs tokens
constexpr int kMaxSelBlocks = 4096;   // floor(k / bs) limit of the block rule (blocks listed in LDS)

struct RuleParams {
    int32_t* S;                    // [B, Hkv, k]: retrieval rows hold the top-min(k, n) set, ascending
    const uint32_t* score;         // [B*Hkv, max_ctx]: every token's selection key (the attention
                                   //                   kernel's score buffer)
    unsigned long long* comp;      // [B*Hkv, max_ctx]: scratch (the candidate buffer, free after
                                   //                   the attention kernel)
    uint32_t* bkey;                // [B*Hkv, bkey_stride]: block rule: each block's largest key
                                   //                   (restored to zero here)
    uint32_t* zpart;               // [nslots, 4]: Top-p: the attention kernel's normaliser partials
                                   //                   (tag bg + 1, m, z as double; tags restored to 0)
    const int32_t* n_ctx;          // [B]
    uint32_t* err;                 // device error flag (bit 2: an S entry outside [0, n))
    uint64_t role_bits;            // bit g set = KV head g is a retrieval head
    int32_t B, Hkv, max_ctx, k;
    int32_t mode;                  // kRuleTopP or kRuleBlock
    int32_t block;                 // block rule: tokens per block (a power of two, 16..256)
    int32_t bkey_stride;           // block words per head
    int32_t nslots;                // partial slots the attention launch may have written
    float c_log2;                  // Top-p: log2(e) / (G sqrt(d)), key units -> log2 of the share
    unsigned long long P;          // Top-p: p as 52-bit fixed point
};

hipError_t launch_rule_select(const RuleParams& p, hipStream_t stream);

}  // namespace lychee
