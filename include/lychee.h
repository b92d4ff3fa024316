/*
 * lychee.h -- C ABI of the hybrid-head decode-attention step (gfx950 / MI355X).
 *
 * One call computes the attention part of one decoder layer for one decode
 * step, as defined on the long-form digest "LycheeDecode: Accelerating
 * Long-Context LLM Inference via Hybrid-Head Sparse Decoding"
 * (paper-graph-ui), section 3.4:
 *   - retrieval heads: dense single-query attention over all cached tokens
 *     (Eq. 1) and S^(l+1) = argsTopK(A, k) (Eq. 2);
 *   - sparse heads: attention over only the k rows named by the inherited set
 *     S^(l) (Eq. 3), and S^(l+1) = S^(l);
 *   - layer 0 is all retrieval (so the first call of a step passes S_in = NULL);
 *   - with grouped-query attention the query heads of a KV head are average-
 *     pooled before token selection (hyper-parameter summary).
 * The split-K partials + log-sum-exp combine and the pooling of retrieval and
 * sparse work into one set of equal-size work units follow the kernel
 * description of the same section ("Custom Hybrid-Head Block-Sparse Decoding
 * Kernel"), re-designed for CDNA4.
 *
 * Conventions
 *   - Pointers are device pointers unless marked (host).
 *   - Roles and critical-token sets are per KV head: query head h uses KV head
 *     h / G (G = n_q_heads / n_kv_heads) and shares that head's role and S.
 *   - Selection score of KV head g at token j: mean over its G query heads of
 *     the pre-softmax logit q_h.K_j / sqrt(d); larger first, ties to the lower
 *     token index.  S rows are ascending; when n_ctx[b] < k only the first
 *     n_ctx[b] entries are valid and the rest are -1.
 *   - Ownership: the caller owns every tensor and the workspace.  The library
 *     never allocates or frees device memory; a handle holds host state only.
 *   - Asynchrony: calls enqueue on the handle's stream and return at once.
 *     No call in the decode path synchronises or copies to the host, so a
 *     sequence of calls can be captured into a HIP graph.
 *   - Errors: an integer status, never an exception.  Argument checks happen
 *     on the host, before anything is enqueued.  A detail string is kept per
 *     thread (lychee_last_error).
 *   - Workspace invariant: the library's counters and histograms inside the
 *     workspace are zero between calls; every call restores them.  Calls on
 *     one workspace must be ordered (one stream, or explicit dependencies).
 *   - Supported: head_dim 64 or 128; G in {1, 2, 4, 8}; n_kv_heads <= 64;
 *     batch * n_kv_heads <= 1024; max_ctx <= 262144; dtype fp32 or bf16.
 */
#ifndef LYCHEE_H
#define LYCHEE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LYCHEE_OK = 0,
    LYCHEE_ERR_INVALID_ARG = -1,   /* null pointer, bad size, overlap, role/S mismatch */
    LYCHEE_ERR_UNSUPPORTED = -2,   /* valid request outside the compiled variants */
    LYCHEE_ERR_HIP = -3,           /* a HIP runtime call or kernel launch failed */
    LYCHEE_ERR_WORKSPACE = -4,     /* workspace too small or misaligned */
    LYCHEE_ERR_DEVICE_CHECK = -5   /* device-side contract violation seen (see lychee_check_device_errors) */
} lychee_status;

typedef enum { LYCHEE_F32 = 0, LYCHEE_BF16 = 1 } lychee_dtype;

/* Problem dimensions fixed for the life of a handle. */
typedef struct {
    int32_t batch;        /* B */
    int32_t n_q_heads;    /* Hq */
    int32_t n_kv_heads;   /* Hkv, divides Hq */
    int32_t head_dim;     /* d */
    int32_t max_ctx;      /* rows per (sequence, KV head) in the cache */
    int32_t k_max;        /* largest critical-token budget k that will be passed */
    int32_t dtype;        /* lychee_dtype of q, k_cache and v_cache */
} lychee_dims;

typedef struct lychee_handle lychee_handle;

/* (host) Bytes of device workspace a handle with these dims needs; 0 if the
 * dims are invalid or unsupported (see lychee_last_error). */
size_t lychee_workspace_bytes(const lychee_dims* dims);

/* Bind dims, a caller-owned device workspace (>= lychee_workspace_bytes,
 * 256-byte aligned) and a HIP stream (hipStream_t passed as void*; NULL = the
 * null stream) into a handle.  Enqueues one clear of the workspace's counter
 * region on the stream (so do not call it inside graph capture). */
lychee_status lychee_create(const lychee_dims* dims, void* workspace, size_t workspace_bytes,
                            void* stream, lychee_handle** out_handle);

/* One layer of the hybrid-head step (the per-layer attention of Algorithm 1
 * in section 3.4 of the digest; Eq. 1, 2, 3 and the propagation rules).
 *   q          [B, Hq, d]               dtype
 *   k_cache    [B, Hkv, max_ctx, d]     dtype; rows >= n_ctx[b] are never read
 *   v_cache    [B, Hkv, max_ctx, d]     dtype
 *   role_mask  (host) [Hkv] uint8, nonzero = retrieval head, 0 = sparse head
 *   S_in       [B, Hkv, k] int32 from the previous layer's S_out; may be NULL
 *              only when every role is retrieval (layer 0).  Entries of a
 *              sparse head's row must lie in [0, n_ctx[b]) or be -1 (padding
 *              of a set shorter than min(k, n_ctx[b]), skipped) for the first
 *              min(k, n_ctx[b]) positions; later entries are copied, not read.
 *              The entries other than -1 must be strictly ascending (the form
 *              S_out has), which rules out duplicates.
 *              A sparse head whose entries are all padding outputs zeros.
 *   S_out      [B, Hkv, k] int32; retrieval rows get the new set (ascending,
 *              -1 padded), sparse rows a copy of S_in's row.  S_out may equal
 *              S_in (in place); any other overlap is rejected.
 *   out        [B, Hq, d] fp32, fully overwritten
 *   n_ctx      [B] int32 on the device, 1 <= n_ctx[b] <= max_ctx
 *   k          1 <= k <= k_max
 * Device-side contract checks (each latches a flag that
 * lychee_check_device_errors reports; nothing is read out of bounds):
 *   - an S_in entry outside [0, n_ctx[b]) other than -1 is skipped;
 *   - S_in entries (other than -1) that are not strictly ascending inside a
 *     row, e.g. a duplicate, are flagged and attended as given (a duplicated
 *     row counts twice).  A pair whose two entries fall in the parts of the
 *     row that different workgroups take, with only -1 entries between
 *     them, is not seen;
 *   - n_ctx[b] outside [1, max_ctx] is clamped to [0, max_ctx]; a sequence
 *     clamped to 0 rows gets zeros in out, -1 in its retrieval rows of S_out
 *     and a copy of S_in in its sparse rows. */
lychee_status lychee_decode_layer(lychee_handle* h,
                                  const void* q, const void* k_cache, const void* v_cache,
                                  const uint8_t* role_mask, const int32_t* S_in, int32_t* S_out,
                                  float* out, const int32_t* n_ctx, int32_t k);

/* Selection rules of lychee_decode_layer_select.  The digest's ablation of
 * selection methods (section 4.4.1, Figure 6) compares top-k with a ratio and
 * a threshold rule without giving their formulas; these are the plain
 * readings, with s_j the score Eq. 2 ranks (the mean over a KV head's G
 * query heads of q . k_j / sqrt(d)) and n = n_ctx[b]:
 *   TOPK       the min(k, n) highest-scoring tokens (lychee_decode_layer);
 *   RATIO      the min(k, ceil(theta n)) highest (at least one), theta =
 *              param in (0, 1], theta n evaluated in double;
 *   THRESHOLD  the tokens with s_j >= tau (param), the k highest of them if
 *              there are more.  The kernel compares the fp32 sum over the G
 *              heads of q . k_j with tau G sqrt(d) rounded to fp32, so a score
 *              within fp32 rounding of tau may fall on either side.
 *   TOPP       the shortest prefix of the ranking whose share of softmax(s)
 *              over all n tokens reaches p = param in (0, 1], at most
 *              min(k, n) tokens.  Shares are fp32 exponentials over an fp64
 *              normaliser, summed as 52-bit fixed point, so a cut within that
 *              rounding of p may land one token either side.  Cut inside the
 *              attention kernel, after the top-min(k, n) set.
 *   BLOCK      block-granular selection (the digest's kernel works on blocks
 *              of 64 tokens and states no rule for a block's score): blocks of
 *              bs = param tokens (16, 32, 64, 128 or 256; the last block may
 *              be shorter), a block scored by the largest s_j of its tokens,
 *              the floor(k / bs) highest blocks kept (at most 4096 blocks;
 *              k >= bs), their tokens listed ascending.  Cut inside the
 *              attention kernel (no second kernel).
 * Ties go to the lower index (token or block) under every rule. */
enum {
    LYCHEE_SELECT_TOPK = 0,
    LYCHEE_SELECT_RATIO = 1,
    LYCHEE_SELECT_THRESHOLD = 2,
    LYCHEE_SELECT_TOPP = 3,
    LYCHEE_SELECT_BLOCK = 4
};

/* lychee_decode_layer with a selection rule for the retrieval heads (above).
 * A retrieval row of S_out holds its selected tokens ascending, then -1 up to
 * k; a later sparse head skips the -1 entries.  Arguments as for
 * lychee_decode_layer, plus `rule` (a LYCHEE_SELECT_* value) and `param`
 * (theta for RATIO, tau for THRESHOLD, p for TOPP, the block size for BLOCK,
 * unused for TOPK).  Returns LYCHEE_ERR_INVALID_ARG for an unknown rule, theta
 * or p outside (0, 1], a NaN tau or a block size or k the block rule does not
 * take, after which nothing is enqueued. */
lychee_status lychee_decode_layer_select(lychee_handle* h,
                                         const void* q, const void* k_cache, const void* v_cache,
                                         const uint8_t* role_mask, const int32_t* S_in, int32_t* S_out,
                                         float* out, const int32_t* n_ctx, int32_t k, int32_t rule,
                                         double param);

/* For callers that cannot allocate device memory or own a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): lychee_decode_layer without a handle or workspace.  Same
 * arguments, layouts, results and host-side checks as lychee_decode_layer,
 * plus the dims (host) and the HIP stream (hipStream_t as void*; NULL = the
 * null stream).  The kernels' scratch (partial records, counters, selection
 * candidates) lives in a 64 MiB device array inside the library, one per GPU,
 * held until the process ends; this call allocates and frees nothing.
 *   - Dims whose decode scratch exceeds 64 MiB return LYCHEE_ERR_WORKSPACE
 *     before anything is enqueued.  The scratch is about 12 bytes per cached
 *     row (batch * n_kv_heads * max_ctx) plus 4 * 66 * G * (d + 2) + 16 KiB
 *     per (sequence, KV head) plus 4 MiB: the Llama3-8B shape fits at
 *     batch 1 up to max_ctx 2^18 and at batch 8 up to 64K.
 *   - The first call on a device (and any call whose layout needs a longer
 *     zeroed region than earlier calls left) enqueues one small clearing
 *     kernel before the attention kernel.
 *   - Every call on one GPU uses that GPU's one array: calls that may overlap
 *     on a GPU (different streams without ordering, several threads) race and
 *     give wrong results.  Order them on one stream.
 *   - Device-side contract flags latch inside the array and are not
 *     reported; check a suspect input through lychee_decode_layer. */
lychee_status lychee_decode_layer_static(const lychee_dims* dims, void* stream,
                                         const void* q, const void* k_cache, const void* v_cache,
                                         const uint8_t* role_mask, const int32_t* S_in, int32_t* S_out,
                                         float* out, const int32_t* n_ctx, int32_t k);

/* Dense all-heads decode attention over the same layout (every head attends
 * to all n_ctx[b] tokens, Eq. 1 without selection): the baseline the hybrid
 * step is compared with.  Same argument meanings as above. */
lychee_status lychee_dense_decode_layer(lychee_handle* h, const void* q, const void* k_cache,
                                        const void* v_cache, float* out, const int32_t* n_ctx);

/* (host) Validate the arguments of lychee_decode_layer for these dims without
 * touching the device: the same checks lychee_decode_layer runs first. */
lychee_status lychee_validate_layer(const lychee_dims* dims,
                                    const void* q, const void* k_cache, const void* v_cache,
                                    const uint8_t* role_mask, const int32_t* S_in,
                                    const int32_t* S_out, const float* out,
                                    const int32_t* n_ctx, int32_t k);

/* Rebind the handle to another stream (hipStream_t as void*). */
lychee_status lychee_set_stream(lychee_handle* h, void* stream);

/* Optional timing hook: when both are non-NULL (hipEvent_t as void*), every
 * following decode/dense call records `start` right before its attention
 * kernel and `stop` right after it, on the handle's stream.  NULL disables. */
lychee_status lychee_set_profile_events(lychee_handle* h, void* start, void* stop);

/* Algorithm 1's cache append, the step after a token's attention (the
 * multi-step loop around the layer; digest section 3.4): row n_ctx[b] of
 * every KV head of sequence b receives the new token's K and V rows, then
 * n_ctx[b] grows by one, all on the device (so a captured loop of steps
 * advances by itself).
 *   k_new, v_new  [B, Hkv, d] dtype
 *   k_cache, v_cache, n_ctx  as for lychee_decode_layer (written)
 * A sequence whose cache is full (n_ctx[b] == max_ctx) is left unchanged and
 * latches a flag reported by lychee_check_device_errors. */
lychee_status lychee_kv_append(lychee_handle* h, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               int32_t* n_ctx);

/* The attention of Cache Correction (digest section 4.2.2: after every 32
 * decoded tokens, a dense prefill over those tokens refreshes their K and V;
 * the projections need the model, the attention is this call).  Each of the
 * last T positions p = n_ctx[b] - T + t of a sequence attends, for every query
 * head h (KV head h / G), densely and causally to cache rows 0..p with scale
 * 1/sqrt(d):
 *   q     [B, T, Hq, d] bf16, row t is position n_ctx[b] - T + t
 *   out   [B, T, Hq, d] fp32, fully overwritten
 *   T     1..32;  1 <= T <= n_ctx[b] on the device (else a flag latches and
 *         the rows are undefined)
 * Runs on the matrix cores (bf16 operands, fp32 accumulation), so it needs a
 * bf16 cache, head_dim 128 and n_q_heads / n_kv_heads in {1, 2, 4, 8}
 * (LYCHEE_ERR_UNSUPPORTED otherwise).  Two kernels: context-chunk partials,
 * then their log-sum-exp merge.  Profile events bracket both. */
lychee_status lychee_correction_attention(lychee_handle* h, const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* n_ctx, int32_t T, float* out);

/* Synchronise the stream, read and clear the device-side error flag.
 * Returns LYCHEE_ERR_DEVICE_CHECK if any call since the last check skipped an
 * out-of-range S_in entry, saw S_in entries out of ascending order (a
 * duplicate), clamped an n_ctx outside [1, max_ctx], appended to a full cache
 * or ran a correction over a context shorter than T; the detail string
 * (lychee_last_error) lists the flag bits. */
lychee_status lychee_check_device_errors(lychee_handle* h);

/* Release the handle (host memory only). */
void lychee_destroy(lychee_handle* h);

/* Static string for a status code. */
const char* lychee_status_str(lychee_status s);

/* Detail message of the last failing call on this thread ("" if none). */
const char* lychee_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LYCHEE_H */
