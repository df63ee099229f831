/*
 * mla_decode.h — C ABI of an MI355X (gfx950) paged MLA decode library.
 *
 * The operation (plain reading of the pages):
 *   "[WIP][Attention] FlashAttn MLA", description: MLA's decode step is
 *   computed as multi-query attention — every query head attends to one
 *   shared latent KV head.
 *   "[Attention] Blackwell FP8 MLA support with CUTLASS_MLA backend", review
 *   thread (the failing kernel test): h_kv = 1, d = 576, dv = 512, a paged
 *   cache (page size 64 in the test; "[NVIDIA] Add Cutlass MLA backend" serves
 *   DeepSeek-V3 with --block-size=128), causal and varlen options, the cache in
 *   bf16 or torch.float8_e4m3fn.
 *
 * For sequence b with L = seq_lens[b] cached tokens (the s_q new tokens are
 * the last s_q of them), query token i in [0, s_q) and head h in [0, H):
 *   Leff    = causal ? L - s_q + 1 + i : L                (keys it may see)
 *   k_t     = decode(kv_cache[block_table[b][t / bs]][t % bs][0..575]) * kv_scale
 *   s_t     = softmax_scale * dot(q[b][i][h][0..575], k_t)          t < Leff
 *   out[b][i][h][0..511] = sum_t softmax(s)_t * k_t[0..511]   (V = latent part)
 *   lse[b][i][h]         = ln(sum_t exp(s_t))                  (natural log)
 * A row that sees no key gets out = 0 and lse = -inf.
 *
 * Input range: the kernels keep each row's softmax reference max from the
 * first key tile it sees and move it only when a later score exceeds it by
 * more than 64 (base 2), so un-normalised weights stay below 2^64 and the fp32
 * output accumulators below 2^64 * max|v| * L. Caches whose latent values
 * reach about 2^60 / L would overflow where the textbook algorithm would not;
 * real latent caches are many orders of magnitude below that.
 *
 * Every entry point is safe to call without a GPU as long as it returns an
 * error before launching (argument checks never touch the device).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_D_QK 576          /* 512 latent + 64 rotary columns per cached row */
#define MLA_D_V 512           /* the latent part of the row serves as V */
#define MLA_MAX_HEADS 128
#define MLA_MAX_SQ 512        /* query tokens per sequence, up to the decode threshold */
#define MLA_MAX_BATCH 16384
#define MLA_ABI_VERSION 1
/* Size of the device array mla_decode_noalloc uses instead of a workspace. */
#define MLA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misalignment, non-finite scale */
    MLA_ERR_UNSUPPORTED = 2,        /* heads, s_q, block size or dtype outside the supported set */
    MLA_ERR_WORKSPACE_TOO_SMALL = 3,
    MLA_ERR_HIP = 4                 /* a HIP launch or query failed */
} mla_status_t;

typedef enum mla_dtype {
    MLA_DTYPE_BF16 = 0,
    MLA_DTYPE_FP8_E4M3FN = 1        /* OCP OFP8 E4M3: bias 7, max 448, no inf */
} mla_dtype_t;

/* Problem description (the kernel test's parameter set, minus the fixed
 * h_kv = 1, d = 576, dv = 512). */
typedef struct mla_decode_desc {
    int32_t batch;               /* 0 <= B <= MLA_MAX_BATCH (B == 0 is a no-op) */
    int32_t num_heads;           /* H, 1..128 */
    int32_t block_size;          /* bs, 64 or 128 tokens per page */
    int32_t num_blocks;          /* pages in kv_cache, >= 1 */
    int32_t max_blocks_per_seq;  /* columns of block_table, >= 1 */
    int32_t kv_dtype;            /* mla_dtype_t */
    int32_t causal;              /* 0 or 1 */
    int32_t split_keys;          /* tuning/test override, 0 in production: 0 = automatic
                                    split-KV; else every sequence is cut into chunks of this
                                    many keys (multiple of 64) */
} mla_decode_desc_t;

/* Bytes of device workspace mla_decode needs for this problem (host-only
 * arithmetic; returns 0 for an invalid or unsupported description). */
size_t mla_decode_workspace_size(int32_t s_q, const mla_decode_desc_t* desc);

/*
 * Paged MLA decode.
 *
 * All pointers are device pointers (HIP), row-major and contiguous:
 *   q            bf16  [B, s_q, H, 576]                16-byte aligned
 *   kv_cache     bf16 or e4m3fn [num_blocks, bs, 576]  16-byte aligned
 *   block_table  int32 [B, max_blocks_per_seq]; entries past ceil(L/bs) are never read
 *   seq_lens     int32 [B], 0 <= L <= max_blocks_per_seq * bs (values outside are clamped
 *                and flagged in the workspace header)
 *   out          bf16  [B, s_q, H, 512]                16-byte aligned
 *   lse          fp32  [B, s_q, H], natural log; may be NULL
 *   workspace    >= mla_decode_workspace_size() bytes, 256-byte aligned
 *   stream       a hipStream_t (NULL = the default stream)
 * softmax_scale and kv_scale must be finite and > 0; pass kv_scale = 1 for a
 * bf16 cache (it is applied either way: k = decode(code) * kv_scale).
 *
 * Ownership: the caller owns every buffer; nothing is allocated or retained.
 * Every element of out (and lse) is written, so they need no initialisation.
 * Inputs are not modified. The work is enqueued on `stream` with no host
 * synchronisation; calls that share a workspace must be ordered on a stream.
 * Errors: on any MLA_ERR_* other than MLA_ERR_HIP nothing is launched and
 * nothing is written.
 *
 * Block-table entries inside a sequence's range [0, ceil(L / bs)) must name a
 * page in [0, num_blocks). An entry outside that range is not read: its
 * tokens are left out of the softmax (as if they were not cached) and flag
 * bit 2 below is set. Entries past ceil(L / bs) are never read.
 *
 * Workspace layout after a call (for inspection by tests): int32 header
 * [0] work items, [1] chunk keys, [2] partial slots, [3] flags (bit 0: a
 * seq_len was clamped; bit 1: the plan did not fit the workspace bounds, which
 * the bounds exclude, and nothing was computed; bit 2: a block-table entry in
 * range was outside [0, num_blocks); bit 3: a work item or split of the plan
 * in the workspace did not fit this call's description, and was skipped (see
 * mla_decode_with_plan)); at byte 256 the work items, 8 x int32 each:
 * {b, row_group, key_begin, key_end, partial_slot (-1 = written directly), 0, 0, 0}.
 */
mla_status_t mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                        float kv_scale, void* out, float* lse, const mla_decode_desc_t* desc,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode on a plan made earlier: launches the decode kernel and the LSE
 * combine but not the split planner. A decode step runs the same batch
 * (same seq_lens values, s_q and description) through every layer of a model,
 * so the plan can be made once per step ("[NVIDIA] Add Cutlass MLA backend",
 * review thread on the ahead-of-time scheduler metadata: planning once per
 * batch rather than once per call) and reused for each layer's q and cache.
 *
 * `workspace` must hold the plan that mla_decode or mla_decode_plan left
 * there for the same seq_lens values, s_q and description, and nothing else
 * may have used it since. q, kv_cache, block_table (same lengths), out and
 * lse may differ from the planning call. Flag bit 2 accumulates over the calls
 * that reuse one plan. Arguments, ownership and errors as for mla_decode.
 * A plan that does not match (a stale or foreign workspace) is not trusted:
 * every work item and split is checked against this call's description
 * before any address is formed from it, and one that does not fit is skipped
 * and sets flag bit 3; the rows it would have written are then left as they
 * were (so out and lse are incomplete: a set bit 3 means the call's results
 * must not be used).
 */
mla_status_t mla_decode_with_plan(const void* q, const void* kv_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                                  float kv_scale, void* out, float* lse,
                                  const mla_decode_desc_t* desc, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* TIMING / TEST HOOK, not for production use: launches only the decode
 * kernel (no planner, no combine), for timing that kernel on its own:
 * `workspace` must already hold the plan of a preceding mla_decode or
 * mla_decode_plan call with the same seq_lens and description.
 * Rows of work items that were split get their partials in the workspace
 * instead of out/lse (fp16 rows scaled by a per-row power of two, with a
 * base-2 lse per row). Same arguments, checks and errors as mla_decode. */
mla_status_t mla_decode_fwd_only(const void* q, const void* kv_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                                 float kv_scale, void* out, float* lse,
                                 const mla_decode_desc_t* desc, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Runs only the split planner (the first kernel mla_decode launches) and
 * leaves the header and work items in the workspace as described above, ready
 * for mla_decode_with_plan (also used by tests to inspect the plan). */
mla_status_t mla_decode_plan(const int32_t* seq_lens, int32_t s_q, const mla_decode_desc_t* desc,
                             void* workspace, size_t workspace_bytes, void* stream);

/* TEST HOOK, not for production use: host mirror of the planner; fills
 * items[8 * n] for host seq_lens; returns the number of items, or -1 if the
 * description is invalid or max_items is short. Also reports rows per work
 * item and the chunk length chosen. */
int32_t mla_plan_host(const int32_t* seq_lens_host, int32_t s_q, const mla_decode_desc_t* desc,
                      int32_t* items, int32_t max_items, int32_t* rows_per_item,
                      int32_t* chunk_keys);

/*
 * Write new latent rows into the paged cache (the step before decode; the
 * cache dtype is torch.float8_e4m3fn in "[Attention] Blackwell FP8 MLA support
 * with CUTLASS_MLA backend", Purpose and Test Plan).
 *
 *   rows          bf16 [n_tokens, 576], device, 16-byte aligned
 *   slot_mapping  int32 [n_tokens], device: row n goes to cache slot
 *                 slot_mapping[n] = page * block_size + offset; a negative slot
 *                 (padding) or one >= num_blocks * block_size writes nothing
 *   kv_cache      [num_blocks, block_size, 576] bf16 or e4m3fn, device, 16-byte aligned
 * Each value is stored as y = x / kv_scale (float32, correctly rounded): for
 * fp8 clamped to +-448 and rounded to the nearest e4m3fn value (ties to the
 * even mantissa; NaN stays NaN), for bf16 rounded to nearest even. Decoding
 * (mla_decode) multiplies by kv_scale again.
 * Ownership and errors as for mla_decode; slots that repeat within one call
 * race. n_tokens == 0 is a no-op.
 */
mla_status_t mla_kv_append(const void* rows, const int32_t* slot_mapping, int32_t n_tokens,
                           float kv_scale, void* kv_cache, int32_t num_blocks, int32_t block_size,
                           int32_t kv_dtype, void* stream);

/*
 * The absorbed projections around the decode MQA ("[WIP][Attention] FlashAttn
 * MLA", description: MLA's decode step is computed as MQA over the latent
 * cache, so the per-head up-projections move onto the query and the output).
 * Reading used (the pages give no shapes): per token t and head h,
 *   mla_absorb_q:   q_out[t][h][0:512]   = q_nope[t][h][0:d_nope] . w_uk[h]
 *                   q_out[t][h][512:576] = q_pe[t][h][0:64]   (copied)
 *   mla_absorb_out: out[t][h][0:d_v]     = o[t][h][0:512] . w_uv[h]
 * All device pointers, bf16, row-major, 16-byte aligned:
 *   q_nope [tokens, heads, d_nope]; q_pe [tokens, heads, 64];
 *   w_uk [heads, d_nope, 512]; q_out [tokens, heads, 576] (the q of mla_decode);
 *   o [tokens, heads, 512] (the out of mla_decode); w_uv [heads, 512, d_v];
 *   out [tokens, heads, d_v].
 * fp32 accumulation, bf16 result rounded to nearest even. d_nope: a multiple
 * of 32; d_v: a multiple of 64 (both <= 4096); 1 <= heads <= 128. tokens == 0
 * is a no-op. Errors as for mla_decode.
 */
mla_status_t mla_absorb_q(const void* q_nope, const void* q_pe, const void* w_uk, void* q_out,
                          int32_t tokens, int32_t heads, int32_t d_nope, void* stream);
mla_status_t mla_absorb_out(const void* o, const void* w_uv, void* out, int32_t tokens,
                            int32_t heads, int32_t d_v, void* stream);

/*
 * mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same decode, with the workspace replaced by a fixed device array of
 * MLA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU it
 * runs on until the process ends. Nothing is allocated per call.
 *
 * When mla_decode_workspace_size() fits the array, the plan and the results
 * are those of mla_decode; otherwise (long 128-head batches) the automatic
 * split uses fewer partial slots (longer key chunks) so that it fits.
 * Descriptions that do not fit even unsplit, or a split_keys override that
 * does not fit, return MLA_ERR_WORKSPACE_TOO_SMALL and launch nothing.
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or host threads without ordering) race and must
 * be serialised by the caller; calls on one stream are ordered. Every value
 * the kernels read from the array is written earlier in the same call.
 * Arguments (no workspace), ownership and errors as for mla_decode;
 * MLA_ERR_HIP also when the array's device address cannot be obtained.
 */
mla_status_t mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                const int32_t* seq_lens, int32_t s_q, float softmax_scale,
                                float kv_scale, void* out, float* lse,
                                const mla_decode_desc_t* desc, void* stream);
/* MLA_NOALLOC_SCRATCH_BYTES, as compiled into the library. */
size_t mla_decode_noalloc_scratch_bytes(void);

const char* mla_status_string(mla_status_t status);
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
