/*
 * bsattn.h - C ABI of the selected-block (block-sparse) attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method has two phases (vllm-omni PR #8335 "[Core] Add shared
 * block-sparse attention adapters with FlashAttention-4", Purpose): a
 * selector produces, per query head and query block, a list of KV-block
 * indices and a count; an attention backend then executes exactly that
 * selection. The protected KV prefix, suffix padding and the native
 * MHA/MQA/GQA head mapping are part of the contract (same section). An error
 * of the provider reaches the caller: it is never answered by dense attention
 * or by repeating K/V heads, under any condition (same section).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers to tensors are device pointers the caller owns (hipMalloc or a
 *   framework allocator). The library allocates no memory on any call path.
 * - Every call is asynchronous on `stream` (0 = the null stream). No call
 *   synchronises the host, and none copies host memory to the device: all
 *   metadata travels as kernel arguments. (The list-checking build is the
 *   exception: see attn_block_sparse_fwd.)
 * - q, k, v, out: bf16, 16-byte aligned, head_dim contiguous, element
 *   strides given per (batch, sequence, head) in `attn_shape`, each a
 *   multiple of 8.
 * - block_idx / block_cnt: int32, contiguous, [batch][num_q_heads][NQ][row]
 *   and [batch][num_q_heads][NQ] with NQ = q_len / block_q and row stride
 *   `idx_row_stride`.
 * - lse (optional, may be NULL): fp32, contiguous [batch][num_q_heads][q_len],
 *   natural-log log-sum-exp of the scaled logits of each query row.
 * - Arguments are validated on the host before any launch. On error nothing
 *   is launched, no output is touched, the status is returned and
 *   attn_last_error() describes the failure (per calling thread).
 * - Results are deterministic: equal inputs give bitwise equal outputs.
 *
 * Sequence layout (diffusers examples/cosmos3/cosmos_parallel.py,
 * shard_cosmos3_sequence / build_gen_key_mask / cosmos3_cp_attention): the
 * queries are the generation tokens; the keys and values are the
 * concatenation of a protected prefix segment and the generation segment,
 * each padded on its own to a multiple of block_k. Padded keys take no
 * attention weight; padded query rows produce zero output and lse = -inf.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* inconsistent or out-of-range argument */
  ATTN_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels implement */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  ATTN_ERR_LAUNCH = 4,      /* a kernel launch failed */
  ATTN_ERR_DEVICE = 5,      /* no device, or the current device is not gfx950 */
  ATTN_ERR_SELF_TEST = 6    /* attn_self_test: a result differs from its known value */
} attn_status;

typedef struct attn_shape {
  int32_t batch;         /* >= 1 */
  int32_t num_q_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;  /* Hkv >= 1, Hq % Hkv == 0; query head h reads KV head h / (Hq/Hkv) */
  int32_t head_dim;      /* D in {64, 128} */
  int32_t block_q;       /* query rows per block, in {64, 128, 256} */
  int32_t block_k;       /* keys per block, in {64, 128} */
  int32_t q_len;         /* padded query length, multiple of block_q */
  int32_t q_valid;       /* real query rows [0, q_valid) */
  int32_t kv_prefix_len;   /* protected segment [0, kv_prefix_len), multiple of block_k;
                              its P = kv_prefix_len / block_k blocks are always kept */
  int32_t kv_prefix_valid; /* real keys [0, kv_prefix_valid) of the prefix segment */
  int32_t kv_len;          /* padded key length, multiple of block_k, >= kv_prefix_len */
  int32_t kv_suffix_valid; /* real keys [kv_prefix_len, kv_prefix_len + kv_suffix_valid) */
  int64_t q_stride[3];   /* element strides of q for (batch, seq, head) */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  float softmax_scale;   /* <= 0 selects head_dim ** -0.5 (mstar PR #927, automated review) */
} attn_shape;

/* Kept KV blocks per query-block row for a target sparsity in percent: the
 * protected prefix blocks count inside the budget;
 * clamp(ceil(n_kv_blocks * (100 - sparsity_pct) / 100), n_protected, n_kv_blocks).
 * The 75 % target of vllm-omni PR #8335 (Purpose) gives 191 of 764 blocks.
 * Returns -1 if 0 <= n_protected <= n_kv_blocks or 0 <= sparsity_pct <= 100
 * does not hold. Pure host arithmetic. */
int32_t attn_keep_blocks(int32_t n_kv_blocks, int32_t n_protected, int32_t sparsity_pct);

/* Bytes of device workspace attn_select_blocks needs for `shape` (pooled
 * queries and keys and their norms). The caller takes this scratch once, up
 * front, and passes it to every call, so no call path allocates (mstar PR
 * #927, Since the review: the attention wrappers share one workspace taken
 * at build). 0 if the shape is invalid. */
size_t attn_select_workspace_size(const attn_shape* shape);

/* Block selector (vllm-omni PR #8335, Purpose: a list of KV blocks and its
 * length per query head and query block; protected KV prefixes).
 *
 * For each (batch b, query head h, query block i) with at least one real row:
 *  1. mean-pool the real rows of the query block and the real keys of every KV
 *     block of KV head h / (Hq/Hkv): exact sum, one fp64 division, one
 *     rounding to fp32;
 *  2. score KV block j as the fp32 value nearest to the exact dot product of
 *     the two pooled vectors (no softmax scale);
 *  3. keep every protected block that holds a real key, then the best other
 *     non-empty blocks by (score descending, index ascending) until
 *     keep_blocks blocks are kept or none is left.
 * The pages leave the scoring rule open; block-mean pooling is the reading
 * this library implements.
 *
 * Writes block_idx rows in ascending order, unused slots set to -1, and
 * block_cnt. Query blocks without a real row get count 0.
 *
 * Requirements: P <= keep_blocks <= NK (P = kv_prefix_len / block_k,
 * NK = kv_len / block_k); idx_row_stride >= keep_blocks; NK <= 4096;
 * workspace of at least attn_select_workspace_size(shape) bytes, 256-byte
 * aligned, whose contents are scratch. Real (non-padding) inputs must be
 * finite; padding may hold anything. */
attn_status attn_select_blocks(const attn_shape* shape, const void* q, const void* k,
                               int32_t keep_blocks, int32_t* block_idx, int32_t* block_cnt,
                               int32_t idx_row_stride, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Bytes of the selector scratch array the library holds on each device for
 * attn_select_blocks_noalloc (64 MiB: the 48k-token and 720p workloads need
 * 28 MB and 45 MB). */
#define ATTN_SELECT_STATIC_WORKSPACE_BYTES (64u << 20)

/* attn_select_blocks without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments (minus the workspace),
 * same results, bit for bit. The pooled vectors live in a fixed array of
 * ATTN_SELECT_STATIC_WORKSPACE_BYTES that the library keeps on every device
 * it runs on until the process ends; the call allocates nothing. Returns
 * ATTN_ERR_WORKSPACE if attn_select_workspace_size(shape) exceeds the array.
 * Every call on a device shares that device's array: calls that overlap on
 * one device (other streams, other threads) race and must be serialised by
 * the caller. */
attn_status attn_select_blocks_noalloc(const attn_shape* shape, const void* q, const void* k,
                                       int32_t keep_blocks, int32_t* block_idx,
                                       int32_t* block_cnt, int32_t idx_row_stride,
                                       hipStream_t stream);

/* Block-sparse attention (vllm-omni PR #8335, Purpose: the backend executes
 * the selection; diffusers cosmos_parallel.py, cosmos3_cp_attention: the
 * generation pathway's non-causal attention over cat(prefix, gen)).
 *
 * For each real query row t of block i of query head h in batch b:
 *   out[b,t,h,:] = sum_u softmax_u(scale * q.k_u) v_u
 * over the real keys u of the blocks block_idx[b,h,i,0 .. cnt-1] of KV head
 * h / (Hq/Hkv), cnt = block_cnt[b,h,i] clamped to [0, idx_row_stride].
 * bf16 inputs, fp32 accumulation and softmax, bf16 output. Rows with no key
 * (cnt 0, or only padded keys) and padded rows give 0 and lse -inf. Listed
 * blocks should be distinct and in [0, NK); the order of the list does not
 * matter. The release build skips entries outside [0, NK) and counts a
 * repeated block twice. The list-checking build (libbsattn_checked.so,
 * compiled with BSATTN_CHECK_LISTS=1) first checks the list of every query
 * block that has a real row, on `stream`, and waits for the check: a count
 * outside [0, idx_row_stride], an entry outside [0, NK) or a repeated entry
 * returns ATTN_ERR_INVALID_ARG naming the lowest such (batch, head, query
 * block), and nothing is written. */
attn_status attn_block_sparse_fwd(const attn_shape* shape, const void* q, const void* k,
                                  const void* v, const int32_t* block_idx,
                                  const int32_t* block_cnt, int32_t idx_row_stride, void* out,
                                  float* lse, hipStream_t stream);

/* Dense attention: attn_block_sparse_fwd with every KV block listed (the
 * 0 % sparsity case), through the same kernel; no index list is read. */
attn_status attn_dense_fwd(const attn_shape* shape, const void* q, const void* k, const void* v,
                           void* out, float* lse, hipStream_t stream);

/* Causal dense attention (diffusers cosmos_parallel.py, cosmos3_cp_attention:
 * the understanding pathway attends to itself causally; mstar PR #927,
 * automated review: the dense pass keeps the bottom-right causal alignment of
 * the FA3 call).
 *
 * Same arguments and layout as attn_dense_fwd. Keys are ranked in order among
 * the real keys only (the prefix segment's real keys, then the generation
 * segment's); with n_k real keys and n_q = q_valid real rows, real row t
 * attends the real keys of rank <= t + (n_k - n_q), so the last real row sees
 * every real key (bottom-right alignment). For a stream attending to itself
 * (n_k == n_q, e.g. kv_prefix_len = 0 and kv_suffix_valid = q_valid) this is
 * the usual mask "key <= query". Rows left with no key (n_q > n_k) give 0 and
 * lse -inf, as padded rows do. Blocks past a query block's last reachable key
 * are not visited. */
attn_status attn_dense_causal_fwd(const attn_shape* shape, const void* q, const void* k,
                                  const void* v, void* out, float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Step/layer attention strategy: a thin host layer over the calls above that
 * picks dense or selected-sparse attention per (denoising step, layer)
 * (vllm-omni PR #8583, Purpose: dense or sparse chosen per step and layer,
 * recipes that turn every layer sparse from one step on or only some layers,
 * and every layout run once before the first timed step; PR #8644, Purpose:
 * the first twenty iterations dense, then every layer sparse).
 *
 * Steps [0, dense_steps) run every layer dense. From step dense_steps on,
 * layer l runs sparse when bit l of sparse_layers is set, dense otherwise.
 * Examples: the Cosmos3 mixed recipe is {36, 10, bits 8..35, 75}; always
 * sparse is {36, 0, all 36 bits, 75}; the H3 switch is {50, 20, all 50 bits,
 * 75}. */
typedef struct attn_strategy {
  int32_t num_layers;     /* layers per denoising step, 1..64 */
  int32_t dense_steps;    /* >= 0 */
  uint64_t sparse_layers; /* bit l = layer l sparse after dense_steps; no bit at or above num_layers */
  int32_t sparsity_pct;   /* target sparsity of the sparse calls, 0..100 (attn_keep_blocks) */
} attn_strategy;

/* 1 if the call of `layer` in denoising step `step` is sparse, 0 if dense,
 * -1 if the strategy or (step, layer) is invalid. Pure host arithmetic. */
int32_t attn_strategy_is_sparse(const attn_strategy* strategy, int32_t step, int32_t layer);

/* Bytes of device workspace attn_strategy_fwd and attn_strategy_warmup need
 * for `shape`: the block lists and counts of a sparse call followed by the
 * selector's workspace. 0 if the shape or the strategy is invalid. */
size_t attn_strategy_workspace_size(const attn_shape* shape, const attn_strategy* strategy);

/* The attention of (step, layer) under `strategy`: attn_dense_fwd for a dense
 * call; for a sparse call attn_select_blocks with keep_blocks =
 * attn_keep_blocks(NK, P, sparsity_pct) into the workspace, then
 * attn_block_sparse_fwd. Arguments as for those calls; the workspace
 * (256-byte aligned, attn_strategy_workspace_size bytes) is scratch owned by
 * the caller. Errors of the underlying calls propagate unchanged. */
attn_status attn_strategy_fwd(const attn_shape* shape, const attn_strategy* strategy,
                              int32_t step, int32_t layer, const void* q, const void* k,
                              const void* v, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Warmup across layouts: runs once every kind of call the strategy can make
 * for `shape` (dense and/or select + sparse), so the first launch of each
 * kernel (which loads its code object) happens before the first denoising
 * step. `out` is overwritten; the workspace is as for attn_strategy_fwd. */
attn_status attn_strategy_warmup(const attn_shape* shape, const attn_strategy* strategy,
                                 const void* q, const void* k, const void* v, void* out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Whether `shape` is supported by the sparse path, checked without touching
 * the device (vllm-omni PR #8335, Purpose: sparse compatibility is checked
 * independently of dense-kernel restrictions). ATTN_OK or the error the
 * entry points would return; attn_last_error() says why. */
attn_status attn_query_support(const attn_shape* shape);

/* Start-up check (the tiny plan-and-run check at boot of mstar PR #927,
 * "Since the review"): selects and runs a tiny case on the current device
 * (2 query heads, 1 KV head, head_dim 128, 64x64 blocks, 100 of 128 query
 * rows real, a protected prefix of 40 real keys and 88 generation keys, NaN
 * in every padded row) through attn_select_blocks, attn_block_sparse_fwd,
 * attn_dense_fwd and attn_dense_causal_fwd, and compares every output with
 * the value its construction fixes: the keys are scaled one-hot vectors, so
 * each row's softmax is exactly one-hot on its target key or exactly
 * uniform over the visible keys; the block list is checked for count, order,
 * range, the protected block and the -1 fill.
 * Unlike every other entry point this one allocates (about 0.2 MB of device
 * memory, freed before it returns), runs on the null stream and synchronises
 * the device: it is meant for start-up, not for a call path. Returns ATTN_OK;
 * ATTN_ERR_DEVICE if the device is missing, not a gfx950 or a HIP call fails;
 * the status of a failing entry point; or ATTN_ERR_SELF_TEST when a result
 * differs. attn_last_error() then names the device, its architecture, the
 * check, the position and the values, and the library version. */
attn_status attn_self_test(void);

/* Description of the last failure on the calling thread ("" if none): the
 * entry point, what failed, the library version and target architecture
 * (mstar PR #927, Since the review: a misconfigured backend fails at start-up
 * with an error that names the backend, the GPU and the version).
 * The string belongs to the library and stays valid until the next call of
 * an entry point on the same thread. */
const char* attn_last_error(void);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
