/*
 * pkv.h - C ABI of libpkv: an int8 ("C8") paged KV cache for one AMD Instinct
 * MI355X (gfx950).  Three operations, after the pages that define them:
 *
 *   pkv_store_c8    quantize new bf16 K/V tokens and write them into the
 *                   block-table-indexed cache (MojoStorePagedKVCacheC8 in
 *                   Mojo Opset PR #379; its bf16 sibling MojoStorePagedKVCache
 *                   in the README's Op List).
 *   pkv_dequant     gather a sequence's cache back to bf16 rows
 *                   (MojoDequantFromPagedKVCache in PR #379).
 *   pkv_decode_gqa  grouped-query attention of the new queries over the paged
 *                   cache (MojoPagedDecodeGQA in the README's Op List), with
 *                   split-KV partitions and a log-sum-exp merge; decode (one
 *                   query per sequence), causal chunks and whole-prompt prefill
 *                   (MojoPagedPrefillGQA), optionally over a sliding window
 *                   (MojoSlidingWindowAttention).
 *   pkv_mla_store_c8 / pkv_mla_decode  the same for a latent (MLA) cache
 *                   (MojoStorePagedMLAKVCache, MojoPagedDecodeMLA; see the MLA
 *                   section below).
 *
 * Conventions shared by every call
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates: scratch space for decode is the caller's
 *    workspace, sized by pkv_decode_workspace_size.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns a pkv_status.  Only host-checkable conditions are
 *    reported (null pointers, unsupported shapes, modes or alignments, a small
 *    workspace, a failed launch).  When a call returns an error nothing has
 *    been launched.
 *  - Device-resident index data (block_table, context_lengths, cu_q_lens,
 *    slot_mapping, seq_offsets) are preconditions, not checked: reading them
 *    on the host would need a synchronisation.  They must be in range
 *    (pkv_check_indices checks them on the device, for debugging).
 *  - context_lengths[b] counts every position of sequence b AFTER the call's
 *    new tokens are stored; the new tokens of b occupy positions
 *    [context_lengths[b] - q_len_b, context_lengths[b]).
 *  - Results are deterministic: fixed split plan, fixed merge order, no
 *    floating-point atomics.  Calls are reentrant; the only state kept is the
 *    device's compute-unit count (and, for pkv_decode_gqa_noalloc, the address
 *    of its per-device scratch array, whose calls share that array).
 *
 * Cache layout (caller-owned; element (block, kv head, slot, channel)):
 *   K       [num_blocks][num_kv_heads][block_size][head_dim]  (token-major page)
 *   V       [num_blocks][num_kv_heads][block_size/16][head_dim][16]  (the page in
 *           16-slot tiles, each channel-major: slots 16i .. 16i+15 of one channel are
 *           16 adjacent elements)
 *   scales  PKV_QUANT_PER_TOKEN: float [num_blocks][num_kv_heads][block_size]
 *           PKV_QUANT_PER_BLOCK: float [num_blocks][num_kv_heads]
 *           PKV_QUANT_NONE_BF16: none (K and V hold bf16)
 *           PKV_QUANT_PER_CHANNEL: float [num_kv_heads][head_dim], static (set by
 *           the caller, e.g. from a calibration; the library never writes them)
 *   int8 codes for the quantized modes, bf16 for PKV_QUANT_NONE_BF16.
 *   K, V and the scale arrays: 16-byte aligned.
 *   Supported: head_dim 64 or 128; block_size 16, 32, 64 or 128.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent arguments */
    PKV_ERR_UNSUPPORTED = -2, /* head_dim / block_size / mode outside the supported set */
    PKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    PKV_ERR_HIP = -4          /* a kernel launch or device query failed */
} pkv_status;

typedef enum {
    /* one fp32 scale per token and KV head: scale = absmax/127 of the token's
       head_dim values (dynamic symmetric quantization, MojoDynamicQuant in the
       README's Op List) */
    PKV_QUANT_PER_TOKEN = 0,
    /* one fp32 scale per block and KV head (PR #379's per-block scale layout
       for quant_mode != 0): absmax/127 of every value the block holds */
    PKV_QUANT_PER_BLOCK = 1,
    /* no quantization: K and V pages hold bf16 */
    PKV_QUANT_NONE_BF16 = 2,
    /* static per-channel scales, one per (KV head, channel), broadcast over the
       tokens (the scale[..., None, :] layout that PR #379's review passes name
       for the C8 dequant): code = clamp(rne(fl32(x / s_c)), -128, 127), which
       saturates values beyond the calibrated range; the store writes codes only.
       Decoded by the int8-score kernel only (kernel 3). */
    PKV_QUANT_PER_CHANNEL = 3
} pkv_quant_mode;

/* A caller-owned paged cache.  Shapes travel with the pointers. */
typedef struct {
    void *k;        /* int8 (or bf16) pages, layout above */
    void *v;        /* int8 (or bf16) pages, layout above */
    float *k_scale; /* NULL in PKV_QUANT_NONE_BF16 */
    float *v_scale; /* NULL in PKV_QUANT_NONE_BF16 */
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t head_dim;
    int32_t quant_mode; /* pkv_quant_mode */
} pkv_cache_t;

/* Human-readable name of a pkv_status. Never NULL. */
const char *pkv_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int pkv_version(void);

/*
 * pkv_store_c8 - quantize new tokens and write them into the cache.
 *
 * k_new, v_new  bf16 [num_tokens][num_kv_heads][head_dim], row-major.
 * Slot of new token t, in one of two forms:
 *  - slot_mapping != NULL (int64 [num_tokens]): block = slot / block_size,
 *    slot in block = slot % block_size; a negative entry skips the token.
 *    cu_q_lens, context_lengths and block_table are then ignored.
 *    Not available with PKV_QUANT_PER_BLOCK.
 *  - slot_mapping == NULL: cu_q_lens (int32 [batch + 1], prefix sums of the
 *    per-sequence new-token counts; NULL means one new token per sequence,
 *    token b belongs to sequence b, num_tokens == batch), context_lengths
 *    (int32 [batch]) and block_table (int32 [batch][max_blocks_per_seq]):
 *    token i of sequence b lands at position
 *    p = context_lengths[b] - q_len_b + i, block block_table[b][p/block_size].
 * max_q_len     host-known upper bound of the per-sequence new-token counts
 *               (used to size the per-block launch; <= 0 means num_tokens).
 * quant_mode    must equal cache->quant_mode.
 *
 * Per token (mode 0), for each token and KV head independently:
 *   scale = fl32(absmax / 127),  code = clamp(rne(fl32(x / scale)), -128, 127)
 *   (code 0 when scale == 0); rne rounds halves to even (PR #379 reviews:
 *   symmetric int8 codes, x over the scale, rounded and clamped; the division
 *   in fp32).
 * Per block (mode 1), for each (sequence, block touched, KV head):
 *   s = max(s_old, fl32(absmax_new / 127)) where s_old is the block's scale
 *   when positions before the new tokens already live in the block; if s
 *   grows, the block's existing codes are re-quantized from fl32(code * s_old);
 *   the new tokens are quantized with s.  Precondition: no physical block is
 *   shared between sequences.
 * bf16 (mode 2): the values are copied.
 * Per channel (mode 3): code = clamp(rne(fl32(x / s_c)), -128, 127) with the
 *   static scale s_c of the value's (KV head, channel) (code 0 when s_c == 0);
 *   the scale arrays are read, never written.
 *
 * num_tokens == 0 returns PKV_OK without launching anything.
 */
int pkv_store_c8(const pkv_cache_t *cache, const void *k_new, const void *v_new,
                 int32_t num_tokens, const int64_t *slot_mapping, const int32_t *cu_q_lens,
                 const int32_t *context_lengths, const int32_t *block_table, int32_t batch,
                 int32_t max_blocks_per_seq, int32_t max_q_len, int32_t quant_mode, void *stream);

/*
 * pkv_dequant - gather every sequence's cache back to bf16
 * (MojoDequantFromPagedKVCache, PR #379).
 *
 * For b < batch, position p < context_lengths[b], KV head h, channel c:
 *   out[(off_b + p) * token_stride + h * head_stride + c] = bf16_rne(fl32(code * scale))
 * (the product in fp32, PR #379 reviews), or the stored bf16 value in mode 2.
 * off_b = seq_offsets[b] (int64 [batch]) or, when seq_offsets is NULL, the
 * exclusive prefix sum of context_lengths.  Rows outside every sequence (the
 * padding of a padded layout) are not written.  Strides are in elements;
 * channels are contiguous.  k_out or v_out may be NULL to skip that half.
 */
int pkv_dequant(const pkv_cache_t *cache, const int32_t *block_table, int32_t max_blocks_per_seq,
                const int32_t *context_lengths, const int64_t *seq_offsets, int32_t batch,
                void *k_out, void *v_out, int64_t token_stride, int64_t head_stride, void *stream);

/*
 * pkv_cache_walk - a measurement aid: the read ceiling of the int8 decode's
 * access pattern over this cache (not an operation of the pages).
 *
 * One wave per (sequence b, KV head h, split s of split_tokens keys), launched
 * in the order of pkv_decode_gqa's fixed partition, reads what the decode of
 * keys [s * split_tokens, min((s + 1) * split_tokens, context_lengths[b])) reads
 * from the cache - their K rows, the whole 16-slot V tiles that hold them, and
 * their per-token K and V scales (mode 0) or the per-block scales of the pages
 * they touch, each page once per wave (mode 1; none in mode 3) - and computes
 * nothing else, with `depth` (1..3) blocks of 64 keys in flight per wave (the
 * decode keeps 1).  out[(b * num_kv_heads + h) * nsplit + s] receives the
 * wrapping uint32 sum of the 32-bit words that wave read (0 for a split past
 * the context), nsplit = ceil(max_blocks_per_seq * block_size / split_tokens);
 * out holds batch * num_kv_heads * nsplit entries (device, 4-byte aligned).
 * split_tokens: a multiple of 64 in [64, 4096].  Int8 modes only (mode 2:
 * PKV_ERR_UNSUPPORTED).  Errors as pkv_dequant.
 */
int pkv_cache_walk(const pkv_cache_t *cache, const int32_t *block_table, int32_t max_blocks_per_seq,
                   const int32_t *context_lengths, int32_t batch, int32_t split_tokens, int32_t depth,
                   uint32_t *out, void *stream);

/* Bits of pkv_check_indices' result[0]. */
enum {
    PKV_CHECK_CONTEXT = 1, /* a context length outside [0, max_blocks_per_seq * block_size] */
    PKV_CHECK_BLOCK = 2,   /* a block-table entry the context reaches outside [0, num_blocks) */
    PKV_CHECK_QLEN = 4,    /* cu_q_lens[0] != 0, cu_q_lens decreasing, or a q_len above the
                              sequence's context length or above max_q_len (when > 0) */
    PKV_CHECK_SLOT = 8     /* a slot-mapping entry >= num_blocks * block_size */
};

/*
 * pkv_check_indices - optional debug validator (not an operation of the pages):
 * checks on the device the index arrays that the other calls take as unchecked
 * preconditions (see "Device-resident index data" above), before a call that
 * would read out of bounds with them is made.
 *
 * num_blocks, block_size  the pool's size (a pkv_cache_t's or an MLA cache's).
 * block_table   int32 [batch][max_blocks_per_seq] or NULL; entries j with
 *               j * block_size < context_lengths[b] are checked (the calls read
 *               no others).  Needs context_lengths.
 * context_lengths  int32 [batch] or NULL.
 * cu_q_lens     int32 [batch + 1] or NULL; max_q_len <= 0: no upper bound.
 * slot_mapping  int64 [num_tokens] or NULL (negative entries are valid: the
 *               store skips them).
 * result        device int32 [4], 4-byte aligned, fully written by the call:
 *               [0] the PKV_CHECK_* bits of every violated condition (0: all
 *               hold), [1] the lowest offending sequence (-1: none), [2] the
 *               lowest offending token of slot_mapping (-1: none), [3] 0.
 * One launch of one workgroup, asynchronous on `stream`; the caller reads
 * `result` once the stream has reached the call.  The check reads only inside
 * the arrays' stated sizes, whatever their contents.  Not checked: that no
 * physical block is shared between sequences (pkv_store_c8's per-block mode).
 * Errors (nothing launched): PKV_ERR_INVALID_ARG for a NULL or misaligned
 * result, negative sizes, a block table without context lengths, batch > 0
 * with no array to check, or num_tokens > 0 without slot_mapping.
 */
int pkv_check_indices(int32_t num_blocks, int32_t block_size, const int32_t *block_table,
                      int32_t max_blocks_per_seq, const int32_t *context_lengths,
                      const int32_t *cu_q_lens, int32_t max_q_len, int32_t batch,
                      const int64_t *slot_mapping, int32_t num_tokens, int32_t *result,
                      void *stream);

/* Optional knobs of pkv_decode_gqa (pass NULL for the defaults). */
typedef struct {
    int32_t split_tokens; /* keys per fixed split-KV partition, rounded up to a multiple
                             of 128 (64 for kernel 3), at most 4096; 0 = sized from the
                             shapes.  A value
                             > 0 selects fixed splits.  The balanced partition cuts all
                             64-key blocks of all query groups into near-equal ranges,
                             as many as the GPU holds waves of the kernel at once (or a
                             multiple of that, several rounds, when the query groups
                             are not few against those waves). */
    int32_t kernel;       /* 0 = choose (3 for int8 caches, 2 for bf16); 1 = VALU split-KV kernel
                             (dot2 + DPP reductions); 2 = MFMA kernel with fp16 / bf16
                             scores; 3 = MFMA kernel with exact int8 scores and key
                             subsets packed into the tile columns (int8 caches; a bf16
                             cache falls back to 2); 4 = tile kernel for many query rows
                             per KV head (prompts, multi-token chunks): one workgroup per
                             128 rows of a (sequence, KV head), each 64-key block loaded
                             once per workgroup and shared through LDS, fp16 scores;
                             one pass over each tile's keys where the tiles fill two rounds
                             of the GPU's workgroups (4 per CU), else contexts above 4096
                             keys (and split_tokens > 0 always) in key splits with a
                             log-sum-exp merge and a workspace (per-token or per-block int8
                             caches, head_dim 128, no window, partition 0; otherwise
                             PKV_ERR_UNSUPPORTED) */
    int32_t partition;    /* how the keys are cut into work (kernels 3 and 2):
                             0 = planned: kernel 3 takes the balanced partition for
                             contexts of 16384 keys or more with query groups at most
                             half its resident waves, kernel 2 (bf16 caches, head_dim
                             128, one 16-row tile) for contexts of 4096 keys or more,
                             planned over several rounds; otherwise fixed splits;
                             1 = fixed splits of split_tokens keys; 2 = balanced
                             partition whenever the shapes allow it (at most 4096
                             sequences; kernel 2: bf16, head_dim 128, up to 16 query
                             rows per KV head). */
    int32_t window;       /* > 0: sliding window, each query attends only to its
                             last `window` positions (itself included; the
                             MojoSlidingWindowAttention row of the README's Op
                             List); 0: every earlier position */
    int32_t reserved[4];  /* must be zero */
} pkv_decode_opts_t;

/* Bytes of workspace pkv_decode_gqa needs for these shapes (0 when it needs
 * none).  Depends on the current device's compute-unit count. */
size_t pkv_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t max_q_len, int32_t quant_mode,
                                 const pkv_decode_opts_t *opts);

/*
 * pkv_decode_gqa - attention of the new queries over the paged cache
 * (MojoPagedDecodeGQA, README Op List).
 *
 * q        bf16 [Tq][num_q_heads][head_dim]; Tq = batch when cu_q_lens is NULL
 *          (one query per sequence), else cu_q_lens[batch].
 * Query i < q_len_b of sequence b sits at position p = context_lengths[b] -
 * q_len_b + i and attends to keys 0..p (causal within its chunk).  Query head
 * hq reads KV head hq / G, G = num_q_heads / num_kv_heads.
 *   out = softmax(scale * q K^T) V   over the dequantized keys and values,
 * accumulated in fp32 and written as bf16 [Tq][num_q_heads][head_dim].
 * lse_out  optional fp32 [Tq][num_q_heads]: natural log of the softmax
 *          denominator of the scaled logits; -inf for a sequence with no keys
 *          (whose output is 0).
 * max_q_len host-known upper bound of q_len_b (1 for pure decode).
 * workspace / workspace_bytes: caller scratch of at least
 *          pkv_decode_workspace_size(...) bytes, 16-byte aligned (split
 *          partials; no initial contents needed).  Calls that run
 *          concurrently must not share a workspace.
 */
int pkv_decode_gqa(const void *q, int32_t num_q_heads, const pkv_cache_t *cache,
                   const int32_t *block_table, int32_t max_blocks_per_seq,
                   const int32_t *context_lengths, const int32_t *cu_q_lens, int32_t batch,
                   int32_t max_q_len, float scale, void *out, float *lse_out, void *workspace,
                   size_t workspace_bytes, const pkv_decode_opts_t *opts, void *stream);

/*
 * pkv_store_decode_gqa - one decode step in one call: store each sequence's
 * new K/V token, then attend (MojoStorePagedKVCacheC8 of PR #379 followed by
 * MojoPagedDecodeGQA of the README's Op List, one query per sequence).
 *
 * The result equals pkv_store_c8(cache, k_new, v_new, batch, NULL, NULL,
 * context_lengths, block_table, batch, max_blocks_per_seq, 1, mode) followed
 * by pkv_decode_gqa(q, ..., cu_q_lens = NULL, max_q_len = 1, ...):
 * k_new, v_new  bf16 [batch][num_kv_heads][head_dim], 4-byte aligned; the
 *               token of sequence b goes to position context_lengths[b] - 1
 *               (a sequence with context length 0 stores nothing).
 * Other arguments, the workspace and errors as pkv_decode_gqa.  For per-token
 * and per-channel caches decoded by the int8-score kernel with one row group
 * per KV head (up to 16 query heads per KV head) the store happens inside the
 * decode launch: the wave that attends to the new position quantizes the
 * token, writes it to the cache and uses its codes directly; otherwise a
 * store launch precedes the decode.
 */
int pkv_store_decode_gqa(const void *q, const void *k_new, const void *v_new, int32_t num_q_heads,
                         const pkv_cache_t *cache, const int32_t *block_table,
                         int32_t max_blocks_per_seq, const int32_t *context_lengths, int32_t batch,
                         float scale, void *out, float *lse_out, void *workspace,
                         size_t workspace_bytes, const pkv_decode_opts_t *opts, void *stream);

/* The split plan pkv_decode_gqa would use, for tests and benchmarks.
 * Writes the keys per partition and the number of partitions per row group
 * (for a balanced partition: 0 and the number of waves), and the kernel
 * (1 VALU, 2 or 3 MFMA); any output pointer may be NULL. */
int pkv_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t max_blocks_per_seq, int32_t block_size, int32_t max_q_len,
                    int32_t quant_mode, const pkv_decode_opts_t *opts, int32_t *split_tokens,
                    int32_t *num_splits, int32_t *kernel);

/* Size of the fixed device array that pkv_decode_gqa_noalloc takes its
 * workspace from (one copy per GPU, held until the process ends). */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * pkv_decode_gqa_noalloc - pkv_decode_gqa for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and result as pkv_decode_gqa, minus
 * the workspace: the split partials go to a file-scope device array of
 * PKV_NOALLOC_SCRATCH_BYTES inside the library.  The call allocates nothing
 * (no hipMalloc, no hipFree).
 *
 * Limits and errors:
 *  - PKV_ERR_WORKSPACE (nothing launched) when the plan needs more than
 *    PKV_NOALLOC_SCRATCH_BYTES (pkv_decode_workspace_size tells beforehand).
 *    32 MiB covers every single-token decode plan up to 8192 (batch x KV head)
 *    items; the chunked multi-token plans of many sequences may need more.
 *  - The stream must belong to the current device (PKV_ERR_INVALID_ARG
 *    otherwise): the array's address is the current device's.
 *  - Every call on one GPU shares that GPU's array and the array keeps the
 *    last call's contents (the decode needs no initial contents).  Calls that
 *    overlap in time on one GPU (other streams, other threads) race on it.
 *  - Otherwise as pkv_decode_gqa.
 */
int pkv_decode_gqa_noalloc(const void *q, int32_t num_q_heads, const pkv_cache_t *cache,
                           const int32_t *block_table, int32_t max_blocks_per_seq,
                           const int32_t *context_lengths, const int32_t *cu_q_lens, int32_t batch,
                           int32_t max_q_len, float scale, void *out, float *lse_out,
                           const pkv_decode_opts_t *opts, void *stream);

/* ------------------------------------------------------------------------- */
/* Paged MLA (latent) cache                                                   */
/* ------------------------------------------------------------------------- */
/*
 * MojoStorePagedMLAKVCache and MojoPagedDecodeMLA (README Op List; the pages
 * give no definition).  Read as multi-head latent attention in its absorbed
 * decode form: each token keeps one latent row c (512 channels) and one
 * rotary-key row r (64 channels), shared by every query head.  Each row is
 * stored as int8 codes with its own per-token scale, as in
 * PKV_QUANT_PER_TOKEN: s = fl32(absmax / 127), code = clamp(rne(fl32(x / s)),
 * -128, 127), 0 when s == 0.
 *
 * Layout (caller-owned, 16-byte aligned; row = block * block_size + slot):
 *   latent        int8  [num_blocks][block_size][512]
 *   rope          int8  [num_blocks][block_size][64]
 *   latent_scale  float [num_blocks][block_size]
 *   rope_scale    float [num_blocks][block_size]
 * Supported: latent_dim 512, rope_dim 64; block_size 16, 32, 64 or 128.
 */
typedef struct {
    void *latent;
    void *rope;
    float *latent_scale;
    float *rope_scale;
    int32_t num_blocks;
    int32_t block_size;
    int32_t latent_dim;  /* 512 */
    int32_t rope_dim;    /* 64 */
} pkv_mla_cache_t;

/*
 * pkv_mla_store_c8 - quantize new tokens' latent rows (bf16 [T][512], 16-byte
 * aligned) and rotary-key rows (bf16 [T][64]) into the MLA cache.  Slots are
 * resolved exactly as in pkv_store_c8: slot_mapping[t] (row index block *
 * block_size + slot; negative = skip), or cu_q_lens / context_lengths /
 * block_table (cu_q_lens NULL: one token per sequence, num_tokens == batch;
 * a sequence with context length 0 stores nothing).  num_tokens == 0 launches
 * nothing.
 */
int pkv_mla_store_c8(const pkv_mla_cache_t *cache, const void *latent_new, const void *rope_new,
                     int32_t num_tokens, const int64_t *slot_mapping, const int32_t *cu_q_lens,
                     const int32_t *context_lengths, const int32_t *block_table, int32_t batch,
                     int32_t max_blocks_per_seq, void *stream);

/* Bytes of workspace pkv_mla_decode needs (0 when it needs none; 0 also for
 * arguments it rejects).  split_tokens: 0 = the library's plan, else keys per
 * split (rounded up to a multiple of 64).  The library's plan, when the
 * (sequence, group of 16 heads) items are at most half the decode workgroups
 * the current device holds at once, is a balanced partition: every 64-key
 * block of every item in one list, cut into about that many near-equal
 * segments (the kernel computes each workgroup's segment from
 * context_lengths, so no host copy of them is needed); otherwise one
 * workgroup per item (or per fixed split).  Depends on the current device's
 * compute-unit count and the kernel's occupancy. */
size_t pkv_mla_decode_workspace_size(int32_t batch, int32_t num_heads, int32_t max_blocks_per_seq,
                                     int32_t block_size, int32_t split_tokens);

/* The split plan pkv_mla_decode would use: keys per split and splits per
 * (sequence, group of 16 heads); for the balanced partition, split_len 0 and
 * num_splits = the workgroups it is planned over.  Either output pointer may
 * be NULL. */
int pkv_mla_decode_plan(int32_t batch, int32_t num_heads, int32_t max_blocks_per_seq,
                        int32_t block_size, int32_t split_tokens, int32_t *split_len,
                        int32_t *num_splits);

/*
 * pkv_mla_decode - latent attention of one new query per sequence over the
 * MLA cache (MojoPagedDecodeMLA, README Op List).
 *
 * q_latent bf16 [batch][num_heads][512] (the query already multiplied into the
 *          latent space), q_rope bf16 [batch][num_heads][64]; both 16-byte
 *          aligned.  Sequence b attends to keys 0 .. context_lengths[b] - 1
 *          (its new token included):
 *   l_t = scale * (q_latent . c^_t + q_rope . r^_t)   (c^, r^ dequantized)
 *   out = sum_t softmax(l)_t c^_t    bf16 [batch][num_heads][512], 16-byte
 *          aligned (the value up-projection that follows is not part of it)
 * lse_out  optional fp32 [batch][num_heads]: natural log of the softmax
 *          denominator; -inf for a sequence with no keys (output 0).
 * workspace: at least pkv_mla_decode_workspace_size(...) bytes with the same
 *          split_tokens, 16-byte aligned, no initial contents needed; calls
 *          that run concurrently must not share it.
 */
int pkv_mla_decode(const void *q_latent, const void *q_rope, int32_t num_heads,
                   const pkv_mla_cache_t *cache, const int32_t *block_table,
                   int32_t max_blocks_per_seq, const int32_t *context_lengths, int32_t batch,
                   float scale, void *out, float *lse_out, void *workspace, size_t workspace_bytes,
                   int32_t split_tokens, void *stream);

/*
 * pkv_mla_store_decode - one MLA decode step in one call: store each
 * sequence's new latent and rotary token, then attend (MojoStorePagedMLAKVCache
 * followed by MojoPagedDecodeMLA, README Op List).
 *
 * The result equals pkv_mla_store_c8(cache, latent_new, rope_new, batch, NULL,
 * NULL, context_lengths, block_table, batch, max_blocks_per_seq) followed by
 * pkv_mla_decode(q_latent, q_rope, ...):
 * latent_new, rope_new  bf16 [batch][512] (16-byte aligned) and [batch][64];
 *               the token of sequence b goes to position context_lengths[b] - 1
 *               (a sequence with context length 0 stores nothing).
 * Other arguments, the workspace and errors as pkv_mla_decode.  With up to 16
 * heads (one head group per sequence) the store happens inside the decode
 * launch: the workgroup whose keys end at the new position quantizes the
 * token, writes it to the cache and uses its codes directly; otherwise a store
 * launch precedes the decode.
 */
int pkv_mla_store_decode(const void *q_latent, const void *q_rope, const void *latent_new,
                         const void *rope_new, int32_t num_heads, const pkv_mla_cache_t *cache,
                         const int32_t *block_table, int32_t max_blocks_per_seq,
                         const int32_t *context_lengths, int32_t batch, float scale, void *out,
                         float *lse_out, void *workspace, size_t workspace_bytes,
                         int32_t split_tokens, void *stream);

/*
 * pkv_mla_cache_walk - a measurement aid: the read ceiling of the MLA decode's
 * access pattern over this cache (not an operation of the pages).
 *
 * One workgroup of four waves per (sequence b, split s of split_tokens keys),
 * the splits of one sequence launched consecutively, reads what the decode of
 * keys [s * split_tokens, min((s + 1) * split_tokens, context_lengths[b]))
 * reads from the cache - their latent and rotary rows and their two scales,
 * with the decode's lane layout and two 64-key blocks in flight per wave - and
 * computes nothing else.  out[b * nsplit + s] receives the wrapping uint32 sum
 * of the 32-bit words of those keys' rows and scales (0 for a split past the
 * context), nsplit = ceil(max_blocks_per_seq * block_size / split_tokens); out
 * holds batch * nsplit entries (device, 4-byte aligned).  split_tokens: a
 * multiple of 64 in [64, 4096].  Errors as pkv_mla_store_c8.
 */
int pkv_mla_cache_walk(const pkv_mla_cache_t *cache, const int32_t *block_table,
                       int32_t max_blocks_per_seq, const int32_t *context_lengths, int32_t batch,
                       int32_t split_tokens, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
