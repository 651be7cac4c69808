// pkv_api.cpp - the C ABI of libpkv (include/pkv.h): argument validation, split planning and
// kernel launches on the caller's stream.  No allocation, no host synchronisation.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kDefaultCUs = 256;  // MI355X, used when no device is visible (planning only)
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = kDefaultCUs;
    g_cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_cache(const pkv_cache_t* c) {
    if (!c || !c->k || !c->v) return PKV_ERR_INVALID_ARG;
    if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
    if (c->head_dim != 64 && c->head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (!pow2(c->block_size) || c->block_size < 16 || c->block_size > 128) return PKV_ERR_UNSUPPORTED;
    if (c->quant_mode < 0 || c->quant_mode > 3) return PKV_ERR_UNSUPPORTED;
    if (c->quant_mode != PKV_QUANT_NONE_BF16 && (!c->k_scale || !c->v_scale)) return PKV_ERR_INVALID_ARG;
    if (!aligned(c->k, 16) || !aligned(c->v, 16)) return PKV_ERR_INVALID_ARG;
    if (c->k_scale && !aligned(c->k_scale, 16)) return PKV_ERR_INVALID_ARG;
    if (c->v_scale && !aligned(c->v_scale, 16)) return PKV_ERR_INVALID_ARG;
    return PKV_OK;
}

constexpr int64_t kMaxSplit = 4096;      // keys per split the decode kernel accepts
constexpr int64_t kMaxSplits = 1 << 16;   // key splits per row group

struct DecodePlan {
    int kernel;        // 1 VALU, 2 MFMA (fp16 / bf16 scores), 3 MFMA (int8 scores, int8 cache only),
                       // 4 tile (128 rows per workgroup, keys shared through LDS)
    int rg;            // VALU: rows per row group (1, 2, 4, 8); MFMA: 16-row tiles per group
    int classes;       // kernel 3: key-subset classes per column tile (1, 2, 4)
    int rows_per_item; // query rows one row group covers
    int prs;           // partial rows stored per (item, split)
    int nrg;
    int nsplit;
    int split_len;
    int sk_waves;      // kernel 3, no forced split: balanced partition over this many waves
    size_t ws_bytes;
};

int pow2_at_least(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

int make_plan(int32_t batch, int32_t hq, int32_t hkv, int32_t head_dim, int32_t mbs, int32_t bs,
              int32_t max_q_len, int32_t mode, const pkv_decode_opts_t* opts, DecodePlan* p) {
    if (batch < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || mbs <= 0) return PKV_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (!pow2(bs) || bs < 16 || bs > 128) return PKV_ERR_UNSUPPORTED;
    if (mode < 0 || mode > 3) return PKV_ERR_UNSUPPORTED;
    if (max_q_len < 1) max_q_len = 1;
    int kernel = mode == 2 ? 2 : 3;  // int8 pages: exact int8 scores; bf16 pages: bf16 scores
    if (opts) {
        for (int i = 0; i < 4; ++i)
            if (opts->reserved[i] != 0) return PKV_ERR_INVALID_ARG;
        if (opts->window < 0) return PKV_ERR_INVALID_ARG;
        if (opts->partition < 0 || opts->partition > 2) return PKV_ERR_INVALID_ARG;
        if (opts->split_tokens < 0) return PKV_ERR_INVALID_ARG;
        if (opts->kernel < 0 || opts->kernel > 4) return PKV_ERR_INVALID_ARG;
        if (opts->kernel != 0) kernel = opts->kernel;
    }
    if (kernel == 3 && mode == 2) kernel = 2;  // the int8-score kernel needs int8 pages
    // prompts (at least one full tile of 128 query rows per KV head, tiles enough to fill the GPU
    // twice): the tile kernel, whose workgroups share each key block among 128 rows (measured on
    // MI355X, 4 prompts of 2048 tokens: 277 against 340 us).  Chunks of fewer rows keep the
    // int8-score kernel, whose key splits balance long contexts (64 chunks of up to 16 tokens over
    // up to 16K keys: 444 against 698 us per step).
    if ((!opts || opts->kernel == 0) && kernel == 3 && (mode == 0 || mode == 1) && head_dim == 128 &&
        !(opts && (opts->window > 0 || opts->split_tokens > 0 || opts->partition != 0))) {
        const int64_t rows_hkv = (int64_t)max_q_len * (hq / hkv);
        const int64_t tiles = (int64_t)batch * hkv * cdiv(rows_hkv, 128);
        if (rows_hkv >= 128 && tiles >= 2LL * device_cus()) kernel = 4;
    }
    if (mode == 3 && kernel != 3) return PKV_ERR_UNSUPPORTED;  // per-channel scales: int8-score kernel only
    const int g = hq / hkv;
    const int64_t rows = (int64_t)max_q_len * g;
    if (rows > (1 << 20)) return PKV_ERR_UNSUPPORTED;
    p->kernel = kernel;
    p->classes = 1;
    if (kernel == 4) {
        // one workgroup per 128-row tile and key split; the partials as two 64-row items per tile
        // for the merge.  No splits where the tiles fill two rounds of the GPU's workgroups (two
        // per CU; prompts: splits would only add partials, and the longest tiles start first),
        // splits of 4096 keys where they do not and a context exceeds 4096 (one round of tiles
        // would wait on its longest: 698 against 443 us on the chunked multi-token decode)
        if (head_dim != 128 || (mode != 0 && mode != 1)) return PKV_ERR_UNSUPPORTED;
        if (opts && (opts->window > 0 || opts->partition != 0)) return PKV_ERR_UNSUPPORTED;
        p->rg = 8;
        p->rows_per_item = 128;
        p->nrg = (int)cdiv(rows, 128);
        p->prs = 64;
        p->sk_waves = 0;
        const int64_t max_ctx = (int64_t)mbs * bs;
        const int64_t tiles = (int64_t)batch * hkv * cdiv(rows, 128);
        int64_t L = opts && opts->split_tokens > 0 ? cdiv(opts->split_tokens, 64) * 64
                                                   : (tiles >= 4LL * device_cus() ? max_ctx : kMaxSplit);
        if (opts && opts->split_tokens > 0 && L > kMaxSplit) L = kMaxSplit;
        if (L >= max_ctx) L = cdiv(max_ctx, 64) * 64;
        if (cdiv(max_ctx, L) > kMaxSplits) return PKV_ERR_UNSUPPORTED;
        p->split_len = (int)L;
        p->nsplit = (int)cdiv(max_ctx, L);
        const int64_t pitems = 2LL * batch * hkv * p->nrg;
        p->ws_bytes = p->nsplit > 1 ? (size_t)(pitems * p->nsplit * 64) * (size_t)(head_dim + 1) * 4 : 0;
        return PKV_OK;
    }
    if (kernel == 3) {
        // columns of a 16-wide tile = (row, key-subset class): 4 classes for up to 4 rows, 2 for
        // up to 8, else one class and one or two 16-row tiles per row group
        if (rows <= 4) {
            p->classes = 4;
            p->rg = 1;
            p->rows_per_item = 4;
        } else if (rows <= 8) {
            p->classes = 2;
            p->rg = 1;
            p->rows_per_item = 8;
        } else {
            // 16-row groups for chunks of decode size (up to 96 rows: the 32-row variant needs
            // more than 256 registers, one wave per SIMD, the 16-row one keeps two; the groups of
            // one (sequence, KV head) run on one XCD at about the same time, so their repeated
            // key reads come from its L2); 32-row groups for prompts, where the matrix-core work
            // per key read dominates (both measured on MI355X)
            p->classes = 1;
            p->rg = rows <= 96 ? 1 : 2;
            p->rows_per_item = 16 * p->rg;
        }
        p->nrg = (int)cdiv(rows, p->rows_per_item);
        p->prs = (int)(rows < p->rows_per_item ? rows : p->rows_per_item);
    } else if (kernel == 1) {
        p->rg = pow2_at_least((int)(rows < 8 ? rows : 8));
        p->rows_per_item = p->rg;
        p->nrg = (int)cdiv(rows, p->rg);
        p->prs = p->rg;
    } else {
        // up to three (head_dim 64) or two (head_dim 128) 16-row tiles per wave, so the wave's
        // accumulators and double-buffered key blocks stay in registers; more rows take several
        // row groups
        const int64_t max_rows = head_dim == 64 ? 48 : 32;
        p->nrg = (int)cdiv(rows, max_rows);
        p->rg = (int)cdiv(cdiv(rows, p->nrg), 16);
        p->rows_per_item = 16 * p->rg;
        p->prs = (int)(rows < p->rows_per_item ? rows : p->rows_per_item);
    }
    // keys one row group can need: the whole table, or with a sliding window of W keys at most
    // W + (max_q_len - 1) (its rows' positions differ by less than max_q_len) + 127 (the range
    // starts 128-aligned)
    int64_t max_ctx = (int64_t)mbs * bs;
    const int window = opts ? opts->window : 0;
    if (window > 0 && (int64_t)window + max_q_len - 1 + 127 < max_ctx) max_ctx = (int64_t)window + max_q_len - 1 + 127;
    const int64_t items = (int64_t)batch * hkv * p->nrg;
    p->sk_waves = 0;
    const int partition = opts ? opts->partition : 0;
    const bool fixed = partition == 1 || (opts && opts->split_tokens > 0);
    if (kernel == 3 && !fixed && items > 0 && (partition == 2 || max_ctx >= 16384)) {
        // balanced partition: every key block of every item in one list, cut into as many equal
        // ranges as the GPU holds waves of the kernel at once (no partly filled rounds of waves).
        // It pays one more memory round trip per wave (the plan), which only long contexts
        // amortise, and needs the items to be few against the waves.
        // one wave per SIMD (four per compute unit) even where two fit: on the long-context decode
        // the segments are then twice as long, their merge half as large, and no wave shares its
        // SIMD (measured on MI355X: 284 against 290 us; three or four per CU are best, two and
        // five slower)
        const int fit = pkv::decode_c8_waves_per_cu(head_dim, p->classes, p->rg, mode, batch, window > 0);
        const int per_cu = fit < 4 ? fit : 4;
        const int64_t W = (int64_t)per_cu * device_cus();
        // more items than half the waves: the library's plan takes fixed splits (measured faster
        // on the chunked multi-token decode: 397 against 483 us); a forced balanced partition
        // takes several rounds of waves, enough that the items are at most half the segments
        const int64_t rounds = W > 0 && items * 2 > W ? cdiv(2 * items, W) : 1;
        if (per_cu > 0 && (rounds == 1 || partition == 2) && W * rounds + items <= (int64_t)0x7fffffff / 2) {
            p->sk_waves = (int)(W * rounds);
            p->split_len = 0;
            p->nsplit = p->sk_waves;
            const size_t slots = (size_t)(p->sk_waves + items) * (size_t)p->prs;
            p->ws_bytes = slots * (size_t)(head_dim + 1) * 4 + (size_t)items * 2 * 4;
            return PKV_OK;
        }
    }
    if (kernel == 2 && mode == 2 && p->rg == 1 && !fixed && items > 0 && (partition == 2 || max_ctx >= 4096)) {
        // bf16 pages: the same balanced partition, over as many rounds of the waves the GPU holds
        // as keep the items at most a third of the segments (sequences of very different lengths
        // otherwise leave most waves idle behind the longest splits; measured on the bf16
        // large-batch decode: 316 us with three rounds, 328 with two, the same with four)
        const int per_cu = pkv::decode_mfma_waves_per_cu(head_dim, p->rg, mode, batch, window > 0);
        if (per_cu > 0) {
            const int64_t W = (int64_t)per_cu * device_cus();
            int64_t rounds = cdiv(3 * items, W);
            if (rounds < 1) rounds = 1;
            if (W * rounds + items <= (int64_t)0x7fffffff / 2) {
                p->sk_waves = (int)(W * rounds);
                p->split_len = 0;
                p->nsplit = p->sk_waves;
                const size_t slots = (size_t)(p->sk_waves + items) * (size_t)p->prs;
                p->ws_bytes = slots * (size_t)(head_dim + 1) * 4 + (size_t)items * 2 * 4;
                return PKV_OK;
            }
        }
    }
    int64_t L;
    if (opts && opts->split_tokens > 0) {
        const int64_t gran = kernel == 3 ? 64 : 128;  // the int8-score kernel walks 64-key blocks
        L = cdiv(opts->split_tokens, gran) * gran;
    } else {
        // Aim for ~16 (int8-score kernel: ~11) workgroups per compute unit counting every
        // (possibly empty) split, with partitions of 256..2048 keys (bf16 matrix-core kernel:
        // ..4096, measured faster on many mid-length sequences: fewer waves than the GPU holds
        // at once instead of a second, partly filled round): long enough to amortise the
        // per-workgroup query load and partial write, short enough to spread a few long
        // sequences over the whole chip.
        const int64_t target = (kernel == 3 ? 11LL : 16LL) * device_cus();
        const int64_t want_splits = items > 0 ? (target + items - 1) / items : 1;
        L = cdiv(cdiv(max_ctx, want_splits), 128) * 128;
        if (L < 256) L = 256;
        const int64_t cap = kernel == 2 ? 4096 : 2048;
        if (L > cap) L = cap;
    }
    if (L > kMaxSplit) L = kMaxSplit;
    if (L >= max_ctx) L = cdiv(max_ctx, 128) * 128;
    if (cdiv(max_ctx, L) > kMaxSplits) return PKV_ERR_UNSUPPORTED;
    p->split_len = (int)L;
    p->nsplit = (int)cdiv(max_ctx, L);
    p->ws_bytes = p->nsplit > 1 ? (size_t)(items * p->nsplit * p->prs) * (size_t)(head_dim + 1) * 4 : 0;
    return PKV_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace

extern "C" {

const char* pkv_status_string(int status) {
    switch (status) {
        case PKV_OK: return "PKV_OK";
        case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG: invalid argument";
        case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED: unsupported shape or mode";
        case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE: workspace missing or too small";
        case PKV_ERR_HIP: return "PKV_ERR_HIP: HIP launch or device query failed";
        default: return "PKV_ERR_UNKNOWN";
    }
}

int pkv_version(void) { return 100; }

int pkv_store_c8(const pkv_cache_t* cache, const void* k_new, const void* v_new, int32_t num_tokens,
                 const int64_t* slot_mapping, const int32_t* cu_q_lens, const int32_t* context_lengths,
                 const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                 int32_t max_q_len, int32_t quant_mode, void* stream) {
    int st = check_cache(cache);
    if (st != PKV_OK) return st;
    if (quant_mode != cache->quant_mode) return PKV_ERR_INVALID_ARG;
    if (num_tokens < 0) return PKV_ERR_INVALID_ARG;
    if (num_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !aligned(k_new, 4) || !aligned(v_new, 4)) return PKV_ERR_INVALID_ARG;
    if (slot_mapping) {
        if (quant_mode == PKV_QUANT_PER_BLOCK) return PKV_ERR_UNSUPPORTED;
    } else {
        if (!context_lengths || !block_table || batch < 0 || max_blocks_per_seq <= 0)
            return PKV_ERR_INVALID_ARG;
        if (!cu_q_lens && num_tokens != batch) return PKV_ERR_INVALID_ARG;
    }
    pkv::StoreArgs a;
    std::memset(&a, 0, sizeof a);
    a.k = cache->k;
    a.v = cache->v;
    a.ks = cache->k_scale;
    a.vs = cache->v_scale;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.slot_mapping = slot_mapping;
    a.cu_q = cu_q_lens;
    a.ctx = context_lengths;
    a.bt = block_table;
    a.num_tokens = num_tokens;
    a.hkv = cache->num_kv_heads;
    a.bs = cache->block_size;
    a.log2bs = ilog2(cache->block_size);
    a.mbs = max_blocks_per_seq;
    a.batch = batch;
    int q = cu_q_lens ? (max_q_len > 0 ? max_q_len : num_tokens) : 1;
    a.nbt = (int)((q + cache->block_size - 2) / cache->block_size + 1);
    if (a.nbt > max_blocks_per_seq && !slot_mapping) a.nbt = max_blocks_per_seq;
    // chunks of more than one token per sequence are stored by 16-slot tiles (q tokens from any
    // position touch at most (q + 14) / 16 + 1 tiles); single tokens by the per-token kernel
    a.ntile = (cu_q_lens && !slot_mapping && q > 1) ? (int)((q + 14) / 16 + 1) : 0;
    if (a.ntile > max_blocks_per_seq * (cache->block_size / 16)) a.ntile = max_blocks_per_seq * (cache->block_size / 16);
    return hip_status(pkv::launch_store(a, cache->head_dim, quant_mode, static_cast<hipStream_t>(stream)));
}

int pkv_dequant(const pkv_cache_t* cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                const int32_t* context_lengths, const int64_t* seq_offsets, int32_t batch, void* k_out,
                void* v_out, int64_t token_stride, int64_t head_stride, void* stream) {
    int st = check_cache(cache);
    if (st != PKV_OK) return st;
    if (!block_table || !context_lengths || batch < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
    if (!k_out && !v_out) return PKV_ERR_INVALID_ARG;
    if (token_stride <= 0 || head_stride <= 0) return PKV_ERR_INVALID_ARG;
    if ((k_out && !aligned(k_out, 2)) || (v_out && !aligned(v_out, 2))) return PKV_ERR_INVALID_ARG;
    if (batch == 0) return PKV_OK;
    pkv::DequantArgs a;
    std::memset(&a, 0, sizeof a);
    a.k = cache->k;
    a.v = cache->v;
    a.ks = cache->k_scale;
    a.vs = cache->v_scale;
    a.bt = block_table;
    a.ctx = context_lengths;
    a.seq_off = seq_offsets;
    a.k_out = static_cast<uint16_t*>(k_out);
    a.v_out = static_cast<uint16_t*>(v_out);
    a.token_stride = token_stride;
    a.head_stride = head_stride;
    a.hkv = cache->num_kv_heads;
    a.bs = cache->block_size;
    a.log2bs = ilog2(cache->block_size);
    a.mbs = max_blocks_per_seq;
    a.batch = batch;
    a.vec_ok = (token_stride % 8 == 0) && (head_stride % 8 == 0) && (!k_out || aligned(k_out, 16)) &&
               (!v_out || aligned(v_out, 16));
    a.nchunk = (int)cdiv((int64_t)max_blocks_per_seq * cache->block_size, 128);
    return hip_status(pkv::launch_dequant(a, cache->head_dim, cache->quant_mode, static_cast<hipStream_t>(stream)));
}

int pkv_cache_walk(const pkv_cache_t* cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                   const int32_t* context_lengths, int32_t batch, int32_t split_tokens, int32_t depth,
                   uint32_t* out, void* stream) {
    int st = check_cache(cache);
    if (st != PKV_OK) return st;
    if (cache->quant_mode == PKV_QUANT_NONE_BF16) return PKV_ERR_UNSUPPORTED;
    if (!block_table || !context_lengths || !out || batch < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
    if (split_tokens < 64 || split_tokens > 4096 || split_tokens % 64 != 0) return PKV_ERR_INVALID_ARG;
    if (depth < 1 || depth > 3 || !aligned(out, 4)) return PKV_ERR_INVALID_ARG;
    if (batch == 0) return PKV_OK;
    pkv::WalkArgs a;
    std::memset(&a, 0, sizeof a);
    a.k = cache->k;
    a.v = cache->v;
    a.ks = cache->k_scale;
    a.vs = cache->v_scale;
    a.bt = block_table;
    a.ctx = context_lengths;
    a.out = out;
    a.hkv = cache->num_kv_heads;
    a.bs = cache->block_size;
    a.log2bs = ilog2(cache->block_size);
    a.mbs = max_blocks_per_seq;
    a.split_len = split_tokens;
    a.nsplit = (int)cdiv((int64_t)max_blocks_per_seq * cache->block_size, split_tokens);
    return hip_status(pkv::launch_walk(a, batch, cache->head_dim, cache->quant_mode, depth,
                                       static_cast<hipStream_t>(stream)));
}

int pkv_check_indices(int32_t num_blocks, int32_t block_size, const int32_t* block_table,
                      int32_t max_blocks_per_seq, const int32_t* context_lengths, const int32_t* cu_q_lens,
                      int32_t max_q_len, int32_t batch, const int64_t* slot_mapping, int32_t num_tokens,
                      int32_t* result, void* stream) {
    if (!result || !aligned(result, 4)) return PKV_ERR_INVALID_ARG;
    if (num_blocks < 0 || block_size <= 0 || batch < 0 || num_tokens < 0) return PKV_ERR_INVALID_ARG;
    if (block_table && (!context_lengths || max_blocks_per_seq <= 0)) return PKV_ERR_INVALID_ARG;
    if (context_lengths && max_blocks_per_seq < 0) return PKV_ERR_INVALID_ARG;
    if (batch > 0 && !context_lengths && !cu_q_lens && !slot_mapping) return PKV_ERR_INVALID_ARG;
    if (num_tokens > 0 && !slot_mapping) return PKV_ERR_INVALID_ARG;
    pkv::CheckArgs a;
    std::memset(&a, 0, sizeof a);
    a.bt = block_table;
    a.ctx = context_lengths;
    a.cu = cu_q_lens;
    a.slot = slot_mapping;
    a.result = result;
    a.num_blocks = num_blocks;
    a.bs = block_size;
    a.mbs = max_blocks_per_seq;
    a.batch = batch;
    a.max_q_len = max_q_len;
    a.num_tokens = slot_mapping ? num_tokens : 0;
    return hip_status(pkv::launch_check(a, static_cast<hipStream_t>(stream)));
}

size_t pkv_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t max_q_len, int32_t quant_mode, const pkv_decode_opts_t* opts) {
    DecodePlan p;
    if (make_plan(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size, max_q_len,
                  quant_mode, opts, &p) != PKV_OK)
        return 0;
    return p.ws_bytes;
}

int pkv_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t max_blocks_per_seq, int32_t block_size, int32_t max_q_len, int32_t quant_mode,
                    const pkv_decode_opts_t* opts, int32_t* split_tokens, int32_t* num_splits,
                    int32_t* kernel) {
    DecodePlan p;
    int st = make_plan(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
                       max_q_len, quant_mode, opts, &p);
    if (st != PKV_OK) return st;
    if (split_tokens) *split_tokens = p.split_len;
    if (num_splits) *num_splits = p.nsplit;
    if (kernel) *kernel = p.kernel;
    return PKV_OK;
}

}  // extern "C"

namespace {

// pkv_decode_gqa, and with k_new / v_new (one decode step's new tokens, cu_q_lens NULL) the store
// of those tokens first: fused into the int8-score decode where it serves the call (per-token and
// per-channel caches, one row group per KV head), else a store launch before the decode.  Every
// argument is checked before anything is launched.
int decode_impl(const void* q, int32_t num_q_heads, const pkv_cache_t* cache, const int32_t* block_table,
                int32_t max_blocks_per_seq, const int32_t* context_lengths, const int32_t* cu_q_lens,
                int32_t batch, int32_t max_q_len, float scale, void* out, float* lse_out,
                void* workspace, size_t workspace_bytes, const pkv_decode_opts_t* opts, void* stream,
                const void* k_new, const void* v_new) {
    int st = check_cache(cache);
    if (st != PKV_OK) return st;
    if (!q || !out || !block_table || !context_lengths) return PKV_ERR_INVALID_ARG;
    if (k_new || v_new) {
        if (!k_new || !v_new || cu_q_lens || !aligned(k_new, 4) || !aligned(v_new, 4)) return PKV_ERR_INVALID_ARG;
        if (batch < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
    }
    if (!aligned(q, 16) || !aligned(out, 2) || (lse_out && !aligned(lse_out, 4))) return PKV_ERR_INVALID_ARG;
    if (!cu_q_lens) max_q_len = 1;
    if (max_q_len < 1) return PKV_ERR_INVALID_ARG;
    DecodePlan p;
    st = make_plan(batch, num_q_heads, cache->num_kv_heads, cache->head_dim, max_blocks_per_seq,
                   cache->block_size, max_q_len, cache->quant_mode, opts, &p);
    if (st != PKV_OK) return st;
    if (batch == 0) return PKV_OK;
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 16)))
        return PKV_ERR_WORKSPACE;
    pkv::DecodeArgs a;
    std::memset(&a, 0, sizeof a);
    a.q = static_cast<const uint16_t*>(q);
    a.k = cache->k;
    a.v = cache->v;
    a.ks = cache->k_scale;
    a.vs = cache->v_scale;
    a.bt = block_table;
    a.ctx = context_lengths;
    a.cu = cu_q_lens;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse_out;
    a.hq = num_q_heads;
    a.hkv = cache->num_kv_heads;
    a.g = num_q_heads / cache->num_kv_heads;
    a.bs = cache->block_size;
    a.log2bs = ilog2(cache->block_size);
    a.mbs = max_blocks_per_seq;
    a.nrg = p.nrg;
    a.nsplit = p.nsplit;
    a.split_len = p.split_len;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.window = opts ? opts->window : 0;
    const int64_t items = (int64_t)batch * a.hkv * p.nrg;
    if (p.sk_waves > 0) {
        float* ws = static_cast<float*>(workspace);
        const int64_t slots = (p.sk_waves + items) * p.prs;
        a.part_o = ws;
        a.part_lse = ws + slots * cache->head_dim;
        a.seg = reinterpret_cast<int32_t*>(a.part_lse + slots);
        a.sk_waves = p.sk_waves;
    } else if (p.nsplit > 1) {
        float* ws = static_cast<float*>(workspace);
        const int64_t pitems = p.kernel == 4 ? 2 * items : items;  // the tile kernel: two 64-row items per tile
        a.part_o = ws;
        a.part_lse = ws + pitems * p.nsplit * p.prs * cache->head_dim;
    }
    a.prs = p.prs;
    hipStream_t st_ = static_cast<hipStream_t>(stream);
    if (k_new) {
        const bool fused = p.kernel == 3 && p.nrg == 1 &&
                           (cache->quant_mode == PKV_QUANT_PER_TOKEN || cache->quant_mode == PKV_QUANT_PER_CHANNEL);
        if (fused) {
            a.k_new = static_cast<const uint16_t*>(k_new);
            a.v_new = static_cast<const uint16_t*>(v_new);
        } else {
            pkv::StoreArgs sa;
            std::memset(&sa, 0, sizeof sa);
            sa.k = cache->k;
            sa.v = cache->v;
            sa.ks = cache->k_scale;
            sa.vs = cache->v_scale;
            sa.k_new = static_cast<const uint16_t*>(k_new);
            sa.v_new = static_cast<const uint16_t*>(v_new);
            sa.ctx = context_lengths;
            sa.bt = block_table;
            sa.num_tokens = batch;
            sa.hkv = cache->num_kv_heads;
            sa.bs = cache->block_size;
            sa.log2bs = ilog2(cache->block_size);
            sa.mbs = max_blocks_per_seq;
            sa.batch = batch;
            sa.nbt = 1;
            const hipError_t e = pkv::launch_store(sa, cache->head_dim, cache->quant_mode, st_);
            if (e != hipSuccess) return PKV_ERR_HIP;
        }
    }
    if (p.kernel == 1)
        return hip_status(pkv::launch_decode_valu(a, batch, cache->head_dim, p.rg, cache->quant_mode, st_));
    if (p.kernel == 4)
        return hip_status(pkv::launch_decode_tile(a, batch, cache->head_dim, cache->quant_mode, st_));
    if (p.kernel == 3)
        return hip_status(
            pkv::launch_decode_c8(a, batch, cache->head_dim, p.classes, p.rg, cache->quant_mode, st_));
    return hip_status(pkv::launch_decode_mfma(a, batch, cache->head_dim, p.rg, cache->quant_mode, st_));
}

}  // namespace

extern "C" {

int pkv_decode_gqa(const void* q, int32_t num_q_heads, const pkv_cache_t* cache, const int32_t* block_table,
                   int32_t max_blocks_per_seq, const int32_t* context_lengths, const int32_t* cu_q_lens,
                   int32_t batch, int32_t max_q_len, float scale, void* out, float* lse_out,
                   void* workspace, size_t workspace_bytes, const pkv_decode_opts_t* opts, void* stream) {
    return decode_impl(q, num_q_heads, cache, block_table, max_blocks_per_seq, context_lengths, cu_q_lens, batch,
                       max_q_len, scale, out, lse_out, workspace, workspace_bytes, opts, stream, nullptr, nullptr);
}

int pkv_store_decode_gqa(const void* q, const void* k_new, const void* v_new, int32_t num_q_heads,
                         const pkv_cache_t* cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* context_lengths, int32_t batch, float scale, void* out, float* lse_out,
                         void* workspace, size_t workspace_bytes, const pkv_decode_opts_t* opts, void* stream) {
    if (!k_new || !v_new) return PKV_ERR_INVALID_ARG;
    return decode_impl(q, num_q_heads, cache, block_table, max_blocks_per_seq, context_lengths, nullptr, batch, 1,
                       scale, out, lse_out, workspace, workspace_bytes, opts, stream, k_new, v_new);
}

}  // extern "C"
