// mla_api.cpp - the C ABI of the paged MLA (latent cache) entry points of libpkv (include/pkv.h):
// argument validation, split planning and launches on the caller's stream.  No allocation, no
// host synchronisation.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/pkv.h"
#include "mla_internal.h"

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

std::atomic<int> g_mla_wgs[kMaxDevices];

// Decode workgroups one compute unit of the current device holds at once (cached per device).
int mla_wgs_per_cu() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = g_mla_wgs[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    n = pkv::mla_decode_wgs_per_cu();
    if (n > 0) g_mla_wgs[dev].store(n, std::memory_order_relaxed);
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

int check_mla_cache(const pkv_mla_cache_t* c) {
    if (!c || !c->latent || !c->rope || !c->latent_scale || !c->rope_scale) return PKV_ERR_INVALID_ARG;
    if (c->num_blocks <= 0) return PKV_ERR_INVALID_ARG;
    if (c->latent_dim != pkv::kMlaLatent || c->rope_dim != pkv::kMlaRope) return PKV_ERR_UNSUPPORTED;
    if (!pow2(c->block_size) || c->block_size < 16 || c->block_size > 128) return PKV_ERR_UNSUPPORTED;
    if (!aligned(c->latent, 16) || !aligned(c->rope, 16) || !aligned(c->latent_scale, 16) ||
        !aligned(c->rope_scale, 16))
        return PKV_ERR_INVALID_ARG;
    return PKV_OK;
}

constexpr int64_t kMlaBlock = 64;        // keys per block of the decode kernel
constexpr int64_t kMaxSplits = 1 << 16;  // key splits per (sequence, head group)
// workspace bytes per partial row (one head of one split): 512 fp16 channels, then (after all
// rows) its log-sum-exp and latent scale
constexpr size_t kPartRowBytes = pkv::kMlaLatent * 2 + 2 * 4;

struct MlaPlan {
    int nhg;
    int nsplit;
    int split_len;
    int sk_wgs;  // > 0: balanced partition over this many workgroups
    size_t ws_bytes;
};

int mla_plan(int32_t batch, int32_t heads, int32_t mbs, int32_t bs, int32_t split_tokens, MlaPlan* p) {
    if (batch < 0 || heads <= 0 || mbs <= 0 || split_tokens < 0) return PKV_ERR_INVALID_ARG;
    if (!pow2(bs) || bs < 16 || bs > 128) return PKV_ERR_UNSUPPORTED;
    p->nhg = (int)cdiv(heads, pkv::kMlaHeads);
    const int64_t items = (int64_t)batch * p->nhg;
    const int64_t max_ctx = (int64_t)mbs * bs;
    p->sk_wgs = 0;
    if (split_tokens == 0 && items > 0) {
        // balanced partition: all key blocks of all items cut into as many near-equal segments as
        // the GPU holds workgroups at once (one round, no partly filled second round); only when
        // the items are few against those workgroups, else one workgroup per item needs no merge
        const int per_cu = mla_wgs_per_cu();
        const int64_t W = (int64_t)per_cu * device_cus();
        if (per_cu > 0 && items * 2 <= W && max_ctx > kMlaBlock) {
            p->sk_wgs = (int)W;
            p->split_len = 0;
            p->nsplit = (int)W;
            const size_t slots = (size_t)(W + items);
            p->ws_bytes = slots * pkv::kMlaHeads * kPartRowBytes + (size_t)items * 2 * 4;
            return PKV_OK;
        }
    }
    int64_t L;
    if (split_tokens > 0) {
        L = cdiv(split_tokens, kMlaBlock) * kMlaBlock;
    } else {
        // about four workgroups per compute unit counting every (possibly empty) split, with
        // splits of 256 .. 8192 keys: a split's partial output (16 heads x 512 fp16, written and
        // read back) costs as much HBM traffic as ~56 of its keys, so splits stay long
        const int64_t target = 4LL * device_cus();
        const int64_t want = items > 0 ? cdiv(target, items) : 1;
        L = cdiv(cdiv(max_ctx, want), kMlaBlock) * kMlaBlock;
        if (L < 256) L = 256;
        if (L > 8192) L = 8192;
    }
    if (L >= max_ctx) L = cdiv(max_ctx, kMlaBlock) * kMlaBlock;
    if (cdiv(max_ctx, L) > kMaxSplits) return PKV_ERR_UNSUPPORTED;
    p->split_len = (int)L;
    p->nsplit = (int)cdiv(max_ctx, L);
    p->ws_bytes = p->nsplit > 1 ? (size_t)(items * p->nsplit) * pkv::kMlaHeads * kPartRowBytes : 0;
    return PKV_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// The decode, and with latent_new / rope_new (bf16 [batch][512] / [batch][64]) one decode step: each
// sequence's new token stored at position context_lengths[b] - 1 first.  With one head group per
// sequence the decode launch stores it (the workgroup whose keys end there); otherwise a store
// launch precedes the decode.
int mla_decode_impl(const void* q_latent, const void* q_rope, const void* latent_new, const void* rope_new,
                    int32_t num_heads, const pkv_mla_cache_t* cache, const int32_t* block_table,
                    int32_t max_blocks_per_seq, const int32_t* context_lengths, int32_t batch, float scale,
                    void* out, float* lse_out, void* workspace, size_t workspace_bytes, int32_t split_tokens,
                    void* stream) {
    int st = check_mla_cache(cache);
    if (st != PKV_OK) return st;
    if (!q_latent || !q_rope || !out || !block_table || !context_lengths) return PKV_ERR_INVALID_ARG;
    if (!aligned(q_latent, 16) || !aligned(q_rope, 16) || !aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
        return PKV_ERR_INVALID_ARG;
    if (latent_new && (!aligned(latent_new, 16) || !aligned(rope_new, 2))) return PKV_ERR_INVALID_ARG;
    MlaPlan p;
    st = mla_plan(batch, num_heads, max_blocks_per_seq, cache->block_size, split_tokens, &p);
    if (st != PKV_OK) return st;
    if (batch == 0) return PKV_OK;
    if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes || !aligned(workspace, 16)))
        return PKV_ERR_WORKSPACE;
    pkv::MlaArgs a;
    std::memset(&a, 0, sizeof a);
    a.latent = static_cast<int8_t*>(cache->latent);
    a.rope = static_cast<int8_t*>(cache->rope);
    a.ls = cache->latent_scale;
    a.rs = cache->rope_scale;
    a.ql = static_cast<const uint16_t*>(q_latent);
    a.qr = static_cast<const uint16_t*>(q_rope);
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse_out;
    a.bt = block_table;
    a.ctx = context_lengths;
    a.batch = batch;
    a.heads = num_heads;
    a.nhg = p.nhg;
    a.bs = cache->block_size;
    a.log2bs = ilog2(cache->block_size);
    a.mbs = max_blocks_per_seq;
    a.nsplit = p.nsplit;
    a.split_len = p.split_len;
    a.sk_wgs = p.sk_wgs;
    a.scale_log2 = scale * 1.4426950408889634f;
    if (p.sk_wgs > 0) {
        uint16_t* ws = static_cast<uint16_t*>(workspace);
        const int64_t rows = ((int64_t)p.sk_wgs + (int64_t)batch * p.nhg) * pkv::kMlaHeads;
        a.part_o = ws;
        a.part_lse = reinterpret_cast<float*>(ws + rows * pkv::kMlaLatent);
        a.seg = reinterpret_cast<int*>(a.part_lse + 2 * rows);
    } else if (p.nsplit > 1) {
        uint16_t* ws = static_cast<uint16_t*>(workspace);
        const int64_t rows = (int64_t)batch * p.nhg * p.nsplit * pkv::kMlaHeads;
        a.part_o = ws;
        a.part_lse = reinterpret_cast<float*>(ws + rows * pkv::kMlaLatent);
    }
    if (latent_new) {
        a.latent_new = static_cast<const uint16_t*>(latent_new);
        a.rope_new = static_cast<const uint16_t*>(rope_new);
        if (p.nhg == 1) {
            a.fuse_store = 1;
        } else {  // several head groups read the new key: store it first
            a.num_tokens = batch;
            const hipError_t e = pkv::launch_mla_store(a, static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return PKV_ERR_HIP;
        }
    }
    return hip_status(pkv::launch_mla_decode(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int pkv_mla_store_c8(const pkv_mla_cache_t* cache, const void* latent_new, const void* rope_new,
                     int32_t num_tokens, const int64_t* slot_mapping, const int32_t* cu_q_lens,
                     const int32_t* context_lengths, const int32_t* block_table, int32_t batch,
                     int32_t max_blocks_per_seq, void* stream) {
    int st = check_mla_cache(cache);
    if (st != PKV_OK) return st;
    if (num_tokens < 0) return PKV_ERR_INVALID_ARG;
    if (num_tokens == 0) return PKV_OK;
    if (!latent_new || !rope_new || !aligned(latent_new, 16) || !aligned(rope_new, 2)) return PKV_ERR_INVALID_ARG;
    if (!slot_mapping) {
        if (!context_lengths || !block_table || batch < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
        if (!cu_q_lens && num_tokens != batch) return PKV_ERR_INVALID_ARG;
    }
    pkv::MlaArgs a;
    std::memset(&a, 0, sizeof a);
    a.latent = static_cast<int8_t*>(cache->latent);
    a.rope = static_cast<int8_t*>(cache->rope);
    a.ls = cache->latent_scale;
    a.rs = cache->rope_scale;
    a.latent_new = static_cast<const uint16_t*>(latent_new);
    a.rope_new = static_cast<const uint16_t*>(rope_new);
    a.slot_mapping = slot_mapping;
    a.cu_q = cu_q_lens;
    a.ctx = context_lengths;
    a.bt = block_table;
    a.num_tokens = num_tokens;
    a.batch = batch;
    a.bs = cache->block_size;
    a.log2bs = ilog2(cache->block_size);
    a.mbs = max_blocks_per_seq;
    return hip_status(pkv::launch_mla_store(a, static_cast<hipStream_t>(stream)));
}

size_t pkv_mla_decode_workspace_size(int32_t batch, int32_t num_heads, int32_t max_blocks_per_seq,
                                     int32_t block_size, int32_t split_tokens) {
    MlaPlan p;
    if (mla_plan(batch, num_heads, max_blocks_per_seq, block_size, split_tokens, &p) != PKV_OK) return 0;
    return p.ws_bytes;
}

int pkv_mla_decode_plan(int32_t batch, int32_t num_heads, int32_t max_blocks_per_seq, int32_t block_size,
                        int32_t split_tokens, int32_t* split_len, int32_t* num_splits) {
    MlaPlan p;
    int st = mla_plan(batch, num_heads, max_blocks_per_seq, block_size, split_tokens, &p);
    if (st != PKV_OK) return st;
    if (split_len) *split_len = p.split_len;
    if (num_splits) *num_splits = p.nsplit;
    return PKV_OK;
}

int pkv_mla_decode(const void* q_latent, const void* q_rope, int32_t num_heads, const pkv_mla_cache_t* cache,
                   const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lengths,
                   int32_t batch, float scale, void* out, float* lse_out, void* workspace,
                   size_t workspace_bytes, int32_t split_tokens, void* stream) {
    return mla_decode_impl(q_latent, q_rope, nullptr, nullptr, num_heads, cache, block_table, max_blocks_per_seq,
                           context_lengths, batch, scale, out, lse_out, workspace, workspace_bytes, split_tokens,
                           stream);
}

int pkv_mla_store_decode(const void* q_latent, const void* q_rope, const void* latent_new, const void* rope_new,
                         int32_t num_heads, const pkv_mla_cache_t* cache, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* context_lengths, int32_t batch, float scale,
                         void* out, float* lse_out, void* workspace, size_t workspace_bytes, int32_t split_tokens,
                         void* stream) {
    if (!latent_new || !rope_new) return PKV_ERR_INVALID_ARG;
    return mla_decode_impl(q_latent, q_rope, latent_new, rope_new, num_heads, cache, block_table, max_blocks_per_seq,
                           context_lengths, batch, scale, out, lse_out, workspace, workspace_bytes, split_tokens,
                           stream);
}

int pkv_mla_cache_walk(const pkv_mla_cache_t* cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* context_lengths, int32_t batch, int32_t split_tokens, uint32_t* out,
                       void* stream) {
    int st = check_mla_cache(cache);
    if (st != PKV_OK) return st;
    if (!block_table || !context_lengths || !out || batch < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
    if (split_tokens < 64 || split_tokens > 4096 || split_tokens % 64 != 0 || !aligned(out, 4))
        return PKV_ERR_INVALID_ARG;
    if (batch == 0) return PKV_OK;
    pkv::MlaWalkArgs a;
    std::memset(&a, 0, sizeof a);
    a.latent = static_cast<const int8_t*>(cache->latent);
    a.rope = static_cast<const int8_t*>(cache->rope);
    a.ls = cache->latent_scale;
    a.rs = cache->rope_scale;
    a.bt = block_table;
    a.ctx = context_lengths;
    a.out = out;
    a.bs = cache->block_size;
    a.log2bs = ilog2(cache->block_size);
    a.mbs = max_blocks_per_seq;
    a.split_len = split_tokens;
    a.nsplit = (int)cdiv((int64_t)max_blocks_per_seq * cache->block_size, split_tokens);
    return hip_status(pkv::launch_mla_walk(a, batch, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
