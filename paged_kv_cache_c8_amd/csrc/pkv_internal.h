// pkv_internal.h - argument blocks and kernel launchers shared between the C-ABI layer
// (pkv_api.cpp) and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct StoreArgs {
    void* k;
    void* v;
    float* ks;
    float* vs;
    const uint16_t* k_new;
    const uint16_t* v_new;
    const int64_t* slot_mapping;
    const int32_t* cu_q;
    const int32_t* ctx;
    const int32_t* bt;
    int num_tokens;
    int hkv;
    int bs;
    int log2bs;
    int mbs;
    int batch;
    int nbt;    // blocks a sequence's new tokens can touch (per-block launch)
    int ntile;  // 16-slot tiles a sequence's new tokens can touch (tile launch; 0: per-token kernel)
};

struct DequantArgs {
    const void* k;
    const void* v;
    const float* ks;
    const float* vs;
    const int32_t* bt;
    const int32_t* ctx;
    const int64_t* seq_off;
    uint16_t* k_out;
    uint16_t* v_out;
    int64_t token_stride;
    int64_t head_stride;
    int hkv;
    int bs;
    int log2bs;
    int mbs;
    int batch;
    int vec_ok;  // outputs and strides allow 16-byte stores
    int nchunk;  // 128-position chunks of the longest sequence the block table holds
};

struct WalkArgs {
    const void* k;
    const void* v;
    const float* ks;
    const float* vs;
    const int32_t* bt;
    const int32_t* ctx;
    uint32_t* out;
    int hkv;
    int bs;
    int log2bs;
    int mbs;
    int split_len;
    int nsplit;
};

struct DecodeArgs {
    const uint16_t* q;
    const void* k;
    const void* v;
    const float* ks;
    const float* vs;
    const int32_t* bt;
    const int32_t* ctx;
    const int32_t* cu;
    uint16_t* out;
    float* lse;
    float* part_o;    // [items][nsplit][RG][D]
    float* part_lse;  // [items][nsplit][RG]  (base-2 log-sum-exp)
    int hq;
    int hkv;
    int g;
    int bs;
    int log2bs;
    int mbs;
    int nrg;
    int nsplit;
    int split_len;
    int prs;           // partial rows per (item, split) in part_o / part_lse
    float scale_log2;  // softmax scale * log2(e)
    int sk_waves;      // > 0: balanced partition into about this many segments (waves)
    int32_t* seg;      // balanced partition: first / last wave of each item [items][2]
    int window;        // > 0: sliding window, a query sees only its last `window` keys
    // one decode step's new tokens (bf16 [batch][hkv][D], position ctx - 1 of each sequence), stored
    // by the decode itself (int8-score kernel, one query per sequence); nullptr: nothing to store
    const uint16_t* k_new;
    const uint16_t* v_new;
};

// Sliding window: the first key a query at position pos sees (key 0 without a window).
__host__ __device__ inline int win_lo(int window, int pos) {
    return window > 0 && pos + 1 > window ? pos + 1 - window : 0;
}
// First key of the key range of a row group whose first row sits at position pos, aligned down to
// 128 keys (a multiple of every kernel's block and of every split length).
__host__ __device__ inline int win_begin(int window, int pos) { return win_lo(window, pos) & ~127; }

hipError_t launch_store(const StoreArgs& a, int head_dim, int mode, hipStream_t stream);
hipError_t launch_dequant(const DequantArgs& a, int head_dim, int mode, hipStream_t stream);
hipError_t launch_walk(const WalkArgs& a, int batch, int head_dim, int mode, int depth, hipStream_t stream);

// pkv_check_indices (check.hip): the arrays to check (NULL: not checked) and the sizes that bound them
struct CheckArgs {
    const int32_t* bt;
    const int32_t* ctx;
    const int32_t* cu;
    const int64_t* slot;
    int32_t* result;
    int num_blocks;
    int bs;
    int mbs;
    int batch;
    int max_q_len;
    int num_tokens;
};
// result bits (the same values as pkv.h's PKV_CHECK_*)
constexpr int kCheckContext = 1, kCheckBlock = 2, kCheckQlen = 4, kCheckSlot = 8;
hipError_t launch_check(const CheckArgs& a, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeArgs& a, int batch, int head_dim, int rg, int mode,
                              hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs& a, int batch, int head_dim, int row_tiles, int mode,
                              hipStream_t stream);
// int8 cache (modes 0, 1): classes = subset classes per column tile (1, 2, 4), row_tiles = 1 or 2
hipError_t launch_decode_c8(const DecodeArgs& a, int batch, int head_dim, int classes, int row_tiles,
                            int mode, hipStream_t stream);
// Many query rows per KV head (prompts, multi-token chunks): one workgroup per 128-row tile (and key
// split, where tiles are few), key blocks shared through LDS (decode_tile.hip); head_dim 128, int8
// modes 0 and 1, no window.
hipError_t launch_decode_tile(const DecodeArgs& a, int batch, int head_dim, int mode, hipStream_t stream);
// resident waves per compute unit of the balanced-partition kernel (0: not available)
int decode_c8_waves_per_cu(int head_dim, int classes, int row_tiles, int mode, int batch, bool windowed);
// Waves of the balanced bf16 matrix-core decode one compute unit holds (0: not available for
// these arguments).
int decode_mfma_waves_per_cu(int head_dim, int row_tiles, int mode, int batch, bool windowed);
// log-sum-exp merge of the split partials; rows_per_item = query rows of one row group
hipError_t launch_merge(const DecodeArgs& a, int batch, int head_dim, int rows_per_item, hipStream_t stream);

}  // namespace pkv
