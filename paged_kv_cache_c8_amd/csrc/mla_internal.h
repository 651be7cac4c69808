// mla_internal.h - argument block and launchers of the paged MLA (latent cache) kernels, shared
// between the C-ABI layer (mla_api.cpp) and mla.hip.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kMlaLatent = 512;  // latent channels of a token row
constexpr int kMlaRope = 64;     // rotary-key channels of a token row
constexpr int kMlaHeads = 16;    // query heads per work item (one 16-column matrix tile)

struct MlaArgs {
    // cache: latent [NB][BS][512] and rope [NB][BS][64] int8, one fp32 scale per token for each
    int8_t* latent;
    int8_t* rope;
    float* ls;
    float* rs;
    // store
    const uint16_t* latent_new;  // bf16 [T][512]
    const uint16_t* rope_new;    // bf16 [T][64]
    const int64_t* slot_mapping;
    const int32_t* cu_q;
    int num_tokens;
    // decode
    const uint16_t* ql;  // bf16 [B][H][512]
    const uint16_t* qr;  // bf16 [B][H][64]
    uint16_t* out;       // bf16 [B][H][512]
    float* lse;          // [B][H] or null
    uint16_t* part_o;    // fp16, in latent-code units: fixed splits [nsplit][items][16][512];
                         // balanced: [slots][16][512]
    float* part_lse;     // per row of part_o: its base-2 log-sum-exp and its latent scale
    int* seg;            // balanced partition: per item, its first partial slot and segment count
    // both
    const int32_t* bt;
    const int32_t* ctx;
    int batch;
    int heads;
    int nhg;  // head groups of 16 per sequence
    int bs;
    int log2bs;
    int mbs;
    int nsplit;
    int split_len;     // keys per split, a multiple of 64
    int sk_wgs;        // > 0: balanced partition over this many workgroups (split_len unused)
    float scale_log2;  // softmax scale * log2(e)
    int fuse_store;    // decode: also store latent_new / rope_new row b at position ctx[b] - 1 (nhg == 1)
};

// The MLA decode's cache reads alone (pkv_mla_cache_walk): one workgroup of four waves per
// (sequence, split of split_len keys); out[b * nsplit + s] gets the wrapping sum of the 32-bit
// words of the keys' latent rows, rotary rows and scales.
struct MlaWalkArgs {
    const int8_t* latent;
    const int8_t* rope;
    const float* ls;
    const float* rs;
    const int32_t* bt;
    const int32_t* ctx;
    uint32_t* out;
    int bs;
    int log2bs;
    int mbs;
    int split_len;  // a multiple of 64, at most 4096
    int nsplit;
};

// Workgroups of the decode kernel one compute unit holds at once (0 if unknown).
int mla_decode_wgs_per_cu();

hipError_t launch_mla_store(const MlaArgs& a, hipStream_t stream);
hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t stream);
hipError_t launch_mla_walk(const MlaWalkArgs& a, int batch, hipStream_t stream);

}  // namespace pkv
