// noalloc.hip - pkv_decode_gqa_noalloc: the grouped-query decode with its split partials in a
// fixed device array of the library instead of a caller workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
//
// `scratch` is a file-scope device array of PKV_NOALLOC_SCRATCH_BYTES.  Each GPU the library runs
// on holds its own copy at its own address until the process ends.  On the first call on a device
// (with that device current) its address is taken with hipGetSymbolAddress and kept per device;
// host code uses only that address, never the array's name (which on the host is a stand-in, not
// a device address).  The decode kernels need no initial contents in their workspace, so nothing
// is cleared.  Every call on one GPU shares that GPU's array: calls that overlap in time on one
// GPU (different streams, different threads) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/pkv.h"

namespace {

constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_init;

// Device address of `scratch` on the current device (taken once per device).
int scratch_address(int dev, void** out) {
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_init);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return PKV_OK;
}

}  // namespace

extern "C" int pkv_decode_gqa_noalloc(const void* q, int32_t num_q_heads, const pkv_cache_t* cache,
                                      const int32_t* block_table, int32_t max_blocks_per_seq,
                                      const int32_t* context_lengths, const int32_t* cu_q_lens, int32_t batch,
                                      int32_t max_q_len, float scale, void* out, float* lse_out,
                                      const pkv_decode_opts_t* opts, void* stream) {
    if (!cache) return PKV_ERR_INVALID_ARG;
    const int32_t mql = cu_q_lens ? max_q_len : 1;
    const size_t need = pkv_decode_workspace_size(batch, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                                  max_blocks_per_seq, cache->block_size, mql, cache->quant_mode,
                                                  opts);
    if (need > kScratchBytes) return PKV_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_HIP;
        if (stream) {  // the scratch address is the current device's: the stream must run there
            hipDevice_t sdev = -1;
            if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return PKV_ERR_HIP;
            if (sdev != dev) return PKV_ERR_INVALID_ARG;
        }
        const int st = scratch_address(dev, &ws);
        if (st != PKV_OK) return st;
    }
    // everything else (argument checks, plan, kernels) is pkv_decode_gqa's
    return pkv_decode_gqa(q, num_q_heads, cache, block_table, max_blocks_per_seq, context_lengths, cu_q_lens,
                          batch, max_q_len, scale, out, lse_out, ws, need > 0 ? kScratchBytes : 0, opts, stream);
}
