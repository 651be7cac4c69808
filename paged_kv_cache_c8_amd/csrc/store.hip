// store.hip - quantizing store of new K/V tokens into the paged cache (gfx950).
//
// Implements MojoStorePagedKVCacheC8 of Mojo Opset PR #379 (and its bf16 sibling
// MojoStorePagedKVCache from the README's Op List) without the torch reference's per-chunk host
// loop: every (token, KV head) or (sequence, block, KV head) is one device work item, resolved
// from the block table on the GPU, so no host synchronisation happens on this path.
//
//   per token (mode 0): one wave per (token, KV head); the wave's lanes hold the head_dim
//       values, a DPP/shuffle max gives the absmax, scale = fl32(absmax / 127), each lane
//       divides (IEEE) and rounds half to even.  K rows are written as contiguous bytes; V goes
//       to the slot's channel-major 16-slot tile (one byte per channel, stride 16).
//   per block (mode 1): one workgroup per (sequence, block touched, KV head) - the single writer
//       of that block's scale.  s = max(s_old, fl32(absmax_new / 127)); when s grows the codes
//       already in the block are re-quantized from fl32(code * s_old).
//   bf16 (mode 2): a copy into the same layout.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// Physical block and slot of new token t; false when the token is skipped.
__device__ __forceinline__ bool resolve_slot(const StoreArgs& a, int t, int64_t& blk, int& slot) {
    if (a.slot_mapping) {
        const int64_t s = a.slot_mapping[t];
        if (s < 0) return false;
        blk = s >> a.log2bs;
        slot = (int)(s & (a.bs - 1));
        return true;
    }
    int b, i;
    if (a.cu_q) {
        // largest b with cu_q[b] <= t (skips sequences without new tokens)
        int lo = 0, hi = a.batch;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu_q[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        b = lo;
        if (b >= a.batch) return false;  // t beyond cu_q_lens[batch]: nothing to store
        i = t - a.cu_q[b];
        const int qlen = a.cu_q[b + 1] - a.cu_q[b];
        const int pos = a.ctx[b] - qlen + i;
        blk = a.bt[(int64_t)b * a.mbs + (pos >> a.log2bs)];
        slot = pos & (a.bs - 1);
    } else {
        b = t;
        const int pos = a.ctx[b] - 1;
        if (pos < 0) return false;
        blk = a.bt[(int64_t)b * a.mbs + (pos >> a.log2bs)];
        slot = pos & (a.bs - 1);
    }
    return true;
}

template <int D, int MODE>
__global__ __launch_bounds__(256) void store_token_kernel(StoreArgs a) {
    constexpr int EPL = D / kWave;  // values per lane (1 or 2)
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (item >= (int64_t)a.num_tokens * a.hkv) return;  // uniform per wave
    const int t = (int)(item / a.hkv);
    const int h = (int)(item % a.hkv);
    int64_t blk;
    int slot;
    if (!resolve_slot(a, t, blk, slot)) return;
    const int64_t page = blk * a.hkv + h;
    const int c0 = lane * EPL;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = (which ? a.v_new : a.k_new) + ((int64_t)t * a.hkv + h) * D + c0;
        uint32_t bits[EPL];
        if constexpr (EPL == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
            bits[0] = w & 0xffffu;
            bits[1] = w >> 16;
        } else {
            bits[0] = src[0];
        }
        if constexpr (MODE == 2) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(which ? a.v : a.k);
            if (which == 0) {
                uint16_t* row = dst + (page * a.bs + slot) * D + c0;
#pragma unroll
                for (int e = 0; e < EPL; ++e) row[e] = (uint16_t)bits[e];
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) dst[v_elem(page, D, a.bs, c0 + e, slot)] = (uint16_t)bits[e];
            }
        } else if constexpr (MODE == 3) {  // static per-channel scales: codes only
            const float* sc = (which ? a.vs : a.ks) + (int64_t)h * D + c0;
            int8_t* dst = reinterpret_cast<int8_t*>(which ? a.v : a.k);
            if (which == 0) {
                int8_t* row = dst + (page * a.bs + slot) * D + c0;
#pragma unroll
                for (int e = 0; e < EPL; ++e) row[e] = (int8_t)quant_code(bf16_to_f32(bits[e]), sc[e]);
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    dst[v_elem(page, D, a.bs, c0 + e, slot)] = (int8_t)quant_code(bf16_to_f32(bits[e]), sc[e]);
            }
        } else {
            float x[EPL];
            float am = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                x[e] = bf16_to_f32(bits[e]);
                am = fmaxf(am, fabsf(x[e]));
            }
            am = group_max<kWave>(am);
            const float s = absmax_scale(am);
            int8_t* dst = reinterpret_cast<int8_t*>(which ? a.v : a.k);
            if (which == 0) {
                int8_t* row = dst + (page * a.bs + slot) * D + c0;
#pragma unroll
                for (int e = 0; e < EPL; ++e) row[e] = (int8_t)quant_code(x[e], s);
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    dst[v_elem(page, D, a.bs, c0 + e, slot)] = (int8_t)quant_code(x[e], s);
            }
            if (lane == 0) (which ? a.vs : a.ks)[page * a.bs + slot] = s;
        }
    }
}

__device__ __forceinline__ float block_max256(float x, float* red) {
    x = group_max<kWave>(x);
    const int w = threadIdx.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[w] = x;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int D>
__global__ __launch_bounds__(256) void store_block_kernel(StoreArgs a) {
    __shared__ float red[4];
    int r = blockIdx.x;
    const int h = r % a.hkv;
    r /= a.hkv;
    const int jj = r % a.nbt;
    const int b = r / a.nbt;
    const int qlen = a.cu_q ? a.cu_q[b + 1] - a.cu_q[b] : 1;
    if (qlen <= 0) return;
    const int t0 = a.cu_q ? a.cu_q[b] : b;
    const int ctx = a.ctx[b];
    const int prior = ctx - qlen;
    if (prior < 0) return;  // inactive decode slot (context length 0): nothing to store
    const int j = (prior >> a.log2bs) + jj;
    if (j * a.bs >= ctx) return;
    const int lo = max(prior, j * a.bs);
    const int hi = min(ctx, (j + 1) * a.bs);
    const int n_new = hi - lo;
    const int n_old = lo - j * a.bs;
    const int64_t page = (int64_t)a.bt[(int64_t)b * a.mbs + j] * a.hkv + h;

    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = which ? a.v_new : a.k_new;
        float* sc = which ? a.vs : a.ks;
        int8_t* dst = reinterpret_cast<int8_t*>(which ? a.v : a.k);
        const float s_old = n_old > 0 ? sc[page] : 0.0f;  // read by every thread before any write
        float am = 0.0f;
        for (int e = threadIdx.x; e < n_new * D; e += blockDim.x) {
            const int p = lo + e / D;
            const int c = e % D;
            const uint16_t bits = src[((int64_t)(t0 + p - prior) * a.hkv + h) * D + c];
            am = fmaxf(am, fabsf(bf16_to_f32(bits)));
        }
        am = block_max256(am, red);
        const float s_new = absmax_scale(am);
        const float s = fmaxf(s_old, s_new);
        if (n_old > 0 && s > s_old) {
            for (int e = threadIdx.x; e < n_old * D; e += blockDim.x) {
                const int slot = e / D;
                const int c = e % D;
                const int64_t idx = which ? v_elem(page, D, a.bs, c, slot) : (page * a.bs + slot) * D + c;
                const float old_value = (float)dst[idx] * s_old;
                dst[idx] = (int8_t)quant_code(old_value, s);
            }
        }
        for (int e = threadIdx.x; e < n_new * D; e += blockDim.x) {
            const int p = lo + e / D;
            const int c = e % D;
            const int slot = p - j * a.bs;
            const float x = bf16_to_f32(src[((int64_t)(t0 + p - prior) * a.hkv + h) * D + c]);
            const int64_t idx = which ? v_elem(page, D, a.bs, c, slot) : (page * a.bs + slot) * D + c;
            dst[idx] = (int8_t)quant_code(x, s);
        }
        if (threadIdx.x == 0) sc[page] = s;
        __syncthreads();  // red[] is reused by the V pass
    }
}

template <int D>
hipError_t launch_store_d(const StoreArgs& a, int mode, hipStream_t stream) {
    if (mode == 1) {
        const int64_t grid = (int64_t)a.batch * a.nbt * a.hkv;
        if (grid == 0) return hipSuccess;
        if (grid > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL(store_block_kernel<D>, dim3((unsigned)grid), dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    const int64_t items = (int64_t)a.num_tokens * a.hkv;
    const int64_t grid = (items + 3) / 4;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (mode == 0)
        hipLaunchKernelGGL((store_token_kernel<D, 0>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    else if (mode == 3)
        hipLaunchKernelGGL((store_token_kernel<D, 3>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((store_token_kernel<D, 2>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_store(const StoreArgs& a, int head_dim, int mode, hipStream_t stream) {
    if (head_dim == 64) return launch_store_d<64>(a, mode, stream);
    if (head_dim == 128) return launch_store_d<128>(a, mode, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
