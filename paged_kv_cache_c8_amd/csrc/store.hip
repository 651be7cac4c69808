// store.hip - quantizing store of new K/V tokens into the paged cache (gfx950).
//
// Implements MojoStorePagedKVCacheC8 of Mojo Opset PR #379 (and its bf16 sibling
// MojoStorePagedKVCache from the README's Op List) without the torch reference's per-chunk host
// loop: every (token, KV head) or (sequence, block, KV head) is one device work item, resolved
// from the block table on the GPU, so no host synchronisation happens on this path.
//
//   Chunk and prompt stores (cu_q_lens given, up to more than one token per sequence) go by
//   16-slot tiles, the unit of the V page: one wave per (sequence, tile of 16 positions, KV head).
//   Lane (s, q) = (lane / 4, lane % 4) loads channels q D/4 .. of slot s's new token as 16-byte
//   bf16 loads; a quad DPP max gives each token's absmax, scale = fl32(absmax / 127), each lane
//   divides (IEEE) and rounds half to even.  The K rows of the tile are 16 D contiguous bytes,
//   written 16 bytes per store; the V codes go through 16 D bytes of LDS (token rows in,
//   channel columns out), so each lane writes whole 16-slot channel rows of the channel-major V
//   tile, 16 bytes per store.  A tile the call fills only in part keeps the bytes of its other
//   slots (read back and merged; one wave is the tile's only writer).
//   per token (mode 0): as above.  Decode-size stores (one token per sequence) and the
//       slot_mapping form keep one wave per (token, KV head): each token is its own tile row.
//   per block (mode 1): one workgroup per (sequence, block touched, KV head) - the single writer
//       of that block's scale - of one tile wave per 16 slots of the block.  s = max(s_old,
//       fl32(absmax_new / 127)) (the waves' maxima meet in LDS); when s grows the codes already
//       in the block are re-quantized from fl32(code * s_old).
//   per channel (mode 3): codes from static per-channel scales, the scales untouched.
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

// =============================================================================================
// Tile stores
// =============================================================================================

constexpr int TS = kVTile;  // slots per tile

template <int N>
__device__ __forceinline__ void load_bf16_row(const uint16_t* src, bool on, float* x) {
#pragma unroll
    for (int l = 0; l < N / 8; ++l) {
        const u32x4 w = on ? load16(src + 8 * l) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * l + e] = bf16_at(w, e);
    }
}

// N int8 codes (N a multiple of 16) packed four to a dword and stored as 16-byte pieces
template <int N>
__device__ __forceinline__ void store_codes(uint8_t* dst, const int* c) {
#pragma unroll
    for (int l = 0; l < N / 16; ++l) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)(c[16 * l + 4 * i] & 255) | ((uint32_t)(c[16 * l + 4 * i + 1] & 255) << 8) |
                   ((uint32_t)(c[16 * l + 4 * i + 2] & 255) << 16) | ((uint32_t)(c[16 * l + 4 * i + 3] & 255) << 24);
        *reinterpret_cast<uint4*>(dst + 16 * l) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// byte mask of dword w (slots 4w .. 4w+3) of a 16-slot int8 channel row: slots in [lo, hi)
__device__ __forceinline__ uint32_t slot_mask8(int w, int lo, int hi) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m |= (4 * w + i >= lo && 4 * w + i < hi) ? (0xffu << (8 * i)) : 0u;
    return m;
}

// The V codes of the tile, written row-major (slot s, channels q D/4 ..) to lds by the lanes that
// hold a slot, read back as the channel rows this lane writes: channels (D/64) lane .. + D/64 - 1,
// 16 slots each, four dwords per channel (byte i of dword w = slot 4w + i).
template <int D>
__device__ __forceinline__ void transpose_codes(uint8_t* lds, int lane, bool on, const int* codes,
                                                uint32_t (*col)[4]) {
    constexpr int CPL = D / 4;
    if (on) store_codes<CPL>(lds + (lane >> 2) * D + (lane & 3) * CPL, codes);
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < D / 64; ++cc)
#pragma unroll
        for (int w = 0; w < 4; ++w) col[cc][w] = 0u;
#pragma unroll
    for (int sl = 0; sl < TS; ++sl) {
        if constexpr (D == 128) {
            const uint32_t v = *reinterpret_cast<const uint16_t*>(lds + sl * D + 2 * lane);
            col[0][sl >> 2] |= (v & 0xffu) << (8 * (sl & 3));
            col[1][sl >> 2] |= ((v >> 8) & 0xffu) << (8 * (sl & 3));
        } else {
            const uint32_t v = lds[sl * D + lane];
            col[0][sl >> 2] |= v << (8 * (sl & 3));
        }
    }
    __syncthreads();  // lds is free again
}

// One wave per (sequence, 16-position tile, KV head) of a chunk store; modes 0 (per token), 3 (per
// channel) and 2 (bf16).
template <int D, int MODE>
__global__ __launch_bounds__(64) void store_tile_kernel(StoreArgs a) {
    constexpr int ESZ = MODE == 2 ? 2 : 1;
    constexpr int CPL = D / 4;
    __shared__ __attribute__((aligned(16))) uint8_t lds[TS * D * ESZ];
    int r = blockIdx.x;
    const int h = r % a.hkv;
    r /= a.hkv;
    const int kk = r % a.ntile;
    const int b = r / a.ntile;
    const int qlen = a.cu_q[b + 1] - a.cu_q[b];
    if (qlen <= 0) return;
    const int ctx = a.ctx[b];
    const int prior = ctx - qlen;
    if (prior < 0) return;
    const int p0 = ((prior >> 4) + kk) * TS;  // first position of the tile
    if (p0 >= ctx) return;
    const int lo = max(prior, p0) - p0;       // the call's slots of the tile: [lo, hi)
    const int hi = min(ctx, p0 + TS) - p0;
    const int64_t page = (int64_t)a.bt[(int64_t)b * a.mbs + (p0 >> a.log2bs)] * a.hkv + h;
    const int sib = p0 & (a.bs - 1);  // the tile's first slot in its block
    const int lane = threadIdx.x;
    const int sl = lane >> 2, q = lane & 3;
    const bool on = sl >= lo && sl < hi;
    const int64_t tok = (int64_t)a.cu_q[b] + (p0 + sl - prior);  // (only read when on)
    const bool partial = lo > 0 || hi < TS;
    const int64_t vtile = page * D * a.bs + (int64_t)(sib / TS) * D * TS;  // element offset of the V tile

#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = (which ? a.v_new : a.k_new) + (tok * a.hkv + h) * D + q * CPL;
        if constexpr (MODE == 2) {
            uint16_t* kd = reinterpret_cast<uint16_t*>(a.k);
            uint16_t* vd = reinterpret_cast<uint16_t*>(a.v);
            u32x4 raw[CPL / 8];
#pragma unroll
            for (int l = 0; l < CPL / 8; ++l) raw[l] = on ? load16(src + 8 * l) : u32x4{0u, 0u, 0u, 0u};
            if (which == 0) {
                if (on) {
                    uint16_t* row = kd + (page * a.bs + sib + sl) * D + q * CPL;
#pragma unroll
                    for (int l = 0; l < CPL / 8; ++l)
                        *reinterpret_cast<uint4*>(row + 8 * l) = make_uint4(raw[l].x, raw[l].y, raw[l].z, raw[l].w);
                }
                continue;
            }
            // V: rows of bf16 to LDS, channel rows of 16 slots (32 bytes) out
            if (on) {
#pragma unroll
                for (int l = 0; l < CPL / 8; ++l)
                    *reinterpret_cast<uint4*>(lds + (sl * D + q * CPL + 8 * l) * 2) =
                        make_uint4(raw[l].x, raw[l].y, raw[l].z, raw[l].w);
            }
            __syncthreads();
#pragma unroll
            for (int cc = 0; cc < D / 64; ++cc) {
                const int c = lane * (D / 64) + cc;
                uint32_t o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t e0 = *reinterpret_cast<const uint16_t*>(lds + ((2 * i) * D + c) * 2);
                    const uint32_t e1 = *reinterpret_cast<const uint16_t*>(lds + ((2 * i + 1) * D + c) * 2);
                    o[i] = e0 | (e1 << 16);
                }
                uint16_t* dst = vd + vtile + (int64_t)c * TS;
                if (partial) {
                    const u32x4 o0 = load16(dst), o1 = load16(dst + 8);
                    const uint32_t old[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t m = ((2 * i >= lo && 2 * i < hi) ? 0xffffu : 0u) |
                                           ((2 * i + 1 >= lo && 2 * i + 1 < hi) ? 0xffff0000u : 0u);
                        o[i] = (o[i] & m) | (old[i] & ~m);
                    }
                }
                *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
                *reinterpret_cast<uint4*>(dst + 8) = make_uint4(o[4], o[5], o[6], o[7]);
            }
        } else {
            float x[CPL];
            load_bf16_row<CPL>(src, on, x);
            int codes[CPL];
            float s = 0.0f;
            if constexpr (MODE == 3) {  // static per-channel scales
                const float* sc = (which ? a.vs : a.ks) + (int64_t)h * D + q * CPL;
#pragma unroll
                for (int e = 0; e < CPL; ++e) codes[e] = quant_code(x[e], sc[e]);
            } else {
                float am = 0.0f;
#pragma unroll
                for (int e = 0; e < CPL; ++e) am = fmaxf(am, fabsf(x[e]));
                am = group_max<4>(am);  // the four lanes of the slot
                s = absmax_scale(am);
#pragma unroll
                for (int e = 0; e < CPL; ++e) codes[e] = quant_code(x[e], s);
            }
            if (which == 0) {
                if (on) store_codes<CPL>(reinterpret_cast<uint8_t*>(a.k) + (page * a.bs + sib + sl) * D + q * CPL, codes);
            } else {
                uint32_t col[D / 64][4];
                transpose_codes<D>(lds, lane, on, codes, col);
#pragma unroll
                for (int cc = 0; cc < D / 64; ++cc) {
                    uint8_t* dst = reinterpret_cast<uint8_t*>(a.v) + vtile + (int64_t)(lane * (D / 64) + cc) * TS;
                    if (partial) {
                        const u32x4 o = load16(dst);
                        const uint32_t old[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const uint32_t m = slot_mask8(w, lo, hi);
                            col[cc][w] = (col[cc][w] & m) | (old[w] & ~m);
                        }
                    }
                    *reinterpret_cast<uint4*>(dst) = make_uint4(col[cc][0], col[cc][1], col[cc][2], col[cc][3]);
                }
            }
            if constexpr (MODE == 0) {
                if (on && q == 0) (which ? a.vs : a.ks)[page * a.bs + sib + sl] = s;
            }
        }
    }
}

// Per-block scales: one workgroup of bs/16 tile waves per (sequence, block touched, KV head).
template <int D>
__global__ __launch_bounds__(512) void store_block_tiles_kernel(StoreArgs a) {
    constexpr int CPL = D / 4;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_all[];  // [bs / 16][TS * D]
    __shared__ float red[8];
    __shared__ float sold_s;
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
    if (j * a.bs >= ctx) return;  // (uniform over the workgroup)
    const int lo_pos = max(prior, j * a.bs);  // the call's positions in the block: [lo_pos, hi_pos)
    const int hi_pos = min(ctx, (j + 1) * a.bs);
    const int n_old = lo_pos - j * a.bs;      // positions already in the block
    const int64_t page = (int64_t)a.bt[(int64_t)b * a.mbs + j] * a.hkv + h;

    const int w = threadIdx.x >> 6;  // tile of the block
    const int nw = blockDim.x >> 6;
    const int lane = threadIdx.x & 63;
    uint8_t* lds = lds_all + w * TS * D;
    const int p0 = j * a.bs + w * TS;
    const int nlo = min(max(lo_pos - p0, 0), TS), nhi = min(max(hi_pos - p0, 0), TS);  // new slots
    const int nold = min(max(n_old - w * TS, 0), TS);                                  // old slots [0, nold)
    const int sl = lane >> 2, q = lane & 3;
    const bool on = sl >= nlo && sl < nhi;
    const int64_t tok = (int64_t)t0 + (p0 + sl - prior);
    const int64_t vtile = page * D * a.bs + (int64_t)w * D * TS;
    const int64_t krow = (page * a.bs + w * TS + sl) * D + q * CPL;

#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = (which ? a.v_new : a.k_new) + (tok * a.hkv + h) * D + q * CPL;
        float* sc = which ? a.vs : a.ks;
        uint8_t* dst = reinterpret_cast<uint8_t*>(which ? a.v : a.k);
        // the block's scale is read by thread 0 only (which also writes it last) and shared via LDS
        if (threadIdx.x == 0) sold_s = n_old > 0 ? sc[page] : 0.0f;
        float x[CPL];
        load_bf16_row<CPL>(src, on, x);
        float am = 0.0f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) am = fmaxf(am, fabsf(x[e]));
        am = group_max<kWave>(am);
        if (lane == 0) red[w] = am;
        __syncthreads();
        const float s_old = sold_s;
        float a_new = red[0];
        for (int i = 1; i < nw; ++i) a_new = fmaxf(a_new, red[i]);
        const float s = fmaxf(s_old, absmax_scale(a_new));
        const bool requant = n_old > 0 && s > s_old;
        int codes[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) codes[e] = quant_code(x[e], s);
        if (which == 0) {
            if (on) {
                store_codes<CPL>(dst + krow, codes);
            } else if (requant && sl < nold) {  // an old row: re-quantize its codes to the new scale
                int old[CPL];
#pragma unroll
                for (int l = 0; l < CPL / 16; ++l) {
                    const u32x4 v = load16(dst + krow + 16 * l);
#pragma unroll
                    for (int e = 0; e < 16; ++e) old[16 * l + e] = quant_code((float)(int8_t)((word(v, e >> 2) >> (8 * (e & 3))) & 0xffu) * s_old, s);
                }
                store_codes<CPL>(dst + krow, old);
            }
        } else {
            uint32_t col[D / 64][4];
            transpose_codes<D>(lds, lane, on, codes, col);
            const bool any_new = nhi > nlo;
            if (any_new || (requant && nold > 0)) {
#pragma unroll
                for (int cc = 0; cc < D / 64; ++cc) {
                    uint8_t* vd = dst + vtile + (int64_t)(lane * (D / 64) + cc) * TS;
                    if (nlo > 0 || nhi < TS) {  // other slots: kept, or re-quantized when old and the scale grew
                        const u32x4 o = load16(vd);
                        uint32_t old[4] = {o.x, o.y, o.z, o.w};
                        if (requant) {
#pragma unroll
                            for (int ww = 0; ww < 4; ++ww) {
                                uint32_t nw8 = 0;
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const int slot = 4 * ww + i;
                                    uint32_t byte = (old[ww] >> (8 * i)) & 0xffu;
                                    if (slot < nold) byte = (uint32_t)(quant_code((float)(int8_t)byte * s_old, s) & 255);
                                    nw8 |= byte << (8 * i);
                                }
                                old[ww] = nw8;
                            }
                        }
#pragma unroll
                        for (int ww = 0; ww < 4; ++ww) {
                            const uint32_t m = slot_mask8(ww, nlo, nhi);
                            col[cc][ww] = (col[cc][ww] & m) | (old[ww] & ~m);
                        }
                    }
                    *reinterpret_cast<uint4*>(vd) = make_uint4(col[cc][0], col[cc][1], col[cc][2], col[cc][3]);
                }
            }
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
        hipLaunchKernelGGL(store_block_tiles_kernel<D>, dim3((unsigned)grid), dim3(64 * (a.bs / TS)),
                           (size_t)(a.bs / TS) * TS * D, stream, a);
        return hipGetLastError();
    }
    if (a.cu_q && !a.slot_mapping && a.ntile > 0) {  // chunk / prompt store: by tiles
        const int64_t grid = (int64_t)a.batch * a.ntile * a.hkv;
        if (grid == 0) return hipSuccess;
        if (grid > 0x7fffffff) return hipErrorInvalidValue;
        if (mode == 0)
            hipLaunchKernelGGL((store_tile_kernel<D, 0>), dim3((unsigned)grid), dim3(64), 0, stream, a);
        else if (mode == 3)
            hipLaunchKernelGGL((store_tile_kernel<D, 3>), dim3((unsigned)grid), dim3(64), 0, stream, a);
        else
            hipLaunchKernelGGL((store_tile_kernel<D, 2>), dim3((unsigned)grid), dim3(64), 0, stream, a);
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
