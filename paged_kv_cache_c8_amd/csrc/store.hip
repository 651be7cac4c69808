// store.hip - quantizing store of new K/V tokens into the paged cache (gfx950).
//
// Implements MojoStorePagedKVCacheC8 of Mojo Opset PR #379 (and its bf16 sibling
// MojoStorePagedKVCache from the README's Op List) without the torch reference's per-chunk host
// loop: every (token, KV head) or (sequence, block, KV head) is one device work item, resolved
// from the block table on the GPU, so no host synchronisation happens on this path.
//
//   Chunk and prompt stores (cu_q_lens given, up to more than one token per sequence) go by
//   16-slot tiles, the unit of the V page: one wave per (sequence, tile of 16 positions, KV head).
//   In each step the wave reads whole token rows of its tile (16-byte bf16 loads; a row's lanes
//   meet in a DPP max for its absmax; scale = fl32(absmax / 127); codes rounded half to even from
//   one reciprocal per row, the same codes as IEEE division) and writes whole 128-byte K rows; the
//   V codes go through 16 D bytes of LDS (token rows in, channel rows out), so each 16-byte store
//   covers 64 consecutive channel rows of the channel-major V tile.  A tile the call fills only in
//   part keeps the bytes of its other slots (read back and merged; one wave is the tile's only
//   writer).
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
            int codes[EPL];
            quant_row_absmax<EPL>(x, s, codes);
            int8_t* dst = reinterpret_cast<int8_t*>(which ? a.v : a.k);
            if (which == 0) {
                int8_t* row = dst + (page * a.bs + slot) * D + c0;
#pragma unroll
                for (int e = 0; e < EPL; ++e) row[e] = (int8_t)codes[e];
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) dst[v_elem(page, D, a.bs, c0 + e, slot)] = (int8_t)codes[e];
            }
            if (lane == 0) (which ? a.vs : a.ks)[page * a.bs + slot] = s;
        }
    }
}

// =============================================================================================
// Tile stores
//
// A tile wave walks the tile's 16 token rows in steps: in step j, lane L takes the 8-channel chunk
// L % CH of row j RPI + L / CH (CH = D / 8 chunks per row, RPI = 64 / CH rows per step), so each
// load of the bf16 input rows and each store of K code rows covers RPI whole rows, and a row's
// absmax is a max over its CH lanes.  The V codes go to LDS as token rows and come back out as
// channel rows: lane L writes channels L + 64 c, so each 16-byte store covers 64 consecutive
// 16-slot channel rows of the tile.  A tile the call fills only in part keeps the bytes of its other
// slots (read back and merged; one wave is the tile's only writer).
// =============================================================================================

constexpr int TS = kVTile;  // slots per tile

template <int D>
struct TileMap {
    static constexpr int CH = D / 8;        // 8-channel chunks per row
    static constexpr int RPI = kWave / CH;  // rows per step
    static constexpr int NJ = TS / RPI;     // steps per tile
    static constexpr int CPW = D / 64;      // V channel rows per lane
};

__device__ __forceinline__ void unpack_bf16x8(const u32x4& w, float* x) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = bf16_at(w, e);
}

__device__ __forceinline__ uint2 pack_codes8(const int* c) {
    uint32_t w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        w[i] = (uint32_t)(c[4 * i] & 255) | ((uint32_t)(c[4 * i + 1] & 255) << 8) |
               ((uint32_t)(c[4 * i + 2] & 255) << 16) | ((uint32_t)(c[4 * i + 3] & 255) << 24);
    return make_uint2(w[0], w[1]);
}

// byte mask of dword w (slots 4w .. 4w+3) of a 16-slot int8 channel row: slots in [lo, hi)
__device__ __forceinline__ uint32_t slot_mask8(int w, int lo, int hi) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m |= (4 * w + i >= lo && 4 * w + i < hi) ? (0xffu << (8 * i)) : 0u;
    return m;
}

// The tile's V codes from LDS token rows (byte slot * D + channel) to the lane's channel rows,
// channels lane + 64 cc: four dwords of 16 slots each (byte i of dword w = slot 4w + i).
template <int D>
__device__ __forceinline__ void lds_channel_rows(const uint8_t* lds, int lane, uint32_t (*col)[4]) {
    constexpr int CPW = TileMap<D>::CPW;
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
        for (int w = 0; w < 4; ++w) col[cc][w] = 0u;
#pragma unroll
    for (int t = 0; t < TS; ++t)
#pragma unroll
        for (int cc = 0; cc < CPW; ++cc) col[cc][t >> 2] |= (uint32_t)lds[t * D + lane + 64 * cc] << (8 * (t & 3));
}

// One wave per (sequence, 16-position tile, KV head) of a chunk store; modes 0 (per token), 3 (per
// channel) and 2 (bf16).
template <int D, int MODE>
__global__ __launch_bounds__(64) void store_tile_kernel(StoreArgs a) {
    using M = TileMap<D>;
    constexpr int ESZ = MODE == 2 ? 2 : 1;
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
    const int rl = lane / M::CH, c8 = (lane % M::CH) * 8;
    const bool partial = lo > 0 || hi < TS;
    const int64_t vtile = page * D * a.bs + (int64_t)(sib / TS) * D * TS;  // element offset of the V tile
    const int64_t tok0 = (int64_t)a.cu_q[b] + (p0 - prior);                // token of slot 0

#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = which ? a.v_new : a.k_new;
        if constexpr (MODE == 2) {
            uint16_t* kd = reinterpret_cast<uint16_t*>(a.k);
#pragma unroll
            for (int j = 0; j < M::NJ; ++j) {
                const int sl = j * M::RPI + rl;
                const bool on = sl >= lo && sl < hi;
                const u32x4 v = on ? load16(src + ((tok0 + sl) * a.hkv + h) * D + c8) : u32x4{0u, 0u, 0u, 0u};
                if (which == 0) {
                    if (on) *reinterpret_cast<uint4*>(kd + (page * a.bs + sib + sl) * D + c8) = make_uint4(v.x, v.y, v.z, v.w);
                } else {
                    *reinterpret_cast<uint4*>(lds + (sl * D + c8) * 2) = make_uint4(v.x, v.y, v.z, v.w);
                }
            }
            if (which == 0) continue;
            __builtin_amdgcn_wave_barrier();
            // channel rows out: step k, lane L: channel 32 k + L / 2, slots 8 (L % 2) .. + 8
            uint16_t* vd = reinterpret_cast<uint16_t*>(a.v);
#pragma unroll
            for (int k = 0; k < D / 32; ++k) {
                const int c = 32 * k + (lane >> 1), s0 = 8 * (lane & 1);
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t e0 = *reinterpret_cast<const uint16_t*>(lds + ((s0 + 2 * i) * D + c) * 2);
                    const uint32_t e1 = *reinterpret_cast<const uint16_t*>(lds + ((s0 + 2 * i + 1) * D + c) * 2);
                    o[i] = e0 | (e1 << 16);
                }
                uint16_t* dst = vd + vtile + (int64_t)c * TS + s0;
                if (partial) {
                    const u32x4 ov = load16(dst);
                    const uint32_t old[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = s0 + 2 * i;
                        const uint32_t m = ((t >= lo && t < hi) ? 0xffffu : 0u) | ((t + 1 >= lo && t + 1 < hi) ? 0xffff0000u : 0u);
                        o[i] = (o[i] & m) | (old[i] & ~m);
                    }
                }
                *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        } else {
            float* scales = which ? a.vs : a.ks;
            uint8_t* kd = reinterpret_cast<uint8_t*>(a.k);
#pragma unroll
            for (int j = 0; j < M::NJ; ++j) {
                const int sl = j * M::RPI + rl;
                const bool on = sl >= lo && sl < hi;
                float x[8];
                unpack_bf16x8(on ? load16(src + ((tok0 + sl) * a.hkv + h) * D + c8) : u32x4{0u, 0u, 0u, 0u}, x);
                int codes[8];
                float s = 0.0f;
                if constexpr (MODE == 3) {  // static per-channel scales
                    const float* sc = scales + (int64_t)h * D + c8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) codes[e] = quant_code(x[e], sc[e]);
                } else {
                    float am = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[e]));
                    am = group_max<M::CH>(am);  // the row's CH lanes
                    s = absmax_scale(am);
                    quant_row_absmax<8>(x, s, codes);
                }
                const uint2 pk = pack_codes8(codes);
                if (which == 0) {
                    if (on) *reinterpret_cast<uint2*>(kd + (page * a.bs + sib + sl) * D + c8) = pk;
                } else {
                    *reinterpret_cast<uint2*>(lds + sl * D + c8) = pk;
                }
                if constexpr (MODE == 0) {
                    if (on && (lane % M::CH) == 0) scales[page * a.bs + sib + sl] = s;
                }
            }
            if (which == 0) continue;
            __builtin_amdgcn_wave_barrier();
            uint32_t col[M::CPW][4];
            lds_channel_rows<D>(lds, lane, col);
#pragma unroll
            for (int cc = 0; cc < M::CPW; ++cc) {
                uint8_t* dst = reinterpret_cast<uint8_t*>(a.v) + vtile + (int64_t)(lane + 64 * cc) * TS;
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
    }
}

// Per-block scales: one workgroup of bs/16 tile waves per (sequence, block touched, KV head).
template <int D>
__global__ __launch_bounds__(512) void store_block_tiles_kernel(StoreArgs a) {
    using M = TileMap<D>;
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
    const int rl = lane / M::CH, c8 = (lane % M::CH) * 8;
    const int64_t tok0 = (int64_t)t0 + (p0 - prior);
    const int64_t vtile = page * D * a.bs + (int64_t)w * D * TS;
    const int64_t krow0 = (page * a.bs + w * TS) * D + c8;

#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = which ? a.v_new : a.k_new;
        float* sc = which ? a.vs : a.ks;
        uint8_t* dst = reinterpret_cast<uint8_t*>(which ? a.v : a.k);
        // the block's scale is read by thread 0 only (which also writes it last) and shared via LDS
        if (threadIdx.x == 0) sold_s = n_old > 0 ? sc[page] : 0.0f;
        float x[M::NJ][8];
        float am = 0.0f;
#pragma unroll
        for (int jj2 = 0; jj2 < M::NJ; ++jj2) {
            const int sl = jj2 * M::RPI + rl;
            const bool on = sl >= nlo && sl < nhi;
            unpack_bf16x8(on ? load16(src + ((tok0 + sl) * a.hkv + h) * D + c8) : u32x4{0u, 0u, 0u, 0u}, x[jj2]);
#pragma unroll
            for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[jj2][e]));
        }
        am = group_max<kWave>(am);
        if (lane == 0) red[w] = am;
        __syncthreads();
        const float s_old = sold_s;
        float a_new = red[0];
        for (int i = 1; i < nw; ++i) a_new = fmaxf(a_new, red[i]);
        const float s = fmaxf(s_old, absmax_scale(a_new));
        const bool requant = n_old > 0 && s > s_old;
#pragma unroll
        for (int jj2 = 0; jj2 < M::NJ; ++jj2) {
            const int sl = jj2 * M::RPI + rl;
            const bool on = sl >= nlo && sl < nhi;
            int codes[8];
            quant_row_absmax<8>(x[jj2], s, codes);  // s is fl32(A / 127) of the block's bf16 absmax A >= |x|
            if (which == 0) {
                if (on) {
                    *reinterpret_cast<uint2*>(dst + krow0 + sl * D) = pack_codes8(codes);
                } else if (requant && sl < nold) {  // an old row: re-quantize its codes to the new scale
                    const uint2 ov = *reinterpret_cast<const uint2*>(dst + krow0 + sl * D);
                    int oc[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        oc[e] = quant_code((float)(int8_t)(((e < 4 ? ov.x : ov.y) >> (8 * (e & 3))) & 0xffu) * s_old, s);
                    *reinterpret_cast<uint2*>(dst + krow0 + sl * D) = pack_codes8(oc);
                }
            } else {
                *reinterpret_cast<uint2*>(lds + sl * D + c8) = pack_codes8(codes);
            }
        }
        if (which == 1 && (nhi > nlo || (requant && nold > 0))) {
            __builtin_amdgcn_wave_barrier();
            uint32_t col[M::CPW][4];
            lds_channel_rows<D>(lds, lane, col);
#pragma unroll
            for (int cc = 0; cc < M::CPW; ++cc) {
                uint8_t* vd = dst + vtile + (int64_t)(lane + 64 * cc) * TS;
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
        if (threadIdx.x == 0) sc[page] = s;
        __syncthreads();  // red[] and sold_s are reused by the V pass
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
