// decode_mfma.hip - grouped-query attention over the paged cache on the matrix cores (gfx950).
//
// Same result as decode_valu.hip (MojoPagedDecodeGQA, Mojo Opset README Op List), built for the
// HBM roofline of MI355X: at 8 TB/s a compute unit has about 80 SIMD-cycles per (key, KV head),
// while int8 -> fp16 conversion plus dot products on the vector ALUs need more than that, so
// both contractions of every key block run as v_mfma_f32_16x16x32_{f16,bf16} and the vector
// ALUs only convert codes and do the softmax bookkeeping.
//
// One wave per (sequence, KV head, row group, key range): a fixed split, or a segment of the
// balanced partition (sk_partition.h; bf16 pages, planned over several rounds of
// the resident waves); no barriers in the main loop.  A row group is RT tiles of 16 query rows
// (row r = i * G + g: query i of the chunk, head g of the KV head's group); the keys of the range
// are walked in blocks of 32, the next block's K, V and scales in flight while the current one
// computes.
//
//   scores  S^T (keys x rows) = K . Q^T: K is the A operand - lane (rho, kg) holds 32 contiguous
//           bytes (int8) or four 16-byte pieces 64 bytes apart (bf16: the lane groups of a row
//           read 64 contiguous bytes per load) of one token-major K row - and the query tile is B.  The
//           key behind row slot rho of score tile u is 8*(rho/4) + 4u + rho%4, so that in the
//           output lane (n, g) holds keys 8g .. 8g+7 of query row n.  int8 codes become fp16 exactly
//           (byte permute into 0x64xx, subtract 1152); the query row is pre-scaled by a power of two
//           into fp16's normal range and the factor removed with the per-key K scale.
//   softmax online over blocks, per query row (lane column n; rows meet across lanes n+16k).
//           The weights p * s_v / S (S = running max of the V scales, so the fp16 weights stay in
//           [0, 1]) of keys 8g .. 8g+7 are exactly lane (n, g)'s slice of the P operand.
//   P.V     O (rows x channels) += P . V: the channel-major V tile gives the 8 keys of one channel
//           as 8 contiguous bytes - the B operand - with no transpose.  When a row's running max
//           or S grows, its accumulator row is rescaled (rows 4g+i of lane g; factors fetched from
//           the lanes that own those rows).
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"
#include "sk_partition.h"

namespace pkv {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr int BLK = 32;                 // keys per block
constexpr int MAX_SPLIT = 4096;         // keys per split (planner limit)
constexpr int MAX_SPLIT_BLOCKS = MAX_SPLIT / 16;

template <int D, int MODE>
struct MCfg {
    static constexpr int ESZ = MODE == 2 ? 2 : 1;
    static constexpr int KS = D / 32;        // 32-channel k-steps of the score MFMA
    static constexpr int DT = D / 16;        // 16-channel tiles of the output
    static constexpr int KB = 8 * KS * ESZ;  // K bytes per lane per score tile
    static constexpr int KL = KB / 16;       // 16-byte K loads per lane per score tile
    static constexpr int VW = 2 * ESZ;       // V dwords per lane per channel tile (8 keys)
};

template <int D, int MODE>
struct BlockRegs {
    using C = MCfg<D, MODE>;
    u32x4 k[2][C::KL];
    uint32_t v[C::DT][C::VW];
    float ks[8];
    float vs[8];
};

// eight int8 codes (two dwords) -> an fp16 MFMA operand holding 1152 + code (exact): the byte
// permute alone, the constant 1152 removed from the accumulated results instead of every value
__device__ __forceinline__ h8 biased_h8(uint32_t w0, uint32_t w1) {
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;  // code + 128 as unsigned bytes
    const uint32_t r[4] = {__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u),
                           __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)};
    return __builtin_bit_cast(h8, r);
}

// Reductions over the four lanes n, n+16, n+32, n+48 (one query row).  gfx950's permlane swaps
// exchange 16-lane rows (odd rows of one copy with even rows of the other) and 32-lane halves
// in the VALU, instead of a round trip through the LDS crossbar.
__device__ __forceinline__ float xor16_max(float x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// One wave's work: the rows of row group rg of (sequence b, KV head h) over keys
// [t_seg0, t_seg1) (a split or a balanced segment), walked in ranges of at most MAX_SPLIT keys
// (each with its block-table slice in LDS; the softmax state carries over).  The result goes to
// the output (pslot < 0) or to partial slot pslot for the merge.
template <int D, int MODE, int RT>
__device__ __forceinline__ void mfma_segment(const DecodeArgs& a, const int b, const int h, const int rg,
                                             const int t_seg0, const int t_seg1, const int64_t pslot,
                                             int* const bt_s) {
    using C = MCfg<D, MODE>;

    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane & 15;   // query row within a tile (score/P layout), channel (output layout)
    const int g = lane >> 4;   // lane group

    const int qlen = a.cu ? a.cu[b + 1] - a.cu[b] : 1;
    const int qrow0 = a.cu ? a.cu[b] : b;
    const int prior = a.ctx[b] - qlen;
    const int nrows = qlen * a.g;
    const int r0 = rg * (16 * RT);
    const int nvalid = min(16 * RT, nrows - r0);
    int t_begin = t_seg0, t_end = t_seg1;  // the current range (set per range below)
    const int lo_hi = win_lo(a.window, prior + (r0 + nvalid - 1) / a.g);

    // ---- query tiles (B operand of the score MFMA): lane (n, g) holds 8 channels of row n per
    //      k-step m, the same channels its K operand holds (below).
    //      int8 pages: the K operand carries 1152 + code, so every score carries 1152 * sum(q) of
    //      its row in excess; qbias holds that amount (the row's fp16 values summed in fp32).
    uint32_t qb[RT][C::KS][4];
    float rowmul[RT], qbias[RT];
    int lim[RT];
    int lo[RT];           // first key the row may see (sliding window)
    bool causal = false;  // some row of the group cannot see every key of the split
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int j = rt * 16 + n;
        const bool rv = j < nvalid;
        const int r = r0 + j;
        lim[rt] = rv ? prior + r / a.g : 0x7fffffff;
        lo[rt] = rv ? win_lo(a.window, lim[rt]) : 0;
        causal |= lim[rt] < t_end - 1;
        uint32_t raw[C::KS][4];
        if (rv) {
            // k-step m: channels g*8*KS + 8m .. (int8 pages) or 32m + 8g .. (bf16 pages, whose K
            // loads then read 64 contiguous bytes of a row per lane group and instruction)
            const uint16_t* qp = a.q + ((int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g) * D +
                                 (MODE == 2 ? g * 8 : g * 8 * C::KS);
#pragma unroll
            for (int m = 0; m < C::KS; ++m) {
                const u32x4 w = load16(qp + (MODE == 2 ? 32 : 8) * m);
                raw[m][0] = w.x; raw[m][1] = w.y; raw[m][2] = w.z; raw[m][3] = w.w;
            }
        } else {
#pragma unroll
            for (int m = 0; m < C::KS; ++m) raw[m][0] = raw[m][1] = raw[m][2] = raw[m][3] = 0;
        }
        if constexpr (MODE == 2) {
#pragma unroll
            for (int m = 0; m < C::KS; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) qb[rt][m][e] = raw[m][e];
            rowmul[rt] = a.scale_log2;
            qbias[rt] = 0.0f;
        } else {
            float mx = 0.0f;
#pragma unroll
            for (int m = 0; m < C::KS; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    mx = fmaxf(mx, fmaxf(fabsf(bf16_to_f32(raw[m][e] & 0xffffu)), fabsf(bf16_to_f32(raw[m][e] >> 16))));
            mx = xor16_max(mx);
            int ex = 0;
            if (mx > 0.0f) (void)frexpf(mx, &ex);       // mx in [2^(ex-1), 2^ex)
            const int k = min(120, max(-120, 15 - ex));  // mx * 2^k in [2^14, 2^15)
            const float up = ldexpf(1.0f, k);
            float qs = 0.0f;
#pragma unroll
            for (int m = 0; m < C::KS; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const h2 v = {(_Float16)(bf16_to_f32(raw[m][e] & 0xffffu) * up),
                                  (_Float16)(bf16_to_f32(raw[m][e] >> 16) * up)};
                    qb[rt][m][e] = __builtin_bit_cast(uint32_t, v);
                    qs += (float)v.x + (float)v.y;
                }
            qbias[rt] = 1152.0f * xor16_sum(qs);
            rowmul[rt] = ldexpf(a.scale_log2, -k);
        }
    }
    causal = __any(causal);

    int blk0 = 0;  // first page of the current range's block-table slice

    // softmax state per row (lane column n), lazily rescaled: m_ref only moves when a block's max
    // exceeds it by more than 8 (weights stay <= 2^8), s_ref when a V scale exceeds 16x it.
    float m_ref[RT], l_run[RT];
    f4 acc[RT][C::DT];
    f4 pacc[RT];  // per-row sums of the fp16 weights, to remove the 1152 code bias
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m_ref[rt] = -INFINITY;
        l_run[rt] = 0.0f;
        pacc[rt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) acc[rt][dt] = f4{0.f, 0.f, 0.f, 0.f};
    }
    float s_ref = MODE == 2 ? 1.0f : 0.0f;

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v);
    const int rho = lane & 15;
    const int kg = lane >> 4;
    const int64_t page_bytes = (int64_t)a.hkv * a.bs * D * C::ESZ;  // one physical block, all heads
    const int64_t head_bytes = (int64_t)h * a.bs * D * C::ESZ;
    const int krow_off = 8 * (rho >> 2) + (rho & 3);                 // score tile u adds 4u
    // bf16 pages: lane group kg holds channels 32m + 8kg .. of k-step m (bytes 64m + 16kg ..), so
    // the four lane groups of a row read 64 contiguous bytes per load; int8 pages: 32 bytes
    // (channels kg*32 ..) per lane group
    const int k_lane_bytes = MODE == 2 ? kg * 16 : kg * C::KB;
    constexpr int K_LOAD_STRIDE = MODE == 2 ? 64 : 16;
    const int v_lane_bytes = n * kVTile * C::ESZ;                    // channel n of each 16-channel tile

    auto load_block = [&](int T, BlockRegs<D, MODE>& R) {
        {
            int t = T + krow_off;  // keys t and t + 4 share a page (same 8-key group)
            if (t >= t_end) t = t_begin;  // in-bounds stand-in, masked later
            const uint8_t* kp = kbase + (int64_t)bt_s[(t >> a.log2bs) - blk0] * page_bytes + head_bytes +
                                (t & (a.bs - 1)) * (D * C::ESZ) + k_lane_bytes;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                int tu = T + krow_off + 4 * u;
                const uint8_t* kpu = (tu < t_end) ? kp + u * 4 * D * C::ESZ : kp;
#pragma unroll
                for (int l = 0; l < C::KL; ++l) R.k[u][l] = load16(kpu + K_LOAD_STRIDE * l);
            }
        }
        int t0 = T + 8 * g;
        if (t0 >= t_end) t0 = t_begin;
        const int64_t bt0 = bt_s[(t0 >> a.log2bs) - blk0];
        const int slot0 = t0 & (a.bs - 1);
        const uint8_t* vp = vbase + bt0 * page_bytes + head_bytes + v_lane_bytes +
                            ((slot0 / kVTile) * D * kVTile + slot0 % kVTile) * C::ESZ;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            const uint8_t* vpd = vp + dt * 16 * kVTile * C::ESZ;
            if constexpr (C::VW == 2) {
                const uint2 w = *reinterpret_cast<const uint2*>(vpd);
                R.v[dt][0] = w.x; R.v[dt][1] = w.y;
            } else {
                const uint4 w = *reinterpret_cast<const uint4*>(vpd);
                R.v[dt][0] = w.x; R.v[dt][1] = w.y; R.v[dt][2] = w.z; R.v[dt][3] = w.w;
            }
        }
        const int64_t sidx = (bt0 * a.hkv + h) * a.bs + slot0;
        if constexpr (MODE == 0) {
            const float4* kq = reinterpret_cast<const float4*>(a.ks + sidx);
            const float4* vq = reinterpret_cast<const float4*>(a.vs + sidx);
            const float4 k0 = kq[0], k1 = kq[1], v0 = vq[0], v1 = vq[1];
            R.ks[0] = k0.x; R.ks[1] = k0.y; R.ks[2] = k0.z; R.ks[3] = k0.w;
            R.ks[4] = k1.x; R.ks[5] = k1.y; R.ks[6] = k1.z; R.ks[7] = k1.w;
            R.vs[0] = v0.x; R.vs[1] = v0.y; R.vs[2] = v0.z; R.vs[3] = v0.w;
            R.vs[4] = v1.x; R.vs[5] = v1.y; R.vs[6] = v1.z; R.vs[7] = v1.w;
        } else if constexpr (MODE == 1) {
            const float kk = a.ks[bt0 * a.hkv + h], vv = a.vs[bt0 * a.hkv + h];
#pragma unroll
            for (int e = 0; e < 8; ++e) { R.ks[e] = kk; R.vs[e] = vv; }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) { R.ks[e] = 1.0f; R.vs[e] = 1.0f; }
        }
    };

    // One 32-key block on registers R (loaded one block earlier).
    auto process = [&](int T, const BlockRegs<D, MODE>& R) {
        // masked: the block runs past the split's keys, past a row's causal limit or below a row's
        // window start (the group's last row has the largest)
        const bool MASKED = causal || T + BLK > t_end || T < lo_hi;
        // -------------------------------------------- scores: two 16-key tiles per row tile
        f4 sc[RT][2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sc[rt][u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < C::KS; ++m) {
                if constexpr (MODE == 2) {
                    const u32x4 w = R.k[u][m];  // 8 bf16 = one 16-byte load per k-step
                    const uint32_t r[4] = {w.x, w.y, w.z, w.w};
                    const b8 av = __builtin_bit_cast(b8, r);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        sc[rt][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av, __builtin_bit_cast(b8, qb[rt][m]), sc[rt][u], 0, 0, 0);
                } else {
                    const u32x4 w = R.k[u][m / 2];  // 8 codes per k-step: dwords (2m, 2m+1)
                    const h8 av = (m & 1) ? biased_h8(w.z, w.w) : biased_h8(w.x, w.y);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        sc[rt][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            av, __builtin_bit_cast(h8, qb[rt][m]), sc[rt][u], 0, 0, 0);
                }
            }
        }

        // -------------------------------------------- scores in log2 units
        float sv[RT][8];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float raw = sc[rt][e >> 2][e & 3] - qbias[rt];
                sv[rt][e] = raw * (R.ks[e] * rowmul[rt]);
            }
        float vs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vs[e] = R.vs[e];
        // -------------------------------------------- the mask, one scalar branch for the whole block:
        //      hidden keys score -inf; slots past the keys may never have been written, so their
        //      scales (and bf16 values) must not reach a weight or the V-scale reference
        uint32_t vcode[C::DT][C::VW];  // this block's V operand words (bf16: cleared past the keys)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int i = 0; i < C::VW; ++i) vcode[dt][i] = R.v[dt][i];
        if (MASKED) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = T + 8 * g + e;
                if (!(t < t_end)) vs[e] = 0.0f;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    if (!(t < t_end && t <= lim[rt] && t >= lo[rt])) sv[rt][e] = -INFINITY;
            }
            if constexpr (MODE == 2) {  // the lane's 8 keys, two per dword of each channel's V
                const int tk = T + 8 * g;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const uint32_t keep = tk + 2 * e2 + 1 < t_end ? ~0u : (tk + 2 * e2 < t_end ? 0xffffu : 0u);
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt) vcode[dt][e2] &= keep;
                }
            }
        }

        // -------------------------------------------- V-scale reference
        float sf = 1.0f;
        bool s_moved = false;
        float vscale[8];
        if constexpr (MODE != 2) {
            float vmax = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) vmax = fmaxf(vmax, vs[e]);
            vmax = xor16_max(vmax);
            if (vmax > 16.0f * s_ref) {  // (also the first block: s_ref == 0)
                sf = s_ref > 0.0f ? s_ref * __builtin_amdgcn_rcpf(vmax) : 0.0f;
                s_ref = vmax;
                s_moved = true;
            }
            const float inv = s_ref > 0.0f ? __builtin_amdgcn_rcpf(s_ref) : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) vscale[e] = vs[e] * inv;
        }

        // -------------------------------------------- online softmax, P operand
        uint32_t pa[RT][4];
        float factor[RT];
        bool any_rescale = s_moved;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float bmax = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) bmax = fmaxf(bmax, sv[rt][e]);
            bmax = xor16_max(bmax);
            float alpha = 1.0f;
            if (bmax > m_ref[rt] + 8.0f) {  // (also the first block: m_ref == -inf)
                alpha = __builtin_amdgcn_exp2f(m_ref[rt] - bmax);
                m_ref[rt] = bmax;
            }
            // a row with no visible key yet keeps m_ref = -inf; its weights are taken against 0, so
            // that its hidden keys (-inf) weigh exactly 0
            const float mref = m_ref[rt] == -INFINITY ? 0.0f : m_ref[rt];
            float p[8];
            float psum = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(sv[rt][e] - mref);
                psum += p[e];
            }
            psum = xor16_sum(psum);
            l_run[rt] = l_run[rt] * alpha + psum;
            factor[rt] = alpha * sf;
            any_rescale |= alpha != 1.0f;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                if constexpr (MODE == 2) {
                    pa[rt][e2] = f32_to_bf16_rne(p[2 * e2]) | (f32_to_bf16_rne(p[2 * e2 + 1]) << 16);
                } else {
                    const h2 w = {(_Float16)(p[2 * e2] * vscale[2 * e2]), (_Float16)(p[2 * e2 + 1] * vscale[2 * e2 + 1])};
                    pa[rt][e2] = __builtin_bit_cast(uint32_t, w);
                }
            }
        }

        // -------------------------------------------- rescale rows whose reference moved
        if (__any(any_rescale)) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float f = __shfl(factor[rt], 4 * g + i, kWave);  // factor of row 4g+i
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt) acc[rt][dt][i] *= f;
                    pacc[rt][i] *= f;
                }
            }
        }

        // -------------------------------------------- P.V over the 32 keys (+ the weight sums)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            if constexpr (MODE == 2) {
                const uint32_t r[4] = {vcode[dt][0], vcode[dt][1], vcode[dt][2], vcode[dt][3]};
                const b8 bv = __builtin_bit_cast(b8, r);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, pa[rt]), bv,
                                                                          acc[rt][dt], 0, 0, 0);
            } else {
                const h8 bv = biased_h8(vcode[dt][0], vcode[dt][1]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, pa[rt]), bv,
                                                                         acc[rt][dt], 0, 0, 0);
            }
        }
        if constexpr (MODE != 2) {
            const uint32_t ones[4] = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};  // fp16 1.0
            const h8 bo = __builtin_bit_cast(h8, ones);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                pacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, pa[rt]), bo, pacc[rt], 0, 0, 0);
        }
    };

    // Two register sets, alternating: the loads of block k+1 stay in flight while block k computes,
    // and no register set is ever copied (a copy would wait for those loads).  Loads past the
    // split's last block read the in-bounds stand-in, so every iteration issues the same loads.
    for (int tb = t_seg0; tb < t_seg1; tb += MAX_SPLIT) {
        t_begin = tb;
        t_end = min(tb + MAX_SPLIT, t_seg1);
        if (tb != t_seg0) __builtin_amdgcn_wave_barrier();  // the previous range's LDS reads are done
        // block-table slice of the range (the wave reads back its own LDS writes in order)
        blk0 = t_begin >> a.log2bs;
        const int nblk = ((t_end - 1) >> a.log2bs) - blk0 + 1;
        for (int i = lane; i < nblk; i += kWave) bt_s[i] = a.bt[(int64_t)b * a.mbs + blk0 + i];
        __builtin_amdgcn_wave_barrier();

        BlockRegs<D, MODE> ra, rb;
        load_block(t_begin, ra);
        for (int T = t_begin;;) {
            load_block(T + BLK, rb);
            process(T, ra);
            T += BLK;
            if (T >= t_end) break;
            load_block(T + BLK, ra);
            process(T, rb);
            T += BLK;
            if (T >= t_end) break;
        }
    }

    // ---- normalise and write: lane (channel n, group g) holds rows 4g+i of every channel tile
    const bool split_mode = pslot >= 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = rt * 16 + 4 * g + i;  // row within the group
            const float l = __shfl(l_run[rt], 4 * g + i, kWave);
            const float m = __shfl(m_ref[rt], 4 * g + i, kWave);
            if (j >= nvalid) continue;
            const float mul = l > 0.0f ? s_ref / l : 0.0f;
            const float bias = MODE == 2 ? 0.0f : 1152.0f * pacc[rt][i];
            const int r = r0 + j;
            const int64_t orow = (int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g;
            const int64_t prow = pslot * a.prs + j;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                const float o = (acc[rt][dt][i] - bias) * mul;
                const int d = dt * 16 + n;
                if (!split_mode) a.out[orow * D + d] = (uint16_t)f32_to_bf16_rne(o);
                else a.part_o[prow * D + d] = o;
            }
            if (n == 0) {
                const float lse2 = l > 0.0f ? m + log2f(l) : -INFINITY;
                if (!split_mode) {
                    if (a.lse) a.lse[orow] = lse2 * kLn2;
                } else {
                    a.part_lse[prow] = lse2;
                }
            }
        }
    }
}

// Fixed splits: one wave per (item, split of split_len keys), splits fastest.
template <int D, int MODE, int RT>
__global__ __launch_bounds__(64) void decode_mfma_kernel(DecodeArgs a) {
    __shared__ int bt_s[MAX_SPLIT_BLOCKS];
    const int s = blockIdx.x % a.nsplit;
    const int item = blockIdx.x / a.nsplit;
    const ItemGeo it = item_geo<16 * RT>(a, item);
    if (it.nvalid <= 0) return;
    if (it.kmax <= 0) {  // inactive sequence: zero output, lse = -inf
        if (s == 0) zero_rows<D>(a, it, threadIdx.x);
        return;
    }
    const int t_begin = win_begin(a.window, it.prior + it.r0 / a.g) + s * a.split_len;  // (sliding window)
    if (t_begin >= it.kmax) return;
    mfma_segment<D, MODE, RT>(a, it.b, it.h, item % a.nrg, t_begin, min(t_begin + a.split_len, it.kmax),
                              a.nsplit > 1 ? (int64_t)item * a.nsplit + s : -1, bt_s);
}

// Balanced partition (sk_partition.h): one wave per segment of the plan, planned over several
// rounds of the waves the GPU holds when the items are many.
template <int D, int MODE, int RT, bool WIN>
__global__ __launch_bounds__(64) void decode_mfma_sk_kernel(DecodeArgs a, int batch) {
    __shared__ int bt_s[MAX_SPLIT_BLOCKS];
    extern __shared__ int kseq[];  // [batch + 1] prefix sums over sequences of their waves
    SkSegment sg;
    if (!sk_plan<16 * RT, WIN>(a, batch, blockIdx.x, kseq, sg)) return;
    mfma_segment<D, MODE, RT>(a, sg.it.b, sg.it.h, sg.it.r0 / (16 * RT), sg.t0, sg.t1, sg.pslot, bt_s);
}

template <int D, int MODE, int RT>
hipError_t launch_one(const DecodeArgs& a, int batch, hipStream_t stream) {
    const int64_t items = (int64_t)batch * a.hkv * a.nrg;
    if (a.sk_waves > 0) {  // balanced partition (bf16 pages, one row tile)
        if constexpr (MODE == 2 && RT == 1) {
            if (items == 0) return hipSuccess;
            if (batch > SK_MAX_SEQS || a.sk_waves + items > 0x7fffffff) return hipErrorInvalidValue;
            const size_t lds = (size_t)(batch + 1) * sizeof(int);
            if (a.window > 0)
                hipLaunchKernelGGL((decode_mfma_sk_kernel<D, MODE, RT, true>), dim3((unsigned)(a.sk_waves + items)),
                                   dim3(64), lds, stream, a, batch);
            else
                hipLaunchKernelGGL((decode_mfma_sk_kernel<D, MODE, RT, false>), dim3((unsigned)(a.sk_waves + items)),
                                   dim3(64), lds, stream, a, batch);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            constexpr int ROWS = 16 * RT;
            return launch_merge_sk<D, ROWS>(a, items, stream);
        } else {
            return hipErrorInvalidValue;
        }
    }
    const int64_t grid = items * a.nsplit;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_mfma_kernel<D, MODE, RT>), dim3((unsigned)grid), dim3(64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_merge(a, batch, D, 16 * RT, stream);
}

template <int D, int MODE>
hipError_t launch_rt(const DecodeArgs& a, int batch, int rt, hipStream_t stream) {
    switch (rt) {
        case 1: return launch_one<D, MODE, 1>(a, batch, stream);
        case 2: return launch_one<D, MODE, 2>(a, batch, stream);
        case 3: if constexpr (D == 64) return launch_one<D, MODE, 3>(a, batch, stream);
                return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_mode(const DecodeArgs& a, int batch, int rt, int mode, hipStream_t stream) {
    switch (mode) {
        case 0: return launch_rt<D, 0>(a, batch, rt, stream);
        case 1: return launch_rt<D, 1>(a, batch, rt, stream);
        case 2: return launch_rt<D, 2>(a, batch, rt, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Waves of the balanced bf16 kernel one compute unit holds (bf16 pages, one row tile).
int decode_mfma_waves_per_cu(int head_dim, int row_tiles, int mode, int batch, bool windowed) {
    if (batch > SK_MAX_SEQS || row_tiles != 1 || mode != 2 || (head_dim != 64 && head_dim != 128)) return 0;
    const size_t lds = (size_t)(batch + 1) * sizeof(int);
    int per_cu = 0;
    hipError_t e;
    if (head_dim == 64)
        e = windowed ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma_sk_kernel<64, 2, 1, true>, 64, lds)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma_sk_kernel<64, 2, 1, false>, 64, lds);
    else
        e = windowed ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma_sk_kernel<128, 2, 1, true>, 64, lds)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_mfma_sk_kernel<128, 2, 1, false>, 64, lds);
    return e == hipSuccess && per_cu > 0 ? per_cu : 0;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int batch, int head_dim, int row_tiles, int mode,
                              hipStream_t stream) {
    if (a.split_len > MAX_SPLIT || (a.split_len % 128) != 0) return hipErrorInvalidValue;
    if (head_dim == 64) return launch_mode<64>(a, batch, row_tiles, mode, stream);
    if (head_dim == 128) return launch_mode<128>(a, batch, row_tiles, mode, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
