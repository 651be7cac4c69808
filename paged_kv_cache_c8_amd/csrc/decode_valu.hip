// decode_valu.hip - split-KV grouped-query attention over the paged int8 / bf16 cache (gfx950).
//
// Computes MojoPagedDecodeGQA (Mojo Opset README, Op List) directly on the quantized pages:
// out = softmax(scale * q K^T) V with K, V dequantized in registers.  Work is split
// flash-decoding style: one workgroup (4 waves) per (sequence, KV head, row group, key split);
// when a row group's keys span several splits, a second kernel merges the partials with a
// log-sum-exp reduction (the kernel boundary makes every XCD's partials visible; a device-wide
// fence per workgroup instead would write back each XCD's L2 thousands of times).
//
// Rows.  A KV head serves G query heads; a chunk of q_len new queries gives q_len * G rows
// r = i * G + g (query i, head g).  Rows are processed RG at a time; row r may see keys
// 0 .. prior + i (causal).  Plain decode is q_len = 1, RG = G (up to 8).
//
// Per 128-key chunk (the next chunk's K, V and scales are already in flight):
//   1. scores: 8 (int8, head_dim 128) or 16 (bf16) lanes share one key row, each holding 16
//      contiguous bytes of the token-major K page.  int8 codes become fp16 pairs exactly (byte
//      permute into 0x64xx, i.e. 1024 + code + 128, then subtract 1152) and meet fp16 query pairs
//      in v_dot2_f32_f16 (fp32 accumulation); the query row is pre-scaled by a power of two so its
//      bf16 values sit in fp16's normal range.  bf16 pages use v_dot2_f32_bf16 on the raw pairs.
//      The per-row partials are folded across the lanes by a butterfly reduce-scatter on DPP; the
//      per-token K scale is applied once per dot product.  Scores go to LDS in log2 units.
//   2. softmax: one wave per row (two when RG = 8) takes the chunk max, rescales the running
//      sum, and writes the weights of token pairs to LDS: p * s_v / S (fp16; S = the chunk's
//      largest V scale, applied later in fp32) or p (bf16 pages).
//   3. P.V: each thread owns NU channels of one token group.  The channel-major V tiles give 16
//      (8 bf16) consecutive tokens of one channel per 16-byte load, i.e. token pairs for dot2;
//      the pair weights are LDS broadcasts shared by the NU channels.
// At the end the token groups' accumulators are summed through LDS.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr int CH = 128;            // keys per chunk
constexpr int RED_FLOATS = 8192;   // LDS floats for the final cross-group reduction
constexpr int MAX_SPLIT = 4096;    // keys per split (planner limit)
constexpr int MAX_SPLIT_BLOCKS = MAX_SPLIT / 16;

template <int D, int RG, int MODE>
struct Cfg {
    static constexpr int ESZ = MODE == 2 ? 2 : 1;
    static constexpr int LPT = D * ESZ / 16;   // lanes per key row
    static constexpr int EPL = 16 / ESZ;       // values per lane in the score phase
    static constexpr int TPP = 256 / LPT;      // keys per score pass
    static constexpr int NPASS = CH / TPP;
    static constexpr int TPU = 16 / ESZ;       // keys per V unit (16 bytes of one channel)
    static constexpr int NTG = CH / TPU;       // token groups per chunk
    static constexpr int TPT = 256 / NTG;      // threads per token group
    static constexpr int NU = D / TPT;         // channels per thread in P.V
    static constexpr int SCW = TPU * RG + 4;   // score floats per token group (padded)
    static constexpr int PWW = (TPU / 2) * RG + 4;  // pair-weight dwords per token group (padded)
    static constexpr int RPR = (RED_FLOATS / (NTG * D)) < RG ? (RED_FLOATS / (NTG * D)) : RG;
    static constexpr int HELD = RG >= LPT ? RG / LPT : 1;  // rows held per lane after the fold
    static_assert(LPT <= 16, "a key row must fit in one DPP row");
    static_assert(NU >= 1 && D % TPT == 0, "channel split");
    static_assert(RG % RPR == 0, "reduction rounds");
};

__device__ __forceinline__ int sc_index(int tl, int j, int rg, int tpu, int scw) {
    return (tl / tpu) * scw + (tl % tpu) * rg + j;
}

// four int8 codes -> two fp16 pairs, exactly: (code0, code1), (code2, code3)
__device__ __forceinline__ void codes_to_h2(uint32_t w, h2& lo, h2& hi) {
    const uint32_t u = w ^ 0x80808080u;  // code + 128 as an unsigned byte
    const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
    const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = __builtin_bit_cast(h2, a) - bias;
    hi = __builtin_bit_cast(h2, b) - bias;
}

template <int S>
__device__ __forceinline__ float xchg_s(float x) {
    return lane_xchg<S>(x);
}

// Butterfly reduce-scatter of RG partial sums over LPT lanes.  On return lane c holds
// complete sums in v[0 .. HELD): rows c*HELD + k when RG >= LPT, else row c / (LPT / RG).
template <int RG, int LPT>
__device__ __forceinline__ void fold_rows(float (&v)[RG], int c) {
    int n = RG;
#pragma unroll
    for (int s = LPT / 2; s >= 1; s >>= 1) {
        const bool upper = (c & s) != 0;
        if (n > 1) {
            const int half = n / 2;
#pragma unroll
            for (int i = 0; i < RG / 2; ++i) {
                if (i < half) {
                    const float send = upper ? v[i] : v[half + i];
                    const float keep = upper ? v[half + i] : v[i];
                    float recv;
                    if (s == 8) recv = xchg_s<8>(send);
                    else if (s == 4) recv = xchg_s<4>(send);
                    else if (s == 2) recv = xchg_s<2>(send);
                    else recv = xchg_s<1>(send);
                    v[i] = keep + recv;
                }
            }
            n = half;
        } else {
            float recv;
            if (s == 8) recv = xchg_s<8>(v[0]);
            else if (s == 4) recv = xchg_s<4>(v[0]);
            else if (s == 2) recv = xchg_s<2>(v[0]);
            else recv = xchg_s<1>(v[0]);
            v[0] += recv;
        }
    }
}

// Registers of one chunk, loaded one chunk ahead.
template <int NPASS, int NU>
struct ChunkRegs {
    u32x4 k[NPASS];
    float ks[NPASS];
    u32x4 v[NU];
    float vs[2];  // V scales of the softmax lane's token pair
};

template <int D, int RG, int MODE>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
    using C = Cfg<D, RG, MODE>;
    __shared__ __attribute__((aligned(16))) float sc[C::NTG * C::SCW];
    __shared__ __attribute__((aligned(16))) uint32_t pw[C::NTG * C::PWW];
    __shared__ __attribute__((aligned(16))) float red[RED_FLOATS];
    __shared__ int bt_s[MAX_SPLIT_BLOCKS];
    __shared__ float row_alpha[RG], row_m[RG], row_l[RG];
    __shared__ float chunk_vscale;

    const int tid = threadIdx.x;
    int wi = blockIdx.x;
    const int s = wi % a.nsplit;
    wi /= a.nsplit;
    const int item = wi;  // (sequence, KV head, row group)
    const int rg = wi % a.nrg;
    wi /= a.nrg;
    const int h = wi % a.hkv;
    const int b = wi / a.hkv;

    const int qlen = a.cu ? a.cu[b + 1] - a.cu[b] : 1;
    const int qrow0 = a.cu ? a.cu[b] : b;
    const int ctx = a.ctx[b];
    const int prior = ctx - qlen;
    const int nrows = qlen * a.g;
    const int r0 = rg * RG;
    if (r0 >= nrows) return;
    const int nvalid = min(RG, nrows - r0);
    const int kmax = prior + (r0 + nvalid - 1) / a.g + 1;  // keys the group's last row needs
    const int t_begin = win_begin(a.window, prior + r0 / a.g) + s * a.split_len;  // (sliding window)

    if (kmax <= 0) {  // no keys at all (inactive sequence): zero output, lse = -inf
        if (s == 0) {
            for (int o = tid; o < nvalid * D; o += blockDim.x) {
                const int j = o / D, d = o % D;
                const int r = r0 + j;
                const int64_t orow = (int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g;
                a.out[orow * D + d] = 0;
                if (d == 0 && a.lse) a.lse[orow] = -INFINITY;
            }
        }
        return;
    }
    if (t_begin >= kmax) return;
    const int t_end = min(t_begin + a.split_len, kmax);

    // ---- block-table slice of this split
    const int blk0 = t_begin >> a.log2bs;
    const int nblk = ((t_end - 1) >> a.log2bs) - blk0 + 1;
    for (int i = tid; i < nblk; i += blockDim.x) bt_s[i] = a.bt[(int64_t)b * a.mbs + blk0 + i];

    // ---- query rows: this lane's channel slice as fp16 (int8 pages) or bf16 (bf16 pages) pairs
    const int c = tid % C::LPT;
    constexpr int NP = C::EPL / 2;  // pairs per lane
    uint32_t q2[RG][NP];
    float held_mul[C::HELD];  // per held row: 2^-k * scale * log2(e)
    {
        float rowmul[RG];
#pragma unroll
        for (int j = 0; j < RG; ++j) {
            uint32_t raw[NP];
            if (j < nvalid) {
                const int r = r0 + j;
                const uint16_t* qp =
                    a.q + ((int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g) * D + c * C::EPL;
#pragma unroll
                for (int e4 = 0; e4 < NP / 4; ++e4) {
                    const u32x4 w = load16(qp + e4 * 8);
                    raw[e4 * 4 + 0] = w.x; raw[e4 * 4 + 1] = w.y; raw[e4 * 4 + 2] = w.z; raw[e4 * 4 + 3] = w.w;
                }
            } else {
#pragma unroll
                for (int p = 0; p < NP; ++p) raw[p] = 0;
            }
            if constexpr (MODE == 2) {
#pragma unroll
                for (int p = 0; p < NP; ++p) q2[j][p] = raw[p];
                rowmul[j] = a.scale_log2;
            } else {
                float mx = 0.0f;
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    mx = fmaxf(mx, fmaxf(fabsf(bf16_to_f32(raw[p] & 0xffffu)), fabsf(bf16_to_f32(raw[p] >> 16))));
                mx = group_max<C::LPT>(mx);
                int e = 0;
                if (mx > 0.0f) (void)frexpf(mx, &e);  // mx in [2^(e-1), 2^e)
                // mx * 2^k in [2^14, 2^15); the clamp keeps 2^k and 2^-k * scale finite fp32
                const int k = min(120, max(-120, 15 - e));
                const float up = ldexpf(1.0f, k);
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const h2 v = {(_Float16)(bf16_to_f32(raw[p] & 0xffffu) * up),
                                  (_Float16)(bf16_to_f32(raw[p] >> 16) * up)};
                    q2[j][p] = __builtin_bit_cast(uint32_t, v);
                }
                rowmul[j] = ldexpf(a.scale_log2, -k);
            }
        }
#pragma unroll
        for (int k = 0; k < C::HELD; ++k) {
            if constexpr (RG >= C::LPT) held_mul[k] = rowmul[c * C::HELD + k];
            else held_mul[k] = rowmul[c / (C::LPT / RG)];
        }
    }

    // softmax state: wave w owns rows w and w + 4 (uniform across the wave)
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.0f, 0.0f};

    float acc[RG][C::NU];
#pragma unroll
    for (int j = 0; j < RG; ++j)
#pragma unroll
        for (int k = 0; k < C::NU; ++k) acc[j][k] = 0.0f;

    // P.V thread mapping: consecutive threads take consecutive 16-byte segments of a page's channel
    // (one per 16-slot V tile), then the next channel.
    const int seg_per_row = a.bs / C::TPU;
    const int pv_seg = tid % seg_per_row;
    const int pv_dl = (tid / seg_per_row) % C::TPT;
    const int pv_pic = tid / (seg_per_row * C::TPT);  // page within the chunk
    const int pv_tg = pv_pic * seg_per_row + pv_seg;

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v);
    const int64_t head_pages = (int64_t)a.hkv;

    __syncthreads();  // bt_s ready

    // Issue the loads of chunk cb.  Lanes whose key lies past the split read the split's first key
    // instead (always valid) and are masked later, so every load is unconditional and in bounds.
    auto load_chunk = [&](int cb, ChunkRegs<C::NPASS, C::NU>& R) {
#pragma unroll
        for (int pass = 0; pass < C::NPASS; ++pass) {
            int t = cb + pass * C::TPP + tid / C::LPT;
            if (t >= t_end) t = t_begin;
            const int64_t page = (int64_t)bt_s[(t >> a.log2bs) - blk0] * head_pages + h;
            const int off = t & (a.bs - 1);
            R.k[pass] = load16(kbase + ((page * a.bs + off) * D) * C::ESZ + c * 16);
            if constexpr (MODE == 0) R.ks[pass] = a.ks[page * a.bs + off];
            else if constexpr (MODE == 1) R.ks[pass] = a.ks[page];
            else R.ks[pass] = 1.0f;
        }
        {
            int t0 = cb + pv_pic * a.bs + pv_seg * C::TPU;
            if (t0 >= t_end) t0 = t_begin;
            const int64_t page = (int64_t)bt_s[(t0 >> a.log2bs) - blk0] * head_pages + h;
            const int seg = (t0 & (a.bs - 1)) / C::TPU;
#pragma unroll
            for (int k = 0; k < C::NU; ++k) {
                const int d = pv_dl + k * C::TPT;
                R.v[k] = load16(vbase + v_elem(page, D, a.bs, d, seg * C::TPU) * C::ESZ);
            }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            int t = cb + 2 * lane + e;
            if (t >= t_end) t = t_begin;
            const int64_t page = (int64_t)bt_s[(t >> a.log2bs) - blk0] * head_pages + h;
            if constexpr (MODE == 0) R.vs[e] = a.vs[page * a.bs + (t & (a.bs - 1))];
            else if constexpr (MODE == 1) R.vs[e] = a.vs[page];
            else R.vs[e] = 1.0f;
        }
    };

    ChunkRegs<C::NPASS, C::NU> cur, nxt;
    load_chunk(t_begin, cur);

    for (int cb = t_begin; cb < t_end; cb += CH) {
        if (cb + CH < t_end) load_chunk(cb + CH, nxt);

        // ------------------------------------------------------------------ 1. scores
#pragma unroll
        for (int pass = 0; pass < C::NPASS; ++pass) {
            const int tl = pass * C::TPP + tid / C::LPT;
            const int t = cb + tl;
            float part[RG];
#pragma unroll
            for (int j = 0; j < RG; ++j) part[j] = 0.0f;
            const u32x4 kw = cur.k[pass];
            if constexpr (MODE == 2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const b2 kb = __builtin_bit_cast(b2, word(kw, i));
#pragma unroll
                    for (int j = 0; j < RG; ++j)
                        part[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, q2[j][i]), kb, part[j], false);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h2 lo, hi;
                    codes_to_h2(word(kw, i), lo, hi);
#pragma unroll
                    for (int j = 0; j < RG; ++j) {
                        part[j] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, q2[j][2 * i]), lo, part[j], false);
                        part[j] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, q2[j][2 * i + 1]), hi, part[j], false);
                    }
                }
            }
            fold_rows<RG, C::LPT>(part, c);
            const bool valid = t < t_end;
            const float ks = cur.ks[pass];
            if constexpr (RG >= C::LPT) {
#pragma unroll
                for (int k = 0; k < C::HELD; ++k) {
                    const int j = c * C::HELD + k;
                    const int lim = prior + (r0 + j) / a.g;
                    const bool seen = t <= lim && t >= win_lo(a.window, lim);
                    const float v = (valid && j < nvalid && seen) ? part[k] * ks * held_mul[k] : -INFINITY;
                    sc[sc_index(tl, j, RG, C::TPU, C::SCW)] = v;
                }
            } else {
                constexpr int DUP = C::LPT / RG;
                if (c % DUP == 0) {
                    const int j = c / DUP;
                    const int lim = prior + (r0 + j) / a.g;
                    const bool seen = t <= lim && t >= win_lo(a.window, lim);
                    const float v = (valid && j < nvalid && seen) ? part[0] * ks * held_mul[0] : -INFINITY;
                    sc[sc_index(tl, j, RG, C::TPU, C::SCW)] = v;
                }
            }
        }
        __syncthreads();

        // ------------------------------------------------------------------ 2. softmax
        {
            const int tl0 = 2 * lane;
            const bool v0 = cb + tl0 < t_end, v1 = cb + tl0 + 1 < t_end;
            float vmax = 1.0f, inv = 1.0f;
            if constexpr (MODE != 2) {
                vmax = fmaxf(v0 ? cur.vs[0] : 0.0f, v1 ? cur.vs[1] : 0.0f);
                vmax = group_max<kWave>(vmax);
                inv = vmax > 0.0f ? 1.0f / vmax : 0.0f;
                if (tid == 0) chunk_vscale = vmax;
            }
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int j = wave + 4 * rr;
                if (j < RG) {
                    const float s0 = sc[sc_index(tl0, j, RG, C::TPU, C::SCW)];
                    const float s1 = sc[sc_index(tl0 + 1, j, RG, C::TPU, C::SCW)];
                    const float cmax = group_max<kWave>(fmaxf(s0, s1));
                    const float m_new = fmaxf(m_run[rr], cmax);
                    const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run[rr] - m_new);
                    const float p0 = (s0 == -INFINITY) ? 0.0f : exp2f(s0 - m_new);
                    const float p1 = (s1 == -INFINITY) ? 0.0f : exp2f(s1 - m_new);
                    const float psum = group_sum<kWave>(p0 + p1);
                    l_run[rr] = l_run[rr] * alpha + psum;
                    m_run[rr] = m_new;
                    uint32_t packed;
                    if constexpr (MODE == 2) {
                        packed = f32_to_bf16_rne(p0) | (f32_to_bf16_rne(p1) << 16);
                    } else {
                        const h2 wv = {(_Float16)(p0 * (cur.vs[0] * inv)), (_Float16)(p1 * (cur.vs[1] * inv))};
                        packed = __builtin_bit_cast(uint32_t, wv);
                    }
                    pw[(tl0 / C::TPU) * C::PWW + ((tl0 % C::TPU) / 2) * RG + j] = packed;
                    if (lane == 0) row_alpha[j] = alpha;
                }
            }
        }
        __syncthreads();

        // ------------------------------------------------------------------ 3. P.V
        {
            float alpha[RG];
#pragma unroll
            for (int j = 0; j < RG; ++j) alpha[j] = row_alpha[j];
            const float cs = MODE == 2 ? 1.0f : chunk_vscale;
            float part[RG][C::NU];
#pragma unroll
            for (int j = 0; j < RG; ++j)
#pragma unroll
                for (int k = 0; k < C::NU; ++k) part[j][k] = 0.0f;
            const int tok0 = cb + pv_pic * a.bs + pv_seg * C::TPU;
            const uint32_t* wrow = pw + pv_tg * C::PWW;
#pragma unroll
            for (int i = 0; i < 4; ++i) {  // dword i of each unit: tokens 4i .. 4i+3 (int8) / 2i, 2i+1 (bf16)
                constexpr int PPD = MODE == 2 ? 1 : 2;  // token pairs per dword
                uint32_t vp[C::NU][PPD];
#pragma unroll
                for (int k = 0; k < C::NU; ++k) {
                    if constexpr (MODE == 2) {
                        uint32_t vv = word(cur.v[k], i);
                        // bf16 slots past the keys may hold any bit pattern: zero them
                        const int tk = tok0 + 2 * i;
                        if (tk >= t_end) vv = 0;
                        else if (tk + 1 >= t_end) vv &= 0xffffu;
                        vp[k][0] = vv;
                    } else {
                        h2 lo, hi;
                        codes_to_h2(word(cur.v[k], i), lo, hi);
                        vp[k][0] = __builtin_bit_cast(uint32_t, lo);
                        vp[k][PPD - 1] = __builtin_bit_cast(uint32_t, hi);
                    }
                }
#pragma unroll
                for (int pp = 0; pp < PPD; ++pp) {
                    const int pair = i * PPD + pp;
                    uint32_t w[RG];
                    if constexpr (RG >= 4) {
#pragma unroll
                        for (int j4 = 0; j4 < RG; j4 += 4) {
                            const uint4 w4 = *reinterpret_cast<const uint4*>(wrow + pair * RG + j4);
                            w[j4] = w4.x; w[j4 + 1] = w4.y; w[j4 + 2] = w4.z; w[j4 + 3] = w4.w;
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < RG; ++j) w[j] = wrow[pair * RG + j];
                    }
#pragma unroll
                    for (int k = 0; k < C::NU; ++k) {
#pragma unroll
                        for (int j = 0; j < RG; ++j) {
                            if constexpr (MODE == 2)
                                part[j][k] = __builtin_amdgcn_fdot2_f32_bf16(
                                    __builtin_bit_cast(b2, w[j]), __builtin_bit_cast(b2, vp[k][pp]), part[j][k], false);
                            else
                                part[j][k] = __builtin_amdgcn_fdot2(
                                    __builtin_bit_cast(h2, w[j]), __builtin_bit_cast(h2, vp[k][pp]), part[j][k], false);
                        }
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < RG; ++j)
#pragma unroll
                for (int k = 0; k < C::NU; ++k) acc[j][k] = fmaf(cs, part[j][k], acc[j][k] * alpha[j]);
        }
        __syncthreads();
        cur = nxt;
    }

    // ---- publish the softmax state
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int j = wave + 4 * rr;
        if (j < RG && lane == 0) {
            row_m[j] = m_run[rr];
            row_l[j] = l_run[rr];
        }
    }

    const bool split_mode = a.nsplit > 1;
    const int64_t pbase = ((int64_t)item * a.nsplit + s) * a.prs;  // partial rows of this split

    // ---- sum the token groups' accumulators, RPR rows per round; write output or partials
#pragma unroll
    for (int j0 = 0; j0 < RG; j0 += C::RPR) {
#pragma unroll
        for (int jj = 0; jj < C::RPR; ++jj)
#pragma unroll
            for (int k = 0; k < C::NU; ++k)
                red[(pv_tg * C::RPR + jj) * D + pv_dl + k * C::TPT] = acc[j0 + jj][k];
        __syncthreads();
        for (int o = tid; o < C::RPR * D; o += blockDim.x) {
            const int jj = o / D, d = o % D;
            const int j = j0 + jj;
            float sum = 0.0f;
            for (int g2 = 0; g2 < C::NTG; ++g2) sum += red[(g2 * C::RPR + jj) * D + d];
            if (j < nvalid) {
                const float l = row_l[j];
                const float m = row_m[j];
                const float o_val = l > 0.0f ? sum / l : 0.0f;
                const float lse2 = l > 0.0f ? m + log2f(l) : -INFINITY;
                if (!split_mode) {
                    const int r = r0 + j;
                    const int64_t orow = (int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g;
                    a.out[orow * D + d] = (uint16_t)f32_to_bf16_rne(o_val);
                    if (d == 0 && a.lse) a.lse[orow] = lse2 * kLn2;
                } else {
                    a.part_o[(pbase + j) * D + d] = o_val;
                    if (d == 0) a.part_lse[pbase + j] = lse2;
                }
            }
        }
        __syncthreads();
    }
}

template <int D, int RG, int MODE>
hipError_t launch_one(const DecodeArgs& a, int batch, hipStream_t stream) {
    const int64_t items = (int64_t)batch * a.hkv * a.nrg;
    const int64_t grid = items * a.nsplit;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_valu_kernel<D, RG, MODE>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_merge(a, batch, D, RG, stream);
}

template <int D, int MODE>
hipError_t launch_rg(const DecodeArgs& a, int batch, int rg, hipStream_t stream) {
    switch (rg) {
        case 1: return launch_one<D, 1, MODE>(a, batch, stream);
        case 2: return launch_one<D, 2, MODE>(a, batch, stream);
        case 4: return launch_one<D, 4, MODE>(a, batch, stream);
        case 8: return launch_one<D, 8, MODE>(a, batch, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_mode(const DecodeArgs& a, int batch, int rg, int mode, hipStream_t stream) {
    switch (mode) {
        case 0: return launch_rg<D, 0>(a, batch, rg, stream);
        case 1: return launch_rg<D, 1>(a, batch, rg, stream);
        case 2: return launch_rg<D, 2>(a, batch, rg, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs& a, int batch, int head_dim, int rg, int mode,
                              hipStream_t stream) {
    if (a.split_len > MAX_SPLIT || (a.split_len % CH) != 0) return hipErrorInvalidValue;
    if (head_dim == 64) return launch_mode<64>(a, batch, rg, mode, stream);
    if (head_dim == 128) return launch_mode<128>(a, batch, rg, mode, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
