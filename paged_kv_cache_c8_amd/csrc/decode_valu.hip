// decode_valu.hip - split-KV grouped-query attention over the paged int8 / bf16 cache (gfx950).
//
// Computes MojoPagedDecodeGQA (Mojo Opset README, Op List) directly on the quantized pages:
// out = softmax(scale * q K^T) V with K, V dequantized in registers.  Work is split
// flash-decoding style: one workgroup (4 waves) per (sequence, KV head, row group, key split);
// the partials are combined by a log-sum-exp merge kernel (or written directly when one split
// covers the keys).
//
// Rows.  A KV head serves G query heads; a chunk of q_len new queries gives q_len * G rows
// r = i * G + g (query i, head g).  Rows are processed RG at a time; row r may see keys
// 0 .. prior + i (causal).  Plain decode is q_len = 1, RG = G (up to 8).
//
// Per 128-key chunk:
//   1. scores: 8 (int8, D=128) or 16 (bf16) lanes share one key row, each loading 16 contiguous
//      bytes of the token-major K page; the RG partial dot products are folded across those lanes
//      by a butterfly reduce-scatter on DPP, leaving each lane one (or more) complete rows.
//      The per-token K scale is applied once per dot product.  Scores go to LDS in log2 units.
//   2. softmax: one wave per row (two rows per wave when RG = 8) takes the chunk max, rescales
//      the running sum, and stores weight * (per-token V scale) back in LDS.
//   3. P.V: each thread owns NU channels of one 16-token group.  The channel-major V page gives
//      16 consecutive tokens of one channel per 16-byte load; the weights of those tokens are
//      LDS broadcasts shared by the NU channels.
// At the end the token groups' accumulators are summed through LDS.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr int CH = 128;          // keys per chunk
constexpr int RED_FLOATS = 8192; // LDS floats for the final cross-group reduction

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
    static constexpr int SCW = TPU * RG + 4;   // LDS floats per token group (padded)
    static constexpr int RPR = (RED_FLOATS / (NTG * D)) < RG ? (RED_FLOATS / (NTG * D)) : RG;
    static constexpr int HELD = RG >= LPT ? RG / LPT : 1;  // rows held per lane after the fold
    static_assert(LPT <= 16, "a key row must fit in one DPP row");
    static_assert(NU >= 1 && D % TPT == 0, "channel split");
    static_assert(RG % RPR == 0, "reduction rounds");
};

__device__ __forceinline__ int sc_index(int tl, int j, int rg, int tpu, int scw) {
    return (tl / tpu) * scw + (tl % tpu) * rg + j;
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
                    if (s == 8) recv = lane_xchg<8>(send);
                    else if (s == 4) recv = lane_xchg<4>(send);
                    else if (s == 2) recv = lane_xchg<2>(send);
                    else recv = lane_xchg<1>(send);
                    v[i] = keep + recv;
                }
            }
            n = half;
        } else {
            float recv;
            if (s == 8) recv = lane_xchg<8>(v[0]);
            else if (s == 4) recv = lane_xchg<4>(v[0]);
            else if (s == 2) recv = lane_xchg<2>(v[0]);
            else recv = lane_xchg<1>(v[0]);
            v[0] += recv;
        }
    }
}

template <int D, int RG, int MODE>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
    using C = Cfg<D, RG, MODE>;
    __shared__ __attribute__((aligned(16))) float sc[C::NTG * C::SCW];
    __shared__ __attribute__((aligned(16))) float red[RED_FLOATS];
    __shared__ float row_alpha[RG], row_m[RG], row_l[RG];

    const int tid = threadIdx.x;
    int wi = blockIdx.x;
    const int s = wi % a.nsplit;
    wi /= a.nsplit;
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
    const int t_begin = s * a.split_len;

    if (kmax <= 0) {  // no keys at all (inactive sequence): zero output, lse = -inf
        if (s == 0 && a.nsplit == 1) {
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

    // ---- query rows of this group, this lane's channel slice, in fp32 registers
    const int c = tid % C::LPT;
    float qv[RG][C::EPL];
#pragma unroll
    for (int j = 0; j < RG; ++j) {
        if (j < nvalid) {
            const int r = r0 + j;
            const uint16_t* qp =
                a.q + ((int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g) * D + c * C::EPL;
#pragma unroll
            for (int e8 = 0; e8 < C::EPL / 8; ++e8) {
                const u32x4 w = load16(qp + e8 * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) qv[j][e8 * 8 + e] = bf16_at(w, e);
            }
        } else {
#pragma unroll
            for (int e = 0; e < C::EPL; ++e) qv[j][e] = 0.0f;
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

    // P.V thread mapping: consecutive threads walk a page in memory order (channel-major,
    // then 16-byte segment), so each load instruction covers contiguous bytes.
    constexpr int dummy = 0;
    (void)dummy;
    const int seg_per_row = a.bs / C::TPU;          // 16-byte segments per channel row
    const int pv_seg = tid % seg_per_row;
    const int pv_dl = (tid / seg_per_row) % C::TPT;
    const int pv_pic = tid / (seg_per_row * C::TPT);  // page within the chunk
    const int pv_tg = pv_pic * seg_per_row + pv_seg;

    const int64_t bt_row = (int64_t)b * a.mbs;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v);

    for (int cb = t_begin; cb < t_end; cb += CH) {
        // ------------------------------------------------------------------ 1. scores
#pragma unroll
        for (int pass = 0; pass < C::NPASS; ++pass) {
            const int tl = pass * C::TPP + tid / C::LPT;
            const int t = cb + tl;
            const bool valid = t < t_end;
            float part[RG];
#pragma unroll
            for (int j = 0; j < RG; ++j) part[j] = 0.0f;
            float kscale = 1.0f;
            if (valid) {
                const int64_t blk = a.bt[bt_row + (t >> a.log2bs)];
                const int off = t & (a.bs - 1);
                const int64_t page = blk * a.hkv + h;
                const u32x4 kw = load16(kbase + ((page * a.bs + off) * D) * C::ESZ + c * 16);
#pragma unroll
                for (int e = 0; e < C::EPL; ++e) {
                    const float kv = MODE == 2 ? bf16_at(kw, e) : i8_at(kw, e);
#pragma unroll
                    for (int j = 0; j < RG; ++j) part[j] = fmaf(qv[j][e], kv, part[j]);
                }
                if constexpr (MODE == 0) kscale = a.ks[page * a.bs + off];
                else if constexpr (MODE == 1) kscale = a.ks[page];
            }
            fold_rows<RG, C::LPT>(part, c);
            const float mul = kscale * a.scale_log2;
            if constexpr (RG >= C::LPT) {
#pragma unroll
                for (int k = 0; k < C::HELD; ++k) {
                    const int j = c * C::HELD + k;
                    const int lim = prior + (r0 + j) / a.g;
                    const float v = (valid && j < nvalid && t <= lim) ? part[k] * mul : -INFINITY;
                    sc[sc_index(tl, j, RG, C::TPU, C::SCW)] = v;
                }
            } else {
                constexpr int DUP = C::LPT / RG;
                if (c % DUP == 0) {
                    const int j = c / DUP;
                    const int lim = prior + (r0 + j) / a.g;
                    const float v = (valid && j < nvalid && t <= lim) ? part[0] * mul : -INFINITY;
                    sc[sc_index(tl, j, RG, C::TPU, C::SCW)] = v;
                }
            }
        }
        __syncthreads();

        // ------------------------------------------------------------------ 2. softmax
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int j = wave + 4 * rr;
            if (j < RG) {
                float sv[CH / kWave];
                float cmax = -INFINITY;
#pragma unroll
                for (int k = 0; k < CH / kWave; ++k) {
                    sv[k] = sc[sc_index(lane + k * kWave, j, RG, C::TPU, C::SCW)];
                    cmax = fmaxf(cmax, sv[k]);
                }
                cmax = group_max<kWave>(cmax);
                const float m_new = fmaxf(m_run[rr], cmax);
                const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run[rr] - m_new);
                float psum = 0.0f;
#pragma unroll
                for (int k = 0; k < CH / kWave; ++k) {
                    const int tl = lane + k * kWave;
                    const int t = cb + tl;
                    float p = (sv[k] == -INFINITY) ? 0.0f : exp2f(sv[k] - m_new);
                    psum += p;
                    if constexpr (MODE != 2) {
                        if (p != 0.0f) {
                            const int64_t page = (int64_t)a.bt[bt_row + (t >> a.log2bs)] * a.hkv + h;
                            p *= (MODE == 0) ? a.vs[page * a.bs + (t & (a.bs - 1))] : a.vs[page];
                        }
                    }
                    sc[sc_index(tl, j, RG, C::TPU, C::SCW)] = p;
                }
                psum = group_sum<kWave>(psum);
                l_run[rr] = l_run[rr] * alpha + psum;
                m_run[rr] = m_new;
                if (lane == 0) row_alpha[j] = alpha;
            }
        }
        __syncthreads();

        // ------------------------------------------------------------------ 3. P.V
        {
            float alpha[RG];
#pragma unroll
            for (int j = 0; j < RG; ++j) alpha[j] = row_alpha[j];
#pragma unroll
            for (int j = 0; j < RG; ++j)
#pragma unroll
                for (int k = 0; k < C::NU; ++k) acc[j][k] *= alpha[j];

            const int tok0 = cb + pv_pic * a.bs + pv_seg * C::TPU;
            if (tok0 < t_end) {
                const int64_t page = (int64_t)a.bt[bt_row + ((cb + pv_pic * a.bs) >> a.log2bs)] * a.hkv + h;
                u32x4 vw[C::NU];
#pragma unroll
                for (int k = 0; k < C::NU; ++k) {
                    const int d = pv_dl + k * C::TPT;
                    vw[k] = load16(vbase + ((page * D + d) * a.bs) * C::ESZ + pv_seg * 16);
                }
                const float* wrow = sc + pv_tg * C::SCW;
#pragma unroll
                for (int e = 0; e < C::TPU; ++e) {
                    float w[RG];
                    if constexpr (RG >= 4) {
#pragma unroll
                        for (int j4 = 0; j4 < RG; j4 += 4) {
                            const float4 w4 = *reinterpret_cast<const float4*>(wrow + e * RG + j4);
                            w[j4] = w4.x; w[j4 + 1] = w4.y; w[j4 + 2] = w4.z; w[j4 + 3] = w4.w;
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < RG; ++j) w[j] = wrow[e * RG + j];
                    }
                    const bool live = (MODE != 2) || (tok0 + e < t_end);  // bf16 tail may hold junk
#pragma unroll
                    for (int k = 0; k < C::NU; ++k) {
                        float vv = MODE == 2 ? bf16_at(vw[k], e) : i8_at(vw[k], e);
                        if (!live) vv = 0.0f;
#pragma unroll
                        for (int j = 0; j < RG; ++j) acc[j][k] = fmaf(w[j], vv, acc[j][k]);
                    }
                }
            }
        }
        __syncthreads();
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

    // ---- sum the token groups' accumulators, RPR rows per round
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
                const int r = r0 + j;
                const int64_t orow = (int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g;
                if (a.nsplit == 1) {
                    a.out[orow * D + d] = (uint16_t)f32_to_bf16_rne(o_val);
                    if (d == 0 && a.lse) a.lse[orow] = lse2 * kLn2;
                } else {
                    const int64_t pidx = ((((int64_t)b * a.hkv + h) * a.nrg + rg) * a.nsplit + s) * RG + j;
                    a.part_o[pidx * D + d] = o_val;
                    if (d == 0) a.part_lse[pidx] = lse2;
                }
            }
        }
        __syncthreads();
    }
}

// Log-sum-exp merge of the split partials: one workgroup per (sequence, KV head, row group).
template <int D, int RG>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
    int wi = blockIdx.x;
    const int rg = wi % a.nrg;
    wi /= a.nrg;
    const int h = wi % a.hkv;
    const int b = wi / a.hkv;
    const int qlen = a.cu ? a.cu[b + 1] - a.cu[b] : 1;
    const int qrow0 = a.cu ? a.cu[b] : b;
    const int prior = a.ctx[b] - qlen;
    const int nrows = qlen * a.g;
    const int r0 = rg * RG;
    if (r0 >= nrows) return;
    const int nvalid = min(RG, nrows - r0);
    const int kmax = prior + (r0 + nvalid - 1) / a.g + 1;
    const int nact = kmax <= 0 ? 0 : min(a.nsplit, (kmax + a.split_len - 1) / a.split_len);
    const int64_t base = (((int64_t)b * a.hkv + h) * a.nrg + rg) * a.nsplit;
    for (int o = threadIdx.x; o < nvalid * D; o += blockDim.x) {
        const int j = o / D, d = o % D;
        float mx = -INFINITY;
        for (int sp = 0; sp < nact; ++sp) mx = fmaxf(mx, a.part_lse[(base + sp) * RG + j]);
        float wsum = 0.0f, acc = 0.0f;
        if (mx != -INFINITY) {
            for (int sp = 0; sp < nact; ++sp) {
                const float l2 = a.part_lse[(base + sp) * RG + j];
                const float w = l2 == -INFINITY ? 0.0f : exp2f(l2 - mx);
                wsum += w;
                acc = fmaf(w, a.part_o[((base + sp) * RG + j) * D + d], acc);
            }
        }
        const int r = r0 + j;
        const int64_t orow = (int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g;
        a.out[orow * D + d] = (uint16_t)f32_to_bf16_rne(wsum > 0.0f ? acc / wsum : 0.0f);
        if (d == 0 && a.lse) a.lse[orow] = wsum > 0.0f ? (mx + log2f(wsum)) * kLn2 : -INFINITY;
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
    hipLaunchKernelGGL((merge_kernel<D, RG>), dim3((unsigned)items), dim3(256), 0, stream, a);
    return hipGetLastError();
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
    if (head_dim == 64) return launch_mode<64>(a, batch, rg, mode, stream);
    if (head_dim == 128) return launch_mode<128>(a, batch, rg, mode, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
