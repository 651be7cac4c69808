// mla.hip - paged MLA (latent cache) C8 store and decode on gfx950.
//
// MojoStorePagedMLAKVCache and MojoPagedDecodeMLA (Mojo Opset README, Op List), read as
// multi-head latent attention in its absorbed decode form: each token keeps one latent row
// (512 channels) and one rotary-key row (64 channels), shared by every query head; head h scores
// key t as scale * (q_c . c_t + q_r . r_t) and returns the weighted sum of the latent rows.  Both
// rows are stored as int8 codes with their own per-token scale fl32(absmax / 127), rounded half
// to even (the per-token C8 rule of PR #379's MojoStorePagedKVCacheC8).
//
// Store: one wave per token; 8 latent channels and 1 rotary channel per lane, a cross-lane max
// for each row's absmax, IEEE division and rintf.
//
// Decode: one workgroup of four waves per (sequence, group of 16 heads, key split).  The latent
// rows are both the keys and the values, so each 64-key block is read from HBM once and used
// twice:
//  * wave w loads keys 16w .. 16w+15 of the block in the A-operand layout of
//    v_mfma_i32_16x16x64_i8 (lane (g, n): key 16w + n, 16 bytes of channels 64m + 16g for step m)
//    and scores them against the 16 heads with exact integer dot products: each query row is
//    scaled by a power of two and rounded to integers in [-2^14, 2^14], split as 256 hi + lo with
//    int8 hi and lo; the latent part (eight 64-channel steps) and the rotary part (one step) are
//    summed separately, since their scales differ per token.
//  * the same registers go to LDS (one 528-byte row per key), and the next block's loads are
//    issued at once.
//  * the block's maximum logit per head and the largest latent scale are exchanged through LDS;
//    each wave turns its 16 keys into fp16 weights p * s_c / S (S: a lazily raised reference
//    latent scale, so that the weights stay in range) and stores them in LDS.
//  * P.V as O^T (channels x heads) += V^T P^T on v_mfma_f32_16x16x32_f16: wave w owns latent
//    channels 128w .. 128w+127.  Lane (g, n) reads 8 bytes (channels 128w + 8n ..) of each of
//    its 8 keys 32v + 8g + j from LDS; byte j of those eight reads is the A operand of output tile
//    j (channel 128w + 8n + j for A row n).  A code c enters as the fp16 value 1152 + c (one byte
//    permute and one xor per two codes, exact) and 1152 times the weight sums (an all-ones MFMA)
//    is taken off at the end.
// Two barriers per block; the latent tile and the weights are double-buffered in LDS.  Keys past
// the split's end read in-bounds stand-ins (rows of its last page) that get zero weight.
// Splits are merged by a log-sum-exp pass (mla_merge_kernel).
#include "mla_internal.h"
#include "pkv_device.h"

namespace pkv {
namespace {

typedef int i4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr int DC = kMlaLatent;
constexpr int DR = kMlaRope;
constexpr int NW = 4;            // waves per workgroup
constexpr int MBLK = 16 * NW;    // keys per block, 16 per wave
constexpr int LROW = DC + 16;    // LDS pitch of a latent row (bytes): rows start 4 banks apart
constexpr int CW = DC / NW;      // output channels per wave
constexpr int NT = CW / 16;      // 16 x 16 output tiles per wave
constexpr int QSTEPS = DC / 64 + DR / 64;  // 64-channel score steps: 8 latent + 1 rotary

// ------------------------------------------------------------------------------------- store

// Row (block * BS + slot) of new token t in the page arrays; false when the token is skipped.
__device__ __forceinline__ bool mla_row(const MlaArgs& a, int t, int64_t& row) {
    if (a.slot_mapping) {
        row = a.slot_mapping[t];
        return row >= 0;
    }
    int b, pos;
    if (a.cu_q) {
        int lo = 0, hi = a.batch;  // largest b with cu_q[b] <= t
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu_q[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        b = lo;
        if (b >= a.batch) return false;
        pos = a.ctx[b] - (a.cu_q[b + 1] - a.cu_q[b]) + (t - a.cu_q[b]);
    } else {
        b = t;
        pos = a.ctx[b] - 1;
    }
    if (pos < 0) return false;  // inactive decode slot (context length 0)
    row = (int64_t)a.bt[(int64_t)b * a.mbs + (pos >> a.log2bs)] * a.bs + (pos & (a.bs - 1));
    return true;
}

__global__ __launch_bounds__(256) void mla_store_kernel(MlaArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= a.num_tokens) return;  // uniform per wave
    int64_t row;
    if (!mla_row(a, t, row)) return;
    // latent row: channels 8 lane .. 8 lane + 7
    const u32x4 w = load16(a.latent_new + (int64_t)t * DC + 8 * lane);
    float x[8];
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = bf16_at(w, e);
        am = fmaxf(am, fabsf(x[e]));
    }
    const float s = absmax_scale(group_max<kWave>(am));
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        c0 |= (uint32_t)(quant_code(x[e], s) & 255) << (8 * e);
        c1 |= (uint32_t)(quant_code(x[4 + e], s) & 255) << (8 * e);
    }
    *reinterpret_cast<uint2*>(a.latent + row * DC + 8 * lane) = make_uint2(c0, c1);
    // rotary row: channel lane
    const float xr = bf16_to_f32(a.rope_new[(int64_t)t * DR + lane]);
    const float sr = absmax_scale(group_max<kWave>(fabsf(xr)));
    a.rope[row * DR + lane] = (int8_t)quant_code(xr, sr);
    if (lane == 0) {
        a.ls[row] = s;
        a.rs[row] = sr;
    }
}

// ------------------------------------------------------------------------------------ decode

// max / sum over the four lanes n, n+16, n+32, n+48 (gfx950 permlane swaps, no LDS)
__device__ __forceinline__ float col_max(float x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float col_sum(float x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Quantize NS 64-channel steps of the lane's query row (16 channels per step, raw bf16 in
// raw[2m], raw[2m+1]): x * 2^k rounded to integers in [-2^14, 2^14] (k from the row's absmax over
// the four lanes of the column), split exactly as 256 hi + lo.  Returns 2^-k * mul.
template <int NS>
__device__ __forceinline__ float quant_query(const u32x4* raw, i4* hi, i4* lo, float sgn, float mul) {
    float x[16 * NS];
#pragma unroll
    for (int l = 0; l < 2 * NS; ++l)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * l + e] = sgn * bf16_at(raw[l], e);
    float mx = 0.0f;
#pragma unroll
    for (int e = 0; e < 16 * NS; ++e) mx = fmaxf(mx, fabsf(x[e]));
    mx = col_max(mx);
    int ex = 0;
    if (mx > 0.0f) (void)frexpf(mx, &ex);        // mx in [2^(ex-1), 2^ex)
    const int k = min(120, max(-120, 14 - ex));  // |x| * 2^k < 2^14
    const float up = ldexpf(1.0f, k);
#pragma unroll
    for (int m = 0; m < NS; ++m) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t hw = 0, lw = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int qi = (int)__builtin_rintf(x[16 * m + 4 * w + e] * up);  // |qi| <= 2^14
                const int l8 = ((qi + 128) & 255) - 128;
                const int h8v = (qi - l8) >> 8;                                  // |h8v| <= 64
                hw |= (uint32_t)(h8v & 255) << (8 * e);
                lw |= (uint32_t)(l8 & 255) << (8 * e);
            }
            hi[m][w] = (int)hw;
            lo[m][w] = (int)lw;
        }
    }
    return mul * ldexpf(1.0f, -k);
}

struct __align__(16) MlaShared {
    uint8_t lat[2][MBLK * LROW];  // latent rows of the block (keys x 528 bytes)
    _Float16 p[2][16][MBLK];      // weights, head-major
    float mx[2][NW][16];          // per-wave block maximum of each head's logits
    float vmx[2][NW];             // per-wave largest latent scale
    float lsum[NW][16];           // per-wave weight sums, exchanged at the end
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mla_decode_kernel(MlaArgs a, int items) {
    __shared__ MlaShared S;
    const int u = blockIdx.x;
    const int item = u % items;
    const int sp = u / items;
    const int b = item / a.nhg;
    const int h0 = (item % a.nhg) * 16;
    const int nvalid = min(16, a.heads - h0);
    const int ctx = a.ctx[b];
    const int t_begin = sp * a.split_len;
    const int t_end = a.nsplit == 1 ? ctx : min(ctx, t_begin + a.split_len);
    const int w = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane & 15;  // key row (score A operand), head column (scores, weights, output)
    const int g = lane >> 4;
    if (t_begin >= t_end) {  // uniform per workgroup
        if (a.nsplit == 1) {  // a sequence with no key: zero output, lse = -inf
            for (int o = threadIdx.x; o < nvalid * DC; o += blockDim.x)
                a.out[((int64_t)b * a.heads + h0 + o / DC) * DC + o % DC] = 0;
            if ((int)threadIdx.x < nvalid && a.lse) a.lse[(int64_t)b * a.heads + h0 + threadIdx.x] = -INFINITY;
        }
        return;
    }

    // ---- key loads of one block for this wave: key T + 16w + n (the lane's A row), channels
    //      64m + 16g .. of the latent row for m < 8 and 16g .. of the rotary row; the lane's
    //      scales are those of keys T + 16w + 4g + i (its rows of the score tile)
    const int32_t* btb = a.bt + (int64_t)b * a.mbs;
    const int lastpg = (t_end - 1) >> a.log2bs;
    i4 kr[QSTEPS];
    f4 lsv, rsv;
    auto load_k = [&](int T) {
        const int64_t pg = (int64_t)btb[min((T + 16 * w) >> a.log2bs, lastpg)] * a.bs;
        const int64_t row = pg + ((T + 16 * w + n) & (a.bs - 1));
        const uint8_t* lp = reinterpret_cast<const uint8_t*>(a.latent) + row * DC + 16 * g;
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) {
            const u32x4 v = load16(lp + 64 * m);
            kr[m] = i4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
        const u32x4 v = load16(reinterpret_cast<const uint8_t*>(a.rope) + row * DR + 16 * g);
        kr[DC / 64] = i4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        const int64_t srow = pg + ((T + 16 * w + 4 * g) & (a.bs - 1));
        lsv = *reinterpret_cast<const f4*>(a.ls + srow);
        rsv = *reinterpret_cast<const f4*>(a.rs + srow);
    };
    load_k(t_begin);

    // ---- query rows (B operand): lane (g, n) holds head h0 + n, channels 64m + 16g .. + 15
    const bool hv = n < nvalid;
    const int64_t qrow = (int64_t)b * a.heads + h0 + n;
    u32x4 qraw[2 * QSTEPS];
    {
        const uint16_t* qlp = a.ql + qrow * DC + 16 * g;
        const uint16_t* qrp = a.qr + qrow * DR + 16 * g;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) {
            qraw[2 * m] = hv ? load16(qlp + 64 * m) : z;
            qraw[2 * m + 1] = hv ? load16(qlp + 64 * m + 8) : z;
        }
        qraw[2 * (QSTEPS - 1)] = hv ? load16(qrp) : z;
        qraw[2 * QSTEPS - 1] = hv ? load16(qrp + 8) : z;
    }
    const float sgn = a.scale_log2 < 0.0f ? -1.0f : 1.0f;  // a negative scale flips the query
    i4 qhi[QSTEPS], qlo[QSTEPS];
    const float rmul_c = quant_query<DC / 64>(qraw, qhi, qlo, sgn, fabsf(a.scale_log2));
    const float rmul_r = quant_query<1>(qraw + 2 * (DC / 64), qhi + DC / 64, qlo + DC / 64, sgn, fabsf(a.scale_log2));

    const uint32_t ones_w[4] = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};  // fp16 1.0
    const h8 ones = __builtin_bit_cast(h8, ones_w);
    float mr = -INFINITY;  // running reference max (log2 units), raised lazily (by more than 8)
    float lsum = 0.0f;     // the wave's weight sum of its keys, per head
    float sref = 0.0f;     // reference latent scale, raised when a block's scale passes 16x it
    float sinv = 0.0f;
    f4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
    f4 pacc = f4{0.f, 0.f, 0.f, 0.f};

    int bi = 0;
    for (int T = t_begin; T < t_end; T += MBLK, bi ^= 1) {
        // -------------------------------- integer scores of the wave's 16 keys x 16 heads
        i4 c = i4{0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) c = __builtin_amdgcn_mfma_i32_16x16x64_i8(kr[m], qhi[m], c, 0, 0, 0);
        c = c * 256;
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) c = __builtin_amdgcn_mfma_i32_16x16x64_i8(kr[m], qlo[m], c, 0, 0, 0);
        i4 r = __builtin_amdgcn_mfma_i32_16x16x64_i8(kr[DC / 64], qhi[DC / 64], i4{0, 0, 0, 0}, 0, 0, 0);
        r = r * 256;
        r = __builtin_amdgcn_mfma_i32_16x16x64_i8(kr[DC / 64], qlo[DC / 64], r, 0, 0, 0);
        // -------------------------------- latent rows to LDS, next block's loads
        uint8_t* lrow = &S.lat[bi][(16 * w + n) * LROW + 16 * g];
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) *reinterpret_cast<i4*>(lrow + 64 * m) = kr[m];
        const f4 lsc = lsv, rsc = rsv;
        if (T + MBLK < t_end) load_k(T + MBLK);

        // -------------------------------- logits (log2 units) of keys T + 16w + 4g + i
        const bool MASKED = T + MBLK > t_end;
        float x[4], vsl[4];
        float lmax = -INFINITY, vm = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool vis = !MASKED || T + 16 * w + 4 * g + i < t_end;
            x[i] = vis ? __builtin_fmaf((float)c[i] * lsc[i], rmul_c, (float)r[i] * rsc[i] * rmul_r) : -INFINITY;
            vsl[i] = vis ? lsc[i] : 0.0f;  // stand-in keys' scales never reach a weight
            vm = fmaxf(vm, vsl[i]);
            lmax = fmaxf(lmax, x[i]);
        }
        lmax = col_max(lmax);
        vm = col_max(vm);
        if (g == 0) S.mx[bi][w][n] = lmax;
        if (lane == 0) S.vmx[bi][w] = vm;
        __syncthreads();  // the block's latent rows and maxima are visible

        float bmax = S.mx[bi][0][n], vmax = S.vmx[bi][0];
#pragma unroll
        for (int k = 1; k < NW; ++k) {
            bmax = fmaxf(bmax, S.mx[bi][k][n]);
            vmax = fmaxf(vmax, S.vmx[bi][k]);
        }
        float sf = 1.0f;
        if (vmax > 16.0f * sref) {  // (also the first block: sref == 0)
            sf = sref > 0.0f ? sref * __builtin_amdgcn_rcpf(vmax) : 0.0f;
            sref = vmax;
            sinv = __builtin_amdgcn_rcpf(vmax);
        }
        float alpha = 1.0f;
        if (bmax > mr + 8.0f) {  // (also the first block: mr == -inf)
            alpha = __builtin_amdgcn_exp2f(mr - bmax);
            mr = bmax;
        }
        float ps = 0.0f;
        h4 wv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = x[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[i] - mr);
            ps += p;
            wv[i] = (_Float16)(p * vsl[i] * sinv);
        }
        lsum = lsum * alpha + col_sum(ps);
        *reinterpret_cast<h4*>(&S.p[bi][n][16 * w + 4 * g]) = wv;
        const float factor = alpha * sf;
        if (__any(factor != 1.0f)) {
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[j] *= factor;
            pacc *= factor;
        }
        __syncthreads();  // the weights are visible

        // -------------------------------- P.V over the wave's channels, 32 keys per step
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const h8 bq = *reinterpret_cast<const h8*>(&S.p[bi][n][32 * v + 8 * g]);
            uint2 vv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                vv[j] = *reinterpret_cast<const uint2*>(&S.lat[bi][(32 * v + 8 * g + j) * LROW + CW * w + 8 * n]);
#pragma unroll
            for (int tj = 0; tj < NT; ++tj) {
                const uint32_t bsel = tj & 3;
                const uint32_t sel = 0x0c000c00u | ((4u + bsel) << 16) | bsel;  // [code, 0, code', 0]
                uint32_t d[4];
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const uint32_t lo = tj < 4 ? vv[2 * pp].x : vv[2 * pp].y;
                    const uint32_t hi = tj < 4 ? vv[2 * pp + 1].x : vv[2 * pp + 1].y;
                    d[pp] = __builtin_amdgcn_perm(hi, lo, sel) ^ 0x64806480u;  // fp16 1152 + code
                }
                acc[tj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, d), bq, acc[tj], 0, 0, 0);
            }
            pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, bq, pacc, 0, 0, 0);
        }
    }

    // ---- normalise and write.  Lane (g, n) holds channels 128w + 32g + 8i + j (tile j, row
    //      4g + i of the tile) of head h0 + n.
    if (g == 0) S.lsum[w][n] = lsum;
    __syncthreads();
    const float L = S.lsum[0][n] + S.lsum[1][n] + S.lsum[2][n] + S.lsum[3][n];
    const float mul = L > 0.0f ? sref / L : 0.0f;
    const float bias = 1152.0f * pacc[0];
    if (!hv) return;
    const bool split_mode = a.nsplit > 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float o[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) o[j] = (acc[j][i] - bias) * mul;
        const int ch = CW * w + 32 * g + 8 * i;
        if (!split_mode) {
            uint4 pk;
            pk.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
            pk.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
            pk.z = f32_to_bf16_rne(o[4]) | (f32_to_bf16_rne(o[5]) << 16);
            pk.w = f32_to_bf16_rne(o[6]) | (f32_to_bf16_rne(o[7]) << 16);
            *reinterpret_cast<uint4*>(a.out + qrow * DC + ch) = pk;
        } else {
            float* po = a.part_o + ((int64_t)u * 16 + n) * DC + ch;
            *reinterpret_cast<f4*>(po) = f4{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<f4*>(po + 4) = f4{o[4], o[5], o[6], o[7]};
        }
    }
    if (w == 0 && g == 0) {
        const float lse2 = L > 0.0f ? mr + log2f(L) : -INFINITY;
        if (!split_mode) {
            if (a.lse) a.lse[qrow] = lse2 * kLn2;
        } else {
            a.part_lse[(int64_t)u * 16 + n] = lse2;
        }
    }
}

// Log-sum-exp merge of the splits of one (sequence, head): 128 threads, 4 channels each.
__global__ __launch_bounds__(128) void mla_merge_kernel(MlaArgs a, int items) {
    const int b = blockIdx.x / a.heads;
    const int h = blockIdx.x % a.heads;
    const int item = b * a.nhg + h / 16;
    const int row = h % 16;
    const int ctx = a.ctx[b];
    const int nact = ctx <= 0 ? 0 : min(a.nsplit, (ctx + a.split_len - 1) / a.split_len);
    float M = -INFINITY;
    for (int s = 0; s < nact; ++s) M = fmaxf(M, a.part_lse[((int64_t)s * items + item) * 16 + row]);
    const int c = 4 * threadIdx.x;
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    float wsum = 0.0f;
    for (int s = 0; s < nact; ++s) {
        const int64_t pr = ((int64_t)s * items + item) * 16 + row;
        const float wt = __builtin_amdgcn_exp2f(a.part_lse[pr] - M);
        wsum += wt;
        acc += wt * *reinterpret_cast<const f4*>(a.part_o + pr * DC + c);
    }
    const float mul = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    uint2 pk;
    pk.x = f32_to_bf16_rne(acc[0] * mul) | (f32_to_bf16_rne(acc[1] * mul) << 16);
    pk.y = f32_to_bf16_rne(acc[2] * mul) | (f32_to_bf16_rne(acc[3] * mul) << 16);
    *reinterpret_cast<uint2*>(a.out + ((int64_t)b * a.heads + h) * DC + c) = pk;
    if (threadIdx.x == 0 && a.lse)
        a.lse[(int64_t)b * a.heads + h] = wsum > 0.0f ? (M + log2f(wsum)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_mla_store(const MlaArgs& a, hipStream_t stream) {
    const int64_t grid = ((int64_t)a.num_tokens + 3) / 4;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_store_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_mla_decode(const MlaArgs& a, hipStream_t stream) {
    const int64_t items = (int64_t)a.batch * a.nhg;
    const int64_t units = items * a.nsplit;
    if (units == 0) return hipSuccess;
    if (units > 0x7fffffff || (int64_t)a.batch * a.heads > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_decode_kernel, dim3((unsigned)units), dim3(NW * kWave), 0, stream, a, (int)items);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)(a.batch * a.heads)), dim3(DC / 4), 0, stream, a,
                       (int)items);
    return hipGetLastError();
}

}  // namespace pkv
