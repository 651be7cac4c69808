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
// Decode: one workgroup of four waves per (sequence, group of 16 heads, key range).  The latent
// rows are both the keys and the values, so each 64-key block is read from HBM once and used
// twice:
//  * wave w loads keys 16w .. 16w+15 of the block in the A-operand layout of
//    v_mfma_i32_16x16x64_i8 (lane (g, n): key 16w + n, 16 bytes of channels 64m + 16g for step m)
//    and scores them against the 16 heads with exact integer dot products: each query row is
//    scaled by a power of two and rounded to integers in [-2^22, 2^22] (relative rounding 2^-23
//    of the row's largest element), split as 65536 hi + 256 mid + lo with int8 digits; 256 K.hi +
//    K.mid and K.lo are accumulated apart (int32) and joined in fp32; the latent part (eight
//    64-channel steps) and the rotary part (one step) are summed separately, since their scales
//    differ per token.
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
// Three barriers per block (the latent tile, the weights and the maxima are single LDS buffers);
// the key registers are double-buffered (each wave has about two blocks in flight), and the
// quantized query rows, the same for all four waves, are kept in LDS.  Keys past the range's end read
// in-bounds stand-ins (rows of its last page) that get zero weight.
// Key ranges: fixed splits of split_len keys, or (the default) a balanced partition that cuts
// every block of every (sequence, head group) into as many near-equal segments as the GPU holds
// workgroups at once, each workgroup finding its own from the context lengths.  The partial
// results are merged by a log-sum-exp pass (mla_merge_kernel).
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
static_assert(DC / 8 == kWave, "the merge is one wave of 8 latent channels per lane");

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

// Bytes a workgroup keeps of a token it stores for its own decode: latent codes [512], rotary
// codes [64], the latent and rotary scales (fp32).
constexpr int NT_BYTES = DC + DR + 8;

// Quantize token t of latent_new / rope_new (one wave: latent channels 8 lane .., rotary channel
// lane) into cache row `row`; with nt, also keep its codes and scales there (LDS).
__device__ __forceinline__ void mla_quantize_token(const MlaArgs& a, int64_t t, int64_t row, uint8_t* nt) {
    const int lane = threadIdx.x & (kWave - 1);
    // latent row: channels 8 lane .. 8 lane + 7
    const u32x4 w = load16(a.latent_new + t * DC + 8 * lane);
    float x[8];
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = bf16_at(w, e);
        am = fmaxf(am, fabsf(x[e]));
    }
    const float s = absmax_scale(group_max<kWave>(am));
    int codes[8];
    quant_row_absmax<8>(x, s, codes);
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        c0 |= (uint32_t)(codes[e] & 255) << (8 * e);
        c1 |= (uint32_t)(codes[4 + e] & 255) << (8 * e);
    }
    *reinterpret_cast<uint2*>(a.latent + row * DC + 8 * lane) = make_uint2(c0, c1);
    // rotary row: channel lane
    const float xr = bf16_to_f32(a.rope_new[t * DR + lane]);
    const float sr = absmax_scale(group_max<kWave>(fabsf(xr)));
    int cr;
    quant_row_absmax<1>(&xr, sr, &cr);
    a.rope[row * DR + lane] = (int8_t)cr;
    if (lane == 0) {
        a.ls[row] = s;
        a.rs[row] = sr;
    }
    if (nt) {
        *reinterpret_cast<uint2*>(nt + 8 * lane) = make_uint2(c0, c1);
        nt[DC + lane] = (uint8_t)cr;
        if (lane == 0) {
            reinterpret_cast<float*>(nt + DC + DR)[0] = s;
            reinterpret_cast<float*>(nt + DC + DR)[1] = sr;
        }
    }
}

__global__ __launch_bounds__(256) void mla_store_kernel(MlaArgs a) {
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= a.num_tokens) return;  // uniform per wave
    int64_t row;
    if (!mla_row(a, t, row)) return;
    mla_quantize_token(a, t, row, nullptr);
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
// raw[2m], raw[2m+1]): x * 2^k rounded to integers in [-2^22, 2^22] (k from the row's absmax over
// the four lanes of the column), split exactly as 65536 hi + 256 mid + lo.  Returns 2^-k * mul.
template <int NS>
__device__ __forceinline__ float quant_query(const u32x4* raw, i4* hi, i4* md, i4* lo, float sgn, float mul) {
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
    const int k = min(120, max(-120, 22 - ex));  // |x| * 2^k < 2^22
    const float up = ldexpf(1.0f, k);
#pragma unroll
    for (int m = 0; m < NS; ++m) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t hw = 0, mw = 0, lw = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int qi = (int)__builtin_rintf(x[16 * m + 4 * w + e] * up);  // |qi| <= 2^22
                const int l8 = ((qi + 128) & 255) - 128;
                const int r1 = (qi - l8) >> 8;                                   // |r1| <= 2^14
                const int m8 = ((r1 + 128) & 255) - 128;
                const int h8v = (r1 - m8) >> 8;                                  // |h8v| <= 64
                hw |= (uint32_t)(h8v & 255) << (8 * e);
                mw |= (uint32_t)(m8 & 255) << (8 * e);
                lw |= (uint32_t)(l8 & 255) << (8 * e);
            }
            hi[m][w] = (int)hw;
            md[m][w] = (int)mw;
            lo[m][w] = (int)lw;
        }
    }
    return mul * ldexpf(1.0f, -k);
}

struct __align__(16) MlaShared {
    uint8_t lat[MBLK * LROW];     // latent rows of the block (keys x 528 bytes)
    _Float16 p[16][MBLK];         // weights, head-major
    float mx[NW][16];             // per-wave block maximum of each head's logits
    float vmx[NW];                // per-wave largest latent scale
    float lsum[NW][16];           // per-wave weight sums, exchanged at the end
    i4 qhi[QSTEPS][kWave];        // the quantized query rows (B operand of the score MFMA, per
    i4 qmd[QSTEPS][kWave];        // lane), high, middle and low bytes: the same for every wave
    i4 qlo[QSTEPS][kWave];
    int pg[NW][128];              // per wave: page ids of its keys in two 64-block chunks (ring)
    int plan[NW][2];              // balanced partition: per-wave partial sums
    int found[3];                 // balanced partition: the workgroup's sequence, its first slot and length
    __align__(16) uint8_t nt[NT_BYTES];  // a decode step's new token, stored by this workgroup
};

// One wave's key registers for a block: A operand rows of the score MFMA (8 latent steps and
// one rotary step) and the scales of the lane's four score rows.
struct MlaKRegs {
    i4 k[QSTEPS];
    f4 ls, rs;
};

// Sum over the workgroup (NW waves); every thread gets the total.  Ends with a barrier, so the
// shared slots can be reused at once.
__device__ __forceinline__ int wg_sum(int x, int (*red)[2], int slot) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, kWave);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) red[w][slot] = x;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) t += red[k][slot];
    __syncthreads();
    return t;
}

// Balanced partition of every key block of every (sequence, head group) item over the W
// workgroups the GPU holds at once: item i with n_i blocks gets k_i = min(n_i, ceil(n_i Wp / N))
// contiguous, near-equal segments (N blocks in all; Wp = W - A with A non-empty items, so that
// the ceilings keep the total within W and the chip runs one round of equally long workgroups).
// Segments are numbered sequence by sequence, head group by head group.  Workgroup u finds its
// segment from the context lengths alone (two passes over them); false when u has none.  ctx: the
// context length of the segment's sequence.
__device__ bool mla_balanced_segment(const MlaArgs& a, int u, MlaShared& S, int& b, int& hg, int& t_begin,
                                     int& t_end, int& kseg, int& first, int& ctx) {
    const int tid = threadIdx.x;
    const int W = a.sk_wgs;
    auto nblk = [&](int c) { return c > 0 ? (c + MBLK - 1) / MBLK : 0; };
    int c_first = 0;  // context length of sequence tid (first chunk), kept for the second pass
    int N = 0, A = 0;
    for (int c0 = 0; c0 < a.batch; c0 += NW * kWave) {
        const int bb = c0 + tid;
        const int cb = bb < a.batch ? a.ctx[bb] : 0;
        const int nb = nblk(cb);
        if (c0 == 0) c_first = cb;
        N += wg_sum(nb, S.plan, 0);
        A += wg_sum(nb > 0 ? 1 : 0, S.plan, 1);
    }
    if (N == 0) return false;  // every item is empty: the merge writes the zero rows
    const int64_t NN = (int64_t)N * a.nhg;
    const int AA = A * a.nhg;
    const int64_t Wp = W > 2 * AA ? W - AA : (W > AA ? AA : 1);
    auto segs = [&](int nb) { return nb > 0 ? (int)min((int64_t)nb, ((int64_t)nb * Wp + NN - 1) / NN) : 0; };
    int carry = 0;
    for (int c0 = 0; c0 < a.batch; c0 += NW * kWave) {
        const int bb = c0 + tid;
        const int cb = bb < a.batch ? (c0 == 0 ? c_first : a.ctx[bb]) : 0;
        const int nb = nblk(cb);
        const int k = segs(nb) * a.nhg;
        int x = k;  // inclusive scan over the wave, then over the waves
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(x, d, kWave);
            if ((tid & (kWave - 1)) >= d) x += y;
        }
        const int w = tid / kWave;
        if ((tid & (kWave - 1)) == kWave - 1) S.plan[w][0] = x;
        __syncthreads();
        int off = carry, tot = 0;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
            off += q < w ? S.plan[q][0] : 0;
            tot += S.plan[q][0];
        }
        const int incl = off + x;
        if (k > 0 && incl - k <= u && u < incl) {
            S.found[0] = bb;
            S.found[1] = incl - k;
            S.found[2] = cb;
        }
        carry += tot;
        __syncthreads();
    }
    if (u >= carry) return false;
    b = S.found[0];
    const int seq_first = S.found[1];
    ctx = S.found[2];
    const int nb = nblk(ctx);
    kseg = segs(nb);
    const int off = u - seq_first;
    hg = off / kseg;
    const int sg = off - hg * kseg;
    first = seq_first + hg * kseg;
    t_begin = (int)((int64_t)nb * sg / kseg) * MBLK;
    t_end = min(ctx, (int)((int64_t)nb * (sg + 1) / kseg) * MBLK);
    return true;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mla_decode_kernel(MlaArgs a, int items) {
    __shared__ MlaShared S;
    const int u = blockIdx.x;
    int b, hg, t_begin, t_end, ctx;
    int64_t pslot;  // partial slot of this workgroup's output, -1: the output itself
    if (a.sk_wgs > 0) {
        int kseg, first;
        if (!mla_balanced_segment(a, u, S, b, hg, t_begin, t_end, kseg, first, ctx)) return;  // uniform
        if ((int)threadIdx.x == 0 && t_begin == 0) {  // the item's first segment records the item
            a.seg[2 * (b * a.nhg + hg)] = first;
            a.seg[2 * (b * a.nhg + hg) + 1] = kseg;
        }
        pslot = kseg > 1 ? u : -1;
    } else {
        const int item = u % items;
        const int sp = u / items;
        b = item / a.nhg;
        hg = item % a.nhg;
        ctx = a.ctx[b];
        t_begin = sp * a.split_len;
        t_end = a.nsplit == 1 ? ctx : min(ctx, t_begin + a.split_len);
        pslot = a.nsplit > 1 ? u : -1;
    }
    const int h0 = hg * 16;
    const int nvalid = min(16, a.heads - h0);
    const int w = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane & 15;  // key row (score A operand), head column (scores, weights, output)
    const int g = lane >> 4;
    if (t_begin >= t_end) {  // uniform per workgroup (fixed splits only)
        if (a.nsplit == 1) {  // a sequence with no key: zero output, lse = -inf
            for (int o = threadIdx.x; o < nvalid * DC; o += blockDim.x)
                a.out[((int64_t)b * a.heads + h0 + o / DC) * DC + o % DC] = 0;
            if ((int)threadIdx.x < nvalid && a.lse) a.lse[(int64_t)b * a.heads + h0 + threadIdx.x] = -INFINITY;
        }
        return;
    }
    // one decode step with its store (one head group per sequence): the workgroup whose keys end at
    // the new token's position, ctx - 1, quantizes and writes the token and keeps its codes in LDS
    // (its own loads of that slot may predate the write: the block holding it is patched below)
    const int pos = a.fuse_store ? __builtin_amdgcn_readfirstlane(ctx) - 1 : -1;
    const bool own_new = pos >= __builtin_amdgcn_readfirstlane(t_begin) && pos < __builtin_amdgcn_readfirstlane(t_end);

    // ---- key loads of one block for this wave: key T + 16w + n (the lane's A row), channels
    //      64m + 16g .. of the latent row for m < 8 and 16g .. of the rotary row; the lane's
    //      scales are those of keys T + 16w + 4g + i (its rows of the score tile).  Two register
    //      sets: the loads of block k + 2 are issued once block k's codes are in LDS, so every
    //      wave has about two blocks in flight.
    //      Page ids: each wave keeps those of its keys for two chunks of 64 blocks of the range in
    //      an LDS ring (entry j = block j mod 128), read with ds_read; chunk c + 1 is loaded at
    //      the start of chunk c and written to the ring half-way through it.  So no key load
    //      waits for a block-table round trip, and no wait in the key loop is for a page load.
    //      Start-up: the first two chunks' page ids and the query rows are requested together, the
    //      first block's keys as soon as the page ids are in, and the query is quantized while
    //      those keys are on their way.  (The groups stay in this order, so that each wait
    //      covers only its own group and the ones before it.)
    const int32_t* btb = a.bt + (int64_t)b * a.mbs;
    const int lastpg = (t_end - 1) >> a.log2bs;
    auto pages_of = [&](int c) {  // (keys past the range's end: its last page, in bounds)
        const int T = t_begin + MBLK * (64 * c + lane);
        return btb[min((T + 16 * w) >> a.log2bs, lastpg)];
    };
    const int pv0 = pages_of(0);
    int pvn = pages_of(1);  // the next chunk's page ids, on their way to the ring

    // ---- query rows (B operand): lane (g, n) holds head h0 + n, channels 64m + 16g .. + 15 (lanes
    //      of heads past the group's end read head h0's row and use zeros)
    const bool hv = n < nvalid;
    const int64_t qrow = (int64_t)b * a.heads + h0 + (hv ? n : 0);
    u32x4 qraw[2 * QSTEPS];
    __builtin_amdgcn_sched_barrier(0);
    {
        const uint16_t* qlp = a.ql + qrow * DC + 16 * g;
        const uint16_t* qrp = a.qr + qrow * DR + 16 * g;
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) {
            qraw[2 * m] = load16(qlp + 64 * m);
            qraw[2 * m + 1] = load16(qlp + 64 * m + 8);
        }
        qraw[2 * (QSTEPS - 1)] = load16(qrp);
        qraw[2 * QSTEPS - 1] = load16(qrp + 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    S.pg[w][lane] = pv0;
    S.pg[w][64 + lane] = pvn;
    __builtin_amdgcn_wave_barrier();
    auto page_of = [&](int T) { return S.pg[w][((T - t_begin) / MBLK) & 127]; };
    auto load_k = [&](int T, int pid, MlaKRegs& R) {
        const int64_t pg = (int64_t)pid * a.bs;
        const int64_t row = pg + ((T + 16 * w + n) & (a.bs - 1));
        const uint8_t* lp = reinterpret_cast<const uint8_t*>(a.latent) + row * DC + 16 * g;
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) {
            const u32x4 v = load16(lp + 64 * m);
            R.k[m] = i4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
        const u32x4 v = load16(reinterpret_cast<const uint8_t*>(a.rope) + row * DR + 16 * g);
        R.k[DC / 64] = i4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    };
    auto load_s = [&](int T, int pid, MlaKRegs& R) {
        const int64_t pg = (int64_t)pid * a.bs;
        const int64_t srow = pg + ((T + 16 * w + 4 * g) & (a.bs - 1));
        R.ls = *reinterpret_cast<const f4*>(a.ls + srow);
        R.rs = *reinterpret_cast<const f4*>(a.rs + srow);
    };
    MlaKRegs R0, R1;
    {
        const int p0 = page_of(t_begin);
        load_k(t_begin, p0, R0);
        load_s(t_begin, p0, R0);
    }
    const int p1 = page_of(t_begin + MBLK);
    __builtin_amdgcn_sched_barrier(0);

    if (!hv) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 2 * QSTEPS; ++i) qraw[i] = z;
    }
    const float sgn = a.scale_log2 < 0.0f ? -1.0f : 1.0f;  // a negative scale flips the query
    i4 qhi[QSTEPS], qmd[QSTEPS], qlo[QSTEPS];
    const float rmul_c = quant_query<DC / 64>(qraw, qhi, qmd, qlo, sgn, fabsf(a.scale_log2));
    const float rmul_r = quant_query<1>(qraw + 2 * (DC / 64), qhi + DC / 64, qmd + DC / 64, qlo + DC / 64, sgn,
                                        fabsf(a.scale_log2));
    // the quantized query is the same for every wave: kept once in LDS instead of in every
    // wave's registers (room for the second key register set)
    if (w == 0) {
#pragma unroll
        for (int m = 0; m < QSTEPS; ++m) {
            S.qhi[m][lane] = qhi[m];
            S.qmd[m][lane] = qmd[m];
            S.qlo[m][lane] = qlo[m];
        }
    }
    // the new token, by wave 1 while the first block's keys are on their way
    if (own_new && w == 1) {
        const int64_t row = (int64_t)btb[pos >> a.log2bs] * a.bs + (pos & (a.bs - 1));
        mla_quantize_token(a, b, row, S.nt);
    }
    __syncthreads();  // the quantized query and a stored token are visible
    // the second block's loads, after the raw query registers are free (unconditional: past the
    // range's end they read stand-ins on its last page)
    load_k(t_begin + MBLK, p1, R1);
    load_s(t_begin + MBLK, p1, R1);

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

    // one 64-key block at T from register set R.  steady: the loads of block T + 2 are issued
    // unconditionally (past the range's end they read in-bounds stand-ins)
    auto block = [&](const bool steady, const int T, MlaKRegs& R) {
        const int bi = (T - t_begin) / MBLK;
        if ((bi & 63) == 32) {  // chunk bi/64 + 1 (loaded at the chunk's start) to the ring
            S.pg[w][((bi / 64 + 1) & 1) * 64 + lane] = pvn;
            __builtin_amdgcn_wave_barrier();
        }
        if ((bi & 63) == 0 && bi > 0) pvn = pages_of(bi / 64 + 1);  // (its ring half is free)
        const int pg = page_of(T + 2 * MBLK);
        // -------------------------------- integer scores of the wave's 16 keys x 16 heads
        //                                  (hi and lo as two independent accumulation chains)
        i4 ch = i4{0, 0, 0, 0}, cm = i4{0, 0, 0, 0}, cl = i4{0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) {
            ch = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.k[m], S.qhi[m][lane], ch, 0, 0, 0);
            cm = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.k[m], S.qmd[m][lane], cm, 0, 0, 0);
            cl = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.k[m], S.qlo[m][lane], cl, 0, 0, 0);
        }
        const i4 c1 = ch * 256 + cm;  // |256 K.hi + K.mid| <= 512 * 128 * 2^14 = 2^30
        const i4 rh = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.k[DC / 64], S.qhi[DC / 64][lane], i4{0, 0, 0, 0}, 0, 0, 0);
        const i4 rm = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.k[DC / 64], S.qmd[DC / 64][lane], i4{0, 0, 0, 0}, 0, 0, 0);
        const i4 rl = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.k[DC / 64], S.qlo[DC / 64][lane], i4{0, 0, 0, 0}, 0, 0, 0);
        const i4 r1 = rh * 256 + rm;
        // -------------------------------- latent rows to LDS (once every wave is done with the
        //                                  previous block's), loads of the block after next
        __syncthreads();
        uint8_t* lrow = &S.lat[(16 * w + n) * LROW + 16 * g];
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) *reinterpret_cast<i4*>(lrow + 64 * m) = R.k[m];
        const bool more = steady || T + 2 * MBLK < t_end;
        if (more) load_k(T + 2 * MBLK, pg, R);

        // -------------------------------- logits (log2 units) of keys T + 16w + 4g + i
        const bool MASKED = T + MBLK > t_end;
        float x[4], vsl[4];
        float lmax = -INFINITY, vm = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool vis = !MASKED || T + 16 * w + 4 * g + i < t_end;
            const float cs = __builtin_fmaf((float)c1[i], 256.0f, (float)cl[i]);  // latent score
            const float rs = __builtin_fmaf((float)r1[i], 256.0f, (float)rl[i]);  // rotary score
            x[i] = vis ? __builtin_fmaf(cs * R.ls[i], rmul_c, rs * R.rs[i] * rmul_r) : -INFINITY;
            vsl[i] = vis ? R.ls[i] : 0.0f;  // stand-in keys' scales never reach a weight
            vm = fmaxf(vm, vsl[i]);
            lmax = fmaxf(lmax, x[i]);
        }
        // the scales' registers are free once the logits are formed: the next loads go to the same
        // registers (no instruction moves across this point, so no copy of in-flight loads)
        __builtin_amdgcn_sched_barrier(0);
        if (more) load_s(T + 2 * MBLK, pg, R);
        lmax = col_max(lmax);
        vm = col_max(vm);
        if (g == 0) S.mx[w][n] = lmax;
        if (lane == 0) S.vmx[w] = vm;
        __syncthreads();  // the block's latent rows and maxima are visible

        float bmax = S.mx[0][n], vmax = S.vmx[0];
#pragma unroll
        for (int k = 1; k < NW; ++k) {
            bmax = fmaxf(bmax, S.mx[k][n]);
            vmax = fmaxf(vmax, S.vmx[k]);
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
        *reinterpret_cast<h4*>(&S.p[n][16 * w + 4 * g]) = wv;
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
            const h8 bq = *reinterpret_cast<const h8*>(&S.p[n][32 * v + 8 * g]);
            uint2 vv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                vv[j] = *reinterpret_cast<const uint2*>(&S.lat[(32 * v + 8 * g + j) * LROW + CW * w + 8 * n]);
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
    };
    // Every block issues the loads of the block after next, past the range's end too (in-bounds
    // stand-ins on its last page, which the cache holds): with a conditional issue the newest
    // loads could be any block's, and every wait would drain all of them.
    // the block holding the stored token takes its codes and scales from LDS: wave wk's lanes of
    // key row kn (all channel groups) and, for the scales, lane group gk's entry ik
    auto patch_new = [&](const int T, MlaKRegs& R) {
        const int kk = pos - T;
        if (w != (kk >> 4)) return;  // (uniform per wave)
        const bool krow = n == (kk & 15);
#pragma unroll
        for (int m = 0; m < DC / 64; ++m) {
            const i4 v = *reinterpret_cast<const i4*>(S.nt + 64 * m + 16 * g);
            R.k[m] = krow ? v : R.k[m];
        }
        const i4 vr = *reinterpret_cast<const i4*>(S.nt + DC + 16 * g);
        R.k[DC / 64] = krow ? vr : R.k[DC / 64];
        const float* ns = reinterpret_cast<const float*>(S.nt + DC + DR);
        const float nls = ns[0], nrs = ns[1];
        const bool sgrp = g == ((kk & 15) >> 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool hit = sgrp && i == (kk & 3);
            R.ls[i] = hit ? nls : R.ls[i];
            R.rs[i] = hit ? nrs : R.rs[i];
        }
    };
    for (int T = t_begin;;) {
        if (own_new && pos >= T && pos < T + MBLK) patch_new(T, R0);
        block(true, T, R0);
        T += MBLK;
        if (T >= t_end) break;
        if (own_new && pos >= T && pos < T + MBLK) patch_new(T, R1);
        block(true, T, R1);
        T += MBLK;
        if (T >= t_end) break;
    }

    // ---- normalise and write.  Lane (g, n) holds channels 128w + 32g + 8i + j (tile j, row
    //      4g + i of the tile) of head h0 + n.
    if (g == 0) S.lsum[w][n] = lsum;
    __syncthreads();
    const float L = S.lsum[0][n] + S.lsum[1][n] + S.lsum[2][n] + S.lsum[3][n];
    const bool split_mode = pslot >= 0;
    // the output (bf16), or a partial in latent-code units (fp16: every latent scale of the range
    // is within 16x sref, so |partial| <= 127 * 16) whose scale sref the merge applies
    const float mul = L > 0.0f ? (split_mode ? 1.0f : sref) / L : 0.0f;
    const float bias = 1152.0f * pacc[0];
    if (!hv) return;
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
            h8 ph;
#pragma unroll
            for (int j = 0; j < NT; ++j) ph[j] = (_Float16)o[j];
            *reinterpret_cast<h8*>(a.part_o + (pslot * 16 + n) * DC + ch) = ph;
        }
    }
    if (w == 0 && g == 0) {
        const float lse2 = L > 0.0f ? mr + log2f(L) : -INFINITY;
        if (!split_mode) {
            if (a.lse) a.lse[qrow] = lse2 * kLn2;
        } else {
            *reinterpret_cast<float2*>(a.part_lse + 2 * (pslot * 16 + n)) = make_float2(lse2, sref);
        }
    }
}

// Log-sum-exp merge of the partials of one (sequence, head): one wave, 8 channels per lane; the
// partials are read eight at a time.  Fixed splits: split s of item i in slot s * items + i;
// balanced partition: the item's segments in slots seg[2i] .. seg[2i] + seg[2i + 1] - 1 (a
// one-segment item is already written).  A sequence with no key gets a zero row and lse -inf.
__global__ __launch_bounds__(kWave) void mla_merge_kernel(MlaArgs a, int items) {
    const int b = blockIdx.x / a.heads;
    const int h = blockIdx.x % a.heads;
    const int item = b * a.nhg + h / 16;
    const int row = h % 16;
    // the context length and the item's slot range are requested together (the range is stale
    // for an item with no key, and then not used)
    const int ctx = a.ctx[b];
    const int2 range = a.sk_wgs > 0 ? *reinterpret_cast<const int2*>(a.seg + 2 * item) : make_int2(0, 0);
    int nact, first = 0;
    int64_t stride;
    if (ctx <= 0) {
        nact = 0;
        stride = 0;
    } else if (a.sk_wgs > 0) {
        nact = range.y;
        if (nact <= 1) return;
        first = range.x;
        stride = 1;
    } else {
        nact = min(a.nsplit, (ctx + a.split_len - 1) / a.split_len);
        first = item;
        stride = items;
    }
    const int c = 8 * threadIdx.x;
    constexpr int CH = 8;
    float M = -INFINITY, wsum = 0.0f;
    f4 acc0 = f4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    for (int s0 = 0; s0 < nact; s0 += CH) {
        float l2[CH], sr[CH];
        h8 po[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            if (s0 + q < nact) {
                const int64_t pr = (first + (int64_t)(s0 + q) * stride) * 16 + row;
                const float2 ls = *reinterpret_cast<const float2*>(a.part_lse + 2 * pr);
                l2[q] = ls.x;
                sr[q] = ls.y;
                po[q] = *reinterpret_cast<const h8*>(a.part_o + pr * DC + c);
            } else {
                l2[q] = -INFINITY;
                sr[q] = 0.0f;
                po[q] = h8{};
            }
        }
        float mc = M;
#pragma unroll
        for (int q = 0; q < CH; ++q) mc = fmaxf(mc, l2[q]);
        if (mc == -INFINITY) continue;
        const float sc = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - mc);
        M = mc;
        wsum *= sc;
        acc0 *= sc;
        acc1 *= sc;
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            const float wt = l2[q] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(l2[q] - M);
            const float ws = wt * sr[q];
            wsum += wt;
            acc0 += ws * f4{(float)po[q][0], (float)po[q][1], (float)po[q][2], (float)po[q][3]};
            acc1 += ws * f4{(float)po[q][4], (float)po[q][5], (float)po[q][6], (float)po[q][7]};
        }
    }
    const float mul = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    uint4 pk;
    pk.x = f32_to_bf16_rne(acc0[0] * mul) | (f32_to_bf16_rne(acc0[1] * mul) << 16);
    pk.y = f32_to_bf16_rne(acc0[2] * mul) | (f32_to_bf16_rne(acc0[3] * mul) << 16);
    pk.z = f32_to_bf16_rne(acc1[0] * mul) | (f32_to_bf16_rne(acc1[1] * mul) << 16);
    pk.w = f32_to_bf16_rne(acc1[2] * mul) | (f32_to_bf16_rne(acc1[3] * mul) << 16);
    *reinterpret_cast<uint4*>(a.out + ((int64_t)b * a.heads + h) * DC + c) = pk;
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
    const int64_t units = a.sk_wgs > 0 ? (items > 0 ? a.sk_wgs + items : 0) : items * a.nsplit;
    if (units == 0) return hipSuccess;
    if (units > 0x7fffffff || (int64_t)a.batch * a.heads > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_decode_kernel, dim3((unsigned)units), dim3(NW * kWave), 0, stream, a, (int)items);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || (a.sk_wgs == 0 && a.nsplit == 1)) return e;
    hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)(a.batch * a.heads)), dim3(DC / 8), 0, stream, a,
                       (int)items);
    return hipGetLastError();
}

int mla_decode_wgs_per_cu() {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mla_decode_kernel, NW * kWave, 0) != hipSuccess)
        return 0;
    return per_cu > 0 ? per_cu : 0;
}

}  // namespace pkv
