// decode_c8.hip - grouped-query attention over the int8 paged cache (per-token, per-block or
// static per-channel scales) on the matrix cores of gfx950.
//
// Same result as decode_valu.hip and decode_mfma.hip (MojoPagedDecodeGQA, Mojo Opset README Op
// List; the cache of PR #379's MojoStorePagedKVCacheC8), with the vector-ALU work per key cut to
// what the HBM roofline of MI355X leaves room for:
//
//  * Scores on the int8 matrix cores, with no conversion of the K codes.  Each query row is
//    multiplied by a power of two and rounded to integers q in [-2^22, 2^22] (relative rounding
//    2^-23 of the row's largest element, so a row with one channel hundreds of times larger than
//    the rest keeps the small channels' precision); q = 65536 hi + 256 mid + lo with int8 digits
//    (exact).  v_mfma_i32_16x16x64_i8 forms K.hi, shifted left by 8, then accumulates K.mid on
//    top (an exact int32 below 2^28), and K.lo in a second accumulator; the two are joined in
//    fp32 as 256 c1 + c2.  The K scale and the power of two come back in the fp32 softmax.
//  * Keys are walked in blocks of 64.  Lane group g (lanes 16g .. 16g+15) owns the 16 keys
//    16g .. 16g+15 of the block, one 16-slot V tile: it loads them as the 16 consecutive bytes of
//    each channel row of that channel-major tile (one 16-byte load per 16 channels; a block reads
//    its four tiles whole, so no cache line is fetched for half its bytes).  The block is cut
//    into four key subsets s = (v, e) = (s / 2, s % 2); subset s holds keys 16g + 8v + 4e + i
//    (i < 4) of every lane group, so that after its score MFMA lane (g, n) holds the weights of
//    exactly those keys.
//  * The 16 columns of every MFMA tile are (row r, subset class j): column n = J r + j with
//    J = 16 / rows in {1, 2, 4}; class j takes the subsets with s % J == j.  Each column runs its
//    own online softmax (running max, weight sum, V-scale reference), so every lane's softmax
//    values are real (row, key) pairs even when a KV head has only 4 query rows; the J partial
//    softmaxes of a row are merged once, after the last block.
//  * P.V as O^T (channels x columns) += V^T P^T on v_mfma_f32_16x16x32_f16, one per 8 keys of
//    each lane group (v = 0, 1) and 16 channels; a code c enters as the fp16 value 1152 + c
//    (exact: a byte permute) and 1152 times the weight sums (an all-ones MFMA) is taken off at
//    the end.  The weights are p * s_v / S with S the column's running max V scale, so they stay
//    in [0, 2^8] in fp16.
//
// One wave per (sequence, KV head, row group, key range), no barriers in the loop; the key ranges
// are fixed splits or the segments of the balanced partition (below), and start at the window
// when a sliding window is set.  The K, V and scale loads of block k+1 are issued while block k
// computes; past the range's keys they read in-bounds stand-ins (the range's last page) that the
// masks give zero weight.  Per-channel scales: the K scales join the query before it is rounded,
// the V scales multiply the output channels, and no scale is loaded per key.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "sk_partition.h"

namespace pkv {
namespace {

typedef int i4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr int BLK = 64;                  // keys per block (four 16-key subsets)
constexpr int MAX_SPLIT = 4096;          // keys per split (planner limit)
constexpr int MAX_SPLIT_PAGES = MAX_SPLIT / 16;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// eight int8 codes (two dwords) -> the fp16 MFMA operand 1152 + code (exact)
__device__ __forceinline__ h8 biased_h8(uint32_t w0, uint32_t w1) {
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;  // code + 128 as unsigned bytes
    const uint32_t r[4] = {__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u),
                           __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)};
    return __builtin_bit_cast(h8, r);
}

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

template <int D, int J>
struct C8Regs {
    i4 k[4][D / 64];         // per subset: the lane's 16 * (D/64) code bytes of one K row
    f4 ks[4 / J], vs[4 / J]; // per slot: the scales of the lane's 4 keys (per-block mode: .x)
};

template <int D>
struct C8V {
    u32x4 v[D / 16];         // per channel tile: the lane group's 16 keys of one channel
};

// The attention of one work item (sequence b, KV head h, row group starting at row r0) over its
// keys [t_seg0, t_seg1) (t_seg0 a multiple of 64).  pslot < 0: the segment is the item's whole key
// range and the result goes to out / lse; else it is a partial, written to rows pslot * prs + j of
// the workspace for the merge.  WIN: a sliding window (DecodeArgs::window) limits each row's keys.
// qs: the wave's LDS for its quantized query rows, QS_I4<D, RT> 16-byte entries.
template <int D, int RT>
constexpr int QS_I4 = 3 * (D / 64) * RT * kWave;

// Bytes of the wave's LDS for a new token it stores: K codes [D], V codes [D], K and V scales.
template <int D>
constexpr int NT_BYTES = 2 * D + 16;

// Quantize the new token of (sequence b, KV head h) at position pos, as the per-token store does
// (per-token absmax scale, or the static per-channel scales), write its codes and scale into the
// cache, and keep them in nt (LDS) for the wave's own attention: the wave then reads them from
// there, not from the memory it has just written.  Lane l takes channels D/64 l ..
template <int D, int MODE>
__device__ __forceinline__ void store_new_token(const DecodeArgs& a, int b, int h, int pos, uint8_t* nt) {
    constexpr int EPL = D / kWave;
    const int lane = threadIdx.x & 63;
    const int64_t page = (int64_t)a.bt[(int64_t)b * a.mbs + (pos >> a.log2bs)] * a.hkv + h;
    const int slot = pos & (a.bs - 1);
    float* nts = reinterpret_cast<float*>(nt + 2 * D);
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = (which ? a.v_new : a.k_new) + ((int64_t)b * a.hkv + h) * D + lane * EPL;
        float x[EPL];
        if constexpr (EPL == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
            x[0] = bf16_to_f32(w & 0xffffu);
            x[1] = bf16_to_f32(w >> 16);
        } else {
            x[0] = bf16_to_f32(src[0]);
        }
        // the cache is the caller's writable memory (read through const pointers elsewhere)
        float* scales = const_cast<float*>(which ? a.vs : a.ks);
        uint8_t* cache = reinterpret_cast<uint8_t*>(const_cast<void*>(which ? a.v : a.k));
        int codes[EPL];
        float s = 0.0f;
        if constexpr (MODE == 3) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) codes[e] = quant_code(x[e], scales[(int64_t)h * D + lane * EPL + e]);
        } else {
            float am = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) am = fmaxf(am, fabsf(x[e]));
            am = group_max<kWave>(am);
            s = absmax_scale(am);
            quant_row_absmax<EPL>(x, s, codes);
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int c = lane * EPL + e;
            if (which == 0) cache[(page * a.bs + slot) * D + c] = (uint8_t)codes[e];
            else cache[v_elem(page, D, a.bs, c, slot)] = (uint8_t)codes[e];
            nt[which * D + c] = (uint8_t)codes[e];
        }
        if constexpr (MODE == 0) {
            if (lane == 0) {
                scales[page * a.bs + slot] = s;
                nts[which] = s;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
}

template <int D, int MODE, int J, int RT, bool WIN, int KD = 1>
__device__ __forceinline__ void c8_segment(const DecodeArgs& a, const int b_, const int h_, const int qlen_,
                                           const int qrow0_, const int prior_, const int r0_, const int nvalid_,
                                           const int t_seg0_, const int t_seg1_, const int64_t pslot,
                                           int* const bt_s, i4* const qs, uint8_t* const nt) {
    static_assert(MODE == 0 || MODE == 1 || MODE == 3, "int8 cache modes only");
    static_assert(J == 1 || RT == 1, "several row tiles only with one subset class");
    constexpr int KSTEP = D / 64;                     // 64-channel steps of the score MFMA
    constexpr int DT = D / 16;                        // 16-channel output tiles
    constexpr int NSLOT = 4 / J;                      // subsets per column per block

    // the item's and segment's values are the same in every lane: kept in scalar registers, so the
    // key loop and every branch on them are uniform control flow (lane-divergent control flow
    // around the matrix-core instructions, which read every lane's operands, must not arise)
    const int b = __builtin_amdgcn_readfirstlane(b_), h = __builtin_amdgcn_readfirstlane(h_);
    const int qlen = __builtin_amdgcn_readfirstlane(qlen_), qrow0 = __builtin_amdgcn_readfirstlane(qrow0_);
    const int prior = __builtin_amdgcn_readfirstlane(prior_), r0 = __builtin_amdgcn_readfirstlane(r0_);
    const int nvalid = __builtin_amdgcn_readfirstlane(nvalid_);
    const int t_seg0 = __builtin_amdgcn_readfirstlane(t_seg0_), t_seg1 = __builtin_amdgcn_readfirstlane(t_seg1_);
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;  // column (scores, weights, accumulators); channel (V operand)
    const int g = lane >> 4;  // lane group
    const int jcol = n % J;   // subset class of the lane's column

    // per-channel mode: the K scales of the lane's query channels (g*16*KSTEP ..)
    f4 skq[MODE == 3 ? 4 * KSTEP : 1];
    if constexpr (MODE == 3) {
        const f4* sp = reinterpret_cast<const f4*>(a.ks + (int64_t)h * D + g * 16 * KSTEP);
#pragma unroll
        for (int i = 0; i < 4 * KSTEP; ++i) skq[i] = sp[i];
    }
    // ---- query rows (B operand of the score MFMA): lane (n, g) holds the 16 * KSTEP channels
    //      g*16*KSTEP .. of its column's row, k-step m taking 16 of them.  The raw bf16 loads are
    //      issued first; they are quantized while the first key block is in flight.
    int lim[RT];  // last key the row may see
    int lo[RT];   // first key the row may see (sliding window)
    bool causal = false;
    u32x4 qraw[RT][2 * KSTEP];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int j = J > 1 ? n / J : rt * 16 + n;
        const bool rv = j < nvalid;
        const int r = r0 + j;
        lim[rt] = rv ? prior + r / a.g : 0x7fffffff;
        lo[rt] = WIN && rv ? win_lo(a.window, lim[rt]) : 0;
        causal |= lim[rt] < t_seg1 - 1;
        const uint16_t* qp = a.q + ((int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g) * D + g * 16 * KSTEP;
#pragma unroll
        for (int l = 0; l < 2 * KSTEP; ++l) qraw[rt][l] = rv ? load16(qp + 8 * l) : u32x4{0u, 0u, 0u, 0u};
    }
    causal = __any(causal);
    // the lowest causal limit over the wave's rows: blocks wholly at or below it need no mask
    int lim_lo = 0x7fffffff;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) lim_lo = min(lim_lo, lim[rt]);
    for (int sh = 1; sh < kWave; sh <<= 1) lim_lo = min(lim_lo, __shfl_xor(lim_lo, sh, kWave));
    lim_lo = __builtin_amdgcn_readfirstlane(lim_lo);
    // one decode step with its store: the wave whose keys end at the new token's position stores it
    // (one query per sequence: the position is the item's last key, prior == t_seg1 - 1)
    bool own_new = false;
    if constexpr (MODE == 0 || MODE == 3) {
        own_new = a.k_new != nullptr && prior >= t_seg0 && prior < t_seg1;
        if (own_new) store_new_token<D, MODE>(a, b, h, prior, nt);
    }
    // the largest window start over the group's rows (its last row's): blocks below it are masked
    const int lo_hi = WIN ? win_lo(a.window, prior + (r0 + nvalid - 1) / a.g) : 0;

    const int32_t* btb = a.bt + (int64_t)b * a.mbs;

    // ---- per-column softmax state, lazily rescaled: the reference max (log2 units) moves only when
    //      a block's max passes it by more than 8, the V-scale reference when a scale passes 16x it
    float mr[RT], lsum[RT];
    f4 acc[RT][DT];
    f4 pacc[RT];  // column weight sums (every row of the tile), for the 1152 code bias
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        mr[rt] = -INFINITY;
        lsum[rt] = 0.0f;
        pacc[rt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[rt][dt] = f4{0.f, 0.f, 0.f, 0.f};
    }
    float sref = 0.0f;  // the column's V-scale reference
    float sinv = 0.0f;

    const uint8_t* kb = reinterpret_cast<const uint8_t*>(a.k) + (int64_t)h * a.bs * D;
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.v) + (int64_t)h * a.bs * D;
    const int64_t page_bytes = (int64_t)a.hkv * a.bs * D;  // one physical block, all heads
    const int rho = lane & 15;                             // score A operand: key row slot
    const int kchunk = rho >> 2;                           // ... whose key is 16 kchunk + 8v + 4e + rho % 4
    const int k_lane = (rho & 3) * D + g * 16 * KSTEP;      // its channels g*16*KSTEP ..
    const int v_lane = n * kVTile;                         // V operand: channel row n of a tile

    const uint32_t ones_w[4] = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};  // fp16 1.0
    const h8 ones = __builtin_bit_cast(h8, ones_w);

    // K and the scales of the next block are loaded as soon as the current block has consumed
    // them (K after the scores, the scales after the softmax); V, consumed last, alternates
    // between two buffers and is loaded first.  Every load is in flight for about one block and
    // no register is copied.
    // key of value i of slot u of lane (g, n): subset q = J u + jcol = (v, e) holds 16g + 8v + 4e + i
    auto key_of = [&](int T, int u, int i) {
        const int q = J * u + jcol;
        return T + 16 * g + 8 * (q >> 1) + 4 * (q & 1) + i;
    };
    // the quantized query rows, digit p (0 hi, 1 mid, 2 lo) of k-step m of row tile rt, are the
    // B operands of the score MFMAs; they live in the wave's LDS (qs) and are read back per block,
    // which keeps them out of the registers the key loop needs
    auto qslot = [&](int p, int rt, int m) -> i4& { return qs[((p * RT + rt) * KSTEP + m) * kWave + lane]; };
    float rowmul[RT];  // |softmax scale| * log2(e) / 2^k: integer score units -> log2 units

    // The segment is walked in ranges of at most MAX_SPLIT keys, each with its block-table slice in
    // LDS; the softmax state carries over.
    for (int tb = t_seg0; tb < t_seg1; tb += MAX_SPLIT) {
        const int t_begin = tb;
        const int t_end = min(tb + MAX_SPLIT, t_seg1);
        const int blk0 = t_begin >> a.log2bs;
        const int lastpg = (t_end - 1) >> a.log2bs;
        const int nblk = lastpg - blk0 + 1;
        if (tb != t_seg0) __builtin_amdgcn_wave_barrier();  // the previous range's LDS reads are done

        // Page and first slot of the 16-key chunk c of the block at T (keys past the split's last
        // page read that page again: in bounds, masked later).
        auto chunk_page = [&](int T, int c) { return min((T + 16 * c) >> a.log2bs, lastpg); };
        auto load_k_at = [&](int T, int pid, C8Regs<D, J>& R) {
            const int sl = (T + 16 * kchunk) & (a.bs - 1);
            const uint8_t* kp = kb + (int64_t)pid * page_bytes + sl * D + k_lane;
    #pragma unroll
            for (int q = 0; q < 4; ++q) {
    #pragma unroll
                for (int m = 0; m < KSTEP; ++m) {
                    const u32x4 w = load16(kp + (8 * (q >> 1) + 4 * (q & 1)) * D + 16 * m);
                    R.k[q][m] = i4{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
                }
            }
        };
        auto load_s_at = [&](int T, int pid, C8Regs<D, J>& R) {
            if constexpr (MODE == 3) return;  // per-channel scales: none per key
            const int sl = (T + 16 * g) & (a.bs - 1);
    #pragma unroll
            for (int u = 0; u < NSLOT; ++u) {  // scales of the lane's keys 16g + 8v + 4e + i, s = (v, e)
                const int q = J * u + jcol;
                if constexpr (MODE == 0) {
                    const int64_t si = ((int64_t)pid * a.hkv + h) * a.bs + sl + 8 * (q >> 1) + 4 * (q & 1);
                    R.ks[u] = *reinterpret_cast<const f4*>(a.ks + si);
                    R.vs[u] = *reinterpret_cast<const f4*>(a.vs + si);
                } else {
                    const int64_t si = (int64_t)pid * a.hkv + h;
                    R.ks[u][0] = a.ks[si];
                    R.vs[u][0] = a.vs[si];
                }
            }
        };
        auto load_v_at = [&](int T, int pid, C8V<D>& R) {
            const int sl = (T + 16 * g) & (a.bs - 1);  // first slot of the lane group's V tile
            const uint8_t* vp = vb + (int64_t)pid * page_bytes + sl * D + v_lane;
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt) R.v[dt] = load16(vp + dt * 16 * kVTile);
        };
        auto load_k = [&](int T, C8Regs<D, J>& R) { load_k_at(T, bt_s[chunk_page(T, kchunk) - blk0], R); };
        auto load_s = [&](int T, C8Regs<D, J>& R) { load_s_at(T, bt_s[chunk_page(T, g) - blk0], R); };
        auto load_v = [&](int T, C8V<D>& R) { load_v_at(T, bt_s[chunk_page(T, g) - blk0], R); };

        // ---- first block: its page ids straight from the block table, its loads issued before the
        //      block-table slice goes to LDS and before the query is quantized
        // K and the scales alternate between KD register sets (KD = 2: loaded two blocks ahead)
        C8Regs<D, J> Ra, Rb;
        C8V<D> v0, v1;
        {
            const int pk = btb[chunk_page(t_begin, kchunk)];
            const int pv = btb[chunk_page(t_begin, g)];
            load_v_at(t_begin, pv, v0);
            load_k_at(t_begin, pk, Ra);
            load_s_at(t_begin, pv, Ra);
        }
        // block-table slice of the split (the wave reads back its own LDS writes in order)
        for (int i = lane; i < nblk; i += kWave) bt_s[i] = btb[blk0 + i];
        __builtin_amdgcn_wave_barrier();
        if constexpr (KD == 2) {  // the second block's K and scales (past the range: in-bounds stand-ins)
            load_k(t_begin + BLK, Rb);
            load_s(t_begin + BLK, Rb);
        }

        if (tb == t_seg0) {
            // ---- quantize the query rows: q * 2^k rounded to integers in [-2^22, 2^22], split exactly as
            //      65536 hi + 256 mid + lo with int8 digits
            const float sgn = a.scale_log2 < 0.0f ? -1.0f : 1.0f;  // a negative scale flips the query
        #pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                float x[16 * KSTEP];
        #pragma unroll
                for (int l = 0; l < 2 * KSTEP; ++l)
        #pragma unroll
                    for (int e = 0; e < 8; ++e) x[8 * l + e] = sgn * bf16_at(qraw[rt][l], e);
                if constexpr (MODE == 3) {  // q . (code * s_K) = (q * s_K) . code: s_K joins the query
        #pragma unroll
                    for (int e = 0; e < 16 * KSTEP; ++e) x[e] *= skq[e / 4][e % 4];
                }
                float mx = 0.0f;
        #pragma unroll
                for (int e = 0; e < 16 * KSTEP; ++e) mx = fmaxf(mx, fabsf(x[e]));
                mx = col_max(mx);
                int ex = 0;
                if (mx > 0.0f) (void)frexpf(mx, &ex);        // mx in [2^(ex-1), 2^ex)
                const int k = min(120, max(-120, 22 - ex));  // |x| * 2^k < 2^22
                const float up = ldexpf(1.0f, k);
        #pragma unroll
                for (int m = 0; m < KSTEP; ++m) {
                    i4 qh, qm, ql;
        #pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        uint32_t hw = 0, mw = 0, lw = 0;
        #pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int qi = (int)__builtin_rintf(x[16 * m + 4 * w + e] * up);  // |qi| <= 2^22
                            const int lo = ((qi + 128) & 255) - 128;
                            const int r1 = (qi - lo) >> 8;                                  // |r1| <= 2^14
                            const int md = ((r1 + 128) & 255) - 128;
                            const int hi = (r1 - md) >> 8;                                  // |hi| <= 64
                            hw |= (uint32_t)(hi & 255) << (8 * e);
                            mw |= (uint32_t)(md & 255) << (8 * e);
                            lw |= (uint32_t)(lo & 255) << (8 * e);
                        }
                        qh[w] = (int)hw;
                        qm[w] = (int)mw;
                        ql[w] = (int)lw;
                    }
                    qslot(0, rt, m) = qh;
                    qslot(1, rt, m) = qm;
                    qslot(2, rt, m) = ql;
                }
                // floored at 2^-126: a hidden key's -inf score must stay -inf (a zero scale would
                // make it NaN), and below the floor every logit difference is far under fp32's
                // resolution of exp2 near 1, so a zero scale still weighs every visible key 1
                rowmul[rt] = fmaxf(fabsf(a.scale_log2) * ldexpf(1.0f, -k), 0x1p-126f);
            }

        }

        auto block = [&](const int T, const C8V<D>& VC, C8V<D>& VN, C8Regs<D, J>& R) {
            // masked: the block runs past the split's keys, past some row's causal limit or below
            // some row's window start
            const bool MASKED = (causal && T + BLK - 1 > lim_lo) || T + BLK > t_end || (WIN && T < lo_hi);
            // the next block's V: loaded first (past the split's end: in-bounds stand-ins, never
            // weighted), except with one 16-row tile and one subset class, where it is loaded after
            // this block's P.V into the same registers: that keeps those kernels within 256
            // registers, two waves per SIMD (measured on the chunked decode: 390 against 398 us)
            constexpr bool V_LATE = RT == 1 && J == 1;
            if constexpr (!V_LATE) load_v(T + BLK, VN);
            // keep the next block's loads ahead of this block's waits (the scheduler would otherwise
            // sink them below the first score MFMA, whose wait then drains every load in flight)
            __builtin_amdgcn_sched_barrier(0);

            // -------------------------------------------- scores: two int32 tiles per subset,
            //      c1 = 256 K.hi + K.mid and c2 = K.lo (the score is 256 c1 + c2)
            i4 sc[RT][4], sc2[RT][4];
    #pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                i4 qb[KSTEP];
    #pragma unroll
                for (int m = 0; m < KSTEP; ++m) qb[m] = qslot(0, rt, m);
    #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    i4 c = i4{0, 0, 0, 0};
    #pragma unroll
                    for (int m = 0; m < KSTEP; ++m)
                        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.k[q][m], qb[m], c, 0, 0, 0);
                    sc[rt][q] = c * 256;
                }
    #pragma unroll
                for (int m = 0; m < KSTEP; ++m) qb[m] = qslot(1, rt, m);
    #pragma unroll
                for (int q = 0; q < 4; ++q)
    #pragma unroll
                    for (int m = 0; m < KSTEP; ++m)
                        sc[rt][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.k[q][m], qb[m], sc[rt][q], 0, 0, 0);
    #pragma unroll
                for (int m = 0; m < KSTEP; ++m) qb[m] = qslot(2, rt, m);
    #pragma unroll
                for (int q = 0; q < 4; ++q) {
                    i4 c2 = i4{0, 0, 0, 0};
    #pragma unroll
                    for (int m = 0; m < KSTEP; ++m)
                        c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(R.k[q][m], qb[m], c2, 0, 0, 0);
                    sc2[rt][q] = c2;
                }
            }
            load_k(T + KD * BLK, R);
            __builtin_amdgcn_sched_barrier(0);

            // -------------------------------------------- scores in integer units times the K scales
            float x[RT][NSLOT][4];
    #pragma unroll
            for (int rt = 0; rt < RT; ++rt)
    #pragma unroll
                for (int u = 0; u < NSLOT; ++u) {
                    i4 S = sc[rt][J * u], S2 = sc2[rt][J * u];
    #pragma unroll
                    for (int c = 1; c < J; ++c)
                        if (jcol == c) {
                            S = sc[rt][J * u + c];
                            S2 = sc2[rt][J * u + c];
                        }
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float si = __builtin_fmaf((float)S[i], 256.0f, (float)S2[i]);
                        x[rt][u][i] = si * (MODE == 0 ? R.ks[u][i] : (MODE == 1 ? R.ks[u][0] : 1.0f));
                    }
                }
            float vsl[NSLOT][4];
    #pragma unroll
            for (int u = 0; u < NSLOT; ++u)
    #pragma unroll
                for (int i = 0; i < 4; ++i) vsl[u][i] = MODE == 0 ? R.vs[u][i] : (MODE == 1 ? R.vs[u][0] : 1.0f);
            // -------------------------------------------- the mask, one scalar branch for the whole block:
            //      hidden keys score -inf; slots past the keys may never have been written, so their
            //      (possibly non-finite) V scales must not reach a weight or the column's reference
            if (MASKED) {
    #pragma unroll
                for (int u = 0; u < NSLOT; ++u)
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = key_of(T, u, i);
                        if (!(t < t_end)) vsl[u][i] = 0.0f;
    #pragma unroll
                        for (int rt = 0; rt < RT; ++rt)
                            if (!(t < t_end && t <= lim[rt] && (!WIN || t >= lo[rt]))) x[rt][u][i] = -INFINITY;
                    }
            }

            // -------------------------------------------- V-scale reference of the column
            float sf = 1.0f;
            bool s_moved = false;
            {
                float vmax = 0.0f;
    #pragma unroll
                for (int u = 0; u < NSLOT; ++u)
    #pragma unroll
                    for (int i = 0; i < 4; ++i) vmax = fmaxf(vmax, vsl[u][i]);
                vmax = col_max(vmax);
                if (vmax > 16.0f * sref) {  // (also the first block: sref == 0)
                    sf = sref > 0.0f ? sref * __builtin_amdgcn_rcpf(vmax) : 0.0f;
                    sref = vmax;
                    sinv = __builtin_amdgcn_rcpf(vmax);
                    s_moved = true;
                }
            }
    #pragma unroll
            for (int u = 0; u < NSLOT; ++u)
    #pragma unroll
                for (int i = 0; i < 4; ++i) vsl[u][i] *= sinv;

            // -------------------------------------------- online softmax per column, P operands
            uint32_t wpk[RT][NSLOT][2];
            float factor[RT];
            bool any_rescale = s_moved;
    #pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                float bmax = -INFINITY;
    #pragma unroll
                for (int u = 0; u < NSLOT; ++u)
    #pragma unroll
                    for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, x[rt][u][i]);
                bmax = col_max(bmax) * rowmul[rt];
                float alpha = 1.0f;
                if (bmax > mr[rt] + 8.0f) {  // (also the first block: mr == -inf)
                    alpha = __builtin_amdgcn_exp2f(mr[rt] - bmax);
                    mr[rt] = bmax;
                }
                // a column with no visible key yet keeps mr = -inf; its weights are taken against 0,
                // so that a hidden key (-inf times the positive rowmul) weighs exactly 0
                const float mref = mr[rt] == -INFINITY ? 0.0f : mr[rt];
                float ps = 0.0f;
    #pragma unroll
                for (int u = 0; u < NSLOT; ++u) {
                    float p[4];
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[rt][u][i], rowmul[rt], -mref));
                        ps += p[i];
                    }
                    const h4 w = {(_Float16)(p[0] * vsl[u][0]), (_Float16)(p[1] * vsl[u][1]),
                                  (_Float16)(p[2] * vsl[u][2]), (_Float16)(p[3] * vsl[u][3])};
                    const auto wb = __builtin_bit_cast(uint2, w);
                    wpk[rt][u][0] = wb.x;
                    wpk[rt][u][1] = wb.y;
                }
                lsum[rt] = lsum[rt] * alpha + ps;
                factor[rt] = alpha * sf;
                any_rescale |= alpha != 1.0f;
            }

            load_s(T + KD * BLK, R);
            __builtin_amdgcn_sched_barrier(0);

            // -------------------------------------------- rescale the columns whose references moved
            if (__any(any_rescale)) {
    #pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
    #pragma unroll
                    for (int dt = 0; dt < DT; ++dt) acc[rt][dt] *= factor[rt];
                    pacc[rt] *= factor[rt];
                }
            }

            // -------------------------------------------- P.V (+ weight sums): per lane group, keys
            //      16g + 8v .. +8 of subset pair (v, 0), (v, 1)
    #pragma unroll
            for (int v = 0; v < 2; ++v) {
                h8 bq[RT];
    #pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    uint32_t ww[4];
    #pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int q = 2 * v + e;  // subset of keys 16g + 8v + 4e ..
                        const int u = q / J;
                        const bool mine = J == 1 || jcol == q % J;  // else the subset is another class's
                        ww[2 * e] = mine ? wpk[rt][u][0] : 0u;
                        ww[2 * e + 1] = mine ? wpk[rt][u][1] : 0u;
                    }
                    bq[rt] = __builtin_bit_cast(h8, ww);
                }
    #pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const h8 av = v == 0 ? biased_h8(VC.v[dt].x, VC.v[dt].y) : biased_h8(VC.v[dt].z, VC.v[dt].w);
    #pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bq[rt], acc[rt][dt], 0, 0, 0);
                }
    #pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    pacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, bq[rt], pacc[rt], 0, 0, 0);
            }
            if constexpr (V_LATE) load_v(T + BLK, VN);
        };
        // The block that holds the stored new token takes its codes and scales from nt (the cache
        // was written by this wave a moment ago; its loads of that slot are replaced, not trusted).
        // The block is the same for the whole wave; which lanes hold the key depends on the lane,
        // so the replacement is made of selects, with no lane-divergent branch.
        auto patch_new = [&](const int T, C8V<D>& VC, C8Regs<D, J>& R) {
            const int kk = prior - T;  // the new key within the block
            const int kc = kk >> 4, qn = 2 * ((kk >> 3) & 1) + ((kk >> 2) & 1), ii = kk & 3;
            const bool krow = rho == 4 * kc + ii;  // K: the score row of that key, channels g 16 KSTEP ..
    #pragma unroll
            for (int m = 0; m < KSTEP; ++m) {
                const uint4 w = *reinterpret_cast<const uint4*>(nt + g * 16 * KSTEP + 16 * m);
                const i4 val = i4{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
    #pragma unroll
                for (int qq = 0; qq < 4; ++qq) R.k[qq][m] = krow && qq == qn ? val : R.k[qq][m];
            }
            const bool vgrp = g == kc;  // the lane group whose keys hold it
            if constexpr (MODE == 0) {  // its K and V scales
                const float* nts = reinterpret_cast<const float*>(nt + 2 * D);
                const float ksn = nts[0], vsn = nts[1];
                const bool col = vgrp && jcol == qn % J;
    #pragma unroll
                for (int u = 0; u < NSLOT; ++u)
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool hit = col && u == qn / J && i == ii;
                        R.ks[u][i] = hit ? ksn : R.ks[u][i];
                        R.vs[u][i] = hit ? vsn : R.vs[u][i];
                    }
            }
            // V: byte kk % 16 of the lane's 16-slot rows of channels n + 16 dt
            const int sh = 8 * (kk & 3), wd = (kk >> 2) & 3;
            const uint32_t keep = ~(0xffu << sh);
    #pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint32_t put = (uint32_t)nt[D + n + 16 * dt] << sh;
                const u32x4 o = VC.v[dt];
                VC.v[dt] = u32x4{vgrp && wd == 0 ? (o.x & keep) | put : o.x, vgrp && wd == 1 ? (o.y & keep) | put : o.y,
                                 vgrp && wd == 2 ? (o.z & keep) | put : o.z, vgrp && wd == 3 ? (o.w & keep) | put : o.w};
            }
        };
        for (int T = t_begin;;) {
            if (own_new && prior >= T && prior < T + BLK) patch_new(T, v0, Ra);
            block(T, v0, v1, Ra);
            T += BLK;
            if (T >= t_end) break;
            if (own_new && prior >= T && prior < T + BLK) patch_new(T, v1, KD == 2 ? Rb : Ra);
            block(T, v1, v0, KD == 2 ? Rb : Ra);
            T += BLK;
            if (T >= t_end) break;
        }

    }


    // ---- merge the J columns of each row, normalise, write.  Lane (g, n) holds channels
    //      16 dt + 4g + i of column n.  Per-channel mode: sum_t w_t code_t,c * s_V,c is the
    //      accumulator times the channel's V scale (loaded here, in flight during the merge).
    f4 svc[MODE == 3 ? DT : 1];
    if constexpr (MODE == 3) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            svc[dt] = *reinterpret_cast<const f4*>(a.vs + (int64_t)h * D + dt * 16 + 4 * g);
    }
    const bool split_mode = pslot >= 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const float l = col_sum(lsum[rt]);
        float M = mr[rt];
        if constexpr (J >= 2) M = fmaxf(M, lane_xchg<1>(M));
        if constexpr (J >= 4) M = fmaxf(M, lane_xchg<2>(M));
        const float f = mr[rt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mr[rt] - M);
        float L = l * f;
        if constexpr (J >= 2) L += lane_xchg<1>(L);
        if constexpr (J >= 4) L += lane_xchg<2>(L);
        const float cm = f * sref;
        const float bias = 1152.0f * pacc[rt][0];
        f4 o[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = (acc[rt][dt][i] - bias) * cm;
                if constexpr (MODE == 3) v *= svc[dt][i];
                if constexpr (J >= 2) v += lane_xchg<1>(v);
                if constexpr (J >= 4) v += lane_xchg<2>(v);
                o[dt][i] = v;
            }
        }
        const int j = J > 1 ? n / J : rt * 16 + n;  // row within the group
        if (jcol != 0 || j >= nvalid) continue;
        const float mul = L > 0.0f ? 1.0f / L : 0.0f;
        const int r = r0 + j;
        const int64_t orow = (int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g;
        const int64_t prow = pslot * a.prs + j;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = dt * 16 + 4 * g;
            if (!split_mode) {
                uint2 pk;
                pk.x = f32_to_bf16_rne(o[dt][0] * mul) | (f32_to_bf16_rne(o[dt][1] * mul) << 16);
                pk.y = f32_to_bf16_rne(o[dt][2] * mul) | (f32_to_bf16_rne(o[dt][3] * mul) << 16);
                *reinterpret_cast<uint2*>(a.out + orow * D + d) = pk;
            } else {
                *reinterpret_cast<f4*>(a.part_o + prow * D + d) = o[dt] * mul;
            }
        }
        if (g == 0) {
            const float lse2 = L > 0.0f ? M + log2f(L) : -INFINITY;
            if (!split_mode) {
                if (a.lse) a.lse[orow] = lse2 * kLn2;
            } else {
                a.part_lse[prow] = lse2;
            }
        }
    }
}

// Fixed partition: one wave per (item, split of split_len keys).  Pairs u = (split, sequence x
// KV head) go fastest, so consecutive workgroups go round-robin over the XCDs and each XCD gets an
// even share whatever the number of empty splits; the row groups of one pair (which read the
// same keys) take workgroups 8 apart, so they run on one XCD at about the same time and all but
// the first read the keys from its L2.  Workgroup 8 (q nrg + c) + x takes row group nrg - 1 - c of
// pair 8 q + x: a causal chunk's or prompt's last row groups, which see the most keys, start first
// and the short ones fill the end of the launch (measured on a 4 x 2048-token prefill: 323 against
// 358 us with the short ones first).
template <int D, int MODE, int J, int RT, bool WIN>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(J > 1 ? 2 : 1))) void decode_c8_kernel(DecodeArgs a, int pairs) {
    constexpr int ROWS = J > 1 ? 16 / J : 16 * RT;
    __shared__ int bt_s[MAX_SPLIT_PAGES];
    __shared__ i4 qs[QS_I4<D, RT>];
    __shared__ __attribute__((aligned(16))) uint8_t nt[NT_BYTES<D>];
    const int wi = blockIdx.x;
    const int rest = wi >> 3;
    const int u = (rest / a.nrg) * 8 + (wi & 7);
    if (u >= pairs) return;
    const int nbh = pairs / a.nsplit;
    const int s = u / nbh;
    const int item = (u % nbh) * a.nrg + (a.nrg - 1 - rest % a.nrg);
    const ItemGeo it = item_geo<ROWS, WIN>(a, item);
    if (it.nvalid <= 0) return;
    if (it.kmax <= 0) {
        if (s == 0) zero_rows<D>(a, it, threadIdx.x);
        return;
    }
    const int t_begin = it.kmin + s * a.split_len;
    if (t_begin >= it.kmax) return;
    const int t_end = min(t_begin + a.split_len, it.kmax);
    c8_segment<D, MODE, J, RT, WIN>(a, it.b, it.h, it.qlen, it.qrow0, it.prior, it.r0, it.nvalid, t_begin, t_end,
                               a.nsplit > 1 ? (int64_t)item * a.nsplit + s : -1, bt_s, qs, nt);
}

// Balanced partition (sk_partition.h): one wave per segment of the plan.
template <int D, int MODE, int J, int RT, bool WIN>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1))) void decode_c8_sk_kernel(DecodeArgs a, int batch) {
    constexpr int ROWS = J > 1 ? 16 / J : 16 * RT;
    __shared__ int bt_s[MAX_SPLIT_PAGES];
    __shared__ i4 qs[QS_I4<D, RT>];
    __shared__ __attribute__((aligned(16))) uint8_t nt[NT_BYTES<D>];
    extern __shared__ int kseq[];  // [batch + 1] prefix sums over sequences of their waves
    SkSegment sg;
    if (!sk_plan<ROWS, WIN>(a, batch, blockIdx.x, kseq, sg)) return;
    const ItemGeo& it = sg.it;
    // one wave per SIMD (the planner's choice) leaves registers for K two blocks ahead; measured on
    // MI355X: 284.6 -> 282.0 us on the long-context decode with per-token scales, while with
    // static per-channel scales (no scale loads per key) it measured slower (269.5 -> 272.8 us)
    constexpr int KD = RT == 1 && MODE != 3 ? 2 : 1;
    c8_segment<D, MODE, J, RT, WIN, KD>(a, it.b, it.h, it.qlen, it.qrow0, it.prior, it.r0, it.nvalid, sg.t0, sg.t1,
                                    sg.pslot, bt_s, qs, nt);
}

template <int D, int MODE, int J, int RT, bool WIN>
hipError_t launch_one_w(const DecodeArgs& a, int batch, hipStream_t stream) {
    constexpr int ROWS = J > 1 ? 16 / J : 16 * RT;
    const int64_t items = (int64_t)batch * a.hkv * a.nrg;
    if (items == 0) return hipSuccess;
    if (a.sk_waves > 0) {  // balanced partition
        if (batch > SK_MAX_SEQS) return hipErrorInvalidValue;
        const size_t lds = (size_t)(batch + 1) * sizeof(int);
        hipLaunchKernelGGL((decode_c8_sk_kernel<D, MODE, J, RT, WIN>), dim3((unsigned)(a.sk_waves + items)), dim3(64),
                           lds, stream, a, batch);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_merge_sk<D, ROWS>(a, items, stream);
    }
    const int64_t pairs = (int64_t)batch * a.hkv * a.nsplit;  // (split, sequence x KV head)
    const int64_t grid = (pairs + 7) / 8 * 8 * a.nrg;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_c8_kernel<D, MODE, J, RT, WIN>), dim3((unsigned)grid), dim3(64), 0, stream, a, (int)pairs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_merge(a, batch, D, ROWS, stream);
}

template <int D, int MODE, int J, int RT>
hipError_t launch_one(const DecodeArgs& a, int batch, hipStream_t stream) {
    return a.window > 0 ? launch_one_w<D, MODE, J, RT, true>(a, batch, stream)
                        : launch_one_w<D, MODE, J, RT, false>(a, batch, stream);
}

template <int D, int MODE, int J, int RT>
int sk_waves_one(int batch, bool windowed) {
    int per_cu = 0;
    const size_t lds = (size_t)(batch + 1) * sizeof(int);
    const hipError_t e = windowed
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_c8_sk_kernel<D, MODE, J, RT, true>, 64, lds)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_c8_sk_kernel<D, MODE, J, RT, false>, 64, lds);
    if (e != hipSuccess || per_cu <= 0) return 0;
    return per_cu;
}

template <int D, int MODE>
hipError_t launch_shape(const DecodeArgs& a, int batch, int j, int rt, hipStream_t stream) {
    if (j == 4 && rt == 1) return launch_one<D, MODE, 4, 1>(a, batch, stream);
    if (j == 2 && rt == 1) return launch_one<D, MODE, 2, 1>(a, batch, stream);
    if (j == 1 && rt == 1) return launch_one<D, MODE, 1, 1>(a, batch, stream);
    if (j == 1 && rt == 2) return launch_one<D, MODE, 1, 2>(a, batch, stream);
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_mode(const DecodeArgs& a, int batch, int j, int rt, int mode, hipStream_t stream) {
    if (mode == 0) return launch_shape<D, 0>(a, batch, j, rt, stream);
    if (mode == 1) return launch_shape<D, 1>(a, batch, j, rt, stream);
    if (mode == 3) return launch_shape<D, 3>(a, batch, j, rt, stream);
    return hipErrorInvalidValue;
}

template <int D, int MODE>
int sk_shape(int j, int rt, int batch, bool w) {
    if (j == 4 && rt == 1) return sk_waves_one<D, MODE, 4, 1>(batch, w);
    if (j == 2 && rt == 1) return sk_waves_one<D, MODE, 2, 1>(batch, w);
    if (j == 1 && rt == 1) return sk_waves_one<D, MODE, 1, 1>(batch, w);
    if (j == 1 && rt == 2) return sk_waves_one<D, MODE, 1, 2>(batch, w);
    return 0;
}

}  // namespace

int decode_c8_waves_per_cu(int head_dim, int classes, int row_tiles, int mode, int batch, bool windowed) {
    if (batch > SK_MAX_SEQS) return 0;
    const int c = classes, r = row_tiles;
    const bool w = windowed;
    if (head_dim == 64)
        return mode == 0 ? sk_shape<64, 0>(c, r, batch, w)
                         : (mode == 1 ? sk_shape<64, 1>(c, r, batch, w) : sk_shape<64, 3>(c, r, batch, w));
    if (head_dim == 128)
        return mode == 0 ? sk_shape<128, 0>(c, r, batch, w)
                         : (mode == 1 ? sk_shape<128, 1>(c, r, batch, w) : sk_shape<128, 3>(c, r, batch, w));
    return 0;
}

hipError_t launch_decode_c8(const DecodeArgs& a, int batch, int head_dim, int classes, int row_tiles,
                            int mode, hipStream_t stream) {
    if (a.sk_waves <= 0 && (a.split_len > MAX_SPLIT || (a.split_len % BLK) != 0)) return hipErrorInvalidValue;
    if (head_dim == 64) return launch_mode<64>(a, batch, classes, row_tiles, mode, stream);
    if (head_dim == 128) return launch_mode<128>(a, batch, classes, row_tiles, mode, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
