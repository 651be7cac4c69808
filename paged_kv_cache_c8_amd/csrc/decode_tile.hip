// decode_tile.hip - grouped-query attention of many query rows per KV head over the int8 paged cache
// (paged prefill and multi-token chunks; MojoPagedPrefillGQA / MojoPagedDecodeGQA, Mojo Opset README
// Op List), on the matrix cores of gfx950.
//
// The per-wave decode kernels stream every key block once per row group; with tens or hundreds of
// query rows per KV head the same block is then read (and its V codes converted) once per group.
// Here one workgroup of four waves takes a tile of 128 query rows of one (sequence, KV head), 32
// rows per wave (rows 16w .. 16w + 15 and 64 + 16w .. 64 + 16w + 15, so that a tile partly filled
// still spreads over the four SIMDs; a wave whose second 16 rows are all past the tile's rows does
// the work of its first 16 only), and walks the keys the tile's last row sees in blocks of 64:
//   * the four waves load each block together (16 bytes of K, 16 of V and one scale per thread
//     per load, two blocks in flight), convert the int8 codes to fp16 once (exact: code and
//     1152 + code are both fp16 integers) and store K token-major and V channel-major in LDS,
//     double-buffered, with one workgroup barrier per block;
//   * each wave forms its rows' scores on the matrix cores in fp16 (v_mfma_f32_16x16x32_f16):
//     S^T (keys x rows) = K . Q^T, the query rows pre-scaled by a power of two into fp16's range
//     (the factor and the per-key K scale applied to the fp32 scores);
//   * online softmax per row, lazily rescaled (the reference max moves only when a block's max
//     passes it by more than 8, the V-scale reference when a V scale passes 16x it);
//   * O^T (channels x rows) += V^T . P^T, so that every lane holds channels of its own row and the
//     rescaling never leaves the lane.
// Key splits: with a.nsplit > 1 the workgroup takes split s (keys [s L, (s + 1) L) of the tile's
// range, L = a.split_len) and writes partials that the log-sum-exp merge combines; the
// rows' causal limits are clamped to the split's last key.  Each thread loads the two block-table
// entries its loads of a block need one block ahead of those loads (no table slice in LDS, no
// limit on the context).  Per-token and per-block scales only: with static
// per-channel scales the K scale sits inside each dot product, and folding it into an fp16 query
// would round it to 11 bits (the int8-score kernel serves those caches).
#include <cstddef>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"
#include "sk_partition.h"

namespace pkv {
namespace {

typedef _Float16 th8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float tf2 __attribute__((ext_vector_type(2)));
typedef _Float16 th2 __attribute__((ext_vector_type(2)));
typedef const float __attribute__((address_space(3))) lds_cf;  // LDS pointers (32-bit)
typedef const f4 __attribute__((address_space(3))) lds_cf4;

constexpr int TD = 128;          // head dim
constexpr int TW = 4;            // waves per workgroup
constexpr int TROWS = 32 * TW;   // query rows per tile
constexpr int TBLK = 64;         // keys per block
constexpr int KP = TD + 8;       // LDS pitch of a K row (halves): rows start 4 banks apart
constexpr int VP = TBLK + 8;     // LDS pitch of a V channel row (halves)
constexpr float kLn2t = 0.6931471805599453f;

struct __align__(16) TileShared {
    _Float16 k[2][TBLK][KP];   // K codes of the block, token-major (rows in score-operand order)
    _Float16 v[2][TD][VP];     // V codes of the block, channel-major
    float ks[2][TBLK];         // per-key K scale (0 past the keys)
    float vs[2][TBLK];         // per-key V scale (0 past the keys)
};
static_assert(offsetof(TileShared, vs) == offsetof(TileShared, ks) + 2 * TBLK * sizeof(float),
              "the V scales follow the K scales");

// the raw loads of one block by one thread: 32 K codes (a quarter of a key row), 32 V codes (two
// channel rows of a 16-slot tile) and one scale
struct TileRaw {
    u32x4 k0, k1, v0, v1;
    float s;
};

// the block-table entries of one thread's loads of a block: the page of its key (K) and of its V tile
struct TilePg {
    int k, v;
};

// eight int8 codes (two dwords) -> eight fp16 values, exactly: the byte permute makes 1152 + code,
// one packed subtraction removes 1152
__device__ __forceinline__ th8 codes_h8(uint32_t w0, uint32_t w1) {
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;  // code + 128 as unsigned bytes
    const uint32_t r[4] = {__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u),
                           __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u),
                           __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)};
    const th8 bias = {(_Float16)1152.0f, (_Float16)1152.0f, (_Float16)1152.0f, (_Float16)1152.0f,
                      (_Float16)1152.0f, (_Float16)1152.0f, (_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(th8, r) - bias;
}

// max / sum over the four lanes n, n+16, n+32, n+48 (one query row), by permlane swaps
__device__ __forceinline__ float row_max4(float x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}
__device__ __forceinline__ int wave_min(int x) {
    for (int d = 1; d < kWave; d <<= 1) x = min(x, __shfl_xor(x, d, kWave));
    return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ int wave_max(int x) {
    for (int d = 1; d < kWave; d <<= 1) x = max(x, __shfl_xor(x, d, kWave));
    return __builtin_amdgcn_readfirstlane(x);
}

// Workgroup u takes split u / V of row tile nrg - 1 - v / (batch * hkv) of pair v % (batch * hkv),
// v = u % V, V = batch * hkv * nrg: the tiles that see the most keys (a chunk's last rows) first,
// split-major.  Workgroups go to the XCDs round-robin, so with batch * hkv a multiple of 8 every
// tile and split of a (sequence, KV head) pair lands on one XCD, whose L2 then serves that pair's
// keys to all of them (with the splits of a tile adjacent, each XCD would take one key range of
// every pair instead: about twice the time per block on long prompts).
template <int MODE>
__global__ __launch_bounds__(TW * kWave) __attribute__((amdgpu_waves_per_eu(2))) void decode_tile_kernel(
    DecodeArgs a, int nbh) {
    __shared__ TileShared S;
    const int nv = nbh * a.nrg;
    const int sp = blockIdx.x / nv;
    const int v = blockIdx.x % nv;
    const int item = (v % nbh) * a.nrg + (a.nrg - 1 - v / nbh);
    const ItemGeo it = item_geo<TROWS, false>(a, item);
    if (it.nvalid <= 0) return;  // uniform per workgroup
    const int b = it.b, h = it.h;
    // keys [t0, kmax): this split of what the tile's last row sees (nsplit 1: all of it)
    const int t0 = sp * a.split_len;
    if (t0 >= it.kmax) return;  // (uniform; the merge reads no partial past the keys)
    const int kmax = a.nsplit > 1 ? min(t0 + a.split_len, it.kmax) : it.kmax;
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int n = lane & 15;
    const int g = lane >> 4;

    // ---- cooperative loads of the block at T: thread tid takes key T + tid / 4 (bytes 32 (tid % 4)
    //      .. of its K row), channels 2 (tid % 64), + 1 of V tile tid / 64, and (tid % 4 < 2) the
    //      key's K (0) or V (1) scale.  Keys past kmax read the last key's row and the V tile
    //      holding it (in bounds), and get scale 0.
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k);
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v);
    const int64_t hd = (int64_t)a.bs * TD;  // bytes of one (page, head)
    const int32_t* btrow = a.bt + (int64_t)b * a.mbs;
    auto load_pg = [&](int T, TilePg& P) __attribute__((always_inline)) {
        const int key = min(T + (tid >> 2), kmax - 1);
        const int tt = min(T + 16 * (tid >> 6), (kmax - 1) & ~15);  // first key of the V tile
        P.k = btrow[key >> a.log2bs];
        P.v = btrow[tt >> a.log2bs];
    };
    auto load_raw = [&](int T, const TilePg& P, TileRaw& R) __attribute__((always_inline)) {
        const int key = min(T + (tid >> 2), kmax - 1);
        const int64_t pk = (int64_t)P.k * a.hkv + h;
        const uint8_t* kp = kbase + pk * hd + (key & (a.bs - 1)) * TD + (tid & 3) * 32;
        R.k0 = load16(kp);
        R.k1 = load16(kp + 16);
        const int tt = min(T + 16 * (tid >> 6), (kmax - 1) & ~15);  // first key of the V tile
        const int64_t pv = (int64_t)P.v * a.hkv + h;
        const uint8_t* vp = vbase + pv * hd + ((tt & (a.bs - 1)) >> 4) * (TD * kVTile) + (tid & 63) * 32;
        R.v0 = load16(vp);
        R.v1 = load16(vp + 16);
        R.s = 0.0f;
        if constexpr (MODE == 0) {
            if ((tid & 2) == 0) R.s = ((tid & 1) ? a.vs : a.ks)[pk * a.bs + (key & (a.bs - 1))];
        } else {
            if ((tid & 2) == 0) R.s = ((tid & 1) ? a.vs : a.ks)[pk];
        }
    };
    auto store_lds = [&](const TileRaw& R, int buf, int T) __attribute__((always_inline)) {
        const int kl = tid >> 2;
        // key kl of the block goes to row 32 hf + 16 u + rho, the row slot rho of score tile u of
        // half hf that holds it (kl = 32 hf + 8 (rho / 4) + 4 u + rho % 4): a tile's 16 lanes then
        // read 16 consecutive rows, 4 banks apart, without conflicts
        const int krow_l = (kl & 32) + ((kl & 4) << 2) + ((kl & 24) >> 1) + (kl & 3);
        _Float16* kd = &S.k[buf][krow_l][(tid & 3) * 32];
        *reinterpret_cast<th8*>(kd) = codes_h8(R.k0.x, R.k0.y);
        *reinterpret_cast<th8*>(kd + 8) = codes_h8(R.k0.z, R.k0.w);
        *reinterpret_cast<th8*>(kd + 16) = codes_h8(R.k1.x, R.k1.y);
        *reinterpret_cast<th8*>(kd + 24) = codes_h8(R.k1.z, R.k1.w);
        const int c = 2 * (tid & 63), s0 = 16 * (tid >> 6);
        *reinterpret_cast<th8*>(&S.v[buf][c][s0]) = codes_h8(R.v0.x, R.v0.y);
        *reinterpret_cast<th8*>(&S.v[buf][c][s0 + 8]) = codes_h8(R.v0.z, R.v0.w);
        *reinterpret_cast<th8*>(&S.v[buf][c + 1][s0]) = codes_h8(R.v1.x, R.v1.y);
        *reinterpret_cast<th8*>(&S.v[buf][c + 1][s0 + 8]) = codes_h8(R.v1.z, R.v1.w);
        if ((tid & 2) == 0) {
            const bool in = T + kl < kmax;  // past the keys: 0, so that nothing unwritten is used
            ((tid & 1) ? S.vs[buf] : S.ks[buf])[kl] = in ? R.s : 0.0f;
        }
    };

    // ---- this wave's query rows (B operand of the score MFMA): rows 64rt + 16w + n of the tile;
    //      lane (n, g) holds channels 32m + 8g .. + 7 of k-step m, scaled by 2^k into fp16's range
    //      (exact: a bf16 value times a power of two fits fp16's 11 significant bits)
    uint32_t qf[2][4][4];
    float rowmul[2];  // |softmax scale| * log2(e) / 2^k, floored at 2^-126 (below)
    const float sgn = a.scale_log2 < 0.0f ? -1.0f : 1.0f;  // a negative scale flips the query
    int lim[2];       // last key the row sees (invalid rows: none masked, nothing written)
    bool rowv[2];
    u32x4 qraw[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int j = 64 * rt + 16 * w + n;
        rowv[rt] = j < it.nvalid;
        const int r = it.r0 + j;
        // (a split: clamped to its last key, so that the next split's keys are masked like causal ones)
        lim[rt] = rowv[rt] ? min(it.prior + r / a.g, kmax - 1) : 0x7fffffff;
        // (loaded unconditionally, so that nothing waits for them before the conversion: a row
        // past the tile's rows reads its last row, in bounds, and is zeroed below)
        const int rq = it.r0 + min(j, it.nvalid - 1);
        const uint16_t* qp = a.q + ((int64_t)(it.qrow0 + rq / a.g) * a.hq + h * a.g + rq % a.g) * TD + 8 * g;
#pragma unroll
        for (int m = 0; m < 4; ++m) qraw[rt][m] = load16(qp + 32 * m);
    }
    // ---- the key loop's first loads, issued behind the query's: the block-table entries of blocks
    //      0 and 1 travel with the query rows, and the raw loads of blocks 0 and 1 (then block 2's
    //      entries) fly while the query is converted.  The order is the one a step of the loop
    //      leaves outstanding (entries of block k + 2, then the raw loads of block k + 1), so that
    //      the loop's wait counts hold from its first trip.
    TileRaw R0, R1;
    TilePg P0, P1;
    load_pg(t0, P0);
    load_pg(t0 + TBLK, P1);
    load_raw(t0, P0, R0);
    load_pg(t0 + 2 * TBLK, P0);
    load_raw(t0 + TBLK, P1, R1);  // (past kmax: in-bounds stand-ins)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const float sq = rowv[rt] ? sgn : 0.0f;
        float x[32];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[8 * m + e] = sq * bf16_at(qraw[rt][m], e);
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 32; ++e) mx = fmaxf(mx, fabsf(x[e]));
        mx = row_max4(mx);
        int ex = 0;
        if (mx > 0.0f) (void)frexpf(mx, &ex);       // mx in [2^(ex-1), 2^ex)
        const int k = min(120, max(-120, 15 - ex));  // mx * 2^k in [2^14, 2^15)
        const float up = ldexpf(1.0f, k);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const _Float16 lo = (_Float16)(x[8 * m + 2 * e2] * up), hi = (_Float16)(x[8 * m + 2 * e2 + 1] * up);
                qf[rt][m][e2] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
        // floored at 2^-126: a hidden key's -inf score times the row's factor must stay -inf (a zero
        // scale would make it NaN), and below the floor every logit difference is far under fp32's
        // resolution of exp2 near 1, so a zero scale still weighs every visible key 1
        rowmul[rt] = fmaxf(ldexpf(fabsf(a.scale_log2), -k), 0x1p-126f);
    }
    // the wave's lowest and highest causal limits over its valid rows
    const int lim_lo = wave_min(min(lim[0], lim[1]));
    const int lim_hi = wave_max(max(rowv[0] ? lim[0] : -1, rowv[1] ? lim[1] : -1));
    // whether any of the wave's second 16 rows is a row of the tile (uniform)
    const bool rt1_live = __builtin_amdgcn_readfirstlane((int)__any(rowv[1])) != 0;

    float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
    f4 acc[2][8];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
    float s_ref = 0.0f, s_inv = 0.0f;


    // one block from LDS buffer buf: the wave's 32 rows (nrt = 1: its first 16) against its 64 keys,
    // in two halves of 32 keys, each its own online-softmax step
    auto compute = [&](const int T, const int buf, auto nrt) __attribute__((always_inline)) {
        constexpr int NRT = decltype(nrt)::value;
        if (T > lim_hi) return;  // no valid row of the wave sees these keys (uniform)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int T0 = T + 32 * hf;
            if (T0 > lim_hi) break;  // (uniform)
            const bool MASKED = T0 + 31 > lim_lo;
            // ---------------------------- scores: tile u holds keys T0 + 8g' + 4u + i of row n
            f4 sc[2][2];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) sc[rt][0] = sc[rt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
                const _Float16* kr = &S.k[buf][32 * hf + 16 * uu + n][8 * g];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const th8 av = *reinterpret_cast<const th8*>(kr + 32 * m);
#pragma unroll
                    for (int rt = 0; rt < NRT; ++rt)
                        sc[rt][uu] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(th8, qf[rt][m]),
                                                                            sc[rt][uu], 0, 0, 0);
                }
            }
            // ---------------------------- logits (log2 units) of keys T0 + 8g + e, their V scales
            //      (one LDS base made opaque here, so that the four reads take immediate offsets
            //      from it rather than sixteen precomputed addresses held across the key loop)
            lds_cf* sp = (lds_cf*)&S.ks[0][8 * g];
            asm volatile("" : "+v"(sp));
            const f4 k0 = *(lds_cf4*)(sp + buf * TBLK + 32 * hf);
            const f4 k1 = *(lds_cf4*)(sp + buf * TBLK + 32 * hf + 4);
            const f4 v0 = *(lds_cf4*)(sp + (2 + buf) * TBLK + 32 * hf);
            const f4 v1 = *(lds_cf4*)(sp + (2 + buf) * TBLK + 32 * hf + 4);
            const float kss[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
            const float vss[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            // ---------------------------- V-scale reference (the same for every row of the wave)
            float vmax = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) vmax = fmaxf(vmax, vss[e]);
            vmax = row_max4(vmax);
            float sf = 1.0f;
            if (vmax > 16.0f * s_ref) {  // (also the first half-block: s_ref == 0)
                sf = s_ref > 0.0f ? s_ref * __builtin_amdgcn_rcpf(vmax) : 0.0f;
                s_ref = vmax;
                s_inv = __builtin_amdgcn_rcpf(vmax);
            }
            float vr[8];  // the keys' V scales over the reference
#pragma unroll
            for (int e = 0; e < 8; ++e) vr[e] = vss[e] * s_inv;
            // ---------------------------- online softmax, P^T operand (lane (n, g): row n, keys
            //                              T0 + 8g .. + 7)
            uint32_t pb[2][4];
            float factor[2];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                // y: the score times the key's K scale; the logit (log2 units) is y times the row's
                // factor rowmul >= 0, which joins the exponent's FMA (and commutes with the max)
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = sc[rt][e >> 2][e & 3] * kss[e];
                if (MASKED) {  // hidden keys score -inf (keys past kmax are past every valid row's limit)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (T0 + 8 * g + e > lim[rt]) y[e] = -INFINITY;
                }
                float ymax = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) ymax = fmaxf(ymax, y[e]);
                const float bmax = row_max4(ymax) * rowmul[rt];
                float alpha = 1.0f;
                if (bmax > m_ref[rt] + 8.0f) {  // (also the first block: m_ref == -inf)
                    alpha = __builtin_amdgcn_exp2f(m_ref[rt] - bmax);
                    m_ref[rt] = bmax;
                }
                // a row with no visible key yet keeps m_ref = -inf: its weights are taken against
                // 0, so that its hidden keys (-inf) weigh exactly 0
                const float mref = m_ref[rt] == -INFINITY ? 0.0f : m_ref[rt];
                float ps = 0.0f;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(y[2 * e2], rowmul[rt], -mref));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(y[2 * e2 + 1], rowmul[rt], -mref));
                    ps += p0 + p1;
                    const tf2 wv = {p0 * vr[2 * e2], p1 * vr[2 * e2 + 1]};  // one packed conversion (RNE)
                    pb[rt][e2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(wv, th2));
                }
                l_run[rt] = l_run[rt] * alpha + row_sum4(ps);
                factor[rt] = alpha * sf;
            }
            if (__any(factor[0] != 1.0f || (NRT > 1 && factor[NRT - 1] != 1.0f))) {
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 8; ++ct) acc[rt][ct] *= factor[rt];
            }
            // ---------------------------- O^T += V^T . P^T over the 32 keys, channel tile ct
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const th8 av = *reinterpret_cast<const th8*>(&S.v[buf][16 * ct + n][32 * hf + 8 * g]);
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(th8, pb[rt]),
                                                                         acc[rt][ct], 0, 0, 0);
            }
        }
    };

    // ---- the key loop: block k computes from LDS buffer k % 2 while the raw loads of blocks k + 1
    //      (register set (k + 1) % 2) and k + 2 (set k % 2, issued at its start) are in flight; block
    //      k + 1 goes to LDS after block k's compute, then one barrier.  The block-table entries of
    //      block k + 3 are loaded at the start of block k, before its raw loads, so that waiting
    //      for them (at block k + 1) never waits for raw loads issued after them.  Blocks in pairs,
    //      one loop exit, so the register sets and buffers are fixed per half of the pair.  The
    //      loop is written out once per count of live row tiles (the choice is uniform per wave),
    //      so that each copy gets its own register allocation.
    const int nblk = (kmax - t0 + TBLK - 1) / TBLK;
    store_lds(R0, 0, t0);
    __syncthreads();
    auto key_loop = [&](auto nrt) __attribute__((always_inline)) {
        auto step = [&](const int T, const int buf, TileRaw& Rcur, TileRaw& Rnext, TilePg& Pcur, TilePg& Pnext)
                        __attribute__((always_inline)) {
            load_pg(T + 3 * TBLK, Pnext);       // block k + 3's entries (set k + 1's were used)
            load_raw(T + 2 * TBLK, Pcur, Rcur);  // block k + 2 into the set block k came from (already in LDS)
            compute(T, buf, nrt);
            store_lds(Rnext, buf ^ 1, T + TBLK);  // block k + 1
            __syncthreads();
        };
        int T = t0;
        for (int i = 1; i < nblk; i += 2) {
            step(T, 0, R0, R1, P0, P1);
            step(T + TBLK, 1, R1, R0, P1, P0);
            T += 2 * TBLK;
        }
        if (nblk & 1) compute(T, 0, nrt);
    };
    // (waves of one workgroup may take different copies: both run the same blocks and the same
    // number of workgroup barriers, which count arrivals, so they stay in step)
    if (rt1_live)
        key_loop(std::integral_constant<int, 2>{});
    else
        key_loop(std::integral_constant<int, 1>{});

    // ---- normalise and write: lane (n, g) holds channels 16ct + 4g + i of row 64rt + 16w + n.
    //      Splits: fp32 partials and base-2 lse, laid out for a merge of 64-row items: half j / 64
    //      of the tile is item 2 (tile) + j / 64, its row j % 64 of split sp in row
    //      ((item2 * nsplit + sp) * 64 + j % 64).
    //      The lane's indices are taken afresh from an opaque copy of the thread id, so that the
    //      compiler keeps none of the prologue's row offsets live (and spilled) across the loop.
    const bool split_mode = a.nsplit > 1;
    int tid_e = tid;
    asm volatile("" : "+v"(tid_e));
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        if (!rowv[rt]) continue;
        const int j = 64 * rt + 16 * (tid_e / kWave) + (tid_e & 15);
        const int r = it.r0 + j;
        const int64_t orow = (int64_t)(it.qrow0 + r / a.g) * a.hq + h * a.g + r % a.g;
        const int64_t prow = ((int64_t)(2 * item + (j >> 6)) * a.nsplit + sp) * 64 + (j & 63);
        const float l = l_run[rt];
        const float mul = l > 0.0f ? s_ref / l : 0.0f;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int c = 16 * ct + 4 * g;
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = acc[rt][ct][i] * mul;
            if (!split_mode) {
                uint2 pk;
                pk.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
                pk.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
                *reinterpret_cast<uint2*>(a.out + orow * TD + c) = pk;
            } else {
                *reinterpret_cast<f4*>(a.part_o + prow * TD + c) = f4{o[0], o[1], o[2], o[3]};
            }
        }
        if (g == 0) {
            const float lse2 = l > 0.0f ? m_ref[rt] + log2f(l) : -INFINITY;
            if (!split_mode) {
                if (a.lse) a.lse[orow] = lse2 * kLn2t;
            } else {
                a.part_lse[prow] = lse2;
            }
        }
    }
}

}  // namespace

hipError_t launch_decode_tile(const DecodeArgs& a, int batch, int head_dim, int mode, hipStream_t stream) {
    if (head_dim != TD) return hipErrorInvalidValue;
    const int64_t nbh = (int64_t)batch * a.hkv;
    const int64_t grid = nbh * a.nrg * a.nsplit;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 gd((unsigned)grid), bd(TW * kWave);
    if (mode == 0)
        hipLaunchKernelGGL(decode_tile_kernel<0>, gd, bd, 0, stream, a, (int)nbh);
    else if (mode == 1)
        hipLaunchKernelGGL(decode_tile_kernel<1>, gd, bd, 0, stream, a, (int)nbh);
    else
        return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    // the partials as 64-row items (two per tile), merged by the decode's log-sum-exp merge
    DecodeArgs m = a;
    m.nrg = 2 * a.nrg;
    m.prs = 64;
    return launch_merge(m, batch, head_dim, 64, stream);
}

}  // namespace pkv
