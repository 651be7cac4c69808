// walk.hip - the read ceiling of the int8 decode's access pattern (gfx950).
//
// One wave per (sequence, KV head, split of split_len keys), launched in the decode's order, reads
// every cache byte the decode of those keys reads and does nothing with it but add it up:
//   * the K rows of its keys (token-major pages: lane (rho, g) takes 16-byte pieces of the rows of
//     keys 16 (rho / 4) + 8 v + 4 e + rho % 4 of each 64-key block, as the decode's score operand);
//   * the V tiles of its keys (16-slot channel-major tiles: lane (n, g) takes channel rows
//     n + 16 dt of tile g of the block, one 16-byte load each, as the decode's P.V operand);
//   * the per-token K and V scales of its keys, or the per-block scales of the blocks it touches.
// The wave's block-table slice goes to LDS first, as in the decode.  `depth` blocks of 64 keys
// are in flight while one is summed (the decode keeps one).  The sum of the 32-bit words a wave
// read (wrapping) is its checksum, out[(b * hkv + h) * nsplit + s]; keys past the context are not
// read, except for the rest of a V tile that starts inside it (the decode reads whole tiles).
#include "mla_internal.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int BLK = 64;
constexpr int MAX_SPLIT = 4096;

template <int D>
struct WalkBuf {
    u32x4 k[4][D / 64];
    u32x4 v[D / 16];
    float4 s;  // lanes n < 8: four K (n < 4) or V (n >= 4) per-token scales; n == 0: block scales
};

__device__ __forceinline__ uint32_t sum4(const u32x4& w) { return w.x + w.y + w.z + w.w; }

template <int D, int MODE, int DEPTH>
__global__ __launch_bounds__(64) void walk_kernel(WalkArgs a, int pairs) {
    constexpr int KSTEP = D / 64;
    constexpr int DT = D / 16;
    constexpr int NB = DEPTH + 1;
    __shared__ int bt_s[MAX_SPLIT / 16 + 1];
    const int u = blockIdx.x;
    if (u >= pairs * a.nsplit) return;
    const int s = u / pairs;  // pairs (sequence x KV head) fastest, as the decode's fixed partition
    const int bh = u % pairs;
    const int h = bh % a.hkv, b = bh / a.hkv;
    const int lane = threadIdx.x;
    const int n = lane & 15, g = lane >> 4;
    const int ctx = __builtin_amdgcn_readfirstlane(a.ctx[b]);
    const int t0 = s * a.split_len;
    uint32_t acc = 0;
    if (t0 < ctx) {
        const int t1 = min(t0 + a.split_len, ctx);
        const int blk0 = t0 >> a.log2bs;
        const int nblk = ((t1 - 1) >> a.log2bs) - blk0 + 1;
        for (int i = lane; i < nblk; i += kWave) bt_s[i] = a.bt[(int64_t)b * a.mbs + blk0 + i];
        __syncthreads();
        const uint8_t* kb = reinterpret_cast<const uint8_t*>(a.k) + (int64_t)h * a.bs * D;
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.v) + (int64_t)h * a.bs * D;
        const int64_t page_bytes = (int64_t)a.hkv * a.bs * D;
        const int rho = lane & 15, kchunk = rho >> 2;

        auto load = [&](int T, WalkBuf<D>& R) {
            if (T >= t1) return;  // uniform: nothing past the split
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = T + 16 * kchunk + 8 * (q >> 1) + 4 * (q & 1) + (rho & 3);
                const bool on = t < t1;
                const int tt = on ? t : T;
                const uint8_t* kp = kb + (int64_t)bt_s[(tt >> a.log2bs) - blk0] * page_bytes +
                                    (tt & (a.bs - 1)) * D + g * 16 * KSTEP;
#pragma unroll
                for (int m = 0; m < KSTEP; ++m) R.k[q][m] = on ? load16(kp + 16 * m) : u32x4{0u, 0u, 0u, 0u};
            }
            const int tg = T + 16 * g;  // first key of the lane group's V tile
            const bool von = tg < t1;
            const int tv = von ? tg : T;
            const int64_t pid = bt_s[(tv >> a.log2bs) - blk0];
            const uint8_t* vp = vb + pid * page_bytes + (tv & (a.bs - 1)) * D + n * kVTile;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) R.v[dt] = von ? load16(vp + dt * 16 * kVTile) : u32x4{0u, 0u, 0u, 0u};
            R.s = make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (MODE == 0) {
                if (von && n < 8) {
                    const float* sp = (n < 4 ? a.ks : a.vs) + (pid * a.hkv + h) * a.bs + (tv & (a.bs - 1)) + 4 * (n & 3);
                    R.s = *reinterpret_cast<const float4*>(sp);
                }
            } else if constexpr (MODE == 1) {
                // block scales: each page the wave's keys touch, once: read with the tile that
                // starts the page, or with the wave's first tile when the range starts mid-page
                const bool first = (tg & (a.bs - 1)) == 0 || tg == t0;
                if (von && n == 0 && first) {
                    R.s.x = a.ks[pid * a.hkv + h];
                    R.s.y = a.vs[pid * a.hkv + h];
                }
            }
        };
        auto consume = [&](int T, const WalkBuf<D>& R) {
            if (T >= t1) return;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int m = 0; m < KSTEP; ++m) acc += sum4(R.k[q][m]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc += sum4(R.v[dt]);
            if constexpr (MODE == 0) {
                // per-token scales of keys past the context are not counted
                const int tk = T + 16 * g + 4 * (n & 3);
                const float e[4] = {R.s.x, R.s.y, R.s.z, R.s.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n < 8 && tk + i < t1) acc += __float_as_uint(e[i]);
            } else if constexpr (MODE == 1) {
                acc += __float_as_uint(R.s.x) + __float_as_uint(R.s.y);
            }
        };

        WalkBuf<D> buf[NB];
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) load(t0 + BLK * i, buf[i]);
        for (int T = t0; T < t1; T += BLK * NB) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                load(T + BLK * (j + DEPTH), buf[(j + DEPTH) % NB]);
                consume(T + BLK * j, buf[j]);
            }
        }
    }
    // wave sum of the lanes' word sums
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, kWave);
    if (lane == 0) a.out[((int64_t)b * a.hkv + h) * a.nsplit + s] = acc;
}

template <int D, int MODE>
hipError_t launch_d(const WalkArgs& a, int pairs, int depth, hipStream_t stream) {
    const int64_t grid = (int64_t)pairs * a.nsplit;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (depth == 1)
        hipLaunchKernelGGL((walk_kernel<D, MODE, 1>), dim3((unsigned)grid), dim3(64), 0, stream, a, pairs);
    else if (depth == 2)
        hipLaunchKernelGGL((walk_kernel<D, MODE, 2>), dim3((unsigned)grid), dim3(64), 0, stream, a, pairs);
    else
        hipLaunchKernelGGL((walk_kernel<D, MODE, 3>), dim3((unsigned)grid), dim3(64), 0, stream, a, pairs);
    return hipGetLastError();
}

// The MLA decode's reads (latent cache): one workgroup of four waves per (sequence b, split s),
// launched with the splits of one sequence consecutive, as the decode numbers its segments.  Wave
// w reads keys T + 16w .. T + 16w + 15 of each 64-key block with the decode's lane layout: lane
// (g, n) the 16-byte pieces 64m + 16g of key n's latent row (m < 8) and piece 16g of its rotary
// row, and the latent and rotary scales of keys 16w + 4g .. + 3.  Two blocks in flight per wave,
// the loads of block k + 2 issued once block k is summed (past the range's end they read the
// range's last key again); only keys inside the range are summed.
constexpr int MW_WAVES = 4;
constexpr int MW_BLK = 16 * MW_WAVES;

struct MlaWalkBuf {
    u32x4 k[kMlaLatent / 64 + 1];
    float4 ls, rs;
};

__global__ __launch_bounds__(MW_WAVES * kWave) void mla_walk_kernel(MlaWalkArgs a, int units) {
    __shared__ int bt_s[MAX_SPLIT / 16 + 1];
    __shared__ uint32_t red[MW_WAVES];
    const int u = blockIdx.x;
    if (u >= units) return;
    const int b = u / a.nsplit, s = u % a.nsplit;
    const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int n = lane & 15, g = lane >> 4;
    const int ctx = __builtin_amdgcn_readfirstlane(a.ctx[b]);
    const int t0 = s * a.split_len;
    uint32_t acc = 0;
    if (t0 < ctx) {  // uniform per workgroup
        const int t1 = min(t0 + a.split_len, ctx);
        const int blk0 = t0 >> a.log2bs;
        const int nblk = ((t1 - 1) >> a.log2bs) - blk0 + 1;
        for (int i = threadIdx.x; i < nblk; i += blockDim.x) bt_s[i] = a.bt[(int64_t)b * a.mbs + blk0 + i];
        __syncthreads();
        auto row_of = [&](int t) {  // cache row of key t (past the range: its last key)
            const int tt = min(t, t1 - 1);
            return (int64_t)bt_s[(tt >> a.log2bs) - blk0] * a.bs + (tt & (a.bs - 1));
        };
        auto load = [&](int T, MlaWalkBuf& R) {
            const int64_t row = row_of(T + 16 * w + n);
            const uint8_t* lp = reinterpret_cast<const uint8_t*>(a.latent) + row * kMlaLatent + 16 * g;
#pragma unroll
            for (int m = 0; m < kMlaLatent / 64; ++m) R.k[m] = load16(lp + 64 * m);
            R.k[kMlaLatent / 64] = load16(reinterpret_cast<const uint8_t*>(a.rope) + row * kMlaRope + 16 * g);
            // the four scales of keys 16w + 4g .. share one 4-aligned group of a page's rows
            const int64_t srow = row_of(T + 16 * w + 4 * g) & ~(int64_t)3;
            R.ls = *reinterpret_cast<const float4*>(a.ls + srow);
            R.rs = *reinterpret_cast<const float4*>(a.rs + srow);
        };
        auto sum = [&](int T, const MlaWalkBuf& R) {
            if (T + 16 * w + n < t1) {
#pragma unroll
                for (int m = 0; m <= kMlaLatent / 64; ++m) acc += sum4(R.k[m]);
            }
            const int tk = T + 16 * w + 4 * g;
            const float el[4] = {R.ls.x, R.ls.y, R.ls.z, R.ls.w};
            const float er[4] = {R.rs.x, R.rs.y, R.rs.z, R.rs.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (n == 0 && tk + i < t1) acc += __float_as_uint(el[i]) + __float_as_uint(er[i]);
        };
        MlaWalkBuf R0, R1;
        load(t0, R0);
        load(t0 + MW_BLK, R1);
        for (int T = t0; T < t1; T += 2 * MW_BLK) {
            sum(T, R0);
            load(T + 2 * MW_BLK, R0);
            if (T + MW_BLK < t1) sum(T + MW_BLK, R1);
            load(T + 3 * MW_BLK, R1);
        }
    }
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, kWave);
    if (lane == 0) red[w] = acc;
    __syncthreads();
    if (threadIdx.x == 0) a.out[u] = red[0] + red[1] + red[2] + red[3];
}

}  // namespace

hipError_t launch_mla_walk(const MlaWalkArgs& a, int batch, hipStream_t stream) {
    const int64_t units = (int64_t)batch * a.nsplit;
    if (units == 0) return hipSuccess;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_walk_kernel, dim3((unsigned)units), dim3(MW_WAVES * kWave), 0, stream, a, (int)units);
    return hipGetLastError();
}

hipError_t launch_walk(const WalkArgs& a, int batch, int head_dim, int mode, int depth, hipStream_t stream) {
    const int pairs = batch * a.hkv;
    if (head_dim == 64) {
        if (mode == 0) return launch_d<64, 0>(a, pairs, depth, stream);
        if (mode == 1) return launch_d<64, 1>(a, pairs, depth, stream);
        return launch_d<64, 3>(a, pairs, depth, stream);
    }
    if (head_dim == 128) {
        if (mode == 0) return launch_d<128, 0>(a, pairs, depth, stream);
        if (mode == 1) return launch_d<128, 1>(a, pairs, depth, stream);
        return launch_d<128, 3>(a, pairs, depth, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
