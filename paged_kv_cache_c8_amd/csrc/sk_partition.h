// sk_partition.h - the balanced key partition shared by the int8-score decode (decode_c8.hip) and
// the bf16 matrix-core decode (decode_mfma.hip): work-item geometry, the plan each wave computes
// from the sequence lengths, and the merge of the segments' partial results.  Device code; each
// including file gets its own copies (anonymous namespace).
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int SK_BLK = 64;          // keys per block of the partition
constexpr int SK_MAX_SEQS = 4096;   // sequences the plan handles (LDS prefix sums)

// Rows, keys and output position of work item `item` = (sequence b, KV head h, row group rg).
struct ItemGeo {
    int b, h, qlen, qrow0, prior, r0, nrows, nvalid, kmax, kmin;  // keys [kmin, kmax) (kmin 128-aligned)
};
template <int ROWS, bool WIN = false>
__device__ __forceinline__ ItemGeo item_geo(const DecodeArgs& a, int item) {
    ItemGeo it;
    const int rg = item % a.nrg;
    const int bh = item / a.nrg;
    it.h = bh % a.hkv;
    it.b = bh / a.hkv;
    it.qlen = a.cu ? a.cu[it.b + 1] - a.cu[it.b] : 1;
    it.qrow0 = a.cu ? a.cu[it.b] : it.b;
    it.prior = a.ctx[it.b] - it.qlen;
    it.nrows = it.qlen * a.g;
    it.r0 = rg * ROWS;
    it.nvalid = min(ROWS, it.nrows - it.r0);
    it.kmax = it.nvalid > 0 ? it.prior + (it.r0 + it.nvalid - 1) / a.g + 1 : 0;  // keys the last row sees
    it.kmin = WIN && it.nvalid > 0 ? win_begin(a.window, it.prior + it.r0 / a.g) : 0;  // first key of the range
    return it;
}

// zero output and lse = -inf for the rows of an item with no key (a sequence of length 0)
template <int D>
__device__ __forceinline__ void zero_rows(const DecodeArgs& a, const ItemGeo& it, int lane) {
    for (int o = lane; o < it.nvalid * D; o += kWave) {
        const int j = o / D, d = o % D;
        const int r = it.r0 + j;
        const int64_t orow = (int64_t)(it.qrow0 + r / a.g) * a.hq + it.h * a.g + r % a.g;
        a.out[orow * D + d] = 0;
        if (d == 0 && a.lse) a.lse[orow] = -INFINITY;
    }
}

// Balanced partition: with N key blocks (64 keys) over all items and a target of W segments (the
// waves the GPU holds at once, or a multiple of them when the items are not few against those),
// item i with n_i blocks gets k_i = min(n_i, ceil(n_i W' / N)) segments of near-equal length, W' =
// W - A for A non-empty items (so that the ceilings keep the total within W), one wave per
// segment: waves of about the same length, so the GPU runs full rounds of waves instead of rounds
// of very different fill.  The grid holds W + items waves (an upper bound of the sum of the
// k_i); the spare ones return at once.  Wave K_i + s (K = prefix
// sums of k, items in (sequence, KV head, row group) order) takes segment s of item i; a
// one-segment item writes its result, others leave a partial in slot K_i + s, and segment 0
// records K_i and k_i in seg[2i], seg[2i + 1] for the merge.  The plan is computed by every wave
// from the sequence lengths, per sequence (its KV heads share the counts).
struct SkSegment {
    ItemGeo it;      // the work item
    int t0, t1;      // its keys [t0, t1) this wave takes
    int64_t pslot;   // partial slot of the wave, -1: a one-segment item writes its result
};

// The segment of wave `wid` (false: the wave has none).  kseq: LDS of batch + 1 ints.
template <int ROWS, bool WIN>
__device__ __forceinline__ bool sk_plan(const DecodeArgs& a, int batch, int wid, int* kseq, SkSegment& out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int W = a.sk_waves;
    // blocks of row group rg of sequence b (the same for every KV head)
    auto group_blocks = [&](int b, int rg) {
        const int qlen = a.cu ? a.cu[b + 1] - a.cu[b] : 1;
        const int nrows = qlen * a.g;
        const int r0 = rg * ROWS;
        if (r0 >= nrows) return 0;
        const int nvalid = min(ROWS, nrows - r0);
        const int kmax = a.ctx[b] - qlen + (r0 + nvalid - 1) / a.g + 1;
        const int kmin = WIN ? win_begin(a.window, a.ctx[b] - qlen + r0 / a.g) : 0;
        return kmax > 0 ? (kmax - kmin + SK_BLK - 1) / SK_BLK : 0;
    };
    // N = total blocks over every item, A = items with at least one block
    int64_t N = 0;
    int A = 0;
    for (int b0 = 0; b0 < batch; b0 += kWave) {
        int nb = 0, na = 0;
        if (b0 + lane < batch)
            for (int rg = 0; rg < a.nrg; ++rg) {
                const int x = group_blocks(b0 + lane, rg);
                nb += x;
                na += x > 0;
            }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            nb += __shfl_xor(nb, d, kWave);
            na += __shfl_xor(na, d, kWave);
        }
        N += nb;
        A += na;
    }
    if (N == 0) return false;  // every item is empty: the merge writes the zero rows
    N *= a.hkv;
    A *= a.hkv;
    // ceil rounding adds less than one segment per item: planning for W - A waves keeps the total
    // within the W waves the GPU holds at once (one round)
    const int64_t Wp = W > 2 * A ? W - A : (W > A ? A : 1);
    auto segs = [&](int nb, int64_t NN) {
        return nb > 0 ? (int)min((int64_t)nb, ((int64_t)nb * Wp + NN - 1) / NN) : 0;
    };
    // waves of each sequence (all its KV heads and row groups) and their prefix sums
    int carry = 0;
    for (int b0 = 0; b0 < batch; b0 += kWave) {
        const int b = b0 + lane;
        int x = 0;
        if (b < batch)
            for (int rg = 0; rg < a.nrg; ++rg) x += segs(group_blocks(b, rg), N);
        x *= a.hkv;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {  // inclusive scan over the wave
            const int y = __shfl_up(x, d, kWave);
            if (lane >= d) x += y;
        }
        if (b < batch) kseq[b + 1] = carry + x;
        carry += __shfl(x, kWave - 1, kWave);
    }
    if (lane == 0) kseq[0] = 0;
    __builtin_amdgcn_wave_barrier();
    if (wid >= carry) return false;
    int lo = 0, hi = batch;  // kseq[lo] <= wid < kseq[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (kseq[mid] <= wid) lo = mid; else hi = mid;
    }
    const int b = lo;
    // within sequence b: items (h, rg) in order, rg fastest
    int per_head = 0;
    for (int rg = 0; rg < a.nrg; ++rg) per_head += segs(group_blocks(b, rg), N);
    const int off = wid - kseq[b];
    const int h = off / per_head;
    int rem = off - h * per_head, rg = 0, k = segs(group_blocks(b, 0), N);
    int first = kseq[b] + h * per_head;
    while (rem >= k) {
        rem -= k;
        first += k;
        ++rg;
        k = segs(group_blocks(b, rg), N);
    }
    const int seg = rem;
    const int item = (b * a.hkv + h) * a.nrg + rg;
    const ItemGeo it = item_geo<ROWS, WIN>(a, item);
    const int nb = (it.kmax - it.kmin + SK_BLK - 1) / SK_BLK;
    if (seg == 0 && lane == 0) {
        a.seg[2 * item] = first;
        a.seg[2 * item + 1] = k;
    }
    // Every value of the segment is the same in all lanes, but it was read from LDS and memory at
    // lane-varying addresses as far as the compiler can tell: made wave-uniform (scalar registers)
    // here, so that the kernel's key loop and branches are uniform control flow.  Lane-divergent
    // control flow around the matrix-core instructions (which read every lane's operands) is what
    // the key loops must not have.
    auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    out.it.b = uni(it.b);
    out.it.h = uni(it.h);
    out.it.qlen = uni(it.qlen);
    out.it.qrow0 = uni(it.qrow0);
    out.it.prior = uni(it.prior);
    out.it.r0 = uni(it.r0);
    out.it.nrows = uni(it.nrows);
    out.it.nvalid = uni(it.nvalid);
    out.it.kmax = uni(it.kmax);
    out.it.kmin = uni(it.kmin);
    out.t0 = uni(it.kmin + (int)((int64_t)nb * seg / k) * SK_BLK);
    out.t1 = uni(min(it.kmin + (int)((int64_t)nb * (seg + 1) / k) * SK_BLK, it.kmax));
    out.pslot = uni(k) == 1 ? -1 : (int64_t)wid;
    return true;
}

// Merge of the balanced partition: item i's partials sit in slots seg[2i] .. seg[2i] + seg[2i+1] - 1;
// a one-segment item is already written; an item with no key gets zero rows.  Thread (row j,
// 8-channel group c) of thread group g takes the item's segments in chunks of SK_MERGE_CH,
// chunks g, g + ng, ..., so that a long item has all its partials in flight at once (one group
// alone would walk them in as many dependent rounds of loads as it has chunks).  With ng > 1 the
// groups' running (max, weight sum, accumulators) meet in dynamic LDS of 10 * ng * ROWS * D / 8
// floats and group 0 combines them.
constexpr int SK_MERGE_CH = 8;
constexpr int SK_MERGE_THREADS = 1024;

template <int D, int ROWS>
__global__ __launch_bounds__(SK_MERGE_THREADS) void merge_sk_kernel(DecodeArgs a, int ng) {
    constexpr int CG = D / 8;
    constexpr int TPR = ROWS * CG;  // threads of one group
    const int item = blockIdx.x;
    // the item's segment record is read together with its geometry (one round trip less); it is
    // only used once the item is known to have keys, i.e. once this call's decode has written it
    const int k = a.seg[2 * item + 1];
    const int w0 = a.seg[2 * item];
    const ItemGeo it = item_geo<ROWS>(a, item);
    if (it.nvalid <= 0) return;
    if (it.kmax <= 0) {
        if (threadIdx.x < kWave) zero_rows<D>(a, it, threadIdx.x);
        return;
    }
    if (k <= 1) return;  // one segment: the result is already written
    const int w1 = w0 + k - 1;
    const int grp = threadIdx.x / TPR, t = threadIdx.x % TPR;
    const int jr = t / CG, cg = t % CG;
    const bool active = grp < ng && jr < it.nvalid;
    float M = -INFINITY, wsum = 0.0f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    constexpr int CHM = SK_MERGE_CH;
    for (int s0 = w0 + grp * CHM; active && s0 <= w1; s0 += ng * CHM) {
        float l2[CHM];
        float4 p0[CHM], p1[CHM];
#pragma unroll
        for (int c = 0; c < CHM; ++c) {
            const int ww = s0 + c;
            if (ww <= w1) {
                const int64_t row = (int64_t)ww * a.prs + jr;
                l2[c] = a.part_lse[row];
                const float4* pp = reinterpret_cast<const float4*>(a.part_o + row * D) + 2 * cg;
                p0[c] = pp[0];
                p1[c] = pp[1];
            } else {
                l2[c] = -INFINITY;
                p0[c] = p1[c] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        float mc = M;
#pragma unroll
        for (int c = 0; c < CHM; ++c) mc = fmaxf(mc, l2[c]);
        if (mc == -INFINITY) continue;
        const float sc = M == -INFINITY ? 0.0f : exp2f(M - mc);
        M = mc;
        wsum *= sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
        for (int c = 0; c < CHM; ++c) {
            const float wt = l2[c] == -INFINITY ? 0.0f : exp2f(l2[c] - M);
            wsum += wt;
            acc[0] = fmaf(wt, p0[c].x, acc[0]);
            acc[1] = fmaf(wt, p0[c].y, acc[1]);
            acc[2] = fmaf(wt, p0[c].z, acc[2]);
            acc[3] = fmaf(wt, p0[c].w, acc[3]);
            acc[4] = fmaf(wt, p1[c].x, acc[4]);
            acc[5] = fmaf(wt, p1[c].y, acc[5]);
            acc[6] = fmaf(wt, p1[c].z, acc[6]);
            acc[7] = fmaf(wt, p1[c].w, acc[7]);
        }
    }
    if (ng > 1) {
        // every thread of the workgroup reaches this barrier (the returns above are per item)
        extern __shared__ float msh[];
        const int nt = ng * TPR;
        float* sm = msh;
        float* sw = msh + nt;
        float* sa = msh + 2 * nt;
        if (grp < ng) {
            sm[threadIdx.x] = M;
            sw[threadIdx.x] = wsum;
#pragma unroll
            for (int e = 0; e < 8; ++e) sa[e * nt + threadIdx.x] = acc[e];
        }
        __syncthreads();
        if (grp != 0 || !active) return;
        float mt = M;
        for (int g2 = 1; g2 < ng; ++g2) mt = fmaxf(mt, sm[g2 * TPR + t]);
        if (mt != -INFINITY) {
            const float sc = M == -INFINITY ? 0.0f : exp2f(M - mt);
            wsum *= sc;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= sc;
            for (int g2 = 1; g2 < ng; ++g2) {
                const float mg = sm[g2 * TPR + t];
                if (mg == -INFINITY) continue;
                const float f = exp2f(mg - mt);
                wsum = fmaf(f, sw[g2 * TPR + t], wsum);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(f, sa[e * nt + g2 * TPR + t], acc[e]);
            }
            M = mt;
        }
    } else if (!active) {
        return;
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    const int r = it.r0 + jr;
    const int64_t orow = (int64_t)(it.qrow0 + r / a.g) * a.hq + it.h * a.g + r % a.g;
    uint16_t* op = a.out + orow * D + 8 * cg;
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        pk[e] = f32_to_bf16_rne(acc[2 * e] * inv) | (f32_to_bf16_rne(acc[2 * e + 1] * inv) << 16);
    if ((reinterpret_cast<uintptr_t>(op) & 15) == 0) {
        *reinterpret_cast<uint4*>(op) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            op[2 * e] = (uint16_t)(pk[e] & 0xffffu);
            op[2 * e + 1] = (uint16_t)(pk[e] >> 16);
        }
    }
    if (cg == 0 && a.lse) a.lse[orow] = wsum > 0.0f ? (M + log2f(wsum)) * 0.6931471805599453f : -INFINITY;
}

// Launch of the balanced merge: as many thread groups (a power of two, at most 8 and 1024
// threads) as an item of average segment count needs to have its chunks in flight together.
template <int D, int ROWS>
hipError_t launch_merge_sk(const DecodeArgs& a, int64_t items, hipStream_t stream) {
    constexpr int TPR = ROWS * D / 8;
    static_assert(TPR <= SK_MERGE_THREADS, "one group must fit a workgroup");
    const int64_t avg = ((int64_t)a.sk_waves + 2 * items - 1) / items;  // segments per item, rounded up
    int ng = 1;
    while (ng < 8 && (int64_t)ng * SK_MERGE_CH < avg && 2 * ng * TPR <= SK_MERGE_THREADS) ng *= 2;
    const int threads = ((ng * TPR + kWave - 1) / kWave) * kWave;
    const size_t lds = ng > 1 ? (size_t)ng * TPR * 10 * sizeof(float) : 0;
    hipLaunchKernelGGL((merge_sk_kernel<D, ROWS>), dim3((unsigned)items), dim3(threads), lds, stream, a, ng);
    return hipGetLastError();
}

}  // namespace
}  // namespace pkv
