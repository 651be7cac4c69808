// merge.hip - log-sum-exp merge of the split-KV partials of pkv_decode_gqa.
//
// A split s of a row leaves o_s = sum_t w_t v_t / sum_t w_t (fp32) and L_s = log2 sum_t w_t
// (weights taken against a common zero point).  The row's result is
//     out = sum_s 2^(L_s - M) o_s / sum_s 2^(L_s - M),   lse = M + log2 sum_s 2^(L_s - M),
// M = max_s L_s, combined in a fixed order (deterministic).  Splits past the row's keys were
// never written and are never read.
//
// One workgroup per (sequence, KV head, row group); thread (row j, 8-channel group c).  The loads
// of eight splits are issued together, then folded into a running (max, sum, accumulator) so that
// any number of splits costs one memory round trip per eight.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr int CH = 8;  // splits per load round

template <int D>
__global__ __launch_bounds__(1024) void merge_kernel(DecodeArgs a, int rows_per_item) {
    constexpr int CG = D / 8;  // 8-channel groups per row
    const int tid = threadIdx.x;
    const int jr = tid / CG;
    const int cg = tid % CG;

    int wi = blockIdx.x;
    const int item = wi;
    const int rg = wi % a.nrg;
    wi /= a.nrg;
    const int h = wi % a.hkv;
    const int b = wi / a.hkv;
    const int qlen = a.cu ? a.cu[b + 1] - a.cu[b] : 1;
    const int qrow0 = a.cu ? a.cu[b] : b;
    const int prior = a.ctx[b] - qlen;
    const int nrows = qlen * a.g;
    const int r0 = rg * rows_per_item;
    if (r0 >= nrows) return;
    const int nvalid = min(rows_per_item, nrows - r0);
    const int kmax = prior + (r0 + nvalid - 1) / a.g + 1;  // the split count the partials used
    if (kmax <= 0) return;                                  // written by the partial kernel
    if (jr >= nvalid) return;
    const int kmin = win_begin(a.window, prior + r0 / a.g);  // splits start here (sliding window)
    const int nact = min(a.nsplit, (kmax - kmin + a.split_len - 1) / a.split_len);
    const int64_t base = (int64_t)item * a.nsplit * a.prs + jr;  // row jr of split 0

    float M = -INFINITY, wsum = 0.0f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int s0 = 0; s0 < nact; s0 += CH) {
        float l2[CH];
        float4 p0[CH], p1[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int s = s0 + c;
            if (s < nact) {
                const int64_t row = base + (int64_t)s * a.prs;
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
        for (int c = 0; c < CH; ++c) mc = fmaxf(mc, l2[c]);
        if (mc == -INFINITY) continue;  // no key seen yet
        const float sc = M == -INFINITY ? 0.0f : exp2f(M - mc);
        M = mc;
        wsum *= sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float w = l2[c] == -INFINITY ? 0.0f : exp2f(l2[c] - M);
            wsum += w;
            acc[0] = fmaf(w, p0[c].x, acc[0]);
            acc[1] = fmaf(w, p0[c].y, acc[1]);
            acc[2] = fmaf(w, p0[c].z, acc[2]);
            acc[3] = fmaf(w, p0[c].w, acc[3]);
            acc[4] = fmaf(w, p1[c].x, acc[4]);
            acc[5] = fmaf(w, p1[c].y, acc[5]);
            acc[6] = fmaf(w, p1[c].z, acc[6]);
            acc[7] = fmaf(w, p1[c].w, acc[7]);
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    const int r = r0 + jr;
    const int64_t orow = (int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g;
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
    if (cg == 0 && a.lse) a.lse[orow] = wsum > 0.0f ? (M + log2f(wsum)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, int batch, int head_dim, int rows_per_item, hipStream_t stream) {
    const int64_t grid = (int64_t)batch * a.hkv * a.nrg;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    const int threads = ((rows_per_item * head_dim / 8 + kWave - 1) / kWave) * kWave;
    if (threads > 1024) return hipErrorInvalidValue;
    if (head_dim == 64)
        hipLaunchKernelGGL((merge_kernel<64>), dim3((unsigned)grid), dim3(threads), 0, stream, a, rows_per_item);
    else if (head_dim == 128)
        hipLaunchKernelGGL((merge_kernel<128>), dim3((unsigned)grid), dim3(threads), 0, stream, a, rows_per_item);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pkv
