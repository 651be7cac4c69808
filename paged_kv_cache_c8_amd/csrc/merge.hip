// merge.hip - log-sum-exp merge of the split-KV partials of pkv_decode_gqa.
//
// A split s of a row leaves o_s = sum_t w_t v_t / sum_t w_t (fp32) and L_s = log2 sum_t w_t
// (weights taken against a common zero point).  The row's result is
//     out = sum_s 2^(L_s - M) o_s / sum_s 2^(L_s - M),   lse = M + log2 sum_s 2^(L_s - M),
// M = max_s L_s, combined in a fixed order (deterministic).  Splits past the row's keys were
// never written; their workspace rows may be loaded with the first round and are then dropped.
//
// One workgroup per (sequence, KV head, row group); thread (row j, group c of CPT channels).  The
// sequence's lengths and the partials of the first CH splits are loaded together (rows of splits
// the item did not use lie inside the workspace: read, then ignored), so a decode's merge costs
// one memory round trip; further splits are folded in CH at a time into a running (max, sum,
// accumulator).  CPT = 4 (CH = 16) for groups of up to 256 threads, else 8 (CH = 8).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kLn2 = 0.6931471805599453f;

template <int D, int CPT>
__global__ __launch_bounds__(CPT == 4 ? 256 : 1024) void merge_kernel(DecodeArgs a, int rows_per_item) {
    constexpr int CG = D / CPT;       // channel groups per row
    constexpr int CH = CPT == 4 ? 16 : 8;  // splits per load round
    constexpr int NV = CPT / 4;       // float4 per split and thread
    const int tid = threadIdx.x;
    const int jr = tid / CG;
    const int cg = tid % CG;

    int wi = blockIdx.x;
    const int item = wi;
    const int rg = wi % a.nrg;
    wi /= a.nrg;
    const int h = wi % a.hkv;
    const int b = wi / a.hkv;
    // ---- loads: lengths, and the first CH splits' partials of row jr (in the workspace for any jr < prs)
    const int64_t base = (int64_t)item * a.nsplit * a.prs + jr;  // row jr of split 0
    const bool rowok = jr < a.prs;
    float l2[CH];
    float4 p[CH][NV];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        if (rowok && c < a.nsplit) {
            const int64_t row = base + (int64_t)c * a.prs;
            l2[c] = a.part_lse[row];
            const float4* pp = reinterpret_cast<const float4*>(a.part_o + row * D) + NV * cg;
#pragma unroll
            for (int v = 0; v < NV; ++v) p[c][v] = pp[v];
        } else {
            l2[c] = -INFINITY;
#pragma unroll
            for (int v = 0; v < NV; ++v) p[c][v] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
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

    float M = -INFINITY, wsum = 0.0f;
    float acc[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) acc[e] = 0.0f;
    for (int s0 = 0; s0 < nact; s0 += CH) {
        if (s0 > 0) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int s = s0 + c;
                if (s < nact) {
                    const int64_t row = base + (int64_t)s * a.prs;
                    l2[c] = a.part_lse[row];
                    const float4* pp = reinterpret_cast<const float4*>(a.part_o + row * D) + NV * cg;
#pragma unroll
                    for (int v = 0; v < NV; ++v) p[c][v] = pp[v];
                }
            }
        }
        // splits past the row's keys were never written this call: whatever their rows hold (NaN
        // included) must reach neither the max nor the sums
#pragma unroll
        for (int c = 0; c < CH; ++c)
            if (s0 + c >= nact) {
                l2[c] = -INFINITY;
#pragma unroll
                for (int v = 0; v < NV; ++v) p[c][v] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        float mc = M;
#pragma unroll
        for (int c = 0; c < CH; ++c) mc = fmaxf(mc, l2[c]);
        if (mc == -INFINITY) continue;  // no key seen yet
        const float sc = M == -INFINITY ? 0.0f : exp2f(M - mc);
        M = mc;
        wsum *= sc;
#pragma unroll
        for (int e = 0; e < CPT; ++e) acc[e] *= sc;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float w = l2[c] == -INFINITY ? 0.0f : exp2f(l2[c] - M);
            wsum += w;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                acc[4 * v + 0] = fmaf(w, p[c][v].x, acc[4 * v + 0]);
                acc[4 * v + 1] = fmaf(w, p[c][v].y, acc[4 * v + 1]);
                acc[4 * v + 2] = fmaf(w, p[c][v].z, acc[4 * v + 2]);
                acc[4 * v + 3] = fmaf(w, p[c][v].w, acc[4 * v + 3]);
            }
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    const int r = r0 + jr;
    const int64_t orow = (int64_t)(qrow0 + r / a.g) * a.hq + h * a.g + r % a.g;
    uint16_t* op = a.out + orow * D + CPT * cg;
    uint32_t pk[CPT / 2];
#pragma unroll
    for (int e = 0; e < CPT / 2; ++e)
        pk[e] = f32_to_bf16_rne(acc[2 * e] * inv) | (f32_to_bf16_rne(acc[2 * e + 1] * inv) << 16);
    if constexpr (CPT == 8) {
        if ((reinterpret_cast<uintptr_t>(op) & 15) == 0) {
            *reinterpret_cast<uint4*>(op) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                op[2 * e] = (uint16_t)(pk[e] & 0xffffu);
                op[2 * e + 1] = (uint16_t)(pk[e] >> 16);
            }
        }
    } else {
        if ((reinterpret_cast<uintptr_t>(op) & 7) == 0) {
            *reinterpret_cast<uint2*>(op) = make_uint2(pk[0], pk[1]);
        } else {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                op[2 * e] = (uint16_t)(pk[e] & 0xffffu);
                op[2 * e + 1] = (uint16_t)(pk[e] >> 16);
            }
        }
    }
    if (cg == 0 && a.lse) a.lse[orow] = wsum > 0.0f ? (M + log2f(wsum)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_merge_d(const DecodeArgs& a, int64_t grid, int rows_per_item, hipStream_t stream) {
    const int t4 = ((rows_per_item * D / 4 + kWave - 1) / kWave) * kWave;
    const int t8 = ((rows_per_item * D / 8 + kWave - 1) / kWave) * kWave;
    if (t4 <= 256)
        hipLaunchKernelGGL((merge_kernel<D, 4>), dim3((unsigned)grid), dim3(t4), 0, stream, a, rows_per_item);
    else if (t8 <= 1024)
        hipLaunchKernelGGL((merge_kernel<D, 8>), dim3((unsigned)grid), dim3(t8), 0, stream, a, rows_per_item);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, int batch, int head_dim, int rows_per_item, hipStream_t stream) {
    const int64_t grid = (int64_t)batch * a.hkv * a.nrg;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (head_dim == 64) return launch_merge_d<64>(a, grid, rows_per_item, stream);
    if (head_dim == 128) return launch_merge_d<128>(a, grid, rows_per_item, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
