// dequant.hip - gather the paged cache back to bf16 rows (gfx950).
//
// Implements MojoDequantFromPagedKVCache of Mojo Opset PR #379: every position p < ctx_b of
// sequence b is written at row off_b + p, value bf16_rne(fl32(code * scale)) (the product in
// fp32, as that PR's reviews require; the scale per token, per block, or per channel), off_b = caller offsets or the exclusive prefix sum of
// the context lengths.  One workgroup per (sequence, logical block, KV head) page; the reviews'
// per-sequence .item() and list-concatenation loop becomes a single launch with no host sync.
//
// K pages are token-major and stream straight to the output rows.  V pages are channel-major
// within 16-slot tiles, so each workgroup stages its page in LDS (16-byte loads) and reads it
// back transposed.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <int D, int MODE>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
    constexpr int ESZ = MODE == 2 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint8_t vpage[D * 128 * ESZ];
    __shared__ long long part[4];

    int r = blockIdx.x;
    const int h = r % a.hkv;
    r /= a.hkv;
    const int j = r % a.mbs;
    const int b = r / a.mbs;
    const int ctx = a.ctx[b];
    if (j * a.bs >= ctx) return;  // uniform
    const int n = min(a.bs, ctx - j * a.bs);

    int64_t base;
    if (a.seq_off) {
        base = a.seq_off[b];
    } else {
        long long acc = 0;
        for (int i = threadIdx.x; i < b; i += blockDim.x) acc += a.ctx[i];
        for (int s = 1; s < kWave; s <<= 1) acc += __shfl_xor(acc, s, kWave);
        if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
        __syncthreads();
        base = part[0] + part[1] + part[2] + part[3];
    }
    const int64_t page = (int64_t)a.bt[(int64_t)b * a.mbs + j] * a.hkv + h;
    const int64_t row0 = base + (int64_t)j * a.bs;

    // stage the V page (all block_size slots; only the first n are read back)
    if (a.v_out) {
        const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(a.v) + page * D * a.bs * ESZ;
        const int chunks = D * a.bs * ESZ / 16;
        for (int i = threadIdx.x; i < chunks; i += blockDim.x)
            *reinterpret_cast<uint4*>(vpage + i * 16) = *reinterpret_cast<const uint4*>(vsrc + i * 16);
    }
    __syncthreads();

    for (int which = 0; which < 2; ++which) {
        uint16_t* out = which ? a.v_out : a.k_out;
        if (!out) continue;
        const float* scales = which ? a.vs : a.ks;
        for (int e8 = threadIdx.x; e8 < n * D / 8; e8 += blockDim.x) {
            const int slot = (e8 * 8) / D;
            const int c0 = (e8 * 8) % D;
            uint32_t y[8];
            if constexpr (MODE == 2) {
                if (which == 0) {
                    const uint16_t* src =
                        reinterpret_cast<const uint16_t*>(a.k) + (page * a.bs + slot) * D + c0;
                    const uint4 v = *reinterpret_cast<const uint4*>(src);
                    y[0] = v.x & 0xffff; y[1] = v.x >> 16; y[2] = v.y & 0xffff; y[3] = v.y >> 16;
                    y[4] = v.z & 0xffff; y[5] = v.z >> 16; y[6] = v.w & 0xffff; y[7] = v.w >> 16;
                } else {
                    const uint16_t* vp = reinterpret_cast<const uint16_t*>(vpage);
#pragma unroll
                    for (int k = 0; k < 8; ++k) y[k] = vp[v_elem(0, D, a.bs, c0 + k, slot)];
                }
            } else {
                int8_t codes[8];
                if (which == 0) {
                    const int8_t* src = reinterpret_cast<const int8_t*>(a.k) + (page * a.bs + slot) * D + c0;
                    const uint2 v = *reinterpret_cast<const uint2*>(src);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        codes[k] = (int8_t)(v.x >> (8 * k));
                        codes[4 + k] = (int8_t)(v.y >> (8 * k));
                    }
                } else {
                    const int8_t* vp = reinterpret_cast<const int8_t*>(vpage);
#pragma unroll
                    for (int k = 0; k < 8; ++k) codes[k] = vp[v_elem(0, D, a.bs, c0 + k, slot)];
                }
                if constexpr (MODE == 3) {  // static per-channel scales [Hkv][D]
                    const float* sc = scales + (int64_t)h * D + c0;
#pragma unroll
                    for (int k = 0; k < 8; ++k) y[k] = f32_to_bf16_rne((float)codes[k] * sc[k]);
                } else {
                    const float s = MODE == 0 ? scales[page * a.bs + slot] : scales[page];
#pragma unroll
                    for (int k = 0; k < 8; ++k) y[k] = f32_to_bf16_rne((float)codes[k] * s);
                }
            }
            uint16_t* dst = out + (row0 + slot) * a.token_stride + (int64_t)h * a.head_stride + c0;
            if (a.vec_ok) {
                uint4 w;
                w.x = y[0] | (y[1] << 16);
                w.y = y[2] | (y[3] << 16);
                w.z = y[4] | (y[5] << 16);
                w.w = y[6] | (y[7] << 16);
                *reinterpret_cast<uint4*>(dst) = w;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) dst[k] = (uint16_t)y[k];
            }
        }
    }
}

template <int D>
hipError_t launch_d(const DequantArgs& a, int mode, hipStream_t stream) {
    const int64_t grid = (int64_t)a.batch * a.mbs * a.hkv;
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (mode == 0)
        hipLaunchKernelGGL((dequant_kernel<D, 0>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    else if (mode == 1)
        hipLaunchKernelGGL((dequant_kernel<D, 1>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    else if (mode == 3)
        hipLaunchKernelGGL((dequant_kernel<D, 3>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((dequant_kernel<D, 2>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, int head_dim, int mode, hipStream_t stream) {
    if (head_dim == 64) return launch_d<64>(a, mode, stream);
    if (head_dim == 128) return launch_d<128>(a, mode, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
