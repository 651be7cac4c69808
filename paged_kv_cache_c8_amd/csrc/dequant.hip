// dequant.hip - gather the paged cache back to bf16 rows (gfx950).
//
// Implements MojoDequantFromPagedKVCache of Mojo Opset PR #379: every position p < ctx_b of
// sequence b is written at row off_b + p, value bf16_rne(fl32(code * scale)) (the product in
// fp32, as that PR's reviews require; the scale per token, per block, or per channel), off_b =
// caller offsets or the exclusive prefix sum of the context lengths.  The reviews' per-sequence
// .item() and list-concatenation loop becomes a single launch with no host sync.
//
// One workgroup per (sequence, 128 positions, KV head) of four waves of two 16-slot tiles each; the
// default row offset (an exclusive prefix sum of the context lengths) is formed once per workgroup.
// K pages are token-major and stream to the output rows; V pages are channel-major within 16-slot
// tiles, so each wave reads its tile whole and turns it into token rows through LDS.  Every store
// instruction writes whole output rows.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int TS = kVTile;       // slots per tile
constexpr int TPW = 2;            // tiles per wave
constexpr int CHUNK = 4 * TPW * TS;  // positions per workgroup (four waves)

// bf16 bits of two values code * scale (the product in fp32, rounded to nearest even)
__device__ __forceinline__ uint32_t deq_pair(int c0, int c1, float s0, float s1) {
    return f32_to_bf16_rne((float)c0 * s0) | (f32_to_bf16_rne((float)c1 * s1) << 16);
}

__device__ __forceinline__ int code_of(uint32_t w, int i) { return (int)(int8_t)((w >> (8 * i)) & 0xffu); }

// One workgroup of four waves per (sequence, 128 positions, KV head); wave w takes the 16-slot
// tiles of positions 16 (w + 4 i) .., i < 2, and issues every load of both before it converts and
// stores anything.  Rows go out whole: in step j a lane takes the 8-channel chunk L % CH of row
// j RPI + L / CH (CH = D / 8 chunks per row, RPI = 64 / CH rows per step), so every 16-byte store
// instruction writes RPI complete rows of the output.  K comes straight from its token-major rows
// (8 codes, or 8 bf16 values, per lane and step); V is read whole from its channel-major tile (each
// lane D/64 channel rows of 16 slots) and turned into token rows through LDS.
template <int D, int MODE>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
    constexpr int ESZ = MODE == 2 ? 2 : 1;
    constexpr int CH = D / 8;            // 8-channel chunks per row
    constexpr int RPI = kWave / CH;      // rows per step
    constexpr int NJ = TS / RPI;         // steps per tile
    constexpr int CPW = D / 64;          // 16-slot channel rows per lane of the V tile
    constexpr int VL = CPW * TS * ESZ / 16;  // 16-byte loads per lane of V channel rows
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[4][TS * D * ESZ];
    __shared__ long long off_s;
    typedef uint32_t piece_t[ESZ * 2];   // 8 codes (2 dwords) or 8 bf16 values (4 dwords)

    int r = blockIdx.x;
    const int h = r % a.hkv;
    r /= a.hkv;
    const int chunk = r % a.nchunk;
    const int b = r / a.nchunk;
    const int ctx = a.ctx[b];
    const int pc = chunk * CHUNK;
    if (pc >= ctx) return;  // uniform over the workgroup
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int rl = lane / CH;            // row within a step
    const int c8 = (lane % CH) * 8;      // first channel of the lane's chunk
    uint8_t* lds = lds_all[w];

    // ---- issue every load of the wave's tiles
    int p0[TPW];
    int64_t page[TPW];
    piece_t kraw[TPW][NJ];
    u32x4 vraw[TPW][VL];
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
        p0[it] = pc + TS * (w + 4 * it);
        page[it] = 0;
        if (p0[it] >= ctx) continue;  // uniform per wave
        page[it] = (int64_t)a.bt[(int64_t)b * a.mbs + (p0[it] >> a.log2bs)] * a.hkv + h;
        const int sib = p0[it] & (a.bs - 1);
        const uint8_t* kt = reinterpret_cast<const uint8_t*>(a.k) + ((page[it] * a.bs + sib) * D + c8) * ESZ;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
            const int sl = jj * RPI + rl;
            const bool on = a.k_out && sl < ctx - p0[it];
            if constexpr (ESZ == 1) {
                const uint2 v = on ? *reinterpret_cast<const uint2*>(kt + sl * D) : make_uint2(0u, 0u);
                kraw[it][jj][0] = v.x;
                kraw[it][jj][1] = v.y;
            } else {
                const u32x4 v = on ? load16(kt + sl * D * 2) : u32x4{0u, 0u, 0u, 0u};
                kraw[it][jj][0] = v.x; kraw[it][jj][1] = v.y; kraw[it][jj][2] = v.z; kraw[it][jj][3] = v.w;
            }
        }
        const uint8_t* vt = reinterpret_cast<const uint8_t*>(a.v) +
                            (page[it] * D * a.bs + (int64_t)(sib / TS) * D * TS + (int64_t)lane * CPW * TS) * ESZ;
#pragma unroll
        for (int l = 0; l < VL; ++l) vraw[it][l] = a.v_out ? load16(vt + 16 * l) : u32x4{0u, 0u, 0u, 0u};
    }
    // the output row offset of the sequence (while the tile loads are in flight)
    if (a.seq_off) {
        if (threadIdx.x == 0) off_s = a.seq_off[b];
    } else if (threadIdx.x < kWave) {  // exclusive prefix sum of the context lengths, by wave 0
        long long acc = 0;
        for (int i = threadIdx.x; i < b; i += kWave) acc += a.ctx[i];
        for (int sh = 1; sh < kWave; sh <<= 1) acc += __shfl_xor(acc, sh, kWave);
        if (threadIdx.x == 0) off_s = acc;
    }
    __syncthreads();
    const long long off = off_s;

#pragma unroll
    for (int it = 0; it < TPW; ++it) {
        if (p0[it] >= ctx) break;  // uniform per wave; no barrier follows
        const int sib = p0[it] & (a.bs - 1);
        const int n = ctx - p0[it];  // slots of the tile inside the sequence (may exceed 16)
        const int64_t pg = page[it];
        // bf16 of the 8 values of a piece of slot sl; scale per token, per block or per channel
        auto convert = [&](const uint32_t* raw, const float* sc, int sl, uint32_t* y) {
            if constexpr (MODE == 2) {
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = raw[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    float s0, s1;
                    if constexpr (MODE == 0) s0 = s1 = sc[pg * a.bs + sib + sl];
                    else if constexpr (MODE == 1) s0 = s1 = sc[pg];
                    else {
                        s0 = sc[(int64_t)h * D + c8 + e];
                        s1 = sc[(int64_t)h * D + c8 + e + 1];
                    }
                    y[e / 2] = deq_pair(code_of(raw[e >> 2], e & 3), code_of(raw[e >> 2], (e & 3) + 1), s0, s1);
                }
            }
        };
        auto write_piece = [&](uint16_t* out, int sl, const uint32_t* y) {
            uint16_t* dst = out + (off + p0[it] + sl) * a.token_stride + (int64_t)h * a.head_stride + c8;
            if (a.vec_ok) {
                *reinterpret_cast<uint4*>(dst) = make_uint4(y[0], y[1], y[2], y[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dst[2 * e] = (uint16_t)(y[e] & 0xffffu);
                    dst[2 * e + 1] = (uint16_t)(y[e] >> 16);
                }
            }
        };

        if (a.k_out) {
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                const int sl = jj * RPI + rl;
                if (sl < n) {
                    uint32_t y[4];
                    convert(kraw[it][jj], a.ks, sl, y);
                    write_piece(a.k_out, sl, y);
                }
            }
        }
        if (!a.v_out) continue;
        // V: the lane's CPW channel rows -> LDS as token rows
        if (it > 0) __builtin_amdgcn_wave_barrier();  // the previous tile's LDS reads come first
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            if constexpr (MODE == 2) {  // slot t of channels CPW lane ..: 16-bit elements
                const uint32_t e0 = (word(vraw[it][t >> 3], (t >> 1) & 3) >> (16 * (t & 1))) & 0xffffu;
                if constexpr (CPW == 2) {
                    const uint32_t e1 = (word(vraw[it][2 + (t >> 3)], (t >> 1) & 3) >> (16 * (t & 1))) & 0xffffu;
                    *reinterpret_cast<uint32_t*>(lds + (t * D + 2 * lane) * 2) = e0 | (e1 << 16);
                } else {
                    *reinterpret_cast<uint16_t*>(lds + (t * D + lane) * 2) = (uint16_t)e0;
                }
            } else {
                const uint32_t b0 = (word(vraw[it][0], t >> 2) >> (8 * (t & 3))) & 0xffu;
                if constexpr (CPW == 2) {
                    const uint32_t b1 = (word(vraw[it][1], t >> 2) >> (8 * (t & 3))) & 0xffu;
                    *reinterpret_cast<uint16_t*>(lds + t * D + 2 * lane) = (uint16_t)(b0 | (b1 << 8));
                } else {
                    lds[t * D + lane] = (uint8_t)b0;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
            const int sl = jj * RPI + rl;
            if (sl < n) {
                piece_t raw;
                if constexpr (ESZ == 1) {
                    const uint2 v = *reinterpret_cast<const uint2*>(lds + sl * D + c8);
                    raw[0] = v.x;
                    raw[1] = v.y;
                } else {
                    const uint4 v = *reinterpret_cast<const uint4*>(lds + (sl * D + c8) * 2);
                    raw[0] = v.x; raw[1] = v.y; raw[2] = v.z; raw[3] = v.w;
                }
                uint32_t y[4];
                convert(raw, a.vs, sl, y);
                write_piece(a.v_out, sl, y);
            }
        }
    }
}

template <int D>
hipError_t launch_d(const DequantArgs& a, int mode, hipStream_t stream) {
    const int64_t grid = (int64_t)a.batch * a.nchunk * a.hkv;
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
