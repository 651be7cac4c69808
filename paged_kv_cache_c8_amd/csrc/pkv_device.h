// pkv_device.h - device-side helpers shared by the libpkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------------
// Cache page layout: K page (block, KV head) is [BS][D] (token rows); V page is [BS/16][D][16]:
// tiles of 16 slots, each channel-major (the 16 slots of one channel are contiguous).
// ---------------------------------------------------------------------------------------------

constexpr int kVTile = 16;  // slots per V tile

// element offset of V (page = block * Hkv + head, channel c, slot) from the start of the cache
__device__ __forceinline__ int64_t v_elem(int64_t page, int D, int bs, int c, int slot) {
    return page * D * bs + ((int64_t)(slot / kVTile) * D + c) * kVTile + slot % kVTile;
}

// ---------------------------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Nearest bf16 (ties to the even significand) of a finite or infinite fp32; NaN -> quiet NaN.
// Adding 0x7fff plus the lowest kept bit carries into the kept half exactly when the discarded
// half is above the midpoint, or at the midpoint with an odd kept half.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------------------------
// int8 quantization (per token / per block): code = clamp(rne(fl32(x / s)), -128, 127), 0 if s == 0.
// The division is IEEE correctly rounded (the library is built with correctly rounded fp32
// division and without denormal flushing) and rintf rounds halves to even.
// ---------------------------------------------------------------------------------------------

__device__ __forceinline__ int quant_code(float x, float s) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(x / s);
    r = fminf(fmaxf(r, -128.0f), 127.0f);
    return (int)r;
}

__device__ __forceinline__ float absmax_scale(float absmax) { return absmax / 127.0f; }

// The same codes as quant_code for the values x of a row whose scale is an absmax scale,
// s = fl32(A / 127) of a bf16 A >= |x| (per-token rows, per-block rows, MLA rows), with one IEEE
// division per row instead of one per value: r = fl32(1 / s), and per value Markstein's correction
// step (P. Markstein, IBM J. Res. Develop. 34(1), 1990): q0 = fl32(x r), e = x - q0 s (one fused
// rounding), q = fl32(q0 + e r).  q can differ from fl32(x / s) in its last bit, but rint(q) never
// differs from rint(fl32(x / s)) on that domain when s >= 2^-100 (checked on the host for every such
// bf16 pair, about 1.05e9); smaller scales (and s == 0) take quant_code itself.
template <int N>
__device__ __forceinline__ void quant_row_absmax(const float* x, float s, int* codes) {
    if (s >= 0x1p-100f) {
        const float r = 1.0f / s;
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float q0 = x[e] * r;
            const float er = __builtin_fmaf(-q0, s, x[e]);
            float q = __builtin_rintf(__builtin_fmaf(er, r, q0));
            q = fminf(fmaxf(q, -128.0f), 127.0f);
            codes[e] = (int)q;
        }
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) codes[e] = quant_code(x[e], s);
    }
}

// ---------------------------------------------------------------------------------------------
// Cross-lane exchange.  Within a row of 16 lanes, DPP moves data without LDS traffic:
//   stride 1: quad_perm [1,0,3,2]     stride 2: quad_perm [2,3,0,1]
//   stride 4: row_half_mirror (lane i <-> 7 - i in each half row; flips bit 2 and the bits below)
//   stride 8: row_mirror      (lane i <-> 15 - i; flips bit 3 and the bits below)
// Each is a perfect matching whose partner differs in the stride bit, which is all that the
// butterfly reductions below require.  Strides 16 and 32 cross rows and use __shfl_xor (ds_bpermute).
// ---------------------------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

template <int S>
__device__ __forceinline__ float lane_xchg(float x) {
    if constexpr (S == 1) return dpp_mov<0xB1>(x);
    else if constexpr (S == 2) return dpp_mov<0x4E>(x);
    else if constexpr (S == 4) return dpp_mov<0x141>(x);
    else if constexpr (S == 8) return dpp_mov<0x140>(x);
    else return __shfl_xor(x, S, kWave);
}

template <int N>  // reduce over aligned groups of N lanes (N power of two <= 64)
__device__ __forceinline__ float group_max(float x) {
    if constexpr (N >= 2) x = fmaxf(x, lane_xchg<1>(x));
    if constexpr (N >= 4) x = fmaxf(x, lane_xchg<2>(x));
    if constexpr (N >= 8) x = fmaxf(x, lane_xchg<4>(x));
    if constexpr (N >= 16) x = fmaxf(x, lane_xchg<8>(x));
    if constexpr (N >= 32) x = fmaxf(x, lane_xchg<16>(x));
    if constexpr (N >= 64) x = fmaxf(x, lane_xchg<32>(x));
    return x;
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += lane_xchg<1>(x);
    if constexpr (N >= 4) x += lane_xchg<2>(x);
    if constexpr (N >= 8) x += lane_xchg<4>(x);
    if constexpr (N >= 16) x += lane_xchg<8>(x);
    if constexpr (N >= 32) x += lane_xchg<16>(x);
    if constexpr (N >= 64) x += lane_xchg<32>(x);
    return x;
}

// ---------------------------------------------------------------------------------------------
// 16-byte global loads (kept as four dwords)
// ---------------------------------------------------------------------------------------------

struct u32x4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 load16(const void* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return {v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ uint32_t word(const u32x4& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// element e (0..15) of 16 int8 codes, as float (exact)
__device__ __forceinline__ float i8_at(const u32x4& v, int e) {
    return (float)(int8_t)((word(v, e >> 2) >> (8 * (e & 3))) & 0xffu);
}

// element e (0..7) of 8 bf16 values, as float (exact)
__device__ __forceinline__ float bf16_at(const u32x4& v, int e) {
    const uint32_t w = word(v, e >> 1);
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
}

}  // namespace pkv
