// kvq_device.hpp -- device-side helpers shared by the kernels of the library:
// binary16 bit handling, storage-format constants and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Storage types.  f16, q8_0 and q4_0 are the pages' tiers; q4_1, q5_0, q5_1
// and q6_0 are the further scalar types of their served pairs (block sizes 20,
// 22, 24 and 26 bytes per 32 values).
enum : int { T_F16 = 0, T_Q8 = 1, T_Q4 = 2, T_Q4_1 = 4, T_Q5_0 = 5, T_Q5_1 = 6, T_Q6_0 = 7 };

__host__ __device__ constexpr bool valid_type(int t)
{
    return t == T_F16 || t == T_Q8 || t == T_Q4 || t == T_Q4_1 || t == T_Q5_0 || t == T_Q5_1 ||
           t == T_Q6_0;
}

// Bytes of one data-plane row of D values: the low nibbles of every block
// (D/2 bytes) and then, for q5 / q6, every block's high bits (4 or 8 bytes).
__host__ __device__ constexpr int data_row_bytes(int t, int D)
{
    return t == T_F16 ? 2 * D
         : t == T_Q8 ? D
         : (t == T_Q5_0 || t == T_Q5_1) ? D / 2 + D / 8
         : t == T_Q6_0 ? D / 2 + D / 4
         : D / 2;
}

// fp16 entries of the scale plane per 32-value block: the scale d, and for
// q4_1 / q5_1 the block minimum m after it.
__host__ __device__ constexpr int scales_per_block(int t)
{
    return t == T_F16 ? 0 : (t == T_Q4_1 || t == T_Q5_1) ? 2 : 1;
}

// Device view of one cache tensor: row index of (sequence b, KV head g, row t)
// is b * seq_stride + g * head_stride + t in both planes.
struct Plane {
    uint8_t* data;
    uint16_t* scales;
    int64_t seq_stride;
    int64_t head_stride;
};

__device__ __forceinline__ float h2f(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f2h_rne(float x)
{
    // v_cvt_f16_f32 rounds to nearest even in the default float mode and keeps
    // binary16 subnormals (the default denormal mode preserves them).
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Eight consecutive elements [e, e + 8) of a stored row of D values,
// dequantised to fp32 (code * scale is exact in fp32: an 11-bit scale times an
// integer of at most 8 bits; the minimum of q4_1 / q5_1 is added with one
// rounding).  `row` points at the row's first data byte, `srow` at its
// scales.  e must be a multiple of 8.
template <int T>
__device__ __forceinline__ void load8(const uint8_t* row, const uint16_t* srow, int e, int D, float* out)
{
    if constexpr (T == T_F16) {
        uint4 u = *reinterpret_cast<const uint4*>(row + 2 * e);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = h2f((uint16_t)(w[i] & 0xffff));
            out[2 * i + 1] = h2f((uint16_t)(w[i] >> 16));
        }
    } else if constexpr (T == T_Q8) {
        uint2 u = *reinterpret_cast<const uint2*>(row + e);
        const float d = h2f(srow[e >> 5]);
        const uint32_t w[2] = {u.x, u.y};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int8_t c = (int8_t)((w[i >> 2] >> (8 * (i & 3))) & 0xff);
            out[i] = d * (float)c;
        }
    } else if constexpr (T == T_Q4) {
        const int blk = e >> 5, p = e & 31;
        uint2 u = *reinterpret_cast<const uint2*>(row + 16 * blk + (p & 15));
        const float d = h2f(srow[blk]);
        const int sh = p < 16 ? 0 : 4;
        const uint32_t w[2] = {u.x, u.y};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int c = (int)((w[i >> 2] >> (8 * (i & 3) + sh)) & 0xf) - 8;
            out[i] = d * (float)c;
        }
    } else {
        // q4_1, q5_0, q5_1, q6_0: low nibbles as q4_0, high bits after all
        // blocks' nibbles (rows of these types are only 4-byte aligned)
        const int blk = e >> 5, p = e & 31;
        const uint32_t* lo = reinterpret_cast<const uint32_t*>(row + 16 * blk + (p & 15));
        const uint32_t w[2] = {lo[0], lo[1]};
        const int sh = p < 16 ? 0 : 4;
        uint64_t hb = 0;
        if constexpr (T == T_Q5_0 || T == T_Q5_1)
            hb = *reinterpret_cast<const uint32_t*>(row + D / 2 + 4 * blk) >> p;
        if constexpr (T == T_Q6_0) {
            const uint32_t* h = reinterpret_cast<const uint32_t*>(row + D / 2 + 8 * blk);
            hb = ((uint64_t)h[0] | ((uint64_t)h[1] << 32)) >> (2 * p);
        }
        constexpr int HB = (T == T_Q5_0 || T == T_Q5_1) ? 1 : T == T_Q6_0 ? 2 : 0;
        constexpr int SPB = scales_per_block(T);
        const float d = h2f(srow[SPB * blk]);
        const float m = SPB == 2 ? h2f(srow[SPB * blk + 1]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int c = (int)((w[i >> 2] >> (8 * (i & 3) + sh)) & 0xf);
            if constexpr (HB > 0) c |= (int)((hb >> (HB * i)) & ((1u << HB) - 1)) << 4;
            if constexpr (T == T_Q5_0) out[i] = d * (float)(c - 16);
            else if constexpr (T == T_Q6_0) out[i] = d * (float)(c - 32);
            else out[i] = fmaf(d, (float)c, m);
        }
    }
}

}  // namespace kvq
