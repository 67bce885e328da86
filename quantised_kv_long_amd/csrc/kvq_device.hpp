// kvq_device.hpp -- device-side helpers shared by the kernels of the library:
// binary16 bit handling, storage-format constants and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

enum : int { T_F16 = 0, T_Q8 = 1, T_Q4 = 2 };

// Bytes of one data-plane row of D values.
__host__ __device__ constexpr int data_row_bytes(int t, int D)
{
    return t == T_F16 ? 2 * D : (t == T_Q8 ? D : D / 2);
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

// Eight consecutive elements [e, e + 8) of a stored row, dequantised to fp32
// (code * scale is exact in fp32: an 11-bit scale times an integer of at most
// 8 bits).  `row` points at the row's first data byte, `srow` at its scales.
// e must be a multiple of 8.
template <int T>
__device__ __forceinline__ void load8(const uint8_t* row, const uint16_t* srow, int e, float* out)
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
    } else {
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
    }
}

}  // namespace kvq
