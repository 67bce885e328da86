// kvq_quant.hpp -- the block quantiser on the device (HAL #582 "per-layer KV
// compression study", section 5 P2 write path: a token is quantised once, when
// it is written; section 1 gives the block formats).  Shared by the
// quantise/append kernel and by the fused decode step, so both write the same
// bytes.
//
// The arithmetic follows the library's fixed block quantiser exactly (binary32
// division, fp16 round-to-nearest-even of the scale, division of each value by
// the *stored* scale, round half away from zero).  Nothing here is contracted
// into FMAs: the only float operations are divisions, fabs/max, one exact
// multiplication by 1/8 and the final rounding.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

// Quantise the 32 fp16 values at src into one block of type T: data bytes at
// dst (64 / 32 / 16 bytes for f16 / q8_0 / q4_0) and the fp16 scale at *sdst
// (untouched for f16).  src and dst must be 16-byte aligned.
template <int T>
__device__ __forceinline__ void quantize_block(const uint16_t* __restrict__ src,
                                               uint8_t* __restrict__ dst,
                                               uint16_t* __restrict__ sdst)
{
    uint4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = reinterpret_cast<const uint4*>(src)[i];

    if constexpr (T == T_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(dst)[i] = raw[i];
        return;
    } else {
        float x[32];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[8 * i + 2 * j] = h2f((uint16_t)(w[j] & 0xffff));
                x[8 * i + 2 * j + 1] = h2f((uint16_t)(w[j] >> 16));
            }
        }
        if constexpr (T == T_Q8) {
            // scale = fp16(max|x| / 127); code = round_half_away(x / scale)
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
            const uint16_t d16 = f2h_rne(amax / 127.0f);
            const float d = h2f(d16);
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = 0;
            if (d != 0.0f) {
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    float r = roundf(x[i] / d);
                    r = fminf(fmaxf(r, -127.0f), 127.0f);
                    const uint32_t c = (uint32_t)(uint8_t)(int8_t)(int)r;
                    w[i >> 2] |= c << (8 * (i & 3));
                }
            }
            reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
            reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
            *sdst = d16;
        } else {
            // scale = fp16(s / -8) with s the first value of largest magnitude;
            // code = clamp(round_half_away(x / scale), -8, 7) + 8, two per byte
            float amax = 0.0f, smax = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const float a = fabsf(x[i]);
                if (a > amax) { amax = a; smax = x[i]; }
            }
            // smax / -8 rounded to fp16.  Formed as magnitude and sign: the
            // compiler otherwise fuses x * -0.125 and the fp16 conversion into a
            // mixed-precision FMA with a +0 addend, which turns the -0 scale of
            // an all-zero block into +0.  |smax| / 8 is exact in binary32 and
            // round-to-nearest-even is symmetric, so the bits are identical.
            const uint16_t mag16 = f2h_rne(fabsf(smax) * 0.125f);
            const uint16_t d16 = (uint16_t)(mag16 | (smax < 0.0f ? 0 : 0x8000));
            const float d = h2f(d16);
            int n[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (d != 0.0f) {
                    float r = roundf(x[i] / d);
                    r = fminf(fmaxf(r, -8.0f), 7.0f);
                    n[i] = (int)r + 8;
                } else {
                    n[i] = 8;
                }
            }
            uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 16; ++j)
                w[j >> 2] |= (uint32_t)(n[j] | (n[j + 16] << 4)) << (8 * (j & 3));
            reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
            *sdst = d16;
        }
    }
}


}  // namespace kvq
