// quant_append.hip -- quantise-on-write of new K/V rows into the cache
// (HAL #582 "per-layer KV compression study", section 5 P2 write path: a token
// is quantised once, when it is written; section 1 gives the block formats).
//
// One thread per 32-value block.  The arithmetic follows the library's fixed
// block quantiser exactly (binary32 division, fp16 round-to-nearest-even of the
// scale, division of each value by the *stored* scale, round half away from
// zero), so the stored bytes are bit-identical on every run.  Nothing here is
// contracted into FMAs: the only float operations are divisions, fabs/max and
// the final rounding.
#include "kvq_internal.hpp"

namespace kvq {
namespace {

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

__global__ void __launch_bounds__(256) quantize_append_kernel(AppendArgs a)
{
    const int nb = a.D >> 5;
    const int64_t n_blocks = (int64_t)a.B * a.n_new * a.Hkv * nb;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_blocks) return;
    const bool is_v = blockIdx.y == 1;
    const Plane& P = is_v ? a.v : a.k;
    const int t = is_v ? a.tv : a.tk;
    const uint16_t* src = (is_v ? a.v_new : a.k_new) + idx * 32;

    const int blk = (int)(idx % nb);
    int64_t rest = idx / nb;
    const int g = (int)(rest % a.Hkv);
    rest /= a.Hkv;
    const int r = (int)(rest % a.n_new);
    const int b = (int)(rest / a.n_new);
    const int64_t row = (int64_t)b * P.seq_stride + (int64_t)g * P.head_stride + a.positions[b] + r;
    uint8_t* dst = P.data + row * data_row_bytes(t, a.D) + (int64_t)blk * data_row_bytes(t, 32);
    uint16_t* sdst = P.scales + row * nb + blk;
    if (t == T_F16)
        quantize_block<T_F16>(src, dst, sdst);
    else if (t == T_Q8)
        quantize_block<T_Q8>(src, dst, sdst);
    else
        quantize_block<T_Q4>(src, dst, sdst);
}

}  // namespace

hipError_t launch_quantize_append(const AppendArgs& a, hipStream_t s)
{
    const int64_t n_blocks = (int64_t)a.B * a.n_new * a.Hkv * (a.D >> 5);
    if (n_blocks == 0) return hipSuccess;
    dim3 grid((unsigned)((n_blocks + 255) / 256), 2);
    hipLaunchKernelGGL(quantize_append_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
