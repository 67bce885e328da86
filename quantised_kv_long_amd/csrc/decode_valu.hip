// decode_valu.hip -- split-KV decode attention with the dot products on the
// vector ALUs (HAL #582 "per-layer KV compression study", section 3b finding 2:
// a quant reader that dequantises stored blocks in registers; section 5 P2: per
// region partial results merged later by an exact log-sum-exp combine).
//
// One workgroup (256 threads, 4 wave64) per (sequence b, KV head g, split s).
// The whole GQA group of G query heads shares every K and V element read.
// Per tile of 64 rows:
//   QK     : 4 threads per row, each dequantising a quarter of the row (8
//            elements at a time, code * scale exact in fp32) and accumulating
//            the G dot products against Q held in LDS; a 2-step shuffle sums
//            the quarters.  Scores are kept in the log2 domain
//            (Q pre-multiplied by softmax_scale * log2 e).
//   softmax: one wave per head: wave-wide max, exp2, wave-wide sum (shuffle
//            reductions); running max m and sum l per head in LDS.
//   PV     : thread (8-element column chunk, row group) accumulates
//            o[h][8] += p[h][t] * v[t][chunk] over its rows.
// At the end the row groups are summed through LDS and the split partial
// (o / l, ln-domain lse) is written.  Every value is fp32; no atomics.
#include <math.h>

#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr int TILE = 64;
constexpr int NT = 256;

template <int TK, int TV, int GP>
__global__ void __launch_bounds__(NT) decode_valu_kernel(DecodeArgs a)
{
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.D, G = a.G;
    const int L = a.seq_lens[b];
    const int t_begin = s * a.split_tokens;
    const int t_end = min(t_begin + a.split_tokens, L);
    const int h0 = g * G;
    const int64_t ho_stride = (int64_t)a.max_splits * D;  // part_o stride between heads
    float* po = a.part_o + (((int64_t)b * a.Hq + h0) * a.max_splits + s) * D;
    float* pl = a.part_lse + ((int64_t)b * a.Hq + h0) * a.max_splits + s;

    // a split at or past ceil(L / split_tokens) holds no row: the merge never
    // reads its partials, so nothing is written
    if (t_begin >= t_end) return;

    extern __shared__ float smem[];
    float* qs = smem;                // [GP][D]   Q * scale * log2(e)
    float* sc = qs + GP * D;         // [GP][TILE] scores, then probabilities
    float* mrun = sc + GP * TILE;    // [GP] running max (log2 domain)
    float* lrun = mrun + GP;         // [GP] running sum
    float* alph = lrun + GP;         // [GP] rescale factor of the current tile
    float* red = alph + GP;          // [NT / (D/8)][D] row-group reduction

    for (int i = tid; i < GP * D; i += NT) {
        const int h = i / D;
        qs[i] = h < G ? h2f(a.q[((int64_t)b * a.Hq + h0 + h) * D + (i % D)]) * a.scale_log2 : 0.0f;
    }
    if (tid < GP) { mrun[tid] = -INFINITY; lrun[tid] = 0.0f; }

    const int rbK = data_row_bytes(TK, D), rbV = data_row_bytes(TV, D);
    const int nsK = (D >> 5) * scales_per_block(TK), nsV = (D >> 5) * scales_per_block(TV);
    const int64_t krow0 = (int64_t)b * a.k.seq_stride + (int64_t)g * a.k.head_stride;
    const int64_t vrow0 = (int64_t)b * a.v.seq_stride + (int64_t)g * a.v.head_stride;
    const uint8_t* kdata = a.k.data + krow0 * rbK;
    const uint16_t* kscl = a.k.scales + krow0 * nsK;
    const uint8_t* vdata = a.v.data + vrow0 * rbV;
    const uint16_t* vscl = a.v.scales + vrow0 * nsV;

    // QK mapping: row = tid / 4, quarter = tid % 4
    const int qk_row = tid >> 2, qk_part = tid & 3;
    const int qk_e0 = qk_part * (D >> 2), qk_e1 = qk_e0 + (D >> 2);
    // PV mapping: 8-element chunk c, row group rg
    const int NC = D >> 3, NG = NT / NC;
    const int pv_c = tid % NC, pv_g = tid / NC;
    const bool pv_on = pv_g < NG;

    float o[GP][8];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[h][j] = 0.0f;

    __syncthreads();

    for (int t0 = t_begin; t0 < t_end; t0 += TILE) {
        const int nt = min(TILE, t_end - t0);
        // ---- QK
        {
            float acc[GP];
#pragma unroll
            for (int h = 0; h < GP; ++h) acc[h] = 0.0f;
            const int t = t0 + qk_row;
            if (qk_row < nt) {
                const uint8_t* row = kdata + (int64_t)t * rbK;
                const uint16_t* srow = kscl + (int64_t)t * nsK;
                for (int e = qk_e0; e < qk_e1; e += 8) {
                    float kv[8];
                    load8<TK>(row, srow, e, D, kv);
#pragma unroll
                    for (int h = 0; h < GP; ++h) {
                        if (h < G) {
                            const float4 qa = *reinterpret_cast<const float4*>(qs + h * D + e);
                            const float4 qb = *reinterpret_cast<const float4*>(qs + h * D + e + 4);
                            acc[h] += qa.x * kv[0] + qa.y * kv[1] + qa.z * kv[2] + qa.w * kv[3] +
                                      qb.x * kv[4] + qb.y * kv[5] + qb.z * kv[6] + qb.w * kv[7];
                        }
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                acc[h] += __shfl_xor(acc[h], 1, 64);
                acc[h] += __shfl_xor(acc[h], 2, 64);
            }
            if (qk_part == 0) {
#pragma unroll
                for (int h = 0; h < GP; ++h)
                    if (h < G) sc[h * TILE + qk_row] = qk_row < nt ? acc[h] : -INFINITY;
            }
        }
        __syncthreads();
        // ---- online softmax, one wave per head
        for (int h = wave; h < G; h += NT / 64) {
            const float x = sc[h * TILE + lane];
            const float m_old = mrun[h];
            const float m_new = fmaxf(m_old, wave_max(x));
            const float p = exp2f(x - m_new);
            const float psum = wave_sum(p);
            sc[h * TILE + lane] = p;
            if (lane == 0) {
                const float al = exp2f(m_old - m_new);
                alph[h] = al;
                lrun[h] = lrun[h] * al + psum;
                mrun[h] = m_new;
            }
        }
        __syncthreads();
        // ---- PV
        if (pv_on) {
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                if (h < G) {
                    const float al = alph[h];
#pragma unroll
                    for (int j = 0; j < 8; ++j) o[h][j] *= al;
                }
            }
            for (int r = pv_g; r < nt; r += NG) {
                const int t = t0 + r;
                float vv[8];
                load8<TV>(vdata + (int64_t)t * rbV, vscl + (int64_t)t * nsV, pv_c * 8, D, vv);
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    if (h < G) {
                        const float p = sc[h * TILE + r];
#pragma unroll
                        for (int j = 0; j < 8; ++j) o[h][j] += p * vv[j];
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- sum the row groups per head and write the partial
    for (int h = 0; h < G; ++h) {
        // o[][] must stay in registers: select head h with an unrolled loop
        // rather than a runtime index
        if (pv_on) {
#pragma unroll
            for (int hh = 0; hh < GP; ++hh)
                if (hh == h)
#pragma unroll
                    for (int j = 0; j < 8; ++j) red[pv_g * D + pv_c * 8 + j] = o[hh][j];
        }
        __syncthreads();
        const float inv_l = 1.0f / lrun[h];
        for (int d = tid; d < D; d += NT) {
            float v = 0.0f;
            for (int r = 0; r < NG; ++r) v += red[r * D + d];
            po[h * ho_stride + d] = v * inv_l;
        }
        if (tid == 0) pl[(int64_t)h * a.max_splits] = (mrun[h] + log2f(lrun[h])) * 0.69314718055994531f;
        __syncthreads();
    }
}

template <int TK, int TV>
hipError_t launch_tv(const DecodeArgs& a, hipStream_t s)
{
    const int NC = a.D >> 3, NG = NT / NC;
    dim3 grid(grid_splits(a), a.Hkv, a.B);
    if (a.G <= 8) {
        const size_t lds = sizeof(float) * (8 * a.D + 8 * TILE + 3 * 8 + NG * a.D);
        hipLaunchKernelGGL((decode_valu_kernel<TK, TV, 8>), grid, dim3(NT), lds, s, a);
    } else {
        const size_t lds = sizeof(float) * (16 * a.D + 16 * TILE + 3 * 16 + NG * a.D);
        hipLaunchKernelGGL((decode_valu_kernel<TK, TV, 16>), grid, dim3(NT), lds, s, a);
    }
    return hipGetLastError();
}

template <int TK>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s)
{
    switch (a.tv) {
    case T_F16: return launch_tv<TK, T_F16>(a, s);
    case T_Q8: return launch_tv<TK, T_Q8>(a, s);
    case T_Q4: return launch_tv<TK, T_Q4>(a, s);
    case T_Q4_1: return launch_tv<TK, T_Q4_1>(a, s);
    case T_Q5_0: return launch_tv<TK, T_Q5_0>(a, s);
    case T_Q5_1: return launch_tv<TK, T_Q5_1>(a, s);
    case T_Q6_0: return launch_tv<TK, T_Q6_0>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Every pair of storage types (K and V chosen independently).
hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t s)
{
    switch (a.tk) {
    case T_F16: return launch_t<T_F16>(a, s);
    case T_Q8: return launch_t<T_Q8>(a, s);
    case T_Q4: return launch_t<T_Q4>(a, s);
    case T_Q4_1: return launch_t<T_Q4_1>(a, s);
    case T_Q5_0: return launch_t<T_Q5_0>(a, s);
    case T_Q5_1: return launch_t<T_Q5_1>(a, s);
    case T_Q6_0: return launch_t<T_Q6_0>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
