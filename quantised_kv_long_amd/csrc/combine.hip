// combine.hip -- exact log-sum-exp merge of split partials (HAL #582
// "per-layer KV compression study", section 5 P2 read path: regions are merged
// by an exact online-softmax combine; here the regions are the splits).
//
// One workgroup (256 threads) per (sequence, query head).  fp32 throughout:
//   LSE = m + ln sum_s exp(lse_s - m),  m = max_s lse_s
//   out = sum_s exp(lse_s - LSE) * o_s
// The weights go to LDS; then each thread owns four adjacent columns (one
// 16-byte load per split row) and a residue class of splits, with UNROLL
// independent loads in flight so the pass costs about one memory round trip
// rather than one per split.  The split groups are summed through LDS.
#include <math.h>

#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr int NT = 256;
constexpr int WCHUNK = 4096;
constexpr int UNROLL = 8;

__device__ float block_reduce(float v, bool is_max, float* tmp)
{
    v = is_max ? wave_max(v) : wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) tmp[wave] = v;
    __syncthreads();
    float r = tmp[0];
    for (int w = 1; w < NT / 64; ++w) r = is_max ? fmaxf(r, tmp[w]) : r + tmp[w];
    return r;
}

__global__ void __launch_bounds__(NT) combine_kernel(CombineArgs a)
{
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const int D = a.D;
    const int L = a.seq_lens[b];
    const int S = L > 0 ? min((L + a.split_tokens - 1) / a.split_tokens, a.max_splits) : 0;
    const int64_t bh = (int64_t)b * a.Hq + h;
    const float* pl = a.part_lse + bh * a.max_splits;
    const float4* po = reinterpret_cast<const float4*>(a.part_o + bh * a.max_splits * D);

    __shared__ float tmp[NT / 64];
    __shared__ float w[WCHUNK];
    __shared__ float4 red[NT];

    float m = -INFINITY;
    for (int s = tid; s < S; s += NT) m = fmaxf(m, pl[s]);
    m = block_reduce(m, true, tmp);

    float lse = -INFINITY;
    if (m != -INFINITY) {
        float sum = 0.0f;
        for (int s = tid; s < S; s += NT) sum += expf(pl[s] - m);
        sum = block_reduce(sum, false, tmp);
        lse = m + logf(sum);
    }

    const int D4 = D >> 2;                 // float4 columns (D <= 512: at most 128)
    const int R = NT / D4;                 // split residue classes
    const int c = tid % D4, r = tid / D4;
    const bool on = r < R;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);

    if (lse != -INFINITY) {
        for (int c0 = 0; c0 < S; c0 += WCHUNK) {
            const int n = min(WCHUNK, S - c0);
            __syncthreads();
            for (int i = tid; i < n; i += NT) w[i] = expf(pl[c0 + i] - lse);
            __syncthreads();
            if (on) {
                for (int i0 = r; i0 < n; i0 += R * UNROLL) {
                    float4 v[UNROLL];
                    float wi[UNROLL];
#pragma unroll
                    for (int u = 0; u < UNROLL; ++u) {
                        const int i = i0 + u * R;
                        if (i < n) {
                            v[u] = po[(int64_t)(c0 + i) * D4 + c];
                            wi[u] = w[i];
                        } else {
                            v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                            wi[u] = 0.0f;
                        }
                    }
#pragma unroll
                    for (int u = 0; u < UNROLL; ++u) {
                        acc.x += wi[u] * v[u].x;
                        acc.y += wi[u] * v[u].y;
                        acc.z += wi[u] * v[u].z;
                        acc.w += wi[u] * v[u].w;
                    }
                }
            }
        }
    }

    __syncthreads();
    if (on) red[r * D4 + c] = acc;
    __syncthreads();
    if (tid < D4) {
        float4 v = red[tid];
        for (int k = 1; k < R; ++k) {
            const float4 u = red[k * D4 + tid];
            v.x += u.x;
            v.y += u.y;
            v.z += u.z;
            v.w += u.w;
        }
        if (a.out_f16) {
            uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + bh * D + 4 * tid;
            o[0] = f2h_rne(v.x);
            o[1] = f2h_rne(v.y);
            o[2] = f2h_rne(v.z);
            o[3] = f2h_rne(v.w);
        } else {
            reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + bh * D)[tid] = v;
        }
    }
    if (tid == 0 && a.lse_out) a.lse_out[bh] = lse;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s)
{
    dim3 grid(a.Hq, a.B);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
