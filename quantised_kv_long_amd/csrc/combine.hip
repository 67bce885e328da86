// combine.hip -- exact log-sum-exp merge of split partials (HAL #582
// "per-layer KV compression study", section 5 P2 read path: regions are merged
// by an exact online-softmax combine; here the regions are the splits).
//
// One workgroup (256 threads) per (sequence, query head).  fp32 throughout:
//   LSE = m + ln sum_s exp(lse_s - m),  m = max_s lse_s
//   out = sum_s exp(lse_s - LSE) * o_s
// The weights are staged in LDS in chunks; threads stride over the D columns
// (coalesced reads of each partial row) and over splits when D < 256.
#include <math.h>

#include "kvq_internal.hpp"

namespace kvq {
namespace {

constexpr int NT = 256;
constexpr int WCHUNK = 1024;

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
    const float* po = a.part_o + bh * a.max_splits * D;

    __shared__ float tmp[NT / 64];
    __shared__ float w[WCHUNK];
    __shared__ float red[NT * 2];

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

    const int nd = D < NT ? D : NT;       // threads per split row
    const int R = NT / nd;                // splits processed side by side
    const int dd = tid % nd, rr = tid / nd;
    const bool on = rr < R;
    constexpr int MAXD_PER_THREAD = 2;    // D <= 512
    float acc[MAXD_PER_THREAD] = {0.0f, 0.0f};

    if (lse != -INFINITY) {
        for (int c0 = 0; c0 < S; c0 += WCHUNK) {
            const int n = min(WCHUNK, S - c0);
            __syncthreads();
            for (int i = tid; i < n; i += NT) w[i] = expf(pl[c0 + i] - lse);
            __syncthreads();
            if (on) {
                for (int i = rr; i < n; i += R) {
                    const float wi = w[i];
                    const float* row = po + (int64_t)(c0 + i) * D;
#pragma unroll
                    for (int k = 0; k < MAXD_PER_THREAD; ++k) {
                        const int d = dd + k * nd;
                        if (d < D) acc[k] += wi * row[d];
                    }
                }
            }
        }
    }

    // sum the R split groups (each thread holds up to 2 columns)
    for (int k = 0; k < MAXD_PER_THREAD; ++k) {
        __syncthreads();
        if (on) red[rr * nd + dd] = acc[k];
        __syncthreads();
        const int d = tid + k * nd;
        if (tid < nd && d < D) {
            float v = 0.0f;
            for (int r = 0; r < R; ++r) v += red[r * nd + tid];
            if (a.out_f16)
                reinterpret_cast<uint16_t*>(a.out)[bh * D + d] = f2h_rne(v);
            else
                reinterpret_cast<float*>(a.out)[bh * D + d] = v;
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
