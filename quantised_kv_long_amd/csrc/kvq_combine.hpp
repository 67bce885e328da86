// kvq_combine.hpp -- exact log-sum-exp merge of the split partials of one
// (sequence, query head) by a whole workgroup (HAL #582 "per-layer KV
// compression study", section 5 P2 read path: regions merged by an exact
// online-softmax combine; here the regions are the splits).  Used by the
// standalone combine kernel and by the fused decode step.
//
// fp32 throughout:
//   LSE = m + ln sum_s exp(lse_s - m),  m = max_s lse_s
//   out = sum_s exp(lse_s - LSE) * o_s
// The weights go to LDS in chunks; each thread owns four adjacent columns (one
// 16-byte load per split row) and a residue class of splits, with UNROLL
// independent loads in flight, so a pass costs about one memory round trip
// rather than one per split.  The split groups are summed through LDS.
#pragma once

#include <math.h>

#include "kvq_device.hpp"

namespace kvq {

constexpr int CMB_NT = 256;        // threads of the calling workgroup
constexpr int CMB_WCHUNK = 1024;   // weights staged per pass
constexpr int CMB_UNROLL = 8;

struct CombineLds {
    float tmp[CMB_NT / 64];
    float w[CMB_WCHUNK];
    float4 red[CMB_NT];
};

__device__ __forceinline__ float cmb_block_reduce(float v, bool is_max, float* tmp)
{
    v = is_max ? wave_max(v) : wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) tmp[wave] = v;
    __syncthreads();
    float r = tmp[0];
    for (int w = 1; w < CMB_NT / 64; ++w) r = is_max ? fmaxf(r, tmp[w]) : r + tmp[w];
    return r;
}

// pl: the S partial lse values; po: the S partial rows of D floats (16-byte
// aligned); writes D outputs at out (fp16 or fp32) and, if lse_dst is not
// NULL, the merged lse.  S == 0 (or all splits empty) gives out = 0, lse = -inf.
__device__ __forceinline__ void combine_rows(const float* pl, const float* po, int S, int D,
                                             bool out_f16, void* out, float* lse_dst, CombineLds& sm)
{
    const int tid = threadIdx.x;
    float m = -INFINITY;
    for (int s = tid; s < S; s += CMB_NT) m = fmaxf(m, pl[s]);
    m = cmb_block_reduce(m, true, sm.tmp);

    float lse = -INFINITY;
    if (m != -INFINITY) {
        float sum = 0.0f;
        for (int s = tid; s < S; s += CMB_NT) sum += expf(pl[s] - m);
        sum = cmb_block_reduce(sum, false, sm.tmp);
        lse = m + logf(sum);
    }

    const int D4 = D >> 2;                 // float4 columns (D <= 512: at most 128)
    const int R = CMB_NT / D4;             // split residue classes
    const int c = tid % D4, r = tid / D4;
    const bool on = r < R;
    const float4* po4 = reinterpret_cast<const float4*>(po);
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);

    if (lse != -INFINITY) {
        for (int c0 = 0; c0 < S; c0 += CMB_WCHUNK) {
            const int n = min(CMB_WCHUNK, S - c0);
            __syncthreads();
            for (int i = tid; i < n; i += CMB_NT) sm.w[i] = expf(pl[c0 + i] - lse);
            __syncthreads();
            if (on) {
                for (int i0 = r; i0 < n; i0 += R * CMB_UNROLL) {
                    float4 v[CMB_UNROLL];
                    float wi[CMB_UNROLL];
#pragma unroll
                    for (int u = 0; u < CMB_UNROLL; ++u) {
                        const int i = i0 + u * R;
                        if (i < n) {
                            v[u] = po4[(int64_t)(c0 + i) * D4 + c];
                            wi[u] = sm.w[i];
                        } else {
                            v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                            wi[u] = 0.0f;
                        }
                    }
#pragma unroll
                    for (int u = 0; u < CMB_UNROLL; ++u) {
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
    if (on) sm.red[r * D4 + c] = acc;
    __syncthreads();
    if (tid < D4) {
        float4 v = sm.red[tid];
        for (int k = 1; k < R; ++k) {
            const float4 u = sm.red[k * D4 + tid];
            v.x += u.x;
            v.y += u.y;
            v.z += u.z;
            v.w += u.w;
        }
        if (out_f16) {
            uint16_t* o = reinterpret_cast<uint16_t*>(out) + 4 * tid;
            o[0] = f2h_rne(v.x);
            o[1] = f2h_rne(v.y);
            o[2] = f2h_rne(v.z);
            o[3] = f2h_rne(v.w);
        } else {
            reinterpret_cast<float4*>(out)[tid] = v;
        }
    }
    if (tid == 0 && lse_dst) *lse_dst = lse;
    __syncthreads();
}

// ---------------------------------------------------------------------------
// The same merge for the G query heads of one KV head at once, by one
// workgroup of CMB_NT threads (the fused decode step's last workgroup).  Head n
// has its S lse values at pl + n * pl_stride and its S rows of D floats at
// po + n * po_stride; outputs go to out (G rows of D, fp16 or fp32) and, if
// lse_dst is not NULL, lse_dst[n].  `lds` is scratch of lds_floats floats, at
// least CMB_GROUP_LDS_MIN(G); G * D / 4 must not exceed MAXI * CMB_NT.
//
// The per-head LSE is reduced by a group of CMB_NT / Gp threads per head (Gp
// = G rounded up to a power of two); the weighted sum gives each thread one
// float4 column of one head and a residue class of splits, with CMB_GUNROLL
// loads in flight, so reading all G * S partial rows takes few round trips.
constexpr int CMB_GUNROLL = 16;

__host__ __device__ constexpr int CMB_GROUP_LDS_MIN(int G) { return 32 + 4 * CMB_NT + 8 * G; }

__device__ __forceinline__ float cmb_group_reduce(float v, bool is_max, int tph, float* red)
{
    // reduce over groups of tph consecutive threads; tph is a power of two
    const int tid = threadIdx.x;
    const int w = tph < 64 ? tph : 64;
    for (int off = w >> 1; off >= 1; off >>= 1) {
        const float o = __shfl_xor(v, off, 64);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    if (tph > 64) {
        __syncthreads();
        if ((tid & 63) == 0) red[tid >> 6] = v;
        __syncthreads();
        const int g0 = (tid / tph) * (tph >> 6);
        v = red[g0];
        for (int k = 1; k < (tph >> 6); ++k) v = is_max ? fmaxf(v, red[g0 + k]) : v + red[g0 + k];
    }
    return v;
}

template <int MAXI>
__device__ __forceinline__ void combine_group(const float* pl, int64_t pl_stride, const float* po,
                                              int64_t po_stride, int G, int S, int D, bool out_f16,
                                              void* out, float* lse_dst, float* lds, int lds_floats)
{
    const int tid = threadIdx.x;
    int gp = 1;
    while (gp < G) gp <<= 1;
    const int tph = CMB_NT / gp;          // threads per head for the LSE
    const int hn = tid / tph, hj = tid % tph;
    float* red = lds;                     // [CMB_NT / 64]
    float* lse_s = lds + 16;              // [G]
    float4* acc_s = reinterpret_cast<float4*>(lds + 32);   // [CMB_NT] float4
    float* w = lds + 32 + 4 * CMB_NT;     // weights, [G][chunk]
    const int chunk = (lds_floats - 32 - 4 * CMB_NT) / G;

    // -- LSE of every head
    float m = -INFINITY;
    if (hn < G)
        for (int s = hj; s < S; s += tph) m = fmaxf(m, pl[hn * pl_stride + s]);
    m = cmb_group_reduce(m, true, tph, red);
    float sum = 0.0f;
    if (hn < G && m != -INFINITY)
        for (int s = hj; s < S; s += tph) sum += expf(pl[hn * pl_stride + s] - m);
    sum = cmb_group_reduce(sum, false, tph, red);
    __syncthreads();
    if (hn < G && hj == 0) lse_s[hn] = m == -INFINITY ? -INFINITY : m + logf(sum);
    __syncthreads();

    // -- weighted sum: item = (head, float4 column), R residue classes of splits
    const int D4 = D >> 2;
    const int items = G * D4;
    const int R = items >= CMB_NT ? 1 : CMB_NT / items;
    float4 acc[MAXI];                     // items per thread (G * D / 4 <= MAXI * CMB_NT)
#pragma unroll
    for (int k = 0; k < MAXI; ++k) acc[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const int r = tid / (items < CMB_NT ? items : CMB_NT);
    for (int c0 = 0; c0 < S; c0 += chunk) {
        const int n = min(chunk, S - c0);
        __syncthreads();
        for (int i = tid; i < G * n; i += CMB_NT) {
            const int h = i / n, s = i % n;
            const float L = lse_s[h];
            w[h * chunk + s] = L == -INFINITY ? 0.0f : expf(pl[h * pl_stride + c0 + s] - L);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < MAXI; ++k) {
            const int item = (items < CMB_NT ? tid % items : tid) + k * CMB_NT;
            if (item >= items || r >= R) continue;
            const int h = item / D4, c = item % D4;
            const float4* src = reinterpret_cast<const float4*>(po + h * po_stride) + c;
            const float* wh = w + h * chunk;
            float4 a = acc[k];
            for (int i0 = r; i0 < n; i0 += R * CMB_GUNROLL) {
                float4 v[CMB_GUNROLL];
                float wi[CMB_GUNROLL];
#pragma unroll
                for (int u = 0; u < CMB_GUNROLL; ++u) {
                    const int i = i0 + u * R;
                    if (i < n) {
                        v[u] = src[(int64_t)(c0 + i) * D4];
                        wi[u] = wh[i];
                    } else {
                        v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                        wi[u] = 0.0f;
                    }
                }
#pragma unroll
                for (int u = 0; u < CMB_GUNROLL; ++u) {
                    a.x += wi[u] * v[u].x;
                    a.y += wi[u] * v[u].y;
                    a.z += wi[u] * v[u].z;
                    a.w += wi[u] * v[u].w;
                }
            }
            acc[k] = a;
        }
    }

    // -- sum the residue classes and write
    if (items < CMB_NT) {
        __syncthreads();
        if (r < R) acc_s[r * items + tid % items] = acc[0];
        __syncthreads();
    }
    for (int item = tid; item < items; item += CMB_NT) {
        float4 v;
        if (items < CMB_NT) {
            v = acc_s[item];
            for (int k = 1; k < R; ++k) {
                const float4 u = acc_s[k * items + item];
                v.x += u.x;
                v.y += u.y;
                v.z += u.z;
                v.w += u.w;
            }
        } else {
            v = acc[(item - tid) / CMB_NT];
        }
        const int h = item / D4, c = item % D4;
        if (out_f16) {
            uint16_t* o = reinterpret_cast<uint16_t*>(out) + (int64_t)h * D + 4 * c;
            o[0] = f2h_rne(v.x);
            o[1] = f2h_rne(v.y);
            o[2] = f2h_rne(v.z);
            o[3] = f2h_rne(v.w);
        } else {
            reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (int64_t)h * D)[c] = v;
        }
    }
    if (lse_dst && tid < G) lse_dst[tid] = lse_s[tid];
    __syncthreads();
}

}  // namespace kvq
