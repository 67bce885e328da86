// kvq_combine.hpp -- exact log-sum-exp merge of the split partials of one
// (sequence, query head) by a whole workgroup (HAL #582 "per-layer KV
// compression study", section 5 P2 read path: regions merged by an exact
// online-softmax combine; here the regions are the splits).
//
// fp32 throughout.  The mathematical result is
//   LSE = ln sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) * o_s .
// Each thread owns four adjacent columns (one 16-byte load per split row) and
// a residue class r of the splits (s = r, r + R, ...).  It issues the loads of
// up to U (8 or 16) of its splits at once (lse values and rows together) and
// folds them into a running (max m, sum l, weighted row a) -- the same online
// softmax as within a split -- so a merge of up to R * U splits costs
// one memory round trip.  The R running triples of a column are then merged
// through LDS:  M = max m_r,  l = sum exp(m_r - M) l_r,  a = sum exp(m_r - M) a_r,
// out = a / l,  LSE = M + ln l.
#pragma once

#include <math.h>

#include "kvq_device.hpp"

namespace kvq {

constexpr int CMB_NT = 256;        // threads of the calling workgroup
constexpr float CMB_LOG2E = 1.4426950408889634f;

struct CombineLds {
    float m[CMB_NT];
    float l[CMB_NT];
    float4 a[CMB_NT];
};

// The running merge of one thread: max m, sum l, weighted row a.
struct CombineState {
    float m, l;
    float4 a;
};

__device__ __forceinline__ CombineState combine_init()
{
    return CombineState{-INFINITY, 0.0f, make_float4(0.0f, 0.0f, 0.0f, 0.0f)};
}

// Partials of one region: lse values at pl, rows of D floats at po (16-byte
// aligned).  load(sp, c) gives split sp's lse and its float4 column c.
struct CombineSrc1 {
    const float* pl;
    const float4* po4;
    int D4;
    __device__ __forceinline__ void load(int sp, int c, float& ls, float4& v) const
    {
        ls = pl[sp];
        v = po4[(int64_t)sp * D4 + c];
    }
};

// Folds S partials (split sp read by src.load) into the thread's running
// state: its four columns of its residue class of the splits.  Splits with
// lse = -inf carry no weight.  U splits are loaded per batch.  Weights are
// exp2((lse - m) * log2 e) on the hardware exp2: the relative error of a
// weight is a few fp32 ulps times |lse - m|.
template <int U, class Src>
__device__ __forceinline__ void combine_fold_src(const Src& src, int S, int D, CombineState& st)
{
    const int tid = threadIdx.x;
    const int D4 = D >> 2;                 // float4 columns (D <= 512: at most 128)
    const int R = CMB_NT / D4;             // split residue classes
    const int c = tid % D4, r = tid / D4;

    float m = st.m, l = st.l;
    float4 a = st.a;
    for (int s0 = r; s0 < S; s0 += R * U) {
        float ls[U];
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = s0 + u * R;
            if (sp < S) {
                src.load(sp, c, ls[u], v[u]);
            } else {
                ls[u] = -INFINITY;
                v[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
        float bm = ls[0];
#pragma unroll
        for (int u = 1; u < U; ++u) bm = fmaxf(bm, ls[u]);
        if (bm > m) {                      // move the reference (m = -inf: nothing to scale)
            const float f = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m - bm) * CMB_LOG2E);
            l *= f;
            a.x *= f;
            a.y *= f;
            a.z *= f;
            a.w *= f;
            m = bm;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = ls[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((ls[u] - m) * CMB_LOG2E);
            l += w;
            a.x += w * v[u].x;
            a.y += w * v[u].y;
            a.z += w * v[u].z;
            a.w += w * v[u].w;
        }
    }
    st.m = m;
    st.l = l;
    st.a = a;
}

// The S partials at pl / po.
template <int U>
__device__ __forceinline__ void combine_fold(const float* pl, const float* po, int S, int D,
                                             CombineState& st)
{
    combine_fold_src<U>(CombineSrc1{pl, reinterpret_cast<const float4*>(po), D >> 2}, S, D, st);
}

// Merges the residue classes' states through LDS and writes D outputs at out
// (fp16 or fp32) and, if lse_dst is not NULL, the merged lse.  No weight at
// all (no splits, or all empty) gives out = 0, lse = -inf.
__device__ __forceinline__ void combine_finish(const CombineState& st, int D, bool out_f16, void* out,
                                               float* lse_dst, CombineLds& sm)
{
    const int tid = threadIdx.x;
    const int D4 = D >> 2;
    const int R = CMB_NT / D4;
    __syncthreads();
    sm.m[tid] = st.m;
    sm.l[tid] = st.l;
    sm.a[tid] = st.a;
    __syncthreads();
    if (tid < D4) {
        float M = -INFINITY;
        for (int k = 0; k < R; ++k) M = fmaxf(M, sm.m[k * D4 + tid]);
        float L = 0.0f;
        float4 A = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (M != -INFINITY) {
            for (int k = 0; k < R; ++k) {
                const float mk = sm.m[k * D4 + tid];
                const float f = mk == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mk - M) * CMB_LOG2E);
                const float4 ak = sm.a[k * D4 + tid];
                L += f * sm.l[k * D4 + tid];
                A.x += f * ak.x;
                A.y += f * ak.y;
                A.z += f * ak.z;
                A.w += f * ak.w;
            }
        }
        float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (L > 0.0f) {
            const float inv = 1.0f / L;
            o = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
        }
        if (out_f16) {
            uint16_t* op = reinterpret_cast<uint16_t*>(out) + 4 * tid;
            op[0] = f2h_rne(o.x);
            op[1] = f2h_rne(o.y);
            op[2] = f2h_rne(o.z);
            op[3] = f2h_rne(o.w);
        } else {
            reinterpret_cast<float4*>(out)[tid] = o;
        }
        if (tid == 0 && lse_dst) *lse_dst = L > 0.0f ? M + logf(L) : -INFINITY;
    }
}

// The whole merge of the S partials of one (sequence, query head).
template <int U>
__device__ __forceinline__ void combine_rows(const float* pl, const float* po, int S, int D,
                                             bool out_f16, void* out, float* lse_dst, CombineLds& sm)
{
    CombineState st = combine_init();
    combine_fold<U>(pl, po, S, D, st);
    combine_finish(st, D, out_f16, out, lse_dst, sm);
}

}  // namespace kvq
