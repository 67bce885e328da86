// kvq_combine.hpp -- exact log-sum-exp merge of the split partials of one
// (sequence, query head) by a whole workgroup (HAL #582 "per-layer KV
// compression study", section 5 P2 read path: regions merged by an exact
// online-softmax combine; here the regions are the splits).
//
// fp32 throughout.  The mathematical result is
//   LSE = ln sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) * o_s .
// Each thread owns four adjacent columns (one 16-byte load per split row) and
// a residue class r of the splits (s = r, r + R, ...); the R classes of a
// column are R adjacent lanes of one wave.  A thread issues the loads of up to
// U (2 to 16) of its splits at once (lse values and rows together) and folds
// them into a running (max m, sum l, weighted row a) -- the same online
// softmax as within a split -- so a merge of up to R * U splits costs one
// memory round trip, which does not wait for the sequence length: the splits
// loaded follow from the launch arguments, and those past the sequence's last
// split are masked out afterwards.  The R running triples of a column are then
// merged across the lanes in log2 R exchange steps (no LDS, no barrier):
//   M = max(m, m'),  l = e^(m - M) l + e^(m' - M) l',  a likewise,
// and finally out = a / l,  LSE = M + ln l.
#pragma once

#include <math.h>

#include "kvq_device.hpp"

namespace kvq {

constexpr int CMB_NT = 256;        // threads of the calling workgroup
constexpr float CMB_LOG2E = 1.4426950408889634f;

// Split residue classes of a chunk of W4 float4 columns (W4 = 8, 16 or 32):
// CMB_NT / W4, so that every thread has a column.
__host__ __device__ constexpr int cmb_classes(int W4)
{
    return CMB_NT / W4;
}

// The running merge of one thread: max m, sum l, weighted row a.
struct CombineState {
    float m, l;
    float4 a;
};

__device__ __forceinline__ CombineState combine_init()
{
    return CombineState{-INFINITY, 0.0f, make_float4(0.0f, 0.0f, 0.0f, 0.0f)};
}

typedef uint32_t cmb_u32x4 __attribute__((ext_vector_type(4)));

// A buffer resource over `bytes` bytes at p: a load at or past the end reads
// zero and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t cmb_rsrc(const void* p, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Partials of one region.  Splits [0, n) are loaded: n follows from the launch
// arguments alone, so no load waits for the sequence length; splits [0, S)
// hold rows, the rest are masked out.  settle() reads the sequence length
// (called once the first batch of loads is in flight).
struct CombineSrc1 {
    __amdgpu_buffer_rsrc_t rl;     // lse values of splits 0, 1, ...
    __amdgpu_buffer_rsrc_t ro;     // rows of D floats, from the chunk's first column
    const int32_t* len;            // the sequence length
    int split_tokens;
    int D, n, S;
    // split su + r (su the same for the whole workgroup): a per-lane offset
    // that stays the same over the batches and a uniform one
    __device__ __forceinline__ void load(int su, int r, int c, uint32_t& ls, cmb_u32x4& v) const
    {
        ls = __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * r, 4 * su, 0);
        v = __builtin_amdgcn_raw_buffer_load_b128(ro, 4 * (r * D + 4 * c), 4 * su * D, 0);
    }
    __device__ __forceinline__ void settle()
    {
        const int L = max(*len, 0);
        S = min((L + split_tokens - 1) / split_tokens, n);
    }
    __device__ __forceinline__ bool live(int sp) const { return sp < S; }
    // no split at or past end() holds rows
    __device__ __forceinline__ int end() const { return S; }
};

// Folds the partials of src into the thread's running state: its four
// columns of its residue class of the splits [0, src.n).  Splits that hold no
// rows, or whose lse is -inf, carry no weight (their loaded values are
// replaced, not multiplied by zero: they may be anything).  U splits are
// loaded per batch; the first batch is issued before src.settle() reads the
// sequence lengths, and each batch's loads are all issued before any of
// their values is used (one memory round trip per batch).
// Weights are exp2((lse - m) * log2 e) on the hardware exp2: the relative
// error of a weight is a few fp32 ulps times |lse - m|.
template <int U, class Src>
__device__ __forceinline__ void combine_fold_src(Src& src, int W, CombineState& st)
{
    const int tid = threadIdx.x;
    const int W4 = W >> 2;                 // float4 columns of the chunk (at most 32)
    const int R = cmb_classes(W4);         // split residue classes (adjacent lanes)
    const int r = tid % R, c = tid / R;

    float m = st.m, l = st.l;
    float4 a = st.a;
    uint32_t lb[U];
    cmb_u32x4 vb[U];
    auto issue = [&](int s0) {
#pragma unroll
        for (int u = 0; u < U; ++u) src.load(s0 + u * R, r, c, lb[u], vb[u]);
    };
    auto fold = [&](int s0) {
        // (the values are opaque from here: the loads stay whole and
        // unconditional, and the wait for them comes after the last is issued)
        // (32-bit operands only: each component of a row is its own operand)
        float ls[U];
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            uint32_t e0 = vb[u][0], e1 = vb[u][1], e2 = vb[u][2], e3 = vb[u][3];
            asm volatile("" : "+v"(lb[u]), "+v"(e0), "+v"(e1), "+v"(e2), "+v"(e3));
            const float x = __builtin_bit_cast(float, lb[u]);
            const bool ok = src.live(s0 + r + u * R) && x != -INFINITY;
            ls[u] = ok ? x : -INFINITY;
            v[u] = ok ? make_float4(__builtin_bit_cast(float, e0), __builtin_bit_cast(float, e1),
                                    __builtin_bit_cast(float, e2), __builtin_bit_cast(float, e3))
                      : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
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
    };
    issue(0);
    __builtin_amdgcn_sched_barrier(0);
    src.settle();
    fold(0);
    for (int s0 = R * U; s0 < src.n && s0 < src.end(); s0 += R * U) {
        issue(s0);
        fold(s0);
    }
    st.m = m;
    st.l = l;
    st.a = a;
}

// Merges the R residue classes of each column across their lanes and writes
// the chunk's W outputs at out (fp16 or fp32) and, if lse_dst is not NULL,
// the merged lse.  No weight at all (no splits, or all empty) gives out = 0,
// lse = -inf.  Every lane of the thread's wave takes part.
__device__ __forceinline__ void combine_finish(const CombineState& st, int W, bool out_f16, void* out,
                                               float* lse_dst)
{
    const int tid = threadIdx.x;
    const int R = cmb_classes(W >> 2);
    const int r = tid % R, c = tid / R;
    float m = st.m, l = st.l;
    float4 a = st.a;
#pragma unroll
    for (int k = 1; k < 32; k <<= 1) {
        if (k < R) {                       // (uniform)
            const float m2 = __shfl_xor(m, k);
            const float l2 = __shfl_xor(l, k);
            const float4 a2 = make_float4(__shfl_xor(a.x, k), __shfl_xor(a.y, k), __shfl_xor(a.z, k),
                                          __shfl_xor(a.w, k));
            const float M = fmaxf(m, m2);
            const float f1 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m - M) * CMB_LOG2E);
            const float f2 = m2 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m2 - M) * CMB_LOG2E);
            l = f1 * l + f2 * l2;
            a = make_float4(f1 * a.x + f2 * a2.x, f1 * a.y + f2 * a2.y, f1 * a.z + f2 * a2.z,
                            f1 * a.w + f2 * a2.w);
            m = M;
        }
    }
    if (r != 0) return;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (l > 0.0f) {
        const float inv = 1.0f / l;
        o = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    }
    if (out_f16) {
        uint16_t* op = reinterpret_cast<uint16_t*>(out) + 4 * c;
        op[0] = f2h_rne(o.x);
        op[1] = f2h_rne(o.y);
        op[2] = f2h_rne(o.z);
        op[3] = f2h_rne(o.w);
    } else {
        reinterpret_cast<float4*>(out)[c] = o;
    }
    if (c == 0 && lse_dst) *lse_dst = l > 0.0f ? m + logf(l) : -INFINITY;
}

}  // namespace kvq
