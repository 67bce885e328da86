// combine.hip -- exact log-sum-exp merge of split partials (HAL #582
// "per-layer KV compression study", section 5 P2 read path: regions are merged
// by an exact online-softmax combine; here the regions are the splits).
//
// One workgroup (256 threads) per (sequence, query head, chunk of at most
// 128 columns, chosen by chunk_cols); the merge itself is combine_fold_src() /
// combine_finish() in kvq_combine.hpp.  A chunk of W columns gives its 256
// threads 256 / (W / 4) residue classes of the splits (8 for 128 columns),
// each folding its splits in batches of 8 or 16 loads; every chunk reads all
// the lse values and writes its own columns (the first chunk also writes the
// LSE).
#include "kvq_combine.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

// Columns of one merge workgroup for rows of D columns (a multiple of 32) and
// up to S splits: the whole row up to 128 columns, else the largest multiple
// of 32 up to 128 that divides it; then narrower divisors while a thread
// would fold more than 16 splits (one batch of loads), since a chunk of w
// columns has 256 / (w / 4) residue classes.
inline int chunk_cols(int D, int S)
{
    auto next_down = [D](int w) {
        for (int v = w - 32; v >= 32; v -= 32)
            if (D % v == 0) return v;
        return 32;
    };
    int w = D <= 128 ? D : next_down(160);
    while (w > 32 && (S + CMB_NT / (w / 4) - 1) / (CMB_NT / (w / 4)) > 16) w = next_down(w);
    return w;
}

__global__ void __launch_bounds__(CMB_NT) combine_kernel(CombineArgs a)
{
    __shared__ CombineLds sm;
    const int h = blockIdx.x, b = blockIdx.y;
    const int W = a.D / (int)gridDim.z, c0 = blockIdx.z * W;
    const int L = a.seq_lens[b];
    const int S = L > 0 ? min((L + a.split_tokens - 1) / a.split_tokens, a.max_splits) : 0;
    const int64_t bh = (int64_t)b * a.Hq + h;
    void* out = a.out_f16 ? (void*)(reinterpret_cast<uint16_t*>(a.out) + bh * a.D + c0)
                          : (void*)(reinterpret_cast<float*>(a.out) + bh * a.D + c0);
    const float* pl = a.part_lse + bh * a.max_splits;
    const CombineSrc1 src{pl, reinterpret_cast<const float4*>(a.part_o + bh * a.max_splits * a.D + c0),
                          a.D >> 2};
    float* lse = a.lse_out && blockIdx.z == 0 ? a.lse_out + bh : nullptr;
    // one batch of loads covers S <= 8 * (256 / (W / 4)) splits with U = 8
    CombineState st = combine_init();
    if (S <= 8 * (CMB_NT / (W / 4)))
        combine_fold_src<8>(src, S, W, st);
    else
        combine_fold_src<16>(src, S, W, st);
    combine_finish(st, W, a.out_f16, out, lse, sm);
}

// The splits of all regions of one (sequence, query head) as one list:
// region 0's splits, then region 1's, ... so that one batch of loads spans
// the regions.
struct CombineSrcN {
    const float* pl[MAX_REGIONS];
    const float4* po4[MAX_REGIONS];
    int first[MAX_REGIONS];   // index of each region's split 0 in the list
    int n, D4;
    __device__ __forceinline__ void load(int sp, int c, float& ls, float4& v) const
    {
        // the last region whose first split is at or before sp (static
        // indices only: the arrays stay in registers)
        const float* p = pl[0];
        const float4* o = po4[0];
        int f = 0;
#pragma unroll
        for (int k = 1; k < MAX_REGIONS; ++k) {
            if (k < n && sp >= first[k]) {
                p = pl[k];
                o = po4[k];
                f = first[k];
            }
        }
        ls = p[sp - f];
        v = o[(int64_t)(sp - f) * D4 + c];
    }
};

// The same merge over the partials of several regions (HAL #582 section 5
// P2: each region of a mixed cache, the fp16 window and the quantised tail,
// has its own typed attention; their partials are merged exactly).
__global__ void __launch_bounds__(CMB_NT) combine_regions_kernel(CombineRegionsArgs a)
{
    __shared__ CombineLds sm;
    const int h = blockIdx.x, b = blockIdx.y;
    const int W = a.D / (int)gridDim.z, c0 = blockIdx.z * W;
    const int64_t bh = (int64_t)b * a.Hq + h;
    void* out = a.out_f16 ? (void*)(reinterpret_cast<uint16_t*>(a.out) + bh * a.D + c0)
                          : (void*)(reinterpret_cast<float*>(a.out) + bh * a.D + c0);
    CombineSrcN src;
    src.n = a.n;
    src.D4 = a.D >> 2;                 // row stride in float4 (each row starts at column c0)
    int S = 0;
#pragma unroll
    for (int i = 0; i < MAX_REGIONS; ++i) {
        src.first[i] = S;
        if (i >= a.n) continue;
        const int L = a.seq_lens[i][b];
        S += L > 0 ? min((L + a.split_tokens[i] - 1) / a.split_tokens[i], a.max_splits[i]) : 0;
        src.pl[i] = a.part_lse[i] + bh * a.max_splits[i];
        src.po4[i] = reinterpret_cast<const float4*>(a.part_o[i] + bh * a.max_splits[i] * a.D + c0);
    }
    CombineState st = combine_init();
    if (S <= 8 * (CMB_NT / (W / 4)))
        combine_fold_src<8>(src, S, W, st);
    else
        combine_fold_src<16>(src, S, W, st);
    combine_finish(st, W, a.out_f16, out, a.lse_out && blockIdx.z == 0 ? a.lse_out + bh : nullptr, sm);
}

}  // namespace

hipError_t launch_combine_regions(const CombineRegionsArgs& a, hipStream_t s)
{
    int S = 0;
    for (int i = 0; i < a.n; ++i) S += a.max_splits[i];
    dim3 grid(a.Hq, a.B, a.D / chunk_cols(a.D, S));
    hipLaunchKernelGGL(combine_regions_kernel, grid, dim3(CMB_NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s)
{
    dim3 grid(a.Hq, a.B, a.D / chunk_cols(a.D, a.max_splits));
    hipLaunchKernelGGL(combine_kernel, grid, dim3(CMB_NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
