// combine.hip -- exact log-sum-exp merge of split partials (HAL #582
// "per-layer KV compression study", section 5 P2 read path: regions are merged
// by an exact online-softmax combine; here the regions are the splits).
//
// One workgroup (256 threads) per (sequence, query head, chunk of at most
// 128 columns, chosen by chunk_cols); the merge itself is combine_fold_src() /
// combine_finish() in kvq_combine.hpp.  A chunk of W columns gives its 256
// threads cmb_classes(W / 4) residue classes of the splits (8 for 128
// columns), each folding its splits in batches of 2 to 16 loads; every chunk reads all
// the lse values and writes its own columns (the first chunk also writes the
// LSE).  The splits loaded are those that can hold rows given the launch
// arguments (live_splits), so the loads do not wait for the sequence lengths;
// with several sequences (LEN_FIRST) the length is read first instead and
// the loads are range-checked to the sequence's own splits, so a short
// sequence's dead splits cost no memory traffic.
#include "kvq_combine.hpp"
#include "kvq_internal.hpp"

namespace kvq {
namespace {

#ifndef KVQ_CMB_TARGET_U
#define KVQ_CMB_TARGET_U 4
#endif

// Columns of one merge workgroup for rows of D columns (a multiple of 32) and
// n splits to load: 128, 64 or 32, the widest that divides D, then halved
// while a thread would load more than KVQ_CMB_TARGET_U splits (a chunk of w
// columns has cmb_classes(w / 4) residue classes): narrower chunks mean more
// workgroups and fewer loads per thread.  Every chunk width gives all 256
// threads a column.
inline int chunk_cols(int D, int n)
{
    int w = D % 128 == 0 ? 128 : D % 64 == 0 ? 64 : 32;
    while (w > 32 && (n + cmb_classes(w / 4) - 1) / cmb_classes(w / 4) > KVQ_CMB_TARGET_U) w /= 2;
    return w;
}

// Splits one thread loads per batch: the fewest of 2, 4, 8, 16 that cover n
// splits in one batch (16 beyond).
inline int batch_splits(int n, int W)
{
    const int R = cmb_classes(W / 4);
    return n <= 2 * R ? 2 : n <= 4 * R ? 4 : n <= 8 * R ? 8 : 16;
}

// Scalar arguments, 14 dwords: the build preloads the first 14 argument
// dwords into scalar registers (a struct argument gets none), so no
// argument is read from memory.  hdw packs Hq (bits 0-15), D / 32 (bits
// 16-20) and the chunk width W / 32 (bits 26-28).
template <int U, bool F16, bool LEN_FIRST>
__global__ void __launch_bounds__(CMB_NT)
combine_kernel(const float* part_o, const float* part_lse, int hdw, int max_splits, int live_splits,
               int split_tokens, const int32_t* seq_lens, void* out_p, float* lse_out)
{
    const int Hq = hdw & 0xFFFF, D = ((hdw >> 16) & 31) * 32, W = ((hdw >> 26) & 7) * 32;
    const int h = blockIdx.x, b = blockIdx.y;
    const int c0 = blockIdx.z * W;
    const int64_t bh = (int64_t)b * Hq + h;
    CombineSrc1 src;
    src.len = seq_lens + b;
    src.split_tokens = split_tokens;
    src.D = D;
    src.n = live_splits;
    src.S = 0;
    // the splits a load may touch: all that can hold rows (the loads are
    // issued before the sequence length arrives), or with LEN_FIRST those of
    // this sequence (past them a load reads zero and touches no memory)
    int nr = max_splits;
    if constexpr (LEN_FIRST) {
        src.settle();
        nr = src.S;
    }
    src.rl = cmb_rsrc(part_lse + bh * max_splits, (int64_t)nr * 4);
    const int64_t ro_floats = (int64_t)nr * D - c0;
    src.ro = cmb_rsrc(part_o + bh * max_splits * D + c0, (ro_floats > 0 ? ro_floats : 0) * 4);
    void* out = F16 ? (void*)(reinterpret_cast<uint16_t*>(out_p) + bh * D + c0)
                    : (void*)(reinterpret_cast<float*>(out_p) + bh * D + c0);
    float* lse = lse_out && blockIdx.z == 0 ? lse_out + bh : nullptr;
    CombineState st = combine_init();
    combine_fold_src<U>(src, W, st);
    combine_finish(st, W, F16, out, lse);
}

// The splits of all regions of one (sequence, query head) as one list of
// slots: region 0's live_splits slots, then region 1's, ... (slot offsets from
// the launch arguments), so that one batch of loads spans the regions and
// needs no sequence length; slots past a region's own split count are masked.
struct CombineSrcN {
    const float* pl[MAX_REGIONS];   // lse values of the (sequence, head)
    const float* po[MAX_REGIONS];   // its rows, from the chunk's first column
    int first[MAX_REGIONS];         // slot of each region's split 0
    int last[MAX_REGIONS];          // max_splits - 1: loads clamp to it
    int S[MAX_REGIONS];             // splits holding rows, per region
    int live_n[MAX_REGIONS];        // each region's slots
    int split_tokens[MAX_REGIONS];
    const int32_t* len[MAX_REGIONS];   // the sequence's length in each region
    int nreg, D, n, e;
    // (global loads with per-lane addresses: the lanes of one load may fall
    // in different regions; every address stays inside the region's partials)
    __device__ __forceinline__ void load(int su, int r, int c, uint32_t& ls, cmb_u32x4& v) const
    {
        const int sp = su + r;
        const float* l = pl[0];
        const float* o = po[0];
        int f = 0, z = last[0];
#pragma unroll
        for (int i = 1; i < MAX_REGIONS; ++i) {
            if (i < nreg && sp >= first[i]) {
                l = pl[i];
                o = po[i];
                f = first[i];
                z = last[i];
            }
        }
        const int j = min(sp - f, z);
        ls = *reinterpret_cast<const uint32_t*>(l + j);
        v = *reinterpret_cast<const cmb_u32x4*>(o + (int64_t)j * D + 4 * c);
    }
    __device__ __forceinline__ void settle()
    {
        e = 0;
#pragma unroll
        for (int i = 0; i < MAX_REGIONS; ++i) {
            // (an unused region has live_n = 0, so S = 0)
            const int L = max(*len[i], 0);
            S[i] = min((L + split_tokens[i] - 1) / split_tokens[i], live_n[i]);
            e = S[i] > 0 ? first[i] + S[i] : e;
        }
    }
    __device__ __forceinline__ bool live(int sp) const
    {
        bool ok = false;
#pragma unroll
        for (int i = 0; i < MAX_REGIONS; ++i)
            if (i < nreg && sp >= first[i] && sp < first[i] + S[i]) ok = true;
        return ok;
    }
    __device__ __forceinline__ int end() const { return e; }
};

// The same merge over the partials of several regions (HAL #582 section 5
// P2: each region of a mixed cache, the fp16 window and the quantised tail,
// has its own typed attention; their partials are merged exactly).
template <int U>
__global__ void __launch_bounds__(CMB_NT) combine_regions_kernel(CombineRegionsArgs a)
{
    // every argument is read in one round (pinned here, or the compiler
    // spreads the loads over several)
    asm volatile("" ::"s"(a.part_o[0]), "s"(a.part_o[1]), "s"(a.part_o[2]), "s"(a.part_o[3]));
    asm volatile("" ::"s"(a.part_lse[0]), "s"(a.part_lse[1]), "s"(a.part_lse[2]), "s"(a.part_lse[3]));
    asm volatile("" ::"s"(a.seq_lens[0]), "s"(a.seq_lens[1]), "s"(a.seq_lens[2]), "s"(a.seq_lens[3]));
    asm volatile("" ::"s"(a.live_splits[0]), "s"(a.live_splits[1]), "s"(a.live_splits[2]), "s"(a.live_splits[3]));
    asm volatile("" ::"s"(a.max_splits[0]), "s"(a.max_splits[1]), "s"(a.max_splits[2]), "s"(a.max_splits[3]));
    asm volatile("" ::"s"(a.split_tokens[0]), "s"(a.split_tokens[1]), "s"(a.split_tokens[2]),
                 "s"(a.split_tokens[3]));
    asm volatile("" ::"s"(a.Hq), "s"(a.D), "s"(a.W), "s"(a.n), "s"(a.out), "s"(a.lse_out));
    const int h = blockIdx.x, b = blockIdx.y;
    const int W = a.W, c0 = blockIdx.z * W;
    const int64_t bh = (int64_t)b * a.Hq + h;
    CombineSrcN src;
    src.nreg = a.n;
    src.D = a.D;
    // every field of every region is read without a branch: the launcher
    // fills an unused region with region 0's pointers and no splits
    int n = 0;
#pragma unroll
    for (int i = 0; i < MAX_REGIONS; ++i) {
        src.first[i] = n;
        src.S[i] = 0;
        src.live_n[i] = a.live_splits[i];
        src.split_tokens[i] = a.split_tokens[i];
        src.last[i] = a.max_splits[i] - 1;
        src.pl[i] = a.part_lse[i] + bh * a.max_splits[i];
        src.po[i] = a.part_o[i] + bh * a.max_splits[i] * a.D + c0;
        src.len[i] = a.seq_lens[i] + b;
        n += src.live_n[i];
    }
    src.n = n;
    src.e = 0;
    void* out = a.out_f16 ? (void*)(reinterpret_cast<uint16_t*>(a.out) + bh * a.D + c0)
                          : (void*)(reinterpret_cast<float*>(a.out) + bh * a.D + c0);
    float* lse = a.lse_out && blockIdx.z == 0 ? a.lse_out + bh : nullptr;
    CombineState st = combine_init();
    combine_fold_src<U>(src, W, st);
    combine_finish(st, W, a.out_f16, out, lse);
}

}  // namespace

hipError_t launch_combine_regions(const CombineRegionsArgs& args, hipStream_t s)
{
    CombineRegionsArgs a = args;
    for (int i = a.n; i < MAX_REGIONS; ++i) {
        // an unused region: valid pointers, no splits
        a.part_o[i] = a.part_o[0];
        a.part_lse[i] = a.part_lse[0];
        a.seq_lens[i] = a.seq_lens[0];
        a.split_tokens[i] = a.split_tokens[0];
        a.max_splits[i] = a.max_splits[0];
        a.live_splits[i] = 0;
    }
    int n = 0;
    for (int i = 0; i < a.n; ++i) n += a.live_splits[i];
    const int W = chunk_cols(a.D, n);
    a.W = W;
    const dim3 grid(a.Hq, a.B, a.D / W);
    switch (batch_splits(n, W)) {
    case 2: hipLaunchKernelGGL(combine_regions_kernel<2>, grid, dim3(CMB_NT), 0, s, a); break;
    case 4: hipLaunchKernelGGL(combine_regions_kernel<4>, grid, dim3(CMB_NT), 0, s, a); break;
    case 8: hipLaunchKernelGGL(combine_regions_kernel<8>, grid, dim3(CMB_NT), 0, s, a); break;
    default: hipLaunchKernelGGL(combine_regions_kernel<16>, grid, dim3(CMB_NT), 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s)
{
    const int W = chunk_cols(a.D, a.live_splits);
    const dim3 grid(a.Hq, a.B, a.D / W);
    // (Hq <= 65535 and D <= 512, a multiple of 32, are validated by the caller)
    const int hdw = a.Hq | ((a.D / 32) << 16) | ((W / 32) << 26);
    // one sequence: its length is the largest, every split up to live_splits
    // holds rows and the loads need not wait for it; several: the length
    // first, so that the dead splits of the shorter ones are not read
#define KVQ_CMB(UU, FF, LL)                                                                                 \
    hipLaunchKernelGGL((combine_kernel<UU, FF, LL>), grid, dim3(CMB_NT), 0, s, a.part_o, a.part_lse, hdw,      \
                       a.max_splits, a.live_splits, a.split_tokens, a.seq_lens, a.out, a.lse_out)
#define KVQ_CMB2(UU)                  \
    if (a.out_f16) {                  \
        if (a.B > 1)                  \
            KVQ_CMB(UU, true, true);  \
        else                          \
            KVQ_CMB(UU, true, false); \
    } else {                          \
        if (a.B > 1)                  \
            KVQ_CMB(UU, false, true); \
        else                          \
            KVQ_CMB(UU, false, false);\
    }
    switch (batch_splits(a.live_splits, W)) {
    case 2: KVQ_CMB2(2) break;
    case 4: KVQ_CMB2(4) break;
    case 8: KVQ_CMB2(8) break;
    default: KVQ_CMB2(16) break;
    }
#undef KVQ_CMB2
#undef KVQ_CMB
    return hipGetLastError();
}

}  // namespace kvq
