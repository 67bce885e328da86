// quant_append.hip -- quantise-on-write of new K/V rows into the cache
// (HAL #582 "per-layer KV compression study", section 5 P2 write path: a token
// is quantised once, when it is written; section 1 gives the block formats).
//
// One thread per 32-value block; the block quantiser itself is in
// kvq_quant.hpp.  The source rows are addressed through strides, so the same
// kernel takes new tokens ([B][n_new][Hkv][D]) and rows of fp16 cache planes
// (the rolling fp16 window of a mixed cache, quantised when it is evicted).
#include "kvq_internal.hpp"
#include "kvq_quant.hpp"

namespace kvq {
namespace {

__global__ void __launch_bounds__(256) quantize_append_kernel(AppendArgs a)
{
    const int nb = a.D >> 5;
    const int64_t n_blocks = (int64_t)a.B * a.n_new * a.Hkv * nb;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_blocks) return;
    const bool is_v = blockIdx.y == 1;
    const Plane& P = is_v ? a.v : a.k;
    const int t = is_v ? a.tv : a.tk;

    const int blk = (int)(idx % nb);
    int64_t rest = idx / nb;
    const int g = (int)(rest % a.Hkv);
    rest /= a.Hkv;
    const int r = (int)(rest % a.n_new);
    const int b = (int)(rest / a.n_new);
    if (a.counts && r >= a.counts[b]) return;
    const uint16_t* src = is_v ? a.v_new + b * a.v_sb + r * a.v_sr + g * a.v_sg
                               : a.k_new + b * a.k_sb + r * a.k_sr + g * a.k_sg;
    src += 32 * blk;
    const int pos0 = a.positions ? a.positions[b] : a.seq_lens[b] - a.n_new;
    if (pos0 + r < 0) return;  // a sequence shorter than its new rows: nothing before row 0
    const int64_t row = (int64_t)b * P.seq_stride + (int64_t)g * P.head_stride + pos0 + r;
    uint8_t* rowp = P.data + row * data_row_bytes(t, a.D);
    uint16_t* srow = P.scales + row * nb * scales_per_block(t);
    switch (t) {
    case T_F16: quantize_block<T_F16>(src, rowp + 64 * blk, nullptr); break;
    case T_Q8: quantize_block<T_Q8>(src, rowp + 32 * blk, srow + blk); break;
    case T_Q4: quantize_block<T_Q4>(src, rowp + 16 * blk, srow + blk); break;
    case T_Q4_1: quantize_block_ext<T_Q4_1>(src, rowp, srow, blk, a.D); break;
    case T_Q5_0: quantize_block_ext<T_Q5_0>(src, rowp, srow, blk, a.D); break;
    case T_Q5_1: quantize_block_ext<T_Q5_1>(src, rowp, srow, blk, a.D); break;
    default: quantize_block_ext<T_Q6_0>(src, rowp, srow, blk, a.D); break;
    }
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
