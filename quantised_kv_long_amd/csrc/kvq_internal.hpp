// kvq_internal.hpp -- host-side interface between the C ABI layer (argument
// validation, kvq_api.cpp) and the kernel launchers (*.hip).  Every launcher
// assumes its arguments were validated and only enqueues kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"
#include "kvq_device.hpp"

namespace kvq {

struct AppendArgs {
    Plane k, v;
    int tk, tv;
    // the source rows: value d of row r of KV head g of sequence b is at
    // k_new + b*k_sb + r*k_sr + g*k_sg + d (fp16; likewise for V)
    const uint16_t* k_new;
    const uint16_t* v_new;
    int64_t k_sb, k_sr, k_sg, v_sb, v_sr, v_sg;
    const int32_t* counts;     // rows written per sequence; or null: n_new each
    const int32_t* positions;  // first row per sequence; or null: seq_lens[b] - n_new
    const int32_t* seq_lens;
    int B, n_new, Hkv, D;
};

struct DecodeArgs {
    Plane k, v;
    int tk, tv;
    const uint16_t* q;
    const int32_t* seq_lens;
    int B, Hq, Hkv, D, G;
    // query tokens per sequence (1: single-token decode).  With nq > 1 (the
    // matrix-core kernel only) q is [B][nq][Hq][D], the partials are
    // [B][nq*Hq][max_splits][D], and token i of b sees rows [0, L_b - nq + 1 + i)
    int nq;
    float scale_log2;  // softmax scale * log2(e)
    int max_seq_len, split_tokens, max_splits;
    float* part_o;
    float* part_lse;
    // decode step only (null otherwise): the new K/V rows, [B][nq][Hkv][D]
    // fp16, row i of sequence b written at row seq_lens[b] - nq + i by the
    // workgroup whose split holds that row, before it reads it
    const uint16_t* k_new;
    const uint16_t* v_new;
};

// Splits a decode launch covers: those that can hold a row below
// max_seq_len (every length is at most max_seq_len), at most max_splits.
// Partials past them are never read by the merge.
__host__ __device__ inline int grid_splits(const DecodeArgs& a)
{
    const int n = (a.max_seq_len + a.split_tokens - 1) / a.split_tokens;
    return n < a.max_splits ? n : a.max_splits;
}

// Partials of up to MAX_REGIONS regions (separate decode launches over
// separate caches) merged into one output.
constexpr int MAX_REGIONS = 4;
struct CombineRegionsArgs {
    int n;
    const float* part_o[MAX_REGIONS];
    const float* part_lse[MAX_REGIONS];
    const int32_t* seq_lens[MAX_REGIONS];
    int split_tokens[MAX_REGIONS];
    int max_splits[MAX_REGIONS];
    // splits of each region that can hold rows: min(max_splits,
    // ceil(max_seq_len / split_tokens)) where max_seq_len is known, else
    // max_splits
    int live_splits[MAX_REGIONS];
    int B, Hq, D;
    int W;             // merge chunk width (set by the launcher)
    bool out_f16;
    void* out;
    float* lse_out;
};

struct CombineArgs {
    const float* part_o;
    const float* part_lse;
    const int32_t* seq_lens;
    int B, Hq, D, split_tokens, max_splits;
    int live_splits;   // as in CombineRegionsArgs
    bool out_f16;
    void* out;
    float* lse_out;
};

// Every host-side check of kvq_decode_step (no HIP call); KVQ_OK or the
// status the call returns.
int validate_step(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache, const void* k_new,
                  const void* v_new, const void* q, const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                  float softmax_scale, int max_seq_len, int split_tokens, int max_splits, const float* part_o,
                  const float* part_lse, int out_type, const void* out, const float* lse_out);

hipError_t launch_quantize_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode_valu(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s);
bool decode_mfma_supports(const DecodeArgs& a);
// whether the matrix-core kernel writes the new rows of a decode step itself
// (every type it is built for)
inline bool decode_mfma_writes_new_rows(const DecodeArgs&) { return true; }
// the tail (quantised K and V) and the fp16 window of a mixed cache in one launch
hipError_t launch_decode_mfma_dual(const DecodeArgs& tail, const DecodeArgs& window, hipStream_t s);
bool decode_mfma_dual_supports(const DecodeArgs& tail, const DecodeArgs& window);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_combine_regions(const CombineRegionsArgs& a, hipStream_t s);

}  // namespace kvq
