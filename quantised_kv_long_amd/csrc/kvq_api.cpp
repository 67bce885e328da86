// kvq_api.cpp -- the C ABI (include/kvq.h): argument validation on the host,
// then one launch per kernel on the caller's stream.  No HIP call is made
// before every scalar argument has been checked, so every error status can be
// produced without a GPU.
#include "kvq.h"

#include <math.h>

#include "kvq_internal.hpp"

namespace {

bool known_type(int t) { return kvq::valid_type(t); }

bool valid_head_dim(int D) { return D >= 32 && D <= KVQ_MAX_HEAD_DIM && D % 32 == 0; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Checks one plane descriptor; rows [0, rows_needed) of every (b < B, g < Hkv)
// must be addressable.
int check_plane(const kvq_plane_desc* p, int B, int Hkv, int64_t rows_needed)
{
    if (!p) return KVQ_ERR_NULL;
    if (!known_type(p->type)) return KVQ_ERR_TYPE;
    if (!p->data) return KVQ_ERR_NULL;
    if (p->type != KVQ_F16 && !p->scales) return KVQ_ERR_NULL;
    if (!aligned(p->data, 16) || (p->scales && !aligned(p->scales, 4))) return KVQ_ERR_ALIGN;
    if (p->capacity < 0 || p->seq_stride_rows < 0 || p->head_stride_rows < 0) return KVQ_ERR_SHAPE;
    if (B > 1 && p->seq_stride_rows == 0) return KVQ_ERR_SHAPE;
    if (Hkv > 1 && p->head_stride_rows == 0) return KVQ_ERR_SHAPE;
    if (rows_needed > p->capacity) return KVQ_ERR_CAPACITY;
    return KVQ_OK;
}

kvq::Plane to_plane(const kvq_plane_desc* p)
{
    return kvq::Plane{static_cast<uint8_t*>(p->data), static_cast<uint16_t*>(p->scales),
                      p->seq_stride_rows, p->head_stride_rows};
}

int finish(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH; }

int validate_decode(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache, const void* q,
                    const int32_t* seq_lens, int B, int Hq, int Hkv, int D, float softmax_scale,
                    int max_seq_len, int split_tokens, int max_splits, const float* part_o,
                    const float* part_lse)
{
    if (!q || !seq_lens || !part_o || !part_lse) return KVQ_ERR_NULL;
    if (B < 1 || Hkv < 1 || Hq < 1 || Hq % Hkv != 0 || Hq / Hkv > KVQ_MAX_GROUP) return KVQ_ERR_SHAPE;
    if (!valid_head_dim(D)) return KVQ_ERR_SHAPE;
    if (!isfinite(softmax_scale)) return KVQ_ERR_SHAPE;
    if (max_seq_len < 1) return KVQ_ERR_SHAPE;
    int rc = check_plane(k_cache, B, Hkv, max_seq_len);
    if (rc != KVQ_OK) return rc;
    rc = check_plane(v_cache, B, Hkv, max_seq_len);
    if (rc != KVQ_OK) return rc;
    if (!aligned(q, 16) || !aligned(part_o, 16) || !aligned(part_lse, 4) || !aligned(seq_lens, 4))
        return KVQ_ERR_ALIGN;
    if (split_tokens < KVQ_SPLIT_GRANULE || split_tokens % KVQ_SPLIT_GRANULE != 0) return KVQ_ERR_SPLITS;
    if (max_splits < 1 || max_splits > 65535) return KVQ_ERR_SPLITS;
    if ((int64_t)max_splits * split_tokens < max_seq_len) return KVQ_ERR_SPLITS;
    if ((int64_t)B * Hkv > 65535LL * 65535LL) return KVQ_ERR_SHAPE;
    return KVQ_OK;
}

kvq::DecodeArgs decode_args(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                            const void* q, const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                            float softmax_scale, int max_seq_len, int split_tokens, int max_splits,
                            float* part_o, float* part_lse)
{
    kvq::DecodeArgs a;
    a.k = to_plane(k_cache);
    a.v = to_plane(v_cache);
    a.tk = k_cache->type;
    a.tv = v_cache->type;
    a.q = static_cast<const uint16_t*>(q);
    a.seq_lens = seq_lens;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.G = Hq / Hkv;
    a.nq = 1;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.max_seq_len = max_seq_len;
    a.split_tokens = split_tokens;
    a.max_splits = max_splits;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.k_new = nullptr;
    a.v_new = nullptr;
    return a;
}

}  // namespace

namespace kvq {

int validate_step(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache, const void* k_new,
                  const void* v_new, const void* q, const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                  float softmax_scale, int max_seq_len, int split_tokens, int max_splits, const float* part_o,
                  const float* part_lse, int out_type, const void* out, const float* lse_out)
{
    const int rc = validate_decode(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale, max_seq_len,
                                   split_tokens, max_splits, part_o, part_lse);
    if (rc != KVQ_OK) return rc;
    if (!k_new || !v_new || !out) return KVQ_ERR_NULL;
    if (out_type != KVQ_F16 && out_type != KVQ_OUT_F32) return KVQ_ERR_TYPE;
    if (B > 65535 || Hq > 65535) return KVQ_ERR_SHAPE;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
        return KVQ_ERR_ALIGN;
    return KVQ_OK;
}

}  // namespace kvq

extern "C" {

size_t kvq_data_row_bytes(int type, int head_dim)
{
    if (!known_type(type) || head_dim <= 0 || head_dim % 32 != 0) return 0;
    return (size_t)kvq::data_row_bytes(type, head_dim);
}

size_t kvq_scale_row_bytes(int type, int head_dim)
{
    if (!known_type(type) || head_dim <= 0 || head_dim % 32 != 0) return 0;
    return (size_t)(2 * kvq::scales_per_block(type) * (head_dim / 32));
}

int64_t kvq_tier_cache_bytes(int tier, int64_t n_ctx, int n_layers, int Hkv, int D)
{
    if (n_ctx <= 0 || n_layers <= 0 || Hkv <= 0 || D <= 0 || D % 32 != 0) return -1;
    // bytes of 32 values: f16 64, q8_0 34, q4_0 18, q5_1 24
    int kb, vb;
    switch (tier) {
    case KVQ_TIER_F16: kb = 64; vb = 64; break;
    case KVQ_TIER_Q8_Q8: kb = 34; vb = 34; break;
    case KVQ_TIER_Q8_Q4: kb = 34; vb = 18; break;
    case KVQ_TIER_Q51_Q4: kb = 24; vb = 18; break;
    default: return -1;
    }
    return n_ctx * (int64_t)n_layers * Hkv * (D / 32) * (int64_t)(kb + vb);
}

int kvq_select_kv_tier(int64_t n_ctx, int n_layers, int Hkv, int D, int64_t free_bytes,
                       int64_t resident_bytes, int64_t vram_target_bytes, int64_t* budget_bytes,
                       int64_t* cache_bytes)
{
    if (n_ctx <= 0 || n_layers <= 0 || Hkv <= 0 || D <= 0 || D % 32 != 0) return KVQ_ERR_SHAPE;
    if (free_bytes < 0 || resident_bytes < 0 || vram_target_bytes < 0) return KVQ_ERR_SHAPE;
    const int64_t reserve = 3LL << 29;  // 1.5 GiB for compute
    const int64_t cap = vram_target_bytes > 0 && vram_target_bytes < free_bytes ? vram_target_bytes
                                                                                : free_bytes;
    const int64_t budget = cap - resident_bytes - reserve;
    int tier = KVQ_TIER_Q51_Q4;
    for (int t = KVQ_TIER_F16; t <= KVQ_TIER_Q51_Q4; ++t) {
        if (kvq_tier_cache_bytes(t, n_ctx, n_layers, Hkv, D) <= budget) {
            tier = t;
            break;
        }
    }
    if (budget_bytes) *budget_bytes = budget;
    if (cache_bytes) *cache_bytes = kvq_tier_cache_bytes(tier, n_ctx, n_layers, Hkv, D);
    return tier;
}

int kvq_tier_types(int tier, int* type_k, int* type_v)
{
    int tk, tv;
    switch (tier) {
    case KVQ_TIER_F16: tk = KVQ_F16; tv = KVQ_F16; break;
    case KVQ_TIER_Q8_Q8: tk = KVQ_Q8_0; tv = KVQ_Q8_0; break;
    case KVQ_TIER_Q8_Q4: tk = KVQ_Q8_0; tv = KVQ_Q4_0; break;
    case KVQ_TIER_Q51_Q4: tk = KVQ_Q5_1; tv = KVQ_Q4_0; break;
    default: return KVQ_ERR_TYPE;
    }
    if (type_k) *type_k = tk;
    if (type_v) *type_v = tv;
    return KVQ_OK;
}

const char* kvq_status_string(int status)
{
    switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "a required pointer is NULL";
    case KVQ_ERR_SHAPE: return "a size is out of range or inconsistent";
    case KVQ_ERR_TYPE: return "unknown storage, output type or variant";
    case KVQ_ERR_ALIGN: return "a plane or array is not aligned as required";
    case KVQ_ERR_CAPACITY: return "rows requested beyond a cache's capacity";
    case KVQ_ERR_SPLITS: return "split arithmetic does not fit";
    case KVQ_ERR_LAUNCH: return "the HIP runtime reported an error at launch";
    default: return "unknown status";
    }
}

int kvq_quantize_append(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                        const void* k_new, const void* v_new, const int32_t* positions, int B,
                        int n_new, int Hkv, int D, int max_end, void* stream)
{
    if (B < 0 || n_new < 0 || Hkv < 1 || !valid_head_dim(D)) return KVQ_ERR_SHAPE;
    if (B == 0 || n_new == 0) return KVQ_OK;  // nothing to write (pointers may be NULL)
    if (!k_new || !v_new || !positions) return KVQ_ERR_NULL;
    if (max_end < n_new) return KVQ_ERR_SHAPE;
    int rc = check_plane(k_cache, B, Hkv, max_end);
    if (rc != KVQ_OK) return rc;
    rc = check_plane(v_cache, B, Hkv, max_end);
    if (rc != KVQ_OK) return rc;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(positions, 4)) return KVQ_ERR_ALIGN;
    const int64_t n_blocks = (int64_t)B * n_new * Hkv * (D / 32);
    if ((n_blocks + 255) / 256 > 0x7fffffffLL) return KVQ_ERR_SHAPE;

    kvq::AppendArgs a;
    a.k = to_plane(k_cache);
    a.v = to_plane(v_cache);
    a.tk = k_cache->type;
    a.tv = v_cache->type;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    // [B][n_new][Hkv][D]
    a.k_sb = a.v_sb = (int64_t)n_new * Hkv * D;
    a.k_sr = a.v_sr = (int64_t)Hkv * D;
    a.k_sg = a.v_sg = D;
    a.counts = nullptr;
    a.positions = positions;
    a.seq_lens = nullptr;
    a.B = B;
    a.n_new = n_new;
    a.Hkv = Hkv;
    a.D = D;
    (void)hipGetLastError();
    return finish(kvq::launch_quantize_append(a, static_cast<hipStream_t>(stream)));
}

int kvq_quantize_rows(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                      const kvq_plane_desc* k_src, const kvq_plane_desc* v_src, const int32_t* counts,
                      const int32_t* positions, int B, int max_rows, int Hkv, int D, int max_end,
                      void* stream)
{
    if (B < 0 || max_rows < 0 || Hkv < 1 || !valid_head_dim(D)) return KVQ_ERR_SHAPE;
    if (B == 0 || max_rows == 0) return KVQ_OK;  // nothing to write (pointers may be NULL)
    if (!counts || !positions) return KVQ_ERR_NULL;
    if (max_end < 0) return KVQ_ERR_SHAPE;
    int rc = check_plane(k_src, B, Hkv, max_rows);
    if (rc != KVQ_OK) return rc;
    rc = check_plane(v_src, B, Hkv, max_rows);
    if (rc != KVQ_OK) return rc;
    if (k_src->type != KVQ_F16 || v_src->type != KVQ_F16) return KVQ_ERR_TYPE;
    rc = check_plane(k_cache, B, Hkv, max_end);
    if (rc != KVQ_OK) return rc;
    rc = check_plane(v_cache, B, Hkv, max_end);
    if (rc != KVQ_OK) return rc;
    if (!aligned(counts, 4) || !aligned(positions, 4)) return KVQ_ERR_ALIGN;
    const int64_t n_blocks = (int64_t)B * max_rows * Hkv * (D / 32);
    if ((n_blocks + 255) / 256 > 0x7fffffffLL) return KVQ_ERR_SHAPE;

    kvq::AppendArgs a;
    a.k = to_plane(k_cache);
    a.v = to_plane(v_cache);
    a.tk = k_cache->type;
    a.tv = v_cache->type;
    a.k_new = static_cast<const uint16_t*>(k_src->data);
    a.v_new = static_cast<const uint16_t*>(v_src->data);
    // rows of fp16 planes: D values per row
    a.k_sb = k_src->seq_stride_rows * D;
    a.k_sr = D;
    a.k_sg = k_src->head_stride_rows * D;
    a.v_sb = v_src->seq_stride_rows * D;
    a.v_sr = D;
    a.v_sg = v_src->head_stride_rows * D;
    a.counts = counts;
    a.positions = positions;
    a.seq_lens = nullptr;
    a.B = B;
    a.n_new = max_rows;
    a.Hkv = Hkv;
    a.D = D;
    (void)hipGetLastError();
    return finish(kvq::launch_quantize_append(a, static_cast<hipStream_t>(stream)));
}

int kvq_decode_attn_variant(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                            const void* q, const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                            float softmax_scale, int max_seq_len, int split_tokens, int max_splits,
                            float* part_o, float* part_lse, int variant, void* stream)
{
    if (variant != KVQ_VARIANT_AUTO && variant != KVQ_VARIANT_VALU && variant != KVQ_VARIANT_MFMA)
        return KVQ_ERR_TYPE;
    const int rc = validate_decode(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale,
                                   max_seq_len, split_tokens, max_splits, part_o, part_lse);
    if (rc != KVQ_OK) return rc;
    const kvq::DecodeArgs a = decode_args(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale,
                                          max_seq_len, split_tokens, max_splits, part_o, part_lse);
    const bool mfma_ok = kvq::decode_mfma_supports(a);
    if (variant == KVQ_VARIANT_MFMA && !mfma_ok) return KVQ_ERR_SHAPE;
    const bool use_mfma = variant == KVQ_VARIANT_MFMA || (variant == KVQ_VARIANT_AUTO && mfma_ok);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return finish(use_mfma ? kvq::launch_decode_mfma(a, s) : kvq::launch_decode_valu(a, s));
}

int kvq_decode_attn(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache, const void* q,
                    const int32_t* seq_lens, int B, int Hq, int Hkv, int D, float softmax_scale,
                    int max_seq_len, int split_tokens, int max_splits, float* part_o,
                    float* part_lse, void* stream)
{
    return kvq_decode_attn_variant(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale,
                                   max_seq_len, split_tokens, max_splits, part_o, part_lse,
                                   KVQ_VARIANT_AUTO, stream);
}

int kvq_decode_attn_multi(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                          const void* q, const int32_t* seq_lens, int B, int n_q, int Hq, int Hkv,
                          int D, float softmax_scale, int max_seq_len, int split_tokens,
                          int max_splits, float* part_o, float* part_lse, void* stream)
{
    int rc = validate_decode(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale, max_seq_len,
                             split_tokens, max_splits, part_o, part_lse);
    if (rc != KVQ_OK) return rc;
    if (n_q < 1 || (int64_t)n_q * (Hq / Hkv) > 16 || max_seq_len < n_q) return KVQ_ERR_SHAPE;
    if ((int64_t)B * n_q * Hq > 65535LL * 65535LL) return KVQ_ERR_SHAPE;
    kvq::DecodeArgs a = decode_args(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale,
                                    max_seq_len, split_tokens, max_splits, part_o, part_lse);
    a.nq = n_q;
    if (!kvq::decode_mfma_supports(a)) return KVQ_ERR_SHAPE;
    (void)hipGetLastError();
    return finish(kvq::launch_decode_mfma(a, static_cast<hipStream_t>(stream)));
}

int kvq_decode_step_multi(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache, const void* k_new,
                          const void* v_new, const void* q, const int32_t* seq_lens, int B, int n_q, int Hq,
                          int Hkv, int D, float softmax_scale, int max_seq_len, int split_tokens,
                          int max_splits, float* part_o, float* part_lse, int out_type, void* out,
                          float* lse_out, void* stream)
{
    int rc = validate_decode(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale, max_seq_len,
                             split_tokens, max_splits, part_o, part_lse);
    if (rc != KVQ_OK) return rc;
    if (n_q < 1 || (int64_t)n_q * (Hq / Hkv) > 16 || max_seq_len < n_q) return KVQ_ERR_SHAPE;
    if ((int64_t)n_q * Hq > 65535 || B > 65535) return KVQ_ERR_SHAPE;
    if (!k_new || !v_new || !out) return KVQ_ERR_NULL;
    if (out_type != KVQ_F16 && out_type != KVQ_OUT_F32) return KVQ_ERR_TYPE;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16) ||
        (lse_out && !aligned(lse_out, 4)))
        return KVQ_ERR_ALIGN;
    kvq::DecodeArgs a = decode_args(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale,
                                    max_seq_len, split_tokens, max_splits, part_o, part_lse);
    a.nq = n_q;
    if (!kvq::decode_mfma_supports(a)) return KVQ_ERR_SHAPE;
    // the attention kernel writes the n_q new rows itself
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (kvq::launch_decode_mfma(a, s) != hipSuccess) return KVQ_ERR_LAUNCH;
    kvq::CombineArgs c;
    c.part_o = part_o;
    c.part_lse = part_lse;
    c.seq_lens = seq_lens;
    c.B = B;
    c.Hq = n_q * Hq;
    c.D = D;
    c.split_tokens = split_tokens;
    c.max_splits = max_splits;
    c.live_splits = kvq::grid_splits(a);
    c.out_f16 = out_type == KVQ_F16;
    c.out = out;
    c.lse_out = lse_out;
    return finish(kvq::launch_combine(c, s));
}

int kvq_combine(const float* part_o, const float* part_lse, const int32_t* seq_lens, int B, int Hq,
                int D, int split_tokens, int max_splits, int out_type, void* out, float* lse_out,
                void* stream)
{
    if (!part_o || !part_lse || !seq_lens || !out) return KVQ_ERR_NULL;
    if (out_type != KVQ_F16 && out_type != KVQ_OUT_F32) return KVQ_ERR_TYPE;
    if (B < 1 || Hq < 1 || !valid_head_dim(D)) return KVQ_ERR_SHAPE;
    if (B > 65535 || Hq > 65535) return KVQ_ERR_SHAPE;
    if (split_tokens < KVQ_SPLIT_GRANULE || split_tokens % KVQ_SPLIT_GRANULE != 0) return KVQ_ERR_SPLITS;
    if (max_splits < 1 || max_splits > 65535) return KVQ_ERR_SPLITS;
    if (!aligned(part_o, 16) || !aligned(part_lse, 4) || !aligned(seq_lens, 4) ||
        !aligned(out, 16) || (lse_out && !aligned(lse_out, 4)))
        return KVQ_ERR_ALIGN;
    kvq::CombineArgs a;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.seq_lens = seq_lens;
    a.B = B;
    a.Hq = Hq;
    a.D = D;
    a.split_tokens = split_tokens;
    a.max_splits = max_splits;
    a.live_splits = max_splits;
    a.out_f16 = out_type == KVQ_F16;
    a.out = out;
    a.lse_out = lse_out;
    (void)hipGetLastError();
    return finish(kvq::launch_combine(a, static_cast<hipStream_t>(stream)));
}

int kvq_decode_attn_mixed(const kvq_plane_desc* k_tail, const kvq_plane_desc* v_tail,
                          const kvq_plane_desc* k_win, const kvq_plane_desc* v_win, const void* q,
                          const int32_t* tail_lens, const int32_t* win_lens, int B, int Hq, int Hkv,
                          int D, float softmax_scale, int tail_max_len, int tail_split_tokens,
                          int tail_max_splits, float* tail_part_o, float* tail_part_lse,
                          int win_max_len, int win_split_tokens, int win_max_splits,
                          float* win_part_o, float* win_part_lse, void* stream)
{
    int rc = validate_decode(k_tail, v_tail, q, tail_lens, B, Hq, Hkv, D, softmax_scale, tail_max_len,
                             tail_split_tokens, tail_max_splits, tail_part_o, tail_part_lse);
    if (rc != KVQ_OK) return rc;
    rc = validate_decode(k_win, v_win, q, win_lens, B, Hq, Hkv, D, softmax_scale, win_max_len,
                         win_split_tokens, win_max_splits, win_part_o, win_part_lse);
    if (rc != KVQ_OK) return rc;
    if (k_win->type != KVQ_F16 || v_win->type != KVQ_F16) return KVQ_ERR_TYPE;
    const kvq::DecodeArgs t = decode_args(k_tail, v_tail, q, tail_lens, B, Hq, Hkv, D, softmax_scale,
                                          tail_max_len, tail_split_tokens, tail_max_splits, tail_part_o,
                                          tail_part_lse);
    const kvq::DecodeArgs w = decode_args(k_win, v_win, q, win_lens, B, Hq, Hkv, D, softmax_scale,
                                          win_max_len, win_split_tokens, win_max_splits, win_part_o,
                                          win_part_lse);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (kvq::decode_mfma_dual_supports(t, w)) return finish(kvq::launch_decode_mfma_dual(t, w, s));
    // otherwise one launch per region, each with the kernel its shape takes
    hipError_t e = kvq::decode_mfma_supports(t) ? kvq::launch_decode_mfma(t, s) : kvq::launch_decode_valu(t, s);
    if (e == hipSuccess)
        e = kvq::decode_mfma_supports(w) ? kvq::launch_decode_mfma(w, s) : kvq::launch_decode_valu(w, s);
    return finish(e);
}

int kvq_decode_step_mixed(const kvq_plane_desc* k_tail, const kvq_plane_desc* v_tail,
                          const kvq_plane_desc* k_win, const kvq_plane_desc* v_win, const void* k_new,
                          const void* v_new, const void* q, const int32_t* tail_lens,
                          const int32_t* win_lens, int B, int Hq, int Hkv, int D, float softmax_scale,
                          int tail_max_len, int tail_split_tokens, int tail_max_splits,
                          float* tail_part_o, float* tail_part_lse, int win_max_len,
                          int win_split_tokens, int win_max_splits, float* win_part_o,
                          float* win_part_lse, int out_type, void* out, float* lse_out, void* stream)
{
    int rc = validate_decode(k_tail, v_tail, q, tail_lens, B, Hq, Hkv, D, softmax_scale, tail_max_len,
                             tail_split_tokens, tail_max_splits, tail_part_o, tail_part_lse);
    if (rc != KVQ_OK) return rc;
    rc = validate_decode(k_win, v_win, q, win_lens, B, Hq, Hkv, D, softmax_scale, win_max_len,
                         win_split_tokens, win_max_splits, win_part_o, win_part_lse);
    if (rc != KVQ_OK) return rc;
    if (k_win->type != KVQ_F16 || v_win->type != KVQ_F16) return KVQ_ERR_TYPE;
    if (!k_new || !v_new || !out) return KVQ_ERR_NULL;
    if (out_type != KVQ_F16 && out_type != KVQ_OUT_F32) return KVQ_ERR_TYPE;
    if (B > 65535 || Hq > 65535) return KVQ_ERR_SHAPE;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16) ||
        (lse_out && !aligned(lse_out, 4)))
        return KVQ_ERR_ALIGN;
    const kvq::DecodeArgs t = decode_args(k_tail, v_tail, q, tail_lens, B, Hq, Hkv, D, softmax_scale,
                                          tail_max_len, tail_split_tokens, tail_max_splits, tail_part_o,
                                          tail_part_lse);
    kvq::DecodeArgs w = decode_args(k_win, v_win, q, win_lens, B, Hq, Hkv, D, softmax_scale,
                                    win_max_len, win_split_tokens, win_max_splits, win_part_o,
                                    win_part_lse);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t e;
    const bool window_mfma = kvq::decode_mfma_supports(w);
    if (window_mfma) {
        // the window's attention workgroup that holds row win_lens[b] - 1
        // writes the new row before reading it
        w.k_new = static_cast<const uint16_t*>(k_new);
        w.v_new = static_cast<const uint16_t*>(v_new);
    }
    if (kvq::decode_mfma_dual_supports(t, w)) {
        e = kvq::launch_decode_mfma_dual(t, w, s);
    } else {
        e = kvq::decode_mfma_supports(t) ? kvq::launch_decode_mfma(t, s) : kvq::launch_decode_valu(t, s);
        if (e == hipSuccess && !window_mfma) {
            kvq::AppendArgs ap;
            ap.k = w.k;
            ap.v = w.v;
            ap.tk = w.tk;
            ap.tv = w.tv;
            ap.k_new = static_cast<const uint16_t*>(k_new);
            ap.v_new = static_cast<const uint16_t*>(v_new);
            ap.k_sb = ap.v_sb = (int64_t)Hkv * D;  // [B][Hkv][D], one row
            ap.k_sr = ap.v_sr = 0;
            ap.k_sg = ap.v_sg = D;
            ap.counts = nullptr;
            ap.positions = nullptr;  // row win_lens[b] - 1
            ap.seq_lens = win_lens;
            ap.B = B;
            ap.n_new = 1;
            ap.Hkv = Hkv;
            ap.D = D;
            e = kvq::launch_quantize_append(ap, s);
        }
        if (e == hipSuccess) e = window_mfma ? kvq::launch_decode_mfma(w, s) : kvq::launch_decode_valu(w, s);
    }
    if (e != hipSuccess) return KVQ_ERR_LAUNCH;

    kvq::CombineRegionsArgs c{};
    c.n = 2;
    const kvq::DecodeArgs* r[2] = {&t, &w};
    for (int i = 0; i < 2; ++i) {
        c.part_o[i] = r[i]->part_o;
        c.part_lse[i] = r[i]->part_lse;
        c.seq_lens[i] = r[i]->seq_lens;
        c.split_tokens[i] = r[i]->split_tokens;
        c.max_splits[i] = r[i]->max_splits;
        c.live_splits[i] = kvq::grid_splits(*r[i]);
    }
    c.B = B;
    c.Hq = Hq;
    c.D = D;
    c.out_f16 = out_type == KVQ_F16;
    c.out = out;
    c.lse_out = lse_out;
    return finish(kvq::launch_combine_regions(c, s));
}

int kvq_combine_regions(int n_regions, const float* const* part_o, const float* const* part_lse,
                        const int32_t* const* seq_lens, const int* split_tokens, const int* max_splits,
                        int B, int Hq, int D, int out_type, void* out, float* lse_out, void* stream)
{
    if (n_regions < 1 || n_regions > kvq::MAX_REGIONS) return KVQ_ERR_SHAPE;
    if (!part_o || !part_lse || !seq_lens || !split_tokens || !max_splits || !out) return KVQ_ERR_NULL;
    if (out_type != KVQ_F16 && out_type != KVQ_OUT_F32) return KVQ_ERR_TYPE;
    if (B < 1 || Hq < 1 || !valid_head_dim(D)) return KVQ_ERR_SHAPE;
    if (B > 65535 || Hq > 65535) return KVQ_ERR_SHAPE;
    if (!aligned(out, 16) || (lse_out && !aligned(lse_out, 4))) return KVQ_ERR_ALIGN;
    kvq::CombineRegionsArgs a{};
    a.n = n_regions;
    for (int i = 0; i < n_regions; ++i) {
        if (!part_o[i] || !part_lse[i] || !seq_lens[i]) return KVQ_ERR_NULL;
        if (split_tokens[i] < KVQ_SPLIT_GRANULE || split_tokens[i] % KVQ_SPLIT_GRANULE != 0)
            return KVQ_ERR_SPLITS;
        if (max_splits[i] < 1 || max_splits[i] > 65535) return KVQ_ERR_SPLITS;
        if (!aligned(part_o[i], 16) || !aligned(part_lse[i], 4) || !aligned(seq_lens[i], 4))
            return KVQ_ERR_ALIGN;
        a.part_o[i] = part_o[i];
        a.part_lse[i] = part_lse[i];
        a.seq_lens[i] = seq_lens[i];
        a.split_tokens[i] = split_tokens[i];
        a.max_splits[i] = max_splits[i];
        a.live_splits[i] = max_splits[i];
    }
    a.B = B;
    a.Hq = Hq;
    a.D = D;
    a.out_f16 = out_type == KVQ_F16;
    a.out = out;
    a.lse_out = lse_out;
    (void)hipGetLastError();
    return finish(kvq::launch_combine_regions(a, static_cast<hipStream_t>(stream)));
}

int kvq_decode_step(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache, const void* k_new,
                    const void* v_new, const void* q, const int32_t* seq_lens, int B, int Hq, int Hkv,
                    int D, float softmax_scale, int max_seq_len, int split_tokens, int max_splits,
                    float* part_o, float* part_lse, int out_type, void* out, float* lse_out,
                    void* stream)
{
    const int rc = kvq::validate_step(k_cache, v_cache, k_new, v_new, q, seq_lens, B, Hq, Hkv, D,
                                      softmax_scale, max_seq_len, split_tokens, max_splits, part_o,
                                      part_lse, out_type, out, lse_out);
    if (rc != KVQ_OK) return rc;

    kvq::DecodeArgs a = decode_args(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale,
                                    max_seq_len, split_tokens, max_splits, part_o, part_lse);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t e;
    const bool mfma = kvq::decode_mfma_supports(a);
    if (mfma && kvq::decode_mfma_writes_new_rows(a)) {
        // the attention kernel writes the new row itself
        a.k_new = static_cast<const uint16_t*>(k_new);
        a.v_new = static_cast<const uint16_t*>(v_new);
        e = kvq::launch_decode_mfma(a, s);
    } else {
        kvq::AppendArgs ap;
        ap.k = a.k;
        ap.v = a.v;
        ap.tk = a.tk;
        ap.tv = a.tv;
        ap.k_new = static_cast<const uint16_t*>(k_new);
        ap.v_new = static_cast<const uint16_t*>(v_new);
        // [B][Hkv][D], one row
        ap.k_sb = ap.v_sb = (int64_t)Hkv * D;
        ap.k_sr = ap.v_sr = 0;
        ap.k_sg = ap.v_sg = D;
        ap.counts = nullptr;
        ap.positions = nullptr;  // row seq_lens[b] - 1
        ap.seq_lens = seq_lens;
        ap.B = B;
        ap.n_new = 1;
        ap.Hkv = Hkv;
        ap.D = D;
        e = kvq::launch_quantize_append(ap, s);
        if (e == hipSuccess) e = mfma ? kvq::launch_decode_mfma(a, s) : kvq::launch_decode_valu(a, s);
    }
    if (e != hipSuccess) return KVQ_ERR_LAUNCH;

    kvq::CombineArgs c;
    c.part_o = part_o;
    c.part_lse = part_lse;
    c.seq_lens = seq_lens;
    c.B = B;
    c.Hq = Hq;
    c.D = D;
    c.split_tokens = split_tokens;
    c.max_splits = max_splits;
    c.live_splits = kvq::grid_splits(a);
    c.out_f16 = out_type == KVQ_F16;
    c.out = out;
    c.lse_out = lse_out;
    return finish(kvq::launch_combine(c, s));
}

}  // extern "C"
