// kvq_api.cpp -- the C ABI (include/kvq.h): argument validation on the host,
// then one launch per kernel on the caller's stream.  No HIP call is made
// before every scalar argument has been checked, so every error status can be
// produced without a GPU.
#include "kvq.h"

#include <math.h>

#include "kvq_internal.hpp"

namespace {

bool known_type(int t) { return t == KVQ_F16 || t == KVQ_Q8_0 || t == KVQ_Q4_0; }

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
    if (!aligned(p->data, 16) || (p->scales && !aligned(p->scales, 16))) return KVQ_ERR_ALIGN;
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

extern "C" {

size_t kvq_data_row_bytes(int type, int head_dim)
{
    if (!known_type(type) || head_dim <= 0 || head_dim % 32 != 0) return 0;
    return (size_t)kvq::data_row_bytes(type, head_dim);
}

size_t kvq_scale_row_bytes(int type, int head_dim)
{
    if (!known_type(type) || head_dim <= 0 || head_dim % 32 != 0) return 0;
    return type == KVQ_F16 ? 0 : (size_t)(head_dim / 16);
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
    a.positions = positions;
    a.seq_lens = nullptr;
    a.B = B;
    a.n_new = n_new;
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
    a.out_f16 = out_type == KVQ_F16;
    a.out = out;
    a.lse_out = lse_out;
    (void)hipGetLastError();
    return finish(kvq::launch_combine(a, static_cast<hipStream_t>(stream)));
}

int kvq_decode_step(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache, const void* k_new,
                    const void* v_new, const void* q, const int32_t* seq_lens, int B, int Hq, int Hkv,
                    int D, float softmax_scale, int max_seq_len, int split_tokens, int max_splits,
                    float* part_o, float* part_lse, int out_type, void* out, float* lse_out,
                    void* stream)
{
    const int rc = validate_decode(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale,
                                   max_seq_len, split_tokens, max_splits, part_o, part_lse);
    if (rc != KVQ_OK) return rc;
    if (!k_new || !v_new || !out) return KVQ_ERR_NULL;
    if (out_type != KVQ_F16 && out_type != KVQ_OUT_F32) return KVQ_ERR_TYPE;
    if (B > 65535 || Hq > 65535) return KVQ_ERR_SHAPE;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16) ||
        (lse_out && !aligned(lse_out, 4)))
        return KVQ_ERR_ALIGN;

    kvq::DecodeArgs a = decode_args(k_cache, v_cache, q, seq_lens, B, Hq, Hkv, D, softmax_scale,
                                    max_seq_len, split_tokens, max_splits, part_o, part_lse);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t e;
    if (kvq::decode_mfma_supports(a)) {
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
        ap.positions = nullptr;  // row seq_lens[b] - 1
        ap.seq_lens = seq_lens;
        ap.B = B;
        ap.n_new = 1;
        ap.Hkv = Hkv;
        ap.D = D;
        e = kvq::launch_quantize_append(ap, s);
        if (e == hipSuccess) e = kvq::launch_decode_valu(a, s);
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
    c.out_f16 = out_type == KVQ_F16;
    c.out = out;
    c.lse_out = lse_out;
    return finish(kvq::launch_combine(c, s));
}

}  // extern "C"
