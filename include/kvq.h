/*
 * kvq.h -- C ABI of the block-quantised KV-cache decode-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (HAL #582 "per-layer KV compression study"):
 *   - section 1 (size model table): each token's K and V row per KV head is
 *     stored either as f16 or as 32-value blocks with one fp16 scale:
 *     q8_0 = 32 int8 codes (34 bytes per block), q4_0 = 32 four-bit codes
 *     (18 bytes per block).  K and V types are chosen independently (section 2
 *     quality bar and section 5 P1: "-ctk/-ctv", asymmetric q8_0 K + q4_0 V).
 *   - section 5 P2 "write path": a new token is quantised once, when written.
 *   - section 3b and section 5 P0: decode attention reads the stored blocks and
 *     dequantises them in registers, so the bytes moved per token fall with
 *     the format (the bandwidth-bound reader the study asks for).
 *   - section 5 P2 "read path": attention over separate regions is merged
 *     with an exact online-softmax combine; here the regions are the splits of
 *     a split-KV (flash-decoding) launch.
 *
 * Conventions shared by every entry point:
 *   - The caller owns all memory.  Every pointer marked "device" is HIP device
 *     memory of the current device; the library allocates nothing and keeps
 *     no state between calls, so calls are thread-safe.  The one exception is
 *     kvq_decode_step_noalloc, whose partials live in a device array the
 *     library holds per GPU (see there: its calls on one GPU must not
 *     overlap).
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL means the
 *     legacy default stream) and return.  KVQ_OK means "enqueued".
 *   - Scalar arguments are validated on the host before any HIP call; an
 *     invalid call returns a negative status and enqueues nothing.  Contents
 *     of device arrays (positions, lengths) are preconditions and are not
 *     checked.
 *   - Layouts are row-major C arrays unless stated otherwise.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of one cache tensor (K or V). */
typedef enum {
    KVQ_F16 = 0,  /* IEEE binary16 values, 2*D bytes per row, no scale plane   */
    KVQ_Q8_0 = 1, /* per 32-value block: 32 int8 codes + one fp16 scale        */
    KVQ_Q4_0 = 2, /* per 32-value block: 32 codes in [0,15] (value = code - 8),
                     packed two per byte, + one fp16 scale                     */
    /* Further scalar types of the pages' served pairs (HAL #582 section 1 size
     * table and section 5; block sizes 20, 22, 24 and 26 bytes per 32 values).
     * A row's data plane holds the low 4 bits of every code (D/2 bytes, block
     * b at 16*b, byte j = code j | code j+16 << 4), then for q5 / q6 every
     * block's high bits (a little-endian 32-bit word per block, bit j = bit 4
     * of code j; or a 64-bit word, bits 2j and 2j+1 = bits 4 and 5).  Rows of
     * these types are 4-byte aligned.  The value 3 is not a storage type (it
     * names fp32 output, KVQ_OUT_F32). */
    KVQ_Q4_1 = 4, /* codes in [0,15], value = d * code + m; scales d, m        */
    KVQ_Q5_0 = 5, /* codes in [0,31], value = d * (code - 16); scale d         */
    KVQ_Q5_1 = 6, /* codes in [0,31], value = d * code + m; scales d, m        */
    KVQ_Q6_0 = 7  /* codes in [0,63], value = d * (code - 32); scale d         */
} kvq_type;

/* Status codes (negative = error, nothing was enqueued). */
enum {
    KVQ_OK = 0,
    KVQ_ERR_NULL = -1,     /* a required pointer is NULL                        */
    KVQ_ERR_SHAPE = -2,    /* a size is out of range or inconsistent            */
    KVQ_ERR_TYPE = -3,     /* unknown storage or output type                    */
    KVQ_ERR_ALIGN = -4,    /* a plane or array is not aligned as required       */
    KVQ_ERR_CAPACITY = -5, /* rows requested beyond a cache's capacity          */
    KVQ_ERR_SPLITS = -6,   /* split arithmetic does not fit                     */
    KVQ_ERR_LAUNCH = -7    /* the HIP runtime reported an error at launch       */
};

/* Granule of `split_tokens`: every split is a whole number of this many rows. */
#define KVQ_SPLIT_GRANULE 64

/* Largest head dimension and query-group size the kernels accept. */
#define KVQ_MAX_HEAD_DIM 512
#define KVQ_MAX_GROUP 16

/*
 * One cache tensor (K or V) of one layer, stored as two planes in device
 * memory (the same bytes as the 34-/18-byte blocks of the storage format,
 * split so that every data row starts on a 16-byte boundary):
 *   data plane : rows of kvq_data_row_bytes(type, D) bytes.
 *                f16: D binary16 values.  q8_0: D int8 codes, block b at
 *                bytes [32b, 32b+32).  q4_0: D/2 bytes, block b at bytes
 *                [16b, 16b+16); byte j of a block holds the code of element j
 *                in its low nibble and of element j+16 in its high nibble.
 *                q4_1: as q4_0.  q5_0, q5_1: the q4_0 bytes of the low
 *                nibbles, then D/8 bytes of high bits (block b's 32-bit word
 *                at D/2 + 4b).  q6_0: the low nibbles, then D/4 bytes (block
 *                b's 64-bit word at D/2 + 8b).
 *   scale plane: rows of D/32 binary16 scales (scale of block b at index b),
 *                or for q4_1 / q5_1 D/16 entries (block b: scale at 2b,
 *                minimum at 2b+1); unused (may be NULL) for f16.
 * Row t of KV head g of sequence b is row index
 *     b * seq_stride_rows + g * head_stride_rows + t
 * in both planes; rows t in [0, capacity) are addressable.  The usual layout
 * is head_stride_rows = capacity, seq_stride_rows = Hkv * capacity.
 * Alignment: the data plane must be 16-byte aligned, the scale plane 4-byte
 * aligned.
 */
typedef struct {
    int32_t type;             /* kvq_type                                   */
    int32_t capacity;         /* addressable rows per (sequence, KV head)   */
    void* data;               /* device: data plane                         */
    void* scales;             /* device: scale plane (NULL for f16)         */
    int64_t seq_stride_rows;  /* rows between sequences                     */
    int64_t head_stride_rows; /* rows between KV heads of one sequence      */
} kvq_plane_desc;

/* Bytes of one data-plane row: 2*D (f16), D (q8_0), D/2 (q4_0, q4_1),
 * 5*D/8 (q5_0, q5_1), 3*D/4 (q6_0); 0 for an unknown type or a D that is not
 * a positive multiple of 32. */
size_t kvq_data_row_bytes(int type, int head_dim);

/* Bytes of one scale-plane row: 0 (f16), D/16 (q8_0, q4_0, q5_0, q6_0), D/8
 * (q4_1, q5_1); 0 when invalid. */
size_t kvq_scale_row_bytes(int type, int head_dim);

/*
 * KV tier ladder (HAL #582 section 5 P1, the automatic KV tier at start-up:
 * pick the least compression whose whole cache stays resident).
 *
 * Tiers, from least to most compressing (K type / V type):
 *   KVQ_TIER_F16     f16 / f16
 *   KVQ_TIER_Q8_Q8   q8_0 / q8_0
 *   KVQ_TIER_Q8_Q4   q8_0 / q4_0
 *   KVQ_TIER_Q51_Q4  q5_1 / q4_0   (the last resort; q5_1 blocks are 24 bytes
 *                    per 32 values)
 */
enum { KVQ_TIER_F16 = 0, KVQ_TIER_Q8_Q8 = 1, KVQ_TIER_Q8_Q4 = 2, KVQ_TIER_Q51_Q4 = 3 };

/*
 * Bytes of a whole cache of the tier: n_layers * Hkv * n_ctx rows of K and of
 * V (f16: 2*D bytes a row; q8_0: 34*D/32; q4_0: 18*D/32; q5_1: 24*D/32).
 * -1 for an unknown tier or non-positive sizes, or D % 32 != 0.
 */
int64_t kvq_tier_cache_bytes(int tier, int64_t n_ctx, int n_layers, int Hkv, int D);

/*
 * The tier chosen for a context of n_ctx tokens: the first of the ladder
 * (least compressing) whose whole cache fits the budget
 *   budget = min(free_bytes, vram_target_bytes if > 0) - resident_bytes - 1.5 GiB
 * (the compute reserve), or KVQ_TIER_Q51_Q4 when none fits.  Writes the budget
 * and the chosen tier's cache bytes if the pointers are not NULL.  Returns the
 * tier, or KVQ_ERR_SHAPE for non-positive sizes, negative byte counts or
 * D % 32 != 0.  Host-only; no HIP call.
 */
int kvq_select_kv_tier(int64_t n_ctx, int n_layers, int Hkv, int D, int64_t free_bytes,
                       int64_t resident_bytes, int64_t vram_target_bytes, int64_t* budget_bytes,
                       int64_t* cache_bytes);

/* K and V storage types of a tier; KVQ_ERR_TYPE for an unknown tier (types
 * not written). */
int kvq_tier_types(int tier, int* type_k, int* type_v);

/* Static, human-readable name of a status code. */
const char* kvq_status_string(int status);

/*
 * Quantise-on-write (HAL #582 section 5 P2 write path: tokens are quantised
 * once when written; section 1 gives the block formats).
 *
 * For every sequence b < B, new row r < n_new and KV head g < Hkv, converts
 * the f16 row k_new[b][r][g][0..D) into k_cache's type and stores it at row
 * positions[b] + r of KV head g of sequence b; likewise v_new into v_cache.
 * Block quantiser (the pages do not print one; this is the library's fixed
 * definition, bit-exact):
 *   q8_0: d = fp16_rne(max_i |x_i| / 127) (binary32 division);
 *         code_i = round_half_away_from_zero(x_i / d) clamped to [-127, 127]
 *         (binary32 division by the stored d); all codes 0 when d == 0.
 *   q4_0: s = the x_i of largest magnitude (lowest i on ties, +0 if none);
 *         d = fp16_rne(s / -8); code_i = clamp(round_half_away(x_i / d),
 *         -8, 7) + 8; all codes 8 when d == 0.
 *   q5_0, q6_0: as q4_0 with -16 / -32 in place of -8: code_i =
 *         clamp(round_half_away(x_i / d), -16, 15) + 16 or (-32, 31) + 32.
 *   q4_1, q5_1: m = fp16(min_i x_i) (exact), d = fp16_rne((max_i x_i -
 *         min_i x_i) / 15 or 31) (binary32 subtraction and division);
 *         code_i = clamp(round_half_away((x_i - m) / d), 0, 15 or 31) with
 *         the stored m and d; all codes 0 when d == 0.
 *   f16 : the bits are copied unchanged.
 * Inputs of the quantised types must be finite: a block holding an infinity
 * or a NaN gets unspecified codes (the method defines none).
 *
 *   k_cache, v_cache : plane descriptors (host memory, read during the call).
 *   k_new, v_new     : device, [B][n_new][Hkv][D] binary16.
 *   positions        : device, [B] int32, first row written per sequence.
 *   max_end          : host, max over b of positions[b] + n_new; must not
 *                      exceed either cache's capacity (KVQ_ERR_CAPACITY).
 *   Requirements: B >= 0, n_new >= 0, Hkv >= 1, D % 32 == 0, 32 <= D <= 512.
 *   B == 0 or n_new == 0 (with valid Hkv and D) enqueues nothing and returns
 *   KVQ_OK without looking at any pointer.
 */
int kvq_quantize_append(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                        const void* k_new, const void* v_new, const int32_t* positions,
                        int B, int n_new, int Hkv, int D, int max_end, void* stream);

/*
 * Quantise rows of fp16 cache planes into a cache (HAL #582 section 5 P2, the
 * position-axis mixed cache: recent tokens stay fp16 in a rolling window and
 * are quantised once, in batches, when they leave it for the compressed
 * tail).  For every sequence b < B, row r < counts[b] and KV head g < Hkv,
 * converts row r of KV head g of sequence b of the fp16 planes k_src / v_src
 * with the block quantiser of kvq_quantize_append and stores it at row
 * positions[b] + r of k_cache / v_cache.
 *
 *   k_src, v_src : plane descriptors of type KVQ_F16 (host memory, read
 *                  during the call); rows [0, max_rows) must be addressable.
 *   counts       : device, [B] int32, 0 <= counts[b] <= max_rows.
 *   positions    : device, [B] int32, first row written per sequence.
 *   max_end      : host, max over b of positions[b] + counts[b]; must not
 *                  exceed either cache's capacity (KVQ_ERR_CAPACITY).
 *   Sources and destinations must not overlap.  B == 0 or max_rows == 0
 *   (with valid Hkv and D) enqueues nothing and returns KVQ_OK.
 *   KVQ_ERR_TYPE if a source plane is not fp16.
 */
int kvq_quantize_rows(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                      const kvq_plane_desc* k_src, const kvq_plane_desc* v_src,
                      const int32_t* counts, const int32_t* positions, int B, int max_rows,
                      int Hkv, int D, int max_end, void* stream);

/*
 * Split-KV decode attention (HAL #582 section 3b finding 2 and section 5 P0:
 * a reader that streams the stored blocks and dequantises them in registers;
 * section 5 P2: regions merged exactly by log-sum-exp).
 *
 * One query row per query head.  Query head h reads KV head h / (Hq / Hkv).
 * Sequence b attends over its rows [0, seq_lens[b]) with no mask.  The rows
 * are cut into splits of split_tokens rows; split s of sequence b covers rows
 * [s*split_tokens, min((s+1)*split_tokens, L_b)).  For every (b, h, s) with
 * s < S_b = ceil(L_b / split_tokens) (the splits that hold a row) the call
 * writes, in fp32,
 *   part_lse[b][h][s]   = ln sum_t exp(score_t)
 *   part_o[b][h][s][:]  = sum_t exp(score_t - part_lse) * v_t
 * with score_t = softmax_scale * sum_d q[b][h][d] * k_t[d] and k_t, v_t the
 * dequantised rows (code * scale, exactly).  Splits from S_b up to
 * max_splits hold no row and are left as they are: kvq_combine reads only
 * the first S_b splits of sequence b (a caller merging partials itself knows
 * S_b from L_b), and the launch spends no workgroups on splits from
 * ceil(max_seq_len / split_tokens) on.
 *
 *   q              : device, [B][Hq][D] binary16.
 *   seq_lens       : device, [B] int32, 0 <= L_b <= max_seq_len <= capacity
 *                    (L_b = 0: no split of b holds a row; nothing is written
 *                    for b).
 *   max_seq_len    : host, an upper bound of every L_b.
 *   split_tokens   : host, a positive multiple of KVQ_SPLIT_GRANULE.
 *   max_splits     : host, >= ceil(max_seq_len / split_tokens).
 *   part_o         : device, [B][Hq][max_splits][D] fp32, 16-byte aligned.
 *   part_lse       : device, [B][Hq][max_splits] fp32.
 *   Requirements: B >= 1, Hkv >= 1, Hq % Hkv == 0, Hq / Hkv <= 16,
 *   D % 32 == 0, 32 <= D <= 512, K and V caches with the same strides' meaning.
 *
 * Choosing split_tokens: the result changes only by rounding; the time
 * depends on it.  Measured on an MI355X (256 CUs): for one long sequence the
 * fastest splits give one or two workgroups per CU, Hkv * ceil(max_seq_len /
 * split_tokens) = 256 or 512 at head_dim 128 (8 KV heads: 1024 or 2048 rows
 * at 65536, within 1 %; 4096 or 8192 at 262144, 8192 up to 3 % faster), and
 * 256 at head_dim 256 (2 KV heads: 256 rows at 32768); counts in between
 * leave some CUs with one workgroup and others with two (13 % slower at
 * 65536).  Short contexts take at least 128 rows per split at head_dim 128
 * (128 at 4096).  A batch of ragged sequences of 16k-128k rows was
 * fastest with 2048 rows at head_dim 128 and 1024 at head_dim 512.  Fewer
 * rows per split mean more partials for the merge to read.
 */
int kvq_decode_attn(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                    const void* q, const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                    float softmax_scale, int max_seq_len, int split_tokens, int max_splits,
                    float* part_o, float* part_lse, void* stream);

/*
 * Decode attention for n_q query tokens per sequence at once (the
 * speculative-decoding verify step: n_q draft tokens checked in one pass; the
 * pages gate their quantised decode route on n_q <= 16).  The last n_q rows of
 * each sequence are the query tokens' own K/V rows (appended before the
 * call), and token i (0-based) attends causally over rows
 * [0, L_b - n_q + 1 + i).  Query token i, head h reads KV head h / (Hq / Hkv);
 * every (token, head) is one column of the matrix-core tile, so
 * n_q * (Hq / Hkv) <= 16 and the K/V stream is read once for all of them.
 *
 *   q        : device, [B][n_q][Hq][D] binary16.
 *   seq_lens : device, [B] int32, n_q <= L_b <= max_seq_len <= capacity.
 *   part_o   : device, [B][n_q * Hq][max_splits][D] fp32 (row i*Hq + h for
 *              token i, head h); part_lse [B][n_q * Hq][max_splits].  A
 *              split with no row a token sees is written empty for it.
 *   The partials merge with kvq_combine called with n_q * Hq heads, giving
 *   out [B][n_q][Hq][D].  Other arguments as for kvq_decode_attn.
 *   KVQ_ERR_SHAPE if n_q < 1, n_q * Hq / Hkv > 16, or the matrix-core kernel
 *   does not cover D and the types (see KVQ_VARIANT_MFMA).
 */
int kvq_decode_attn_multi(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                          const void* q, const int32_t* seq_lens, int B, int n_q, int Hq, int Hkv,
                          int D, float softmax_scale, int max_seq_len, int split_tokens,
                          int max_splits, float* part_o, float* part_lse, void* stream);

/*
 * One multi-query decode step: the n_q new tokens' K and V rows are written
 * at rows L_b - n_q .. L_b - 1 (row i of k_new / v_new at row L_b - n_q + i),
 * then kvq_decode_attn_multi and kvq_combine over n_q * Hq heads run.
 * Results equal kvq_quantize_append of the n_q rows (positions L_b - n_q)
 * followed by those two calls, bit for bit.  Two kernel launches: each
 * attention workgroup whose split holds some of the new rows writes them
 * before it reads them, then the merge runs.
 *
 *   k_new, v_new : device, [B][n_q][Hkv][D] binary16.
 *   out          : device, [B][n_q][Hq][D] of out_type; lse_out [B][n_q][Hq]
 *                  fp32 or NULL.
 *   Other arguments as for kvq_decode_attn_multi and kvq_combine.
 */
int kvq_decode_step_multi(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                          const void* k_new, const void* v_new, const void* q,
                          const int32_t* seq_lens, int B, int n_q, int Hq, int Hkv, int D,
                          float softmax_scale, int max_seq_len, int split_tokens, int max_splits,
                          float* part_o, float* part_lse, int out_type, void* out, float* lse_out,
                          void* stream);

/* Kernel family for kvq_decode_attn_variant.  The matrix-core kernel covers
 * D = 128, 256 and 512 with every pair of f16, q8_0 and q4_0 and the pairs
 * q8_0/q6_0, q8_0/q5_0, q6_0/q6_0, q6_0/q4_0, q5_0/q5_0, q5_1/q5_1,
 * q4_1/q4_1 and q5_1/q4_0.  The vector-ALU kernel
 * covers every pair of types at every valid D; AUTO picks the matrix cores
 * where they cover the call. */
enum {
    KVQ_VARIANT_AUTO = 0, /* what kvq_decode_attn uses                         */
    KVQ_VARIANT_VALU = 1, /* dot products on the vector ALUs                   */
    KVQ_VARIANT_MFMA = 2  /* dot products on the matrix cores (16x16x32 f16)   */
};

/*
 * kvq_decode_attn with an explicit kernel family; same arguments and results
 * (within floating-point rounding).  KVQ_ERR_TYPE for an unknown variant;
 * KVQ_ERR_SHAPE for KVQ_VARIANT_MFMA where the matrix cores do not cover the
 * call.
 */
int kvq_decode_attn_variant(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                            const void* q, const int32_t* seq_lens, int B, int Hq, int Hkv,
                            int D, float softmax_scale, int max_seq_len, int split_tokens,
                            int max_splits, float* part_o, float* part_lse, int variant,
                            void* stream);

/*
 * Exact log-sum-exp merge of split partials (HAL #582 section 5 P2 read path:
 * regions merged by an exact online-softmax combine).  For each (b, h), with
 * S_b = ceil(seq_lens[b] / split_tokens) (at most max_splits):
 *   LSE = ln sum_{s<S_b} exp(part_lse[b][h][s])
 *   out[b][h][:] = sum_{s<S_b} exp(part_lse[b][h][s] - LSE) * part_o[b][h][s][:]
 * computed in fp32; a sequence whose splits are all empty gets out = 0 and
 * LSE = -inf.
 *
 *   part_o, part_lse : device, as written by kvq_decode_attn.
 *   seq_lens         : device, [B] int32 (the same lengths).
 *   out_type         : KVQ_F16 or a value of 3 for fp32 (KVQ_OUT_F32).
 *   out              : device, [B][Hq][D] of out_type, 16-byte aligned.
 *   lse_out          : device, [B][Hq] fp32, or NULL.
 */
#define KVQ_OUT_F32 3
int kvq_combine(const float* part_o, const float* part_lse, const int32_t* seq_lens, int B,
                int Hq, int D, int split_tokens, int max_splits, int out_type, void* out,
                float* lse_out, void* stream);

/*
 * Split-KV attention over both regions of a mixed cache (HAL #582 section 5
 * P2: a quantised tail and an fp16 window of recent tokens) in one call.
 * Equivalent to kvq_decode_attn over the tail (k_tail / v_tail, tail_lens,
 * tail_* splits and partials) followed by kvq_decode_attn over the window
 * (k_win / v_win, fp16, win_lens, win_* splits and partials) with the same q,
 * and bit-identical to it.  Where the matrix-core kernel covers the shape
 * (tail K and V of q8_0 / q4_0 at D = 128, 256 or 512, or a pair with the
 * further types that KVQ_VARIANT_MFMA lists at D = 128) both regions run in one
 * launch: a small window then costs its bytes, not a second launch's start
 * and end.  Otherwise the two launches are made.  The partials merge with
 * kvq_combine_regions.
 *
 *   k_win, v_win : fp16 planes (KVQ_ERR_TYPE otherwise).
 *   Each region's lengths, max_len, splits and partials follow the rules of
 *   kvq_decode_attn; a region's lengths may be 0.
 */
int kvq_decode_attn_mixed(const kvq_plane_desc* k_tail, const kvq_plane_desc* v_tail,
                          const kvq_plane_desc* k_win, const kvq_plane_desc* v_win, const void* q,
                          const int32_t* tail_lens, const int32_t* win_lens, int B, int Hq, int Hkv,
                          int D, float softmax_scale, int tail_max_len, int tail_split_tokens,
                          int tail_max_splits, float* tail_part_o, float* tail_part_lse,
                          int win_max_len, int win_split_tokens, int win_max_splits,
                          float* win_part_o, float* win_part_lse, void* stream);

/*
 * One decode step over a mixed cache (HAL #582 section 5 P2: a quantised tail
 * and an fp16 window that receives the new token): the new row is written into
 * the window at row win_lens[b] - 1, attention runs over both regions as in
 * kvq_decode_attn_mixed, and the partials are merged as by
 * kvq_combine_regions with n_regions = 2 (tail, then window).  Results equal
 * kvq_quantize_append of the row into the window followed by those two calls,
 * bit for bit.  Where the matrix-core kernel covers the shape this is two
 * launches: the window's attention workgroup that holds row win_lens[b] - 1
 * writes it before reading it, then the merge runs.
 *
 *   k_new, v_new   : device, [B][Hkv][D] binary16: the new token's K and V.
 *   win_lens       : lengths of the window *including* the new token,
 *                    1 <= win_lens[b] <= win_max_len (a sequence with
 *                    win_lens[b] = 0 gets no new row).
 *   tail_lens      : 0 <= tail_lens[b] <= tail_max_len.
 *   out_type, out, lse_out : as for kvq_combine.
 *   The remaining arguments are those of kvq_decode_attn_mixed.
 * Moving full windows into the tail (eviction) is kvq_quantize_rows, called
 * by the owner of the cache between steps.
 */
int kvq_decode_step_mixed(const kvq_plane_desc* k_tail, const kvq_plane_desc* v_tail,
                          const kvq_plane_desc* k_win, const kvq_plane_desc* v_win, const void* k_new,
                          const void* v_new, const void* q, const int32_t* tail_lens,
                          const int32_t* win_lens, int B, int Hq, int Hkv, int D, float softmax_scale,
                          int tail_max_len, int tail_split_tokens, int tail_max_splits,
                          float* tail_part_o, float* tail_part_lse, int win_max_len,
                          int win_split_tokens, int win_max_splits, float* win_part_o,
                          float* win_part_lse, int out_type, void* out, float* lse_out, void* stream);

/*
 * Exact log-sum-exp merge of the partials of several regions (HAL #582
 * section 5 P2 read path: each region of a mixed cache -- the fp16 window and
 * the compressed tail -- runs its own typed attention launch, and the regions
 * are merged by an exact online-softmax combine).  Region i was written by
 * kvq_decode_attn with lengths seq_lens[i], split_tokens[i] and
 * max_splits[i]; for each (b, h) the merge runs over the S_b,i =
 * ceil(seq_lens[i][b] / split_tokens[i]) splits of every region, as
 * kvq_combine does over one region.  The result is the attention over the
 * union of the regions' rows.
 *
 *   n_regions    : 1 .. 4.
 *   part_o, part_lse, seq_lens, split_tokens, max_splits : host arrays of
 *                  n_regions entries; the pointers are device pointers laid
 *                  out as for kvq_combine.
 *   out_type, out, lse_out : as for kvq_combine.
 */
int kvq_combine_regions(int n_regions, const float* const* part_o, const float* const* part_lse,
                        const int32_t* const* seq_lens, const int* split_tokens,
                        const int* max_splits, int B, int Hq, int D, int out_type, void* out,
                        float* lse_out, void* stream);

/*
 * One decode step of one layer in a single call: quantise-on-write of the new
 * token, split-KV attention over every row including the new one, and the
 * exact log-sum-exp merge (HAL #582 section 5 P2: the write path quantises a
 * token once, the read path streams the stored blocks and merges regions by an
 * exact online-softmax combine).
 *
 * Results equal kvq_quantize_append (one new row per sequence, written at row
 * seq_lens[b] - 1) followed by kvq_decode_attn and kvq_combine with the same
 * arguments: the cache rows are bit-identical, and the split partials and
 * out / lse_out agree within floating-point rounding.  Where the matrix-core
 * kernel covers the call (see KVQ_VARIANT_MFMA) the step is two kernel
 * launches: attention, then the merge.  The attention kernel's workgroup whose
 * split holds row seq_lens[b] - 1 writes that row; for types f16, q8_0 and
 * q4_0 it takes the row's decoded values straight from its quantiser as one
 * more term of its split, with an fp32 weight where the three calls round
 * that row's weight to fp16 for the matrix cores (the two differ by at most
 * 2^-11 of the weight times the row's largest value); for the further types
 * it reads the row back after writing it.  Other calls run the three kernels
 * in order.
 *
 *   k_new, v_new : device, [B][Hkv][D] binary16: the new token's K and V rows.
 *   seq_lens     : device, [B] int32: lengths *including* the new token,
 *                  1 <= L_b <= max_seq_len <= capacity.
 *   out_type     : KVQ_F16 or KVQ_OUT_F32.
 *   out          : device, [B][Hq][D] of out_type, 16-byte aligned.
 *   lse_out      : device, [B][Hq] fp32 (natural-log LSE of the scores), or
 *                  NULL.
 *   Other arguments and requirements as for kvq_decode_attn; part_o and
 *   part_lse are scratch of the same shapes, overwritten.
 */
int kvq_decode_step(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                    const void* k_new, const void* v_new, const void* q, const int32_t* seq_lens,
                    int B, int Hq, int Hkv, int D, float softmax_scale, int max_seq_len,
                    int split_tokens, int max_splits, float* part_o, float* part_lse,
                    int out_type, void* out, float* lse_out, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * step as kvq_decode_step, with the split partials (max_splits =
 * ceil(max_seq_len / split_tokens)) in a device array of
 * KVQ_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * from load until the process ends, instead of caller memory.  The call
 * allocates nothing.  Results are those of kvq_decode_step with partials of
 * that shape.
 *
 *   Arguments as for kvq_decode_step, without part_o, part_lse and
 *   max_splits.
 *   KVQ_ERR_CAPACITY if the partials need more than the array
 *   (kvq_decode_step_noalloc_bytes gives the bytes a call needs); the other
 *   statuses as for kvq_decode_step, all checked before any HIP call.
 *   Every call on one GPU uses that GPU's one array and leaves its partials
 *   there: calls that overlap on one GPU (other streams, other host threads)
 *   race and must be serialised by the caller.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t kvq_decode_step_noalloc_bytes(int B, int Hq, int D, int max_seq_len, int split_tokens);
int kvq_decode_step_noalloc(const kvq_plane_desc* k_cache, const kvq_plane_desc* v_cache,
                            const void* k_new, const void* v_new, const void* q,
                            const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                            float softmax_scale, int max_seq_len, int split_tokens, int out_type,
                            void* out, float* lse_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
