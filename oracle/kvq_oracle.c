/*
 * kvq_oracle.c -- plain, slow, obviously-correct CPU oracle for block-quantised
 * KV-cache decode attention.  TEST INFRASTRUCTURE ONLY: the product path never
 * links, loads or calls this file.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it.
 *
 * What it computes, and where that comes from:
 *   - Storage types (HAL #582 "per-layer KV compression study", section 1 size
 *     model table): q8_0 = 32-value blocks of int8 plus one fp16 scale
 *     (34 bytes, 8.5 bits/value); q4_0 = 32-value blocks of 4-bit codes plus
 *     one fp16 scale (18 bytes, 4.5 bits/value); f16 = unquantised rows.
 *   - Quantise on write (same study, section 5 P2 "write path": tokens are
 *     quantised once when they are written).  The pages never print the
 *     quantiser, so the block formulas below are this project's readings:
 *     q8_0 scale = max|x| / 127, q4_0 scale = (signed value of largest
 *     magnitude) / -8, codes = round-half-away-from-zero of x / stored scale,
 *     q4_0 codes offset by 8 into [0, 15].
 *   - Decode attention: plain softmax attention of one query row per query
 *     head over the dequantised cache, in fp64 (an exact result with a plain
 *     definition, so the oracle is that definition written out).
 *   - Split + exact log-sum-exp merge of the per-split partial results (same
 *     study, section 5 P2 "read path": two regions merged by an exact online
 *     softmax combine; here generalised to S regions).
 *
 * Every function below is pinned by the CPU tests (hand-worked blocks,
 * exhaustive fp16 sweeps against numpy's IEEE arithmetic, round-trip error
 * bounds, identity inputs, a stdlib brute force, closed forms and
 * invariances); none is "parity unpinned".
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread.
 * fp32 arithmetic relies on x86-64 SSE (FLT_EVAL_METHOD == 0): every float
 * operation is one correctly rounded IEEE binary32 operation.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(FLT_EVAL_METHOD) && FLT_EVAL_METHOD != 0
#error "the oracle needs IEEE binary32 evaluation of float expressions"
#endif

/* Planted-mistake switch used only by the CPU test that proves the pins can
 * see a plausible error.  0 = the oracle as specified. */
#ifndef KVO_MUTANT
#define KVO_MUTANT 0
#endif

enum { KVO_F16 = 0, KVO_Q8_0 = 1, KVO_Q4_0 = 2,
       /* more scalar types (the pages' served pairs name them and give their
        * block sizes; the layouts and quantisers are this project's readings,
        * documented at their quantisers below) */
       KVO_Q4_1 = 4, KVO_Q5_0 = 5, KVO_Q5_1 = 6, KVO_Q6_0 = 7 };

/* ---------------------------------------------------------------- fp16 -- */

/* Exact value of an IEEE 754 binary16 bit pattern (non-finite -> inf/nan). */
double kvo_f16_value(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

float kvo_f16_to_f32(uint16_t h) { return (float)kvo_f16_value(h); }

/* Round a binary32 value to the nearest binary16 value, ties to even,
 * including the subnormal range.  Overflow gives infinity. */
uint16_t kvo_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double v = fabs((double)x);
    if (isnan(x)) return 0x7e00;
    if (v >= 65520.0) return sign | 0x7c00;     /* halfway to 2^16 and up */
    if (v < ldexp(1.0, -14)) {
        /* subnormal grid: multiples of 2^-24 */
        double n = rint(ldexp(v, 24));           /* default mode: ties-to-even */
        return sign | (uint16_t)n;               /* n == 1024 is 2^-14 itself */
    }
    int ex;
    frexp(v, &ex);                               /* v = f * 2^ex, f in [0.5,1) */
    int e = ex - 1;                              /* v in [2^e, 2^(e+1)) */
    double n = rint(ldexp(v, 10 - e));           /* in [1024, 2048] */
    if (n >= 2048.0) { n = 1024.0; e += 1; }
    if (e + 15 >= 31) return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)n - 1024));
}

/* Array form of the conversion above (used by the CPU tests' sweeps). */
void kvo_f32_to_f16_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = kvo_f32_to_f16(x[i]);
}

/* Round half away from zero, evaluated exactly in fp64. */
double kvo_round_half_away(double v)
{
#if KVO_MUTANT == 1
    return rint(v);                              /* planted: ties-to-even */
#else
    double r = floor(fabs(v) + 0.5);
    return v < 0 ? -r : r;
#endif
}

/* --------------------------------------------------------- quantisers -- */

/* q8_0 block of 32 values.  Scale = max|x| / 127 in binary32, rounded to
 * binary16 and stored; codes are round-half-away(x / stored scale) in
 * [-127, 127] (the clamp only bites when the stored scale is subnormal). */
static void quant_block_q8_0(const uint16_t* x, int8_t* q, uint16_t* scale)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float a = fabsf(kvo_f16_to_f32(x[i]));
        if (a > amax) amax = a;
    }
    float d32 = amax / 127.0f;
    uint16_t d16 = kvo_f32_to_f16(d32);
    float d = kvo_f16_to_f32(d16);
#if KVO_MUTANT == 2
    d = d32;                                     /* planted: unrounded scale */
#endif
    *scale = d16;
    for (int i = 0; i < 32; ++i) {
        if (d == 0.0f) { q[i] = 0; continue; }
        float v = kvo_f16_to_f32(x[i]) / d;
        double r = kvo_round_half_away((double)v);
        if (r > 127.0) r = 127.0;
        if (r < -127.0) r = -127.0;
        q[i] = (int8_t)r;
    }
}

/* q4_0 block of 32 values.  The signed value of largest magnitude (first index
 * on ties) divided by -8 gives the scale; codes are round-half-away(x / stored
 * scale) clamped to [-8, 7], offset by 8 to [0, 15], and packed so that byte j
 * holds element j in its low nibble and element j + 16 in its high nibble. */
static void quant_block_q4_0(const uint16_t* x, uint8_t* packed, uint16_t* scale)
{
    float amax = 0.0f, smax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float v = kvo_f16_to_f32(x[i]);
#if KVO_MUTANT == 3
        if (fabsf(v) >= amax) { amax = fabsf(v); smax = v; }  /* planted: last index */
#else
        if (fabsf(v) > amax) { amax = fabsf(v); smax = v; }
#endif
    }
    float d32 = smax / -8.0f;
    uint16_t d16 = kvo_f32_to_f16(d32);
    float d = kvo_f16_to_f32(d16);
    *scale = d16;
    int n[32];
    for (int i = 0; i < 32; ++i) {
        if (d == 0.0f) { n[i] = 8; continue; }
        float v = kvo_f16_to_f32(x[i]) / d;
        double r = kvo_round_half_away((double)v);
        if (r > 7.0) r = 7.0;
        if (r < -8.0) r = -8.0;
        n[i] = (int)r + 8;
    }
    for (int j = 0; j < 16; ++j) {
#if KVO_MUTANT == 4
        packed[j] = (uint8_t)(n[2 * j] | (n[2 * j + 1] << 4));   /* planted: adjacent pairs */
#else
        packed[j] = (uint8_t)(n[j] | (n[j + 16] << 4));
#endif
    }
}

/* ----------------------------------------- more scalar types (readings) --
 *
 * Block sizes on the pages: q5_0 22 bytes per 32 values (HAL #582 section 1
 * size table: 66 KiB per token for q5_0/q5_0 at 48 layers x 8 KV heads x 128),
 * q5_1 24 bytes (section 5 P1 ladder figures), q4_1 20 and q6_0 26 bytes (the
 * same family: 16 bytes of low nibbles, 4 or 8 bytes of high bits, one fp16
 * scale, and for the "_1" types one fp16 minimum).  The pages print no
 * layout; this oracle's readings:
 *   - a row's data plane holds the low 4 bits of every code first (D/2
 *     bytes, block b at 16*b, byte j of a block = element j in the low nibble
 *     and element j+16 in the high nibble, as q4_0), then the high bits:
 *     q5_0 / q5_1 one little-endian 32-bit word per block whose bit j is bit 4
 *     of element j's code; q6_0 one little-endian 64-bit word per block whose
 *     bits 2j, 2j+1 are bits 4, 5 of element j's code;
 *   - the scale plane holds one fp16 per block (q5_0, q6_0: the scale d) or
 *     two (q4_1, q5_1: d, then the minimum m);
 *   - q5_0 / q6_0 extend q4_0: d = fp16(s / -16) or fp16(s / -32) with s the
 *     first value of largest magnitude; code = clamp(round_half_away(x / d),
 *     -16, 15) + 16 or clamp(..., -32, 31) + 32; value = d * (code - 16 or
 *     32); d = 0 gives every code the offset;
 *   - q4_1 / q5_1 map [min, max] onto the codes: m = fp16(min x), d =
 *     fp16((max x - min x) / 15 or 31) (binary32 subtraction and division),
 *     code = clamp(round_half_away((x - m) / d), 0, 15 or 31) with the stored
 *     m and d (binary32 subtraction and division); d = 0 gives code 0;
 *     value = d * code + m. */

/* The value of largest magnitude, first index on ties (+0 for a block of
 * zeros). */
static float first_absmax(const uint16_t* x)
{
    float amax = 0.0f, smax = 0.0f;
    for (int i = 0; i < 32; ++i) {
        float v = kvo_f16_to_f32(x[i]);
        if (fabsf(v) > amax) { amax = fabsf(v); smax = v; }
    }
    return smax;
}

/* Codes of a symmetric block with 2^(bits-1) negative levels: q5_0 (bits 5)
 * and q6_0 (bits 6).  Writes n[32] in [0, 2^bits) and the fp16 scale. */
static void quant_codes_sym(const uint16_t* x, int bits, int* n, uint16_t* scale)
{
    const int half = 1 << (bits - 1);
    float smax = first_absmax(x);
    uint16_t d16 = kvo_f32_to_f16(smax / -(float)half);
    float d = kvo_f16_to_f32(d16);
    *scale = d16;
    for (int i = 0; i < 32; ++i) {
        if (d == 0.0f) { n[i] = half; continue; }
        float v = kvo_f16_to_f32(x[i]) / d;
        double r = kvo_round_half_away((double)v);
#if KVO_MUTANT == 8
        if (r > half) r = half;                  /* planted: clamp one level too high */
#else
        if (r > half - 1) r = half - 1;
#endif
        if (r < -half) r = -half;
        n[i] = (int)r + half;
    }
}

/* Codes of a min/max block: q4_1 (levels 15) and q5_1 (levels 31).  Writes
 * n[32] in [0, levels] and the fp16 scale and minimum. */
static void quant_codes_minmax(const uint16_t* x, int levels, int* n, uint16_t* scale, uint16_t* minv)
{
    float mn = kvo_f16_to_f32(x[0]), mx = mn;
    for (int i = 1; i < 32; ++i) {
        float v = kvo_f16_to_f32(x[i]);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    uint16_t d16 = kvo_f32_to_f16((mx - mn) / (float)levels);
    uint16_t m16 = kvo_f32_to_f16(mn);
    float d = kvo_f16_to_f32(d16), m = kvo_f16_to_f32(m16);
#if KVO_MUTANT == 6
    d = (mx - mn) / (float)levels;               /* planted: unrounded min/max scale */
#endif
    *scale = d16;
    *minv = m16;
    for (int i = 0; i < 32; ++i) {
        if (d == 0.0f) { n[i] = 0; continue; }
        float v = (kvo_f16_to_f32(x[i]) - m) / d;
        double r = kvo_round_half_away((double)v);
        if (r > levels) r = levels;
        if (r < 0.0) r = 0.0;
        n[i] = (int)r;
    }
}

/* Writes the low nibbles of block b (16 bytes at lo + 16*b) and its high
 * bits (hb_bits 1 or 2 per element, at hi + 4*b or 8*b, little endian). */
static void pack_codes(const int* n, int hb_bits, uint8_t* lo, uint8_t* hi, int b)
{
    for (int j = 0; j < 16; ++j)
        lo[16 * b + j] = (uint8_t)((n[j] & 15) | ((n[j + 16] & 15) << 4));
    if (hb_bits == 0) return;
    uint64_t w = 0;
    for (int j = 0; j < 32; ++j)
#if KVO_MUTANT == 7
        w |= (uint64_t)(n[j] >> 4) << (hb_bits * (j ^ 1));   /* planted: high bits of pairs swapped */
#else
        w |= (uint64_t)(n[j] >> 4) << (hb_bits * j);
#endif
    int nbytes = 4 * hb_bits;
    for (int k = 0; k < nbytes; ++k) hi[nbytes * b + k] = (uint8_t)(w >> (8 * k));
}

/* Code of element i of a row (low nibble plus high bits). */
static int unpack_code(int type, const uint8_t* row, int D, int i)
{
    int b = i / 32, e = i % 32;
    uint8_t byte = row[16 * b + (e % 16)];
    int n = e < 16 ? (byte & 0x0f) : (byte >> 4);
    if (type == KVO_Q5_0 || type == KVO_Q5_1) {
        const uint8_t* hi = row + D / 2 + 4 * b;
        n |= ((hi[e / 8] >> (e % 8)) & 1) << 4;
    } else if (type == KVO_Q6_0) {
        const uint8_t* hi = row + D / 2 + 8 * b;
        n |= ((hi[e / 4] >> (2 * (e % 4))) & 3) << 4;
    }
    return n;
}

static int is_quant_type(int type)
{
    return type == KVO_Q8_0 || type == KVO_Q4_0 || type == KVO_Q4_1 || type == KVO_Q5_0 ||
           type == KVO_Q5_1 || type == KVO_Q6_0;
}

/* fp16 entries of the scale plane per block: 2 for the min/max types. */
static int scales_per_block(int type)
{
    return type == KVO_Q4_1 || type == KVO_Q5_1 ? 2 : type == KVO_F16 ? 0 : 1;
}

/* Bytes of the data plane per row of D values, and of the scale plane
 * (0 for an unknown type). */
int64_t kvo_data_row_bytes(int type, int D)
{
    switch (type) {
    case KVO_F16: return 2 * (int64_t)D;
    case KVO_Q8_0: return D;
    case KVO_Q4_0:
    case KVO_Q4_1: return D / 2;
    case KVO_Q5_0:
    case KVO_Q5_1: return D / 2 + D / 8;
    case KVO_Q6_0: return D / 2 + D / 4;
    default: return 0;
    }
}
int64_t kvo_scale_row_bytes(int type, int D)
{
    return is_quant_type(type) ? 2 * (int64_t)scales_per_block(type) * (D / 32) : 0;
}

/* Quantise nrows rows of D f16 values (D a multiple of 32) into a data plane
 * (nrows x data_row_bytes) and a scale plane (nrows x scale_row_bytes / 2
 * fp16), or copy the f16 bits unchanged for the f16 type.  Returns 0, or -1
 * on bad arguments. */
int kvo_quantize_rows(int type, const uint16_t* src, int64_t nrows, int D,
                      uint8_t* data, uint16_t* scales)
{
    if (D <= 0 || D % 32 != 0 || nrows < 0) return -1;
    int nb = D / 32;
    for (int64_t r = 0; r < nrows; ++r) {
        const uint16_t* x = src + r * D;
        if (type == KVO_F16) {
            memcpy(data + r * 2 * (int64_t)D, x, 2 * (size_t)D);
        } else if (type == KVO_Q8_0) {
            for (int b = 0; b < nb; ++b)
                quant_block_q8_0(x + 32 * b, (int8_t*)(data + r * D + 32 * b),
                                 scales + r * nb + b);
        } else if (type == KVO_Q4_0) {
            for (int b = 0; b < nb; ++b)
                quant_block_q4_0(x + 32 * b, data + r * (D / 2) + 16 * b,
                                 scales + r * nb + b);
        } else if (type == KVO_Q5_0 || type == KVO_Q6_0) {
            int bits = type == KVO_Q5_0 ? 5 : 6;
            uint8_t* row = data + r * kvo_data_row_bytes(type, D);
            for (int b = 0; b < nb; ++b) {
                int n[32];
                quant_codes_sym(x + 32 * b, bits, n, scales + r * nb + b);
                pack_codes(n, bits - 4, row, row + D / 2, b);
            }
        } else if (type == KVO_Q4_1 || type == KVO_Q5_1) {
            int levels = type == KVO_Q4_1 ? 15 : 31;
            uint8_t* row = data + r * kvo_data_row_bytes(type, D);
            for (int b = 0; b < nb; ++b) {
                int n[32];
                uint16_t* sc = scales + r * 2 * nb + 2 * b;
                quant_codes_minmax(x + 32 * b, levels, n, sc, sc + 1);
                pack_codes(n, type == KVO_Q4_1 ? 0 : 1, row, row + D / 2, b);
            }
        } else {
            return -1;
        }
    }
    return 0;
}

/* ------------------------------------------------------------ dequant -- */

/* Value of element i of row r, exactly (the product of an fp16 scale and a
 * small integer is exact in fp64). */
static double deq(int type, const uint8_t* data, const uint16_t* scales,
                  int64_t r, int D, int i)
{
    if (type == KVO_F16) {
        uint16_t h;
        memcpy(&h, data + (r * D + i) * 2, 2);
        return kvo_f16_value(h);
    }
    if (type != KVO_Q8_0 && type != KVO_Q4_0) {
        const uint8_t* row = data + r * kvo_data_row_bytes(type, D);
        int n = unpack_code(type, row, D, i);
        int spb = scales_per_block(type);
        const uint16_t* sc = scales + r * spb * (D / 32) + spb * (i / 32);
        double ds = kvo_f16_value(sc[0]);
        switch (type) {
        case KVO_Q5_0: return ds * (double)(n - 16);
        case KVO_Q6_0: return ds * (double)(n - 32);
        default: return ds * (double)n + kvo_f16_value(sc[1]);   /* q4_1, q5_1 */
        }
    }
    double d = kvo_f16_value(scales[r * (D / 32) + i / 32]);
    if (type == KVO_Q8_0) {
        int8_t q = (int8_t)data[r * D + i];
        return d * (double)q;
    }
    int b = i / 32, e = i % 32;
    uint8_t byte = data[r * (D / 2) + 16 * b + (e % 16)];
    int n = e < 16 ? (byte & 0x0f) : (byte >> 4);
#if KVO_MUTANT == 12
    return d * (double)(n - 7);                   /* planted: q4_0 offset off by one */
#else
    return d * (double)(n - 8);
#endif
}

/* Whole row r dequantised into out[0..D) (the same values as deq()). */
static void deq_row(int type, const uint8_t* data, const uint16_t* scales,
                    int64_t r, int D, double* out)
{
    for (int i = 0; i < D; ++i) out[i] = deq(type, data, scales, r, D, i);
}

int kvo_dequant_rows(int type, const uint8_t* data, const uint16_t* scales,
                     int64_t nrows, int D, double* out)
{
    if (D <= 0 || D % 32 != 0 || nrows < 0) return -1;
    if (type != KVO_F16 && !is_quant_type(type)) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        for (int i = 0; i < D; ++i)
            out[r * D + i] = deq(type, data, scales, r, D, i);
    return 0;
}

/* ----------------------------------------------------------- attention -- */

/* Cache layout shared by K and V: for sequence b and KV head g, row t lives
 * at row index (b * Hkv + g) * capacity + t of the data and scale planes. */
typedef struct {
    int B, Hq, Hkv, D, capacity;
    const int32_t* seq_lens;    /* [B] */
    const uint16_t* q;          /* [B][Hq][D] f16 bits */
    int tK, tV;
    const uint8_t* k_data; const uint16_t* k_scales;
    const uint8_t* v_data; const uint16_t* v_scales;
    double scale;
    int split_tokens, max_splits; /* split_tokens <= 0: one region [0, L) */
    double* out;                /* [B][Hq][D]              or [B][Hq][S][D] */
    double* lse;                /* [B][Hq]                 or [B][Hq][S]    */
    int nthreads;
    int64_t next_item;
    pthread_mutex_t lock;
} attn_job;

/* Softmax attention of one query row over rows [t0, t1) of one KV head:
 * s_t = scale * sum_d q_d k_td;  o = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m);
 * lse = m + ln sum_t exp(s_t - m).  An empty range gives o = 0, lse = -inf. */
static void attend_region(const attn_job* J, int b, int h, int t0, int t1,
                          double* o, double* lse, double* s, double* row)
{
#if KVO_MUTANT == 9
    int D = J->D, g = h % J->Hkv;                 /* planted: heads interleaved over KV heads */
#else
    int D = J->D, G = J->Hq / J->Hkv, g = h / G;
#endif
    int64_t row0 = ((int64_t)b * J->Hkv + g) * J->capacity;
    for (int i = 0; i < D; ++i) o[i] = 0.0;
    if (t1 <= t0) { *lse = -INFINITY; return; }
    const uint16_t* qh = J->q + ((int64_t)b * J->Hq + h) * D;
    double* qd = row + D;
    for (int i = 0; i < D; ++i) qd[i] = kvo_f16_value(qh[i]);
    double m = -INFINITY;
    for (int t = t0; t < t1; ++t) {
        deq_row(J->tK, J->k_data, J->k_scales, row0 + t, D, row);
        double acc = 0.0;
        for (int i = 0; i < D; ++i) acc += qd[i] * row[i];
#if KVO_MUTANT == 10
        s[t - t0] = acc;                          /* planted: softmax scale dropped */
#else
        s[t - t0] = J->scale * acc;
#endif
        if (s[t - t0] > m) m = s[t - t0];
    }
    double l = 0.0;
    for (int t = t0; t < t1; ++t) {
        double p = exp(s[t - t0] - m);
        l += p;
#if KVO_MUTANT == 11
        deq_row(J->tK, J->k_data, J->k_scales, row0 + t, D, row);   /* planted: V read from K */
#else
        deq_row(J->tV, J->v_data, J->v_scales, row0 + t, D, row);
#endif
        for (int i = 0; i < D; ++i) o[i] += p * row[i];
    }
    for (int i = 0; i < D; ++i) o[i] /= l;
    *lse = m + log(l);
}

static void* attn_worker(void* arg)
{
    attn_job* J = (attn_job*)arg;
    int64_t n_items = (int64_t)J->B * J->Hq;
    int64_t maxL = 0;
    for (int b = 0; b < J->B; ++b) if (J->seq_lens[b] > maxL) maxL = J->seq_lens[b];
    double* s = (double*)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
    double* row = (double*)malloc(sizeof(double) * 2 * (size_t)J->D);
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t it = J->next_item++;
        pthread_mutex_unlock(&J->lock);
        if (it >= n_items) break;
        int b = (int)(it / J->Hq), h = (int)(it % J->Hq);
        int L = J->seq_lens[b];
        if (J->split_tokens <= 0) {
            attend_region(J, b, h, 0, L, J->out + it * J->D, J->lse + it, s, row);
        } else {
            for (int sp = 0; sp < J->max_splits; ++sp) {
                int t0 = sp * J->split_tokens;
                int t1 = t0 + J->split_tokens;
                if (t0 > L) t0 = L;
                if (t1 > L) t1 = L;
                int64_t k = it * J->max_splits + sp;
                attend_region(J, b, h, t0, t1, J->out + k * J->D, J->lse + k, s, row);
            }
        }
    }
    free(s);
    free(row);
    return NULL;
}

static int run_attn(attn_job* J)
{
    if (J->B < 0 || J->Hq <= 0 || J->Hkv <= 0 || J->Hq % J->Hkv != 0) return -1;
    if (J->D <= 0 || J->D % 32 != 0 || J->capacity < 0) return -1;
    for (int b = 0; b < J->B; ++b)
        if (J->seq_lens[b] < 0 || J->seq_lens[b] > J->capacity) return -1;
    if (J->split_tokens > 0)
        for (int b = 0; b < J->B; ++b)
            if ((int64_t)J->max_splits * J->split_tokens < J->seq_lens[b]) return -1;
    int nt = J->nthreads < 1 ? 1 : J->nthreads;
    J->next_item = 0;
    pthread_mutex_init(&J->lock, NULL);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    for (int i = 0; i < nt; ++i) pthread_create(&th[i], NULL, attn_worker, J);
    for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J->lock);
    return 0;
}

/* Whole-context attention: out [B][Hq][D], lse [B][Hq].  Query head h reads
 * KV head floor(h / (Hq / Hkv)). */
int kvo_attend(int B, int Hq, int Hkv, int D, int capacity, const int32_t* seq_lens,
               const uint16_t* q, int tK, const uint8_t* k_data, const uint16_t* k_scales,
               int tV, const uint8_t* v_data, const uint16_t* v_scales,
               double scale, double* out, double* lse, int nthreads)
{
    attn_job J = {B, Hq, Hkv, D, capacity, seq_lens, q, tK, tV, k_data, k_scales,
                  v_data, v_scales, scale, 0, 1, out, lse, nthreads, 0};
    return run_attn(&J);
}

/* Per-split attention: split sp covers rows [sp*split_tokens, (sp+1)*split_tokens)
 * clipped to [0, L_b).  out [B][Hq][max_splits][D], lse [B][Hq][max_splits]. */
int kvo_attend_split(int B, int Hq, int Hkv, int D, int capacity, const int32_t* seq_lens,
                     const uint16_t* q, int tK, const uint8_t* k_data, const uint16_t* k_scales,
                     int tV, const uint8_t* v_data, const uint16_t* v_scales,
                     double scale, int split_tokens, int max_splits,
                     double* out, double* lse, int nthreads)
{
    if (split_tokens <= 0 || max_splits <= 0) return -1;
    attn_job J = {B, Hq, Hkv, D, capacity, seq_lens, q, tK, tV, k_data, k_scales,
                  v_data, v_scales, scale, split_tokens, max_splits, out, lse, nthreads, 0};
    return run_attn(&J);
}

/* Exact merge of S partial results per (b, h): LSE = ln sum_s exp(lse_s),
 * out = sum_s exp(lse_s - LSE) * o_s.  All splits empty: out = 0, LSE = -inf. */
int kvo_combine(int BH, int S, int D, const double* part_o, const double* part_lse,
                double* out, double* lse)
{
    if (BH < 0 || S <= 0 || D <= 0) return -1;
    for (int64_t r = 0; r < BH; ++r) {
        const double* ls = part_lse + r * S;
        double m = -INFINITY;
        for (int s = 0; s < S; ++s) if (ls[s] > m) m = ls[s];
        double* o = out + r * D;
        for (int i = 0; i < D; ++i) o[i] = 0.0;
        if (m == -INFINITY) { lse[r] = -INFINITY; continue; }
        double sum = 0.0;
        for (int s = 0; s < S; ++s) sum += exp(ls[s] - m);
        double L = m + log(sum);
#if KVO_MUTANT == 5
        int s_end = S - 1;                        /* planted: last split dropped */
#else
        int s_end = S;
#endif
        for (int s = 0; s < s_end; ++s) {
            double w = exp(ls[s] - L);
            for (int i = 0; i < D; ++i) o[i] += w * part_o[(r * S + s) * D + i];
        }
        lse[r] = L;
    }
    return 0;
}
