// decode_mfma.hip -- split-KV decode attention with both contractions on the
// CDNA4 matrix cores (HAL #582 "per-layer KV compression study", section 3b
// finding 2 and section 5 P0: the quant reader is given the same matrix-core
// route as f16 and reads the raw blocks in registers; section 5 P2: per-region
// partials merged by an exact log-sum-exp combine).
//
// One workgroup (4 wave64) per (sequence, KV head, split); each wave walks its
// own 32-row tiles of the split (tiles w, w+4, ...) with private LDS buffers,
// so waves never wait for each other until the final merge.
//
// Per 32-row tile:
//   QK^T as S^T = K * Q^T with v_mfma_f32_16x16x32_f16: A = 16 K rows x 32
//     values of one 32-value block (the raw codes, exactly representable in
//     fp16), B = the GQA group's Q (16 columns, G used).  One MFMA per block;
//     its fp32 result is multiplied by the row's block scale (exact products,
//     fp32 sums).  K goes straight from HBM to registers with coalesced
//     16-byte loads; a 4x4 exchange between the four 16-lane rows
//     (v_permlane32_swap / v_permlane16_swap) turns "lane row q holds block q"
//     into "lane row q holds a quarter of every block".
//   online softmax in fp32, log2 domain; the running maximum is only moved
//     when a score exceeds it by more than 2^8 (exact either way: every
//     partial sum is kept relative to the same reference), so rescaling the
//     accumulators is rare.
//   PV as O^T = V^T * P'^T: V is staged in LDS with direct global->LDS 16-byte
//     loads and read back transposed (ds_read_b64_tr_b4 / _b8 / _b16) so each
//     lane holds one value column for 8 rows; codes become fp16 exactly
//     (nibble | 0x6400 minus 1032, byte ^ 0x80 | 0x6400 minus 1152).  The
//     V block scale is folded into P (P' = p * scale per row and block, fp16),
//     since every 16-column MFMA tile lies inside one 32-value block.
// The four waves' (max, sum, O) are merged through LDS into one normalised
// partial per (head, split).
#include <math.h>

#include "kvq_internal.hpp"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int WAVES = 4;
constexpr int NT = 64 * WAVES;
constexpr int TT = 32;          // rows per tile
constexpr float TAU = 8.0f;     // lazy rescale threshold, log2 units

__host__ __device__ constexpr int rb(int t, int D) { return data_row_bytes(t, D); }

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ half8 make_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    u32x4 u = {a, b, c, d};
    return __builtin_bit_cast(half8, u);
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_add_h(uint32_t x, uint32_t c)
{
    half2v a = __builtin_bit_cast(half2v, x), b = __builtin_bit_cast(half2v, c);
    return __builtin_bit_cast(uint32_t, a + b);
}

__device__ __forceinline__ uint32_t pk_mul_h(uint32_t x, uint32_t c)
{
    half2v a = __builtin_bit_cast(half2v, x), b = __builtin_bit_cast(half2v, c);
    return __builtin_bit_cast(uint32_t, a * b);
}

__device__ __forceinline__ uint32_t cvt_pk_h(float lo, float hi)
{
    half2v r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

// 8 nibbles of one dword -> 8 fp16 values (code - 8), element order
// [nib0, nib4, nib1, nib5, nib2, nib6, nib3, nib7].
__device__ __forceinline__ half8 q4_dword_to_half8(uint32_t w)
{
    const uint32_t M = 0x000F000Fu, MAGIC = 0x64006400u, BIAS = 0xE408E408u;  // -1032, -1032
    const uint32_t p0 = pk_add_h((w & M) | MAGIC, BIAS);
    const uint32_t p1 = pk_add_h(((w >> 4) & M) | MAGIC, BIAS);
    const uint32_t p2 = pk_add_h(((w >> 8) & M) | MAGIC, BIAS);
    const uint32_t p3 = pk_add_h(((w >> 12) & M) | MAGIC, BIAS);
    return make_half8(p0, p1, p2, p3);
}

// 8 signed bytes (two dwords) -> 8 fp16 values in byte order.
__device__ __forceinline__ half8 q8_dwords_to_half8(uint32_t w0, uint32_t w1)
{
    const uint32_t BIAS = 0xE480E480u;  // -1152, -1152
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    const uint32_t K64 = 0x64646464u;
    // v_perm_b32: bytes 0..3 from the second operand, 4..7 from the first
    const uint32_t a = pk_add_h(__builtin_amdgcn_perm(K64, u0, 0x04010400u), BIAS);
    const uint32_t b = pk_add_h(__builtin_amdgcn_perm(K64, u0, 0x04030402u), BIAS);
    const uint32_t c = pk_add_h(__builtin_amdgcn_perm(K64, u1, 0x04010400u), BIAS);
    const uint32_t d = pk_add_h(__builtin_amdgcn_perm(K64, u1, 0x04030402u), BIAS);
    return make_half8(a, b, c, d);
}

// 4x4 exchange between the four 16-lane rows: on entry lane row g holds
// x[w] = X[g][w]; on exit it holds x[w] = X[w][g].
__device__ __forceinline__ void xpose4(uint32_t& r0, uint32_t& r1, uint32_t& r2, uint32_t& r3)
{
    auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
    r0 = a[0]; r2 = a[1];
    auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
    r1 = b[0]; r3 = b[1];
    auto c = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
    r0 = c[0]; r1 = c[1];
    auto d = __builtin_amdgcn_permlane16_swap(r2, r3, false, false);
    r2 = d[0]; r3 = d[1];
}

__device__ __forceinline__ float xmax4(float v)
{
    // max over the four lanes l, l^16, l^32, l^48
    auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    v = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}

__device__ __forceinline__ float xsum4(float v)
{
    auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    v = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                              __builtin_bit_cast(uint32_t, v), false, false);
    return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

// Explicit waits for the direct global->LDS loads, whose completion the
// compiler does not track for later LDS reads.  The memory clobber also keeps
// the compiler from moving loads across the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkm0()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void lds_load16(const void* g, LDS_AS void* l)
{
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

__device__ __forceinline__ void lds_load4(const void* g, LDS_AS void* l)
{
    __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
}

// --------------------------------------------------------------- the kernel

template <int TK, int TV, int D>
struct Cfg {
    static constexpr int NB = D / 32;               // blocks per row
    static constexpr int NBG = D / 128;             // groups of 4 blocks
    static constexpr int RBK = rb(TK, D);
    static constexpr int RBV = rb(TV, D);
    static constexpr int KU = TK == T_Q4 ? 1 : (TK == T_Q8 ? 2 : 4);   // dwords per lane per block
    static constexpr int KDW = 4 * KU * NBG;                           // dwords per lane per subtile
    static constexpr int V_BYTES = TT * RBV;                           // V tile bytes
    static constexpr int V_LOADS = V_BYTES / 1024;                     // 16-byte direct loads per tile
    static constexpr int S_BYTES = TT * 2 * NB;                        // one scale tile
    static constexpr int S_LOADS = S_BYTES / 256;                      // 4-byte direct loads per tile
    static constexpr int K_SCALE = TK != T_F16;
    static constexpr int V_SCALE = TV != T_F16;
    // per-wave LDS buffer: V tile, K scales, V scales
    static constexpr int BUF = V_BYTES + S_BYTES * (K_SCALE + V_SCALE);
    static constexpr int KS_OFF = V_BYTES;
    static constexpr int VS_OFF = V_BYTES + S_BYTES * K_SCALE;
    static constexpr int WAVE_LDS = 2 * BUF;
    static constexpr int NDT = D / 16;                                 // PV output tiles
    // vector-memory ops issued per tile (for the explicit LDS wait)
    static constexpr int K_VM = 2 * NBG * KU;                          // 16-byte K loads (2 subtiles)
    static constexpr int TILE_VM = K_VM + V_LOADS + (K_SCALE ? S_LOADS : 0) + (V_SCALE ? S_LOADS : 0);
    static constexpr bool VALID = V_BYTES % 1024 == 0 && S_BYTES % 256 == 0 && TILE_VM < 64 &&
                                  WAVES * WAVE_LDS <= 160 * 1024;
};

template <int TK, int TV, int D>
__global__ void __launch_bounds__(NT) decode_mfma_kernel(DecodeArgs a)
{
    using C = Cfg<TK, TV, D>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lq = lane >> 4;       // column / lane row of the 16x16 layouts
    const int G = a.G;
    const int L = a.seq_lens[b];
    const int t_begin = s * a.split_tokens;
    const int t_end = min(t_begin + a.split_tokens, L);
    const int h0 = g * G;
    const int64_t ho_stride = (int64_t)a.max_splits * D;
    float* po = a.part_o + (((int64_t)b * a.Hq + h0) * a.max_splits + s) * D;
    float* pl = a.part_lse + ((int64_t)b * a.Hq + h0) * a.max_splits + s;

    if (t_begin >= t_end) {
        for (int i = tid; i < G * D; i += NT) po[(i / D) * ho_stride + (i % D)] = 0.0f;
        if (tid < G) pl[(int64_t)tid * a.max_splits] = -INFINITY;
        return;
    }

    const int64_t krow0 = (int64_t)b * a.k.seq_stride + (int64_t)g * a.k.head_stride;
    const int64_t vrow0 = (int64_t)b * a.v.seq_stride + (int64_t)g * a.v.head_stride;
    const uint8_t* kdata = a.k.data + krow0 * C::RBK;
    const uint8_t* kscl = reinterpret_cast<const uint8_t*>(a.k.scales + krow0 * C::NB);
    const uint8_t* vdata = a.v.data + vrow0 * C::RBV;
    const uint8_t* vscl = reinterpret_cast<const uint8_t*>(a.v.scales + vrow0 * C::NB);

    // ---- Q as the B operand of S^T = K Q^T: column ln = head, lane row lq
    half8 qop[C::NB];
    {
        const uint16_t* qh = a.q + ((int64_t)b * a.Hq + h0 + min(ln, G - 1)) * D;
#pragma unroll
        for (int kb = 0; kb < C::NB; ++kb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                int el;
                if constexpr (TK == T_Q4) {
                    const int p = e >> 1, hi = e & 1, nib = p + 4 * hi;
                    el = 4 * lq + (nib >> 1) + 16 * (nib & 1);
                } else {
                    el = 8 * lq + e;
                }
                qop[kb][e] = ln < G ? __builtin_bit_cast(_Float16, qh[32 * kb + el]) : (_Float16)0.0f;
            }
        }
    }

    uint8_t* wbuf = smem + wave * C::WAVE_LDS;
    floatx4 oacc[C::NDT];
#pragma unroll
    for (int i = 0; i < C::NDT; ++i) oacc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_ref = -INFINITY, l_part = 0.0f;

    const int ntiles = (t_end - t_begin + TT - 1) / TT;

    // ---- issue all loads of tile `it` (K rows to registers, V rows and both
    //      scale tiles to LDS buffer `buf`)
    auto issue = [&](int it, uint32_t (&kr)[2][C::KDW], int buf) {
        const int t0 = t_begin + it * TT;
        uint8_t* vb = wbuf + buf * C::BUF;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int tok = t0 + 8 * (ln >> 2) + 4 * j + (ln & 3);
            const uint8_t* row = kdata + (int64_t)min(tok, L - 1) * C::RBK;
#pragma unroll
            for (int bg = 0; bg < C::NBG; ++bg) {
#pragma unroll
                for (int u = 0; u < C::KU; ++u) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(
                        row + bg * (C::RBK / C::NBG) + lq * (16 * C::KU) + 16 * u);
#pragma unroll
                    for (int c = 0; c < 4; ++c) kr[j][(bg * C::KU + u) * 4 + c] = v[c];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < C::V_LOADS; ++k) {
            const int c16 = k * 64 + lane;
            const int tok = c16 / (C::RBV / 16), off = c16 % (C::RBV / 16);
            lds_load16(vdata + (int64_t)min(t0 + tok, L - 1) * C::RBV + 16 * off,
                       (LDS_AS void*)(vb + 1024 * k));
        }
        if constexpr (C::K_SCALE) {
#pragma unroll
            for (int k = 0; k < C::S_LOADS; ++k) {
                const int c4 = k * 64 + lane;
                const int tok = c4 / (C::NB / 2), dw = c4 % (C::NB / 2);
                lds_load4(kscl + (int64_t)min(t0 + tok, L - 1) * (2 * C::NB) + 4 * dw,
                          (LDS_AS void*)(vb + C::KS_OFF + 256 * k));
            }
        }
        if constexpr (C::V_SCALE) {
#pragma unroll
            for (int k = 0; k < C::S_LOADS; ++k) {
                const int c4 = k * 64 + lane;
                const int tok = c4 / (C::NB / 2), dw = c4 % (C::NB / 2);
                lds_load4(vscl + (int64_t)min(t0 + tok, L - 1) * (2 * C::NB) + 4 * dw,
                          (LDS_AS void*)(vb + C::VS_OFF + 256 * k));
            }
        }
    };

    // ---- compute tile `it` whose data is in kr / LDS buffer `buf`
    auto compute = [&](int it, uint32_t (&kr)[2][C::KDW], int buf) {
        const int t0 = t_begin + it * TT;
        const uint8_t* vb = wbuf + buf * C::BUF;
        const uint8_t* ksb = vb + C::KS_OFF;
        const uint8_t* vsb = vb + C::VS_OFF;

        // -- QK: S^T for the two 16-row subtiles; lane (ln, lq) reg i holds the
        //    score of row t0 + 8*lq + 4*j + i for head ln
        floatx4 sacc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            uint32_t* x = kr[j];
            // exchange: lane row lq loaded all of block (4*bg + lq), dword
            // delta at x[bg*4*KU + delta]; quarter w of a block is dwords
            // [w*KU, (w+1)*KU).  Afterwards lane row lq holds quarter lq of
            // block 4*bg + w at x[bg*4*KU + w*KU + v].
#pragma unroll
            for (int bg = 0; bg < C::NBG; ++bg) {
                uint32_t* base = x + bg * 4 * C::KU;
#pragma unroll
                for (int u = 0; u < C::KU; ++u)
                    xpose4(base[0 * C::KU + u], base[1 * C::KU + u], base[2 * C::KU + u],
                           base[3 * C::KU + u]);
            }
            floatx4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
            // block scales of this lane's four rows (t0 + 8*lq + 4*j + i)
            const uint16_t* srow = reinterpret_cast<const uint16_t*>(ksb) + (8 * lq + 4 * j) * C::NB;
#pragma unroll
            for (int bg = 0; bg < C::NBG; ++bg) {
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4) {
                    const int kb = 4 * bg + kb4;
                    const uint32_t* q = x + bg * 4 * C::KU + kb4 * C::KU;
                    half8 av;
                    if constexpr (TK == T_Q4) av = q4_dword_to_half8(q[0]);
                    else if constexpr (TK == T_Q8) av = q8_dwords_to_half8(q[0], q[1]);
                    else av = make_half8(q[0], q[1], q[2], q[3]);
                    const floatx4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const floatx4 c = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qop[kb], z, 0, 0, 0);
                    if constexpr (C::K_SCALE) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            sc[i] = fmaf(c[i], h2f(srow[i * C::NB + kb]), sc[i]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) sc[i] += c[i];
                    }
                }
            }
            sacc[j] = sc;
        }

        // -- online softmax (log2 domain)
        float sv[8];
        const bool tail = t0 + TT > t_end;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = sacc[j][i] * a.scale_log2;
                sv[4 * j + i] = (tail && t0 + 8 * lq + 4 * j + i >= t_end) ? -INFINITY : x;
            }
        float mx = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
        const bool need = mx > m_ref + TAU;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float hmax = xmax4(mx);
            const float m_new = hmax > m_ref + TAU ? hmax : m_ref;
            const float al = exp2f(m_ref - m_new);
            l_part *= al;
#pragma unroll
            for (int t = 0; t < C::NDT; ++t) oacc[t] *= al;
            m_ref = m_new;
        }
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = exp2f(sv[e] - m_ref);
            l_part += p[e];
        }
        uint32_t pp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pp[k] = cvt_pk_h(p[2 * k], p[2 * k + 1]);

        // -- the LDS data of this tile must have landed (the next tile's loads
        //    may still be in flight)
        // (the caller waits before calling compute)

        // -- P' = P * V block scale for the rows of this lane row (8*lq + e)
        uint32_t ps[C::NB][4];
        if constexpr (C::V_SCALE) {
            const uint16_t* vs = reinterpret_cast<const uint16_t*>(vsb) + (8 * lq) * C::NB;
#pragma unroll
            for (int kb = 0; kb < C::NB; ++kb)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t sp = (uint32_t)vs[(2 * k) * C::NB + kb] |
                                        ((uint32_t)vs[(2 * k + 1) * C::NB + kb] << 16);
                    ps[kb][k] = pk_mul_h(pp[k], sp);
                }
        }

        // -- PV: O^T tile t (16 value columns) += V^T(16 x 32 rows) * P'^T
        const LDS_AS uint8_t* vl = (const LDS_AS uint8_t*)vb;
        if constexpr (TV == T_Q4) {
            // one transposed read gives two column tiles (chunks 2c2, 2c2+1);
            // lane r of the row group addresses row 8*lq + pi(r&7), chunk 2c2 + (r>>3)
            const int r = ln;
            const int rr = r & 7;
            const int trow = 8 * lq + ((rr < 4) ? 2 * rr : 2 * (rr - 4) + 1);
#pragma unroll
            for (int c2 = 0; c2 < C::NDT / 2; ++c2) {
                const int chunk = 2 * c2 + (r >> 3);
                const int2v w = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                    (LDS_AS int2v*)(vl + trow * C::RBV + 8 * chunk));
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int t = 2 * c2 + h;           // column tile = chunk
                    const int kb = t >> 1;              // its block
                    const half8 av = q4_dword_to_half8((uint32_t)w[h]);
                    const half8 bv = make_half8(ps[kb][0], ps[kb][1], ps[kb][2], ps[kb][3]);
                    oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, oacc[t], 0, 0, 0);
                }
            }
        } else if constexpr (TV == T_Q8) {
            // column tile t = chunks 2t, 2t+1; lane r addresses row 8*lq + r/2, chunk 2t + (r&1)
            const int r = ln;
            const int trow = 8 * lq + (r >> 1);
#pragma unroll
            for (int t = 0; t < C::NDT; ++t) {
                const int2v w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (LDS_AS int2v*)(vl + trow * C::RBV + 8 * (2 * t + (r & 1))));
                const half8 av = q8_dwords_to_half8((uint32_t)w[0], (uint32_t)w[1]);
                const int kb = t >> 1;
                const half8 bv = make_half8(ps[kb][0], ps[kb][1], ps[kb][2], ps[kb][3]);
                oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, oacc[t], 0, 0, 0);
            }
        } else {
            // column tile t = chunks 4t..4t+3 (4 halves each); two reads of 4 rows;
            // lane r addresses row 8*lq + 4*R + r/4, chunk 4t + (r&3)
            const int r = ln;
            const half8 bv = make_half8(pp[0], pp[1], pp[2], pp[3]);
#pragma unroll
            for (int t = 0; t < C::NDT; ++t) {
                uint32_t d[4];
#pragma unroll
                for (int R = 0; R < 2; ++R) {
                    const int trow = 8 * lq + 4 * R + (r >> 2);
                    const short4v w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (LDS_AS short4v*)(vl + trow * C::RBV + 8 * (4 * t + (r & 3))));
                    const u32x2 u = __builtin_bit_cast(u32x2, w);
                    d[2 * R] = u[0];
                    d[2 * R + 1] = u[1];
                }
                const half8 av = make_half8(d[0], d[1], d[2], d[3]);
                oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, oacc[t], 0, 0, 0);
            }
        }
    };

    // ---- main loop over this wave's tiles, double-buffered
    uint32_t kA[2][C::KDW], kB[2][C::KDW];
    int it = wave;
    if (it < ntiles) issue(it, kA, 0);
    while (it < ntiles) {
        const int nx = it + WAVES;
        if (nx < ntiles) {
            wait_lgkm0();
            issue(nx, kB, 1);
            wait_vmcnt<C::TILE_VM>();
        } else {
            wait_vmcnt<0>();
        }
        compute(it, kA, 0);
        it = nx;
        if (it >= ntiles) break;
        const int nx2 = it + WAVES;
        if (nx2 < ntiles) {
            wait_lgkm0();
            issue(nx2, kA, 0);
            wait_vmcnt<C::TILE_VM>();
        } else {
            wait_vmcnt<0>();
        }
        compute(it, kB, 1);
        it = nx2;
    }

    // ---- merge the four waves: (m, l, O) per head through LDS
    const float l_head = xsum4(l_part);
    __syncthreads();
    float* mw = reinterpret_cast<float*>(smem);           // [WAVES][16]
    float* lw = mw + WAVES * 16;                          // [WAVES][16]
    float* ow = lw + WAVES * 16;                          // [WAVES][G][D]
    if (lq == 0) {
        mw[wave * 16 + ln] = m_ref;
        lw[wave * 16 + ln] = l_head;
    }
    if (ln < G) {
#pragma unroll
        for (int t = 0; t < C::NDT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * lq + i;
                int d;
                if constexpr (TV == T_Q4) d = 32 * (t >> 1) + 8 * (t & 1) + (m >> 1) + 16 * (m & 1);
                else d = 16 * t + m;
                ow[(wave * G + ln) * D + d] = oacc[t][i];
            }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += NT) {
        const int n = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, mw[w * 16 + n]);
        float lsum = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float f = exp2f(mw[w * 16 + n] - M);   // exp2(-inf) = 0 for idle waves
            lsum += f * lw[w * 16 + n];
            o += f * ow[(w * G + n) * D + d];
        }
        po[n * ho_stride + d] = o / lsum;
        if (d == 0) pl[(int64_t)n * a.max_splits] = (M + log2f(lsum)) * 0.69314718055994531f;
    }
}

template <int TK, int TV, int D>
constexpr bool cfg_valid() { return Cfg<TK, TV, D>::VALID; }

template <int TK, int TV, int D>
size_t lds_bytes(int G)
{
    using C = Cfg<TK, TV, D>;
    const size_t stage = (size_t)WAVES * C::WAVE_LDS;
    const size_t merge = sizeof(float) * ((size_t)WAVES * 32 + (size_t)WAVES * G * D);
    return stage > merge ? stage : merge;
}

template <int TK, int TV, int D>
hipError_t launch3(const DecodeArgs& a, hipStream_t s)
{
    if constexpr (!Cfg<TK, TV, D>::VALID) {
        return hipErrorInvalidConfiguration;
    } else {
        dim3 grid(a.max_splits, a.Hkv, a.B);
        const size_t lds = lds_bytes<TK, TV, D>(a.G);
        if (lds > 64 * 1024) {
            const hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void*>(&decode_mfma_kernel<TK, TV, D>),
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL((decode_mfma_kernel<TK, TV, D>), grid, dim3(NT), lds, s, a);
        return hipGetLastError();
    }
}

template <int TK, int TV>
hipError_t launch2(const DecodeArgs& a, hipStream_t s)
{
    switch (a.D) {
    case 128: return launch3<TK, TV, 128>(a, s);
    case 256: return launch3<TK, TV, 256>(a, s);
    default: return hipErrorInvalidConfiguration;
    }
}

template <int TK>
hipError_t launch1(const DecodeArgs& a, hipStream_t s)
{
    switch (a.tv) {
    case T_F16: return launch2<TK, T_F16>(a, s);
    case T_Q8: return launch2<TK, T_Q8>(a, s);
    default: return launch2<TK, T_Q4>(a, s);
    }
}

}  // namespace

bool decode_mfma_supports(const DecodeArgs& a)
{
    // head_dim 512 needs more registers than the kernel can hold without
    // spilling; it stays on the vector-ALU kernel
    if (a.D != 128 && a.D != 256) return false;
    if (a.G < 1 || a.G > 16) return false;
    // LDS: staging buffers of the four waves, or the merge area if larger
    size_t need = 0;
    switch (a.tk * 3 + a.tv) {
#define KVQ_CASE(TKV, TVV)                                                               \
    case TKV * 3 + TVV:                                                                  \
        if (a.D == 128) { if (!cfg_valid<TKV, TVV, 128>()) return false; need = lds_bytes<TKV, TVV, 128>(a.G); } \
        else if (a.D == 256) { if (!cfg_valid<TKV, TVV, 256>()) return false; need = lds_bytes<TKV, TVV, 256>(a.G); } \
        else { return false; } \
        break;
        KVQ_CASE(0, 0) KVQ_CASE(0, 1) KVQ_CASE(0, 2)
        KVQ_CASE(1, 0) KVQ_CASE(1, 1) KVQ_CASE(1, 2)
        KVQ_CASE(2, 0) KVQ_CASE(2, 1) KVQ_CASE(2, 2)
#undef KVQ_CASE
    default: return false;
    }
    return need <= 160 * 1024;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s)
{
    switch (a.tk) {
    case T_F16: return launch1<T_F16>(a, s);
    case T_Q8: return launch1<T_Q8>(a, s);
    default: return launch1<T_Q4>(a, s);
    }
}

}  // namespace kvq
