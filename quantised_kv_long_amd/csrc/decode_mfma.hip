// decode_mfma.hip -- split-KV decode attention with both contractions on the
// CDNA4 matrix cores (HAL #582 "per-layer KV compression study", section 3b
// finding 2 and section 5 P0: the quant reader is given the same matrix-core
// route as f16 and reads the raw blocks in registers; section 5 P2: per-region
// partials merged by an exact log-sum-exp combine).
//
// One workgroup (4 wave64) per (sequence, KV head, split); each wave walks its
// own 32-row tiles of the split (tiles w, w+4, ...) with a private LDS buffer,
// so waves never wait for each other until the final merge.  The global loads
// of a wave's next tile are issued before its current tile is computed.
//
// Codes enter the matrix cores as fp16 *subnormals*: the bit pattern of a
// nibble n (or of a byte u = code + 128) in the low bits of an fp16 is the
// value n * 2^-24, exact, and one AND (or one byte permute) builds two of them.
// The offset (8 for q4_0, 128 for q8_0) is removed exactly once per block:
//   QK  : the MFMA accumulator starts at -offset * 2^-24 * sum(q over the block);
//   PV  : one extra MFMA per block and tile accumulates offset * 2^-24 * sum(P'),
//         subtracted at the end.
// The 2^24 is applied once to the scores and once to the final output.
//
// Per 32-row tile:
//   QK^T as S^T = K * Q^T with v_mfma_f32_16x16x32_f16: A = 16 K rows x 32
//     values of one 32-value block, B = the GQA group's Q (16 columns, G
//     used).  One MFMA per block; its fp32 result is multiplied by the row's
//     block scale (exact products, fp32 sums).  K goes straight from HBM to
//     registers with coalesced 16-byte loads; for q8_0 / q4_0 a 4x4 exchange
//     between the four 16-lane rows (v_permlane32_swap / v_permlane16_swap)
//     turns "lane row q holds block q" into "lane row q holds a quarter of
//     every block" (f16 rows are loaded in that layout directly).
//   online softmax in fp32, log2 domain; the running maximum is only moved
//     when a score exceeds it by more than 2^8 (exact either way: every
//     partial sum is kept relative to the same reference), so rescaling the
//     accumulators is rare.
//   PV as O^T = V^T * P'^T: V rows are loaded with coalesced 16-byte loads,
//     written to the wave's LDS buffer and read back transposed
//     (ds_read_b64_tr_b4 / _b8 / _b16) so each lane holds one value column
//     for 8 rows.  The V block scale is folded into P (P' = p * scale per row
//     and block, fp16), since every 16-column MFMA tile lies inside one block.
//   Block scales are kept in LDS transposed ([block][row]) so the per-row
//   scales a lane needs are contiguous.
// The four waves' (max, sum, O) are merged through LDS into one normalised
// partial per (head, split).
#include <math.h>

#include "kvq_internal.hpp"
#include "kvq_quant.hpp"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int WAVES = 4;
constexpr int TT = 32;                 // rows per tile
constexpr float TAU = 8.0f;            // lazy rescale threshold, log2 units
constexpr float TWO24 = 16777216.0f;   // 2^24
constexpr float TWOM24 = 1.0f / 16777216.0f;
constexpr int VMCNT0 = 0x0F70;         // s_waitcnt vmcnt(0) (expcnt, lgkmcnt unconstrained)
// Per-workgroup timeline points: empty in the library.  The timeline probe
// build defines KVQ_TL to record the workgroup's clock at its start (0), after
// wave 0's last tile (1), at its end (2) and, in the four-wave merge, once
// every wave's loop is done (3) and once the merge area is written (4).
#ifndef KVQ_TL
#define KVQ_TL(point)
#endif
// Build-time knobs of the load ring (the defaults are the measured best):
// register sets of the quantised head_dim-128 ring, of the head_dim 256/512
// ring (quantised rows; fp16 rows), and the waves per SIMD a head_dim 256/512
// instance is built for (1 lets it use up to 512 registers).
#ifndef KVQ_RING
#define KVQ_RING 2
#endif
#ifndef KVQ_RING_WIDE
#define KVQ_RING_WIDE 2
#endif
#ifndef KVQ_RING_WIDE_F16
#define KVQ_RING_WIDE_F16 1
#endif
#ifndef KVQ_WPE_WIDE
#define KVQ_WPE_WIDE 2
#endif

__host__ __device__ constexpr int rb(int t, int D) { return data_row_bytes(t, D); }

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ half8 make_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    u32x4 u = {a, b, c, d};
    return __builtin_bit_cast(half8, u);
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

// 8 nibbles of one dword as fp16 subnormals, element order [nib0, nib4, nib1,
// nib5, nib2, nib6, nib3, nib7] (one AND per pair, one shift for all): the
// even pairs as nibble * 2^-24, the odd pairs ([nib1, nib5], [nib3, nib7])
// left in bits 4-7 of their halves, i.e. 16 * nibble * 2^-24 (still exact);
// the other operand of the product holds those slots divided by 16.
__device__ __forceinline__ half8 q4_sub8x(uint32_t w)
{
    const uint32_t M = 0x000F000Fu, M4 = 0x00F000F0u;
    const uint32_t w8 = w >> 8;
    return make_half8(w & M, w & M4, w8 & M, w8 & M4);
}

// 8 signed bytes (two dwords) as fp16 subnormals of (byte + 128) * 2^-24, in
// byte order.  v_perm_b32 selector 0x0C produces a zero byte.
__device__ __forceinline__ half8 q8_sub8(uint32_t w0, uint32_t w1)
{
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    return make_half8(__builtin_amdgcn_perm(u0, u0, 0x0C010C00u), __builtin_amdgcn_perm(u0, u0, 0x0C030C02u),
                      __builtin_amdgcn_perm(u1, u1, 0x0C010C00u), __builtin_amdgcn_perm(u1, u1, 0x0C030C02u));
}

// 8 unsigned bytes (two dwords) as fp16 subnormals of byte * 2^-24, in byte
// order.
__device__ __forceinline__ half8 u8_sub8(uint32_t w0, uint32_t w1)
{
    return make_half8(__builtin_amdgcn_perm(w0, w0, 0x0C010C00u), __builtin_amdgcn_perm(w0, w0, 0x0C030C02u),
                      __builtin_amdgcn_perm(w1, w1, 0x0C010C00u), __builtin_amdgcn_perm(w1, w1, 0x0C030C02u));
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

// --------------------------------------------------------------- the kernel

template <int TK, int TV, int D>
struct Cfg {
    // head_dim 256 / 512: the two / four waves of a workgroup walk the same
    // tiles, each owning one 128-column slice of the head dimension (partial
    // scores are summed through LDS); otherwise the four waves each walk their
    // own tiles over the full head dimension
    static constexpr int DS = D == 512 ? 4 : (D == 256 ? 2 : 1);   // waves sharing a tile
    static constexpr int WV = DS > 1 ? DS : WAVES;                   // waves per workgroup
    static constexpr int NTH = 64 * WV;                              // threads per workgroup
    static constexpr int DW = D / DS;              // head-dim slice of a wave
    static constexpr int NB = DW / 32;             // blocks per slice
    static constexpr int NBG = DW / 128;           // groups of 4 blocks
    static constexpr int NB_ROW = D / 32;          // blocks per row
    static constexpr int RBK = rb(TK, DW);         // bytes of a row's slice
    static constexpr int RBV = rb(TV, DW);
    static constexpr int RBK_ROW = rb(TK, D);      // bytes of a row (row stride)
    static constexpr int RBV_ROW = rb(TV, D);
    // storage-type traits: 4-bit low codes (the q4_0 family), high bits per
    // code (q5: 1, q6: 2, after all of a row's nibbles), a block minimum (q4_1,
    // q5_1: value = d * code + m), fp16 scale-plane entries per block
    static constexpr bool KNIB = TK == T_Q4 || TK == T_Q4_1 || TK == T_Q5_0 || TK == T_Q5_1 || TK == T_Q6_0;
    static constexpr int KHB = (TK == T_Q5_0 || TK == T_Q5_1) ? 1 : (TK == T_Q6_0 ? 2 : 0);
    static constexpr bool KMIN = TK == T_Q4_1 || TK == T_Q5_1;
    static constexpr int SPBK = scales_per_block(TK);
    static constexpr int VHB = (TV == T_Q5_0 || TV == T_Q5_1) ? 1 : (TV == T_Q6_0 ? 2 : 0);
    static constexpr bool VMIN = TV == T_Q4_1 || TV == T_Q5_1;
    static constexpr int SPBV = scales_per_block(TV);
    // V rows of the further types (q4_1, q5_0, q5_1, q6_0) are staged in LDS
    // as one unsigned code byte per value and take the byte route of PV
    static constexpr bool VBYTES = TV == T_Q4_1 || TV == T_Q5_0 || TV == T_Q5_1 || TV == T_Q6_0;
    static constexpr bool NEWT = VBYTES || TK == T_Q4_1 || TK == T_Q5_0 || TK == T_Q5_1 || TK == T_Q6_0;
    // LDS row stride of a staged V row (slice): its bytes plus 16, so that
    // the rows one transposed read gathers (16 rows, 16 bytes each for the
    // 4- and 8-bit codes) fall in different banks; unpadded, rows 64, 128 or
    // 256 bytes apart share banks and the reads conflict 4- to 8-fold
    static constexpr int RBV_LDS = (VBYTES ? DW : RBV) + 16;
    static constexpr int VCH = RBV / 16;                               // 16-byte chunks of a V row (slice)
    static constexpr int KU = KNIB ? 1 : (TK == T_Q8 ? 2 : 4);         // dwords per lane per block
    static constexpr int KDW = 4 * KU * NBG;                           // K code dwords per lane per subtile
    static constexpr int KHW = KHB * NB;                               // K high-bit dwords of a row (slice)
    // a row of the 4-bit-code types holds the D/2 nibble bytes of all its
    // blocks, then (q5, q6) the high-bit words of all its blocks: slice w's
    // codes start w * DW/2 bytes in, its high bits D/2 + w * NB * 4 * KHB
    // bytes in; the other types' slices are contiguous (w * RBK)
    static constexpr int KSL = KNIB ? DW / 2 : RBK;                   // code bytes before slice 1 (K)
    static constexpr int VSL = VBYTES ? DW / 2 : RBV;                 // the same for V
    static constexpr int BBK = KNIB ? 16 : RBK / NB;                   // code bytes of a block (K row)
    static constexpr int V_BYTES = TT * RBV_LDS;                       // V tile bytes in LDS (slice)
    static constexpr int V_LOADS = VBYTES ? 0 : TT * RBV / 1024;       // 16-byte loads per lane
    // byte route: one (row, block) unit per lane and load: 16 nibble bytes
    // plus the block's high-bit words
    static constexpr int V_UNITS = VBYTES ? TT * NB / 64 : 0;
    static constexpr int V_DW = VBYTES ? V_UNITS * (4 + VHB) : 4 * V_LOADS;
    static constexpr int K_SCALE = TK != T_F16;
    static constexpr int V_SCALE = TV != T_F16;
    static constexpr int SK_BYTES = TT * 2 * NB * SPBK;                // K scale tile (slice)
    static constexpr int SV_BYTES = TT * 2 * NB * SPBV;
    static constexpr int SK_LOADS = SK_BYTES / 256;                    // 4-byte loads per lane
    static constexpr int SV_LOADS = SV_BYTES / 256;
    static constexpr int S_DW = SK_LOADS + SV_LOADS > 0 ? SK_LOADS + SV_LOADS : 1;
    static constexpr int KS_OFF = V_BYTES;
    static constexpr int VS_OFF = V_BYTES + SK_BYTES;
    static constexpr int BUF = V_BYTES + SK_BYTES + SV_BYTES;
    static constexpr int NDT = DW / 16;                                // PV output tiles
    // register sets of the load ring: two (a third, where it fits in 256
    // registers, measured slower), one where a slice shared by several waves
    // has f16 rows (their registers do not fit twice)
    static constexpr int NSET = DW == 128 && (DS == 1 || (TK != T_F16 && TV != T_F16))
                                    ? (DS == 1 && TK != T_F16 && TV != T_F16 ? KVQ_RING : (DS > 1 ? KVQ_RING_WIDE : 2))
                                    : (DS > 1 ? KVQ_RING_WIDE_F16 : 1);
    static constexpr int WPE = DS > 1 ? KVQ_WPE_WIDE : 2;              // waves per SIMD the build targets
    static constexpr int SX_FLOATS = DS > 1 ? 2 * WV * 64 * 8 : 1;     // partial-score exchange
    static constexpr float KOFF = TK == T_Q4 ? 8.0f : TK == T_Q8 ? 128.0f : TK == T_Q5_0 ? 16.0f
                                : TK == T_Q6_0 ? 32.0f : 0.0f;
    // the V code offset as an fp16 subnormal pair (0: no offset, min types)
    static constexpr uint32_t VOFF_BITS = TV == T_Q4 ? 0x00080008u : TV == T_Q8 ? 0x00800080u
                                        : TV == T_Q5_0 ? 0x00100010u : TV == T_Q6_0 ? 0x00200020u : 0u;
    // a decode step's new row merged from registers (the base types: each
    // aligned half-wave quantises NEW_IT of the row's 2 * NB_ROW blocks)
    static constexpr bool NEWROW = !NEWT;
    static constexpr int NEW_IT = (2 * NB_ROW * 32 + NTH - 1) / NTH;   // new-row blocks per half-wave
    static constexpr bool VALID = (VBYTES || ((TT * RBV) % 1024 == 0 && 64 % VCH == 0)) && SK_BYTES % 256 == 0 &&
                                  SV_BYTES % 256 == 0 &&
                                  (!VBYTES || (TT * NB) % 64 == 0) && V_DW <= (DW == 128 ? 32 : 64) &&
                                  WV * BUF <= 64 * 1024;
};

// Bytes of the four-wave merge area: per wave and score column the running
// max and sum, the V offset sums per block, and the nc x D accumulators of
// every wave (nc = query tokens x heads per KV head).
template <int TK, int TV, int D>
__host__ __device__ constexpr size_t merge_lds_bytes(int nc)
{
    return Cfg<TK, TV, D>::DS > 1 ? 0
                                  : sizeof(float) * ((size_t)WAVES * 16 * 2 + (size_t)WAVES * 16 * (D / 32) +
                                                     (size_t)WAVES * nc * D);   // (DS == 1: WV = WAVES)
}

// Every instance is built for two waves per SIMD (at most 256 registers):
// each wave holds a 128-column slice of the head dimension.
// The work of one workgroup: split s of (sequence blockIdx.z, KV head
// blockIdx.y).  LDS: lds_a (WAVES * BUF bytes: one buffer per wave, the V
// rows of the current tile, then the K and V scale tiles transposed to
// [block][row]), lds_sx (the partial-score exchange of a 512-wide head) and
// lds_merge (the four-wave merge area of whole rows, merge_lds_bytes: its
// own memory, so a wave writes its part as soon as its last tile is done).
// MQ: several query tokens per sequence (a.nq > 1); a separate instance, so
// that the single-token kernels carry none of its per-column index arithmetic
// One 32-value block of a new row, quantised by the 32 lanes of an aligned
// half-wave (j = lane & 31) into row `row` of plane P (a row of D values).
template <int T, int D>
__device__ __forceinline__ void write_block_lanes_d(const uint16_t* src, const Plane& P, int64_t row, int blk, int j)
{
    if constexpr (T == T_F16 || T == T_Q8 || T == T_Q4)
        quantize_block_lanes<T>(src, P.data + row * rb(T, D) + blk * rb(T, 32), P.scales + row * (D / 32) + blk, j);
    else
        quantize_block_ext_lanes<T>(src, P.data + row * rb(T, D), P.scales + row * (D / 32) * scales_per_block(T),
                                    blk, D, j);
}

template <int TK, int TV, int D, bool MQ, bool SHORT = false>
__device__ __forceinline__ void decode_wg(const DecodeArgs& a, const int32_t* const seq_lens, const int s,
                                          uint8_t* const lds_a, float* const lds_sx, uint8_t* const lds_merge,
                                          float* const lds_new)
{
    using C = Cfg<TK, TV, D>;
    const int g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index is uniform across a wave: held in a scalar register, the
    // tile loop and the tile base addresses are scalar work
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lq = lane >> 4;       // column / lane row of the 16x16 layouts
    const int G = a.G;
    // score columns: NQ query tokens x G heads; column c is token c / G (the
    // last NQ rows of the sequence are the query tokens: token i sees rows
    // [0, L - NQ + 1 + i)) and head h0 + c % G
    const int NQ = MQ ? a.nq : 1, NC = NQ * G;
    const int L = seq_lens[b];                      // (seq_lens == a.seq_lens)
    // the plane arguments are read together with the length (pinned here, or
    // the compiler loads them only after the test for an empty split below)
    asm volatile("" ::"s"(a.k.data), "s"(a.v.data), "s"(a.k.scales), "s"(a.v.scales));
    asm volatile("" ::"s"(a.k.seq_stride), "s"(a.k.head_stride), "s"(a.v.seq_stride), "s"(a.v.head_stride));
    asm volatile("" ::"s"(a.q), "s"(a.k_new), "s"(a.part_o), "s"(a.part_lse));
    asm volatile("" ::"s"(a.G), "s"(a.Hq), "s"(a.Hkv), "s"(a.max_splits));
    const int t_begin = s * a.split_tokens;
    const int t_end_all = min(t_begin + a.split_tokens, L);
    // Decode step with one new token (NEWROW, the base types): the workgroup
    // whose split holds row L-1 leaves that row out of its tiles, quantises
    // the new row into it while its first tiles are loading, and merges the
    // row's decoded values as one more term: no load reads the stored row.
    constexpr bool NEWROW_OK = C::NEWROW && !MQ;
    const bool newrow = NEWROW_OK && a.k_new != nullptr && t_end_all == L;
    const int Lr = newrow ? L - 1 : L;             // rows the tiles read
    const int t_end = min(t_begin + a.split_tokens, Lr);
    const int h0 = g * G;
    const int64_t ho_stride = (int64_t)a.max_splits * D;
    const int64_t HQT = (int64_t)NQ * a.Hq;        // rows of the partials' head axis
    float* po = a.part_o + (((int64_t)b * HQT + h0) * a.max_splits + s) * D;
    float* pl = a.part_lse + ((int64_t)b * HQT + h0) * a.max_splits + s;
    // partial row of column c, relative to (b, h0)
    auto crow = [&](int c) -> int64_t { return MQ ? (int64_t)(c / G) * a.Hq + c % G : (int64_t)c; };

    const int64_t krow0 = (int64_t)b * a.k.seq_stride + (int64_t)g * a.k.head_stride;
    const int64_t vrow0 = (int64_t)b * a.v.seq_stride + (int64_t)g * a.v.head_stride;
    const int wsl = C::DS > 1 ? wave : 0;          // this wave's head-dim slice
    // Each plane of (sequence b, KV head g) is read through a buffer resource
    // that covers its rows [0, L): a load of a row at or past L returns zeros
    // without a memory access, so a split's last tile and a prefetch past a
    // wave's last tile need neither a clamp nor a branch, and every tile's
    // loads are one scalar tile offset plus per-lane offsets fixed for the
    // whole loop.  (Offsets are 32-bit: rows below max_seq_len span < 2^31
    // bytes per plane.)
    auto make_rsrc = [](const void* p, int64_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k.data + krow0 * C::RBK_ROW, (int64_t)Lr * C::RBK_ROW);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v.data + vrow0 * C::RBV_ROW, (int64_t)Lr * C::RBV_ROW);
    constexpr int SRK = 2 * C::NB_ROW * C::SPBK, SRV = 2 * C::NB_ROW * C::SPBV;   // scale-row bytes
    const __amdgpu_buffer_rsrc_t rks =
        make_rsrc(C::K_SCALE ? (const void*)(a.k.scales + krow0 * C::NB_ROW * C::SPBK) : (const void*)a.k.data,
                  C::K_SCALE ? (int64_t)Lr * SRK : 0);
    const __amdgpu_buffer_rsrc_t rvs =
        make_rsrc(C::V_SCALE ? (const void*)(a.v.scales + vrow0 * C::NB_ROW * C::SPBV) : (const void*)a.v.data,
                  C::V_SCALE ? (int64_t)Lr * SRV : 0);
    // a split at or past ceil(L / split_tokens) holds no row: the merge never
    // reads its partials, so nothing is written.  (Tested after the resource
    // set-up, so that the argument loads it needs go out with the length's.)
    if (t_begin >= t_end_all) return;

    // ---- decode step with the new tokens: the workgroup whose split holds
    //      row L-1 (multi-query: each workgroup whose split holds some of the
    //      rows [L-NQ, L)) first quantises the new K and V rows of its KV head
    //      into those rows (the same block quantiser as kvq_quantize_append),
    //      then makes them visible to its own loads
    if constexpr (MQ) {
        const int r_lo = max(L - NQ, t_begin);
        const int nrows = t_end - r_lo;
        if (a.k_new != nullptr && nrows > 0) {
            // nrows * 2*NB_ROW blocks (per row: K then V), one aligned
            // half-wave of 32 lanes per block
            for (int it = tid >> 5; it < nrows * 2 * C::NB_ROW; it += C::NTH / 32) {
                const int r = r_lo + it / (2 * C::NB_ROW);
                const int blk2 = it % (2 * C::NB_ROW);
                const bool isv = blk2 >= C::NB_ROW;
                const int blk = isv ? blk2 - C::NB_ROW : blk2;
                const int i = r - (L - NQ);                  // new row i of this sequence
                const uint16_t* src =
                    (isv ? a.v_new : a.k_new) + (((int64_t)b * NQ + i) * a.Hkv + g) * D + 32 * blk;
                const int64_t row = (isv ? vrow0 : krow0) + r;
                if (isv) write_block_lanes_d<TV, D>(src, a.v, row, blk, tid & 31);
                else write_block_lanes_d<TK, D>(src, a.k, row, blk, tid & 31);
            }
            __builtin_amdgcn_s_waitcnt(VMCNT0);
            __syncthreads();
        }
    } else if constexpr (C::NEWT) {
        if (a.k_new != nullptr && t_end == L) {
            // 2*NB_ROW blocks (K then V), one aligned half-wave of 32 lanes
            // per block
            for (int blk2 = tid >> 5; blk2 < 2 * C::NB_ROW; blk2 += C::NTH / 32) {
                const bool isv = blk2 >= C::NB_ROW;
                const int blk = isv ? blk2 - C::NB_ROW : blk2;
                const uint16_t* src = (isv ? a.v_new : a.k_new) + ((int64_t)b * a.Hkv + g) * D + 32 * blk;
                const int64_t row = (isv ? vrow0 : krow0) + (L - 1);
                if (isv) write_block_lanes_d<TV, D>(src, a.v, row, blk, tid & 31);
                else write_block_lanes_d<TK, D>(src, a.k, row, blk, tid & 31);
            }
            // the row is read back only by this workgroup, whose loads of that
            // tile are issued after the barrier: the stores must be complete
            // (acknowledged by L2) first; no other workgroup reads these lines
            __builtin_amdgcn_s_waitcnt(VMCNT0);
            __syncthreads();
        }
    }

    // ---- Q as the B operand of S^T = K Q^T: column ln = head, lane row lq
    //      holds k-slots 8*lq .. 8*lq+7 of each block, in the element order
    //      the K codes arrive in (q8_0 / f16: elements 8*lq .. 8*lq+7; q4_0:
    //      4*lq + {0, 2, 16, 18, 1, 3, 17, 19}, the nibble order of one dword)
    half8 qop[C::NB];
    floatx4 kbias[C::NB];
    float kmq[C::KMIN ? C::NB : 1];
    // Q is loaded before the first tiles (load_q) and formed into operands
    // after they are issued (init_q), so the tiles' loads stay in flight while
    // it is waited for
    uint32_t qraw[C::NB][4];
    auto load_q = [&]() {
        const int c = min(ln, NC - 1);
        const uint16_t* qh = MQ ? a.q + (((int64_t)b * NQ + c / G) * a.Hq + h0 + c % G) * D + wsl * C::DW
                                : a.q + ((int64_t)b * a.Hq + h0 + c) * D + wsl * C::DW;
#pragma unroll
        for (int kb = 0; kb < C::NB; ++kb) {
            if constexpr (C::KNIB) {
                const u32x2 ra = *reinterpret_cast<const u32x2*>(qh + 32 * kb + 4 * lq);
                const u32x2 rb = *reinterpret_cast<const u32x2*>(qh + 32 * kb + 4 * lq + 16);
                qraw[kb][0] = ra[0];
                qraw[kb][1] = ra[1];
                qraw[kb][2] = rb[0];
                qraw[kb][3] = rb[1];
            } else {
                const u32x4 r = *reinterpret_cast<const u32x4*>(qh + 32 * kb + 8 * lq);
#pragma unroll
                for (int c = 0; c < 4; ++c) qraw[kb][c] = r[c];
            }
        }
    };
    auto init_q = [&]() {
        const half2v one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int kb = 0; kb < C::NB; ++kb) {
            uint32_t w[4];
            if constexpr (C::KNIB) {
                w[0] = __builtin_amdgcn_perm(qraw[kb][1], qraw[kb][0], 0x05040100u);
                w[1] = __builtin_amdgcn_perm(qraw[kb][3], qraw[kb][2], 0x05040100u);
                w[2] = __builtin_amdgcn_perm(qraw[kb][1], qraw[kb][0], 0x07060302u);
                w[3] = __builtin_amdgcn_perm(qraw[kb][3], qraw[kb][2], 0x07060302u);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) w[c] = qraw[kb][c];
            }
            float part = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (ln >= NC) w[c] = 0;
                part = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, w[c]), one2, part, false);
            }
            if constexpr (C::KNIB && C::KHB == 0) {
                // (q4_sub8x codes: slots 2, 3, 6, 7 hold 16 * code)
                w[1] = pk_mul_h(w[1], 0x2C002C00u);
                w[3] = pk_mul_h(w[3], 0x2C002C00u);
            }
            qop[kb] = make_half8(w[0], w[1], w[2], w[3]);
            // the accumulator's start removes the code offset exactly once
            const float qsum = xsum4(part);
            const float bias = -C::KOFF * TWOM24 * qsum;
            kbias[kb] = floatx4{bias, bias, bias, bias};
            // block minimum m: the score gains m * sum(q over the block), in
            // the MFMA sums' units (2^-24)
            if constexpr (C::KMIN) kmq[kb] = qsum * TWOM24;
        }
    };

    // scores: fp32 MFMA sums times block scale, then softmax scale * log2(e)
    // (and 2^24 for the subnormal codes)
    const float cK = a.scale_log2 * (C::K_SCALE ? TWO24 : 1.0f);

    uint8_t* const wbuf = lds_a + wave * C::BUF;
    floatx4 oacc[C::NDT];
    floatx4 bacc[C::NB];
#pragma unroll
    for (int i = 0; i < C::NDT; ++i) oacc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < C::NB; ++i) bacc[i] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    // running maximum starts at a finite floor: a column can see no row at all
    // in a wave (a query token's causal limit lies before the wave's tiles),
    // and its weights must then be exp2(-inf - floor) = 0, not NaN
    constexpr float M_FLOOR = -1.0e30f;
    float m_ref = MQ ? M_FLOOR : -INFINITY, l_part = 0.0f;
    // rows this lane's column sees: [0, c_end), the split's end included;
    // below t_lim every column sees every row of the split
    const int c_end = MQ ? min(t_end, L - NQ + 1 + min(ln, NC - 1) / G) : t_end;
    const int t_lim = MQ ? min(t_end, L - NQ + 1) : t_end;

    const int ntiles = (t_end - t_begin + TT - 1) / TT;
    // Every prefetch is issued on every path, so the compiler's wait counts
    // are exact and a wait never drains the loads issued after the one it
    // needs: a prefetch past this wave's last tile reads only out-of-range
    // rows (zeros, no memory access), and its registers are never read.
    // First row of tile `it`; a tile past the wave's last one reads rows from
    // Lr on, which are all out of range.
    auto tile_row = [&](int it) -> int { return it < ntiles ? t_begin + it * TT : Lr; };
    // K row of subtile j read by this lane (tile-relative): rows of the A
    // operand are ordered so that the score layout gives lane row lq the rows
    // 8*lq .. 8*lq+7 of the tile.  Lane (ln, lq) needs k-slots 8*lq .. 8*lq+7
    // of every block: its quarter lq of the block (QB bytes).
    //   f16 (QB = 16): each lane loads its quarters directly, 16 bytes each.
    //   q8_0 / q4_0: 16-byte loads stay coalesced: lane row lq loads the whole
    //   of block 4*bg + lq (BB bytes), and a 4x4 exchange between lane rows
    //   (xpose4) then gives each lane row its quarter of every block.
    //   q5 / q6 high bits: every lane loads its row's high-bit words whole.
    constexpr int QB = 4 * C::KU;                  // bytes of a block quarter
    constexpr int BB = C::BBK;                     // code bytes of a block
    constexpr bool KDIRECT = C::KU == 4;
    constexpr int KR = C::KDW + C::KHW;            // K dwords per lane and row
    const int krow_rel0 = 8 * (ln >> 2) + (ln & 3);
    const uint32_t kpart = (uint32_t)(lq * (KDIRECT ? QB : BB));
    // Per-lane byte offsets inside a tile (the tile's first row is added per
    // tile).  V row chunks and scale words of a tile: 16-byte chunk k*64 +
    // lane of the slice is row c16 / (RBV/16), column c16 % (RBV/16); scale
    // word k*64 + lane is row c4 / wpr, word c4 % wpr (wpr: words per row of
    // the slice).  Whole rows (DS == 1) make one contiguous tile: offsets
    // 16*c16 and 4*c4.
    auto voff = [&](int k) -> uint32_t {
        const int c16 = k * 64 + lane;
        if constexpr (C::DS == 1) return (uint32_t)(16 * lane + 1024 * k);
        else return (uint32_t)((c16 / (C::RBV / 16)) * C::RBV_ROW + wsl * C::RBV + 16 * (c16 % (C::RBV / 16)));
    };
    auto soff = [&](int k, int spb, int srow) -> uint32_t {
        const int wpr = C::NB * spb / 2;
        const int c4 = k * 64 + lane;
        if constexpr (C::DS == 1) return (uint32_t)(4 * c4);
        else return (uint32_t)((c4 / wpr) * srow + wsl * C::NB * spb * 2 + 4 * (c4 % wpr));
    };
    const uint32_t krow_off[2] = {(uint32_t)(krow_rel0 * C::RBK_ROW + wsl * C::KSL),
                                  (uint32_t)((krow_rel0 + 4) * C::RBK_ROW + wsl * C::KSL)};
    // the slice's K high-bit words, relative to its codes
    const uint32_t khoff = (uint32_t)(D / 2 + wsl * (C::KHB * 4 * C::NB - C::KSL));

    // one K row's share of this lane (ro: the row's byte offset in the plane)
    auto load_k_row = [&](uint32_t ro, uint32_t (&x)[KR]) {
        if constexpr (C::KHB > 0) {
            // the slice's high-bit words, after the row's D/2 nibble bytes
#pragma unroll
            for (int u = 0; u < C::KHW / 4; ++u) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rk, ro + khoff + 16 * u, 0, 0);
#pragma unroll
                for (int c = 0; c < 4; ++c) x[C::KDW + 4 * u + c] = v[c];
            }
        }
        const uint32_t p = ro + kpart;
        if constexpr (KDIRECT) {
#pragma unroll
            for (int kb = 0; kb < C::NB; ++kb) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rk, p + kb * BB, 0, 0);
#pragma unroll
                for (int c = 0; c < 4; ++c) x[4 * kb + c] = v[c];
            }
        } else {
#pragma unroll
            for (int bg = 0; bg < C::NBG; ++bg)
#pragma unroll
                for (int u = 0; u < C::KU; ++u) {
                    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rk, p + bg * 4 * BB + 16 * u, 0, 0);
#pragma unroll
                    for (int c = 0; c < 4; ++c) x[(bg * C::KU + u) * 4 + c] = v[c];
                }
        }
    };

    // ---- global loads of tile `it` into registers: K rows in the MFMA layout
    //      (issue_k), and the V rows and scale rows (issue_vs) that stage()
    //      then copies to this wave's LDS buffer
    auto issue_k = [&](int it, uint32_t (&kr)[2][KR]) {
        const uint32_t tb = (uint32_t)tile_row(it) * C::RBK_ROW;
        load_k_row(tb + krow_off[0], kr[0]);
        load_k_row(tb + krow_off[1], kr[1]);
    };
    // scale words of a tile: the K and V scale planes have SPBK / SPBV fp16
    // entries per block (scale, then minimum)
    auto load_all_scales = [&](int t0, uint32_t (&sr)[C::S_DW]) {
        if constexpr (C::K_SCALE) {
            const uint32_t tb = (uint32_t)t0 * SRK;
#pragma unroll
            for (int k = 0; k < C::SK_LOADS; ++k)
                sr[k] = __builtin_amdgcn_raw_buffer_load_b32(rks, tb + soff(k, C::SPBK, SRK), 0, 0);
        }
        if constexpr (C::V_SCALE) {
            const uint32_t tb = (uint32_t)t0 * SRV;
#pragma unroll
            for (int k = 0; k < C::SV_LOADS; ++k)
                sr[C::SK_LOADS + k] = __builtin_amdgcn_raw_buffer_load_b32(rvs, tb + soff(k, C::SPBV, SRV), 0, 0);
        }
    };
    auto issue_vs = [&](int it, uint32_t (&vr)[C::V_DW], uint32_t (&sr)[C::S_DW]) {
        const int t0 = tile_row(it);
        if constexpr (C::VBYTES) {
            // unit k*64 + lane = (row u / NB, block u % NB): its 16 nibble
            // bytes and its high-bit words
#pragma unroll
            for (int k = 0; k < C::V_UNITS; ++k) {
                const int u = k * 64 + lane;
                const uint32_t ro = (uint32_t)(t0 + u / C::NB) * C::RBV_ROW;   // the row's start
                const u32x4 v =
                    __builtin_amdgcn_raw_buffer_load_b128(rv, ro + wsl * C::VSL + 16 * (u % C::NB), 0, 0);
#pragma unroll
                for (int c = 0; c < 4; ++c) vr[k * (4 + C::VHB) + c] = v[c];
                // the slice's high-bit words: D/2 + (slice block) * 4 * VHB
                const uint32_t vho = ro + D / 2 + 4 * C::VHB * (wsl * C::NB + u % C::NB);
                if constexpr (C::VHB == 1) {
                    vr[k * 5 + 4] = __builtin_amdgcn_raw_buffer_load_b32(rv, vho, 0, 0);
                } else if constexpr (C::VHB == 2) {
                    const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(rv, vho, 0, 0);
                    vr[k * 6 + 4] = h[0];
                    vr[k * 6 + 5] = h[1];
                }
            }
        } else {
            const uint32_t tb = (uint32_t)t0 * C::RBV_ROW;
#pragma unroll
            for (int k = 0; k < C::V_LOADS; ++k) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rv, tb + voff(k), 0, 0);
#pragma unroll
                for (int c = 0; c < 4; ++c) vr[4 * k + c] = v[c];
            }
        }
        load_all_scales(t0, sr);
    };

    // one (row, block) unit of a further type as 32 unsigned code bytes
    // (element j at byte j): the low nibbles (byte j of the block holds
    // elements j and j+16), plus the high bits moved to bit 4 of each byte
    auto unit_bytes = [&](const uint32_t* x, uint32_t (&o)[8]) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            o[m] = x[m] & 0x0F0F0F0Fu;               // elements 4m .. 4m+3
            o[m + 4] = (x[m] >> 4) & 0x0F0F0F0Fu;    // elements 16+4m .. 16+4m+3
        }
        if constexpr (C::VHB == 1) {
            // bit e of the word is bit 4 of element e: four bits to the four
            // bytes' bit 4 (the multiply spreads 4 bits 8 apart, no carries)
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint32_t f = __builtin_amdgcn_ubfe(x[4], 4 * m, 4);
                o[m] |= ((f * 0x00204081u) & 0x01010101u) << 4;
            }
        } else if constexpr (C::VHB == 2) {
            // bits 2e, 2e+1 of the 64-bit word are bits 4, 5 of element e:
            // the two-bit fields of four elements go to bits 4-5 of the four
            // bytes (even and odd fields spread separately, no carries)
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint32_t f = __builtin_amdgcn_ubfe(x[4 + (m >> 2)], 8 * (m & 3), 8);
                const uint32_t ev = ((f & 0x33u) * 0x1001u) & 0x00030003u;          // fields 0, 2 -> 0, 16
                const uint32_t od = (((f >> 2) & 0x33u) * 0x1001u) & 0x00030003u;   // fields 1, 3 -> 0, 16
                o[m] |= (ev | (od << 8)) << 4;
            }
        }
    };

    // ---- copy the staged V rows (natural order, [32 rows][row bytes]; the
    //      further types as code bytes) and the scale rows (transposed to
    //      [entry][32 rows], entry = block * SPB + (0: scale, 1: minimum)) to
    //      the wave's LDS buffer
    auto stage_scales = [&](const uint32_t* src, int spb, int nloads, uint16_t* st) {
        const int wpr = C::NB * spb / 2;
        for (int k = 0; k < nloads; ++k) {
            const int c4 = k * 64 + lane;
            const int tok = c4 / wpr, e = 2 * (c4 % wpr);
            st[e * TT + tok] = (uint16_t)(src[k] & 0xffff);
            st[(e + 1) * TT + tok] = (uint16_t)(src[k] >> 16);
        }
    };
    auto stage = [&](const uint32_t (&vr)[C::V_DW], const uint32_t (&sr)[C::S_DW]) {
        uint8_t* vb = wbuf;
        if constexpr (C::VBYTES) {
#pragma unroll
            for (int k = 0; k < C::V_UNITS; ++k) {
                const int u = k * 64 + lane;
                uint32_t o[8];
                unit_bytes(vr + k * (4 + C::VHB), o);
                uint8_t* dst = vb + (u / C::NB) * C::RBV_LDS + 32 * (u % C::NB);
                *reinterpret_cast<u32x4*>(dst) = u32x4{o[0], o[1], o[2], o[3]};
                *reinterpret_cast<u32x4*>(dst + 16) = u32x4{o[4], o[5], o[6], o[7]};
            }
        } else {
            // chunk k*64 + lane of the tile is row (k*64 + lane) / VCH, chunk
            // (k*64 + lane) % VCH (VCH divides 64)
            uint8_t* const vrow = vb + (lane / C::VCH) * C::RBV_LDS + 16 * (lane % C::VCH);
#pragma unroll
            for (int k = 0; k < C::V_LOADS; ++k) {
                const u32x4 v = {vr[4 * k], vr[4 * k + 1], vr[4 * k + 2], vr[4 * k + 3]};
                *reinterpret_cast<u32x4*>(vrow + k * (64 / C::VCH) * C::RBV_LDS) = v;
            }
        }
        if constexpr (C::K_SCALE)
            stage_scales(sr, C::SPBK, C::SK_LOADS, reinterpret_cast<uint16_t*>(vb + C::KS_OFF));
        if constexpr (C::V_SCALE)
            stage_scales(sr + C::SK_LOADS, C::SPBV, C::SV_LOADS, reinterpret_cast<uint16_t*>(vb + C::VS_OFF));
    };

    // ---- compute tile `it` whose K rows are in kr and V rows / scales in LDS
    auto compute = [&](int it, uint32_t (&kr)[2][KR], int next_it) {
        const int t0 = t_begin + it * TT;
        const uint8_t* vb = wbuf;
        const uint16_t* kst = reinterpret_cast<const uint16_t*>(vb + C::KS_OFF);
        const uint16_t* vst = reinterpret_cast<const uint16_t*>(vb + C::VS_OFF);

        // -- QK: S^T for the two 16-row subtiles; lane (ln, lq) reg i holds the
        //    score of row t0 + 8*lq + 4*j + i for head ln
        floatx4 sacc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            uint32_t* x = kr[j];
            if constexpr (!KDIRECT) {
                // lane row lq loaded all of block 4*bg + lq (dwords bg*4*KU +
                // [0, 4*KU)); afterwards it holds quarter lq of block 4*bg + w
                // at x[bg*4*KU + w*KU + v]
#pragma unroll
                for (int bg = 0; bg < C::NBG; ++bg) {
                    uint32_t* base = x + bg * 4 * C::KU;
#pragma unroll
                    for (int u = 0; u < C::KU; ++u)
                        xpose4(base[0 * C::KU + u], base[1 * C::KU + u], base[2 * C::KU + u],
                               base[3 * C::KU + u]);
                }
            }
            floatx4 cb[C::NB];
#pragma unroll
            for (int bg = 0; bg < C::NBG; ++bg) {
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4) {
                    const int kb = 4 * bg + kb4;
                    const uint32_t* q = x + bg * 4 * C::KU + kb4 * C::KU;
                    half8 av;
                    if constexpr (C::KHB > 0) {
                        // nibble pair k of the dword is elements (e0_k, e1_k) of
                        // quarter lq: e0 = 4lq + {0, 16, 1, 17}[k], e1 = e0 + 2;
                        // their high bits go to bits 4 and 20 (bit 4 of each half)
                        const uint32_t w = q[0];
                        uint32_t d[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const int e0 = 4 * lq + ((k & 1) ? 16 : 0) + (k >> 1);
                            uint32_t h0, h1;
                            if constexpr (C::KHB == 1) {
                                const uint32_t hw = x[C::KDW + kb];
                                h0 = __builtin_amdgcn_ubfe(hw, e0, 1);
                                h1 = __builtin_amdgcn_ubfe(hw, e0 + 2, 1);
                            } else {
                                // element e's two bits are bits 2e, 2e+1 of the
                                // block's 64-bit word (e0, e0 + 2 in one half)
                                const uint32_t hw = x[C::KDW + 2 * kb + (e0 >> 4)];
                                h0 = __builtin_amdgcn_ubfe(hw, 2 * (e0 & 15), 2);
                                h1 = __builtin_amdgcn_ubfe(hw, 2 * ((e0 + 2) & 15), 2);
                            }
                            d[k] = ((w >> (4 * k)) & 0x000F000Fu) | (h0 << 4) | (h1 << 20);
                        }
                        av = make_half8(d[0], d[1], d[2], d[3]);
                    } else if constexpr (C::KNIB) {
                        av = q4_sub8x(q[0]);
                    } else if constexpr (TK == T_Q8) {
                        av = q8_sub8(q[0], q[1]);
                    } else {
                        av = make_half8(q[0], q[1], q[2], q[3]);
                    }
                    cb[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, qop[kb], kbias[kb], 0, 0, 0);
                }
            }
            floatx4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (C::K_SCALE) {
                // block scales of this lane's four rows (8*lq + 4*j + i): four
                // contiguous fp16 values per block in the transposed tile
#pragma unroll
                for (int kb = 0; kb < C::NB; ++kb) {
                    const u32x2 sw =
                        *reinterpret_cast<const u32x2*>(kst + (kb * C::SPBK) * TT + 8 * lq + 4 * j);
                    // the element is copied out first: hipcc (clang) bit-casts
                    // a vector-element lvalue from the vector's first element
                    const half2v s01 = __builtin_bit_cast(half2v, (uint32_t)sw[0]);
                    const half2v s23 = __builtin_bit_cast(half2v, (uint32_t)sw[1]);
                    sc[0] = fmaf(cb[kb][0], (float)s01[0], sc[0]);
                    sc[1] = fmaf(cb[kb][1], (float)s01[1], sc[1]);
                    sc[2] = fmaf(cb[kb][2], (float)s23[0], sc[2]);
                    sc[3] = fmaf(cb[kb][3], (float)s23[1], sc[3]);
                    if constexpr (C::KMIN) {
                        // + m * sum(q over the block), m of each row
                        const u32x2 mw =
                            *reinterpret_cast<const u32x2*>(kst + (kb * 2 + 1) * TT + 8 * lq + 4 * j);
                        const half2v m01 = __builtin_bit_cast(half2v, (uint32_t)mw[0]);
                        const half2v m23 = __builtin_bit_cast(half2v, (uint32_t)mw[1]);
                        sc[0] = fmaf((float)m01[0], kmq[kb], sc[0]);
                        sc[1] = fmaf((float)m01[1], kmq[kb], sc[1]);
                        sc[2] = fmaf((float)m23[0], kmq[kb], sc[2]);
                        sc[3] = fmaf((float)m23[1], kmq[kb], sc[3]);
                    }
                }
            } else {
#pragma unroll
                for (int kb = 0; kb < C::NB; ++kb) sc += cb[kb];
            }
            sacc[j] = sc;
        }
        // the K registers are free: start loading the next tile's K rows
        issue_k(next_it, kr);

        if constexpr (C::DS > 1) {
            // each wave holds the scores over its head-dim slice: sum the
            // four in a fixed order, so every wave gets the same bits (one
            // barrier per tile; the two halves of lds_sx alternate by tile)
            float* mine = lds_sx + ((it & 1) * C::WV + wave) * 512 + lane * 8;
            *reinterpret_cast<floatx4*>(mine) = sacc[0];
            *reinterpret_cast<floatx4*>(mine + 4) = sacc[1];
            __syncthreads();
            floatx4 f0 = {0.0f, 0.0f, 0.0f, 0.0f}, f1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int w = 0; w < C::WV; ++w) {
                const float* theirs = lds_sx + ((it & 1) * C::WV + w) * 512 + lane * 8;
                f0 += *reinterpret_cast<const floatx4*>(theirs);
                f1 += *reinterpret_cast<const floatx4*>(theirs + 4);
            }
            sacc[0] = f0;
            sacc[1] = f1;
        }

        // -- online softmax (log2 domain)
        float sv[8];
        // the split's last tile, or a tile holding query tokens' rows: rows
        // past the split's end or the column's causal limit drop out
        const bool tail = t0 + TT > t_lim;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[4 * j + i] = sacc[j][i] * cK;
        if constexpr (C::NSET > 1) {
            if (tail) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (t0 + 8 * lq + e >= c_end) sv[e] = -INFINITY;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (tail && t0 + 8 * lq + e >= c_end) sv[e] = -INFINITY;
        }
        float mx = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
        if (__builtin_amdgcn_ballot_w64(mx > m_ref + TAU) != 0) {
            const float hmax = xmax4(mx);
            const float m_new = hmax > m_ref + TAU ? hmax : m_ref;
            const float al = exp2f(m_ref - m_new);
            l_part *= al;
#pragma unroll
            for (int t = 0; t < C::NDT; ++t) oacc[t] *= al;
#pragma unroll
            for (int t = 0; t < C::NB; ++t) bacc[t] *= al;
            m_ref = m_new;
        }
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(sv[e] - m_ref);
            l_part += p[e];
        }
        uint32_t pp[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) pp[k] = cvt_pk_h(p[2 * k], p[2 * k + 1]);

        // (q4_0 V with q4_sub8x codes: slots 2, 3, 6, 7 of P' divided by 16,
        // and their code offset 16 times as large)
        constexpr bool VN16 = TV == T_Q4;
        const uint32_t pq1 = VN16 ? pk_mul_h(pp[1], 0x2C002C00u) : pp[1];
        const uint32_t pq3 = VN16 ? pk_mul_h(pp[3], 0x2C002C00u) : pp[3];
        // P' for block kb: p times the V scale of each of this lane row's
        // rows 8*lq + e (eight contiguous fp16 values of the transposed tile)
        auto pscaled = [&](int kb) -> half8 {
            const u32x4 sv4 = *reinterpret_cast<const u32x4*>(vst + (kb * C::SPBV) * TT + 8 * lq);
            return make_half8(pk_mul_h(pp[0], sv4[0]), pk_mul_h(pq1, sv4[1]),
                              pk_mul_h(pp[2], sv4[2]), pk_mul_h(pq3, sv4[3]));
        };
        constexpr uint32_t VOFF_ODD = VN16 ? 0x00800080u : C::VOFF_BITS;
        const half8 voff = __builtin_bit_cast(half8, u32x4{C::VOFF_BITS, VOFF_ODD, C::VOFF_BITS, VOFF_ODD});

        // -- PV: O^T tile t (16 value columns) += V^T(16 x 32 rows) * P'^T
        const LDS_AS uint8_t* vl = (const LDS_AS uint8_t*)vb;
        if constexpr (TV == T_Q4) {
            // one transposed read gives the two column tiles of block c2
            // (chunks 2*c2 and 2*c2+1); lane r of the row group addresses row
            // 8*lq + pi(r&7), chunk 2*c2 + (r>>3), pi = [0,2,4,6,1,3,5,7] so the
            // nibble pairs come out in row order
            const int r = ln;
            const int rr = r & 7;
            const int trow = 8 * lq + ((rr < 4) ? 2 * rr : 2 * (rr - 4) + 1);
            const LDS_AS uint8_t* tbase = vl + trow * C::RBV_LDS + 8 * (r >> 3);
#pragma unroll
            for (int c2 = 0; c2 < C::NB; ++c2) {
                const int2v w = __builtin_amdgcn_ds_read_tr4_b64_v2i32((LDS_AS int2v*)(tbase + 16 * c2));
                const half8 bv = pscaled(c2);
                const half8 a0 = q4_sub8x((uint32_t)w[0]);
                const half8 a1 = q4_sub8x((uint32_t)w[1]);
                oacc[2 * c2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bv, oacc[2 * c2], 0, 0, 0);
                oacc[2 * c2 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bv, oacc[2 * c2 + 1], 0, 0, 0);
                bacc[c2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(voff, bv, bacc[c2], 0, 0, 0);
            }
        } else if constexpr (TV == T_Q8 || C::VBYTES) {
            // column tile t = chunks 2t, 2t+1; lane r addresses row 8*lq + r/2,
            // chunk 2t + (r&1).  q8_0: signed bytes (+128 for the subnormal
            // codes); the further types: unsigned code bytes
            const int r = ln;
            const LDS_AS uint8_t* tbase = vl + (8 * lq + (r >> 1)) * C::RBV_LDS + 8 * (r & 1);
#pragma unroll
            for (int kb = 0; kb < C::NB; ++kb) {
                const half8 bv = pscaled(kb);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int t = 2 * kb + h;
                    const int2v w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS int2v*)(tbase + 16 * t));
                    const half8 av = C::VBYTES ? u8_sub8((uint32_t)w[0], (uint32_t)w[1])
                                               : q8_sub8((uint32_t)w[0], (uint32_t)w[1]);
                    oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, oacc[t], 0, 0, 0);
                }
                if constexpr (C::VOFF_BITS != 0)
                    bacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(voff, bv, bacc[kb], 0, 0, 0);
            }
            if constexpr (C::VMIN) {
                // sum over the tile's rows of p * m per block: A row b (lane b
                // < NB) holds block b's minima of this lane row's eight rows,
                // B the unscaled p; row b of the result is block b
                const int e = ln < C::NB ? 2 * ln + 1 : 1;
                const u32x4 mv = *reinterpret_cast<const u32x4*>(vst + e * TT + 8 * lq);
                const half8 am = ln < C::NB ? make_half8(mv[0], mv[1], mv[2], mv[3])
                                            : make_half8(0u, 0u, 0u, 0u);
                bacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, make_half8(pp[0], pp[1], pp[2], pp[3]),
                                                                 bacc[0], 0, 0, 0);
            }
        } else {
            // column tile t = chunks 4t..4t+3 (4 halves each); two reads of 4
            // rows; lane r addresses row 8*lq + 4*R + r/4, chunk 4t + (r&3)
            const int r = ln;
            const half8 bv = make_half8(pp[0], pp[1], pp[2], pp[3]);
            const LDS_AS uint8_t* tbase = vl + (8 * lq + (r >> 2)) * C::RBV_LDS + 8 * (r & 3);
#pragma unroll
            for (int t = 0; t < C::NDT; ++t) {
                uint32_t d[4];
#pragma unroll
                for (int R = 0; R < 2; ++R) {
                    const short4v w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (LDS_AS short4v*)(tbase + 4 * R * C::RBV_LDS + 32 * t));
                    const u32x2 u = __builtin_bit_cast(u32x2, w);
                    d[2 * R] = u[0];
                    d[2 * R + 1] = u[1];
                }
                oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(make_half8(d[0], d[1], d[2], d[3]), bv,
                                                                oacc[t], 0, 0, 0);
            }
        }
    };

    // ---- main loop over this wave's tiles, with a ring of NS register sets
    //      so that loads run ahead: K of the tile NS places ahead in the
    //      wave's sequence is issued as soon as the current tile's QK products
    //      are done (into the registers they free); after the current tile's
    //      PV the V rows and scales of the next tile go to LDS (a wave's LDS
    //      reads and writes are performed in order, so one buffer suffices)
    //      and V of the tile NS + 1 places ahead is issued into the registers
    //      that frees.
    //    Wave w of a whole-row workgroup takes tiles w, w + W, ...; with a
    //    head wider than 128 all waves walk every tile, each over its slice.
    constexpr int W = C::DS > 1 ? 1 : WAVES;
    constexpr int NS = C::NSET;
    int it = C::DS > 1 ? 0 : wave;
    uint32_t krs[NS][2][KR];
    uint32_t vrs[NS][C::V_DW];
    uint32_t srs[NS][C::S_DW];
    // the new row's value of this thread (element tid & 31 of block tid >> 5:
    // K blocks, then V blocks), loaded first so it arrives with the tiles
    uint16_t xnew[C::NEW_IT];
    if constexpr (NEWROW_OK) {
        if (newrow) {
#pragma unroll
            for (int k = 0; k < C::NEW_IT; ++k) {
                // (half-waves past the row's blocks load its last block again:
                // no branch, so the loads stay in flight through the tile loop)
                const int blk2 = min((tid >> 5) + k * (C::NTH / 32), 2 * C::NB_ROW - 1);
                const bool isv = blk2 >= C::NB_ROW;
                xnew[k] = ((isv ? a.v_new : a.k_new) + ((int64_t)b * a.Hkv + g) * D +
                           32 * (isv ? blk2 - C::NB_ROW : blk2))[tid & 31];
            }
        }
    }
    // The new row: quantised into row L-1 (the block quantiser of
    // kvq_quantize_append, bit for bit), its decoded values (scale * code,
    // exact) kept in lds_new: K in [0, D), V in [D, 2D).
    auto newrow_quantise = [&]() {
        const int j = tid & 31, h = tid >> 5;
        if constexpr (C::NEW_IT >= 2) {
            // (head_dim 256 / 512) each half-wave h holds NK K blocks, h + k
            // HW, then as many V blocks: the 2 NK blocks are quantised in
            // lockstep and stored after all of them are computed
            constexpr int HW = C::NTH / 32, NK = C::NEW_IT / 2;
            static_assert(C::NEW_IT * C::NTH == 2 * C::NB_ROW * 32 && NK * HW == C::NB_ROW, "new-row blocks");
            uint16_t xk[NK], xv[NK];
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                // the raw values are opaque to the compiler until here, so
                // their loads are waited for only now
                uint32_t tk = xnew[k], tv = xnew[NK + k];
                asm volatile("" : "+v"(tk), "+v"(tv));
                xk[k] = (uint16_t)tk;
                xv[k] = (uint16_t)tv;
            }
            uint32_t wk[NK], wv[NK];
            uint16_t dk[NK], dv[NK];
            float ek[NK], ev[NK];
            quantize_blocks_lanes_compute<TK, NK>(xk, j, wk, dk, ek);
            quantize_blocks_lanes_compute<TV, NK>(xv, j, wv, dv, ev);
            uint8_t* pk[NK];
            uint8_t* pv[NK];
            uint16_t* sk[NK];
            uint16_t* sv[NK];
            const int64_t rk = krow0 + (L - 1), rv = vrow0 + (L - 1);
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const int blk = h + k * HW;
                pk[k] = a.k.data + rk * rb(TK, D) + blk * rb(TK, 32);
                sk[k] = a.k.scales + rk * (D / 32) + blk;
                pv[k] = a.v.data + rv * rb(TV, D) + blk * rb(TV, 32);
                sv[k] = a.v.scales + rv * (D / 32) + blk;
            }
            quantize_blocks_lanes_store<TK, NK>(pk, sk, j, wk, dk);
            quantize_blocks_lanes_store<TV, NK>(pv, sv, j, wv, dv);
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                lds_new[32 * (h + k * HW) + j] = ek[k];
                lds_new[32 * (C::NB_ROW + h + k * HW) + j] = ev[k];
            }
        } else {
            // (head_dim 128) one block per half-wave: K for h < NB_ROW, else V
            if (h >= 2 * C::NB_ROW) return;           // (uniform over the half-wave)
            uint32_t t = xnew[0];
            asm volatile("" : "+v"(t));
            const uint16_t xk = (uint16_t)t;
            const bool isv = h >= C::NB_ROW;
            const int blk = isv ? h - C::NB_ROW : h;
            const int64_t row = (isv ? vrow0 : krow0) + (L - 1);
            lds_new[32 * h + j] =
                isv ? quantize_block_lanes_v<TV>(xk, a.v.data + row * rb(TV, D) + blk * rb(TV, 32),
                                                 a.v.scales + row * (D / 32) + blk, j)
                    : quantize_block_lanes_v<TK>(xk, a.k.data + row * rb(TK, D) + blk * rb(TK, 32),
                                                 a.k.scales + row * (D / 32) + blk, j);
        }
    };
    // The new row's score of column ln over this wave's slice of the head
    // dimension (the same for the four lanes of the column): Q (the MFMA
    // operand, k-slot e of block kb holds element 32 kb + kel(e)) times the
    // decoded K row, in fp32.
    auto newrow_score_part = [&]() -> float {
        float acc = 0.0f;
#pragma unroll
        for (int kb = 0; kb < C::NB; ++kb) {
            const u32x4 qu = __builtin_bit_cast(u32x4, qop[kb]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w2 = (uint32_t)qu[e >> 1];
                const half2v h2 = __builtin_bit_cast(half2v, w2);
                const int kel = C::KNIB ? 4 * lq + ((e & 1) ? 2 : 0) + ((e & 2) ? 16 : 0) + (e >> 2) : 8 * lq + e;
                // (slots 2, 3, 6, 7 of a q4_sub8x operand hold q / 16)
                const float qe = (float)h2[e & 1] * (C::KNIB && C::KHB == 0 && (e & 2) ? 16.0f : 1.0f);
                acc = fmaf(qe, lds_new[wsl * C::DW + 32 * kb + kel], acc);
            }
        }
        return xsum4(acc);
    };
    load_q();
    // (issued on every path: a wave with no tile reads only out-of-range rows)
#pragma unroll
    for (int x = 0; x < NS; ++x) {
        issue_k(it + x * W, krs[x]);
        issue_vs(it + x * W, vrs[x], srs[x]);
    }
    // the tiles' loads go out before anything waits for Q
    __builtin_amdgcn_sched_barrier(0);
    init_q();
    // The new row is quantised and scored while the first tiles are in
    // flight: its score (log2 units) in m_new (head_dim 256 / 512: the sum of
    // the waves' slice scores, in a fixed order) or, over whole rows, in
    // lds_new[2D + column] (written by wave 0).  Its stores precede the
    // loop's later loads; no load of this launch reads row L-1.
    float m_new = -INFINITY;
    if constexpr (NEWROW_OK) {
        if (newrow) {
            newrow_quantise();
            __syncthreads();
            if constexpr (C::DS > 1) {
                const float sc = newrow_score_part();
                if (lq == 0) lds_new[2 * D + 16 * wave + ln] = sc;
                __syncthreads();
                float tot = 0.0f;
#pragma unroll
                for (int w = 0; w < C::WV; ++w) tot += lds_new[2 * D + 16 * w + ln];
                m_new = tot * a.scale_log2;
            } else {
                if (wave == 0) {
                    const float sc = newrow_score_part();
                    if (lq == 0) lds_new[2 * D + ln] = sc * a.scale_log2;
                }
            }
        }
    }
    // tile it uses K set x; V of tile it is in LDS, V of the next tile in set
    // (x + 1) % NS.  The loop runs whole rounds of the ring with no branch
    // around a load, so the compiler's wait before each use counts exactly
    // the loads issued after it.  A slot past the wave's last tile (at most
    // NS - 1 per wave) runs on rows at or past L: its loads are out of range
    // (zeros, no memory access) and every row is masked out of the softmax.
    //   SHORT (splits of fewer tiles per wave than a round holds, chosen
    //   on the host): the last round runs only the slots whose tile exists (a
    //   branch per slot, after the loop), so a wave with one tile computes one
    //   tile, not a whole round.  Otherwise every round is whole.
    if (it < ntiles) {
        stage(vrs[0], srs[0]);
        issue_vs(it + NS * W, vrs[0], srs[0]);
        const int rounds = ((ntiles - it + W - 1) / W + NS - 1) / NS;
        for (int r = 0; r < (SHORT ? rounds - 1 : rounds); ++r) {
#pragma unroll
            for (int x = 0; x < NS; ++x) {
                compute(it, krs[x], it + NS * W);
                const int y = (x + 1) % NS;
                stage(vrs[y], srs[y]);
                issue_vs(it + (NS + 1) * W, vrs[y], srs[y]);
                it += W;
            }
        }
        if constexpr (SHORT) {
#pragma unroll
            for (int x = 0; x < NS; ++x) {
                if (it < ntiles) {
                    compute(it, krs[x], it + NS * W);
                    const int y = (x + 1) % NS;
                    stage(vrs[y], srs[y]);
                    issue_vs(it + (NS + 1) * W, vrs[y], srs[y]);
                }
                it += W;
            }
        }
    }

    KVQ_TL(1);
    if constexpr (C::DS > 1) {
        // every wave holds the same (m, l) and its own slice of O: write it
        const float l_head = xsum4(l_part);
        // V with block minima (q4_1, q5_1): block kb's sum of p * m for head
        // ln, held by lane ln (lane row 0) in bacc[0][kb], enters in the
        // accumulators' units (2^-24)
        float vmin[C::VMIN ? C::NB : 1];
        if constexpr (C::VMIN) {
            static_assert(C::NB <= 4, "block minima of one lane row");
#pragma unroll
            for (int kb = 0; kb < C::NB; ++kb) {
                const float x = bacc[0][kb];
                vmin[kb] = __shfl(x, ln) * TWOM24;
            }
        }
        // (the new row's term: max m_new, sum 1, row v; hardware exp2, rcp
        // and log2, about 1 ulp each, as in the four-wave merge below)
        if (ln < NC) {
            // (a column that saw no row: l = 0, o = 0, lse = -inf)
            const bool nr = NEWROW_OK && newrow;
            const float M = nr ? fmaxf(m_ref, m_new) : m_ref;
            const float al = nr ? __builtin_amdgcn_exp2f(m_ref - M) : 1.0f;
            const float be = nr ? __builtin_amdgcn_exp2f(m_new - M) : 0.0f;
            const float lt = al * l_head + be;
            const float rl = lt > 0.0f ? __builtin_amdgcn_rcpf(lt) : 0.0f;
            const float inv = al * (C::V_SCALE ? TWO24 : 1.0f) * rl;
            const float fn = be * rl;
            const float* vnew = lds_new + D + wsl * C::DW;
            float* prow = po + crow(ln) * ho_stride + wsl * C::DW;
#pragma unroll
            for (int t = 0; t < C::NDT; ++t) {
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = oacc[t][i];
                    if constexpr (C::VMIN) o[i] += vmin[t >> 1];
                    else if constexpr (C::V_SCALE) o[i] -= bacc[t >> 1][i];
                    o[i] *= inv;
                    if (nr) {
                        // the column register i of tile t holds (see the stores below)
                        const int col = TV == T_Q4 ? 32 * (t >> 1) + 8 * (t & 1) + 2 * lq + (i >> 1) + 16 * (i & 1)
                                                   : 16 * t + 4 * lq + i;
                        o[i] = fmaf(fn, vnew[col], o[i]);
                    }
                }
                // register i holds output row m = 4*lq + i of the tile: for
                // q4_0 V column 32*(t/2) + 8*(t%2) + m/2 + 16*(m%2), i.e. two
                // adjacent pairs 16 apart; otherwise column 16*t + m, four
                // adjacent values
                if constexpr (TV == T_Q4) {
                    float* d0 = prow + 32 * (t >> 1) + 8 * (t & 1) + 2 * lq;
                    *reinterpret_cast<float2*>(d0) = make_float2(o[0], o[2]);
                    *reinterpret_cast<float2*>(d0 + 16) = make_float2(o[1], o[3]);
                } else {
                    *reinterpret_cast<float4*>(prow + 16 * t + 4 * lq) = make_float4(o[0], o[1], o[2], o[3]);
                }
            }
            if (wave == 0 && lq == 0)
                pl[crow(ln) * a.max_splits] = (M + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
        }
        return;
    }

    // ---- merge the four waves: (m, l, O) per head through LDS.  Each lane
    //      stores its raw accumulators in the merge area (no other wave reads
    //      or writes it before the barrier); after the one barrier every
    //      thread of the output loop forms its head's four wave weights
    //      itself (and the V code-offset correction of its block), so each
    //      output column is a four-term weighted sum.
    const float l_head = xsum4(l_part);
    (void)m_new;
    KVQ_TL(3);
    uint8_t* marea = lds_merge;
    float* mw = reinterpret_cast<float*>(marea);          // [WAVES][16]   running max
    float* lw = mw + WAVES * 16;                          // [WAVES][16]   running sum
    float* bw = lw + WAVES * 16;                          // [WAVES][16][NB] V offset sums
    float* ow = bw + WAVES * 16 * C::NB;                  // [WAVES][NC][D] accumulators
    if (lq == 0) {
        mw[wave * 16 + ln] = m_ref;
        lw[wave * 16 + ln] = l_head;
        if constexpr (C::VMIN) {
            // the minima's sum enters with the opposite sign of an offset, in
            // the units of the other accumulators (2^-24)
#pragma unroll
            for (int kb = 0; kb < C::NB; ++kb) bw[(wave * 16 + ln) * C::NB + kb] = -bacc[0][kb] * TWOM24;
        } else if constexpr (C::V_SCALE) {
#pragma unroll
            for (int kb = 0; kb < C::NB; ++kb) bw[(wave * 16 + ln) * C::NB + kb] = bacc[kb][0];
        }
    }
    if (ln < NC) {
        float* orow = ow + (wave * NC + ln) * D;
#pragma unroll
        for (int t = 0; t < C::NDT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * lq + i;
                int d;
                if constexpr (TV == T_Q4) d = 32 * (t >> 1) + 8 * (t & 1) + (m >> 1) + 16 * (m & 1);
                else d = 16 * t + m;
                orow[d] = oacc[t][i];
            }
    }
    __syncthreads();
    KVQ_TL(4);
    // (the weights, their sum's reciprocal and the log use the hardware
    // exp2 / rcp / log2, about 1 ulp each: this is the tail of every
    // workgroup, where the library's exact sequences cost more than the
    // rounding they save)
    for (int idx = tid; idx < NC * (D / 4); idx += C::NTH) {
        const int n = idx / (D / 4), c4 = idx % (D / 4);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, mw[w * 16 + n]);
        // the new row's term: max m_new, sum 1, row v (decoded)
        const float m_new = NEWROW_OK && newrow ? lds_new[2 * D + n] : -INFINITY;
        M = fmaxf(M, m_new);
        float f[WAVES], lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            // 0 for waves that saw no row (m at -inf or at the floor)
            f[w] = __builtin_amdgcn_exp2f(mw[w * 16 + n] - M);
            lsum += f[w] * lw[w * 16 + n];
        }
        const float f_new = NEWROW_OK && newrow ? __builtin_amdgcn_exp2f(m_new - M) : 0.0f;
        lsum += f_new;
        // quantised V: O = (acc - offset sum) * 2^24 (a column that sees no
        // row of the split: o = 0, lse = -inf)
        const float rl = lsum > 0.0f ? __builtin_amdgcn_rcpf(lsum) : 0.0f;
        const float inv = (C::V_SCALE ? TWO24 : 1.0f) * rl;
        float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float c = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float fwi = f[w] * inv;
            const float4 v = reinterpret_cast<const float4*>(ow + (w * NC + n) * D)[c4];
            o.x = fmaf(fwi, v.x, o.x);
            o.y = fmaf(fwi, v.y, o.y);
            o.z = fmaf(fwi, v.z, o.z);
            o.w = fmaf(fwi, v.w, o.w);
            if constexpr (C::V_SCALE) c = fmaf(fwi, bw[(w * 16 + n) * C::NB + c4 / 8], c);
        }
        if constexpr (C::V_SCALE) {
            o.x -= c;
            o.y -= c;
            o.z -= c;
            o.w -= c;
        }
        if constexpr (NEWROW_OK) {
            if (newrow) {
                const float fn = f_new * rl;
                const float4 v = reinterpret_cast<const float4*>(lds_new + D)[c4];
                o.x = fmaf(fn, v.x, o.x);
                o.y = fmaf(fn, v.y, o.y);
                o.z = fmaf(fn, v.z, o.z);
                o.w = fmaf(fn, v.w, o.w);
            }
        }
        reinterpret_cast<float4*>(po + crow(n) * ho_stride)[c4] = o;
        if (c4 == 0) pl[crow(n) * a.max_splits] = (M + __builtin_amdgcn_logf(lsum)) * 0.69314718055994531f;
    }
}

// seq_lens is a.seq_lens passed again as the first argument: the build
// preloads leading scalar arguments into registers (not struct ones), so
// the sequence length's load does not wait for the argument buffer.
template <int TK, int TV, int D, bool MQ, bool SHORT>
__global__ void __launch_bounds__((Cfg<TK, TV, D>::NTH)) __attribute__((amdgpu_waves_per_eu(Cfg<TK, TV, D>::WPE)))
decode_mfma_kernel(const int32_t* seq_lens, DecodeArgs a)
{
    using C = Cfg<TK, TV, D>;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[C::WV * C::BUF];
    __shared__ __attribute__((aligned(16))) float lds_sx[C::SX_FLOATS];
    __shared__ __attribute__((aligned(16))) float lds_new[C::NEWROW && !MQ ? 2 * D + 64 : 1];
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_merge[];   // merge_lds_bytes(nc)
    KVQ_TL(0);
    decode_wg<TK, TV, D, MQ, SHORT>(a, seq_lens, blockIdx.x, lds_a, lds_sx, lds_merge, lds_new);
    KVQ_TL(2);
}

// The two regions of a mixed cache in one launch (HAL #582 section 5 P2): the
// workgroups of the tail's splits [0, grid_splits(t)) run over the tail (types
// TK / TV), the others over the fp16 window w; each region writes its own
// partials.
// One launch instead of two saves the second launch's start and end, which
// for a window of a few thousand rows cost more than its bytes.
template <int TK, int TV, int D>
struct DualCfg {
    using T = Cfg<TK, TV, D>;
    using F = Cfg<T_F16, T_F16, D>;
    static constexpr int BUF = T::WV * (T::BUF > F::BUF ? T::BUF : F::BUF);
    static constexpr int SX = T::SX_FLOATS > F::SX_FLOATS ? T::SX_FLOATS : F::SX_FLOATS;
    static constexpr bool VALID = T::VALID && F::VALID;
};

// The leading scalar arguments (the regions' length pointers and the tail's
// split count ts = grid_splits(t)) are preloaded into registers, so neither
// the region test nor a length load waits for the argument structs.
template <int TK, int TV, int D>
__global__ void __launch_bounds__((Cfg<TK, TV, D>::NTH)) __attribute__((amdgpu_waves_per_eu(2)))
decode_mfma_dual_kernel(const int32_t* t_lens, const int32_t* w_lens, int ts, DecodeArgs t, DecodeArgs w)
{
    using DC = DualCfg<TK, TV, D>;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[DC::BUF];
    __shared__ __attribute__((aligned(16))) float lds_sx[DC::SX];
    __shared__ __attribute__((aligned(16))) float lds_new[DC::F::NEWROW || DC::T::NEWROW ? 2 * D + 64 : 1];
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_merge[];   // dual_dyn_bytes(G)
    // the first ts workgroups of each row take the tail
    if ((int)blockIdx.x < ts)
        decode_wg<TK, TV, D, false>(t, t_lens, blockIdx.x, lds_a, lds_sx, lds_merge, lds_new);
    else
        decode_wg<T_F16, T_F16, D, false>(w, w_lens, blockIdx.x - ts, lds_a, lds_sx, lds_merge, lds_new);
}

template <int TK, int TV, int D>
constexpr bool cfg_valid() { return Cfg<TK, TV, D>::VALID; }

// Dynamic LDS of a launch: the merge area (none for heads wider than 128).
template <int TK, int TV, int D>
size_t dyn_lds_bytes(int nc)
{
    return merge_lds_bytes<TK, TV, D>(nc);
}

template <int TK, int TV, int D>
size_t lds_bytes(int nc)
{
    using C = Cfg<TK, TV, D>;
    return (size_t)C::WV * C::BUF + sizeof(float) * (C::SX_FLOATS + (C::NEWROW ? 2 * D + 64 : 1)) +
           dyn_lds_bytes<TK, TV, D>(nc);
}

template <int TK, int TV, int D, bool MQ, bool SHORT>
hipError_t launch5(const DecodeArgs& a, hipStream_t s)
{
    dim3 grid(grid_splits(a), a.Hkv, a.B);
    const int nc = a.nq * a.G;
    const size_t dyn = dyn_lds_bytes<TK, TV, D>(nc);
    if (lds_bytes<TK, TV, D>(nc) > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&decode_mfma_kernel<TK, TV, D, MQ, SHORT>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_mfma_kernel<TK, TV, D, MQ, SHORT>), grid, dim3(Cfg<TK, TV, D>::NTH), dyn, s,
                       a.seq_lens, a);
    return hipGetLastError();
}

template <int TK, int TV, int D, bool MQ>
hipError_t launch4(const DecodeArgs& a, hipStream_t s)
{
    using C = Cfg<TK, TV, D>;
    if constexpr (!MQ && C::DS == 1) {
        // a full split's tiles per wave that are not a whole number of rounds
        // (e.g. 128-row splits: one tile per wave, two slots per round)
        const int tpw = ((a.split_tokens + TT - 1) / TT + WAVES - 1) / WAVES;
        if (tpw % C::NSET != 0) return launch5<TK, TV, D, MQ, true>(a, s);
    }
    return launch5<TK, TV, D, MQ, false>(a, s);
}

template <int TK, int TV, int D>
hipError_t launch3(const DecodeArgs& a, hipStream_t s)
{
    if constexpr (!Cfg<TK, TV, D>::VALID) {
        return hipErrorInvalidConfiguration;
    } else {
        return a.nq > 1 ? launch4<TK, TV, D, true>(a, s) : launch4<TK, TV, D, false>(a, s);
    }
}

// The pairs with the further storage types built for the matrix cores
// (head_dim 128): the pages' served pairs that use them and the tier ladder's
// last rung.
#define KVQ_NEW_PAIRS(X)  \
    X(T_Q8, T_Q6_0)       \
    X(T_Q8, T_Q5_0)       \
    X(T_Q6_0, T_Q6_0)     \
    X(T_Q6_0, T_Q4)       \
    X(T_Q5_0, T_Q5_0)     \
    X(T_Q5_1, T_Q5_1)     \
    X(T_Q4_1, T_Q4_1)     \
    X(T_Q5_1, T_Q4)

bool new_pair(int tk, int tv)
{
#define KVQ_X(K, V) if (tk == K && tv == V) return true;
    KVQ_NEW_PAIRS(KVQ_X)
#undef KVQ_X
    return false;
}

template <int D>
bool new_supports_d(const DecodeArgs& a)
{
#define KVQ_X(K, V) \
    if (a.tk == K && a.tv == V) return cfg_valid<K, V, D>() && lds_bytes<K, V, D>(a.nq * a.G) <= 160 * 1024;
    KVQ_NEW_PAIRS(KVQ_X)
#undef KVQ_X
    return false;
}

bool new_supports(const DecodeArgs& a)
{
    if (a.D == 128) return new_supports_d<128>(a);
    if (a.D == 256) return new_supports_d<256>(a);
    if (a.D == 512) return new_supports_d<512>(a);
    return false;
}

template <int D>
hipError_t new_launch_d(const DecodeArgs& a, hipStream_t s)
{
#define KVQ_X(K, V) if (a.tk == K && a.tv == V) return launch3<K, V, D>(a, s);
    KVQ_NEW_PAIRS(KVQ_X)
#undef KVQ_X
    return hipErrorInvalidConfiguration;
}

hipError_t new_launch(const DecodeArgs& a, hipStream_t s)
{
    if (a.D == 128) return new_launch_d<128>(a, s);
    if (a.D == 256) return new_launch_d<256>(a, s);
    if (a.D == 512) return new_launch_d<512>(a, s);
    return hipErrorInvalidConfiguration;
}

template <int TK, int TV, int D>
size_t dual_dyn_bytes(int G)
{
    const size_t mt = merge_lds_bytes<TK, TV, D>(G), mf = merge_lds_bytes<T_F16, T_F16, D>(G);
    return mt > mf ? mt : mf;
}

template <int TK, int TV, int D>
bool dual_supports3(const DecodeArgs& t)
{
    using DC = DualCfg<TK, TV, D>;
    if constexpr (!DC::VALID) {
        return false;
    } else {
        return (size_t)DC::BUF + sizeof(float) * (DC::SX + 2 * D + 64) + dual_dyn_bytes<TK, TV, D>(t.G) <=
               160 * 1024;
    }
}

template <int TK, int TV, int D>
hipError_t launch_dual3(const DecodeArgs& t, const DecodeArgs& w, hipStream_t s)
{
    using DC = DualCfg<TK, TV, D>;
    if constexpr (!DC::VALID) {
        return hipErrorInvalidConfiguration;
    } else {
        const size_t dyn = dual_dyn_bytes<TK, TV, D>(t.G);
        if ((size_t)DC::BUF + sizeof(float) * (DC::SX + 2 * D + 64) + dyn > 64 * 1024) {
            const hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void*>(&decode_mfma_dual_kernel<TK, TV, D>),
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
            if (e != hipSuccess) return e;
        }
        dim3 grid(grid_splits(t) + grid_splits(w), t.Hkv, t.B);
        hipLaunchKernelGGL((decode_mfma_dual_kernel<TK, TV, D>), grid, dim3(Cfg<TK, TV, D>::NTH), dyn, s,
                           t.seq_lens, w.seq_lens, grid_splits(t), t, w);
        return hipGetLastError();
    }
}

// tail types: the quantised pairs
template <int D>
bool dual_supports2(const DecodeArgs& t)
{
    if (t.tk == T_Q8 && t.tv == T_Q8) return dual_supports3<T_Q8, T_Q8, D>(t);
    if (t.tk == T_Q8 && t.tv == T_Q4) return dual_supports3<T_Q8, T_Q4, D>(t);
    if (t.tk == T_Q4 && t.tv == T_Q8) return dual_supports3<T_Q4, T_Q8, D>(t);
    if (t.tk == T_Q4 && t.tv == T_Q4) return dual_supports3<T_Q4, T_Q4, D>(t);
    if constexpr (D == 128) {
#define KVQ_X(K, V) if (t.tk == K && t.tv == V) return dual_supports3<K, V, 128>(t);
        KVQ_NEW_PAIRS(KVQ_X)
#undef KVQ_X
    }
    return false;
}

template <int D>
hipError_t launch_dual2(const DecodeArgs& t, const DecodeArgs& w, hipStream_t s)
{
    if (t.tk == T_Q8 && t.tv == T_Q8) return launch_dual3<T_Q8, T_Q8, D>(t, w, s);
    if (t.tk == T_Q8 && t.tv == T_Q4) return launch_dual3<T_Q8, T_Q4, D>(t, w, s);
    if (t.tk == T_Q4 && t.tv == T_Q8) return launch_dual3<T_Q4, T_Q8, D>(t, w, s);
    if (t.tk == T_Q4 && t.tv == T_Q4) return launch_dual3<T_Q4, T_Q4, D>(t, w, s);
    if constexpr (D == 128) {
#define KVQ_X(K, V) if (t.tk == K && t.tv == V) return launch_dual3<K, V, 128>(t, w, s);
        KVQ_NEW_PAIRS(KVQ_X)
#undef KVQ_X
    }
    return hipErrorInvalidConfiguration;
}

template <int TK, int TV>
hipError_t launch2(const DecodeArgs& a, hipStream_t s)
{
    switch (a.D) {
    case 128: return launch3<TK, TV, 128>(a, s);
    case 256: return launch3<TK, TV, 256>(a, s);
    case 512: return launch3<TK, TV, 512>(a, s);
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

template <int TK, int TV>
bool supports2(const DecodeArgs& a)
{
    const int nc = a.nq * a.G;
    if (a.D == 128) return cfg_valid<TK, TV, 128>() && lds_bytes<TK, TV, 128>(nc) <= 160 * 1024;
    if (a.D == 256) return cfg_valid<TK, TV, 256>() && lds_bytes<TK, TV, 256>(nc) <= 160 * 1024;
    if (a.D == 512) return cfg_valid<TK, TV, 512>() && lds_bytes<TK, TV, 512>(nc) <= 160 * 1024;
    return false;
}

template <int TK>
bool supports1(const DecodeArgs& a)
{
    switch (a.tv) {
    case T_F16: return supports2<TK, T_F16>(a);
    case T_Q8: return supports2<TK, T_Q8>(a);
    default: return supports2<TK, T_Q4>(a);
    }
}

}  // namespace

bool decode_mfma_supports(const DecodeArgs& a)
{
    // the matrix-core kernel is built for f16, q8_0 and q4_0 rows, and for the
    // listed pairs with the further types
    auto built = [](int t) { return t == T_F16 || t == T_Q8 || t == T_Q4; };
    if (!built(a.tk) || !built(a.tv)) {
        if (!new_pair(a.tk, a.tv)) return false;
        const int64_t rows = a.max_seq_len;
        if (rows * (int64_t)data_row_bytes(a.tk, a.D) >= (1LL << 31)) return false;
        if (rows * (int64_t)data_row_bytes(a.tv, a.D) >= (1LL << 31)) return false;
        return a.G >= 1 && a.nq >= 1 && a.nq * a.G <= 16 && new_supports(a);
    }
    if (a.D != 128 && a.D != 256 && a.D != 512) return false;
    if (a.G < 1 || a.nq < 1 || a.nq * a.G > 16) return false;
    // rows read are below max_seq_len; their offsets inside one (sequence,
    // KV head) plane are computed in 32 bits
    const int64_t rows = a.max_seq_len;
    if (rows * (int64_t)data_row_bytes(a.tk, a.D) >= (1LL << 31)) return false;
    if (rows * (int64_t)data_row_bytes(a.tv, a.D) >= (1LL << 31)) return false;
    switch (a.tk) {
    case T_F16: return supports1<T_F16>(a);
    case T_Q8: return supports1<T_Q8>(a);
    default: return supports1<T_Q4>(a);
    }
}

bool decode_mfma_dual_supports(const DecodeArgs& t, const DecodeArgs& w)
{
    if (w.tk != T_F16 || w.tv != T_F16 || t.nq != 1 || w.nq != 1) return false;
    if (w.D != t.D || w.B != t.B || w.Hkv != t.Hkv || w.Hq != t.Hq) return false;
    if (!decode_mfma_supports(t) || !decode_mfma_supports(w)) return false;
    if ((int64_t)t.max_splits + w.max_splits > 0x7fffffffLL) return false;
    switch (t.D) {
    case 128: return dual_supports2<128>(t);
    case 256: return dual_supports2<256>(t);
    case 512: return dual_supports2<512>(t);
    default: return false;
    }
}

hipError_t launch_decode_mfma_dual(const DecodeArgs& t, const DecodeArgs& w, hipStream_t s)
{
    switch (t.D) {
    case 128: return launch_dual2<128>(t, w, s);
    case 256: return launch_dual2<256>(t, w, s);
    case 512: return launch_dual2<512>(t, w, s);
    default: return hipErrorInvalidConfiguration;
    }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s)
{
    if (new_pair(a.tk, a.tv)) return new_launch(a, s);
    switch (a.tk) {
    case T_F16: return launch1<T_F16>(a, s);
    case T_Q8: return launch1<T_Q8>(a, s);
    default: return launch1<T_Q4>(a, s);
    }
}

}  // namespace kvq
