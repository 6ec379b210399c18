// W4A16 GEMV kernels for gfx950 (CDNA4, wave64).
//
// The operation (local-kimi README, technical-detail section, GEMV-rewrite paragraph): a true
// matrix-vector product over packed INT4 weights, walking the contiguous reduction axis K with a
// single accumulator per output row, instead of a matrix-matrix kernel applied to one token.
//
// Decode path shared by every kernel here. A 32-bit word holds 8 two's-complement nibbles n0..n7
// (n0 in the low bits); they are decoded in the pairs (n0,n4) (n1,n5) (n2,n6) (n3,n7), each pair
// as the two halves of one fp16 pair, by one v_bitop3 (mask and XOR with a magic constant) and
// one v_pk_add_f16:
//   nibbles in bits 0-3 and 16-19:  (w & 0x000F000F) ^ 0x64086408  ->  1032 + q,  minus 1032
//   nibbles in bits 4-7 and 20-23:  (w & 0x00F000F0) ^ 0x54805480  ->    72 + q,  minus 72
// The XOR sets the fp16 exponent at which one step of the nibble's mantissa bits is 1.0 (2^10
// for bits 0-3, 2^6 for bits 4-7) and flips the nibble's top bit, which maps the two's-complement
// code to q + 8; the subtraction leaves q itself, exactly (the magic-number conversion of
// integers to floating point, applied to packed 4-bit codes). Pairs (n2,n6) and (n3,n7) take the
// same two forms on w >> 8. Weights enter every product as the exact integer q: there is no
// constant offset left to cancel later, so the fp32 rounding of a sum stays relative to the sum
// of |q x|.
//
// Activations are staged as fp16 once per work-group (or per wave for register-resident forms).
// Each run of 128 activations of one token (one scale group) is multiplied by a power of two 2^e
// chosen so that its largest magnitude lands in [2^15, 2^16), then rounded to fp16. A bf16 value
// has 8 significant bits, so the scaled value is exact in fp16 unless it falls below 2^-17, i.e.
// unless it is smaller than about 2^-32 times the largest magnitude of its group; such values are
// rounded to a multiple of 2^-24 (scaled). Products q * x' (4 + 11 significant bits) are exact in
// fp32, group or chunk totals are accumulated in fp32 and multiplied by 2^-e (exact) and by the
// group's fp16 scale. Non-finite activations stay non-finite (an infinity or NaN in a group only
// moves that group's exponent), so every output that reads one is non-finite, as in the plain
// definition (0 * inf is NaN there too).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "plan.h"

namespace w4a16 {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// fp32 sum c + a.lo * b.lo + a.hi * b.hi of two fp16 pairs (v_dot2c_f32_f16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                  false);
}

// The two codes in bits 0-3 and 16-19 of `bits` (other bits ignored) as the fp16 pair (q_lo, q_hi).
__device__ __forceinline__ uint32_t decode_pair_lo(uint32_t bits)
{
    const f16x2_t v = __builtin_bit_cast(f16x2_t, (bits & 0x000F000Fu) ^ 0x64086408u);
    return __builtin_bit_cast(uint32_t, v + __builtin_bit_cast(f16x2_t, 0xE408E408u));
}

// The two codes in bits 4-7 and 20-23 of `bits` (other bits ignored) as the fp16 pair.
__device__ __forceinline__ uint32_t decode_pair_hi(uint32_t bits)
{
    const f16x2_t v = __builtin_bit_cast(f16x2_t, (bits & 0x00F000F0u) ^ 0x54805480u);
    return __builtin_bit_cast(uint32_t, v + __builtin_bit_cast(f16x2_t, 0xD480D480u));
}

// Weights are read exactly once per call: stream them past the caches.
__device__ __forceinline__ uint4 load_weights(const uint4 *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

// The fp32 values of the fp16 scales held by lanes 4*(lane/4) + r, r = 0..3: one conversion,
// then DPP quad broadcasts. The full row and bank masks write every lane, so the destination
// needs no previous value.
__device__ __forceinline__ void quad_scales(uint16_t sv, float (&s4)[4])
{
    const int f = __builtin_bit_cast(int, half_bits_to_float(sv));
    s4[0] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(f, 0x00, 0xF, 0xF, false));
    s4[1] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(f, 0x55, 0xF, 0xF, false));
    s4[2] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(f, 0xAA, 0xF, 0xF, false));
    s4[3] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(f, 0xFF, 0xF, 0xF, false));
}

// a if take else b, computed with masks so it never becomes a branch (branches around the loads
// make the compiler fall back to waiting for every outstanding load at the join).
template <typename T>
__device__ __forceinline__ const T *pick(bool take, const T *a, const T *b)
{
    const uintptr_t m = (uintptr_t)0 - (uintptr_t)take;
    return reinterpret_cast<const T *>((reinterpret_cast<uintptr_t>(a) & m) |
                                       (reinterpret_cast<uintptr_t>(b) & ~m));
}

// Nibble pairs (0,4) (1,5) (2,6) (3,7) of w as fp16 pairs holding q.
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t p[4])
{
    const uint32_t w8 = w >> 8;
    p[0] = decode_pair_lo(w);
    p[1] = decode_pair_hi(w);
    p[2] = decode_pair_lo(w8);
    p[3] = decode_pair_hi(w8);
}

// The four words of a 16-byte chunk: p[j][0..3] are the four fp16 pairs of word j.
__device__ __forceinline__ void unpack_chunk(uint4 wv, uint32_t p[4][4])
{
    unpack_word(wv.x, p[0]);
    unpack_word(wv.y, p[1]);
    unpack_word(wv.z, p[2]);
    unpack_word(wv.w, p[3]);
}

// Sum over one 32-weight chunk of q * x', the activations re-paired and staged as fp16.
__device__ __forceinline__ float chunk_dot(uint4 wv, const uint4 xq[4])
{
    uint32_t p[4][4];
    unpack_chunk(wv, p);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc = dot2(p[j][0], xq[j].x, acc);
        acc = dot2(p[j][1], xq[j].y, acc);
        acc = dot2(p[j][2], xq[j].z, acc);
        acc = dot2(p[j][3], xq[j].w, acc);
    }
    return acc;
}

// ---- activation staging: bf16 -> fp16 with a power-of-two scale per 128-value group

// Largest |x| of the two bf16 values of d, as a bf16 bit pattern in both halves (for finite
// magnitudes the bit pattern orders like the value; NaN and infinity compare above them).
__device__ __forceinline__ uint32_t abs_max2(uint32_t d, uint32_t m)
{
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, d & 0x7FFF7FFFu),
                                                        __builtin_bit_cast(u16x2_t, m)));
}

__device__ __forceinline__ uint32_t abs_max8(uint4 v, uint32_t m)
{
    return abs_max2(v.w, abs_max2(v.z, abs_max2(v.y, abs_max2(v.x, m))));
}

// The larger of the two 16-bit halves of m2, as a 32-bit integer (cross-lane maxima compare
// these, never packed pairs).
__device__ __forceinline__ uint32_t fold_halves(uint32_t m2)
{
    return (m2 >> 16) > (m2 & 0xFFFFu) ? (m2 >> 16) : (m2 & 0xFFFFu);
}

// Exponent e of a group from the bf16 pattern m of its largest magnitude: 2^e * max lands in
// [2^15, 2^16). A bf16 pattern with exponent field b is in [2^(b-127), 2^(b-126)), so
// e = 142 - b; e is capped at 126 so that 2^e and 2^-e are normal fp32 numbers (the groups it
// affects hold only values below 2^-110, all exact in fp16 at that scale). An all-zero group
// gets 126 too.
__device__ __forceinline__ int group_exponent(uint32_t m)
{
    const int e = 142 - (int)(m >> 7);
    return e < 126 ? e : 126;
}

__device__ __forceinline__ float pow2f(int e) { return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23); }

// fp16 pair (a * p, b * p) of two fp32 values, each product rounded once (nearest even): one
// v_fma_mixlo_f16 and one v_fma_mixhi_f16 with fp32 sources.
__device__ __forceinline__ uint32_t pack_scaled(float a, float b, float p)
{
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "=v"(r) : "v"(a), "v"(p));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "+v"(r) : "v"(b), "v"(p));
    return r;
}

// Eight consecutive bf16 activations (x0..x7 in natural order) times p = 2^e as fp16, re-paired
// as (x0,x4) (x1,x5) (x2,x6) (x3,x7) to match unpack_word. The products are exact, so each value
// is rounded once, to fp16.
__device__ __forceinline__ uint4 stage_words(uint4 v, float p)
{
    auto lo = [](uint32_t d) { return __builtin_bit_cast(float, d << 16); };
    auto hi = [](uint32_t d) { return __builtin_bit_cast(float, d & 0xFFFF0000u); };
    return make_uint4(pack_scaled(lo(v.x), lo(v.z), p), pack_scaled(hi(v.x), hi(v.z), p),
                      pack_scaled(lo(v.y), lo(v.w), p), pack_scaled(hi(v.y), hi(v.w), p));
}

// Largest of a per-lane value over the 16 lanes of a DPP row (integer compare).
__device__ __forceinline__ uint32_t row_max16(uint32_t m)
{
    int x = (int)m;
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));
    return (uint32_t)x;
}

// Largest over each quad of lanes.
__device__ __forceinline__ uint32_t quad_max(uint32_t m)
{
    int x = (int)m;
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    return (uint32_t)x;
}

// Cross-lane exchange across lane-index bit `bit` without LDS: DPP within a 16-lane row for bits
// 0-3 (quad permutes, then the half-row and row mirrors, each a bijection between the two halves of
// the group), v_permlane16_swap / v_permlane32_swap for bits 4 and 5.
__device__ __forceinline__ float dpp_partner(float v, int bit)
{
    const int x = __builtin_bit_cast(int, v);
    int r;
    switch (bit) {
    case 0: r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true); break;   // quad_perm 1,0,3,2
    case 1: r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true); break;   // quad_perm 2,3,0,1
    case 2: r = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true); break;  // row_half_mirror
    default: r = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, true); break; // row_mirror
    }
    return __builtin_bit_cast(float, r);
}

// Swap the halves selected by lane bit 4 or 5 between a and b: afterwards a + b holds, in lanes with
// the bit clear, a + partner's a, and in lanes with the bit set, b + partner's b.
// v_permlane16_swap (v_permlane32_swap) exchanges the odd 16-lane rows (the upper 32 lanes) of its
// first register with the even rows (the lower 32 lanes) of its second and rewrites both; the
// builtin returns the two new registers, and the compiler inserts the wait states the instruction
// needs after a VALU write of its operands.
__device__ __forceinline__ float swap_fold(float a, float b, int bit)
{
    const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
    const auto r = bit == 5 ? __builtin_amdgcn_permlane32_swap(ua, ub, false, false)
                            : __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Sum U per-lane values over groups of L lanes (L, U powers of two, U <= L). Rows are folded while
// lanes are halved: at each of the first log2(U) steps a lane keeps half of its rows (the upper half
// if its lane bit is set) and adds its partner's copy of them, so U rows cost U-1 exchanges plus
// log2(L/U) plain ones instead of U*log2(L). On return v[0] holds the full sum of row `row`; the lanes
// with (lane % (L/U)) == 0 hold distinct rows and together cover all U of them.
template <int L, int U>
__device__ __forceinline__ int fold_rows(float (&v)[U], int lane)
{
    static_assert(U <= L, "fold_rows needs U <= L");
    static_assert((L & (L - 1)) == 0 && (U & (U - 1)) == 0, "fold_rows needs powers of two");
    constexpr int LB = __builtin_ctz(L);
    constexpr int UB = __builtin_ctz(U);
    int row = 0;
#pragma unroll
    for (int k = 0; k < UB; ++k) {
        const int bit = LB - 1 - k;
        const int m = U >> (k + 1);
        const bool upper = (lane >> bit) & 1;
#pragma unroll
        for (int i = 0; i < m; ++i) {
            if (bit >= 4) {
                v[i] = swap_fold(v[i], v[i + m], bit);
            } else {
                const float lo = v[i] + dpp_partner(v[i], bit);
                const float hi = v[i + m] + dpp_partner(v[i + m], bit);
                v[i] = upper ? hi : lo;
            }
        }
        row += upper ? m : 0;
    }
#pragma unroll
    for (int bit = LB - 1 - UB; bit >= 0; --bit)
        v[0] = bit >= 4 ? swap_fold(v[0], v[0], bit) : v[0] + dpp_partner(v[0], bit);
    return row;
}

// ------------------------------------------------------------------------------------------
// Staged VALU GEMV: MT tokens (1..4). A wave streams U*R rows at a time, R = 64/L rows side by
// side, L lanes per row; lane p of a row owns the 16-byte chunks p, p+L, p+2L, ... of that row, so
// each load instruction covers R runs of L*16 contiguous bytes (whole cache lines). Activations are
// staged once per work-group in LDS, re-paired and laid out [token][word-in-chunk j][chunk c] so
// the L lanes of a row read consecutive 16-byte slots, followed by the per-chunk factors 2^-e
// of their groups and, for the grouped-expert form, the expert ids (so id lookups never wait on
// outstanding weight loads). A wave walks a flat sequence of (row block, chunk batch) items with
// one item of prefetch. Every load is unconditional: rows past the end re-read the last row,
// rows of an out-of-range expert read the activation row (valid memory of at least K*2 bytes, so
// no other expert is touched), and waves without work re-read a valid item; results of all these
// are discarded or written as zero. Straight-line loads let the compiler wait for each load on
// its own, so early rows are multiplied while later ones are in flight.
//
// Modes (one token unless dense):
//   VALU_DENSE    rows of one matrix.
//   VALU_MOE      rows t*N + n of the experts ids[t] (grouped-expert form).
//   VALU_SWIGLU   the grouped form over gate+up experts of 2I rows: a wave's R rows are HALF = R/2
//                 gate rows n0.. and the matching up rows I+n0.., so after the row sums each gate
//                 lane meets its up partner 32 lanes away and writes h = bf16(silu(g) * u).
//   VALU_COMBINE  the grouped down projection with the router-weighted sum: the activation is
//                 the concatenation of the topk rows h[t] (K = topk*I), and chunk batch b of a row
//                 reads slot t = b*L*V / (I/32) from expert ids[t]'s row, its scales multiplied by
//                 w[t], so the row sum is sum_t w[t] * W_{ids[t]}[n] h[t]. A batch never straddles
//                 two slots ((I/32) % (L*V) == 0). An invalid id reads expert 0 with weight 0.
// ------------------------------------------------------------------------------------------
enum ValuMode { VALU_DENSE = 0, VALU_MOE = 1, VALU_SWIGLU = 2, VALU_COMBINE = 3 };

// bf16 bit pattern nearest to f (ties to even); NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f)
{
    uint32_t b = __builtin_bit_cast(uint32_t, f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((b >> 16) | 0x40u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

template <int L, int V, int U>
struct ValuBuf {
    uint4 w[V][U];
    uint16_t s[V][U];
};

template <int MT, int L, int V, int U, int MODE>
__global__ void __launch_bounds__(256)
gemv_valu_kernel(const uint4 *__restrict__ qw, const uint16_t *__restrict__ sc,
                 const uint16_t *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy,
                 const int32_t *__restrict__ ids, int32_t topk, int32_t E, int64_t N, int32_t K,
                 const float *__restrict__ rw, int32_t KR)
{
    constexpr bool MOE = MODE == VALU_MOE || MODE == VALU_SWIGLU;   // rows through expert ids
    constexpr bool TAIL = MODE == VALU_SWIGLU || MODE == VALU_COMBINE;
    static_assert(!TAIL || (MT == 1 && U == 1), "expert-tail modes are single-token, U = 1");
    static_assert(MODE != VALU_SWIGLU || L <= 32, "SwiGLU pairs need two row halves per wave");
    constexpr int R = 64 / L;
    constexpr int ROWS = U * R;
    constexpr int HALF = R / 2;   // SwiGLU: gate rows per wave step
    extern __shared__ uint4 smem[];
    const int KW = K >> 3;    // activation words
    const int CPR = K >> 5;   // activation chunks (16 bytes); chunks per weight row except combine
    const int CPRW = (MODE == VALU_COMBINE ? KR : K) >> 5;   // 16-byte chunks per weight row
    const int GPRW = (MODE == VALU_COMBINE ? KR : K) >> 7;   // scale groups per weight row
    const int GPR = GPRW;
    uint4 *xs = smem;                                            // [MT][4][CPR]
    float *bs = reinterpret_cast<float *>(smem + MT * KW);      // [MT][CPR]
    int32_t *ids_s = reinterpret_cast<int32_t *>(bs + MT * CPR);  // [topk] (expert forms)
    float *rw_s = reinterpret_cast<float *>(ids_s + topk);        // [topk] (combine)
    const int64_t I = N >> 1;                                     // SwiGLU: outputs per slot
    const int64_t bps = MODE == VALU_SWIGLU ? (I + HALF - 1) / HALF : 1;   // SwiGLU blocks per slot

    const int lane = threadIdx.x & 63;
    const int pr = lane & (L - 1);
    const int rr = lane / L;
    const int wpb = blockDim.x >> 6;
    // The wave index is the same in every lane; saying so lets row bases live in scalar registers.
    const int64_t gw = (int64_t)blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t GW = (int64_t)gridDim.x * wpb;
    const int64_t rows_total = MODE == VALU_MOE ? (int64_t)topk * N : N;
    const int64_t n_super =
        MODE == VALU_SWIGLU ? (int64_t)topk * bps : (rows_total + ROWS - 1) / ROWS;
    const int nb = CPR / (L * V);
    const bool active = gw < n_super;
    const int64_t gw_c = active ? gw : n_super - 1;
    const int64_t n_items = ((n_super - 1 - gw_c) / GW + 1) * nb;

    // Dense rows: a wave-uniform base row plus fixed per-lane offsets. The last row block is pulled
    // back to end at the last row (rows computed twice get identical bits); with fewer rows than
    // one block the lane rows are clamped instead.
    const bool full = rows_total >= ROWS;
    // Lane row of row step u (u may be a run-time value: it is recomputed, not indexed, so no
    // per-lane array has to live in scratch memory).
    auto lane_row = [&](int u) -> int {
        const int r = u * R + rr;
        return (!full && r > rows_total - 1) ? (int)rows_total - 1 : r;
    };
    uint32_t woff[U], soff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = lane_row(u);
        woff[u] = (uint32_t)((r * CPRW + pr) * 16);
        soff[u] = (uint32_t)((r * GPRW + (pr >> 2)) * 2);
    }
    auto st_row0 = [&](int64_t st) -> int64_t {
        if (!full)
            return 0;
        const int64_t r0 = st * ROWS;
        return r0 + ROWS <= rows_total ? r0 : rows_total - ROWS;
    };
    struct Rows {
        const uint4 *w[U];
        const uint16_t *s[U];
    };
    // SwiGLU: slot, output index of this lane's row pair, and whether the lane holds the up row.
    auto swiglu_row = [&](int64_t st, int64_t &slot, int64_t &p) {
        slot = st / bps;
        const int64_t b = st - slot * bps;
        int64_t p0 = b * HALF;
        p0 = p0 + HALF <= I ? p0 : (I >= HALF ? I - HALF : 0);
        p = p0 + (rr & (HALF - 1));
        p = p < I ? p : I - 1;
    };
    // Expert id of a slot: from global memory for the first item (no weight load is outstanding
    // yet, so waiting for it costs nothing extra), from the LDS copy afterwards (a global load
    // would complete behind the weight loads in flight).
    auto expert_of = [&](int64_t slot, auto first) -> int32_t {
        if constexpr (decltype(first)::value)
            return ids[slot];
        else
            return ids_s[slot];
    };
    auto rows_of = [&](int64_t st, Rows &r, auto first) {
        if constexpr (MODE == VALU_SWIGLU) {
            int64_t slot, p;
            swiglu_row(st, slot, p);
            const int32_t e = expert_of(slot, first);
            const bool ok = e >= 0 && e < E;
            const int64_t row = (int64_t)(ok ? e : 0) * N + (rr >= HALF ? I : 0) + p;
            r.w[0] = pick(ok, qw + row * CPR, reinterpret_cast<const uint4 *>(X));
            r.s[0] = pick(ok, sc + row * GPR, X);
            return;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t vrow = st * ROWS + u * R + rr;
            vrow = vrow < rows_total ? vrow : rows_total - 1;
            if (MOE) {
                // topk * N < 2^31 (checked by the entry point): a 32-bit division suffices
                const int64_t slot = (uint32_t)vrow / (uint32_t)N;
                const int32_t e = expert_of(slot, first);
                const bool ok = e >= 0 && e < E;
                const int64_t row = (int64_t)(ok ? e : 0) * N + (vrow - slot * N);
                r.w[u] = pick(ok, qw + row * CPR, reinterpret_cast<const uint4 *>(X));
                r.s[u] = pick(ok, sc + row * GPR, X);
            } else {
                r.w[u] = qw + vrow * CPR;
                r.s[u] = sc + vrow * GPR;
            }
        }
    };
    // Loads and computes each walk the items in order with their own cursor (row block, batch).
    // Expert forms look the rows of a row step up once, at its first batch.
    int64_t ld_st = gw_c;
    int ld_b = 0;
    Rows r;
    auto load = [&](ValuBuf<L, V, U> &buf, auto first) {
        if constexpr (MOE) {
            if (decltype(first)::value || ld_b == 0)
                rows_of(ld_st, r, first);
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int c = pr + L * (v + V * ld_b);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    buf.w[v][u] = load_weights(r.w[u] + c);
                    buf.s[v][u] = r.s[u][c >> 2];
                }
            }
        } else {
            const int64_t r0 = st_row0(ld_st);
            const uint4 *wq = qw;
            const uint16_t *sq = sc;
            int cb = L * V * ld_b;   // first chunk of the batch within its weight row
            if constexpr (MODE == VALU_COMBINE) {
                const int slot = cb / CPRW;
                const int32_t e = expert_of(slot, first);
                const int64_t ee = (e >= 0 && e < E) ? e : 0;
                wq += ee * N * CPRW;
                sq += ee * N * GPRW;
                cb -= slot * CPRW;
            }
            const char *wb = reinterpret_cast<const char *>(wq + r0 * CPRW + cb);
            const char *sb = reinterpret_cast<const char *>(sq + r0 * GPRW + (cb >> 2));
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    buf.w[v][u] = load_weights(
                        reinterpret_cast<const uint4 *>(wb + woff[u] + 16 * L * v));
                    buf.s[v][u] =
                        *reinterpret_cast<const uint16_t *>(sb + soff[u] + 2 * (L / 4) * v);
                }
        }
        const bool wrap = ld_b + 1 == nb;
        ld_b = wrap ? 0 : ld_b + 1;
        ld_st += wrap ? GW : 0;
    };

    // Activation words of the first two staging passes are requested first, then the first item's
    // weights (for expert forms after its expert ids); loads complete in issue order, so staging
    // below waits only for the activations while the weights are still in flight. Rows of longer
    // activations (K > 8 * 2 * threads) fetch the rest during staging.
    constexpr int PF = 2;
    uint4 xpre[MT][PF];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const uint4 *xg = reinterpret_cast<const uint4 *>(X + t * ldx);
#pragma unroll
        for (int f = 0; f < PF; ++f) {
            const int w = threadIdx.x + f * blockDim.x;
            xpre[t][f] = xg[w < KW ? w : KW - 1];
        }
    }
    // Expert ids and router weights for the LDS copy (one per thread; larger topk is read during
    // staging).
    int32_t id_pre = 0;
    float rw_pre = 0.0f;
    if constexpr (MODE != VALU_DENSE) {
        const int i = threadIdx.x < topk ? threadIdx.x : topk - 1;
        id_pre = ids[i];
        if constexpr (MODE == VALU_COMBINE)
            rw_pre = rw[i];
    }
    __builtin_amdgcn_sched_barrier(0);
    ValuBuf<L, V, U> bufA, bufB;
    load(bufA, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);

    // ---- stage activations: scale each group to fp16, re-pair, transpose to [j][c], and keep
    // the per-chunk factor 2^-e of its group
    auto stage = [&](int t, int w, uint4 v) {
        // The 16 words of a scale group sit in the 16 lanes of one DPP row (KW is a multiple of
        // 16 and the word index advances by a multiple of 64 per pass), all active or all not.
        const int e = group_exponent(row_max16(fold_halves(abs_max8(v, 0u))));
        xs[t * KW + (w & 3) * CPR + (w >> 2)] = stage_words(v, pow2f(e));
        if ((w & 3) == 0)
            bs[t * CPR + (w >> 2)] = pow2f(-e);
    };
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int f = 0; f < PF; ++f) {
            const int w = threadIdx.x + f * blockDim.x;
            if (w < KW)
                stage(t, w, xpre[t][f]);
        }
        const uint4 *xg = reinterpret_cast<const uint4 *>(X + t * ldx);
        for (int w = threadIdx.x + PF * blockDim.x; w < KW; w += blockDim.x)
            stage(t, w, xg[w]);
    }
    if constexpr (MODE != VALU_DENSE) {
        if ((int)threadIdx.x < topk) {
            ids_s[threadIdx.x] = id_pre;
            if constexpr (MODE == VALU_COMBINE)
                rw_s[threadIdx.x] = (id_pre >= 0 && id_pre < E) ? rw_pre : 0.0f;
        }
        for (int i = threadIdx.x + blockDim.x; i < topk; i += blockDim.x) {
            ids_s[i] = ids[i];
            if constexpr (MODE == VALU_COMBINE)
                rw_s[i] = (ids[i] >= 0 && ids[i] < E) ? rw[i] : 0.0f;
        }
    }
    __syncthreads();
    if (!active)
        return;

    float acc[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < MT; ++t)
            acc[u][t] = 0.0f;

    auto finish = [&](int64_t st) {
        if constexpr (MODE == VALU_SWIGLU) {
            float v[1] = {acc[0][0]};
            fold_rows<L, 1>(v, pr);
            const float up = __shfl_xor(v[0], 32, 64);   // the up row sits 32 lanes above its gate row
            if (pr == 0 && rr < HALF) {
                int64_t slot, p;
                swiglu_row(st, slot, p);
                const int32_t e = ids_s[slot];
                const float g = v[0];
                const float h = g / (1.0f + expf(-g)) * up;
                reinterpret_cast<uint16_t *>(Y)[slot * ldy + p] =
                    (e >= 0 && e < E) ? float_to_bf16_rne(h) : (uint16_t)0;
            }
            acc[0][0] = 0.0f;
            return;
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = acc[u][t];
            const int u = fold_rows<L, U>(v, pr);
            if ((pr & (L / U - 1)) == 0) {
                const int64_t vrow =
                    MODE == VALU_MOE ? st * ROWS + u * R + rr : st_row0(st) + lane_row(u);
                if (vrow < rows_total) {
                    bool zero = false;
                    if (MODE == VALU_MOE) {
                        const int32_t e = ids_s[(uint32_t)vrow / (uint32_t)N];
                        zero = e < 0 || e >= E;
                    }
                    Y[t * ldy + vrow] = zero ? 0.0f : v[0];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                acc[u][t] = 0.0f;
    };

    int64_t cp_st = gw_c;
    int cp_b = 0;
    auto compute = [&](const ValuBuf<L, V, U> &buf) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int c = pr + L * (v + V * cp_b);
            uint4 xq[MT][4];
            float fct[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xq[t][j] = xs[t * KW + j * CPR + c];
                fct[t] = bs[t * CPR + c];
            }
            // Combine form: a slot whose id names no expert adds nothing at all (its loads read
            // expert 0, whose scales or products need not be finite).
            bool take = true;
            float wslot = 1.0f;
            if constexpr (MODE == VALU_COMBINE) {
                const int slot = (L * V * cp_b) / CPRW;
                const int32_t e = ids_s[slot];
                take = e >= 0 && e < E;
                wslot = rw_s[slot];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float s = half_bits_to_float(buf.s[v][u]) * wslot;
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const float a = fmaf(s, chunk_dot(buf.w[v][u], xq[t]) * fct[t], acc[u][t]);
                    acc[u][t] = take ? a : acc[u][t];
                }
            }
        }
        if (cp_b == nb - 1)
            finish(cp_st);
        const bool wrap = cp_b + 1 == nb;
        cp_b = wrap ? 0 : cp_b + 1;
        cp_st += wrap ? GW : 0;
    };

    // Items alternate between the two buffers; each block of code issues the next item's loads
    // and then consumes the previous ones.
    int64_t i = 0;
    for (; i + 2 < n_items; i += 2) {
        load(bufB, std::false_type{});
        compute(bufA);
        load(bufA, std::false_type{});
        compute(bufB);
    }
    if (i + 1 < n_items) {
        load(bufB, std::false_type{});
        compute(bufA);
        compute(bufB);
    } else {
        compute(bufA);
    }
}

// ------------------------------------------------------------------------------------------
// Split-K VALU GEMV (dense calls). The W = CPR / (L*CL) waves of a work-group share one contiguous
// range of rows and split K: wave w owns the K slice of chunks [w*L*CL, (w+1)*L*CL). Inside a wave,
// L lanes walk a row (lane p owns chunks p, p+L, ... of the slice) and R = 64/L rows sit side by
// side, so every load instruction covers R runs of L*16 contiguous bytes. Each lane keeps its CL
// chunks of activations (as fp16, re-paired) and their group factors 2^-e in registers for the whole
// kernel; they are requested before the first weights, so they are ready while the weights are
// still in flight, with no LDS staging and no barrier before the stream starts. Rows go U*R at a
// time with one item of prefetch and unconditional loads (rows past the block's end re-read its
// last row); per-row partial sums of the W slices meet in LDS once, after the last row, and are
// added in slice order.
//
// GATHER (one token): the combine form of the expert tail. The activation is the concatenation
// of the topk rows h[t] (K = topk*KR), and the L chunks that chunk step j of a wave covers lie in
// one slot t_j (KR/32 is a multiple of L), read from expert ids[t_j]'s rows with the partial sum
// scaled by the router weight w[t_j]: the block's rows come out as sum_t w[t] W_{ids[t]}[n] h[t].
// Slot, expert and weight are the same in every lane, so the row bases stay scalar. An invalid
// id reads expert 0 with weight 0.
// ------------------------------------------------------------------------------------------
template <int MT, int L, int CL, int U, bool GATHER>
__global__ void __launch_bounds__(512)
gemv_splitk_kernel(const uint4 *__restrict__ qw, const uint16_t *__restrict__ sc,
                   const uint16_t *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy,
                   int64_t N, int32_t K, int32_t rows_per_block, const int32_t *__restrict__ ids,
                   int32_t E, const float *__restrict__ rw, int32_t KR)
{
    static_assert(!GATHER || MT == 1, "the combine form is single-token");
    constexpr int R = 64 / L;
    constexpr int ROWS = U * R;
    extern __shared__ float red[];      // [MT][rows_per_block][W]
    const int CPR = (GATHER ? KR : K) >> 5;   // 16-byte chunks per weight row
    const int GPR = (GATHER ? KR : K) >> 7;
    const int W = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int pr = lane & (L - 1);
    const int rr = lane / L;
    const int cbase = wave * (L * CL) + pr;            // chunk j of this lane: cbase + L*j
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    const int64_t left = N - r0;
    const int rcount = (int)(left < rows_per_block ? left : rows_per_block);   // >= 1
    const int n_items = (rcount + ROWS - 1) / ROWS;

    struct Buf {
        uint4 w[CL][U];
        uint16_t s[CL][U];
    };
    // Item rows: a uniform first row plus fixed per-lane offsets; the block's last item is pulled
    // back to end at its last row (rows computed twice get identical bits), and a block with fewer
    // rows than one item clamps the lane rows instead.
    const bool full = rcount >= ROWS;
    // Lane row of row step u (recomputed for a run-time u rather than indexed).
    auto lane_row = [&](int u) -> int {
        const int r = u * R + rr;
        return (!full && r > rcount - 1) ? rcount - 1 : r;
    };
    uint32_t woff[U], soff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = lane_row(u);
        woff[u] = (uint32_t)((r * CPR + pr) * 16);
        soff[u] = (uint32_t)((r * GPR + (pr >> 2)) * 2);
    }
    auto item_row0 = [&](int item) -> int {
        if (!full)
            return 0;
        const int r = item * ROWS;
        return r + ROWS <= rcount ? r : rcount - ROWS;
    };
    // Per chunk step j: the weight-row base (in chunks and in scale groups) of its slot's expert
    // and the router weight; dense calls use row 0 of the matrix and weight 1.
    const uint4 *wq[CL];
    const uint16_t *sq[CL];
    float wt[CL];
    bool take[CL];   // combine form: false for a slot whose id names no expert (adds nothing)
#pragma unroll
    for (int j = 0; j < CL; ++j) {
        if constexpr (GATHER) {
            const int c0 = wave * (L * CL) + L * j;   // first chunk of step j, uniform
            const int slot = c0 / CPR;
            const int32_t e = __builtin_amdgcn_readfirstlane(ids[slot]);
            const bool ok = e >= 0 && e < E;
            const int64_t ee = ok ? e : 0;
            wq[j] = qw + ee * N * CPR + (c0 - slot * CPR);
            sq[j] = sc + ee * N * GPR + ((c0 - slot * CPR) >> 2);
            wt[j] = ok ? rw[slot] : 0.0f;
            take[j] = ok;
        } else {
            wq[j] = qw + wave * (L * CL) + L * j;
            sq[j] = sc + ((wave * (L * CL) + L * j) >> 2);
            wt[j] = 1.0f;
            take[j] = true;
        }
    }
    int ld_item = 0;
    auto load = [&](Buf &buf) {
        const int64_t row0 = r0 + item_row0(ld_item);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < CL; ++j) {
                const char *wb = reinterpret_cast<const char *>(wq[j] + row0 * CPR);
                const char *sb = reinterpret_cast<const char *>(sq[j] + row0 * GPR);
                buf.w[j][u] = load_weights(reinterpret_cast<const uint4 *>(wb + woff[u]));
                buf.s[j][u] = *reinterpret_cast<const uint16_t *>(sb + soff[u]);
            }
        ++ld_item;
    };

    // Activations first: load completions are counted in issue order.
    uint4 xq[MT][CL][4];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const uint4 *xg = reinterpret_cast<const uint4 *>(X + t * ldx);
#pragma unroll
        for (int j = 0; j < CL; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xq[t][j][q] = xg[4 * (cbase + L * j) + q];
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the activation loads ahead of the weight loads
    Buf bufA, bufB;
    load(bufA);
    // Stage the activations in registers as fp16: chunk cbase + L*j of a group sits in four
    // consecutive lanes (L is a multiple of 4 and chunk runs start at multiples of 4).
    float fct[MT][CL];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int j = 0; j < CL; ++j) {
            uint32_t m = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                m = abs_max8(xq[t][j][q], m);
            const int e = group_exponent(quad_max(fold_halves(m)));
            const float p = pow2f(e);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xq[t][j][q] = stage_words(xq[t][j][q], p);
            fct[t][j] = pow2f(-e);
        }
    }

    int cp_item = 0;
    auto compute = [&](const Buf &buf) {
        float acc[U][MT];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                acc[u][t] = 0.0f;
#pragma unroll
        for (int j = 0; j < CL; ++j)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float s = half_bits_to_float(buf.s[j][u]) * wt[j];
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const float a =
                        fmaf(s, chunk_dot(buf.w[j][u], xq[t][j]) * fct[t][j], acc[u][t]);
                    acc[u][t] = take[j] ? a : acc[u][t];
                }
            }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = acc[u][t];
            const int u = fold_rows<L, U>(v, pr);
            if ((pr & (L / U - 1)) == 0) {
                const int lr = item_row0(cp_item) + lane_row(u);
                red[((int64_t)t * rows_per_block + lr) * W + wave] = v[0];
            }
        }
        ++cp_item;
    };

    // The scheduling barriers keep each item's loads ahead of the previous item's arithmetic:
    // left alone, the compiler sinks them into it and then waits for every load in flight at the
    // top of the loop (4096 x 14336 and 8192 x 8192 at one token 2 % faster with them, 8192 x 8192
    // at 4 tokens on the 4x4x4 kernel 4 %).
    int i = 0;
    for (; i + 2 < n_items; i += 2) {
        load(bufB);
        __builtin_amdgcn_sched_barrier(0);
        compute(bufA);
        load(bufA);
        __builtin_amdgcn_sched_barrier(0);
        compute(bufB);
    }
    if (i + 1 < n_items) {
        load(bufB);
        __builtin_amdgcn_sched_barrier(0);
        compute(bufA);
        compute(bufB);
    } else {
        compute(bufA);
    }
    __syncthreads();
    for (int k = threadIdx.x; k < MT * rcount; k += blockDim.x) {
        const int t = k / rcount;
        const int lr = k - t * rcount;
        const float *pp = red + ((int64_t)t * rows_per_block + lr) * W;
        float v = 0.0f;
        for (int q = 0; q < W; ++q)
            v += pp[q];
        Y[t * ldy + r0 + lr] = v;
    }
}

// ------------------------------------------------------------------------------------------
// Split-K GEMV on the 4x4x4 matrix cores for 2..16 tokens. v_mfma_f32_4x4x4_16b_f16 computes 16
// independent 4x4x4 blocks per wave: block b lives in lanes 4b..4b+3, lane 4b+q supplies row q of
// A and column q of B (four consecutive k values each) and receives D[r][q], r = 0..3, in its
// four result registers. Here A holds weights and B activations (4 tokens per token group, TG
// groups). The 16 blocks form 16 / BR row groups of BR blocks, and the BR blocks of a row group
// take BR consecutive 16-byte chunks of K: lane 4b+q, b = BR h + c, reads chunk c of row 4h + q
// (per row, one instruction covers BR * 16 contiguous bytes, as a BR-lane row of the split-K VALU
// kernel does) and keeps chunk c of token 4g+q in registers for the whole kernel -- four times
// fewer activation registers than padding the tokens to 16 columns. A row step is 64 / BR rows;
// BR = 8 serves rows whose chunk count is a multiple of 8 but not of 16 (K = 2304). Each
// decoded weight word feeds two MFMAs per token group (k order 0,4,1,5 and 2,6,3,7, the order of
// the re-paired activations); a chunk's block sum is multiplied by the factor 2^-e of the token's
// group and by its row's fp16 scale, broadcast from lane 4b+r by DPP. After an item
// the BR blocks' partials of a row group are added by DPP row rotations and permlane swaps
// (all 16 lanes with the same lane % 4 and row group), and the waves of a
// work-group, which split K as in the split-K kernel, meet in LDS after the last item.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ f16x4_t as_f16x4(uint32_t a, uint32_t b)
{
    const uint2 v = {a, b};
    return __builtin_bit_cast(f16x4_t, v);
}

// Largest of a per-lane value over the lanes 4b + (lane % 4), b = 4k .. 4k + 3, of a DPP row
// (the four blocks that hold the chunks of one scale group of one token).
__device__ __forceinline__ uint32_t blocks_max4(uint32_t m)
{
    int x = (int)m;
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
    return (uint32_t)x;
}

// Sum of v over the BR lanes 4b + (lane % 4) of a row group, b = BR h .. BR h + BR - 1 (one value
// per block of a 4x4x4 MFMA): rotations by 4 and 8 lanes within a DPP row add its 4 blocks, the
// permlane swaps add the rows 16 and 32 lanes away.
template <int BR>
__device__ __forceinline__ float sum_over_blocks(float v)
{
    int x = __builtin_bit_cast(int, v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false));
    x = __builtin_bit_cast(int, v);
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
    v = swap_fold(v, v, 4);
    return BR == 16 ? swap_fold(v, v, 5) : v;
}

// Up to 16 waves when a lane holds one chunk per step (rows of 72 chunks need 9), else 8.
template <int TG, int CL, int U, int BR>
__global__ void __launch_bounds__(CL == 1 ? 1024 : 512)
gemv_mfma4_kernel(const uint4 *__restrict__ qw, const uint16_t *__restrict__ sc,
                  const uint16_t *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy,
                  int32_t M, int64_t N, int32_t K, int32_t rows_per_block)
{
    static_assert(BR == 8 || BR == 16, "a row group is 8 or 16 blocks");
    constexpr int R = 4 * (16 / BR);     // rows per row step: 4 rows per row group
    constexpr int ROWS = U * R;
    extern __shared__ float red[];      // [M][rows_per_block][W]
    const int CPR = K >> 5;
    const int GPR = K >> 7;
    const int W = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int q = lane & 3;              // row of A and token column of B within the block
    const int b = lane >> 2;             // block
    const int h = b / BR;                // row group: rows 4h .. 4h + 3 of a row step
    const int bc = b % BR;               // chunk of each run of BR chunks
    const int cw = wave * (BR * CL) + bc;   // this lane's first chunk; chunk step j adds BR j
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    const int64_t left = N - r0;
    const int rcount = (int)(left < rows_per_block ? left : rows_per_block);   // >= 1
    const int n_items = (rcount + ROWS - 1) / ROWS;
    // Rows of an item: a uniform first row plus row r of step u; the last item is pulled back to
    // end at the block's last row (rows computed twice get identical bits), and a block with fewer
    // rows than one item clamps the rows instead.
    const bool full = rcount >= ROWS;
    auto step_row = [&](int u, int r) -> int {
        const int x = u * R + r;
        return (!full && x > rcount - 1) ? rcount - 1 : x;
    };
    auto item_row0 = [&](int item) -> int {
        if (!full)
            return 0;
        const int r = item * ROWS;
        return r + ROWS <= rcount ? r : rcount - ROWS;
    };
    struct Buf {
        uint4 w[CL][U];
        uint16_t s[CL][U];
    };
    uint32_t woff[U], soff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = step_row(u, 4 * h + q);
        woff[u] = (uint32_t)((r * CPR + cw) * 16);
        soff[u] = (uint32_t)((r * GPR + (cw >> 2)) * 2);
    }
    int ld_item = 0;
    auto load = [&](Buf &buf) {
        const int64_t row0 = r0 + item_row0(ld_item);
        const char *wb = reinterpret_cast<const char *>(qw + row0 * CPR);
        const char *sb = reinterpret_cast<const char *>(sc + row0 * GPR);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < CL; ++j) {
                // chunk step j: BR chunks further along the row, BR / 4 scale groups
                buf.w[j][u] =
                    load_weights(reinterpret_cast<const uint4 *>(wb + woff[u] + 16 * BR * j));
                buf.s[j][u] = *reinterpret_cast<const uint16_t *>(sb + soff[u] + (BR / 2) * j);
            }
        ++ld_item;
    };

    // Activations first (load completions are counted in issue order): chunk cw + 16 j of token
    // 4g + q; token slots past M read token M-1 and their outputs are never stored.
    uint4 xq[TG][CL][4];
#pragma unroll
    for (int g = 0; g < TG; ++g) {
        const int t = 4 * g + q < M ? 4 * g + q : M - 1;
        const uint4 *xg = reinterpret_cast<const uint4 *>(X + (int64_t)t * ldx);
#pragma unroll
        for (int j = 0; j < CL; ++j)
#pragma unroll
            for (int w = 0; w < 4; ++w)
                xq[g][j][w] = xg[4 * (cw + BR * j) + w];
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the activation loads ahead of the weight loads
    Buf bufA, bufB;
    load(bufA);
    // Stage the activations in registers as fp16. The chunks of one scale group of token 4g + q
    // sit in lanes 4b + q for four consecutive blocks b of a DPP row (BR and the chunk steps are
    // multiples of 4).
    float fct[TG][CL];
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
        for (int j = 0; j < CL; ++j) {
            uint32_t m = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                m = abs_max8(xq[g][j][w], m);
            const int e = group_exponent(blocks_max4(fold_halves(m)));
            const float p = pow2f(e);
#pragma unroll
            for (int w = 0; w < 4; ++w)
                xq[g][j][w] = stage_words(xq[g][j][w], p);
            fct[g][j] = pow2f(-e);
        }

    int cp_item = 0;
    auto compute = [&](const Buf &buf) {
        f32x4_t acc[U][TG];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int g = 0; g < TG; ++g)
                acc[u][g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < CL; ++j)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                uint32_t p[4][4];
                unpack_chunk(buf.w[j][u], p);
                // scales of the block's rows 0..3 (lane 4b + r holds row r's)
                const int sv = buf.s[j][u];
                float s4[4];
                quad_scales((uint16_t)sv, s4);
#pragma unroll
                for (int g = 0; g < TG; ++g) {
                    f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint4 xv = xq[g][j][w];
                        d = __builtin_amdgcn_mfma_f32_4x4x4f16(
                            as_f16x4(p[w][0], p[w][1]), as_f16x4(xv.x, xv.y), d, 0, 0, 0);
                        d = __builtin_amdgcn_mfma_f32_4x4x4f16(
                            as_f16x4(p[w][2], p[w][3]), as_f16x4(xv.z, xv.w), d, 0, 0, 0);
                    }
                    const float f = fct[g][j];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[u][g][r] = fmaf(s4[r], d[r] * f, acc[u][g][r]);
                }
            }
        // The BR blocks' partials of each (row, token), then lane 4b + q with bc = r < 4 parks
        // row 4h + r's value for token 4g + q in LDS.
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int g = 0; g < TG; ++g) {
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[r] = sum_over_blocks<BR>(acc[u][g][r]);
                const int t = 4 * g + q;
                if (bc < 4 && t < M) {
                    const float val = bc == 0 ? v[0] : bc == 1 ? v[1] : bc == 2 ? v[2] : v[3];
                    const int lr = item_row0(cp_item) + step_row(u, 4 * h + bc);
                    red[((int64_t)t * rows_per_block + lr) * W + wave] = val;
                }
            }
        ++cp_item;
    };

    // The scheduling barriers keep each item's loads ahead of the previous item's arithmetic:
    // left alone, the compiler sinks them into it and then waits for every load in flight at the
    // top of the loop (4096 x 14336 and 8192 x 8192 at one token 2 % faster with them, 8192 x 8192
    // at 4 tokens on the 4x4x4 kernel 4 %).
    int i = 0;
    for (; i + 2 < n_items; i += 2) {
        load(bufB);
        __builtin_amdgcn_sched_barrier(0);
        compute(bufA);
        load(bufA);
        __builtin_amdgcn_sched_barrier(0);
        compute(bufB);
    }
    if (i + 1 < n_items) {
        load(bufB);
        __builtin_amdgcn_sched_barrier(0);
        compute(bufA);
        compute(bufB);
    } else {
        compute(bufA);
    }
    __syncthreads();
    for (int k = threadIdx.x; k < M * rcount; k += blockDim.x) {
        const int t = k / rcount;
        const int lr = k - t * rcount;
        const float *pp = red + ((int64_t)t * rows_per_block + lr) * W;
        float v = 0.0f;
        for (int w = 0; w < W; ++w)
            v += pp[w];
        Y[t * ldy + r0 + lr] = v;
    }
}

// ------------------------------------------------------------------------------------------
// Set-up shared by the grouped-expert GEMVs for several tokens (every work-group does it, in
// LDS). moe_group_entries groups the P = M*topk entries (token m, slot t) by expert id, in order
// of first appearance; ids outside [0, E) form one group of their own (key -1). A group of c
// entries becomes ceil(c / MT) virtual entries of up to MT entries: ve_e[v] is the expert (or
// -1), ve_tok[v*MT + j] the j-th entry or -1, and *nve_s the number of virtual entries.
// Scratch arrays key_s .. vbase_s hold P ints each. Ends without a barrier.
// ------------------------------------------------------------------------------------------
template <int MT>
__device__ void moe_group_entries(const int32_t *__restrict__ ids, int P, int32_t E,
                                  int32_t *key_s, int32_t *first_s, int32_t *rank_s,
                                  int32_t *cnt_s, int32_t *vbase_s, int32_t *ve_e,
                                  int32_t *ve_tok, int32_t *nve_s)
{
    for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int32_t e = ids[i];
        key_s[i] = (e >= 0 && e < E) ? e : -1;
        ve_e[i] = -1;
#pragma unroll
        for (int j = 0; j < MT; ++j)
            ve_tok[i * MT + j] = -1;
    }
    __syncthreads();
    // One pass over all P keys per entry, four keys per LDS read (the reads past P stay inside
    // the scratch arrays and are masked): the group's first entry f, this entry's rank r among
    // the earlier ones, and the group size c.
    const int4 *key4 = reinterpret_cast<const int4 *>(key_s);
    for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int32_t k = key_s[i];
        int f = i, r = 0, c = 0;
        for (int j0 = 0; j0 < P; j0 += 4) {
            const int4 kk = key4[j0 >> 2];
            const int32_t kv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = j0 + q;
                const bool m = j < P && kv[q] == k;
                const bool before = m && j < i;
                f = (before && r == 0) ? j : f;
                r += before ? 1 : 0;
                c += m ? 1 : 0;
            }
        }
        first_s[i] = f;
        rank_s[i] = r;
        cnt_s[i] = f == i ? (c + MT - 1) / MT : 0;   // virtual entries of the group (at its first)
    }
    __syncthreads();
    // Virtual entries of the groups whose first entry precedes i, summed in entry order.
    for (int i = threadIdx.x; i < P; i += blockDim.x) {
        int base = 0;
        for (int j = 0; j < i; ++j)
            base += cnt_s[j];
        vbase_s[i] = base;
        if (i == P - 1)
            nve_s[0] = base + cnt_s[i];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int v = vbase_s[first_s[i]] + rank_s[i] / MT;
        ve_tok[v * MT + rank_s[i] % MT] = i;
        if (rank_s[i] % MT == 0)
            ve_e[v] = key_s[i];
    }
}

// Activations of every token staged re-paired as [token][word j][chunk] (16 bytes each), with
// the per-chunk group factors 2^-e in bs[token][chunk]. The staging loop runs over the flat
// (token, word) index; its first kMoeXPre passes use words requested by moe_prefetch_activations
// before the expert grouping, so their latency overlaps the id load and the grouping, and only
// the rest (more than kMoeXPre * threads words) is loaded here. Ends without a barrier.
constexpr int kMoeXPre = 2;

__device__ __forceinline__ void moe_prefetch_activations(const uint16_t *__restrict__ X,
                                                         int64_t ldx, int M, int K,
                                                         uint4 (&pre)[kMoeXPre])
{
    const int KW = K >> 3;
    const int total = M * KW;
#pragma unroll
    for (int f = 0; f < kMoeXPre; ++f) {
        int idx = threadIdx.x + f * blockDim.x;
        idx = idx < total ? idx : total - 1;   // past the end: re-read the last word, unused
        const int t = idx / KW;
        pre[f] = reinterpret_cast<const uint4 *>(X + t * ldx)[idx - t * KW];
    }
}

__device__ void moe_stage_activations(const uint16_t *__restrict__ X, int64_t ldx, int M, int K,
                                      uint4 *xs, float *bs, const uint4 (&pre)[kMoeXPre])
{
    const int KW = K >> 3;
    const int CPR = K >> 5;
    const int total = M * KW;
    // The 16 words of a scale group sit in the 16 lanes of one DPP row and the same token (KW
    // and the thread count are multiples of 16), and a row is either all below `total` or all
    // above.
    auto stage = [&](int idx, uint4 v) {
        const int t = idx / KW;
        const int w = idx - t * KW;
        const int e = group_exponent(row_max16(fold_halves(abs_max8(v, 0u))));
        xs[t * KW + (w & 3) * CPR + (w >> 2)] = stage_words(v, pow2f(e));
        if ((w & 3) == 0)
            bs[t * CPR + (w >> 2)] = pow2f(-e);
    };
#pragma unroll
    for (int f = 0; f < kMoeXPre; ++f) {
        const int idx = threadIdx.x + f * blockDim.x;
        if (idx < total)
            stage(idx, pre[f]);
    }
    for (int idx = threadIdx.x + kMoeXPre * blockDim.x; idx < total; idx += blockDim.x) {
        const int t = idx / KW;
        stage(idx, reinterpret_cast<const uint4 *>(X + t * ldx)[idx - t * KW]);
    }
}

// ------------------------------------------------------------------------------------------
// Grouped-expert GEMV for M tokens with their own topk experts each: every expert selected by
// any token is streamed once per call and multiplied with all the tokens that chose it.
//
// Set-up (every work-group, identically, in LDS): the P = M*topk entries (token m, slot t) are
// grouped by expert id, in order of first appearance; ids outside [0, E) form one group of their
// own whose outputs are zero. A group of c entries becomes ceil(c / MT) virtual entries of up to
// MT (token, slot) pairs. Work items are (block of rows, virtual entry), block-major, so the
// virtual entries of one expert read the same rows in consecutive waves of a work-group and a
// second token of an expert finds those rows in the L2 cache; within an item the wave streams R
// rows of the entry's expert like the staged kernel (activations of all M tokens staged in LDS,
// re-paired, with their chunk factors) and accumulates one product per pair. Empty pair slots are
// skipped by wave-uniform branches around the arithmetic only (the loads stay straight-line).
// One pair per virtual entry (MT = 1) measured fastest on MI355X: larger MT costs registers, and
// so waves, on every expert for the few that more than one token chose. Block-major order also
// measured faster than expert-major order (63.9 against 93.6 us for 16 tokens x top-8 of 256),
// and 1024-thread groups no faster than 512.
// ------------------------------------------------------------------------------------------
constexpr int kMoeBatchedMaxThreads = 512;   // launch bound (the plan uses 512-thread groups)

template <int L, int V, int MT>
__global__ void __launch_bounds__(kMoeBatchedMaxThreads)
gemv_moe_batched_kernel(const uint4 *__restrict__ qw, const uint16_t *__restrict__ sc,
                        const uint16_t *__restrict__ X, int64_t ldx, float *__restrict__ Y,
                        const int32_t *__restrict__ ids, int32_t M, int32_t topk, int32_t E,
                        int64_t N, int32_t K)
{
    constexpr int R = 64 / L;
    extern __shared__ uint4 smem[];
    const int KW = K >> 3;
    const int CPR = K >> 5;
    const int GPR = K >> 7;
    const int P = M * topk;
    // Region A holds the grouping scratch first and the staged activations afterwards.
    const int a16 = (M * KW > (5 * P + 3) / 4) ? M * KW : (5 * P + 3) / 4;   // 16-byte units
    uint4 *xs = smem;                                              // [M][4][CPR]
    int32_t *key_s = reinterpret_cast<int32_t *>(smem);           // [P] expert id or -1
    int32_t *first_s = key_s + P;                                   // [P] first entry of the group
    int32_t *rank_s = first_s + P;                                  // [P] position in the group
    int32_t *cnt_s = rank_s + P;                                    // [P] virtual entries (firsts)
    int32_t *vbase_s = cnt_s + P;                                   // [P] first virtual entry
    float *bs = reinterpret_cast<float *>(smem + a16);            // [M][CPR]
    int32_t *ve_e = reinterpret_cast<int32_t *>(bs + M * CPR);    // [P] virtual entry's expert
    int32_t *ve_tok = ve_e + P;                                     // [P][MT] entries or -1
    int32_t *nve_s = ve_tok + P * MT;                               // [1]

    uint4 xpre[kMoeXPre];
    moe_prefetch_activations(X, ldx, M, K, xpre);
    moe_group_entries<MT>(ids, P, E, key_s, first_s, rank_s, cnt_s, vbase_s, ve_e, ve_tok,
                          nve_s);
    __syncthreads();   // the grouping scratch is overwritten by the activations below
    moe_stage_activations(X, ldx, M, K, xs, bs, xpre);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int pr = lane & (L - 1);
    const int rr = lane / L;
    const int wpb = blockDim.x >> 6;
    const int64_t gw = (int64_t)blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t GW = (int64_t)gridDim.x * wpb;
    const int nve = nve_s[0];
    // P * N < 2^31 (checked by the host), so block counts and item indices fit in 32 bits.
    const uint32_t n_blocks = (uint32_t)((N + R - 1) / R);
    const uint32_t n_super = (uint32_t)nve * n_blocks;
    const int nb = CPR / (L * V);
    if (gw >= (int64_t)n_super)
        return;
    const int64_t n_items = ((n_super - 1 - gw) / GW + 1) * nb;

    // Rows of block b of an expert: the last block is pulled back to end at row N - 1 (rows
    // computed twice give identical bits); with fewer than R rows the lane rows are clamped.
    auto lane_row = [&](uint32_t b) -> int64_t {
        if (N < R)
            return rr < N ? rr : N - 1;
        const int64_t r0 = (int64_t)b * R + R <= N ? (int64_t)b * R : N - R;
        return r0 + rr;
    };
    struct Buf {
        uint4 w[V];
        uint16_t s[V];
    };
    uint32_t ld_st = (uint32_t)gw;
    int ld_b = 0;
    auto load = [&](Buf &buf) {
        const uint32_t b = ld_st / (uint32_t)nve;
        const uint32_t v = ld_st - b * (uint32_t)nve;
        const int32_t e = ve_e[v];
        const int64_t row = (int64_t)(e >= 0 ? e : 0) * N + lane_row(b);
        const uint4 *wr = pick(e >= 0, qw + row * CPR, reinterpret_cast<const uint4 *>(X));
        const uint16_t *sr = pick(e >= 0, sc + row * GPR, X);
#pragma unroll
        for (int q = 0; q < V; ++q) {
            const int c = pr + L * (q + V * ld_b);
            buf.w[q] = load_weights(wr + c);
            buf.s[q] = sr[c >> 2];
        }
        const bool wrap = ld_b + 1 == nb;
        ld_b = wrap ? 0 : ld_b + 1;
        ld_st += wrap ? (uint32_t)GW : 0u;
    };

    float acc[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j)
        acc[j] = 0.0f;
    uint32_t cp_st = (uint32_t)gw;
    int cp_b = 0;
    auto compute = [&](const Buf &buf) {
        const uint32_t bb = cp_st / (uint32_t)nve;
        const uint32_t v = cp_st - bb * (uint32_t)nve;
        int tok[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j)
            tok[j] = ve_tok[v * MT + j];
#pragma unroll
        for (int q = 0; q < V; ++q) {
            const int c = pr + L * (q + V * cp_b);
            const float s = half_bits_to_float(buf.s[q]);
#pragma unroll
            for (int j = 0; j < MT; ++j) {
                if (j > 0 && tok[j] < 0)
                    break;
                const int m = tok[j] >= 0 ? tok[j] / topk : 0;
                uint4 xq[4];
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    xq[h] = xs[m * KW + h * CPR + c];
                acc[j] = fmaf(s, chunk_dot(buf.w[q], xq) * bs[m * CPR + c], acc[j]);
            }
        }
        if (cp_b == nb - 1) {
            const int32_t e = ve_e[v];
            const int64_t row = lane_row(bb);
#pragma unroll
            for (int j = 0; j < MT; ++j) {
                if (j > 0 && tok[j] < 0)
                    break;
                float r[1] = {acc[j]};
                fold_rows<L, 1>(r, pr);
                if (pr == 0 && tok[j] >= 0)
                    Y[(int64_t)tok[j] * N + row] = e >= 0 ? r[0] : 0.0f;
                acc[j] = 0.0f;
            }
        }
        const bool wrap = cp_b + 1 == nb;
        cp_b = wrap ? 0 : cp_b + 1;
        cp_st += wrap ? (uint32_t)GW : 0u;
    };

    Buf bufA, bufB;
    load(bufA);
    int64_t i = 0;
    for (; i + 2 < n_items; i += 2) {
        load(bufB);
        compute(bufA);
        load(bufA);
        compute(bufB);
    }
    if (i + 1 < n_items) {
        load(bufB);
        compute(bufA);
        compute(bufB);
    } else {
        compute(bufA);
    }
}

// ------------------------------------------------------------------------------------------
// Grouped-expert GEMV for several tokens on the 4x4x4 matrix cores. The same set-up as the VALU
// form (entries grouped by expert in LDS, activations of every token staged re-paired with their
// chunk factors), with virtual entries of up to 4 entries of one expert. Items are (virtual entry,
// block of rows) in expert-major order: the tokens that share an expert share its items, so the
// block-major order the VALU form needs for L2 reuse is not needed, and consecutive waves stream
// an expert's rows contiguously (16 tokens x top-8 of 256: 58.1 us against 60.5 block-major and
// 63.2 for the VALU form). Within an item the lanes take the 4x4x4 layout of the split-K MFMA
// kernel: lane 4b+q, b = BR h + c, reads chunk c (of each run of BR) of row 4h + q of each row
// step (64 / BR rows; U steps per block, one measured fastest), decodes it once, and supplies the
// activations of the virtual entry's slot q as column q of B -- so the tokens that chose an expert
// share every decode, and the products run on the matrix cores. Empty slots repeat slot 0's token
// (their outputs are never stored). After the last chunk batch of an item the BR blocks' partials
// are added across lanes and the lanes with c < 4 store row 4h + c for their slot's entry.
// ------------------------------------------------------------------------------------------
template <int BR, int CL, int U>
__global__ void __launch_bounds__(512)
gemv_moe_batched_mfma4_kernel(const uint4 *__restrict__ qw, const uint16_t *__restrict__ sc,
                              const uint16_t *__restrict__ X, int64_t ldx, float *__restrict__ Y,
                              const int32_t *__restrict__ ids, int32_t M, int32_t topk, int32_t E,
                              int64_t N, int32_t K)
{
    constexpr int MT = 4;
    constexpr int R = 4 * (16 / BR) * U; // rows per block: U row steps of 64 / BR rows
    extern __shared__ uint4 smem[];
    const int KW = K >> 3;
    const int CPR = K >> 5;
    const int GPR = K >> 7;
    const int P = M * topk;
    // Region A holds the grouping scratch first and the staged activations afterwards.
    const int a16 = (M * KW > (5 * P + 3) / 4) ? M * KW : (5 * P + 3) / 4;   // 16-byte units
    uint4 *xs = smem;                                              // [M][4][CPR]
    int32_t *key_s = reinterpret_cast<int32_t *>(smem);           // grouping scratch, 5 x [P]
    float *bs = reinterpret_cast<float *>(smem + a16);            // [M][CPR]
    int32_t *ve_e = reinterpret_cast<int32_t *>(bs + M * CPR);    // [P]
    int32_t *ve_tok = ve_e + P;                                     // [P][MT]
    int32_t *nve_s = ve_tok + P * MT;                               // [1]
    uint4 xpre[kMoeXPre];
    moe_prefetch_activations(X, ldx, M, K, xpre);
    moe_group_entries<MT>(ids, P, E, key_s, key_s + P, key_s + 2 * P, key_s + 3 * P,
                          key_s + 4 * P, ve_e, ve_tok, nve_s);
    __syncthreads();   // the grouping scratch is overwritten by the activations below
    moe_stage_activations(X, ldx, M, K, xs, bs, xpre);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int blk = lane >> 2;
    const int h = blk / BR;              // row group: rows 4h .. 4h + 3 of the block
    const int bc = blk % BR;             // chunk of each run of BR chunks
    const int wpb = blockDim.x >> 6;
    const int64_t gw = (int64_t)blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t GW = (int64_t)gridDim.x * wpb;
    const int nve = nve_s[0];
    // Token of an entry: entry / topk as a multiply-high by ceil(2^32 / topk), exact for
    // entry, topk <= 256 (entry * topk < 2^32).
    const uint32_t tk_magic = (uint32_t)((0x100000000ull + (uint32_t)topk - 1) / (uint32_t)topk);
    // P * N < 2^31 (checked by the host), so block counts and item indices fit in 32 bits.
    const uint32_t n_blocks = (uint32_t)((N + R - 1) / R);
    const uint32_t n_super = (uint32_t)nve * n_blocks;
    const int nb = CPR / (BR * CL);
    if (gw >= (int64_t)n_super)
        return;
    const int64_t n_items = ((n_super - 1 - gw) / GW + 1) * nb;

    // Rows of block b: a wave-uniform first row (the last block is pulled back to end at row
    // N - 1; rows computed twice give identical bits) plus fixed per-lane offsets (with fewer
    // than R rows, clamped to row N - 1).
    auto block_row0 = [&](uint32_t b) -> int64_t {
        if (N < R)
            return 0;
        return (int64_t)b * R + R <= N ? (int64_t)b * R : N - R;
    };
    auto lane_row = [&](int r) -> int { return N < R && r > N - 1 ? (int)N - 1 : r; };
    uint32_t woff[U], soff[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int r = lane_row((64 / BR) * u + 4 * h + q);
        woff[u] = (uint32_t)(r * CPR + bc);
        soff[u] = (uint32_t)(r * GPR);
    }
    struct Buf {
        uint4 w[CL][U];
        uint16_t s[CL][U];
    };
    // Cursors over the items: virtual entry v and block b (expert-major, st = v * n_blocks + b),
    // advanced by the grid's wave count without divisions after the first item.
    struct Cursor {
        uint32_t v, b;
        int batch;
    };
    const uint32_t gw_v = (uint32_t)GW / n_blocks, gw_b = (uint32_t)GW % n_blocks;
    auto advance = [&](Cursor &cur) {
        if (++cur.batch < nb)
            return;
        cur.batch = 0;
        cur.v += gw_v;
        cur.b += gw_b;
        if (cur.b >= n_blocks) {
            cur.b -= n_blocks;
            cur.v += 1;
        }
    };
    const Cursor first = {(uint32_t)gw / n_blocks, (uint32_t)gw % n_blocks, 0};
    Cursor ld = first;
    auto load = [&](Buf &buf) {
        // past the last item (clamped to a valid entry): loads of valid rows, never consumed
        const uint32_t v = ld.v < (uint32_t)nve ? ld.v : (uint32_t)nve - 1;
        const int32_t e = __builtin_amdgcn_readfirstlane(ve_e[v]);
        const int64_t row0 = (int64_t)(e >= 0 ? e : 0) * N + block_row0(ld.b);
        const uint4 *wr = pick(e >= 0, qw + row0 * CPR, reinterpret_cast<const uint4 *>(X));
        const uint16_t *sr = pick(e >= 0, sc + row0 * GPR, X);
        const uint32_t c0 = (uint32_t)(BR * CL * ld.batch);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // an invalid expert reads the activations (valid memory of K * 2 bytes per row
            // step's first row: the offsets stay below one row there)
            const uint32_t wo = e >= 0 ? woff[u] : (uint32_t)bc;
            const uint32_t so = e >= 0 ? soff[u] : 0u;
#pragma unroll
            for (int jj = 0; jj < CL; ++jj) {
                const uint32_t c = c0 + BR * jj;
                buf.w[jj][u] = load_weights(wr + wo + c);
                buf.s[jj][u] = sr[so + ((bc + c) >> 2)];
            }
        }
        advance(ld);
    };

    f32x4_t acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        acc[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    Cursor cp = first;
    auto compute = [&](const Buf &buf) {
        const uint32_t v = cp.v;
        const int cp_b = cp.batch;
        const int32_t e_q = ve_tok[v * MT + q];
        const uint32_t e_t = (uint32_t)(e_q >= 0 ? e_q : ve_tok[v * MT]);   // empty: slot 0
        const int m = (int)__umulhi(e_t, tk_magic);
#pragma unroll
        for (int j = 0; j < CL; ++j) {
            const int c = bc + BR * (j + CL * cp_b);   // this lane's chunk
            uint4 xv[4];                 // slot q's activations for chunk c, shared by the steps
#pragma unroll
            for (int w = 0; w < 4; ++w)
                xv[w] = xs[m * KW + w * CPR + c];
            const float f = bs[m * CPR + c];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                uint32_t p[4][4];
                unpack_chunk(buf.w[j][u], p);
                const int sv = buf.s[j][u];
                float s4[4];
                quad_scales((uint16_t)sv, s4);
                f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    d = __builtin_amdgcn_mfma_f32_4x4x4f16(
                        as_f16x4(p[w][0], p[w][1]), as_f16x4(xv[w].x, xv[w].y), d, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_4x4x4f16(
                        as_f16x4(p[w][2], p[w][3]), as_f16x4(xv[w].z, xv[w].w), d, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[u][r] = fmaf(s4[r], d[r] * f, acc[u][r]);
            }
        }
        if (cp_b == nb - 1) {
            const int32_t e = __builtin_amdgcn_readfirstlane(ve_e[v]);
            const int64_t r0 = block_row0(cp.b);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vv[r] = sum_over_blocks<BR>(acc[u][r]);
                if (bc < 4 && e_q >= 0) {
                    const float val = bc == 0 ? vv[0] : bc == 1 ? vv[1] : bc == 2 ? vv[2] : vv[3];
                    Y[(int64_t)e_q * N + r0 + lane_row((64 / BR) * u + 4 * h + bc)] =
                        e >= 0 ? val : 0.0f;
                }
                acc[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        advance(cp);
    };

    Buf bufA, bufB;
    load(bufA);
    int64_t i = 0;
    for (; i + 2 < n_items; i += 2) {
        load(bufB);
        compute(bufA);
        load(bufA);
        compute(bufB);
    }
    if (i + 1 < n_items) {
        load(bufB);
        compute(bufA);
        compute(bufB);
    } else {
        compute(bufA);
    }
}

// ------------------------------------------------------------------------------------------
// MFMA GEMV for 2..16 tokens (v_mfma_f32_16x16x32_f16), computed as D = X * W^T so that each
// lane's four outputs belong to one weight row: lane (i = l%16, g = l/16) supplies, for word j of
// chunk 4s+g of a group s, the 8 fp16 activations of token i (A operand, re-paired) and the 8
// decoded weights q of row i (B operand); D[4g+r][i] is token 4g+r of row i over the group. Each
// group total is multiplied by the factor 2^-e of token 4g+r's group and by row i's fp16 scale in
// fp32 -- one 2-byte scale load per tile and group.
//
// XLDS (K*32 bytes fit in LDS): the activations of all 16 token slots are staged once per work-group
// in fragment order ([group][word][lane], 16 bytes each) together with the per-(group, token)
// factors; work-groups are persistent and stream tiles of 16 rows in a flat (row block, group)
// sequence with one item of prefetch. Otherwise each wave reads its activation fragments from
// global memory with its weights, KS waves of a work-group split the groups of K, and their
// partial sums are added through LDS in a fixed order.
// Token slots past M read token M-1 (their outputs are never stored); rows past N re-read row
// N-1 (never stored). Every load is unconditional.
//
// LINES (XLDS, one tile per wave, an even number of groups per item): a lane of the B operand
// reads 16 bytes of one row, so an operand-order load covers 64 bytes of each of 16 rows (half
// lines, the second half served by L2, with L1 tag conflicts). Instead each pair of groups --
// one 128-byte line of every row -- is loaded by two whole-line instructions (lane l: row
// 8h + l/8, chunk l%8 of the line), passed through a per-wave LDS slot, and read back in
// operand order (lane (i, g) takes chunk g, then 4 + g, of row i).
//
// GLINES (activations from global memory, an even number of groups per item): the same
// whole-line weight loads for every tile, and the activation fragments loaded contiguously
// (instruction j' of a group: lane (i, g) reads the 16 bytes 4j' + g of token i's 256-byte
// group, so the four lanes of a token cover 64 contiguous bytes) and exchanged through LDS into
// operand order (lane (i, g), word j comes from lane (i, j) of instruction g).
//
// XROWS (activations from global memory): an operand-order activation load touches 32 lines
// (16 tokens, 16 bytes of each of a token's two lines per lane group). Instead each
// instruction reads the item's GU groups (256 * GU contiguous bytes) of 4 / GU token rows:
// 1 KB in 8 lines when the rows are 128-byte aligned. The item's chunks go through a per-wave
// LDS slot (XOR-swizzled so that the operand-order reads of 16 slots fall in distinct banks)
// and each lane reads its operand chunks back. With 8 slots (M <= 8) MFMA rows 8-15 repeat
// slots 0-7 (never stored) and half the loads go away.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ f16x8_t as_f16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    u32x4_t v = {a, b, c, d};
    return __builtin_bit_cast(f16x8_t, v);
}

__device__ __forceinline__ f16x8_t as_f16x8(uint4 v) { return as_f16x8(v.x, v.y, v.z, v.w); }

// Largest of a per-lane value over the lanes 16 and 32 apart (v_permlane16_swap and
// v_permlane32_swap with both operands holding it; the same exchange as swap_fold).
__device__ __forceinline__ uint32_t max_over_rows(uint32_t m)
{
    const auto r = __builtin_amdgcn_permlane16_swap(m, m, false, false);
    m = r[0] > r[1] ? (uint32_t)r[0] : (uint32_t)r[1];
    const auto q = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    return q[0] > q[1] ? (uint32_t)q[0] : (uint32_t)q[1];
}

// Scale words of an item: word k holds group k's fp16 scale in its low half. One 16-bit load per
// group and tile, so the scales need only their natural 2-byte alignment (dword loads of scale
// pairs would need 4).
template <int GU>
constexpr int mfma_scale_words() { return GU; }

// The 16-byte members come first: an x array placed after an odd number of scale pairs sits
// at an offset that is not a multiple of 16, and the compiler then kept part of the buffer in
// scratch memory.
template <int T, int GU, bool XLDS>
struct MfmaBuf {
    uint4 w[GU][T];
    uint4 x[XLDS ? 1 : GU][4];     // activation fragments (global-memory mode only)
    uint32_t s[mfma_scale_words<GU>()][T];   // raw scale words, converted where they are used
};

// The GU scales of one row for groups s..s+GU-1. The words are kept whole until use:
// converting right after the load would make that point wait for the load.
template <int GU>
__device__ __forceinline__ void load_scales(const char *p, uint32_t (&out)[mfma_scale_words<GU>()])
{
#pragma unroll
    for (int k = 0; k < GU; ++k)
        out[k] = reinterpret_cast<const uint16_t *>(p)[k];
}

// Scale of group u of an item from its raw words.
template <int GU>
__device__ __forceinline__ float mfma_scale(const uint32_t *words, int u)
{
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    return (float)__builtin_bit_cast(h2_t, words[u]).x;
}

template <int T, int KS, int XMODE, int GU, int WPB>
__global__ void __launch_bounds__(64 * WPB)
gemv_mfma_kernel(const uint4 *__restrict__ qw, const uint16_t *__restrict__ sc,
                 const uint16_t *__restrict__ X, int64_t ldx, float *__restrict__ Y, int64_t ldy,
                 int32_t M, int64_t N, int32_t K)
{
    constexpr bool XLDS = XMODE == 1 || XMODE == 2 || XMODE == 4;   // activations staged in LDS
    constexpr bool LINES = XMODE == 2 || XMODE == 4;   // whole-line weight loads permuted via LDS
    // Token slots staged: 16, or 8 when M <= 8 (XMODE 4), where MFMA rows 8-15 read slots 0-7
    // again; their outputs are never stored.
    constexpr int SLOTS = XMODE == 4 ? 8 : 16;
    constexpr bool GLINES = XMODE == 3;        // global activations, whole-line loads via LDS
    constexpr bool XROWS = XMODE == 5 || XMODE == 6;   // global activations, token-row loads
    constexpr int XSLOTS = XMODE == 6 ? 8 : 16;        // XROWS: token slots loaded per item
    constexpr int XCH = 16 * GU;                       // XROWS: 16-byte chunks of a token's item
    constexpr int NXI = XROWS ? XSLOTS * GU / 4 : 4 * GU;   // activation loads per item and lane
    static_assert(!LINES || (T == 1 && GU % 2 == 0), "line loads pair the groups of one tile");
    static_assert(!GLINES || GU % 2 == 0, "line loads pair the groups of an item");
    static_assert(!XROWS || GU == 1 || GU == 2 || GU == 4, "a token's item spans 16-64 lanes");
    static_assert(WPB % KS == 0, "waves per block must be a multiple of the K split");
    constexpr int RG = WPB / KS;               // row groups (waves with distinct rows) per block
    constexpr int TROWS = 16 * T;              // rows per wave item
    using Buf = MfmaBuf<T, GU, XLDS>;
    extern __shared__ uint4 lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15;
    const int g = lane >> 4;
    const int ks = wave % KS;
    const int rg = wave / KS;
    const int CPR = K >> 5;
    const int GPR = K >> 7;
    const int tok = i < M ? i : M - 1;

    // Rows of a wave: base(rb) + lane_row[t] for tile t. The base of the last row block is pulled
    // back so that the block ends at row N-1 (rows computed twice get identical bits); when N is
    // smaller than one row block the lane rows are clamped instead. Addresses are a wave-uniform
    // base plus a per-lane 32-bit byte offset fixed for the whole kernel.
    const int64_t RGT = RG * TROWS;
    const int64_t n_rb = (N + RGT - 1) / RGT;
    const bool full = N >= RGT;
    uint32_t woff[T], soff[T];
    int lane_row[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        int r = rg * TROWS + 16 * t + i;
        if (!full && r > N - 1)
            r = (int)N - 1;
        lane_row[t] = r;
        woff[t] = (uint32_t)((r * CPR + g) * 16);
        soff[t] = (uint32_t)(r * GPR * 2);
    }
    auto rb_row0 = [&](int64_t rb) -> int64_t {
        if (!full)
            return 0;
        const int64_t r0 = rb * RGT;
        return r0 + RGT <= N ? r0 : N - RGT;
    };
    // Whole-line loads: instruction h of a line pair reads rows 8h + lane/8 of tile t.
    uint32_t loff[T][2];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int r = rg * TROWS + 16 * t + 8 * h + (lane >> 3);
            if (!full && r > N - 1)
                r = (int)N - 1;
            loff[t][h] = (uint32_t)((r * CPR + (lane & 7)) * 16);
        }
    // One group of every tile: D[4g+r][i] over the group's 128 k values, times the factor 2^-e of
    // token 4g+r's group (fac[r]) and row i's scale.
    auto mma_group = [&](const uint4 (&wv)[T], const float (&scv)[T], const f16x8_t xb[4],
                         f32x4_t fac, f32x4_t (&acc)[T]) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            uint32_t p[4][4];
            unpack_chunk(wv[t], p);
            f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    xb[j], as_f16x8(p[j][0], p[j][1], p[j][2], p[j][3]), d, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[t][r] = fmaf(scv[t], d[r] * fac[r], acc[t][r]);
        }
    };
    auto store = [&](int64_t rb, const f32x4_t (&acc)[T]) {
        const int64_t r0 = rb_row0(rb);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int64_t row = r0 + lane_row[t];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g + r;
                if (m < M)
                    Y[(int64_t)m * ldy + row] = acc[t][r];
            }
        }
    };
    auto wbase = [&](int64_t rb, int s_) {
        return reinterpret_cast<const char *>(qw + rb_row0(rb) * CPR + 4 * s_);
    };
    auto sbase = [&](int64_t rb, int s_) {
        return reinterpret_cast<const char *>(sc + rb_row0(rb) * GPR + s_);
    };

    if constexpr (XLDS) {
        static_assert(KS == 1, "staged activations serve whole rows");
        uint4 *xl = lds;                                                 // [GPR][4][4*SLOTS]
        float *offl = reinterpret_cast<float *>(lds + GPR * 16 * SLOTS);   // [GPR][16]
        uint4 *stage = lds + GPR * (16 * SLOTS + 4) + wave * GU * 64;     // LINES: [GU/2][2][64]
        // A flat sequence of (row block, run of GU groups) items for this work-group.
        const int cpr_items = GPR / GU;
        const bool active = blockIdx.x < n_rb;
        const int64_t rb_first = active ? blockIdx.x : n_rb - 1;
        const int64_t n_items = ((n_rb - 1 - rb_first) / gridDim.x + 1) * cpr_items;
        int64_t ld_rb = rb_first;
        int ld_s = 0;
        auto load = [&](Buf &buf) {
            const int64_t rb = ld_rb < n_rb ? ld_rb : n_rb - 1;
            const char *wb = wbase(rb, ld_s);
            const char *sb = sbase(rb, ld_s);
            // Scales first: the compiler finishes their words (moves, shifts) where they arrive
            // and waits for them there, which then does not wait for the item's other loads
            // (28672 x 4096 and 163840 x 2304 at 16 tokens 1 % faster, with the scheduling
            // barriers of the loop below).
#pragma unroll
            for (int t = 0; t < T; ++t) {
                uint32_t sv[mfma_scale_words<GU>()];
                load_scales<GU>(sb + soff[t], sv);
#pragma unroll
                for (int k = 0; k < mfma_scale_words<GU>(); ++k)
                    buf.s[k][t] = sv[k];
            }
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int u = 0; u < GU; ++u) {
                    // LINES: buf.w[2p + h] holds instruction h of line pair p (whole lines)
                    const uint32_t o = LINES ? loff[0][u & 1] + 128 * (u >> 1) : woff[t] + 64 * u;
                    buf.w[u][t] = load_weights(reinterpret_cast<const uint4 *>(wb + o));
                }
            const bool wrap = ld_s + GU == GPR;
            ld_s = wrap ? 0 : ld_s + GU;
            ld_rb += wrap ? gridDim.x : 0;
        };
        Buf bufA, bufB;
        load(bufA);

        // Stage the token slots as fp16, one (group s, MFMA row m) per thread: the group's 16
        // activation words of the token in slot m % SLOTS (rows past M repeat token M-1; with 8
        // slots, rows 8-15 read slots 0-7 again), scaled by the group's power of two into
        // fragment order ([group][word j][chunk gg][slot]), and its factor 2^-e for row m.
        for (int idx = threadIdx.x; idx < GPR * 16; idx += blockDim.x) {
            const int s = idx >> 4, m = idx & 15;
            const int slot = m & (SLOTS - 1);
            const int tm = slot < M ? slot : M - 1;
            const uint4 *xr = reinterpret_cast<const uint4 *>(X + (int64_t)tm * ldx) + 16 * s;
            // All 16 words in flight at once, then the maximum and the conversion from registers.
            uint4 xv[16];
#pragma unroll
            for (int q = 0; q < 16; ++q)
                xv[q] = xr[q];
            uint32_t mx = 0;
#pragma unroll
            for (int q = 0; q < 16; ++q)
                mx = abs_max8(xv[q], mx);
            const int e = group_exponent(fold_halves(mx));
            offl[idx] = pow2f(-e);
            if (m < SLOTS) {
                const float pe = pow2f(e);
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    xl[(s * 4 + (q & 3)) * (4 * SLOTS) + (q >> 2) * SLOTS + m] =
                        stage_words(xv[q], pe);
            }
        }
        __syncthreads();
        if (!active)
            return;

        f32x4_t acc[T];
#pragma unroll
        for (int t = 0; t < T; ++t)
            acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        int64_t cp_rb = rb_first;
        int cp_s = 0;
        auto compute = [&](const Buf &buf) {
            uint4 wl[GU][T];
            if constexpr (LINES) {
                // Whole lines in, operand order out: lane (i, g) takes chunk g (even group) and
                // 4 + g (odd group) of row i, held by lane 8 (i % 8) + ... of instruction i / 8.
#pragma unroll
                for (int u = 0; u < GU; ++u)
                    stage[u * 64 + lane] = buf.w[u][0];
                const int src = 8 * (i & 7) + g;
                const int hh = i >> 3;
#pragma unroll
                for (int p2 = 0; p2 < GU / 2; ++p2) {
                    wl[2 * p2][0] = stage[(2 * p2 + hh) * 64 + src];
                    wl[2 * p2 + 1][0] = stage[(2 * p2 + hh) * 64 + src + 4];
                }
            } else {
#pragma unroll
                for (int u = 0; u < GU; ++u)
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        wl[u][t] = buf.w[u][t];
            }
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int s = cp_s + u;
                f16x8_t xb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xb[j] = as_f16x8(xl[(s * 4 + j) * (4 * SLOTS) + (i & (SLOTS - 1)) + SLOTS * g]);
                const float4 f4 = *reinterpret_cast<const float4 *>(offl + s * 16 + 4 * g);
                const f32x4_t fac = {f4.x, f4.y, f4.z, f4.w};
                float scv[T];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    uint32_t sw[mfma_scale_words<GU>()];
#pragma unroll
                    for (int k = 0; k < mfma_scale_words<GU>(); ++k)
                        sw[k] = buf.s[k][t];
                    scv[t] = mfma_scale<GU>(sw, u);
                }
                mma_group(wl[u], scv, xb, fac, acc);
            }
            if (cp_s + GU == GPR) {
                store(cp_rb, acc);
#pragma unroll
                for (int t = 0; t < T; ++t)
                    acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
            const bool wrap = cp_s + GU == GPR;
            cp_s = wrap ? 0 : cp_s + GU;
            cp_rb += wrap ? gridDim.x : 0;
        };
        int64_t it = 0;
        for (; it + 2 < n_items; it += 2) {
            load(bufB);
            __builtin_amdgcn_sched_barrier(0);
            compute(bufA);
            load(bufA);
            __builtin_amdgcn_sched_barrier(0);
            compute(bufB);
        }
        if (it + 1 < n_items) {
            load(bufB);
            __builtin_amdgcn_sched_barrier(0);
            compute(bufA);
            compute(bufB);
        } else {
            compute(bufA);
        }
    } else {
        // One row block per work-group; KS waves split the groups of K into runs of GU.
        f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);           // [WPB][T][64]
        // Staging per wave after the reduction slots. GLINES: weights [T][GU][64], then activation
        // fragments [GU][4][64] (16 bytes each). XROWS: the item's activations, [XSLOTS][XCH]
        // chunks, chunk c of slot m at position (m * XCH + c) ^ (m % 16) (see the loads below).
        constexpr int RED = KS > 1 ? WPB * T * 64 : 0;
        constexpr int STG = GLINES ? (T + 4) * GU * 64 : XROWS ? NXI * 64 : 0;
        uint4 *stage_w = lds + RED + wave * STG;
        uint4 *stage_x = GLINES ? stage_w + T * GU * 64 : stage_w;
        // Per wave, the factors 2^-e of the item's groups for the 16 token rows: [GU][16].
        float *stage_f = reinterpret_cast<float *>(lds + RED + WPB * STG) + wave * GU * 16;
        const int64_t rb = blockIdx.x;
        const int gpk = GPR / KS;
        const int n_items = gpk / GU;
        const uint4 *xp = reinterpret_cast<const uint4 *>(X + (int64_t)tok * ldx) + (GLINES ? g : 4 * g);
        int ld_s = ks * gpk;
        const int s_last = ks * gpk + (n_items - 1) * GU;   // loads past the slice re-read its last item
        // XROWS: instruction q of an item fills positions 64q + lane of the wave's staging slot,
        // so each instruction reads XCH contiguous chunks (GU groups) of 4 / GU token rows: 8
        // whole lines. Position p holds chunk p ^ (m % 16) of slot m = p / XCH (the XOR stays
        // within the slot's 16-chunk group), which spreads the operand-order reads of the 16
        // slots over distinct banks. Slots past M read token M-1.
        int64_t xq[XROWS ? NXI : 1];
        if constexpr (XROWS) {
#pragma unroll
            for (int q = 0; q < NXI; ++q) {
                const int pos = 64 * q + lane;
                const int m = pos / XCH;
                const int c = (pos ^ (m & 15)) % XCH;
                xq[q] = (int64_t)(m < M ? m : M - 1) * (ldx >> 3) + c;
            }
        }
        auto load = [&](Buf &buf) {
            const int s_ = ld_s < s_last ? ld_s : s_last;
            const char *wb = wbase(rb, s_);
            const char *sb = sbase(rb, s_);
            if constexpr (XROWS) {
                const uint4 *xi = reinterpret_cast<const uint4 *>(X) + (int64_t)s_ * 16;
#pragma unroll
                for (int q = 0; q < NXI; ++q)
                    buf.x[q / 4][q % 4] = xi[xq[q]];
            } else {
#pragma unroll
                for (int u = 0; u < GU; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        buf.x[u][j] = xp[16 * (s_ + u) + (GLINES ? 4 * j : j)];
            }
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int u = 0; u < GU; ++u) {
                    const uint32_t o = GLINES ? loff[t][u & 1] + 128 * (u >> 1) : woff[t] + 64 * u;
                    buf.w[u][t] = load_weights(reinterpret_cast<const uint4 *>(wb + o));
                }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                uint32_t sv[mfma_scale_words<GU>()];
                load_scales<GU>(sb + soff[t], sv);
#pragma unroll
                for (int k = 0; k < mfma_scale_words<GU>(); ++k)
                    buf.s[k][t] = sv[k];
            }
            ld_s += GU;
        };
        f32x4_t acc[T];
#pragma unroll
        for (int t = 0; t < T; ++t)
            acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        auto compute = [&](const Buf &buf) {
            uint4 wl[GU][T];
            uint4 xr[GU][4];
            if constexpr (GLINES) {
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int u = 0; u < GU; ++u)
                        stage_w[(t * GU + u) * 64 + lane] = buf.w[u][t];
#pragma unroll
                for (int u = 0; u < GU; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        stage_x[(u * 4 + j) * 64 + lane] = buf.x[u][j];
                const int src = 8 * (i & 7) + g;
                const int hh = i >> 3;
#pragma unroll
                for (int t = 0; t < T; ++t)
#pragma unroll
                    for (int p2 = 0; p2 < GU / 2; ++p2) {
                        wl[2 * p2][t] = stage_w[(t * GU + 2 * p2 + hh) * 64 + src];
                        wl[2 * p2 + 1][t] = stage_w[(t * GU + 2 * p2 + hh) * 64 + src + 4];
                    }
#pragma unroll
                for (int u = 0; u < GU; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        xr[u][j] = stage_x[(u * 4 + g) * 64 + i + 16 * j];
            } else if constexpr (XROWS) {
                // Token rows in, operand order out: lane (i, g) takes chunks 4g..4g+3 of each group
                // of slot i % XSLOTS.
#pragma unroll
                for (int q = 0; q < NXI; ++q)
                    stage_x[64 * q + lane] = buf.x[q / 4][q % 4];
                const int m = i & (XSLOTS - 1);
#pragma unroll
                for (int u = 0; u < GU; ++u) {
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        wl[u][t] = buf.w[u][t];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        xr[u][j] = stage_x[m * XCH + 16 * u + ((4 * g + j) ^ (m & 15))];
                }
            } else {
#pragma unroll
                for (int u = 0; u < GU; ++u) {
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        wl[u][t] = buf.w[u][t];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        xr[u][j] = buf.x[u][j];
                }
            }
            // Stage each group of the item as fp16: lane (i, g) holds chunk g of token i's group,
            // so the four chunks of a token sit 16 lanes apart; lane (i, 0) parks the factor of
            // token i in the wave's LDS slot and lane (i, g) reads those of tokens 4g..4g+3.
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                uint32_t mx = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    mx = abs_max8(xr[u][j], mx);
                const int e = group_exponent(max_over_rows(fold_halves(mx)));
                const float pe = pow2f(e);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xr[u][j] = stage_words(xr[u][j], pe);
                if (g == 0)
                    stage_f[u * 16 + i] = pow2f(-e);
                f16x8_t xb[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xb[j] = as_f16x8(xr[u][j]);
                const float4 f4 = *reinterpret_cast<const float4 *>(stage_f + u * 16 + 4 * g);
                const f32x4_t fac = {f4.x, f4.y, f4.z, f4.w};
                float scv[T];
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    uint32_t sw[mfma_scale_words<GU>()];
#pragma unroll
                    for (int k = 0; k < mfma_scale_words<GU>(); ++k)
                        sw[k] = buf.s[k][t];
                    scv[t] = mfma_scale<GU>(sw, u);
                }
                mma_group(wl[u], scv, xb, fac, acc);
            }
        };
        // Two item buffers: the loads of item it + 1 are issued before item it is computed. These
        // forms hold 16 token slots of activation fragments per item in registers; a third buffer
        // measured slower (8192 x 8192 at 8-16 tokens: 14.5-16.5 against 13.3-16.1 us). Loading
        // the scales first or pinning the loads with scheduling barriers, which helps the staged
        // forms above, measured 1-6 % slower here (14336 x 2048 and 8192 x 8192 at 8-16 tokens).
        Buf bufA, bufB;
        load(bufA);
        int it = 0;
        for (; it + 2 <= n_items; it += 2) {
            load(bufB);
            compute(bufA);
            load(bufA);
            compute(bufB);
        }
        if (it < n_items)
            compute(bufA);
        if (KS > 1) {
            if (ks != 0) {
#pragma unroll
                for (int t = 0; t < T; ++t)
                    red[(wave * T + t) * 64 + lane] = acc[t];
            }
            __syncthreads();
            if (ks != 0)
                return;
#pragma unroll
            for (int k2 = 1; k2 < KS; ++k2)
#pragma unroll
                for (int t = 0; t < T; ++t)
                    acc[t] += red[((rg * KS + k2) * T + t) * 64 + lane];
        }
        store(rb, acc);
    }
}

// ------------------------------------------------------------------------------------------
// Test support: the signed value of every nibble, decoded with the same unpack_word as the GEMVs.
// ------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
unpack_kernel(const uint32_t *__restrict__ qw, int8_t *__restrict__ out, int64_t words)
{
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < words;
         w += (int64_t)gridDim.x * blockDim.x) {
        uint32_t p[4];
        unpack_word(qw[w], p);
        int8_t q[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2_t h = __builtin_bit_cast(f16x2_t, p[i]);
            q[i] = (int8_t)(int)h.x;
            q[i + 4] = (int8_t)(int)h.y;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            out[8 * w + i] = q[i];
    }
}

// ------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------
template <int MT, int L, int V, int U, int MODE>
static hipError_t launch_valu_t(const GemvArgs &a, const Plan &p, hipStream_t stream)
{
    auto kern = gemv_valu_kernel<MT, L, V, U, MODE>;
    void *args[] = {(void *)&a.qweight, (void *)&a.scales, (void *)&a.X,  (void *)&a.ldx,
                    (void *)&a.Y,       (void *)&a.ldy,    (void *)&a.ids, (void *)&a.topk,
                    (void *)&a.E,       (void *)&a.N,      (void *)&a.K,   (void *)&a.route_w,
                    (void *)&a.KR};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(p.blocks), dim3(p.threads),
                           args, (size_t)p.lds_bytes, stream);
}

template <int MT, int L, int CL, int U, bool GATHER>
static hipError_t launch_splitk_t(const GemvArgs &a, const Plan &p, hipStream_t stream)
{
    auto kern = gemv_splitk_kernel<MT, L, CL, U, GATHER>;
    int32_t rpb = (int32_t)p.rows_per_block;
    void *args[] = {(void *)&a.qweight, (void *)&a.scales, (void *)&a.X,   (void *)&a.ldx,
                    (void *)&a.Y,       (void *)&a.ldy,    (void *)&a.N,   (void *)&a.K,
                    (void *)&rpb,       (void *)&a.ids,    (void *)&a.E,   (void *)&a.route_w,
                    (void *)&a.KR};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(p.blocks), dim3(p.threads),
                           args, (size_t)p.lds_bytes, stream);
}

template <int BR, int CL, int U>
static hipError_t launch_moe_batched_mfma4_t(const GemvArgs &a, const Plan &p, hipStream_t stream)
{
    auto kern = gemv_moe_batched_mfma4_kernel<BR, CL, U>;
    void *args[] = {(void *)&a.qweight, (void *)&a.scales, (void *)&a.X,    (void *)&a.ldx,
                    (void *)&a.Y,       (void *)&a.ids,    (void *)&a.M,    (void *)&a.topk,
                    (void *)&a.E,       (void *)&a.N,      (void *)&a.K};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(p.blocks), dim3(p.threads),
                           args, (size_t)p.lds_bytes, stream);
}

template <int TG, int CL, int U, int BR>
static hipError_t launch_mfma4_t(const GemvArgs &a, const Plan &p, hipStream_t stream)
{
    auto kern = gemv_mfma4_kernel<TG, CL, U, BR>;
    int32_t rpb = (int32_t)p.rows_per_block;
    void *args[] = {(void *)&a.qweight, (void *)&a.scales, (void *)&a.X, (void *)&a.ldx,
                    (void *)&a.Y,       (void *)&a.ldy,    (void *)&a.M, (void *)&a.N,
                    (void *)&a.K,       (void *)&rpb};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(p.blocks), dim3(p.threads),
                           args, (size_t)p.lds_bytes, stream);
}

constexpr int kMoeBatchedMT = 1;   // tokens accumulated per pass over an expert's rows

template <int L, int V>
static hipError_t launch_moe_batched_t(const GemvArgs &a, const Plan &p, hipStream_t stream)
{
    auto kern = gemv_moe_batched_kernel<L, V, kMoeBatchedMT>;
    void *args[] = {(void *)&a.qweight, (void *)&a.scales, (void *)&a.X,    (void *)&a.ldx,
                    (void *)&a.Y,       (void *)&a.ids,    (void *)&a.M,    (void *)&a.topk,
                    (void *)&a.E,       (void *)&a.N,      (void *)&a.K};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(p.blocks), dim3(p.threads),
                           args, (size_t)p.lds_bytes, stream);
}

template <int T, int KS, int XMODE, int GU, int WPB>
static hipError_t launch_mfma_t(const GemvArgs &a, const Plan &p, hipStream_t stream)
{
    auto kern = gemv_mfma_kernel<T, KS, XMODE, GU, WPB>;
    void *args[] = {(void *)&a.qweight, (void *)&a.scales, (void *)&a.X, (void *)&a.ldx,
                    (void *)&a.Y,       (void *)&a.ldy,    (void *)&a.M, (void *)&a.N,
                    (void *)&a.K};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(p.blocks), dim3(64 * WPB),
                           args, (size_t)p.lds_bytes, stream);
}

#define W4A16_VALU_CASE(MT_, L_, V_, U_)                                                     \
    if (p.MT == MT_ && p.L == L_ && p.V == V_ && p.U == U_ && p.mode == PLAN_MODE_DENSE)       \
        return launch_valu_t<MT_, L_, V_, U_, VALU_DENSE>(a, p, stream);                      \
    if (MT_ == 1 && p.MT == MT_ && p.L == L_ && p.V == V_ && p.U == U_ &&                    \
        p.mode == PLAN_MODE_MOE)                                                              \
        return launch_valu_t<(MT_ == 1 ? 1 : 1), L_, V_, U_, VALU_MOE>(a, p, stream);

#define W4A16_TAIL_CASE(L_, V_)                                                              \
    if (p.MT == 1 && p.L == L_ && p.V == V_ && p.U == 1 && p.mode == PLAN_MODE_COMBINE)       \
        return launch_valu_t<1, L_, V_, 1, VALU_COMBINE>(a, p, stream);                       \
    if (L_ <= 32 && p.MT == 1 && p.L == L_ && p.V == V_ && p.U == 1 &&                        \
        p.mode == PLAN_MODE_SWIGLU)                                                           \
        return launch_valu_t<1, (L_ <= 32 ? L_ : 32), V_, 1, VALU_SWIGLU>(a, p, stream);

#define W4A16_SPLITK_CASE(MT_, L_, CL_, U_)                                                  \
    if (p.MT == MT_ && p.L == L_ && p.V == CL_ && p.U == U_ && p.mode == PLAN_MODE_DENSE)      \
        return launch_splitk_t<MT_, L_, CL_, U_, false>(a, p, stream);

#define W4A16_GATHER_CASE(L_, CL_)                                                           \
    if (p.MT == 1 && p.L == L_ && p.V == CL_ && p.U == 1 && p.mode == PLAN_MODE_COMBINE)      \
        return launch_splitk_t<1, L_, CL_, 1, true>(a, p, stream);

#define W4A16_MFMA_CASE(T_, KS_, XL_, GU_, WPB_)                                             \
    if (p.T == T_ && p.KS == KS_ && p.xlds == xmode_xlds(XL_) && p.lines == xmode_lines(XL_) && \
        p.slots8 == xmode_slots8(XL_) && p.trows == xmode_trows(XL_) && p.V == GU_ &&          \
        p.threads == 64 * WPB_)                                                              \
        return launch_mfma_t<T_, KS_, XL_, GU_, WPB_>(a, p, stream);

#define W4A16_MFMA4_CASE(TG_, CL_, U_, BR_)                                                  \
    if (p.MT == TG_ && p.V == CL_ && p.U == U_ && p.L == BR_)                                \
        return launch_mfma4_t<TG_, CL_, U_, BR_>(a, p, stream);

#define W4A16_MOE_BATCHED_CASE(L_, V_)                                                       \
    if (p.L == L_ && p.V == V_)                                                              \
        return launch_moe_batched_t<L_, V_>(a, p, stream);

#define W4A16_MOE_BATCHED_MFMA4_CASE(BR_, CL_, U_)                                            \
    if (p.L == BR_ && p.V == CL_ && p.U == U_)                                               \
        return launch_moe_batched_mfma4_t<BR_, CL_, U_>(a, p, stream);

hipError_t launch(const GemvArgs &a, const Plan &p, hipStream_t stream)
{
    if (p.kind == PLAN_MOE_BATCHED) {
        W4A16_MOE_BATCHED_CONFIGS(W4A16_MOE_BATCHED_CASE)
        return hipErrorInvalidConfiguration;
    }
    if (p.kind == PLAN_MOE_BATCHED_MFMA4) {
        W4A16_MOE_BATCHED_MFMA4_CONFIGS(W4A16_MOE_BATCHED_MFMA4_CASE)
        return hipErrorInvalidConfiguration;
    }
    if (p.kind == PLAN_VALU) {
        W4A16_VALU_CONFIGS(W4A16_VALU_CASE)
        W4A16_TAIL_CONFIGS(W4A16_TAIL_CASE)
    } else if (p.kind == PLAN_SPLITK) {
        W4A16_SPLITK_CONFIGS(W4A16_SPLITK_CASE)
        W4A16_GATHER_CONFIGS(W4A16_GATHER_CASE)
    } else if (p.kind == PLAN_MFMA) {
        W4A16_MFMA_CONFIGS(W4A16_MFMA_CASE)
    } else if (p.kind == PLAN_MFMA4) {
        W4A16_MFMA4_CONFIGS(W4A16_MFMA4_CASE)
    }
    return hipErrorInvalidConfiguration;
}

hipError_t launch_unpack(const uint32_t *qw, int8_t *out, int64_t words, int cus,
                         hipStream_t stream)
{
    int64_t blocks = (words + 255) / 256;
    const int64_t cap = (int64_t)cus * 16;
    if (blocks > cap)
        blocks = cap;
    if (blocks < 1)
        blocks = 1;
    void *args[] = {(void *)&qw, (void *)&out, (void *)&words};
    return hipLaunchKernel(reinterpret_cast<const void *>(unpack_kernel), dim3((unsigned)blocks),
                           dim3(256), args, 0, stream);
}

}  // namespace w4a16
