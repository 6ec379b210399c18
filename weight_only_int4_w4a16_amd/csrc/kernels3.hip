// Grouped-expert GEMV over three-bit expert weights for gfx950 (CDNA4, wave64).
//
// The local-kimi README's hardware section says that fitting a 24 GB card needs the expert
// weights near three bits; the pages define no format. The format read here keeps everything of
// the INT4 format but the code width: a code is a 3-bit two's-complement integer q in [-4, 3]
// with the same fp16 scale per 128-wide K group, and a row of K values is K/32 blocks of three
// uint32 words (12 bytes, 32 codes). In block b, code c (value k = 32 b + c) sits
//     c = 10 t + j      (t < 3, j < 5):  bits [3j, 3j+2]        of word t,
//     c = 10 t + 5 + j  (t < 3, j < 5):  bits [16+3j, 16+3j+2]  of word t,
//     c = 30 / c = 31:                   bit i in bit 15 / bit 31 of word i.
// Each word thus holds five code pairs (10t+j, 10t+5+j) at the same position of its two 16-bit
// halves, which is what one v_bitop3 and one v_pk_add_f16 turn into an fp16 pair of exact codes:
//   fields at bits 0-2 / 16-18:  (w & 0x00070007) ^ 0x64046404  -> 1028 + q, minus 1028
//   fields at bits 3-5 / 19-21:  (w & 0x00380038) ^ 0x58205820  ->  132 + q, minus 132
//   fields at bits 6-8 / 22-24:  (w & 0x01C001C0) ^ 0x4D004D00  ->   20 + q, minus 20
// (the XOR sets an fp16 exponent at which the field's lowest bit is worth 1.0 and flips the
// field's top bit, mapping the two's-complement code to q + 4); fields 3 and 4 of each half take
// the first two forms on w >> 9, and the spare bits of the three words gather into the pair
// (30, 31) at bits 0-2 / 16-18. 0.390625 bytes per weight at 128-wide groups, against 0.515625
// for INT4.
//
// Activations are staged once per work-group exactly as in the INT4 kernels (each 128-value
// group scaled by a power of two into fp16), but paired to match the pairs above: chunk c's 32
// values become the 16 fp16 pairs (10t+j, 10t+5+j) for t < 3, j < 5, in that order, then
// (30, 31), held as four 16-byte slots.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace w4a16 {

namespace {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                  false);
}

template <uint32_t MASK, uint32_t MAGIC, uint32_t NEG>
__device__ __forceinline__ uint32_t decode3(uint32_t bits)
{
    const f16x2_t v = __builtin_bit_cast(f16x2_t, (bits & MASK) ^ MAGIC);
    return __builtin_bit_cast(uint32_t, v + __builtin_bit_cast(f16x2_t, NEG));
}

// Sum over one 32-code block of q * x' with the block's activations staged as 16 fp16 pairs.
__device__ __forceinline__ float block_dot3(uint32_t w0, uint32_t w1, uint32_t w2,
                                            const uint4 (&xp)[4])
{
    const uint32_t xw[16] = {xp[0].x, xp[0].y, xp[0].z, xp[0].w, xp[1].x, xp[1].y,
                             xp[1].z, xp[1].w, xp[2].x, xp[2].y, xp[2].z, xp[2].w,
                             xp[3].x, xp[3].y, xp[3].z, xp[3].w};
    const uint32_t w[3] = {w0, w1, w2};
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const uint32_t v = w[t], v9 = w[t] >> 9;
        acc = dot2h(decode3<0x00070007u, 0x64046404u, 0xE404E404u>(v), xw[5 * t + 0], acc);
        acc = dot2h(decode3<0x00380038u, 0x58205820u, 0xD820D820u>(v), xw[5 * t + 1], acc);
        acc = dot2h(decode3<0x01C001C0u, 0x4D004D00u, 0xCD00CD00u>(v), xw[5 * t + 2], acc);
        acc = dot2h(decode3<0x00070007u, 0x64046404u, 0xE404E404u>(v9), xw[5 * t + 3], acc);
        acc = dot2h(decode3<0x00380038u, 0x58205820u, 0xD820D820u>(v9), xw[5 * t + 4], acc);
    }
    const uint32_t spare = ((w0 >> 15) & 0x00010001u) | ((w1 >> 14) & 0x00020002u) |
                           ((w2 >> 13) & 0x00040004u);
    return dot2h(decode3<0x00070007u, 0x64046404u, 0xE404E404u>(spare), xw[15], acc);
}

// ---- activation staging (the same group scaling as the INT4 kernels)
__device__ __forceinline__ uint32_t absmax2(uint32_t d, uint32_t m)
{
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, d & 0x7FFF7FFFu),
                                                        __builtin_bit_cast(u16x2_t, m)));
}

__device__ __forceinline__ uint32_t pack_scaled3(float a, float b, float p)
{
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "=v"(r) : "v"(a), "v"(p));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,0,0]" : "+v"(r) : "v"(b), "v"(p));
    return r;
}

// Value i (0..31) of a chunk held as 16 bf16 pairs, as fp32.
__device__ __forceinline__ float chunk_value(const uint32_t (&d)[16], int i)
{
    return __builtin_bit_cast(float, (i & 1) ? (d[i >> 1] & 0xFFFF0000u) : (d[i >> 1] << 16));
}

// Stage chunk c of one token: the 32 bf16 values of d, scaled by p = 2^e, as the 16 fp16 pairs
// in block order.
__device__ __forceinline__ void stage_chunk3(const uint32_t (&d)[16], float p, uint32_t (&o)[16])
{
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int j = 0; j < 5; ++j)
            o[5 * t + j] =
                pack_scaled3(chunk_value(d, 10 * t + j), chunk_value(d, 10 * t + 5 + j), p);
    o[15] = pack_scaled3(chunk_value(d, 30), chunk_value(d, 31), p);
}

__device__ __forceinline__ uint32_t quadmax(uint32_t m)
{
    int x = (int)m;
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    x = (int)max((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    return (uint32_t)x;
}

// Sum of a per-lane value over groups of L lanes (L a power of two, 4..64): DPP within a row of
// 16 lanes, then cross-row lane exchanges (ds_bpermute) for 32 and 64.
template <int L>
__device__ __forceinline__ float sum_lanes(float v)
{
    static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "lanes per row: a power of two");
    int x;
    if (L > 1) {
        x = __builtin_bit_cast(int, v);
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    }
    if (L > 2) {
        x = __builtin_bit_cast(int, v);
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    }
    if (L > 4) {
        x = __builtin_bit_cast(int, v);
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));
    }
    if (L > 8) {
        x = __builtin_bit_cast(int, v);
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));
    }
    if (L > 16)
        v += __shfl_xor(v, 16, 64);
    if (L > 32)
        v += __shfl_xor(v, 32, 64);
    return v;
}

template <int V>
struct Buf3 {
    uint32_t w[V][3];
    uint16_t s[V];
    int32_t out;   // flat output index of the lane's row, -1 when the row is past the end
    bool ok;       // the row's expert id is in [0, E)
};

}  // namespace

// ------------------------------------------------------------------------------------------
// Grouped-expert three-bit GEMV, one token: y[t][n] = sum_k q3_e[n,k] s_e[n,k/128] x[k] with
// e = ids[t]; rows of slots whose id is outside [0, E) are written as +0.0. The activations and
// the expert ids are staged once per work-group in LDS; waves then stream (row step, batch)
// items with one item of prefetch: a row step is R = 64/L rows of the flat (slot, row) index,
// lane p of a row owns blocks p, p+L, p+2L, ... of it (L*12 contiguous bytes per load
// instruction), and a batch is V of those blocks (L * V divides the K/32 blocks of a row).
// Every load is unconditional: an invalid id reads expert 0's rows (valid memory) and its
// outputs are written as zero.
// ------------------------------------------------------------------------------------------
template <int L, int V>
__global__ void __launch_bounds__(256)
gemv_moe3_kernel(const uint32_t *__restrict__ qw, const uint16_t *__restrict__ sc,
                 const uint16_t *__restrict__ x, float *__restrict__ y,
                 const int32_t *__restrict__ ids, int32_t topk, int32_t E, int64_t N, int32_t K)
{
    constexpr int R = 64 / L;
    extern __shared__ uint4 smem3[];
    const int CPR = K >> 5;         // blocks per row (= 32-value activation chunks)
    const int GPR = K >> 7;         // scale groups per row
    uint4 *xs = smem3;                                              // [4][CPR] fp16 pairs
    float *fs = reinterpret_cast<float *>(smem3 + 4 * CPR);        // [CPR] group factors
    int32_t *ids_s = reinterpret_cast<int32_t *>(fs + CPR);        // [topk]

    const int lane = threadIdx.x & 63;
    const int pr = lane & (L - 1);
    const int rr = lane / L;
    const int wpb = blockDim.x >> 6;
    const int64_t gw = (int64_t)blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t GW = (int64_t)gridDim.x * wpb;
    const int64_t rows_total = (int64_t)topk * N;
    const int64_t n_steps = (rows_total + R - 1) / R;
    const int nb = CPR / (L * V);   // items per row step (the plan makes L * V divide CPR)
    const bool active = gw < n_steps;
    const int64_t gw_c = active ? gw : n_steps - 1;
    const int64_t n_items = ((n_steps - 1 - gw_c) / GW + 1) * nb;

    // The lane's flat (slot, row) index v = step * R + rr advances by GW * R per row step; its
    // slot and row are carried along (one division at the start), and past the last row the
    // lane reads the last row again without storing it.
    const int64_t D = GW * R;
    const int64_t d_slot = D / N;
    const int64_t d_row = D - d_slot * N;
    int64_t cur_v = gw_c * R + rr;
    int64_t cur_slot = cur_v / N;
    int64_t cur_row = cur_v - cur_slot * N;
    const uint32_t *wr = qw;
    const uint16_t *sr = sc;
    int32_t ld_out = -1;
    bool ld_ok = false;
    // Point wr / sr at the current row step's expert row; the first step takes its id from
    // global memory (nothing is in flight yet), later ones from the LDS copy.
    auto seek = [&](bool first) {
        const bool live = cur_v < rows_total;
        const int32_t slot = live ? (int32_t)cur_slot : topk - 1;
        const int64_t row = live ? cur_row : N - 1;
        const int32_t e = first ? ids[slot] : ids_s[slot];
        ld_ok = e >= 0 && e < E;
        ld_out = live ? (int32_t)cur_v : -1;
        const int64_t er = (int64_t)(ld_ok ? e : 0) * N + row;
        wr = qw + er * (3 * CPR);
        sr = sc + er * GPR;
    };
    auto advance = [&]() {
        cur_v += D;
        cur_slot += d_slot;
        cur_row += d_row;
        if (cur_row >= N) {
            cur_row -= N;
            ++cur_slot;
        }
    };
    int ld_b = 0;
    auto load = [&](Buf3<V> &buf, bool first) {
        if (ld_b == 0)
            seek(first);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int b = pr + L * (v + V * ld_b);
#pragma unroll
            for (int q = 0; q < 3; ++q)
                buf.w[v][q] = __builtin_nontemporal_load(wr + 3 * b + q);
            buf.s[v] = sr[b >> 2];
        }
        buf.out = ld_out;
        buf.ok = ld_ok;
        const bool wrap = ld_b + 1 == nb;
        ld_b = wrap ? 0 : ld_b + 1;
        if (wrap)
            advance();
    };

    // Request the activation chunks (one per thread and pass) and the ids, then the first
    // item's weights, so staging waits only for the activations.
    constexpr int PF = 2;
    uint4 xpre[PF][4];
#pragma unroll
    for (int f = 0; f < PF; ++f) {
        int c = threadIdx.x + f * blockDim.x;
        c = c < CPR ? c : CPR - 1;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xpre[f][q] = reinterpret_cast<const uint4 *>(x)[4 * c + q];
    }
    const int32_t id_pre = ids[(int)threadIdx.x < topk ? threadIdx.x : topk - 1];
    __builtin_amdgcn_sched_barrier(0);
    Buf3<V> bufA, bufB;
    load(bufA, true);
    __builtin_amdgcn_sched_barrier(0);

    // One thread per 32-value chunk: the four chunks of a scale group sit in four consecutive
    // lanes (a pass covers a multiple of 4 chunks, and CPR is a multiple of 4), all active or
    // all not.
    auto stage = [&](int c, const uint4 (&v)[4]) {
        const uint32_t d[16] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                                v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            m = absmax2(d[i], m);
        m = (m >> 16) > (m & 0xFFFFu) ? (m >> 16) : (m & 0xFFFFu);
        m = quadmax(m);
        int e = 142 - (int)(m >> 7);
        e = e < 126 ? e : 126;
        uint32_t o[16];
        stage_chunk3(d, __builtin_bit_cast(float, (uint32_t)(e + 127) << 23), o);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xs[q * CPR + c] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        fs[c] = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);
    };
#pragma unroll
    for (int f = 0; f < PF; ++f) {
        const int c = threadIdx.x + f * blockDim.x;
        if (c < CPR)
            stage(c, xpre[f]);
    }
    for (int c = threadIdx.x + PF * blockDim.x; c < CPR; c += blockDim.x) {
        uint4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] = reinterpret_cast<const uint4 *>(x)[4 * c + q];
        stage(c, v);
    }
    if ((int)threadIdx.x < topk)
        ids_s[threadIdx.x] = id_pre;
    for (int i = threadIdx.x + blockDim.x; i < topk; i += blockDim.x)
        ids_s[i] = ids[i];
    __syncthreads();
    if (!active)
        return;

    float acc = 0.0f;
    int cp_b = 0;
    auto compute = [&](const Buf3<V> &buf) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int b = pr + L * (v + V * cp_b);
            uint4 xp[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xp[q] = xs[q * CPR + b];
            const float d = block_dot3(buf.w[v][0], buf.w[v][1], buf.w[v][2], xp);
            acc = fmaf((float)__builtin_bit_cast(_Float16, buf.s[v]), d * fs[b], acc);
        }
        if (cp_b == nb - 1) {
            const float tot = sum_lanes<L>(acc);
            if (pr == 0 && buf.out >= 0)
                y[buf.out] = buf.ok ? tot : 0.0f;
            acc = 0.0f;
        }
        cp_b = cp_b + 1 == nb ? 0 : cp_b + 1;
    };

    int64_t i = 0;
    for (; i + 2 < n_items; i += 2) {
        load(bufB, false);
        compute(bufA);
        load(bufA, false);
        compute(bufB);
    }
    if (i + 1 < n_items) {
        load(bufB, false);
        compute(bufA);
        compute(bufB);
    } else {
        compute(bufA);
    }
}

template <int L, int V>
static hipError_t launch_moe3_t(const Moe3Args &a, const Plan &p, hipStream_t stream)
{
    auto kern = gemv_moe3_kernel<L, V>;
    void *args[] = {(void *)&a.qweight, (void *)&a.scales, (void *)&a.x, (void *)&a.y,
                    (void *)&a.ids,     (void *)&a.topk,   (void *)&a.E, (void *)&a.N,
                    (void *)&a.K};
    return hipLaunchKernel(reinterpret_cast<const void *>(kern), dim3(p.blocks), dim3(p.threads),
                           args, (size_t)p.lds_bytes, stream);
}

#define W4A16_MOE3_CASE(L_, V_)                                                              \
    if (p.L == L_ && p.V == V_)                                                              \
        return launch_moe3_t<L_, V_>(a, p, stream);

hipError_t launch_moe3(const Moe3Args &a, const Plan &p, hipStream_t stream)
{
    if (p.kind == PLAN_MOE3) {
        W4A16_MOE3_CONFIGS(W4A16_MOE3_CASE)
    }
    return hipErrorInvalidConfiguration;
}

}  // namespace w4a16

namespace w4a16 {

// Test support: the signed value of every three-bit code, decoded with the GEMV's decode forms
// (exact fp16 codes converted to int8).
__global__ void __launch_bounds__(256)
unpack3_kernel(const uint32_t *__restrict__ qw, int8_t *__restrict__ out, int64_t blocks)
{
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < blocks;
         b += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t w[3] = {qw[3 * b], qw[3 * b + 1], qw[3 * b + 2]};
        uint32_t p[16];
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const uint32_t v9 = w[t] >> 9;
            p[5 * t + 0] = decode3<0x00070007u, 0x64046404u, 0xE404E404u>(w[t]);
            p[5 * t + 1] = decode3<0x00380038u, 0x58205820u, 0xD820D820u>(w[t]);
            p[5 * t + 2] = decode3<0x01C001C0u, 0x4D004D00u, 0xCD00CD00u>(w[t]);
            p[5 * t + 3] = decode3<0x00070007u, 0x64046404u, 0xE404E404u>(v9);
            p[5 * t + 4] = decode3<0x00380038u, 0x58205820u, 0xD820D820u>(v9);
        }
        p[15] = decode3<0x00070007u, 0x64046404u, 0xE404E404u>(
            ((w[0] >> 15) & 0x00010001u) | ((w[1] >> 14) & 0x00020002u) |
            ((w[2] >> 13) & 0x00040004u));
        int8_t q[32];
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int j = 0; j < 5; ++j) {
                const f16x2_t h = __builtin_bit_cast(f16x2_t, p[5 * t + j]);
                q[10 * t + j] = (int8_t)(int)h.x;
                q[10 * t + 5 + j] = (int8_t)(int)h.y;
            }
        const f16x2_t h = __builtin_bit_cast(f16x2_t, p[15]);
        q[30] = (int8_t)(int)h.x;
        q[31] = (int8_t)(int)h.y;
#pragma unroll
        for (int i = 0; i < 32; ++i)
            out[32 * b + i] = q[i];
    }
}

hipError_t launch_unpack3(const uint32_t *qw, int8_t *out, int64_t blocks, int cus,
                          hipStream_t stream)
{
    int64_t grid = (blocks + 255) / 256;
    const int64_t cap = (int64_t)cus * 16;
    grid = grid > cap ? cap : (grid < 1 ? 1 : grid);
    void *args[] = {(void *)&qw, (void *)&out, (void *)&blocks};
    return hipLaunchKernel(reinterpret_cast<const void *>(unpack3_kernel), dim3((unsigned)grid),
                           dim3(256), args, 0, stream);
}

}  // namespace w4a16
