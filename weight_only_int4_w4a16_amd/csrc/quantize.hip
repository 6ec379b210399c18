// bf16 -> packed INT4 quantisation for gfx950: the step that produces the GEMV's operands from
// a bf16 weight matrix. The local-kimi README (technical-detail section) builds its INT4 artifact
// from the bf16 checkpoint without stating the method; this is the plainest symmetric
// round-to-nearest scheme for the format:
//   per row and 128-wide group: s = fp16(amax / 7) (float32 division, nearest-even, saturating
//   at 65504), q = clamp(rint(w / s), -8, 7) (float32 division, ties to even), q = 0 when s = 0.
// The scale division is an IEEE float32 division (this library is built with correctly rounded
// float32 division), so every scale is a deterministic function of the input bits. A code is
// first estimated from r = 1/s taken with v_rcp_f32 (relative error <= 2^-23): the exact product
// w * r is within 7.004 * 2^-23 < 8.4e-7 of w / s, which is within 7.004 * 2^-24 < 4.2e-7 of the
// float32 quotient fl(w / s). One FMA against C = 1.5 * 2^23 rounds w * r to the nearest integer
// (ties to even) and leaves it in the low mantissa bits of C + q, and a second FMA gives the
// residual w * r - q with one rounding (error < 3e-8). Where every residual of a lane is at most
// 1/2 - 4e-6, fl(w / s) lies strictly within 1/2 - 2.7e-6 of q, so q = rint(fl(w / s)); a lane
// with a residual closer to 1/2 (about one value in 10^5) recomputes its codes with the exact
// division. Codes need no clamp except in groups with a subnormal or saturated scale, which take
// the exact path with a clamp to [-8, 7]; the two's complement nibble is the low 4 bits of
// C + q (C is a multiple of 16).
//
// Layout: 8 lanes per group, a wave quantises 8 groups at a time; lane p of a group loads the 16-byte
// slices p and p + 8 (bf16 values 8p..8p+7 and 64+8p..64+8p+7), so each load instruction covers one
// whole 128-byte line of each of the 8 groups, and writes packed words p and p + 8. The group
// maximum is reduced with DPP inside each half of a 16-lane row. Memory-bound: 2 bytes read and
// 0.5 + 2/128 bytes written per weight.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

__device__ __forceinline__ float dpp_max(float v, int ctrl_id)
{
    const int x = __builtin_bit_cast(int, v);
    int y;
    switch (ctrl_id) {
    case 0: y = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true); break;    // quad [1,0,3,2]
    case 1: y = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true); break;    // quad [2,3,0,1]
    default: y = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true); break;  // half-row mirror
    }
    return fmaxf(v, __builtin_bit_cast(float, y));
}

// Maximum over the 8 lanes of each half of a DPP row: the two quad swaps give every lane its
// quad's maximum, and the half-row mirror pairs each lane with one of the other quad.
__device__ __forceinline__ float row8_max(float v)
{
    return dpp_max(dpp_max(dpp_max(v, 0), 1), 2);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w)
{
    return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// Eight codes, each in the low nibble of b[i], packed with value i in bits 4i..4i+3: the low
// bytes of the even values go to one word and those of the odd values to another (v_perm), and
// one bit-field insert keeps the low nibble of each byte of the first and the low nibble of each
// byte of the second shifted up by 4.
__device__ __forceinline__ uint32_t pack_nibbles(const uint32_t *b)
{
    // perm(hi, lo, sel): selector bytes 0-3 take bytes of lo, 4-7 bytes of hi, 0x0C gives zero
    const uint32_t e01 = __builtin_amdgcn_perm(b[2], b[0], 0x0C0C0400u);   // [b0, b2, 0, 0]
    const uint32_t e23 = __builtin_amdgcn_perm(b[6], b[4], 0x04000C0Cu);   // [0, 0, b4, b6]
    const uint32_t o01 = __builtin_amdgcn_perm(b[3], b[1], 0x0C0C0400u);   // [b1, b3, 0, 0]
    const uint32_t o23 = __builtin_amdgcn_perm(b[7], b[5], 0x04000C0Cu);   // [0, 0, b5, b7]
    const uint32_t even = e01 | e23;
    const uint32_t odd = o01 | o23;
    return (even & 0x0F0F0F0Fu) | ((odd << 4) & 0xF0F0F0F0u);
}

// One group's scale and this lane's two packed words from its 16 values (slices a and b); the
// group's other 112 values sit in the 7 other lanes of the same half row.
__device__ __forceinline__ void unpack8(uint4 v, float (&f)[8])
{
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ void quantize_lane(uint4 a, uint4 b, uint32_t &w0, uint32_t &w1,
                                              uint16_t &sb)
{
    float amax = 0.0f;
    {
        float f[8];
        unpack8(a, f);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(f[i]));
        unpack8(b, f);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(f[i]));
    }
    amax = row8_max(amax);
    const float s32 = amax / 7.0f;
    sb = __builtin_bit_cast(uint16_t, (_Float16)s32);   // nearest even
    if ((sb & 0x7FFFu) >= 0x7C00u && s32 == s32)        // overflow: saturate
        sb = (uint16_t)((sb & 0x8000u) | 0x7BFFu);
    const float s = (float)__builtin_bit_cast(_Float16, sb);
    // r = 0 for a zero scale makes every code 0, as defined (and every residual 0).
    const float r = s != 0.0f ? __builtin_amdgcn_rcpf(s) : 0.0f;
    constexpr float C = 12582912.0f;   // 1.5 * 2^23: C + q is exact for |q| < 2^22
    // With a normal, unsaturated fp16 scale, s >= (amax / 7)(1 - 2^-11), so |w / s| < 7.004 and
    // every estimate rounds into [-7, 7]: no clamp is needed. A subnormal scale (relative
    // rounding error up to 1/2) or a saturated one can give codes outside [-8, 7]; such groups,
    // and lanes with a residual near 1/2, take the exact division with the clamp.
    const uint32_t smag = sb & 0x7FFFu;
    const bool special = smag - 1u < 0x3FFu || smag == 0x7BFFu;
    // The two 8-value slices one after the other, so only one slice's values are live.
    auto slice = [&](uint4 v) -> uint32_t {
        float f[8], y[8];
        unpack8(v, f);
        float emax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            y[i] = fmaf(f[i], r, C);
            emax = fmaxf(emax, fabsf(fmaf(f[i], r, C - y[i])));
        }
        if (emax > 0.5f - 4e-6f || special) {
            // the exact quotient decides (s > 0 here: a zero scale has no residual and smag = 0)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                y[i] = C + __builtin_amdgcn_fmed3f(rintf(f[i] / s), -8.0f, 7.0f);
        }
        uint32_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q[i] = __builtin_bit_cast(uint32_t, y[i]);
        return pack_nibbles(q);
    };
    w0 = slice(a);
    w1 = slice(b);
}

// A wave takes QU steps of 8 groups per pass and works on one pass while the loads of the next
// are in flight (two register buffers), so each lane keeps up to 2 x QU x 32 bytes requested.
// Registers decide how well the arithmetic overlaps the memory traffic: one step per pass and
// one 8-value slice at a time keep the kernel at 67 VGPRs, 7 waves per SIMD (28672 x 4096: 60.0
// us, against 69.0 with both slices live at 75 VGPRs and 71.2-72.1 with two steps at 101).
constexpr int QU = 1;
constexpr int kGroupsPerWave = 8;

struct QuantBuf {
    uint4 a[QU], b[QU];
};

__global__ void __launch_bounds__(256)
quantize_pack_kernel(const uint16_t *__restrict__ W, int64_t ldw, uint32_t *__restrict__ qw,
                     uint16_t *__restrict__ sc, int64_t N, int32_t K)
{
    const int lane = threadIdx.x & 63;
    const int gl = lane >> 3;     // group of the wave's eight
    const int pl = lane & 7;      // slices pl and pl + 8 of the group
    const int64_t gpr = K >> 7;
    const int64_t groups = N * gpr;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t stride = waves * kGroupsPerWave;
    const int64_t first = wave * kGroupsPerWave;
    if (first >= groups)
        return;
    // passes of this wave: the first groups of its passes are first + p * stride * QU < groups
    const int64_t n_pass = (groups - 1 - first) / (stride * QU) + 1;
    // Group of step u of pass p for this lane, and whether it exists (past the end a lane
    // re-reads the last group and stores nothing). Group indices fit in 32 bits (checked by the
    // host), so the row is a 32-bit division.
    auto group_of = [&](int64_t p, int u, uint32_t &n, uint32_t &j) -> bool {
        const int64_t g = first + (p * QU + u) * stride + gl;
        const bool ok = g < groups;
        const uint32_t gc = (uint32_t)(ok ? g : groups - 1);
        n = gc / (uint32_t)gpr;
        j = gc - n * (uint32_t)gpr;
        return ok;
    };
    auto load = [&](QuantBuf &buf, int64_t p) {
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            uint32_t n, j;
            group_of(p, u, n, j);
            const uint4 *src = reinterpret_cast<const uint4 *>(W + (int64_t)n * ldw + (int64_t)j * 128);
            buf.a[u] = src[pl];
            buf.b[u] = src[pl + 8];
        }
    };
    auto compute = [&](const QuantBuf &buf, int64_t p) {
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            uint32_t w0, w1;
            uint16_t sb;
            quantize_lane(buf.a[u], buf.b[u], w0, w1, sb);
            uint32_t n, j;
            if (group_of(p, u, n, j)) {
                uint32_t *dst = qw + (int64_t)n * (K >> 3) + (int64_t)j * 16;
                dst[pl] = w0;
                dst[pl + 8] = w1;
                if (pl == 0)
                    sc[(int64_t)n * gpr + j] = sb;
            }
        }
    };
    QuantBuf bufA, bufB;
    load(bufA, 0);
    int64_t p = 0;
    for (; p + 2 < n_pass; p += 2) {
        load(bufB, p + 1);
        compute(bufA, p);
        load(bufA, p + 2);
        compute(bufB, p + 1);
    }
    if (p + 1 < n_pass) {
        load(bufB, p + 1);
        compute(bufA, p);
        compute(bufB, p + 1);
    } else {
        compute(bufA, p);
    }
}

hipError_t launch_quantize(const uint16_t *W, int64_t ldw, uint32_t *qw, uint16_t *sc, int64_t N,
                           int32_t K, int cus, hipStream_t stream)
{
    // Every wave makes the same number of passes of QU steps of 8 groups: the fewest passes
    // that the resident waves (work-groups of 4 waves per CU, as many as the kernel's registers
    // allow) can cover, then as few waves as that allows, so no work-group waits for a slot.
    static const int per_cu = [] {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &n, reinterpret_cast<const void *>(quantize_pack_kernel), 256, 0) != hipSuccess ||
            n < 1)
            n = 1;
        return n;
    }();
    const int64_t groups = N * (K / 128);
    const int64_t steps = (groups + kGroupsPerWave - 1) / kGroupsPerWave;
    const int64_t cap_waves = (int64_t)cus * per_cu * 4;
    const int64_t passes = (steps + QU * cap_waves - 1) / (QU * cap_waves);
    const int64_t waves = (steps + QU * passes - 1) / (QU * passes);
    int64_t blocks = (waves + 3) / 4;
    if (blocks < 1)
        blocks = 1;
    void *args[] = {(void *)&W, (void *)&ldw, (void *)&qw, (void *)&sc, (void *)&N, (void *)&K};
    return hipLaunchKernel(reinterpret_cast<const void *>(quantize_pack_kernel),
                           dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

}  // namespace w4a16
