// bf16 -> packed INT4 quantisation for gfx950: the step that produces the GEMV's operands from
// a bf16 weight matrix. The local-kimi README (technical-detail section) builds its INT4 artifact
// from the bf16 checkpoint without stating the method; this is the plainest symmetric
// round-to-nearest scheme for the format:
//   per row and 128-wide group: s = fp16(amax / 7) (float32 division, nearest-even, saturating
//   at 65504), q = clamp(rint(w / s), -8, 7) (float32 division, ties to even), q = 0 when s = 0.
// The divisions are IEEE float32 divisions (this library is built with correctly rounded
// float32 division), so every code and scale is a deterministic function of the input bits.
// Only the scale takes a division per group; a code is first estimated as w * fl(1/s), which is
// within 7 * 1.5 * 2^-23 < 1.3e-6 of the quotient fl(w / s) (|w / s| <= 7.004), so rounding the
// estimate gives rint(fl(w / s)) unless it lies within 4e-6 of a half-integer; only those
// values (about one in 10^5) take the exact division.
//
// Layout: a wave quantises 4 groups at a time, 16 lanes per group; lane p of a group loads the
// 8 bf16 values 8p..8p+7 (16 bytes), so a wave reads 4 x 256 contiguous bytes and writes the 16
// words of each group as one 64-byte run. The group maximum is reduced with DPP inside the
// 16-lane row. Memory-bound: 2 bytes read and 0.5 + 2/128 bytes written per weight.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

__device__ __forceinline__ float row16_max(float v)
{
    // Butterfly maximum over the 16 lanes of a DPP row (quad permutes, half-row and row mirror).
    int x = __builtin_bit_cast(int, v);
    x = __builtin_bit_cast(int, fmaxf(v, __builtin_bit_cast(float,
            __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true))));
    v = __builtin_bit_cast(float, x);
    x = __builtin_bit_cast(int, fmaxf(v, __builtin_bit_cast(float,
            __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true))));
    v = __builtin_bit_cast(float, x);
    x = __builtin_bit_cast(int, fmaxf(v, __builtin_bit_cast(float,
            __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true))));
    v = __builtin_bit_cast(float, x);
    x = __builtin_bit_cast(int, fmaxf(v, __builtin_bit_cast(float,
            __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, true))));
    return __builtin_bit_cast(float, x);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w)
{
    return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// One group's codes and scale from the 8 values of lane p (the group's other 120 values sit in
// the 15 other lanes of the same DPP row).
__device__ __forceinline__ void quantize_slice(uint4 v, uint32_t &word, uint16_t &sb)
{
    float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        amax = fmaxf(amax, fabsf(f[i]));
    amax = row16_max(amax);
    const float s32 = amax / 7.0f;
    sb = __builtin_bit_cast(uint16_t, (_Float16)s32);   // nearest even
    if ((sb & 0x7FFFu) >= 0x7C00u && s32 == s32)        // overflow: saturate
        sb = (uint16_t)((sb & 0x8000u) | 0x7BFFu);
    const float s = (float)__builtin_bit_cast(_Float16, sb);
    // rcp = 0 for a zero scale makes every estimate 0, so every code 0, as defined.
    const float rcp = s != 0.0f ? 1.0f / s : 0.0f;
    word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float t = f[i] * rcp;
        float r = rintf(t);
        if (fabsf(t - r) > 0.5f - 4e-6f)            // near a rounding boundary: divide
            r = rintf(f[i] / s);
        const int q = (int)__builtin_amdgcn_fmed3f(r, -8.0f, 7.0f);
        word |= ((uint32_t)q & 0xFu) << (4 * i);
    }
}

// A wave takes QU steps of 4 groups per pass: all QU loads are issued before the first group is
// quantised, so each lane keeps QU x 16 bytes in flight.
constexpr int QU = 4;

__global__ void __launch_bounds__(256)
quantize_pack_kernel(const uint16_t *__restrict__ W, int64_t ldw, uint32_t *__restrict__ qw,
                     uint16_t *__restrict__ sc, int64_t N, int32_t K)
{
    const int lane = threadIdx.x & 63;
    const int gl = lane >> 4;     // group of the wave's four
    const int pl = lane & 15;     // 16-byte slice of the group
    const int64_t gpr = K >> 7;
    const int64_t groups = N * gpr;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t g0 = wave * 4; g0 < groups; g0 += waves * 4 * QU) {
        uint4 v[QU];
        int64_t n[QU], j[QU];
        bool ok[QU];
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int64_t g = g0 + (int64_t)u * waves * 4 + gl;
            ok[u] = g < groups;
            // past the end: re-read the last group. Group indices fit in 32 bits (checked by
            // the host), so the row is a 32-bit division.
            const uint32_t gc = (uint32_t)(ok[u] ? g : groups - 1);
            const uint32_t nn = gc / (uint32_t)gpr;
            n[u] = nn;
            j[u] = gc - nn * (uint32_t)gpr;
            v[u] = reinterpret_cast<const uint4 *>(W + n[u] * ldw + j[u] * 128)[pl];
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            uint32_t word;
            uint16_t sb;
            quantize_slice(v[u], word, sb);
            if (ok[u]) {
                qw[n[u] * (K >> 3) + j[u] * 16 + pl] = word;
                if (pl == 0)
                    sc[n[u] * gpr + j[u]] = sb;
            }
        }
    }
}

hipError_t launch_quantize(const uint16_t *W, int64_t ldw, uint32_t *qw, uint16_t *sc, int64_t N,
                           int32_t K, int cus, hipStream_t stream)
{
    const int64_t groups = N * (K / 128);
    int64_t blocks = (groups + 15) / 16;           // 4 waves x 4 groups per work-group
    const int64_t cap = (int64_t)cus * 8;
    if (blocks > cap)
        blocks = cap;
    if (blocks < 1)
        blocks = 1;
    void *args[] = {(void *)&W, (void *)&ldw, (void *)&qw, (void *)&sc, (void *)&N, (void *)&K};
    return hipLaunchKernel(reinterpret_cast<const void *>(quantize_pack_kernel),
                           dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

}  // namespace w4a16
