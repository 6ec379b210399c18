// bf16 -> packed INT4 quantisation for gfx950: the step that produces the GEMV's operands from
// a bf16 weight matrix. The local-kimi README (technical-detail section) builds its INT4 artifact
// from the bf16 checkpoint without stating the method; this is the plainest symmetric
// round-to-nearest scheme for the format:
//   per row and 128-wide group: s = fp16(amax / 7) (float32 division, nearest-even, saturating
//   at 65504), q = clamp(rint(w / s), -8, 7) (float32 division, ties to even), q = 0 when s = 0.
// The divisions are IEEE float32 divisions (this library is built with correctly rounded
// float32 division), so every code and scale is a deterministic function of the input bits.
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
    for (int64_t g0 = wave * 4; g0 < groups; g0 += waves * 4) {
        const int64_t g = g0 + gl;
        const bool ok = g < groups;
        const int64_t gc = ok ? g : groups - 1;   // lanes past the end re-read the last group
        const int64_t n = gc / gpr;
        const int64_t j = gc - n * gpr;
        const uint4 v = reinterpret_cast<const uint4 *>(W + n * ldw + j * 128)[pl];
        float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(f[i]));
        amax = row16_max(amax);
        const float s32 = amax / 7.0f;
        uint16_t sb = __builtin_bit_cast(uint16_t, (_Float16)s32);   // nearest even
        if ((sb & 0x7FFFu) >= 0x7C00u && s32 == s32)                  // overflow: saturate
            sb = (uint16_t)((sb & 0x8000u) | 0x7BFFu);
        const float s = (float)__builtin_bit_cast(_Float16, sb);
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int q = 0;
            if (s != 0.0f) {
                const float r = rintf(f[i] / s);
                q = r < -8.0f ? -8 : (r > 7.0f ? 7 : (int)r);
            }
            word |= ((uint32_t)q & 0xFu) << (4 * i);
        }
        if (ok) {
            qw[n * (K >> 3) + j * 16 + pl] = word;
            if (pl == 0)
                sc[n * gpr + j] = sb;
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
