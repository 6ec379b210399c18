// Measurement support: a plain streaming read of a device buffer, the empirical bandwidth
// ceiling that the GEMV kernels are compared against. Each lane issues UNR 16-byte
// non-temporal loads per step (the same load form the GEMV kernels use for weights), folds
// them with XOR so the loads cannot be removed, and each wave writes one word.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

template <int UNR>
__global__ void __launch_bounds__(256)
stream_read_kernel(const probe_u32x4 *__restrict__ p, int64_t n16, uint32_t *__restrict__ out)
{
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    probe_u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t i = tid;
    // Every index below is < n16: the loop condition covers the last of the UNR loads.
    for (; i + (UNR - 1) * stride < n16; i += UNR * stride) {
        probe_u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            acc ^= v[u];
    }
    for (; i < n16; i += stride)
        acc ^= __builtin_nontemporal_load(p + i);
    uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    // XOR across the wave so the single store depends on every lane's loads.
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        r ^= (uint32_t)__shfl_xor((int)r, o, 64);
    if ((threadIdx.x & 63) == 0)
        out[tid >> 6] = r;
}

hipError_t launch_stream_read(const void *buf, int64_t n16, uint32_t *out, int blocks,
                              int unroll, hipStream_t stream)
{
    const probe_u32x4 *p = static_cast<const probe_u32x4 *>(buf);
    void *args[] = {(void *)&p, (void *)&n16, (void *)&out};
    const void *k = nullptr;
    switch (unroll) {
    case 1: k = reinterpret_cast<const void *>(stream_read_kernel<1>); break;
    case 2: k = reinterpret_cast<const void *>(stream_read_kernel<2>); break;
    case 4: k = reinterpret_cast<const void *>(stream_read_kernel<4>); break;
    case 8: k = reinterpret_cast<const void *>(stream_read_kernel<8>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

}  // namespace w4a16
