// C ABI of libw4a16.so (declared in include/w4a16.h): host-side validation, device checks and
// kernel dispatch. Nothing here allocates device or host memory.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>
#include <string.h>

#include "plan.h"
#include "w4a16.h"

namespace w4a16 {
hipError_t launch(const GemvArgs &a, const Plan &p, hipStream_t stream);
hipError_t launch_unpack(const uint32_t *qw, int8_t *out, int64_t words, int cus,
                         hipStream_t stream);
hipError_t launch_stream_read(const void *buf, int64_t n16, uint32_t *out, int blocks,
                              int unroll, hipStream_t stream);
hipError_t launch_moe3(const Moe3Args &a, const Plan &p, hipStream_t stream);
hipError_t launch_unpack3(const uint32_t *qw, int8_t *out, int64_t blocks, int cus,
                          hipStream_t stream);
hipError_t launch_quantize(const uint16_t *W, int64_t ldw, uint32_t *qw, uint16_t *sc, int64_t N,
                           int32_t K, int cus, hipStream_t stream);

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxN = (1LL << 31) - 1;
constexpr int64_t kMaxKDense = 65536;
constexpr int64_t kMaxKBatched = 1LL << 20;
constexpr int32_t kMaxTopk = 1024;

struct DeviceInfo {
    bool ok;
    int cus;
    int64_t lds_limit;
};

std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];

void probe_device(int dev)
{
    DeviceInfo info{false, 0, 0};
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
        strncmp(prop.gcnArchName, "gfx950", 6) == 0) {
        info.ok = true;
        info.cus = prop.multiProcessorCount;
        info.lds_limit = (int64_t)prop.sharedMemPerBlock;
    }
    g_info[dev] = info;
}

// Current device's cached properties, or null when it is missing or not gfx950.
const DeviceInfo *current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::call_once(g_once[dev], probe_device, dev);
    return g_info[dev].ok ? &g_info[dev] : nullptr;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

w4a16_status_t check_common(const void *qweight, const void *scales, const void *x,
                            const void *y, int64_t N, int64_t K, int32_t group_size,
                            int64_t max_k)
{
    if (!qweight || !scales || !x || !y)
        return W4A16_ERR_NULL_POINTER;
    if (group_size != W4A16_GROUP_SIZE)
        return W4A16_ERR_BAD_GROUP;
    if (N < 1 || N > kMaxN || K < W4A16_GROUP_SIZE || K % W4A16_GROUP_SIZE != 0 || K > max_k)
        return W4A16_ERR_BAD_SHAPE;
    if (!aligned(qweight, 16) || !aligned(x, 16) || !aligned(scales, 2) || !aligned(y, 4))
        return W4A16_ERR_MISALIGNED;
    return W4A16_OK;
}

w4a16_status_t run(const GemvArgs &a, int M, int topk, hipStream_t stream)
{
    const DeviceInfo *dev = current_device();
    if (!dev)
        return W4A16_ERR_UNSUPPORTED_DEVICE;
    Plan plan;
    if (!make_plan(M, a.N, a.K, topk, dev->cus, dev->lds_limit, &plan))
        return W4A16_ERR_BAD_SHAPE;
    return launch(a, plan, stream) == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

}  // namespace
}  // namespace w4a16

using namespace w4a16;

extern "C" {

w4a16_status_t w4a16_gemv(const uint32_t *qweight, const uint16_t *scales, const uint16_t *x,
                          float *y, int64_t N, int64_t K, int32_t group_size, hipStream_t stream)
{
    const w4a16_status_t st = check_common(qweight, scales, x, y, N, K, group_size, kMaxKDense);
    if (st != W4A16_OK)
        return st;
    GemvArgs a{qweight, scales, x, K, y, N, nullptr, 0, 0, N, (int32_t)K, 1};
    return run(a, 1, 0, stream);
}

w4a16_status_t w4a16_gemv_batched(const uint32_t *qweight, const uint16_t *scales,
                                  const uint16_t *X, int64_t ldx, float *Y, int64_t ldy,
                                  int32_t M, int64_t N, int64_t K, int32_t group_size,
                                  hipStream_t stream)
{
    const int64_t max_k = M == 1 ? kMaxKDense : kMaxKBatched;
    w4a16_status_t st = check_common(qweight, scales, X, Y, N, K, group_size, max_k);
    if (st != W4A16_OK)
        return st;
    if (M < 1 || M > W4A16_MAX_BATCH || ldx < K || ldy < N)
        return W4A16_ERR_BAD_SHAPE;
    if (ldx % 8 != 0)
        return W4A16_ERR_MISALIGNED;
    GemvArgs a{qweight, scales, X, ldx, Y, ldy, nullptr, 0, 0, N, (int32_t)K, M};
    return run(a, M, 0, stream);
}

w4a16_status_t w4a16_moe_gemv(const uint32_t *qweight, const uint16_t *scales,
                              const int32_t *expert_ids, int32_t topk, int32_t num_experts,
                              const uint16_t *x, float *y, int64_t N, int64_t K,
                              int32_t group_size, hipStream_t stream)
{
    w4a16_status_t st = check_common(qweight, scales, x, y, N, K, group_size, kMaxKDense);
    if (st != W4A16_OK)
        return st;
    if (!expert_ids)
        return W4A16_ERR_NULL_POINTER;
    if (topk < 1 || topk > kMaxTopk || num_experts < 1 || (int64_t)topk * N > kMaxN)
        return W4A16_ERR_BAD_SHAPE;
    if (!aligned(expert_ids, 4))
        return W4A16_ERR_MISALIGNED;
    GemvArgs a{qweight, scales, x, K, y, N, expert_ids, topk, num_experts, N, (int32_t)K, 1};
    return run(a, 1, topk, stream);
}

w4a16_status_t w4a16_moe_gemv_batched(const uint32_t *qweight, const uint16_t *scales,
                                      const int32_t *expert_ids, int32_t M, int32_t topk,
                                      int32_t num_experts, const uint16_t *X, int64_t ldx,
                                      float *Y, int64_t N, int64_t K, int32_t group_size,
                                      hipStream_t stream)
{
    w4a16_status_t st = check_common(qweight, scales, X, Y, N, K, group_size, kMaxKDense);
    if (st != W4A16_OK)
        return st;
    if (!expert_ids)
        return W4A16_ERR_NULL_POINTER;
    if (M < 1 || M > W4A16_MAX_BATCH || topk < 1 || M * topk > 256 || num_experts < 1 ||
        ldx < K || (int64_t)M * topk * N > kMaxN)
        return W4A16_ERR_BAD_SHAPE;
    if (ldx % 8 != 0 || !aligned(expert_ids, 4))
        return W4A16_ERR_MISALIGNED;
    const DeviceInfo *dev = current_device();
    if (!dev)
        return W4A16_ERR_UNSUPPORTED_DEVICE;
    Plan plan;
    if (!make_moe_batched_plan(M, N, K, topk, dev->cus, dev->lds_limit, &plan))
        return W4A16_ERR_BAD_SHAPE;
    GemvArgs a{qweight, scales, X, ldx, Y, N, expert_ids, topk, num_experts, N, (int32_t)K, M,
               nullptr, (int32_t)K};
    return launch(a, plan, stream) == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

w4a16_status_t w4a16_moe_gemv_swiglu(const uint32_t *qweight, const uint16_t *scales,
                                     const int32_t *expert_ids, int32_t topk, int32_t num_experts,
                                     const uint16_t *x, uint16_t *h, int64_t I, int64_t K,
                                     int32_t group_size, hipStream_t stream)
{
    if (!qweight || !scales || !expert_ids || !x || !h)
        return W4A16_ERR_NULL_POINTER;
    if (group_size != W4A16_GROUP_SIZE)
        return W4A16_ERR_BAD_GROUP;
    if (I < 1 || 2 * I > kMaxN || K < W4A16_GROUP_SIZE || K % W4A16_GROUP_SIZE != 0 ||
        K > kMaxKDense || topk < 1 || topk > kMaxTopk || num_experts < 1)
        return W4A16_ERR_BAD_SHAPE;
    if (!aligned(qweight, 16) || !aligned(x, 16) || !aligned(scales, 2) || !aligned(h, 2) ||
        !aligned(expert_ids, 4))
        return W4A16_ERR_MISALIGNED;
    const DeviceInfo *dev = current_device();
    if (!dev)
        return W4A16_ERR_UNSUPPORTED_DEVICE;
    Plan plan;
    if (!make_tail_plan(PLAN_MODE_SWIGLU, 2 * I, K, K, topk, dev->cus, dev->lds_limit, &plan))
        return W4A16_ERR_BAD_SHAPE;
    GemvArgs a{qweight, scales, x, K, reinterpret_cast<float *>(h), I, expert_ids, topk,
               num_experts, 2 * I, (int32_t)K, 1, nullptr, (int32_t)K};
    return launch(a, plan, stream) == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

w4a16_status_t w4a16_moe_down_combine(const uint32_t *qweight, const uint16_t *scales,
                                      const int32_t *expert_ids, const float *route_weights,
                                      int32_t topk, int32_t num_experts, const uint16_t *h,
                                      float *out, int64_t H, int64_t I, int32_t group_size,
                                      hipStream_t stream)
{
    if (!qweight || !scales || !expert_ids || !route_weights || !h || !out)
        return W4A16_ERR_NULL_POINTER;
    if (group_size != W4A16_GROUP_SIZE)
        return W4A16_ERR_BAD_GROUP;
    if (H < 1 || H > kMaxN || I < W4A16_GROUP_SIZE || I % W4A16_GROUP_SIZE != 0 ||
        I > kMaxKDense || topk < 1 || topk > kMaxTopk || num_experts < 1 ||
        (int64_t)topk * I > kMaxKDense)
        return W4A16_ERR_BAD_SHAPE;
    if (!aligned(qweight, 16) || !aligned(h, 16) || !aligned(scales, 2) || !aligned(out, 4) ||
        !aligned(expert_ids, 4) || !aligned(route_weights, 4))
        return W4A16_ERR_MISALIGNED;
    const DeviceInfo *dev = current_device();
    if (!dev)
        return W4A16_ERR_UNSUPPORTED_DEVICE;
    Plan plan;
    const int64_t K = (int64_t)topk * I;
    if (!make_tail_plan(PLAN_MODE_COMBINE, H, K, I, topk, dev->cus, dev->lds_limit, &plan))
        return W4A16_ERR_BAD_SHAPE;
    GemvArgs a{qweight, scales, h, K, out, H, expert_ids, topk, num_experts, H, (int32_t)K, 1,
               route_weights, (int32_t)I};
    return launch(a, plan, stream) == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

w4a16_status_t w4a16_quantize_pack(const uint16_t *w, int64_t ldw, uint32_t *qweight,
                                   uint16_t *scales, int64_t N, int64_t K, int32_t group_size,
                                   hipStream_t stream)
{
    if (!w || !qweight || !scales)
        return W4A16_ERR_NULL_POINTER;
    if (group_size != W4A16_GROUP_SIZE)
        return W4A16_ERR_BAD_GROUP;
    if (N < 1 || N > kMaxN || K < W4A16_GROUP_SIZE || K % W4A16_GROUP_SIZE != 0 ||
        K > kMaxKBatched || ldw < K || N * (K / W4A16_GROUP_SIZE) > (int64_t)0xFFFFFFFFLL)
        return W4A16_ERR_BAD_SHAPE;
    if (!aligned(w, 16) || ldw % 8 != 0 || !aligned(qweight, 4) || !aligned(scales, 2))
        return W4A16_ERR_MISALIGNED;
    const DeviceInfo *dev = current_device();
    if (!dev)
        return W4A16_ERR_UNSUPPORTED_DEVICE;
    return launch_quantize(w, ldw, qweight, scales, N, (int32_t)K, dev->cus, stream) == hipSuccess
               ? W4A16_OK
               : W4A16_ERR_LAUNCH;
}

w4a16_status_t w4a16_moe_gemv3(const uint32_t *qweight3, const uint16_t *scales,
                               const int32_t *expert_ids, int32_t topk, int32_t num_experts,
                               const uint16_t *x, float *y, int64_t N, int64_t K,
                               int32_t group_size, hipStream_t stream)
{
    if (!qweight3 || !scales || !expert_ids || !x || !y)
        return W4A16_ERR_NULL_POINTER;
    if (group_size != W4A16_GROUP_SIZE)
        return W4A16_ERR_BAD_GROUP;
    if (N < 1 || N > kMaxN || K < W4A16_GROUP_SIZE || K % W4A16_GROUP_SIZE != 0 ||
        K > kMaxKDense || topk < 1 || topk > kMaxTopk || num_experts < 1 ||
        (int64_t)topk * N > kMaxN)
        return W4A16_ERR_BAD_SHAPE;
    if (!aligned(qweight3, 4) || !aligned(x, 16) || !aligned(scales, 2) || !aligned(y, 4) ||
        !aligned(expert_ids, 4))
        return W4A16_ERR_MISALIGNED;
    const DeviceInfo *dev = current_device();
    if (!dev)
        return W4A16_ERR_UNSUPPORTED_DEVICE;
    Plan plan;
    if (!make_moe3_plan(N, K, topk, dev->cus, dev->lds_limit, &plan))
        return W4A16_ERR_BAD_SHAPE;
    Moe3Args a{qweight3, scales, x, y, expert_ids, topk, num_experts, N, (int32_t)K};
    return launch_moe3(a, plan, stream) == hipSuccess ? W4A16_OK : W4A16_ERR_LAUNCH;
}

w4a16_status_t w4a16_unpack3_debug(const uint32_t *qweight3, int8_t *q_out, int64_t N, int64_t K,
                                   hipStream_t stream)
{
    if (!qweight3 || !q_out)
        return W4A16_ERR_NULL_POINTER;
    if (N < 1 || K < 32 || K % 32 != 0 || N > kMaxN || K > kMaxKBatched)
        return W4A16_ERR_BAD_SHAPE;
    if (!aligned(qweight3, 4))
        return W4A16_ERR_MISALIGNED;
    const DeviceInfo *dev = current_device();
    if (!dev)
        return W4A16_ERR_UNSUPPORTED_DEVICE;
    return launch_unpack3(qweight3, q_out, N * (K / 32), dev->cus, stream) == hipSuccess
               ? W4A16_OK
               : W4A16_ERR_LAUNCH;
}

w4a16_status_t w4a16_describe_moe3_plan(int64_t N, int64_t K, int32_t topk, int32_t cus,
                                        char *buf, int64_t len)
{
    if (!buf || len < 1)
        return W4A16_ERR_NULL_POINTER;
    buf[0] = '\0';
    Plan plan;
    if (cus < 1 || !make_moe3_plan(N, K, topk, cus, 160 * 1024, &plan))
        return W4A16_ERR_BAD_SHAPE;
    describe_plan(plan, buf, (size_t)len);
    return W4A16_OK;
}

w4a16_status_t w4a16_unpack_debug(const uint32_t *qweight, int8_t *q_out, int64_t N, int64_t K,
                                  hipStream_t stream)
{
    if (!qweight || !q_out)
        return W4A16_ERR_NULL_POINTER;
    if (N < 1 || K < 8 || K % 8 != 0 || N > kMaxN || K > kMaxKBatched)
        return W4A16_ERR_BAD_SHAPE;
    if (!aligned(qweight, 4))
        return W4A16_ERR_MISALIGNED;
    const DeviceInfo *dev = current_device();
    if (!dev)
        return W4A16_ERR_UNSUPPORTED_DEVICE;
    return launch_unpack(qweight, q_out, N * (K / 8), dev->cus, stream) == hipSuccess
               ? W4A16_OK
               : W4A16_ERR_LAUNCH;
}

w4a16_status_t w4a16_stream_read(const void *buf, int64_t bytes, uint32_t *out, int32_t blocks,
                                 int32_t unroll, hipStream_t stream)
{
    if (!buf || !out)
        return W4A16_ERR_NULL_POINTER;
    if (bytes < 16 || bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20) ||
        (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8))
        return W4A16_ERR_BAD_SHAPE;
    if (!aligned(buf, 16) || !aligned(out, 4))
        return W4A16_ERR_MISALIGNED;
    if (!current_device())
        return W4A16_ERR_UNSUPPORTED_DEVICE;
    return launch_stream_read(buf, bytes / 16, out, blocks, unroll, stream) == hipSuccess
               ? W4A16_OK
               : W4A16_ERR_LAUNCH;
}

w4a16_status_t w4a16_describe_plan(int32_t M, int64_t N, int64_t K, int32_t topk, int32_t cus,
                                   char *buf, int64_t len)
{
    if (!buf || len < 1)
        return W4A16_ERR_NULL_POINTER;
    buf[0] = '\0';
    Plan plan;
    // 160 KiB of LDS per work-group, as on gfx950.
    if (cus < 1 || !make_plan(M, N, K, topk, cus, 160 * 1024, &plan))
        return W4A16_ERR_BAD_SHAPE;
    describe_plan(plan, buf, (size_t)len);
    return W4A16_OK;
}

w4a16_status_t w4a16_describe_moe_batched_plan(int32_t M, int64_t N, int64_t K, int32_t topk,
                                               int32_t cus, char *buf, int64_t len)
{
    if (!buf || len < 1)
        return W4A16_ERR_NULL_POINTER;
    buf[0] = '\0';
    Plan plan;
    if (cus < 1 || !make_moe_batched_plan(M, N, K, topk, cus, 160 * 1024, &plan))
        return W4A16_ERR_BAD_SHAPE;
    describe_plan(plan, buf, (size_t)len);
    return W4A16_OK;
}

w4a16_status_t w4a16_describe_tail_plan(int32_t step, int64_t rows, int64_t K, int64_t I,
                                        int32_t topk, int32_t cus, char *buf, int64_t len)
{
    if (!buf || len < 1)
        return W4A16_ERR_NULL_POINTER;
    buf[0] = '\0';
    Plan plan;
    const bool ok =
        step == 0   ? make_tail_plan(PLAN_MODE_SWIGLU, 2 * I, K, K, topk, cus, 160 * 1024, &plan)
        : step == 1 ? make_tail_plan(PLAN_MODE_COMBINE, rows, (int64_t)topk * I, I, topk, cus,
                                     160 * 1024, &plan)
                    : false;
    if (cus < 1 || !ok)
        return W4A16_ERR_BAD_SHAPE;
    describe_plan(plan, buf, (size_t)len);
    return W4A16_OK;
}

const char *w4a16_status_string(w4a16_status_t status)
{
    switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_NULL_POINTER: return "null pointer argument";
    case W4A16_ERR_BAD_SHAPE: return "shape out of range";
    case W4A16_ERR_BAD_GROUP: return "group size must be 128";
    case W4A16_ERR_MISALIGNED: return "misaligned pointer or stride";
    case W4A16_ERR_UNSUPPORTED_DEVICE: return "current device is missing or not gfx950";
    case W4A16_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int32_t w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

}  // extern "C"
