/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 decode GEMV library, libw4a16.so.
 *
 * The operation is the matrix-vector product that the local-kimi README
 * (github.1485827954.workers.dev/RightNow-AI/local-kimi), technical-detail section, puts at the centre of
 * single-stream decode: INT4 weights with 16-bit activations, computed as a true GEMV that
 * walks the contiguous reduction axis K with one accumulator per output row (its GEMV-rewrite
 * paragraph), in a dense form and a grouped-expert form over the experts a router selected.
 * The same section states that the fast path allocates no per-call partial buffers; this
 * library allocates no device or host memory in any call.
 *
 *   y[n] = sum_{k=0}^{K-1} q[n,k] * s[n, k/128] * x[k]
 *
 * Storage (all row-major, little-endian):
 *   qweight  uint32[N][K/8]    value k = 8w + i is bits [4i, 4i+3] of word w of its row, a
 *                              two's-complement integer in [-8, 7] (no zero point)
 *   scales   uint16[N][K/128]  IEEE binary16 bit patterns, one per 128-wide group of a row
 *   x        uint16[K]         bfloat16 bit patterns
 *   y        float[N]          IEEE binary32, fully overwritten (no accumulate-into)
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is a DEVICE pointer on the current HIP device, owned by the caller,
 *     who keeps it alive until the work on `stream` has completed.
 *   - Arguments are validated on the host before anything is enqueued. On any error the
 *     call returns a non-zero status and enqueues nothing.
 *   - On W4A16_OK the work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without synchronising. Faults inside a kernel surface at the caller's next
 *     synchronisation, as for any HIP launch.
 *   - Precision. Every weight enters the arithmetic as the exact integer q. The activations of
 *     each 128-value group of a token are multiplied by a power of two 2^e (e chosen from the
 *     group's largest finite-or-not magnitude so that it lands in [2^15, 2^16)) and rounded to
 *     binary16: this is exact for every activation of magnitude at least 2^-32 times the
 *     largest of its group, and a smaller one moves by at most 2^-40 times that largest value.
 *     Products q * x' are exact in fp32 and are summed in fp32 in a fixed order, then scaled by
 *     2^-e (exact) and by the group's scale, so per output
 *         |y - y_exact| <= (K/32 + 64) * 2^-24 * sum_k |q s x|
 *                          + 2^-40 * sum_{k: |x_k| < 2^-32 max_g} |q_k s_k| * max_{g(k)}
 *     (max_g: the largest |x| of k's group), and repeated calls give identical bits. Infinite
 *     and NaN activations propagate as in the plain definition: every output that reads one
 *     is +-inf or NaN exactly where the exact sum is (0 * inf is NaN).
 *   - Calls are thread-safe. The library keeps one cached record of device properties per
 *     device and no other global state.
 *   - No C++ exception crosses this boundary and nothing is printed.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same definition as hip_runtime_api.h, so this header stands alone. */
typedef struct ihipStream_t *hipStream_t;

#define W4A16_ABI_VERSION 1
#define W4A16_GROUP_SIZE 128
#define W4A16_MAX_BATCH 16

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_NULL_POINTER = 1,       /* a required pointer is NULL                          */
    W4A16_ERR_BAD_SHAPE = 2,          /* N, K, M, topk, E, ldx or ldy out of range (below)    */
    W4A16_ERR_BAD_GROUP = 3,          /* group_size != 128                                    */
    W4A16_ERR_MISALIGNED = 4,         /* qweight/x/X not 16-byte aligned, ldx % 8 != 0,
                                         scales not 2-byte aligned, y/Y not 4-byte aligned    */
    W4A16_ERR_UNSUPPORTED_DEVICE = 5, /* no current HIP device, or it is not gfx950           */
    W4A16_ERR_LAUNCH = 6              /* the HIP runtime refused the kernel launch            */
} w4a16_status_t;

/*
 * Dense single-token GEMV: y = W x. This is the dense W4A16 kernel of the local-kimi README
 * (technical-detail section: the kernel-registry paragraph names a dense and a grouped W4A16
 * operation), in the form its GEMV-rewrite paragraph gives both of them: the reduction axis K
 * contiguous in memory and one accumulator per output row instead of a 16-row tile.
 *   qweight uint32[N][K/8], scales fp16 bits [N][K/128], x bf16 bits [K], y float[N].
 *   1 <= N <= 2^31 - 1;  128 <= K <= 65536, K % 128 == 0;  group_size == 128.
 */
w4a16_status_t w4a16_gemv(const uint32_t *qweight, const uint16_t *scales, const uint16_t *x,
                          float *y, int64_t N, int64_t K, int32_t group_size,
                          hipStream_t stream);

/*
 * Small-batch GEMV for decode of M tokens at once: Y = X W^T. The pages measure single-stream
 * decode only and describe no batched kernel; this form (1..16 tokens over one weight
 * matrix) is this library's addition, with the same storage and precision as w4a16_gemv.
 *   X bf16 bits, M rows with row stride ldx elements (ldx >= K, ldx % 8 == 0);
 *   Y float, M rows with row stride ldy elements (ldy >= N).
 *   1 <= M <= 16; N and K as for w4a16_gemv (K up to 2^20 when M >= 2).
 *   Row m of Y equals w4a16_gemv of row m of X to within the fp32 summation order.
 */
w4a16_status_t w4a16_gemv_batched(const uint32_t *qweight, const uint16_t *scales,
                                  const uint16_t *X, int64_t ldx, float *Y, int64_t ldy,
                                  int32_t M, int64_t N, int64_t K, int32_t group_size,
                                  hipStream_t stream);

/*
 * Grouped-expert GEMV for one token: y[t] = W_{expert_ids[t]} x for t < topk. This is the
 * grouped W4A16 kernel of the local-kimi README's technical-detail section (the one its
 * GEMV-rewrite paragraph measures before and after the rewrite), over the experts the router
 * selected.
 *   qweight uint32[E][N][K/8], scales fp16 bits [E][N][K/128] (experts contiguous);
 *   expert_ids int32[topk] in DEVICE memory (read by the kernel, no host synchronisation);
 *   x bf16 bits [K]; y float[topk][N].
 *   Only the weights and scales of the listed experts are read. An id outside [0, E) names
 *   no expert and its output row is written as +0.0f. Repeated ids are computed independently.
 *   1 <= topk <= 1024; 1 <= E; N, K as for w4a16_gemv.
 */
w4a16_status_t w4a16_moe_gemv(const uint32_t *qweight, const uint16_t *scales,
                              const int32_t *expert_ids, int32_t topk, int32_t num_experts,
                              const uint16_t *x, float *y, int64_t N, int64_t K,
                              int32_t group_size, hipStream_t stream);

/*
 * Grouped-expert GEMV for M tokens decoded together, each with its own topk experts:
 *   Y[m][t] = W_e X[m],  e = expert_ids[m * topk + t]
 *   qweight uint32[E][N][K/8], scales fp16 bits [E][N][K/128]; expert_ids int32[M][topk] in
 *   DEVICE memory; X bf16 bits, M rows of stride ldx (ldx >= K, ldx % 8 == 0); Y float
 *   [M][topk][N], fully overwritten. Every expert that any token selected is read once per call
 *   and applied to all the tokens that chose it (the grouped-expert form of the local-kimi
 *   README, technical-detail section, extended to a batch). An id outside [0, E) gives a row of
 *   +0.0; repeated ids are allowed.
 *   1 <= M <= 16; 1 <= topk, M * topk <= 256; N, K as for w4a16_gemv, and the M activation rows
 *   must fit in LDS (about M * K * 2.1 bytes <= 150 KiB), else W4A16_ERR_BAD_SHAPE.
 */
w4a16_status_t w4a16_moe_gemv_batched(const uint32_t *qweight, const uint16_t *scales,
                                      const int32_t *expert_ids, int32_t M, int32_t topk,
                                      int32_t num_experts, const uint16_t *X, int64_t ldx,
                                      float *Y, int64_t N, int64_t K, int32_t group_size,
                                      hipStream_t stream);

/*
 * Expert tail, step 1: the grouped gate+up product of one token with the SwiGLU epilogue. The
 * local-kimi README, technical-detail section, lists a SwiGLU variant of the grouped W4A16 kernel
 * beside the plain one; the split of an expert's rows and the rounding of h are this library's
 * reading (the pages give neither):
 *   qweight uint32[E][2I][K/8], scales fp16 bits [E][2I][K/128]: rows [0, I) of an expert are
 *     the gate projection, rows [I, 2I) the up projection;
 *   expert_ids int32[topk] in DEVICE memory; x bf16 bits [K];
 *   h bf16 bits [topk][I] (output): h[t][n] = bf16(silu(g) * u) with g = W_e[n] x,
 *     u = W_e[I + n] x, e = expert_ids[t], silu(g) = g / (1 + e^-g), evaluated in fp32 and
 *     rounded to nearest-even bfloat16. An id outside [0, E) gives a row of +0.0.
 *   1 <= I, 2I <= 2^31 - 1; K as for w4a16_gemv; 1 <= topk <= 1024; h 2-byte aligned.
 */
w4a16_status_t w4a16_moe_gemv_swiglu(const uint32_t *qweight, const uint16_t *scales,
                                     const int32_t *expert_ids, int32_t topk, int32_t num_experts,
                                     const uint16_t *x, uint16_t *h, int64_t I, int64_t K,
                                     int32_t group_size, hipStream_t stream);

/*
 * Expert tail, step 2: the grouped down projection of every slot's own activation row, summed
 * with the router's weights (the combine that follows the grouped expert kernels in an MoE
 * decode step):
 *   out[n] = sum_t route_weights[t] * sum_k q_e[n,k] * s_e[n, k/128] * h[t][k],  e = expert_ids[t]
 *   qweight uint32[E][H][I/8], scales fp16 bits [E][H][I/128]; expert_ids int32[topk] and
 *   route_weights float[topk] in DEVICE memory; h bf16 bits [topk][I], contiguous, 16-byte
 *   aligned (the output of w4a16_moe_gemv_swiglu); out float[H], fully overwritten.
 *   A slot whose id is outside [0, E) contributes nothing (expert 0's bytes may be read for it).
 *   1 <= H <= 2^31 - 1; 128 <= I, I % 128 == 0; topk * I <= 65536; 1 <= topk <= 1024.
 */
w4a16_status_t w4a16_moe_down_combine(const uint32_t *qweight, const uint16_t *scales,
                                      const int32_t *expert_ids, const float *route_weights,
                                      int32_t topk, int32_t num_experts, const uint16_t *h,
                                      float *out, int64_t H, int64_t I, int32_t group_size,
                                      hipStream_t stream);

/*
 * The step before the path: quantise a bf16 weight matrix into this library's format. The
 * local-kimi README, technical-detail section, builds its INT4 artifact from the bf16 weights
 * without giving the method; this is the plainest symmetric round-to-nearest scheme:
 *   per row n and 128-wide group g: s = fp16(amax / 7), the float32 quotient rounded to the
 *   nearest-even binary16 and saturated at 65504; q = clamp(rint(w / s), -8, 7) with a float32
 *   quotient and ties to even; q = 0 for a group whose s is zero.
 *   w bf16 bits, N rows of stride ldw elements (ldw >= K, ldw % 8 == 0, w 16-byte aligned);
 *   qweight uint32[N][K/8] and scales fp16 bits [N][K/128] (outputs, fully overwritten).
 *   1 <= N <= 2^31 - 1; 128 <= K <= 2^20, K % 128 == 0; N * K / 128 < 2^32. Inputs must be
 *   finite.
 */
w4a16_status_t w4a16_quantize_pack(const uint16_t *w, int64_t ldw, uint32_t *qweight,
                                   uint16_t *scales, int64_t N, int64_t K, int32_t group_size,
                                   hipStream_t stream);

/*
 * Grouped-expert GEMV over THREE-BIT expert weights, one token: y[t] = W3_{expert_ids[t]} x.
 * The local-kimi README, hardware section, says a 24 GB card needs the expert weights near
 * three bits and defines no format; this library reads the format as: a code is a 3-bit
 * two's-complement integer q in [-4, 3] with one fp16 scale per 128-wide K group (as for
 * INT4), and each row of K values is K/32 blocks of three uint32 words holding 32 codes. In
 * block b, code c (k = 32 b + c) sits, for t < 3 and j < 5,
 *     c = 10t + j      in bits [3j, 3j+2] of word t,
 *     c = 10t + 5 + j  in bits [16+3j, 16+3j+2] of word t,
 *     c = 30 / 31      with its bit i in bit 15 / bit 31 of word i (i = 0, 1, 2).
 *   qweight3 uint32[E][N][3K/32] (4-byte aligned), scales fp16 bits [E][N][K/128],
 *   expert_ids int32[topk] in DEVICE memory, x bf16 bits [K] (16-byte aligned),
 *   y float[topk][N]. Only the listed experts are read; an id outside [0, E) gives a row of
 *   +0.0f; 1 <= topk <= 1024, topk * N <= 2^31 - 1; K as for w4a16_gemv. Precision as stated
 *   at the top of this file (codes enter as exact integers).
 */
w4a16_status_t w4a16_moe_gemv3(const uint32_t *qweight3, const uint16_t *scales,
                               const int32_t *expert_ids, int32_t topk, int32_t num_experts,
                               const uint16_t *x, float *y, int64_t N, int64_t K,
                               int32_t group_size, hipStream_t stream);

/*
 * Test support for the three-bit format: q_out int8[N][K] receives every code, decoded with
 * the GEMV's own decode steps. 1 <= N, 32 <= K, K % 32 == 0; qweight3 4-byte aligned.
 */
w4a16_status_t w4a16_unpack3_debug(const uint32_t *qweight3, int8_t *q_out, int64_t N,
                                   int64_t K, hipStream_t stream);

/* Launch plan of w4a16_moe_gemv3 for (N, K, topk) on `cus` compute units (host only). */
w4a16_status_t w4a16_describe_moe3_plan(int64_t N, int64_t K, int32_t topk, int32_t cus,
                                        char *buf, int64_t len);

/*
 * Test support: q_out int8[N][K] receives the signed value of every packed nibble, so the
 * unpacking can be checked bit for bit against the storage format at the top of this file
 * (this library's reading of the packed INT4 weights of the README's GEMV-rewrite paragraph,
 * which fixes only that K is the contiguous axis). 1 <= N, 8 <= K, K % 8 == 0; qweight 4-byte aligned
 * (one word per thread); otherwise W4A16_ERR_MISALIGNED.
 */
w4a16_status_t w4a16_unpack_debug(const uint32_t *qweight, int8_t *q_out, int64_t N, int64_t K,
                                  hipStream_t stream);

/*
 * Measurement support: reads `bytes` bytes of device memory at `buf` once with 16-byte
 * streaming loads (blocks work-groups of 256 lanes, `unroll` loads in flight per lane per step)
 * and writes one XOR digest word per wave to out[0 .. blocks*4 - 1]. It is the plain
 * bandwidth ceiling a GEMV over the same bytes is compared with; it computes nothing of the
 * GEMV. bytes >= 16, bytes % 16 == 0; 1 <= blocks <= 2^20; unroll in {1, 2, 4, 8};
 * buf 16-byte aligned, out 4-byte aligned; the caller owns both.
 */
w4a16_status_t w4a16_stream_read(const void *buf, int64_t bytes, uint32_t *out, int32_t blocks,
                                 int32_t unroll, hipStream_t stream);

/*
 * Host-only introspection: writes into buf (at most len bytes, NUL-terminated) the kernel and
 * launch shape the entry points would choose for (M, N, K, topk) on a device with `cus` compute
 * units; topk = 0 means a dense call. Returns W4A16_OK or W4A16_ERR_BAD_SHAPE. Touches no device.
 */
w4a16_status_t w4a16_describe_plan(int32_t M, int64_t N, int64_t K, int32_t topk, int32_t cus,
                                   char *buf, int64_t len);

/*
 * Host-only introspection of the expert-tail launch: step 0 = w4a16_moe_gemv_swiglu for (I, K,
 * topk), step 1 = w4a16_moe_down_combine for (rows = H, I, topk). Same conventions as
 * w4a16_describe_plan.
 */
w4a16_status_t w4a16_describe_tail_plan(int32_t step, int64_t rows, int64_t K, int64_t I,
                                        int32_t topk, int32_t cus, char *buf, int64_t len);

/* Host-only introspection of w4a16_moe_gemv_batched's launch (same conventions). */
w4a16_status_t w4a16_describe_moe_batched_plan(int32_t M, int64_t N, int64_t K, int32_t topk,
                                               int32_t cus, char *buf, int64_t len);

/* Static, never-NULL description of a status code. */
const char *w4a16_status_string(w4a16_status_t status);

/* W4A16_ABI_VERSION of the loaded library. */
int32_t w4a16_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
