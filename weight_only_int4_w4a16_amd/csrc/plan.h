// Host-side launch planning for the W4A16 kernels. Pure C++ (no HIP types) so the choice of
// kernel and launch shape can be inspected without a device.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

enum PlanKind { PLAN_NONE = 0, PLAN_VALU = 1, PLAN_MFMA = 2, PLAN_SPLITK = 3,
                PLAN_MOE_BATCHED = 4, PLAN_MFMA4 = 5, PLAN_MOE_BATCHED_MFMA4 = 6, PLAN_MOE3 = 7 };

// What the rows of a staged VALU launch are: one matrix, expert rows, the gate+up experts with
// the SwiGLU epilogue, or the down experts summed with router weights.
enum PlanMode { PLAN_MODE_DENSE = 0, PLAN_MODE_MOE = 1, PLAN_MODE_SWIGLU = 2,
                PLAN_MODE_COMBINE = 3 };

// Instantiated kernels (the only ones compiled into the library).
//
// Staged-activation VALU kernels: X(tokens, lanes per row, chunks per lane per item, row steps).
// Every (tokens, L, 1, 1) with L in {4..64} is present so that any K that is a multiple of 128
// has a kernel; the others are the shapes the dispatch rules pick.
#define W4A16_VALU_CONFIGS(X)                                                                \
    X(1, 64, 1, 1) X(1, 32, 1, 1) X(1, 16, 1, 1) X(1, 8, 1, 1) X(1, 4, 1, 1)                 \
    X(1, 32, 1, 2) X(1, 32, 2, 1) X(1, 16, 1, 2) X(1, 8, 1, 2) X(1, 8, 3, 1) X(1, 4, 1, 2)   \
    X(2, 64, 1, 1) X(2, 32, 1, 1) X(2, 16, 1, 1) X(2, 8, 1, 1) X(2, 4, 1, 1) X(2, 8, 1, 2)    \
    X(3, 64, 1, 1) X(3, 32, 1, 1) X(3, 16, 1, 1) X(3, 8, 1, 1) X(3, 4, 1, 1)                 \
    X(4, 64, 1, 1) X(4, 32, 1, 1) X(4, 16, 1, 1) X(4, 8, 1, 1) X(4, 4, 1, 1)

// Expert-tail kernels (staged VALU, one token, one row step): X(lanes per row, chunks per item),
// each instantiated for the SwiGLU gate+up form (lanes per row <= 32) and the combine form.
#define W4A16_TAIL_CONFIGS(X) X(8, 3) X(32, 1) X(16, 1) X(8, 1) X(4, 1)

// Grouped-expert GEMV for several tokens on 4x4x4 MFMA: X(blocks per row group, chunks per lane,
// row steps per item).
#define W4A16_MOE_BATCHED_MFMA4_CONFIGS(X) X(8, 3, 1) X(8, 1, 1) X(16, 1, 1) X(16, 2, 1)
// Grouped-expert kernels for M tokens with their own experts: X(lanes per row, chunks per item).
#define W4A16_MOE_BATCHED_CONFIGS(X) X(8, 3) X(64, 1) X(32, 1) X(16, 1) X(8, 1) X(4, 1)

// Split-K kernels in the combine form of the expert tail: X(lanes per row, chunks per lane).
#define W4A16_GATHER_CONFIGS(X) X(32, 1) X(32, 2) X(16, 2) X(16, 4) X(8, 4) X(8, 8) X(4, 8)

// Split-K VALU kernels (dense calls): X(tokens, lanes per row, chunks per lane, row steps).
#define W4A16_SPLITK_CONFIGS(X)                                                              \
    X(1, 64, 1, 4) X(1, 32, 1, 2) X(1, 32, 1, 4) X(1, 64, 2, 4) X(1, 64, 4, 2)               \
    X(2, 64, 1, 4) X(3, 64, 1, 4) X(4, 64, 1, 4)

// MFMA kernels: X(16-row tiles per wave, waves splitting K, activation mode, groups per item,
// waves per work-group). Activation mode: 0 from global memory, 1 staged in LDS, 2 staged with
// whole-line weight loads, 3 from global memory with whole-line weight and activation loads,
// 4 as 2 with 8 token slots staged (M <= 8), 5 from global memory as whole token rows
// exchanged into operand order via LDS, 6 as 5 with 8 token slots (M <= 8).
#define W4A16_MFMA_CONFIGS(X)                                                                \
    X(1, 1, 1, 6, 8) X(1, 1, 1, 4, 8) X(1, 1, 1, 2, 8) X(1, 1, 1, 1, 8)                       \
    X(1, 1, 2, 6, 8) X(1, 1, 2, 4, 8) X(1, 1, 2, 2, 8) X(1, 1, 2, 6, 4) X(1, 1, 2, 4, 4)      \
    X(1, 1, 2, 2, 4) X(1, 8, 5, 2, 8) X(4, 4, 3, 2, 4)                                       \
    X(2, 4, 0, 2, 4) X(2, 2, 0, 2, 4) X(2, 1, 0, 2, 4) X(1, 1, 0, 2, 4) X(1, 1, 0, 1, 4)      \
    X(1, 1, 4, 2, 8) X(2, 4, 5, 2, 4) X(2, 4, 6, 2, 4)

// 4x4x4-MFMA split-K kernels for 2..8 tokens: X(token groups of 4, chunks per lane, row steps per
// item, blocks per row group). Three and four token groups measured slower than the 16x16x32
// kernels at 12-16 tokens and need more registers than 1024-thread groups allow.
#define W4A16_MFMA4_CONFIGS(X)                                                               \
    X(1, 1, 1, 16) X(1, 2, 1, 16) X(1, 4, 1, 16) X(1, 1, 2, 16) X(1, 2, 2, 16) X(1, 4, 2, 16)  \
    X(2, 1, 1, 16) X(2, 2, 1, 16) X(2, 4, 1, 16) X(2, 1, 2, 16) X(2, 2, 2, 16)               \
    X(1, 1, 1, 8) X(1, 1, 2, 8) X(1, 3, 1, 8) X(2, 1, 1, 8) X(2, 1, 2, 8) X(2, 3, 1, 8)

// Grouped-expert GEMV over three-bit experts: X(lanes per row, 32-code blocks per lane per item).
#define W4A16_MOE3_CONFIGS(X) X(8, 3) X(8, 1) X(4, 3) X(4, 1)

// Activation modes of the 16x16x32 kernel (its XMODE template argument) as plan flags:
// 0 global, operand order; 1 staged; 2 staged, whole-line weights; 3 global, whole-line weights
// and activations; 4 mode 2 with 8 token slots; 5 global, token-row activation loads; 6 mode 5
// with 8 token slots.
constexpr bool xmode_xlds(int x) { return x == 1 || x == 2 || x == 4; }
constexpr bool xmode_lines(int x) { return x >= 2 && x <= 4; }
constexpr bool xmode_slots8(int x) { return x == 4 || x == 6; }
constexpr bool xmode_trows(int x) { return x == 5 || x == 6; }

struct Plan {
    int kind;
    int MT, L, V, U;   // VALU: tokens, lanes per row, chunks per lane per item, row steps per item
    int T, KS;         // MFMA: 16-row tiles per wave, waves splitting K (V: groups per item)
    bool xlds;         // MFMA: activations of all 16 token slots staged in LDS
    bool lines;        // MFMA (staged activations): whole-line weight loads permuted via LDS
    bool slots8;       // MFMA (M <= 8): 8 token slots instead of 16 (staged whole-line or trows)
    bool trows;        // MFMA (global activations): whole token rows loaded, exchanged via LDS
    bool moe;          // rows through expert ids (grouped and SwiGLU forms)
    int mode;          // PlanMode (staged VALU)
    int64_t kr;        // combine form: length of one weight row (K is the activation length)
    int threads;       // work-group size
    int64_t blocks;    // grid size
    int64_t lds_bytes; // dynamic LDS per work-group
    int64_t rows_per_block; // split-K: rows owned by one work-group
};

struct GemvArgs {
    const void *qweight;   // uint32 words, viewed as 16-byte chunks by the kernels
    const void *scales;    // fp16 bits
    const void *X;         // bf16 bits, M rows of stride ldx
    int64_t ldx;
    void *Y;               // fp32, M rows of stride ldy (MoE: [topk][N], ldy = N)
    int64_t ldy;
    const void *ids;       // MoE expert ids (device), else null
    int32_t topk;
    int32_t E;
    int64_t N;
    int32_t K;
    int32_t M;
    const float *route_w;  // combine form: router weights (device), else null
    int32_t KR;            // combine form: weight row length I (K = topk * I); else K
};

struct Moe3Args {
    const void *qweight;   // uint32 [E][N][3K/32]: 32 three-bit codes per 3 words
    const void *scales;    // fp16 bits [E][N][K/128]
    const void *x;         // bf16 bits [K]
    void *y;               // fp32 [topk][N]
    const void *ids;       // int32 [topk] expert ids (device)
    int32_t topk;
    int32_t E;
    int64_t N;
    int32_t K;
};

// Grouped-expert three-bit GEMV, one token. Returns false when no kernel covers the shape.
bool make_moe3_plan(int64_t N, int64_t K, int topk, int cus, int64_t lds_limit, Plan *p);

// Largest K handled by the VALU kernel for MT tokens (activations staged in LDS).
int64_t valu_max_k(int MT, int64_t lds_limit);

// True if the (kind, MT, L, V, U) or (T, KS) tuple is an instantiated kernel.
bool plan_instantiated(const Plan &p);

// Fill `p` with the kernel and launch shape for a call (topk = 0 for dense calls).
// Returns false when no kernel covers the shape.
bool make_plan(int M, int64_t N, int64_t K, int topk, int cus, int64_t lds_limit, Plan *p);

// Expert tail: mode PLAN_MODE_SWIGLU (N = 2I rows per expert, K) or PLAN_MODE_COMBINE (N = H
// rows, K = topk * KR activation values, KR the weight row length). Returns false when no kernel
// covers the shape.
bool make_tail_plan(int mode, int64_t N, int64_t K, int64_t KR, int topk, int cus,
                    int64_t lds_limit, Plan *p);

// Grouped-expert GEMV of M tokens, each with topk experts (M * topk <= 256). Returns false when
// the activations of the M tokens do not fit in LDS.
bool make_moe_batched_plan(int M, int64_t N, int64_t K, int topk, int cus, int64_t lds_limit,
                           Plan *p);
// The grouped-expert plan of one form (PLAN_MOE_BATCHED or PLAN_MOE_BATCHED_MFMA4).
bool make_moe_batched_plan_of(int kind, int M, int64_t N, int64_t K, int topk, int cus,
                              int64_t lds_limit, Plan *p);

// Launch-shape override for tuning: keeps the caller's kernel choice, fills in grid and LDS.
bool finish_plan(int M, int64_t N, int64_t K, int topk, int cus, int64_t lds_limit,
                 int blocks_per_cu, Plan *p);

// Human-readable one-line description; returns the number of characters written.
int describe_plan(const Plan &p, char *buf, size_t len);

}  // namespace w4a16
