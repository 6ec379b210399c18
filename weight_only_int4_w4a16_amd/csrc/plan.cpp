// Launch planning: which kernel and launch shape serves a (M, N, K, topk) call.
#include "plan.h"

#include <stdio.h>

namespace w4a16 {

static constexpr int kMaxWavesPerCu = 32;

int64_t valu_max_k(int MT, int64_t lds_limit)
{
    // Activations (2 bytes per value) plus one fp32 group factor per 32 values, per token.
    const int64_t per_k = 2 * MT;
    int64_t k = (lds_limit * 32) / (per_k * 32 + 4 * MT);
    k -= k % 128;
    return k < 65536 ? k : 65536;
}

bool plan_instantiated(const Plan &p)
{
#define W4A16_VALU_MATCH(MT_, L_, V_, U_)                                                     \
    if (p.kind == PLAN_VALU && p.MT == MT_ && p.L == L_ && p.V == V_ && p.U == U_ &&           \
        (p.mode == PLAN_MODE_DENSE || (p.mode == PLAN_MODE_MOE && MT_ == 1)))                  \
        return true;
#define W4A16_TAIL_MATCH(L_, V_)                                                              \
    if (p.kind == PLAN_VALU && p.MT == 1 && p.L == L_ && p.V == V_ && p.U == 1 &&              \
        (p.mode == PLAN_MODE_COMBINE || (p.mode == PLAN_MODE_SWIGLU && L_ <= 32)))             \
        return true;
#define W4A16_SPLITK_MATCH(MT_, L_, CL_, U_)                                                  \
    if (p.kind == PLAN_SPLITK && p.MT == MT_ && p.L == L_ && p.V == CL_ && p.U == U_ &&        \
        p.mode == PLAN_MODE_DENSE)                                                            \
        return true;
#define W4A16_GATHER_MATCH(L_, CL_)                                                           \
    if (p.kind == PLAN_SPLITK && p.MT == 1 && p.L == L_ && p.V == CL_ && p.U == 1 &&           \
        p.mode == PLAN_MODE_COMBINE)                                                          \
        return true;
#define W4A16_MFMA_MATCH(T_, KS_, XL_, GU_, WPB_)                                            \
    if (p.kind == PLAN_MFMA && p.T == T_ && p.KS == KS_ && p.xlds == xmode_xlds(XL_) &&       \
        p.lines == xmode_lines(XL_) && p.slots8 == xmode_slots8(XL_) &&                       \
        p.trows == xmode_trows(XL_) && p.V == GU_ && (p.threads == 0 || p.threads == 64 * WPB_)) \
        return true;
#define W4A16_MOE_BATCHED_MATCH(L_, V_)                                                       \
    if (p.kind == PLAN_MOE_BATCHED && p.L == L_ && p.V == V_)                                   \
        return true;
#define W4A16_MOE_BATCHED_MFMA4_MATCH(BR_, CL_, U_)                                           \
    if (p.kind == PLAN_MOE_BATCHED_MFMA4 && p.L == BR_ && p.V == CL_ && p.U == U_)              \
        return true;
#define W4A16_MFMA4_MATCH(TG_, CL_, U_, BR_)                                                  \
    if (p.kind == PLAN_MFMA4 && p.MT == TG_ && p.V == CL_ && p.U == U_ && p.L == BR_)           \
        return true;
#define W4A16_MOE3_MATCH(L_, V_)                                                              \
    if (p.kind == PLAN_MOE3 && p.L == L_ && p.V == V_)                                          \
        return true;
    W4A16_VALU_CONFIGS(W4A16_VALU_MATCH)
    W4A16_MOE3_CONFIGS(W4A16_MOE3_MATCH)
    W4A16_TAIL_CONFIGS(W4A16_TAIL_MATCH)
    W4A16_MFMA_CONFIGS(W4A16_MFMA_MATCH)
    W4A16_MFMA4_CONFIGS(W4A16_MFMA4_MATCH)
    W4A16_MOE_BATCHED_CONFIGS(W4A16_MOE_BATCHED_MATCH)
    W4A16_MOE_BATCHED_MFMA4_CONFIGS(W4A16_MOE_BATCHED_MFMA4_MATCH)
    W4A16_SPLITK_CONFIGS(W4A16_SPLITK_MATCH)
    W4A16_GATHER_CONFIGS(W4A16_GATHER_MATCH)
#undef W4A16_SPLITK_MATCH
#undef W4A16_GATHER_MATCH
#undef W4A16_VALU_MATCH
#undef W4A16_TAIL_MATCH
#undef W4A16_MFMA_MATCH
#undef W4A16_MFMA4_MATCH
#undef W4A16_MOE_BATCHED_MATCH
#undef W4A16_MOE_BATCHED_MFMA4_MATCH
#undef W4A16_MOE3_MATCH
    return false;
}

static int lanes_per_row(int64_t cpr)
{
    for (int L = 64; L >= 4; L >>= 1)
        if (cpr % L == 0)
            return L;
    return 0;
}

bool finish_plan(int M, int64_t N, int64_t K, int topk, int cus, int64_t lds_limit,
                 int blocks_per_cu, Plan *p)
{
    if (cus < 1 || blocks_per_cu < 1 || !plan_instantiated(*p))
        return false;
    const int64_t cpr = K / 32;
    const int64_t gpr = K / 128;
    if (p->kind == PLAN_VALU) {
        if (p->MT != M || cpr % ((int64_t)p->L * p->V) != 0)
            return false;
        // The combine form reads batches of L*V chunks that must not straddle two slots.
        if (p->mode == PLAN_MODE_COMBINE &&
            (p->kr < 128 || p->kr % 128 != 0 || (p->kr / 32) % ((int64_t)p->L * p->V) != 0 ||
             K != (int64_t)topk * p->kr))
            return false;
        if (p->mode == PLAN_MODE_SWIGLU && (N % 2 != 0 || N < 2))
            return false;
        if (p->threads == 0)
            p->threads = 256;
        if (p->threads % 64 || p->threads < 64 || p->threads > 256)
            return false;
        p->lds_bytes = (int64_t)p->MT * (K * 2 + cpr * 4) +
                       (p->mode == PLAN_MODE_DENSE ? 0 : 4LL * topk) +
                       (p->mode == PLAN_MODE_COMBINE ? 4LL * topk : 0);
        if (p->lds_bytes > lds_limit)
            return false;
        const int64_t rows = p->mode == PLAN_MODE_MOE ? (int64_t)topk * N : N;
        const int64_t rows_per_wave_step = (int64_t)p->U * (64 / p->L);
        int64_t n_super = (rows + rows_per_wave_step - 1) / rows_per_wave_step;
        if (p->mode == PLAN_MODE_SWIGLU) {
            const int64_t half = rows_per_wave_step / 2;
            n_super = (int64_t)topk * ((N / 2 + half - 1) / half);
        }
        const int wpb = p->threads / 64;
        int64_t blocks = (n_super + wpb - 1) / wpb;
        int per_cu = blocks_per_cu;
        if (per_cu * wpb > kMaxWavesPerCu)
            per_cu = kMaxWavesPerCu / wpb;
        const int64_t by_lds = lds_limit / (p->lds_bytes > 0 ? p->lds_bytes : 1);
        if (per_cu > by_lds)
            per_cu = (int)by_lds;
        if (per_cu < 1)
            per_cu = 1;
        const int64_t cap = (int64_t)cus * per_cu;
        p->blocks = blocks < cap ? blocks : cap;
        return p->blocks >= 1;
    }
    if (p->kind == PLAN_MFMA4) {
        // MT holds the token groups of 4, V the chunks per lane and L the blocks per row group
        // (8 or 16): a wave covers L * V chunks of K and the number of waves follows from K (up
        // to 16 with one chunk per lane, else 8). Dense calls only.
        const int64_t per_wave = (int64_t)p->L * p->V;
        if (p->MT != (M + 3) / 4 || M < 2 || p->moe || (p->L != 8 && p->L != 16) ||
            cpr % per_wave != 0)
            return false;
        const int64_t waves = cpr / per_wave;
        if (waves < 1 || waves > (p->V == 1 ? 16 : 8))
            return false;
        p->threads = (int)(64 * waves);
        int per_cu = blocks_per_cu;
        if (per_cu * waves > kMaxWavesPerCu)
            per_cu = (int)(kMaxWavesPerCu / waves);
        if (per_cu < 1)
            per_cu = 1;
        int64_t blocks = (int64_t)cus * per_cu;
        const int64_t step = 4LL * (16 / p->L) * p->U;     // rows per item
        int64_t rpb = (N + blocks - 1) / blocks;
        rpb = (rpb + step - 1) / step * step;
        const int64_t max_rpb = lds_limit / (4 * waves * M);
        if (rpb > max_rpb)
            rpb = max_rpb / step * step;
        if (rpb < step)
            return false;
        blocks = (N + rpb - 1) / rpb;
        p->rows_per_block = rpb;
        p->blocks = blocks;
        p->lds_bytes = 4 * waves * M * rpb;
        return blocks >= 1 && blocks < (1LL << 31);
    }
    if (p->kind == PLAN_SPLITK) {
        // V holds the chunks per lane; the number of waves follows from K. Dense calls only.
        const int64_t per_wave = (int64_t)p->L * p->V;
        if (p->MT != M || p->moe || cpr % per_wave != 0)
            return false;
        // Combine form: every chunk step of a wave lies in one slot.
        if (p->mode == PLAN_MODE_COMBINE &&
            (p->kr < 128 || p->kr % 128 != 0 || (p->kr / 32) % p->L != 0 ||
             K != (int64_t)topk * p->kr))
            return false;
        const int64_t waves = cpr / per_wave;
        if (waves < 1 || waves > 8)
            return false;
        p->threads = (int)(64 * waves);
        const int64_t rows = p->moe ? (int64_t)topk * N : N;
        int per_cu = blocks_per_cu;
        if (per_cu * waves > kMaxWavesPerCu)
            per_cu = (int)(kMaxWavesPerCu / waves);
        if (per_cu < 1)
            per_cu = 1;
        int64_t blocks = (int64_t)cus * per_cu;
        const int64_t step = (int64_t)p->U * (64 / p->L);     // rows per item
        int64_t rpb = (rows + blocks - 1) / blocks;
        rpb = (rpb + step - 1) / step * step;
        const int64_t max_rpb = lds_limit / (4 * waves * p->MT);
        if (rpb > max_rpb)
            rpb = max_rpb / step * step;
        if (rpb < step)
            return false;
        blocks = (rows + rpb - 1) / rpb;
        p->rows_per_block = rpb;
        p->blocks = blocks;
        p->lds_bytes = 4 * waves * p->MT * rpb;
        return blocks >= 1 && blocks < (1LL << 31);
    }
    if (p->kind == PLAN_MFMA) {
        if (p->threads == 0)
            p->threads = 256;
        const int wpb = p->threads / 64;
        if (p->threads % 64 || wpb < 1 || wpb % p->KS != 0 || !plan_instantiated(*p))
            return false;
        if (p->V < 1 || gpr % p->KS != 0 || (gpr / p->KS) % p->V != 0 || (p->xlds && p->KS != 1))
            return false;
        if (p->lines && (p->V % 2 != 0 || (p->xlds && p->T != 1)))
            return false;
        if (p->slots8 && (M > 8 || !((p->xlds && p->lines) || p->trows)))
            return false;
        if (p->trows && (p->xlds || p->lines || (p->V != 1 && p->V != 2 && p->V != 4)))
            return false;
        const int64_t rows_per_block = 16LL * p->T * (wpb / p->KS);
        const int64_t row_blocks = (N + rows_per_block - 1) / rows_per_block;
        if (p->xlds) {
            // 16 token slots (8 for the 8-slot form) of activation fragments (16 bytes per
            // lane, word and group) plus one fp32 factor per (group, token); with line loads,
            // one 1 KiB staging slot per group of an item and wave.
            p->lds_bytes = gpr * (p->slots8 ? 2048 : 4096) + gpr * 64 +
                           (p->lines ? (int64_t)wpb * p->V * 1024 : 0);
            if (p->lds_bytes > lds_limit)
                return false;
            int per_cu = blocks_per_cu;
            const int64_t by_lds = lds_limit / p->lds_bytes;
            if (per_cu > by_lds)
                per_cu = (int)by_lds;
            if (per_cu < 1)
                per_cu = 1;
            const int64_t cap = (int64_t)cus * per_cu;
            p->blocks = row_blocks < cap ? row_blocks : cap;
        } else {
            // K-split partial sums, with line loads a staging slot per wave for the weights
            // (T x groups per item) and activation fragments (4 x groups per item), with token-row
            // loads one for the item's activations (token slots x groups per item x 256 bytes),
            // and per wave the 16 token rows' group factors of an item (groups per item x 64
            // bytes).
            p->lds_bytes = (p->KS > 1 ? (int64_t)wpb * p->T * 64 * 16 : 0) +
                           (p->lines ? (int64_t)wpb * (p->T + 4) * p->V * 1024 : 0) +
                           (p->trows ? (int64_t)wpb * (p->slots8 ? 8 : 16) * p->V * 256 : 0) +
                           (int64_t)wpb * p->V * 64;
            if (p->lds_bytes > lds_limit)
                return false;
            p->blocks = row_blocks;
        }
        return p->blocks >= 1 && p->blocks < (1LL << 31);
    }
    return false;
}

// Dispatch rules, from launch-shape sweeps on MI355X with weights rotated through more than
// 1 GiB of copies (so the 256 MB memory-side cache cannot serve them):
//  * dense, 1-4 tokens, K a multiple of 2048 up to 16384 (from 4096 for 2-4 tokens): split-K with
//    64 lanes per row and 4 rows per item, about 8 waves per CU (one work-group of K/2048 waves,
//    8/W groups per CU); very short one-token matrices (<= 16 rows per CU) use 32 lanes and 2-row
//    items instead, and tall one-token matrices with K = 4096 (>= 16384 rows) or K = 2048
//    (>= 8192 rows) the staged kernel with 32 lanes per row and 2 chunks per item; K above 16384
//    uses 2 or 4 chunks per lane so that a work-group stays within 8 waves;
//  * other K, and every grouped-expert call: the staged kernel with the widest power-of-two lanes
//    per row dividing the row's 16-byte chunks; rows of 72 chunks (K = 2304) use 8 lanes with
//    3 chunks per item;
//  * 2-16 tokens: MFMA (see mfma_slots8_plan, mfma_rows8_plan, mfma4_plan and mfma_plan), except 2 tokens with K
//    a multiple of 2048, which stay on split-K VALU.
namespace {

int pow2_lanes(int64_t cpr)
{
    for (int L = 64; L >= 4; L >>= 1)
        if (cpr % L == 0)
            return L;
    return 0;
}

bool try_plan(Plan c, int bpc, int M, int64_t N, int64_t K, int topk, int cus, int64_t lds,
              Plan *p)
{
    if (!plan_instantiated(c) || !finish_plan(M, N, K, topk, cus, lds, bpc, &c))
        return false;
    *p = c;
    return true;
}

Plan valu(int MT, int L, int V, int U, bool moe)
{
    Plan c{};
    c.kind = PLAN_VALU;
    c.MT = MT;
    c.L = L;
    c.V = V;
    c.U = U;
    c.moe = moe;
    c.mode = moe ? PLAN_MODE_MOE : PLAN_MODE_DENSE;
    return c;
}

Plan splitk(int MT, int L, int CL, int U, bool moe)
{
    Plan c = valu(MT, L, CL, U, moe);
    c.kind = PLAN_SPLITK;
    return c;
}

}  // namespace

// MFMA forms for 2..16 tokens, in order of preference (launch-shape sweeps on MI355X):
//  1. activations staged in LDS with whole-line weight loads, 8 waves of 16 rows per
//     work-group, when there are enough row blocks to fill the chip (N/128 >= 0.8 * CUs) and the
//     staging fits in LDS: tall matrices (163840 x 2304, 28672 x 4096);
//  2. activations from global memory, K split over 4 waves: four 16-row tiles per wave with
//     whole-line weight and activation loads when that still fills the chip (14336 x 2048:
//     9.7 us against 10.6 with token-row activation loads; 16384 x 4096: 13.8 against 15.9),
//     else two tiles with token-row activation loads (8192 x 8192: 16.1-16.4 us against
//     17.9-18.1 with operand-order loads);
//  3. token-row loads with one tile per wave and K split over 8 waves, for short matrices with
//     long rows (4096 x 14336: 21.2 us against 25.1 with whole-line loads; 4096 x 4096: 9.7
//     against 11.5; 1024 x 2048: 5.9 against 6.3);
//  4. staged activations with whole-line loads in 4-wave work-groups (4096 x 2304, small N);
//  5. the remaining forms, which cover every K that is a multiple of 128.
// Groups per item: even so that line pairs (or both 64-byte halves of a line) go together.
static bool mfma_plan(int M, int64_t N, int64_t K, int cus, int64_t lds_limit, Plan *p)
{
    const int64_t gpr = K / 128;
    // Groups per item: 2 first for 8-wave work-groups (163840 x 2304 at 16 tokens, same-box sweep:
    // 45.1 us against 47.0 with 6), 6 first for the 4-wave form.
    auto lines = [&](int wpb, Plan *out) {
        static const int gus8[] = {2, 6, 4}, gus4[] = {6, 4, 2};
        for (int gu : (wpb == 8 ? gus8 : gus4)) {
            Plan c{};
            c.kind = PLAN_MFMA;
            c.T = 1;
            c.KS = 1;
            c.V = gu;
            c.xlds = true;
            c.lines = true;
            c.threads = 64 * wpb;
            if (gpr % gu == 0 && try_plan(c, 2, M, N, K, 0, cus, lds_limit, out))
                return true;
        }
        return false;
    };
    // Activation loads of the global forms: 0 operand order, 1 whole lines, 2 token rows.
    auto global = [&](int T, int KS, int GU, int wpb, int xload, Plan *out) {
        Plan c{};
        c.kind = PLAN_MFMA;
        c.T = T;
        c.KS = KS;
        c.V = GU;
        c.lines = xload == 1;
        c.trows = xload == 2;
        c.threads = 64 * wpb;
        return gpr % (KS * GU) == 0 && try_plan(c, 1, M, N, K, 0, cus, lds_limit, out);
    };
    if (N / 128 >= (int64_t)cus * 4 / 5 && lines(8, p))
        return true;
    if (N / 64 >= (int64_t)cus * 4 / 5 && global(4, 4, 2, 4, 1, p))
        return true;
    if (N / 32 >= cus && global(2, 4, 2, 4, 2, p))
        return true;
    if (gpr % 16 == 0 && global(1, 8, 2, 8, 2, p))
        return true;
    if (lines(4, p))
        return true;
    if (gpr * 4160 <= lds_limit / 2) {
        static const int gus[] = {6, 4, 2, 1};
        for (int gu : gus) {
            Plan c{};
            c.kind = PLAN_MFMA;
            c.T = 1;
            c.KS = 1;
            c.V = gu;
            c.xlds = true;
            c.threads = 512;
            if (gpr % gu == 0 && try_plan(c, 1, M, N, K, 0, cus, lds_limit, p))
                return true;
        }
    }
    static const int mf[][3] = {{2, 4, 2}, {2, 2, 2}, {2, 1, 2}, {1, 1, 2}, {1, 1, 1}};
    for (int i = 0; i < (int)(sizeof(mf) / sizeof(mf[0])); ++i)
        if (global(mf[i][0], mf[i][1], mf[i][2], 4, 0, p))
            return true;
    return false;
}

// 4x4x4-MFMA split-K for 2..8 tokens (one or two token groups), from launch-shape sweeps on
// MI355X with rotated weights:
// (times are medians of interleaved rounds of the same graph-timed calls):
//  - rows of a multiple of 16 chunks of at least 128 chunks (K >= 4096): 16 blocks per row
//    group, 2 chunks per lane (4 with two token groups or for K = 14336); two row steps per item
//    and 2 work-groups per CU on tall matrices (28672 x 4096 at 4 tokens: 13.6 us against 29.2
//    us for split-K VALU), else one and one (8192 x 8192 at 4 tokens: 10.5 against 12.3 us; at
//    8 tokens with 4 chunks per lane: 13.5 against 14.0 us for the 16x16x32 kernel);
//  - shorter rows of a multiple of 8 chunks (K <= 2048) and rows of 72 chunks (K = 2304): 8
//    blocks per row group; one chunk per lane and two row steps (14336 x 2048 at 4 tokens: 6.6
//    against 9.0 us with 16 blocks, 11.0 for VALU), or 3 chunks per lane for 72 chunks with 4
//    work-groups per CU on tall matrices (163840 x 2304 at 2 tokens: 34.4 against 37.1 us)
//    and 1 otherwise (4096 x 2304 at 4 tokens: 4.3 against 8.7 us).
static bool mfma4_plan(int M, int64_t N, int64_t K, int cus, int64_t lds_limit, Plan *p)
{
    const int64_t cpr = K / 32;
    Plan c{};
    c.kind = PLAN_MFMA4;
    c.MT = (M + 3) / 4;
    const bool tall = N >= 16384;
    int bpc = 1;
    if (cpr % 16 == 0 && cpr >= 128) {
        c.L = 16;
        c.V = cpr / 32 > 8 ? 4 : 2;
        c.U = c.MT == 1 && tall ? 2 : 1;
        bpc = tall ? 2 : 1;
    } else if (cpr % 8 == 0 && cpr <= 64) {
        c.L = 8;
        c.V = 1;
        c.U = c.MT == 1 ? 2 : 1;     // 14336 x 2048 at 8 tokens: 8.6 us with one step, 9.0 two
    } else if (cpr % 8 == 0) {
        c.L = 8;
        c.V = (cpr / 8) % 3 == 0 ? 3 : 1;
        c.U = 1;
        bpc = tall ? 4 : 1;
    } else {
        return false;
    }
    return try_plan(c, bpc, M, N, K, 0, cus, lds_limit, p);
}

// The staged whole-line MFMA form with 8 token slots (M <= 8), 2 groups per item and 8 waves per
// work-group, on matrices with enough 128-row blocks to fill the chip, when two work-groups fit
// in one CU's LDS: halving the staged activations doubles the waves per CU.
static bool mfma_slots8_plan(int M, int64_t N, int64_t K, int cus, int64_t lds_limit, Plan *p)
{
    const int64_t gpr = K / 128;
    if (M > 8 || N / 128 < (int64_t)cus * 4 / 5 || gpr % 2 != 0 ||
        2 * (gpr * 2048 + gpr * 64 + 8 * 2 * 1024) > lds_limit)
        return false;
    Plan c{};
    c.kind = PLAN_MFMA;
    c.T = 1;
    c.KS = 1;
    c.V = 2;
    c.xlds = true;
    c.lines = true;
    c.slots8 = true;
    c.threads = 512;
    return try_plan(c, 2, M, N, K, 0, cus, lds_limit, p);
}

// 5-8 tokens on matrices of up to 16384 rows: the global-activation 16x16x32 form with 8 token
// slots loaded as token rows, two 16-row tiles per wave and K split over 4 waves, when its
// 32-row work-groups spread evenly over the CUs (whole rounds within 10 %). Same-box sweeps
// against the 4x4x4 kernel: 8192 x 8192 at 5-8 tokens 13.1-13.5 us against 13.9-15.3, 8192 x
// 4096 8.6 against 9.8-10.1, 8192 x 14336 20.3-21.4 against 21.9-24.2, 16384 x 4096 13.8-14.5
// against 14.0-14.9; with uneven rounds the 4x4x4 kernel stays ahead (12288 x 8192: 18.6-19.8
// us against 21.9-22.7; 14336 x 2048 at 8: 9.3 against 9.9; 4096 x 14336 at 8: 17.7 against
// 18.3).
static bool mfma_rows8_plan(int M, int64_t N, int64_t K, int cus, int64_t lds_limit, Plan *p)
{
    const int64_t gpr = K / 128;
    const int64_t blocks = (N + 31) / 32;
    const int64_t rounds = (blocks + cus - 1) / cus;
    if (M < 5 || M > 8 || N > 16384 || gpr % 8 != 0 || blocks * 10 < rounds * cus * 9)
        return false;
    Plan c{};
    c.kind = PLAN_MFMA;
    c.T = 2;
    c.KS = 4;
    c.V = 2;
    c.trows = true;
    c.slots8 = true;
    c.threads = 256;
    return try_plan(c, 1, M, N, K, 0, cus, lds_limit, p);
}

// Whether 3 or 4 tokens are better served by the MFMA kernel than by the VALU ones: tall
// matrices whose rows are not a multiple of 2048 values (the split-K VALU kernel's shapes) and
// hold an even number of groups (whole-line loads), where decoding each weight once for all tokens on the matrix cores beats 3-4 dot products
// per weight on the VALU (163840 x 2304 at 3-4 tokens: 38 us against 49-57 us).
static bool mfma_for_few_tokens(int M, int64_t N, int64_t K, int cus)
{
    return M >= 3 && M <= 4 && K % 2048 != 0 && (K / 128) % 2 == 0 &&
           N / 128 >= (int64_t)cus * 4 / 5;
}

bool make_plan(int M, int64_t N, int64_t K, int topk, int cus, int64_t lds_limit, Plan *p)
{
    *p = Plan{};
    if (M < 1 || M > 16 || N < 1 || K < 128 || K % 128 != 0 || topk < 0)
        return false;
    const bool moe = topk > 0;
    if (moe && M != 1)
        return false;
    const int64_t cpr = K / 32;
    const int64_t rows = moe ? (int64_t)topk * N : N;
    const int L = pow2_lanes(cpr);
    const int64_t c64 = cpr / 64;
    const bool k2048 = cpr % 64 == 0;

    const int split_bpc = (int)(c64 >= 8 ? 1 : 8 / (c64 > 0 ? c64 : 1));
    // K = 4096, one token, tall: split K over 4 waves of 32 lanes with 4 row steps in flight,
    // one work-group per CU (28672 x 4096, same-box sweep: 11.84 us against 12.25 with 2 row steps
    // and 2 work-groups per CU and 11.92 for the staged kernel).
    if (!moe && M == 1 && K == 4096 && rows >= 16384 &&
        try_plan(splitk(1, 32, 1, 4, false), 1, M, N, K, topk, cus, lds_limit, p))
        return true;
    // K = 2048, one token: tall matrices take the staged kernel with 32 lanes and 2 chunks per
    // item (14336 x 2048: 4.9 us against 6.9 us for 64 lanes), the others split K like the
    // longer rows below.
    if (!moe && M == 1 && K == 2048 && rows >= 8192 &&
        try_plan(valu(1, 32, 2, 1, false), 4, M, N, K, topk, cus, lds_limit, p))
        return true;
    // 5-8 tokens on tall matrices (at least 0.8 x CUs blocks of 128 rows) whose rows are not a
    // multiple of 2048 values: the staged whole-line 16x16x32 form with 8 token slots and 2 groups
    // per item, where two 8-wave work-groups fit in one CU's LDS. 2-4 tokens take the 4x4x4
    // kernel below (163840 x 2304, same-box sweep: 36.1 us at 2 tokens and 38.3 at 4 against
    // 40.3 and 39.6 for the 8-slot form).
    if (!moe && M >= 5 && M <= 8 && K % 2048 != 0 &&
        mfma_slots8_plan(M, N, K, cus, lds_limit, p))
        return true;
    // 3-4 tokens: the 4x4x4-MFMA split-K kernel wherever its lane layout fits the row.
    if (!moe && M >= 3 && M <= 4 && mfma4_plan(M, N, K, cus, lds_limit, p))
        return true;
    if (!moe && k2048 && (c64 >= 2 || M <= 2) && c64 <= 8 && M <= 4) {
        if (M == 1 && rows <= 16LL * cus &&
            try_plan(splitk(1, 32, 1, 2, false), 2, M, N, K, topk, cus, lds_limit, p))
            return true;
        if (try_plan(splitk(M, 64, 1, 4, false), split_bpc, M, N, K, topk, cus, lds_limit, p))
            return true;
    }
    if (!moe && k2048 && c64 > 8 && M == 1) {
        if (try_plan(splitk(1, 64, 2, 4, false), 1, M, N, K, topk, cus, lds_limit, p) ||
            try_plan(splitk(1, 64, 4, 2, false), 1, M, N, K, topk, cus, lds_limit, p))
            return true;
    }
    // One token, rows of 32k chunks that are not a multiple of 64 (K = 3072, 5120, 7168): split
    // K over 32 lanes, 2 chunks in flight per lane (4096 x 7168: 5.2 us against 6.6 us staged;
    // 16384 x 3072: 6.7 against 7.4).
    if (!moe && M == 1 && !k2048 && cpr % 32 == 0 && cpr >= 96 &&
        try_plan(splitk(1, 32, 1, 2, false), rows < 8192 ? 2 : 4, M, N, K, topk, cus, lds_limit, p))
        return true;
    if (M == 1) {
        // rows of 48 chunks (K = 1536): 8 lanes with 3 chunks per item, like rows of 72 chunks
        if (!moe && L == 16 && (cpr / 8) % 3 == 0 &&
            try_plan(valu(1, 8, 3, 1, false), 4, M, N, K, topk, cus, lds_limit, p))
            return true;
        // Rows of 72 chunks (K = 2304). Dense: 8 lanes x one chunk per item x 2 row steps, 6
        // work-groups per CU (163840 x 2304, same-box sweep: 30.95 us against 32.7 for 3 chunks
        // per item and one row step). Grouped experts: 8 lanes x 3 chunks per item.
        if (!moe && L == 8 && (cpr / 8) % 3 == 0 &&
            try_plan(valu(1, 8, 1, 2, false), 6, M, N, K, topk, cus, lds_limit, p))
            return true;
        if (L == 8 && (cpr / 8) % 3 == 0 &&
            try_plan(valu(1, 8, 3, 1, moe), 8, M, N, K, topk, cus, lds_limit, p))
            return true;
        if (L == 8 && try_plan(valu(1, 8, 1, 2, moe), 6, M, N, K, topk, cus, lds_limit, p))
            return true;
        if (L == 64 && c64 == 1 && try_plan(valu(1, 64, 1, 1, moe), 2, M, N, K, topk, cus, lds_limit, p))
            return true;
        if (L >= 16 && try_plan(valu(1, L == 64 ? 32 : L, 1, 2, moe), 6, M, N, K, topk, cus, lds_limit, p))
            return true;
        if (L == 4 && try_plan(valu(1, 4, 1, 2, moe), 6, M, N, K, topk, cus, lds_limit, p))
            return true;
        return try_plan(valu(1, L, 1, 1, moe), 6, M, N, K, topk, cus, lds_limit, p);
    }
    // 2 tokens where split-K VALU does not apply (it wins where it does: 8192 x 8192 at 2 tokens
    // 9.0 us against 9.7, 14336 x 2048 5.9 against 6.2), and 5-8 tokens on matrices of up to
    // 16384 rows where the 8-slot token-row form does not apply (16384 x 4096 at 8 with the
    // operand-order 16x16x32 form: 13.5 against 13.8; 4096 x 2304 at 8: 5.7 against 10.8).
    // Taller matrices at 5-8 tokens keep the 16x16x32 kernels (28672 x 4096 at 8: 18.5 against
    // 19.5 us; 163840 x 2304 at 6: 37.0 against 48.6).
    if (!moe && mfma_rows8_plan(M, N, K, cus, lds_limit, p))
        return true;
    if (!moe && (M == 2 || (M >= 5 && M <= 8 && N <= 16384)) &&
        mfma4_plan(M, N, K, cus, lds_limit, p))
        return true;
    if (!moe && mfma_for_few_tokens(M, N, K, cus) && mfma_plan(M, N, K, cus, lds_limit, p))
        return true;
    if (M <= 4) {
        if (M == 2 && L == 8 && try_plan(valu(2, 8, 1, 2, false), 4, M, N, K, topk, cus, lds_limit, p))
            return true;
        if (try_plan(valu(M, L, 1, 1, false), M == 2 ? 4 : 8, M, N, K, topk, cus, lds_limit, p))
            return true;
    }
    return mfma_plan(M, N, K, cus, lds_limit, p);
}

// Grouped-expert GEMV over three-bit experts: 8 lanes per row when they divide the row's 32-code
// blocks, else 4; 3 blocks per item when the lanes' share divides by 3 (K = 2304: 72 blocks,
// 8 lanes x 3 x 3 items), else 1; 4-wave work-groups, persistent, up to 8 per CU (the INT4
// grouped-expert launch shape). At 256 experts of 2048 x 2304, top-8, more lanes per row (16,
// 32, 64, with a ragged last item), one item per row step (9 blocks per lane), and 1- or 2-wave
// work-groups all measured slower.
bool make_moe3_plan(int64_t N, int64_t K, int topk, int cus, int64_t lds_limit, Plan *p)
{
    *p = Plan{};
    if (N < 1 || K < 128 || K % 128 != 0 || topk < 1 || cus < 1)
        return false;
    const int64_t cpr = K / 32;
    Plan c{};
    c.kind = PLAN_MOE3;
    c.MT = 1;
    c.L = cpr % 8 == 0 ? 8 : 4;
    c.V = (cpr / c.L) % 3 == 0 ? 3 : 1;
    c.U = 1;
    c.moe = true;
    c.threads = 256;
    c.lds_bytes = cpr * 68 + 4LL * topk;
    if (c.lds_bytes > lds_limit || !plan_instantiated(c))
        return false;
    const int64_t R = 64 / c.L;
    const int64_t steps = ((int64_t)topk * N + R - 1) / R;
    const int64_t waves = c.threads / 64;
    int64_t per_cu = 8;
    const int64_t by_lds = lds_limit / c.lds_bytes;
    if (per_cu > by_lds)
        per_cu = by_lds;
    const int64_t need = (steps + waves - 1) / waves;
    const int64_t cap = (int64_t)cus * per_cu;
    c.blocks = need < cap ? need : cap;
    *p = c;
    return true;
}

// Expert tail. SwiGLU gate+up: the grouped-expert launch shape (8 lanes with 3 chunks per item for
// rows of 72 chunks, else the widest lanes per row up to 32, one chunk per item). Combine: the
// widest lanes per row up to 32 that divide the chunks of one weight row, one chunk per item,
// which keeps the most waves busy on the short down-projection rows.
bool make_tail_plan(int mode, int64_t N, int64_t K, int64_t KR, int topk, int cus,
                    int64_t lds_limit, Plan *p)
{
    *p = Plan{};
    if (N < 1 || K < 128 || K % 128 != 0 || topk < 1)
        return false;
    if (mode == PLAN_MODE_SWIGLU) {
        const int64_t cpr = K / 32;
        const int L = pow2_lanes(cpr) > 32 ? 32 : pow2_lanes(cpr);
        Plan c = valu(1, 8, 3, 1, true);
        c.mode = PLAN_MODE_SWIGLU;
        if (L == 8 && (cpr / 8) % 3 == 0 && try_plan(c, 8, 1, N, K, topk, cus, lds_limit, p))
            return true;
        c = valu(1, L, 1, 1, true);
        c.mode = PLAN_MODE_SWIGLU;
        return L >= 4 && try_plan(c, 8, 1, N, K, topk, cus, lds_limit, p);
    }
    if (mode == PLAN_MODE_COMBINE) {
        if (KR < 128 || KR % 128 != 0)
            return false;
        const int64_t cprw = KR / 32;
        const int L = pow2_lanes(cprw) > 32 ? 32 : pow2_lanes(cprw);
        // Split-K over the slots when the waves fit a work-group, with the fewest chunks per
        // lane that keep the waves within 8 (2 work-groups per CU); else the staged kernel.
        static const int cls[] = {1, 2, 4, 8};
        for (int cl : cls) {
            Plan c = splitk(1, L, cl, 1, false);
            c.mode = PLAN_MODE_COMBINE;
            c.kr = KR;
            if (try_plan(c, 2, 1, N, K, topk, cus, lds_limit, p))
                return true;
        }
        Plan c = valu(1, L, 1, 1, false);
        c.mode = PLAN_MODE_COMBINE;
        c.kr = KR;
        return L >= 4 && try_plan(c, 8, 1, N, K, topk, cus, lds_limit, p);
    }
    return false;
}

constexpr int kMoeBatchedMT = 1;        // tokens per pass (the kernel is built for 1)
constexpr int kMoeBatchedMfma4U = 1;    // row steps per item (2: 74.6 against 58.1 us, 16 tokens)
// chunks per lane for rows of 24k chunks (K = 768k); 9 (one batch per item at K = 2304) needs
// 161 VGPRs, leaves one work-group per CU and was slower (2 tokens: 16.8 against 12.1 us)
constexpr int kMoeBatchedMfma4CL3 = 3;

// Grouped experts for M tokens: the grouped-expert launch shape of the one-token form (8 lanes
// with 3 chunks per item for rows of 72 chunks, else the widest lanes per row), persistent
// work-groups of 8 waves, two per CU (one if LDS holds only one): 16 waves per CU is what the
// kernel's registers allow, and fewer, longer-lived work-groups amortise the grouping set-up
// (measured on MI355X over 2-16 tokens).
bool make_moe_batched_plan_of(int kind, int M, int64_t N, int64_t K, int topk, int cus,
                              int64_t lds_limit, Plan *p)
{
    *p = Plan{};
    if (M < 1 || M > 16 || topk < 1 || M * topk > 256 || N < 1 || K < 128 || K % 128 != 0 ||
        cus < 1)
        return false;
    const int64_t cpr = K / 32;
    const int64_t P = (int64_t)M * topk;
    int64_t R;
    int64_t ve_ints;      // virtual-entry tables in LDS
    if (kind == PLAN_MOE_BATCHED_MFMA4) {
        // 16 blocks per row group with 2 chunks per lane (or 1), else 8 with 3 (K = 2304) or 1.
        if (cpr % 16 == 0) {
            p->L = 16;
            p->V = cpr % 32 == 0 ? 2 : 1;
        } else if (cpr % 8 == 0) {
            p->L = 8;
            p->V = (cpr / 8) % 3 == 0 ? kMoeBatchedMfma4CL3 : 1;
        } else {
            return false;
        }
        if (cpr % (p->L * p->V) != 0)
            return false;
        p->MT = 4;
        p->U = kMoeBatchedMfma4U;
        R = 4 * (16 / p->L) * p->U;
        ve_ints = P + P * 4 + 1;        // experts, entries of up to 4 slots, count
    } else if (kind == PLAN_MOE_BATCHED) {
        int L = pow2_lanes(cpr), V = 1;
        if (L == 8 && (cpr / 8) % 3 == 0)
            V = 3;
        if (L < 4)
            return false;
        p->L = L;
        p->V = V;
        p->MT = kMoeBatchedMT;
        R = 64 / L;
        ve_ints = P + P * kMoeBatchedMT + 1;
    } else {
        return false;
    }
    p->kind = kind;
    if (kind == PLAN_MOE_BATCHED)
        p->U = 1;
    p->moe = true;
    p->threads = 512;
    if (!plan_instantiated(*p))
        return false;
    // Region A (activations, or the grouping scratch before them) + chunk factors + the
    // virtual-entry tables.
    const int64_t xs_bytes = (int64_t)M * K * 2;
    const int64_t scratch = ((20 * P + 15) / 16) * 16;
    p->lds_bytes = (xs_bytes > scratch ? xs_bytes : scratch) + (int64_t)M * cpr * 4 + 4 * ve_ints;
    if (p->lds_bytes > lds_limit)
        return false;
    int64_t per_cu = lds_limit / p->lds_bytes;
    if (per_cu > 2)
        per_cu = 2;
    const int64_t most = (P * ((N + R - 1) / R) + 7) / 8;   // work-groups that could have work
    p->blocks = (int64_t)cus * per_cu;
    if (p->blocks > most)
        p->blocks = most;
    return p->blocks >= 1 && p->blocks < (1LL << 31);
}

// Grouped experts for several tokens: the 4x4x4-MFMA form wherever its lane layout fits the
// rows, which decodes each weight once for all the tokens that chose its expert; else the VALU
// form (one decode and dot product per token).
bool make_moe_batched_plan(int M, int64_t N, int64_t K, int topk, int cus, int64_t lds_limit,
                           Plan *p)
{
    return make_moe_batched_plan_of(PLAN_MOE_BATCHED_MFMA4, M, N, K, topk, cus, lds_limit, p) ||
           make_moe_batched_plan_of(PLAN_MOE_BATCHED, M, N, K, topk, cus, lds_limit, p);
}

int describe_plan(const Plan &p, char *buf, size_t len)
{
    if (!buf || len == 0)
        return 0;
    if (p.kind == PLAN_MOE3)
        return snprintf(buf, len,
                        "moe3 lanes_per_row=%d blocks_per_item=%d threads=%d blocks=%lld lds=%lld",
                        p.L, p.V, p.threads, (long long)p.blocks, (long long)p.lds_bytes);
    int n = 0;
    if (p.kind == PLAN_VALU)
        n = snprintf(buf, len,
                     "valu%s tokens=%d lanes_per_row=%d chunks_per_item=%d row_steps=%d "
                     "threads=%d blocks=%lld lds=%lld",
                     p.mode == PLAN_MODE_MOE       ? "_moe"
                     : p.mode == PLAN_MODE_SWIGLU  ? "_moe_swiglu"
                     : p.mode == PLAN_MODE_COMBINE ? "_moe_combine"
                                                   : "",
                     p.MT, p.L, p.V, p.U, p.threads, (long long)p.blocks,
                     (long long)p.lds_bytes);
    else if (p.kind == PLAN_SPLITK)
        n = snprintf(buf, len,
                     "splitk%s tokens=%d lanes_per_row=%d chunks_per_lane=%d row_steps=%d "
                     "threads=%d blocks=%lld rows_per_block=%lld lds=%lld",
                     p.mode == PLAN_MODE_COMBINE ? "_moe_combine" : "", p.MT, p.L, p.V, p.U, p.threads, (long long)p.blocks,
                     (long long)p.rows_per_block, (long long)p.lds_bytes);
    else if (p.kind == PLAN_MFMA4)
        n = snprintf(buf, len,
                     "mfma4x4x4_splitk token_groups=%d chunks_per_lane=%d row_steps=%d "
                     "blocks_per_row=%d threads=%d blocks=%lld rows_per_block=%lld lds=%lld",
                     p.MT, p.V, p.U, p.L, p.threads, (long long)p.blocks, (long long)p.rows_per_block,
                     (long long)p.lds_bytes);
    else if (p.kind == PLAN_MOE_BATCHED_MFMA4)
        n = snprintf(buf, len,
                     "moe_batched_mfma4x4x4 slots=%d blocks_per_row=%d chunks_per_lane=%d "
                     "threads=%d blocks=%lld lds=%lld",
                     p.MT, p.L, p.V, p.threads, (long long)p.blocks, (long long)p.lds_bytes);
    else if (p.kind == PLAN_MOE_BATCHED)
        n = snprintf(buf, len,
                     "moe_batched tokens_per_pass=%d lanes_per_row=%d chunks_per_item=%d "
                     "threads=%d blocks=%lld lds=%lld",
                     p.MT, p.L, p.V, p.threads, (long long)p.blocks, (long long)p.lds_bytes);
    else if (p.kind == PLAN_MFMA)
        n = snprintf(buf, len,
                     "mfma16x16x32%s tiles_per_wave=%d k_split=%d groups_per_item=%d threads=%d "
                     "blocks=%lld lds=%lld",
                     p.lines   ? (p.xlds ? (p.slots8 ? "_lds8_lines" : "_lds_lines") : "_lines")
                     : p.trows ? (p.slots8 ? "_rows8" : "_rows")
                     : p.xlds  ? "_lds"
                               : "",
                     p.T,
                     p.KS, p.V, p.threads,
                     (long long)p.blocks, (long long)p.lds_bytes);
    else
        n = snprintf(buf, len, "none");
    return n;
}

}  // namespace w4a16
