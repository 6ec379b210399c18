// Launch planning: which kernel and launch shape serves a (M, N, K, topk) call.
#include "plan.h"

#include <stdio.h>

namespace w4a16 {

static constexpr int kMaxWavesPerCu = 32;

int64_t valu_max_k(int MT, int64_t lds_limit)
{
    // Activations (2 bytes per value) plus one fp32 offset per 32 values, per token.
    const int64_t per_k = 2 * MT;
    int64_t k = (lds_limit * 32) / (per_k * 32 + 4 * MT);
    k -= k % 128;
    return k < 65536 ? k : 65536;
}

bool plan_instantiated(const Plan &p)
{
#define W4A16_VALU_MATCH(MT_, L_, V_, U_)                                                     \
    if (p.kind == PLAN_VALU && p.MT == MT_ && p.L == L_ && p.V == V_ && p.U == U_)             \
        return true;
#define W4A16_MFMA_MATCH(T_, KS_)                                                            \
    if (p.kind == PLAN_MFMA && p.T == T_ && p.KS == KS_)                                      \
        return true;
    W4A16_VALU_CONFIGS(W4A16_VALU_MATCH)
    W4A16_MFMA_CONFIGS(W4A16_MFMA_MATCH)
#undef W4A16_VALU_MATCH
#undef W4A16_MFMA_MATCH
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
        if (p->threads == 0)
            p->threads = 256;
        if (p->threads % 64 || p->threads < 64 || p->threads > 256)
            return false;
        p->lds_bytes = (int64_t)p->MT * (K * 2 + cpr * 4);
        if (p->lds_bytes > lds_limit)
            return false;
        const int64_t rows = p->moe ? (int64_t)topk * N : N;
        const int64_t rows_per_wave_step = (int64_t)p->U * (64 / p->L);
        const int64_t n_super = (rows + rows_per_wave_step - 1) / rows_per_wave_step;
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
    if (p->kind == PLAN_MFMA) {
        if (gpr % p->KS != 0)
            return false;
        p->threads = 256;
        p->lds_bytes = 0;
        const int64_t rows_per_block = 16LL * p->T * (4 / p->KS);
        p->blocks = (N + rows_per_block - 1) / rows_per_block;
        return p->blocks >= 1 && p->blocks < (1LL << 31);
    }
    return false;
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
    const int64_t gpr = K / 128;

    const bool valu = M <= 4 && K <= valu_max_k(M, lds_limit);
    if (valu) {
        const int L = lanes_per_row(cpr);
        const int64_t C = cpr / L;
        // Preferred (V, U) per token count: about eight 16-byte loads in flight per lane.
        static const int pref1[][2] = {{2, 4}, {4, 2}, {9, 1}, {7, 1}, {3, 2}, {1, 4},
                                       {2, 2}, {3, 1}, {1, 2}, {2, 1}};
        static const int prefn[][2] = {{2, 2}, {1, 4}, {3, 1}, {1, 2}, {2, 1}};
        const int(*pref)[2] = M == 1 ? pref1 : prefn;
        const int npref = M == 1 ? (int)(sizeof(pref1) / sizeof(pref1[0]))
                                 : (int)(sizeof(prefn) / sizeof(prefn[0]));
        for (int i = 0; i < npref; ++i) {
            Plan c{};
            c.kind = PLAN_VALU;
            c.MT = M;
            c.L = L;
            c.V = pref[i][0];
            c.U = pref[i][1];
            c.moe = moe;
            if (C % c.V != 0 || !plan_instantiated(c))
                continue;
            if (finish_plan(M, N, K, topk, cus, lds_limit, 8, &c)) {
                *p = c;
                return true;
            }
        }
        if (moe)
            return false;
    }
    if (moe)
        return false;
    // MFMA: two 16-row tiles per wave; split K across waves when rows alone leave CUs idle.
    static const int mf[][2] = {{2, 1}, {2, 2}, {1, 2}, {1, 4}, {1, 1}};
    for (int i = 0; i < (int)(sizeof(mf) / sizeof(mf[0])); ++i) {
        Plan c{};
        c.kind = PLAN_MFMA;
        c.T = mf[i][0];
        c.KS = mf[i][1];
        if (gpr % c.KS != 0)
            continue;
        const int64_t rows_per_block = 16LL * c.T * (4 / c.KS);
        const int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
        const bool last = i == (int)(sizeof(mf) / sizeof(mf[0])) - 1;
        if (blocks < 2LL * cus && !last)
            continue;
        if (finish_plan(M, N, K, topk, cus, lds_limit, 1, &c)) {
            *p = c;
            return true;
        }
    }
    return false;
}

int describe_plan(const Plan &p, char *buf, size_t len)
{
    if (!buf || len == 0)
        return 0;
    int n = 0;
    if (p.kind == PLAN_VALU)
        n = snprintf(buf, len,
                     "valu%s tokens=%d lanes_per_row=%d chunks_per_item=%d row_steps=%d "
                     "threads=%d blocks=%lld lds=%lld",
                     p.moe ? "_moe" : "", p.MT, p.L, p.V, p.U, p.threads, (long long)p.blocks,
                     (long long)p.lds_bytes);
    else if (p.kind == PLAN_MFMA)
        n = snprintf(buf, len, "mfma16x16x32 tiles_per_wave=%d k_split=%d threads=%d blocks=%lld",
                     p.T, p.KS, p.threads, (long long)p.blocks);
    else
        n = snprintf(buf, len, "none");
    return n;
}

}  // namespace w4a16
