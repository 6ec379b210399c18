"""GPU parity of the grouped-expert GEMV for M tokens with their own experts
(w4a16_moe_gemv_batched) against the CPU oracle, element by element.

Tolerance as for every GEMV here: |err| <= 1e-3 * sum_k |q s x| + 1e-5 per element.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import par_oracle
import synthetic
import weight_only_int4_w4a16_amd as w
from devhelp import host

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def experts(E, N, K, seed):
    d = synthetic.moe(E, N, K, 1, seed, config_id=950)
    return d.qweight, d.scales


def operands(E, N, K, M, topk, seed, distinct=True):
    qweight, scales = experts(E, N, K, seed)
    rng = np.random.default_rng([951, seed, M])
    if distinct:
        ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(M)]).astype(np.int32)
    else:
        ids = rng.integers(0, E, size=(M, topk)).astype(np.int32)
    X = synthetic.draw_acts(rng, (M, K))
    return qweight, scales, ids, X


def run(qw, sc, ids, X, ldx=None):
    M, K = X.shape
    if ldx is not None and ldx > K:
        Xp = np.zeros((M, ldx), np.uint16)
        Xp[:, :K] = X
        Xt = torch.from_numpy(Xp.view(np.int16)).cuda().view(torch.bfloat16)[:, :K]
    else:
        Xt = torch.from_numpy(X.view(np.int16)).cuda().view(torch.bfloat16)
    Y = w.moe_gemv_batched(torch.from_numpy(qw.view(np.int32)).cuda(),
                           torch.from_numpy(sc.view(np.float16)).cuda(),
                           torch.from_numpy(ids).cuda(), Xt)
    return host(Y).astype(np.float64)


def check(got, ref, mag, what):
    err = np.abs(got - ref)
    ratio = float((err / np.maximum(mag, 1e-30)).max())
    print(f"{what}: n={err.size} max|err|/mag={ratio:.2e}", flush=True)
    assert np.all(err <= oracle.bound(mag)), f"{what}: {int((err > oracle.bound(mag)).sum())} bad"
    assert np.all(np.isfinite(got))


# (E, N, K, M, topk, distinct ids per token): the 2304-wide rows take 8 lanes x 3 chunks,
# others the widest lanes; N below one wave step; E small enough that many tokens share an
# expert (groups larger than the 4 tokens of one pass); M * topk = 256.
SHAPES = [(20, 64, 384, 3, 4, True), (6, 5, 128, 2, 3, True), (50, 300, 4096, 8, 8, True),
          (9, 100, 2304, 16, 16, False), (3, 77, 1024, 1, 2, True), (40, 33, 2304, 16, 8, True),
          (5, 128, 256, 8, 32, False), (7, 5, 2304, 5, 3, True), (12, 40, 1536, 6, 4, False)]


@pytest.mark.parametrize("E,N,K,M,topk,distinct", SHAPES)
@pytest.mark.parametrize("seed", [0, 1])
def test_moe_batched_matches_oracle(E, N, K, M, topk, distinct, seed):
    qw, sc, ids, X = operands(E, N, K, M, topk, seed, distinct)
    print(f"moe_batched E={E} N={N} K={K} M={M} topk={topk} seed={seed} "
          f"plan={w.describe_moe_batched_plan(M, N, K, topk)}", flush=True)
    got = run(qw, sc, ids, X, ldx=K + 8 if seed else None)
    ref, mag = oracle.moe_gemv_batched(qw, sc, ids, X, K)
    check(got, ref, mag, f"moe_batched {E}x{N}x{K} M{M} top{topk}")


def test_moe_batched_invalid_and_repeated_ids():
    qw, sc, _, X = operands(12, 200, 2304, 4, 6, 3)
    ids = np.array([[3, 3, -1, 11, 0, 7], [12, 3, 5, 5, 5, 5], [0, 1, 2, 3, 4, 5],
                    [-7, 99, 3, 3, 3, 3]], np.int32)
    got = run(qw, sc, ids, X)
    ref, mag = oracle.moe_gemv_batched(qw, sc, ids, X, 2304)
    check(got, ref, mag, "moe_batched invalid/repeated")
    assert np.all(got[0, 2] == 0) and np.all(got[1, 0] == 0) and np.all(got[3, :2] == 0)
    assert np.array_equal(got[0, 0], got[0, 1])


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_moe_batched_full_size(M):
    """256 experts of 2048 x 2304 (the fused gate+up experts), top-8 per token; every element
    of every (token, slot) output checked against the oracle."""
    qw, sc, ids, X = operands(256, 2048, 2304, M, 8, 4)
    print(f"moe_batched full M={M} unique experts={len(np.unique(ids))}", flush=True)
    got = run(qw, sc, ids, X)
    ref, mag = par_oracle.moe_gemv_batched(qw, sc, ids, X, 2304, np.arange(2048))
    check(got, ref, mag, f"moe_batched full M{M} (all rows)")


@pytest.mark.parametrize("E,N,K,M,form", [(256, 2048, 2304, 2, "moe_batched_mfma4x4x4"),
                                          (256, 2048, 2304, 16, "moe_batched_mfma4x4x4"),
                                          (40, 64, 384, 5, "moe_batched tokens_per_pass")])
def test_moe_batched_reads_only_selected_experts(E, N, K, M, form):
    """Every expert no token selected has NaN scales; any read of them would poison the
    output (the 4x4x4 grouped form and the VALU form)."""
    assert w.describe_moe_batched_plan(M, N, K, 8).startswith(form)
    qw, sc, ids, X = operands(E, N, K, M, 8, 6)
    poisoned = np.full_like(sc, 0x7E00)
    used = np.unique(ids)
    poisoned[used] = sc[used]
    got = run(qw, poisoned, ids, X)
    assert np.all(np.isfinite(got))
    ref, mag = par_oracle.moe_gemv_batched(qw, sc, ids, X, K, np.arange(N))
    check(got, ref, mag, f"moe_batched M{M} {form} poisoned unselected experts")


def test_moe_batched_deterministic_and_no_allocation():
    qw, sc, ids, X = operands(64, 512, 2304, 16, 8, 5)
    q = torch.from_numpy(qw.view(np.int32)).cuda()
    s = torch.from_numpy(sc.view(np.float16)).cuda()
    i = torch.from_numpy(ids).cuda()
    x = torch.from_numpy(X.view(np.int16)).cuda().view(torch.bfloat16)
    y1 = w.moe_gemv_batched(q, s, i, x)
    y2 = torch.empty_like(y1)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        w.moe_gemv_batched(q, s, i, x, out=y2)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(y1, y2)
