"""GPU parity of the three-bit grouped-expert GEMV (w4a16_moe_gemv3) and its decode
(w4a16_unpack3_debug) against the CPU oracle.

The codes are decoded exactly (integers in [-4, 3]) and the activations are staged exactly for
every value within 2^32 of its 128-group's largest, so the kernel's result differs from the exact
sum only by the order of its fp32 additions: the per-element allowance 1e-3 * sum|q s x| + 1e-5
is loose, and the observed error relative to sum|q s x| must stay near fp32 rounding (< 1e-5).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import weight_only_int4_w4a16_amd as w
from devhelp import bf16, f16, host, i32, words
from oracle_pins import pack3

pytestmark = pytest.mark.gpu


def within(got, ref, mag, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > oracle.bound(mag)
    ratio = float((err / np.maximum(mag, 1e-30)).max()) if err.size else 0.0
    print(f"{what}: n={err.size} max|err|/sum|wx|={ratio:.2e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance"
    assert ratio < 1e-5, f"{what}: error ratio {ratio:.2e} is a bug signal"


def dev3(d):
    return words(d.qweight), f16(d.scales), i32(d.ids), bf16(d.x)


@pytest.mark.parametrize("N,K", [(1, 32), (37, 2304), (5, 65536), (300, 96)])
def test_unpack3_is_bit_exact(N, K):
    rng = np.random.default_rng([9300, N, K])
    qw = rng.integers(0, 1 << 32, size=(N, 3 * K // 32), dtype=np.uint32)
    print(f"unpack3 N={N} K={K}", flush=True)
    got = host(w.unpack3_debug(words(qw)))
    assert np.array_equal(got, oracle.unpack3(qw, K))


def test_unpack3_special_words():
    """All-zero, all-one and single-code blocks decode to the codes packed into them."""
    K = 64
    q = np.zeros((4, K), np.int64)
    q[1] = -1
    q[2, ::2] = -4
    q[2, 1::2] = 3
    q[3, 30], q[3, 31], q[3, 62], q[3, 63] = -4, 3, 2, -3
    got = host(w.unpack3_debug(words(pack3(q))))
    assert np.array_equal(got.astype(np.int64), q)


# (E, N, K, topk, plan prefix): every kernel variant, staging loops past one and two passes of
# 256 threads (K = 24576 and 65536), more slots than threads (topk = 300), N below and not a
# multiple of the rows of one wave step.
SHAPES = [
    (6, 64, 384, 3, "moe3 lanes_per_row=4 blocks_per_item=3"),
    (4, 3, 128, 2, "moe3 lanes_per_row=4 blocks_per_item=1"),
    (5, 37, 2304, 4, "moe3 lanes_per_row=8 blocks_per_item=3"),
    (3, 100, 2048, 2, "moe3 lanes_per_row=8 blocks_per_item=1"),
    (2, 1000, 4096, 1, "moe3 lanes_per_row=8 blocks_per_item=1"),
    (9, 256, 2304, 8, "moe3 lanes_per_row=8 blocks_per_item=3"),
    (3, 40, 24576, 2, "moe3 lanes_per_row=8 blocks_per_item=3"),
    (2, 5, 65536, 2, "moe3 lanes_per_row=8 blocks_per_item=1"),
    (300, 8, 256, 300, "moe3 lanes_per_row=8 blocks_per_item=1"),
]


@pytest.mark.parametrize("E,N,K,topk,form", SHAPES)
@pytest.mark.parametrize("seed", [0, 1])
def test_moe3_matches_oracle(E, N, K, topk, form, seed):
    plan = w.describe_moe3_plan(N, K, topk)
    print(f"moe3 E={E} N={N} K={K} topk={topk} seed={seed} plan={plan}", flush=True)
    assert plan.startswith(form), plan
    d = synthetic.moe3(E, N, K, topk, seed, config_id=930)
    qw, sc, ids, x = dev3(d)
    y = w.moe_gemv3(qw, sc, ids, x)
    ref, mag = oracle.moe_gemv3(d.qweight, d.scales, d.ids, d.x, K)
    within(host(y), ref, mag, f"moe3 {E}x{N}x{K} top{topk}")


@pytest.mark.parametrize("seed", [0, 1])
def test_moe3_full_size_every_row(seed):
    """256 experts of 2048 x 2304 (the grouped gate+up shape), top-8, every output."""
    cid, N, K = synthetic.SHAPES["c4"]
    d = synthetic.moe3(synthetic.MOE_EXPERTS, N, K, synthetic.MOE_TOPK, seed, config_id=cid)
    print(f"moe3 full size seed={seed} plan={w.describe_moe3_plan(N, K, 8)}", flush=True)
    qw, sc, ids, x = dev3(d)
    y = w.moe_gemv3(qw, sc, ids, x)
    ref, mag = oracle.moe_gemv3(d.qweight, d.scales, d.ids, d.x, K)
    within(host(y), ref, mag, "moe3 256x2048x2304 top8")


def test_moe3_invalid_and_repeated_ids():
    d = synthetic.moe3(5, 80, 2304, 4, 3, config_id=931)
    ids = np.array([4, -1, 4, 5], np.int32)
    qw, sc, _, x = dev3(d)
    out = torch.full((4, 80), float("nan"), device="cuda")
    y = host(w.moe_gemv3(qw, sc, i32(ids), x, out=out))
    ref, mag = oracle.moe_gemv3(d.qweight, d.scales, ids, d.x, 2304)
    within(y, ref, mag, "moe3 invalid/repeated ids")
    assert np.all(y[1] == 0) and np.all(y[3] == 0)
    assert np.array_equal(y[0], y[2])


def test_moe3_reads_only_selected_experts():
    """Every expert that no id selects holds NaN scales; the outputs stay finite and match."""
    E, N, K = 12, 130, 2304
    d = synthetic.moe3(E, N, K, 3, 5, config_id=932)
    sc = d.scales.copy()
    for e in range(E):
        if e not in d.ids:
            sc[e] = 0x7E00
    qw, _, ids, x = dev3(d)
    y = host(w.moe_gemv3(qw, f16(sc), ids, x))
    ref, mag = oracle.moe_gemv3(d.qweight, d.scales, d.ids, d.x, K)
    within(y, ref, mag, "moe3 unselected experts poisoned")


def test_moe3_outlier_activations():
    """One activation of 2^14 and one of 2^10 on positions where every code is 0, the rest
    N(0, 1e-3): an error that scaled with |x| instead of |q s x| would break the allowance."""
    E, N, K, topk = 4, 200, 2304, 3
    rng = np.random.default_rng([9301, N, K])
    x = rng.standard_normal(K).astype(np.float32) * np.float32(1e-3)
    j1, j2 = rng.choice(K, size=2, replace=False)
    x[j1], x[j2] = -2.0 ** 14, 2.0 ** 10
    q = rng.integers(-4, 4, size=(E, N, K))
    q[:, :, [j1, j2]] = 0
    qw = np.stack([pack3(q[e]) for e in range(E)])
    sc = rng.uniform(0.001, 0.01, size=(E, N, K // 128)).astype(np.float16).view(np.uint16)
    xb = synthetic.f32_to_bf16_bits(x)
    ids = np.array([2, 0, 3], np.int32)
    y = host(w.moe_gemv3(words(qw), f16(sc), i32(ids), bf16(xb)))
    ref, mag = oracle.moe_gemv3(qw, sc, ids, xb, K)
    within(y, ref, mag, "moe3 outliers")


def test_moe3_infinite_activation():
    """An infinite activation gives +-inf where its code is nonzero and NaN where it is 0
    (0 * inf), as the plain definition does."""
    E, N, K = 2, 64, 256
    rng = np.random.default_rng([9302, N, K])
    q = rng.integers(-4, 4, size=(E, N, K))
    q[:, :8, 5] = 0
    qw = np.stack([pack3(q[e]) for e in range(E)])
    sc = rng.uniform(0.001, 0.01, size=(E, N, K // 128)).astype(np.float16).view(np.uint16)
    x = synthetic.f32_to_bf16_bits(rng.standard_normal(K).astype(np.float32))
    x[5] = 0x7F80
    ids = np.array([1, 0], np.int32)
    y = host(w.moe_gemv3(words(qw), f16(sc), i32(ids), bf16(x)))
    ref, _ = oracle.moe_gemv3(qw, sc, ids, x, K)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(y[fin], ref[fin])
    assert np.isnan(y[:, :8]).all() and np.isinf(y[:, 8:][~np.isnan(y[:, 8:])]).all()
