"""GPU parity with outlier activations, through every kernel form (C ABI against the oracle).

Decode activations are not all of one size: a few channels can be thousands of times larger than
the rest. Here each token carries one activation of magnitude 2^14 and one of 2^10, placed at
positions where every row's code is 0, and the other activations are drawn from N(0, 1e-3). The
products that survive are then all small, so a kernel whose rounding error scales with the size of
the activations rather than with the size of the products q*s*x breaks the per-element tolerance
1e-3 * sum|q s x| + 1e-5 by orders of magnitude. Each case names the dispatch form it exercises,
and the test asserts that the shape really reaches that form.

Three more properties of the staging (activations scaled per 128-value group by a power of two and
held as fp16):
  * values that land in fp16's subnormal range but are still exact there (8 significant bits at a
    step of 2^-24) must not be flushed by the dot-product or matrix-core instructions;
  * a group whose values span more than 2^32 stays within tolerance when the large value meets a
    nonzero code (the rounded tiny values are then far below the allowance);
  * an infinite activation gives +-inf or NaN exactly where the plain definition does.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import weight_only_int4_w4a16_amd as w
from devhelp import bf16, f16, host, i32, words
from oracle_pins import pack_nibbles

pytestmark = pytest.mark.gpu


def within(got, ref, mag, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > oracle.bound(mag)
    ratio = float((err / np.maximum(mag, 1e-30)).max())
    print(f"{what}: n={err.size} max|err|={err.max():.3e} max|err|/sum|wx|={ratio:.2e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance"
    # the rounding error of an exact-product fp32 sum is far below the allowance
    assert ratio < 1e-5, f"{what}: error ratio {ratio:.2e} is a bug signal"


def bf16_bits(v):
    return synthetic.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def outlier_case(N, K, M, seed, E=1):
    """Codes (E, N, K) with zero columns at every outlier position, packed words, fp16 scales in
    [0.001, 0.01], and X bf16 bits [M][K]: N(0, 1e-3) plus +-2^14 and +-2^10 per token."""
    rng = np.random.default_rng([9100, N, K, M, seed])
    X = rng.standard_normal((M, K)).astype(np.float32) * np.float32(1e-3)
    cols = []
    for m in range(M):
        j1, j2 = rng.choice(K, size=2, replace=False)
        X[m, j1] = rng.choice([-1.0, 1.0]) * 2.0 ** 14
        X[m, j2] = rng.choice([-1.0, 1.0]) * 2.0 ** 10
        cols += [j1, j2]
    q = rng.integers(-8, 8, size=(E, N, K))
    q[:, :, cols] = 0
    qw = np.stack([pack_nibbles(q[e]) for e in range(E)])
    s = rng.uniform(0.001, 0.01, size=(E, N, K // 128)).astype(np.float16).view(np.uint16)
    return q, qw, s, bf16_bits(X)


DENSE_FORMS = [
    # (M, N, K, plan prefix)
    (1, 512, 128, "valu tokens=1 lanes_per_row=4"),
    (1, 512, 2304, "valu tokens=1 lanes_per_row=8 chunks_per_item=1 row_steps=2"),
    (1, 512, 4096, "splitk tokens=1"),
    (1, 300, 14336, "splitk tokens=1 lanes_per_row=64"),
    (2, 512, 128, "valu tokens=2"),
    (2, 512, 4096, "splitk tokens=2"),
    (2, 512, 2304, "mfma4x4x4_splitk token_groups=1"),
    (8, 512, 2304, "mfma4x4x4_splitk token_groups=2"),
    (8, 4096, 4096, "mfma4x4x4_splitk token_groups=2"),
    (16, 512, 128, "mfma16x16x32_lds "),
    (16, 512, 2304, "mfma16x16x32_lds_lines"),
    (16, 2048, 4096, "mfma16x16x32_rows tiles_per_wave=1 k_split=8"),
    (16, 14336, 2048, "mfma16x16x32_lines tiles_per_wave=4"),
    (16, 512, 4992, "mfma16x16x32 "),
    (5, 26624, 2304, "mfma16x16x32_lds8_lines"),
    (2, 26624, 2304, "mfma4x4x4_splitk token_groups=1 chunks_per_lane=3"),
    (16, 8192, 8192, "mfma16x16x32_rows tiles_per_wave=2 k_split=4"),
    (8, 8192, 8192, "mfma16x16x32_rows8 tiles_per_wave=2 k_split=4"),
]


@pytest.mark.parametrize("M,N,K,form", DENSE_FORMS)
def test_outlier_activations_dense(M, N, K, form):
    plan = w.describe_plan(M, N, K)
    assert plan.startswith(form), plan
    q, qw, s, X = outlier_case(N, K, M, 0)
    tq, ts = words(qw[0]), f16(s[0])
    rows = None if N <= 4096 else np.random.default_rng(N).choice(N, 1024, replace=False)
    if M == 1:
        got = host(w.gemv(tq, ts, bf16(X[0])))[None, :]
    else:
        got = host(w.gemv_batched(tq, ts, bf16(X)))
    for m in range(M):
        ref, mag = oracle.gemv(qw[0], s[0], X[m], K, rows=rows)
        g = got[m] if rows is None else got[m][rows]
        within(g, ref, mag, f"{form} M={M} {N}x{K} token {m}")


def test_outlier_activations_grouped_experts():
    E, N, K, topk = 6, 256, 2304, 4
    q, qw, s, X = outlier_case(N, K, 1, 1, E=E)
    ids = np.array([5, 0, 3, 5], np.int32)
    y = host(w.moe_gemv(words(qw), f16(s), i32(ids), bf16(X[0])))
    ref, mag = oracle.moe_gemv(qw, s, ids, X[0], K)
    within(y, ref, mag, "grouped experts")


@pytest.mark.parametrize("M", [2, 4, 16])
def test_outlier_activations_grouped_experts_batched(M):
    E, N, K, topk = 8, 256, 2304, 4
    q, qw, s, X = outlier_case(N, K, M, 2, E=E)
    rng = np.random.default_rng(77 + M)
    ids = np.stack([rng.choice(E, topk, replace=False) for _ in range(M)]).astype(np.int32)
    Y = host(w.moe_gemv_batched(words(qw), f16(s), i32(ids), bf16(X)))
    ref, mag = oracle.moe_gemv_batched(qw, s, ids, X, K)
    within(Y.reshape(-1), ref.reshape(-1), mag.reshape(-1), f"batched grouped experts M={M}")


def test_outlier_activations_expert_tail():
    """SwiGLU gate+up with an outlier x, then the down projection with outlier h rows."""
    from test_gpu_tail import check_h, check_out
    E, I, H, K, topk = 6, 256, 384, 2304, 4
    _, qg, sg, X = outlier_case(2 * I, K, 1, 3, E=E)
    ids = np.array([1, 4, 2, 0], np.int32)
    h = w.moe_gemv_swiglu(words(qg), f16(sg), i32(ids), bf16(X[0]))
    check_h(h, oracle.moe_swiglu(qg, sg, ids, X[0], K), "swiglu with outlier x")
    # down projection: each slot's own h row carries outliers at zero-code positions
    rng = np.random.default_rng(91)
    hrows = rng.standard_normal((topk, I)).astype(np.float32) * np.float32(1e-3)
    qd = rng.integers(-8, 8, size=(E, H, I))
    for t in range(topk):
        j = rng.choice(I, 2, replace=False)
        hrows[t, j] = [2.0 ** 14, -(2.0 ** 10)]
        qd[:, :, j] = 0
    hb = bf16_bits(hrows)
    wd = np.stack([pack_nibbles(qd[e]) for e in range(E)])
    sd = rng.uniform(0.001, 0.01, size=(E, H, I // 128)).astype(np.float16).view(np.uint16)
    rw = np.array([0.4, 0.3, 0.2, 0.1], np.float32)
    out = w.moe_down_combine(words(wd), f16(sd), i32(ids), torch.from_numpy(rw).cuda(), bf16(hb))
    ref, mag = oracle.moe_down_combine(wd, sd, ids, rw, hb)
    check_out(out, ref, mag, "down projection + combine with outlier h")
    err = np.abs(host(out).astype(np.float64) - ref)
    assert float((err / np.maximum(mag, 1e-30)).max()) < 1e-5


SUBNORMAL_FORMS = [
    (1, 512, 2304, "valu"),
    (1, 512, 4096, "splitk"),
    (4, 512, 2304, "mfma4x4x4_splitk"),
    (16, 512, 2304, "mfma16x16x32_lds_lines"),
    (16, 2048, 4096, "mfma16x16x32_rows tiles_per_wave=1 k_split=8"),
    (16, 14336, 2048, "mfma16x16x32_lines tiles_per_wave=4"),
]


@pytest.mark.parametrize("M,N,K,form", SUBNORMAL_FORMS)
def test_fp16_subnormal_activations_are_kept(M, N, K, form):
    """In every group one value of 2^14 sits on a zero code and the others lie in
    [2^-18, 2^-15): scaled by 2 they are fp16 subnormals, still exact. With unit scales the
    result is made of those tiny products only; flushing them would leave zero."""
    assert w.describe_plan(M, N, K).startswith(form)
    rng = np.random.default_rng([9200, M, K])
    mant = rng.uniform(1.0, 2.0, size=(M, K)) * rng.choice([-1.0, 1.0], size=(M, K))
    X = (mant * 2.0 ** rng.integers(-18, -15, size=(M, K))).astype(np.float32)
    big = np.arange(0, K, 128) + 5
    X[:, big] = 2.0 ** 14
    q = rng.integers(-8, 8, size=(N, K))
    q[:, big] = 0
    qw = pack_nibbles(q)
    s = np.full((N, K // 128), 0x3C00, np.uint16)              # fp16 1.0
    Xb = bf16_bits(X)
    if M == 1:
        got = host(w.gemv(words(qw), f16(s), bf16(Xb[0])))[None, :]
    else:
        got = host(w.gemv_batched(words(qw), f16(s), bf16(Xb)))
    for m in range(M):
        ref, mag = oracle.gemv(qw, s, Xb[m], K)
        assert np.all(mag > 1e-2)   # the tiny products carry weight
        within(got[m], ref, mag, f"fp16-subnormal staging {form} token {m}")


@pytest.mark.parametrize("M,N,K", [(1, 512, 2304), (1, 512, 4096), (4, 512, 2304), (16, 512, 2304)])
def test_wide_group_with_outlier_on_nonzero_code(M, N, K):
    """Groups spanning 2^14 down to 2^-24: the values below the fp16 grid are rounded at
    staging, which stays far inside the tolerance when the large value meets nonzero codes."""
    rng = np.random.default_rng([9300, M, K])
    X = (rng.standard_normal((M, K)) * 2.0 ** -22).astype(np.float32)
    X[:, np.arange(0, K, 128) + 17] = 2.0 ** 14
    q = rng.integers(1, 8, size=(N, K)) * rng.choice([-1, 1], size=(N, K))
    qw = pack_nibbles(q)
    s = rng.uniform(0.001, 0.01, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    Xb = bf16_bits(X)
    got = host(w.gemv(words(qw), f16(s), bf16(Xb[0])))[None, :] if M == 1 else \
        host(w.gemv_batched(words(qw), f16(s), bf16(Xb)))
    for m in range(M):
        ref, mag = oracle.gemv(qw, s, Xb[m], K)
        within(got[m], ref, mag, f"wide group M={M} token {m}")


@pytest.mark.parametrize("M,N,K", [(1, 512, 2304), (1, 512, 4096), (4, 512, 2304), (16, 512, 2304),
                                   (16, 2048, 4096)])
def test_infinite_activation_matches_plain_definition(M, N, K):
    """One +inf activation per token: rows whose code there is nonzero give +-inf with the sign
    of q*s (or NaN where another infinity of the other sign meets it), rows with a zero code
    give NaN (0 * inf), exactly as the oracle's sum does."""
    rng = np.random.default_rng([9400, M, K])
    X = rng.standard_normal((M, K)).astype(np.float32)
    j = rng.integers(0, K, size=M)
    X[np.arange(M), j] = np.inf
    q = rng.integers(-8, 8, size=(N, K))
    qw = pack_nibbles(q)
    s = rng.uniform(0.001, 0.01, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    Xb = bf16_bits(X)
    got = host(w.gemv(words(qw), f16(s), bf16(Xb[0])))[None, :] if M == 1 else \
        host(w.gemv_batched(words(qw), f16(s), bf16(Xb)))
    for m in range(M):
        ref, _ = oracle.gemv(qw, s, Xb[m], K)
        assert np.array_equal(np.isnan(got[m]), np.isnan(ref)), m
        fin = ~np.isnan(ref)
        assert np.array_equal(got[m][fin].astype(np.float64), ref[fin]), m   # +-inf, signs equal
        assert np.all(np.isinf(ref[fin]))
