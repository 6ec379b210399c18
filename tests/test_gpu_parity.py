"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Tolerance (per element): |y_gpu - y_oracle| <= 1e-3 * sum_k |q s x| + 1e-5. Unpacking, unit-vector
probes, zero-scale groups, power-of-two scaling and negation are required to be bit-exact.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import par_oracle
import synthetic
import weight_only_int4_w4a16_amd as w
from devhelp import bf16, f16, host, i32, words
from oracle_pins import pack_nibbles

pytestmark = pytest.mark.gpu

SEEDS = (0, 1, 2)


def within(got, ref, mag, what=""):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > oracle.bound(mag)
    ratio = float((err / np.maximum(mag, 1e-30)).max()) if err.size else 0.0
    print(f"{what}: n={err.size} max|err|={err.max() if err.size else 0:.3e} "
          f"max|err|/sum|wx|={ratio:.2e}", flush=True)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside tolerance"
    assert np.all(np.isfinite(got))
    return ratio


@functools.lru_cache(maxsize=4)
def cfg(name, seed, M=1):
    return synthetic.config(name, seed, M=M)


# ------------------------------------------------------------------ unpack
def test_unpack_bit_exact_random():
    d = synthetic.dense(N=300, K=1024, seed=0, config_id=700)
    got = host(w.unpack_debug(words(d.qweight)))
    assert np.array_equal(got, oracle.unpack(d.qweight, d.K))


def test_unpack_every_code_every_position():
    q = np.array([[(c + i) % 16 - 8 for i in range(128)] for c in range(16)])
    got = host(w.unpack_debug(words(pack_nibbles(q))))
    assert np.array_equal(got.astype(np.int64), q)


# ------------------------------------------------------------------ exact cases
def _probe_case(N, K, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-8, 8, size=(N, K))
    s = rng.uniform(0.001, 0.01, size=(N, K // 128)).astype(np.float16)
    return q, pack_nibbles(q), s


@pytest.mark.parametrize("N,K", [(64, 2048), (37, 2304), (16, 14336)])
def test_unit_vector_probes_bitwise(N, K):
    """x = e_j returns q[:, j] * s[:, j/128] exactly (one nonzero term, exact in fp32)."""
    q, qw, s = _probe_case(N, K, 3)
    tq, ts = words(qw), f16(s.view(np.uint16))
    js = sorted(set([0, 1, 7, 8, 31, 32, 127, 128, K // 2 + 5, K - 1]))
    for j in js:
        x = np.zeros(K, np.uint16)
        x[j] = 0x3F80
        y = host(w.gemv(tq, ts, bf16(x)))
        expect = (q[:, j] * s[:, j // 128].astype(np.float64)).astype(np.float32)
        assert np.array_equal(y, expect), j


def test_batched_identity_rows_return_columns_bitwise():
    """Batched (MFMA path) with X rows = unit vectors returns columns of W exactly."""
    N, K, M = 48, 2304, 16
    q, qw, s = _probe_case(N, K, 4)
    js = np.array([0, 3, 9, 100, 127, 128, 500, 1000, 1151, 1152, 1500, 2000, 2200, 2290, 2300, 2303])
    X = np.zeros((M, K), np.uint16)
    X[np.arange(M), js] = 0x3F80
    Y = host(w.gemv_batched(words(qw), f16(s.view(np.uint16)), bf16(X)))
    expect = (q[:, js] * s[:, js // 128].astype(np.float64)).T.astype(np.float32)
    assert np.array_equal(Y, expect)


@pytest.mark.parametrize("M", [5, 6, 8])
def test_batched_identity_rows_staged_8_slot_form_bitwise(M):
    """The 8-token-slot staged MFMA form on a tall matrix: X rows = unit vectors return columns
    of W exactly, so every token lands in its own output row."""
    N, K = 26624, 2304
    assert w.describe_plan(M, N, K).startswith("mfma16x16x32_lds8_lines")
    rng = np.random.default_rng(40 + M)
    qw = rng.integers(0, 1 << 32, size=(N, K // 8), dtype=np.uint32)
    s = rng.uniform(0.001, 0.01, size=(N, K // 128)).astype(np.float16)
    js = np.array([0, 9, 127, 128, 1151, 1500, 2200, 2303])[:M]
    # value k of a row: nibble k % 8 of word k // 8, two's complement
    nib = (qw[:, js // 8] >> (4 * (js % 8)).astype(np.uint32)) & 0xF
    q = nib.astype(np.int64) - 16 * (nib >= 8)
    X = np.zeros((M, K), np.uint16)
    X[np.arange(M), js] = 0x3F80
    Y = host(w.gemv_batched(words(qw), f16(s.view(np.uint16)), bf16(X)))
    expect = (q * s[:, js // 128].astype(np.float64)).T.astype(np.float32)
    assert np.array_equal(Y, expect)


def test_zero_scales_give_exact_zero():
    d = synthetic.dense(N=100, K=2048, seed=5, config_id=701)
    y = host(w.gemv(words(d.qweight), f16(np.zeros_like(d.scales)), bf16(d.x[0])))
    assert np.all(y == 0)
    s = d.scales.copy()
    s[:, ::2] = 0
    x = d.x[0].copy()
    x.reshape(-1, 128)[1::2] = 0      # with the odd groups' x removed, y must be exactly zero
    y = host(w.gemv(words(d.qweight), f16(s), bf16(x)))
    assert np.all(y == 0)


def test_negation_and_power_of_two_scaling_bitwise():
    d = synthetic.dense(N=333, K=4096, seed=6, config_id=702)
    tq, ts = words(d.qweight), f16(d.scales)
    y = host(w.gemv(tq, ts, bf16(d.x[0])))
    yn = host(w.gemv(tq, ts, bf16(d.x[0] ^ np.uint16(0x8000))))
    assert np.array_equal(yn, -y)
    x4 = (d.x[0].astype(np.int32) + (2 << 7)).astype(np.uint16)   # x * 4 via the exponent
    y4 = host(w.gemv(tq, ts, bf16(x4)))
    assert np.array_equal(y4, y * 4)


def test_deterministic_across_calls_and_streams():
    d = synthetic.dense(N=4096, K=4096, seed=7, config_id=703)
    tq, ts, tx = words(d.qweight), f16(d.scales), bf16(d.x[0])
    y1 = host(w.gemv(tq, ts, tx))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2 = w.gemv(tq, ts, tx)
    s.synchronize()
    assert np.array_equal(y1, y2.cpu().numpy())


# ------------------------------------------------------------------ shapes that span tiles and tails
@pytest.mark.parametrize("N,K", [
    (1, 128), (3, 256), (17, 384), (64, 1152), (129, 2048), (1000, 2304), (257, 4096),
    (70, 8192), (33, 14336), (5, 65536), (2049, 1024), (4096, 2048), (9000, 2048),
    (300, 3072), (1000, 7168), (9000, 5120), (5000, 1536),
])
def test_gemv_small_shapes(N, K):
    d = synthetic.dense(N=N, K=K, seed=N + K, config_id=800)
    y = host(w.gemv(words(d.qweight), f16(d.scales), bf16(d.x[0])))
    ref, mag = oracle.gemv(d.qweight, d.scales, d.x[0], K)
    within(y, ref, mag, f"gemv {N}x{K}")


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_batched_every_m_ragged(M):
    N, K = 77, 2304
    d = synthetic.dense(N=N, K=K, seed=M, M=M, config_id=801)
    ldx, ldy = K + 64, N + 3
    Xp = np.zeros((M, ldx), np.uint16)
    Xp[:, :K] = d.x
    Xp[:, K:] = 0x7FC0                       # NaN padding beyond K must never be read
    out = torch.full((M, ldy), float("nan"), dtype=torch.float32, device="cuda")
    tX = bf16(Xp)
    w.gemv_batched(words(d.qweight), f16(d.scales), tX[:, :K], out=out[:, :N])
    Y = host(out)
    assert np.all(np.isnan(Y[:, N:])), "wrote past N"
    ref, mag = oracle.gemv_batched(d.qweight, d.scales, d.x, K)
    within(Y[:, :N], ref, mag, f"batched M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(16, 300, 4096), (9, 2049, 1024), (16, 129, 1536), (5, 7, 256),
                                   (12, 1000, 2304), (16, 4096, 2048), (6, 100, 384),
                                   (16, 2048, 4096), (8, 300, 14336), (4, 40000, 2304),
                                   (3, 40000, 1152), (16, 5, 65536), (16, 300, 2688),
                                   (11, 14336, 2048), (7, 8192, 8192), (12, 4096, 14336)])
def test_batched_mfma_plans(M, N, K):
    """Every MFMA form: whole-line loads with 2, 4 and 6 groups per item, rows below and above
    one row block, and the operand-order forms."""
    d = synthetic.dense(N=N, K=K, seed=M + N, M=M, config_id=803)
    print(f"batched M={M} {N}x{K} plan={w.describe_plan(M, N, K)}", flush=True)
    Y = host(w.gemv_batched(words(d.qweight), f16(d.scales), bf16(d.x)))
    ref, mag = oracle.gemv_batched(d.qweight, d.scales, d.x, K)
    within(Y, ref, mag, f"batched M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 300, 2304), (1, 300, 4096), (2, 300, 2304), (8, 512, 2304),
                                   (16, 512, 2304), (16, 2048, 4096), (16, 300, 4992),
                                   (16, 8192, 2048), (6, 26624, 2304), (12, 16384, 4096),
                                   (16, 16384, 2304)])
def test_scales_at_two_byte_offset(M, N, K):
    """Scales need only 2-byte alignment: every form reads them correctly from an address that
    is 2 mod 4 (a view starting one fp16 into its allocation)."""
    plan = w.describe_plan(M, N, K)
    d = synthetic.dense(N=N, K=K, seed=M + 3, M=M, config_id=807)
    sc = torch.empty(N * (K // 128) + 1, dtype=torch.float16, device="cuda")
    sc[1:] = f16(d.scales).reshape(-1)
    view = sc[1:].view(N, K // 128)
    assert view.data_ptr() % 4 == 2
    print(f"scales+2B M={M} {N}x{K} plan={plan}", flush=True)
    Y = host(w.gemv_batched(words(d.qweight), view, bf16(d.x)))
    ref, mag = par_oracle.gemv_batched(d.qweight, d.scales, d.x, K, np.arange(N))
    within(Y, ref, mag, f"scales+2B M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(3, 40, 131072), (2, 3, 1 << 20), (16, 5, 1 << 20)])
def test_batched_long_rows(M, N, K):
    """Batched calls accept K up to 2^20 (single-token calls up to 65536): rows of 2^17 and 2^20
    values, every output against the oracle."""
    plan = w.describe_plan(M, N, K)
    d = synthetic.dense(N=N, K=K, seed=M + N, M=M, config_id=806)
    print(f"batched M={M} {N}x{K} plan={plan}", flush=True)
    Y = host(w.gemv_batched(words(d.qweight), f16(d.scales), bf16(d.x)))
    ref, mag = oracle.gemv_batched(d.qweight, d.scales, d.x, K)
    within(Y, ref, mag, f"batched M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(2, 5000, 2304), (3, 333, 4096), (4, 20001, 4096), (4, 33, 14336),
                                   (3, 1000, 2048), (4, 999, 1024), (5, 77, 2304), (6, 4096, 14336),
                                   (8, 1500, 8192), (7, 3, 4096), (8, 8192, 512), (2, 17, 256),
                                   (3, 16384, 2304), (6, 1, 2304), (2, 26624, 2304), (4, 26700, 2304)])
def test_batched_mfma4_plans(M, N, K):
    """The 4x4x4-MFMA split-K kernel: 16 and 8 blocks per row group, one and two token groups
    (partial groups included), 1-4 chunks per lane, one and two row steps per item, fewer rows
    than one row step, ragged row blocks and the tall launch shapes."""
    plan = w.describe_plan(M, N, K)
    assert plan.startswith("mfma4x4x4_splitk"), plan
    d = synthetic.dense(N=N, K=K, seed=M * 7 + N, M=M, config_id=804)
    print(f"batched M={M} {N}x{K} plan={plan}", flush=True)
    Y = host(w.gemv_batched(words(d.qweight), f16(d.scales), bf16(d.x)))
    ref, mag = oracle.gemv_batched(d.qweight, d.scales, d.x, K)
    within(Y, ref, mag, f"batched M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K", [(5, 26624, 2304), (6, 26624, 2304), (5, 26700, 2304),
                                   (7, 26700, 2304), (8, 26880, 1536), (6, 30000, 256)])
def test_batched_staged_8_slot_plans(M, N, K):
    """The staged whole-line 16x16x32 form with 8 token slots (5-8 tokens, tall matrices): MFMA
    rows 8-15 read slots 0-7 again and are never stored; ragged row counts pull the last block
    back."""
    plan = w.describe_plan(M, N, K)
    assert plan.startswith("mfma16x16x32_lds8_lines"), plan
    d = synthetic.dense(N=N, K=K, seed=M * 11 + N, M=M, config_id=806)
    print(f"batched M={M} {N}x{K} plan={plan}", flush=True)
    Y = host(w.gemv_batched(words(d.qweight), f16(d.scales), bf16(d.x)))
    ref, mag = oracle.gemv_batched(d.qweight, d.scales, d.x, K)
    within(Y, ref, mag, f"batched M={M} {N}x{K}")


@pytest.mark.parametrize("M,N,K,form,pad", [
    (9, 8192, 1024, "mfma16x16x32_rows tiles_per_wave=2", 0),
    (13, 8200, 2048, "mfma16x16x32_rows tiles_per_wave=2", 0),
    (16, 8192, 3072, "mfma16x16x32_rows tiles_per_wave=2", 0),
    (11, 8192, 1024, "mfma16x16x32_rows tiles_per_wave=2", 64),
    (10, 300, 4096, "mfma16x16x32_rows tiles_per_wave=1 k_split=8", 0),
    (15, 33, 6144, "mfma16x16x32_rows tiles_per_wave=1 k_split=8", 8),
    (16, 4096, 2048, "mfma16x16x32_rows tiles_per_wave=1 k_split=8", 0),
    (5, 8192, 1024, "mfma16x16x32_rows8", 0),
    (6, 8192, 3072, "mfma16x16x32_rows8", 8),
    (7, 8160, 2048, "mfma16x16x32_rows8", 0),
    (8, 8190, 1024, "mfma16x16x32_rows8", 64),
    (5, 16384, 1024, "mfma16x16x32_rows8", 0),
    (16, 8192, 1024, "mfma16x16x32_rows tiles_per_wave=2", 1 << 21),
    (7, 8192, 1024, "mfma16x16x32_rows8", 1 << 21),
])
def test_batched_token_row_plans(M, N, K, form, pad):
    """The global-activation 16x16x32 forms that load whole token rows and exchange them into
    operand order through LDS: 16 and 8 token slots (slots past M repeat token M-1), one to
    three items per wave, ragged row blocks pulled back, and activation rows with a stride
    beyond K whose padding (NaN) must never be read, up to 4 MiB between rows."""
    plan = w.describe_plan(M, N, K)
    assert plan.startswith(form), plan
    d = synthetic.dense(N=N, K=K, seed=M * 13 + N, M=M, config_id=808)
    print(f"batched M={M} {N}x{K} pad={pad} plan={plan}", flush=True)
    Xp = np.full((M, K + pad), 0x7FC0, np.uint16)
    Xp[:, :K] = d.x
    Y = host(w.gemv_batched(words(d.qweight), f16(d.scales), bf16(Xp)[:, :K]))
    ref, mag = oracle.gemv_batched(d.qweight, d.scales, d.x, K)
    within(Y, ref, mag, f"batched M={M} {N}x{K} pad={pad}")


def test_batched_rows_match_single_token():
    N, K, M = 500, 8192, 16
    d = synthetic.dense(N=N, K=K, seed=9, M=M, config_id=802)
    tq, ts = words(d.qweight), f16(d.scales)
    Y = host(w.gemv_batched(tq, ts, bf16(d.x)))
    for m in (0, 7, 15):
        y = host(w.gemv(tq, ts, bf16(d.x[m])))
        ref, mag = oracle.gemv(d.qweight, d.scales, d.x[m], K)
        assert np.all(np.abs(Y[m].astype(np.float64) - y) <= 2 * oracle.bound(mag))


# ------------------------------------------------------------------ the five workloads, full size
@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("name", ["c1", "c2", "c3a", "c3b", "c5a", "c5b"])
def test_dense_workloads_m1_all_rows(name, seed):
    d = cfg(name, seed)
    y = host(w.gemv(words(d.qweight), f16(d.scales), bf16(d.x[0])))
    ref, mag = oracle.gemv(d.qweight, d.scales, d.x[0], d.K)
    ratio = within(y, ref, mag, f"{name} seed={seed} M=1")
    assert ratio < 1e-5, "fp32 summation error far above expectation"


@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("M", [2, 4, 8, 16])
@pytest.mark.parametrize("name", ["c5a", "c5b"])
def test_batched_workloads(name, M, seed):
    """Seed 0: every element of Y against the oracle; seeds 1 and 2: the first and last 64 rows
    and 1024 random rows."""
    d = cfg(name, seed, M)
    Y = host(w.gemv_batched(words(d.qweight), f16(d.scales), bf16(d.x)))
    if seed == 0:
        rows = np.arange(d.N)
    else:
        rng = np.random.default_rng(seed)
        rows = np.unique(np.concatenate([np.arange(64), d.N - 64 + np.arange(64),
                                         rng.integers(0, d.N, 1024)]))
    ref, mag = par_oracle.gemv_batched(d.qweight, d.scales, d.x, d.K, rows)
    ratio = within(Y[:, rows], ref, mag, f"{name} seed={seed} M={M} ({rows.size} rows)")
    assert ratio < 1e-5, "fp32 summation error far above expectation"


@functools.lru_cache(maxsize=1)
def moe_cfg(seed):
    return synthetic.config("c4", seed)


@pytest.mark.parametrize("seed", SEEDS)
def test_moe_workload(seed):
    m = moe_cfg(seed)
    y = host(w.moe_gemv(words(m.qweight), f16(m.scales), i32(m.ids), bf16(m.x)))
    ref, mag = oracle.moe_gemv(m.qweight, m.scales, m.ids, m.x, m.K)
    within(y, ref, mag, f"c4 seed={seed} ids={m.ids.tolist()}")


def test_moe_reads_only_selected_experts():
    """Every unselected expert's scales are NaN; any read of them would poison the output."""
    m = moe_cfg(0)
    sc = np.full_like(m.scales, 0x7E00)
    sc[m.ids] = m.scales[m.ids]
    qw = m.qweight.copy()
    y = host(w.moe_gemv(words(qw), f16(sc), i32(m.ids), bf16(m.x)))
    assert np.all(np.isfinite(y))
    ref, mag = oracle.moe_gemv(m.qweight, m.scales, m.ids, m.x, m.K)
    within(y, ref, mag, "c4 poisoned unselected experts")


@pytest.mark.parametrize("E,N,K,topk", [(320, 8, 256, 300), (6, 50, 8192, 3)])
def test_moe_many_slots_and_long_rows(E, N, K, topk):
    """More slots than the 256 threads that stage the expert ids, and activations longer than
    two staging passes (K = 8192), on the grouped-expert kernel."""
    m = synthetic.moe(E=E, N=N, K=K, topk=topk, seed=9, config_id=805)
    print(f"moe E={E} N={N} K={K} topk={topk} plan={w.describe_plan(1, N, K, topk)}", flush=True)
    y = host(w.moe_gemv(words(m.qweight), f16(m.scales), i32(m.ids), bf16(m.x)))
    ref, mag = oracle.moe_gemv(m.qweight, m.scales, m.ids, m.x, K)
    within(y, ref, mag, f"moe E={E} N={N} K={K} top{topk}")


def test_moe_invalid_and_repeated_ids():
    E, N, K = 5, 96, 2304
    m = synthetic.moe(E=E, N=N, K=K, topk=2, seed=3, config_id=803)
    ids = np.array([2, -1, 4, 5, 2, 1000, 0], np.int32)
    out = torch.full((ids.size, N), float("nan"), dtype=torch.float32, device="cuda")
    w.moe_gemv(words(m.qweight), f16(m.scales), i32(ids), bf16(m.x), out=out)
    y = host(out)
    ref, mag = oracle.moe_gemv(m.qweight, m.scales, ids, m.x, K)
    assert np.all(y[[1, 3, 5]] == 0) and not np.any(np.signbit(y[[1, 3, 5]]))
    within(y, ref, mag, "moe invalid/repeated ids")
    assert np.array_equal(y[0], y[4])


# ------------------------------------------------------------------ no per-call allocation
def test_no_device_allocation_per_call():
    d = synthetic.dense(N=4096, K=4096, seed=1, config_id=804)
    tq, ts, tx = words(d.qweight), f16(d.scales), bf16(d.x[0])
    out = torch.empty(d.N, dtype=torch.float32, device="cuda")
    w.gemv(tq, ts, tx, out=out)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(1000):
        w.gemv(tq, ts, tx, out=out)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0
