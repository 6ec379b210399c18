"""Pins that tie the CPU oracle to facts other than itself.

Each pin takes an `oracle.Oracle` and raises AssertionError when the oracle disagrees with
what the storage format and the mathematics fix. They are run against the shipped oracle
(test_oracle_pins.py) and against copies of it with a mistake planted in the C source
(test_oracle_mutants.py), where at least one pin must fail.

The operation pinned is the W4A16 GEMV of the local-kimi README
(github.1485827954.workers.dev/RightNow-AI/local-kimi), technical-detail section, GEMV-rewrite paragraph:
y = W x reduced along K, W stored as packed signed 4-bit values with one fp16 scale per
128-wide K group. The pages print no worked example, no test vector and no error bound,
so the expected values here are hand derivations (tests/golden), IEEE decodes from numpy,
closed forms and exact invariants.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- test-side helpers
def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Pack signed values q[N][K] in [-8, 7] into uint32 words, one nibble at a time.

    Written as the explicit loop over the 8 positions of a word so it reads against the
    format statement: value k = 8w + i goes to bits [4i, 4i+3] of word w, as the low 4 bits
    of its two's-complement byte.
    """
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    codes = (q & 0xF).astype(np.uint64)            # two's complement, low 4 bits
    words = np.zeros((N, K // 8), np.uint64)
    for i in range(8):
        words |= codes[:, i::8] << np.uint64(4 * i)
    return words.astype(np.uint32)


def f16_bits_pow2(e: int) -> int:
    """fp16 bit pattern of 2**e for a normal exponent (e in [-14, 15])."""
    assert -14 <= e <= 15
    return (e + 15) << 10


def bf16_scale_pow2(bits: np.ndarray, a: int) -> np.ndarray:
    """Multiply bf16 values by 2**a by moving the exponent field (normal values only)."""
    b = bits.astype(np.int64)
    expo = (b >> 7) & 0xFF
    normal = (expo > 0) & (expo < 255)
    assert np.all((expo[normal] + a > 0) & (expo[normal] + a < 255))
    out = np.where(normal, b + (a << 7), b)
    return out.astype(np.uint16)


def numpy_dense_weights(words: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """Independent float64 dequantisation with vectorised numpy (for the brute-force check)."""
    w = words.astype(np.uint64)[:, :, None] >> (np.arange(8, dtype=np.uint64) * 4)
    u = (w & 0xF).astype(np.int64).reshape(words.shape[0], K)
    q = np.where(u >= 8, u - 16, u)
    s = scales.view(np.float16).astype(np.float64)
    return q * np.repeat(s, 128, axis=1)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):     # signalling-NaN patterns convert to quiet NaN
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def random_case(N, K, seed, M=None):
    rng = np.random.default_rng(1000 + seed)
    q = rng.integers(-8, 8, size=(N, K))
    s = rng.uniform(0.001, 0.01, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    shape = (K,) if M is None else (M, K)
    xf = rng.standard_normal(shape).astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)       # truncation is fine for inputs
    return q, pack_nibbles(q), s, x


# ---------------------------------------------------------------- pins
def pin_f16_decode(orc):
    """The hand-written binary16 decoder equals numpy's conversion for all 65536 patterns."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_bf16_decode(orc):
    """The bf16 decoder equals the binary32 reading of the same bits, all 65536 patterns."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bf16_bits_to_f64(bits)
    got = np.array([orc.bf16_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_w1(orc):
    g = _golden("w1_sign_and_nibble_order.json")
    N, K = g["N"], g["K"]
    words = np.array([[int(w, 16)] * (K // 8) for w in g["row_word"]], np.uint32)
    scales = np.array([[int(s, 16)] for s in g["scale_bits"]], np.uint16)
    one = int(g["cases"][0]["x_bits"], 16)
    for case in g["cases"]:
        x = np.zeros(K, np.uint16)
        if case["x"] == "ones":
            x[:] = one
        else:
            x[int(case["x"].split("_")[1])] = one
        y, mag = orc.gemv(words, scales, x, K)
        assert np.array_equal(y, np.array(case["y"])), (case["x"], y)
        assert np.array_equal(mag, np.array(case["mag"])), (case["x"], mag)


def pin_w2(orc):
    g = _golden("w2_group_scale_index.json")
    K = g["K"]
    words = np.array([[int(g["group_word"][k // 16], 16) for k in range(K // 8)]], np.uint32)
    scales = np.array([[int(s, 16) for s in g["scale_bits"]]], np.uint16)
    x = np.full(K, int(g["x_bits"], 16), np.uint16)
    y, _ = orc.gemv(words, scales, x, K)
    assert y[0] == g["y"], y
    y2, _ = orc.gemv(words, scales[:, ::-1], x, K)
    assert y2[0] == g["y_if_scales_swapped"], y2


def pin_unpack(orc):
    """Unpack returns exactly the values the test packed, one nibble at a time."""
    rng = np.random.default_rng(7)
    q = rng.integers(-8, 8, size=(6, 256))
    got = orc.unpack(pack_nibbles(q), 256)
    assert np.array_equal(got.astype(np.int64), q)


def pin_unit_probes(orc):
    """x = e_j returns column j times its group scale, exactly, for every j.

    Scales are distinct powers of two per (row, group), so a scale taken from the wrong row
    or group, or a wrong nibble, shows as a different exact value.
    """
    N, K = 5, 384
    rng = np.random.default_rng(11)
    q = rng.integers(-8, 8, size=(N, K))
    exps = np.array([[-(2 + (3 * n + 5 * g) % 11) for g in range(K // 128)] for n in range(N)])
    scales = np.vectorize(f16_bits_pow2)(exps).astype(np.uint16)
    eye = np.zeros((K, K), np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    Y, mag = orc.gemv_batched(pack_nibbles(q), scales, eye, K)
    expect = (q * np.exp2(np.repeat(exps, 128, axis=1))).T     # [K][N]
    assert np.array_equal(Y, expect)
    assert np.array_equal(mag, np.abs(expect))


def pin_zero_scale_groups(orc):
    """A zero scale removes its group exactly: same y as zeroing x over that group."""
    N, K = 7, 512
    _, words, scales, x = random_case(N, K, 1)
    s0 = scales.copy()
    s0[:, 1] = 0x0000
    s0[:, 3] = 0x8000                                   # -0 as well
    x0 = x.copy()
    x0[128:256] = 0
    x0[384:512] = 0
    ya, _ = orc.gemv(words, s0, x, K)
    yb, _ = orc.gemv(words, scales, x0, K)
    assert np.array_equal(ya, yb)
    yz, mz = orc.gemv(words, np.zeros_like(scales), x, K)
    assert np.all(yz == 0) and np.all(mz == 0)


def pin_linearity(orc):
    """y(2^a x) = 2^a y(x) exactly; additivity over disjoint supports."""
    N, K = 9, 1024
    _, words, scales, x = random_case(N, K, 2)
    y, mag = orc.gemv(words, scales, x, K)
    for a in (3, -5):
        ya, _ = orc.gemv(words, scales, bf16_scale_pow2(x, a), K)
        assert np.array_equal(ya, y * 2.0 ** a)
    x1, x2 = x.copy(), x.copy()
    x1[1::2] = 0
    x2[0::2] = 0
    y1, _ = orc.gemv(words, scales, x1, K)
    y2, _ = orc.gemv(words, scales, x2, K)
    assert np.all(np.abs(y1 + y2 - y) <= 1e-12 * mag)
    assert not np.allclose(y1, y) and not np.allclose(y2, y)


def pin_negation(orc):
    N, K = 9, 640
    _, words, scales, x = random_case(N, K, 3)
    y, _ = orc.gemv(words, scales, x, K)
    yn, _ = orc.gemv(words, scales, x ^ np.uint16(0x8000), K)
    assert np.array_equal(yn, -y)


def pin_constant_rows(orc):
    """A row whose nibbles all equal q* gives q* * sum_g s_g * sum_{k in g} x_k."""
    K = 768
    rng = np.random.default_rng(5)
    qs = np.array([-8, -3, -1, 0, 1, 5, 7])
    words = np.array([[(int(v) & 0xF) * 0x11111111] * (K // 8) for v in qs], np.uint32)
    scales = rng.uniform(0.001, 0.01, size=(len(qs), K // 128)).astype(np.float16)
    xf = rng.standard_normal(K).astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)
    xv = bf16_bits_to_f64(x)
    gsum = xv.reshape(-1, 128).sum(axis=1)
    expect = qs * (scales.astype(np.float64) * gsum).sum(axis=1)
    y, mag = orc.gemv(words, scales.view(np.uint16), x, K)
    assert np.all(np.abs(y - expect) <= 1e-13 * np.maximum(mag, 1e-300))
    expect_mag = np.abs(qs) * (scales.astype(np.float64) * np.abs(xv).reshape(-1, 128).sum(1)).sum(1)
    assert np.all(np.abs(mag - expect_mag) <= 1e-13 * np.maximum(expect_mag, 1e-300))


def pin_brute_force(orc):
    """Agrees with an independent vectorised numpy dequantise + BLAS matrix-vector product."""
    N, K = 64, 2048
    _, words, scales, x = random_case(N, K, 4)
    W = numpy_dense_weights(words, scales, K)
    ref = W @ bf16_bits_to_f64(x)
    y, mag = orc.gemv(words, scales, x, K)
    assert np.all(np.abs(y - ref) <= 1e-12 * mag)
    assert np.all(np.abs(mag - np.abs(W * bf16_bits_to_f64(x)).sum(1)) <= 1e-12 * mag)


def pin_mag_nonnegative(orc):
    """With every term non-negative, mag equals y exactly."""
    N, K = 4, 256
    rng = np.random.default_rng(6)
    q = rng.integers(0, 8, size=(N, K))
    s = rng.uniform(0.001, 0.01, size=(N, K // 128)).astype(np.float16).view(np.uint16)
    x = (np.abs(rng.standard_normal(K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y, mag = orc.gemv(pack_nibbles(q), s, x, K)
    assert np.array_equal(y, mag)


def pin_batched(orc):
    """Batched row m equals the single-token product of X[m]; the row stride is honoured."""
    N, K, M, ld = 6, 512, 3, 640
    _, words, scales, X = random_case(N, K, 8, M=M)
    Xp = np.full((M, ld), 0x7FC0, np.uint16)            # NaN padding past K must be ignored
    Xp[:, :K] = X
    Y, mag = orc.gemv_batched(words, scales, Xp, K)
    for m in range(M):
        y, mg = orc.gemv(words, scales, X[m], K)
        assert np.array_equal(Y[m], y) and np.array_equal(mag[m], mg)


def pin_moe(orc):
    """Slot t equals the dense product with expert ids[t]; ids outside [0, E) give zeros."""
    E, N, K = 5, 4, 256
    rng = np.random.default_rng(9)
    q = rng.integers(-8, 8, size=(E, N, K))
    words = np.stack([pack_nibbles(q[e]) for e in range(E)])
    scales = rng.uniform(0.001, 0.01, size=(E, N, K // 128)).astype(np.float16).view(np.uint16)
    x = (rng.standard_normal(K).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ids = np.array([3, 0, -1, 4, 3, 1], np.int32)
    y, mag = orc.moe_gemv(words, scales, ids, x, K)
    for t, e in enumerate(ids):
        if 0 <= e < E:
            ref, rm = orc.gemv(words[e], scales[e], x, K)
            assert np.array_equal(y[t], ref) and np.array_equal(mag[t], rm)
        else:
            assert np.all(y[t] == 0) and np.all(mag[t] == 0)
    assert not np.array_equal(y[0], y[1])


def pin_row_subset(orc):
    N, K = 11, 384
    _, words, scales, x = random_case(N, K, 10)
    y, mag = orc.gemv(words, scales, x, K)
    rows = [10, 0, 5, 5]
    ys, ms = orc.gemv(words, scales, x, K, rows=rows)
    assert np.array_equal(ys, y[rows]) and np.array_equal(ms, mag[rows])


# ---------------------------------------------------------------- expert tail
def _bf16_value(bits: int) -> float:
    """Exact value of a bfloat16 pattern through numpy's binary32 reading (independent)."""
    return float(np.array([bits << 16], np.uint32).view(np.float32)[0])


def brute_bf16_round(v: float) -> int:
    """Nearest bfloat16 pattern to v, ties to the even pattern, by exact rational comparison of
    the two neighbouring patterns found by bisection over the ordered positive patterns."""
    from fractions import Fraction
    if v != v:
        raise ValueError("nan")
    sign = 0x8000 if np.signbit(v) else 0
    a = abs(v)
    if a == 0:
        return sign
    if a == float("inf"):
        return sign | 0x7F80
    lo, hi = 0, 0x7F80                     # decode(lo) <= a < decode(hi), hi = +inf
    if a >= _bf16_value(0x7F7F):
        lo, hi = 0x7F7F, 0x7F80
    else:
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if _bf16_value(mid) <= a:
                lo = mid
            else:
                hi = mid
    fa, flo = Fraction(a), Fraction(_bf16_value(lo))
    if hi == 0x7F80:   # above the largest finite value: the next step up would be 2^128
        fhi = Fraction(2) ** 128
    else:
        fhi = Fraction(_bf16_value(hi))
    d_lo, d_hi = fa - flo, fhi - fa
    if d_lo < d_hi or (d_lo == d_hi and lo % 2 == 0):
        return sign | lo
    return sign | hi


def pin_bf16_round_brute(orc):
    """double -> bfloat16 rounding equals the exact nearest-even choice on random magnitudes
    (subnormal to overflow), on exact midpoints, and on signed zeros and infinities."""
    rng = np.random.default_rng(31)
    vals = list(np.exp2(rng.uniform(-140, 129, size=600)) * rng.choice([-1.0, 1.0], 600))
    for b in rng.integers(0, 0x7F7F, size=300):
        mid = (_bf16_value(int(b)) + _bf16_value(int(b) + 1)) / 2   # exact in double
        vals += [mid, -mid]
    vals += [0.0, -0.0, float("inf"), -float("inf"), 3.3895313892515355e38, 3.4e38]
    for v in vals:
        want = brute_bf16_round(float(v))
        got = orc.double_to_bf16(float(v))
        assert got == want, f"{v!r}: got {got:#06x} want {want:#06x}"


def pin_bf16_round_ties(orc):
    """Worked ties: halfway values go to the even pattern, in the normal and subnormal ranges."""
    cases = {1 + 2.0 ** -8: 0x3F80, 1 + 3 * 2.0 ** -8: 0x3F82, -(1 + 2.0 ** -8): 0xBF80,
             2.0 ** -133: 0x0001, 2.0 ** -134: 0x0000, 3 * 2.0 ** -134: 0x0002,
             1.5: 0x3FC0, 1 + 2.0 ** -8 + 2.0 ** -30: 0x3F81}
    for v, want in cases.items():
        assert orc.double_to_bf16(v) == want, (v, hex(orc.double_to_bf16(v)), hex(want))
    assert np.isnan(_bf16_value(orc.double_to_bf16(float("nan"))))


def pin_silu(orc):
    """silu(g) = g * sigmoid(g): zero at zero, silu(g) - silu(-g) = g, sigmoid(ln 3) = 3/4,
    and the limits g and 0 far from zero."""
    import math
    assert orc.silu(0.0) == 0.0
    for g in (1e-3, 0.25, 1.0, 2.5, 7.0, 30.0):
        assert abs(orc.silu(g) - orc.silu(-g) - g) <= 1e-15 * g
    assert abs(orc.silu(math.log(3.0)) - 0.75 * math.log(3.0)) <= 4e-16
    assert orc.silu(800.0) == 800.0 and abs(orc.silu(-800.0)) == 0.0
    assert orc.silu(-1.0) < 0 and orc.silu(1.0) > 0.5


def pin_swiglu_golden(orc):
    gold = _golden("w3_swiglu_gate_up_order.json")
    words = np.zeros((1, 4, 16), np.uint32)
    words[0, :, 0] = gold["word0"]
    scales = np.full((1, 4, 1), 0x3C00, np.uint16)
    x = np.zeros(128, np.uint16)
    x[0] = 0x3F80
    r = orc.moe_swiglu(words, scales, np.array([0], np.int32), x, 128)
    assert np.allclose(r["h"][0], gold["h"], rtol=1e-15, atol=0)
    assert list(r["h_bf16"][0]) == gold["h_bf16"]


def _tail_case(E, I, H, K, seed):
    rng = np.random.default_rng(seed)
    qg = rng.integers(-8, 8, size=(E, 2 * I, K))
    wg = np.stack([pack_nibbles(qg[e]) for e in range(E)])
    sg = rng.uniform(0.001, 0.01, size=(E, 2 * I, K // 128)).astype(np.float16).view(np.uint16)
    qd = rng.integers(-8, 8, size=(E, H, I))
    wd = np.stack([pack_nibbles(qd[e]) for e in range(E)])
    sd = rng.uniform(0.001, 0.01, size=(E, H, I // 128)).astype(np.float16).view(np.uint16)
    x = (rng.standard_normal(K).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return qg, wg, sg, qd, wd, sd, x, rng


def pin_swiglu_brute(orc):
    """SwiGLU of the grouped product against an independent numpy dequantise + BLAS path:
    g from the first I rows, u from the last I; invalid ids give zeros; h_bf16 is within half a
    bfloat16 step of h."""
    E, I, K = 3, 6, 256
    qg, wg, sg, _, _, _, x, _ = _tail_case(E, I, 4, K, 32)
    ids = np.array([2, -1, 0, 2], np.int32)
    r = orc.moe_swiglu(wg, sg, ids, x, K)
    xv = bf16_bits_to_f64(x)
    for t, e in enumerate(ids):
        if not 0 <= e < E:
            assert all(np.all(r[k][t] == 0) for k in ("h", "g", "u", "mag_g", "mag_u"))
            assert np.all(r["h_bf16"][t] == 0)
            continue
        W = numpy_dense_weights(wg[e], sg[e], K)
        y = W @ xv
        g, u = y[:I], y[I:]
        h = g / (1.0 + np.exp(-g)) * u
        assert np.allclose(r["g"][t], g, rtol=1e-12, atol=1e-14)
        assert np.allclose(r["u"][t], u, rtol=1e-12, atol=1e-14)
        assert np.allclose(r["h"][t], h, rtol=1e-12, atol=1e-14)
        assert np.allclose(r["mag_g"][t], np.abs(W[:I] * xv).sum(1), rtol=1e-12)
        hb = bf16_bits_to_f64(r["h_bf16"][t])
        assert np.all(np.abs(hb - h) <= np.abs(h) * 2.0 ** -9 + 1e-40)


def pin_down_combine(orc):
    """The router-weighted down projection: a one-hot weight gives the plain product of that
    slot's expert with its own h row; doubling w doubles out exactly; permuting slots changes
    nothing; an invalid id contributes nothing; repeated ids add; numpy brute force agrees."""
    E, I, H = 4, 256, 5
    _, _, _, qd, wd, sd, _, rng = _tail_case(E, I, H, 128, 33)
    T = 4
    h = (rng.standard_normal((T, I)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ids = np.array([3, 1, 3, 0], np.int32)
    w = rng.uniform(0.1, 1.0, size=T).astype(np.float32)
    out, mag = orc.moe_down_combine(wd, sd, ids, w, h)
    for t in range(T):
        oh = np.zeros(T, np.float32)
        oh[t] = 1.0
        o1, m1 = orc.moe_down_combine(wd, sd, ids, oh, h)
        ref, rm = orc.gemv(wd[ids[t]], sd[ids[t]], h[t], I)
        assert np.array_equal(o1, ref) and np.array_equal(m1, rm)
    o2, _ = orc.moe_down_combine(wd, sd, ids, 2 * w, h)
    assert np.array_equal(o2, 2 * out)
    o3, m3 = orc.moe_down_combine(wd, sd, ids, -w, h)
    assert np.array_equal(o3, -out) and np.array_equal(m3, mag)
    perm = np.array([2, 0, 3, 1])
    op, mp = orc.moe_down_combine(wd, sd, ids[perm], w[perm], h[perm])
    assert np.allclose(op, out, rtol=1e-12, atol=1e-14) and np.allclose(mp, mag, rtol=1e-12)
    bad = ids.copy()
    bad[1] = E
    ob, _ = orc.moe_down_combine(wd, sd, bad, w, h)
    keep = [0, 2, 3]
    ok_, _ = orc.moe_down_combine(wd, sd, ids[keep], w[keep], h[keep])
    assert np.allclose(ob, ok_, rtol=1e-13, atol=1e-15)
    ref = np.zeros(H)
    for t in range(T):
        ref += float(w[t]) * (numpy_dense_weights(wd[ids[t]], sd[ids[t]], I) @ bf16_bits_to_f64(h[t]))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)
    assert np.all(mag >= np.abs(out))


# ---------------------------------------------------------------- quantise + pack
def pin_quantize_golden(orc):
    gold = _golden("w4_quantize_round_to_even.json")
    row = np.zeros(256, np.uint16)
    row[:8] = gold["group0"]["bf16"]
    row[128:132] = gold["group1"]["bf16"]
    qw, sc = orc.quantize_pack(row[None, :], 256)
    assert list(sc[0]) == [gold["group0"]["scale"], gold["group1"]["scale"]]
    assert int(qw[0, 0]) == gold["group0"]["word0"] and int(qw[0, 16]) == gold["group1"]["word16"]
    assert np.all(qw[0, 1:16] == 0) and np.all(qw[0, 17:] == 0)


def numpy_quantize(w_bits: np.ndarray, K: int):
    """Independent float32 numpy path of the same definition (numpy's own float32 division,
    float16 conversion and rint), used as a brute-force check."""
    w = (w_bits.astype(np.uint32) << 16).view(np.float32).reshape(w_bits.shape[0], K // 128, 128)
    amax = np.abs(w).max(axis=2)
    with np.errstate(over="ignore"):
        s16 = (amax / np.float32(7.0)).astype(np.float16)
    s16 = np.where(np.isinf(s16), np.float16(65504.0), s16)
    s = s16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s == 0, 0, np.clip(np.rint(w / s), -8, 7)).astype(np.int64)
    return q.reshape(w_bits.shape[0], K), s16.view(np.uint16)


def pin_quantize_brute(orc):
    """Codes and scales equal the numpy float32 path bit for bit on random rows with a wide
    magnitude spread, zero groups, huge groups (scale saturation) and tiny ones (subnormal
    scales); packing round-trips through unpack; |w - q s| <= s / 2 off the clamp."""
    rng = np.random.default_rng(41)
    N, K = 12, 512
    w = rng.standard_normal((N, K)).astype(np.float32)
    w *= np.exp2(rng.integers(-30, 20, size=(N, K // 128))).repeat(128, axis=1).astype(np.float32)
    w[3, 128:256] = 0.0                      # zero group
    w[5, :128] *= np.float32(2.0 ** 100)     # scale saturates at 65504
    w[7, 256:384] *= np.float32(2.0 ** -110)  # subnormal or zero scales
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)   # truncated to bf16 (any bf16 will do)
    qw, sc = orc.quantize_pack(bits, K)
    q_ref, s_ref = numpy_quantize(bits, K)
    assert np.array_equal(sc, s_ref)
    assert np.array_equal(orc.unpack(qw, K).astype(np.int64), q_ref)
    s = sc.view(np.float16).astype(np.float64).repeat(128, axis=1)
    wv = bf16_bits_to_f64(bits)
    q = q_ref.astype(np.float64)
    inside = (np.abs(q) < 7) & (s > 0)
    assert np.all(np.abs(wv - q * s)[inside] <= s[inside] / 2 * (1 + 2.0 ** -20))
    assert np.all(q[3, 128:256] == 0) and np.all(sc[3, 1] == 0)
    assert np.all(sc[5, 0] == 0x7BFF)


def pin_quantize_gemv_roundtrip(orc):
    """Quantising a matrix that is already exactly representable (integer codes in [-7, 7]
    times an fp16 scale with amax 7 in every group) returns the same codes and scales, so the
    GEMV of the quantised matrix equals the product with the original values."""
    rng = np.random.default_rng(42)
    N, K = 6, 384
    q = rng.integers(-7, 8, size=(N, K))
    q[:, ::128] = 7                          # amax 7 in every group
    scale_exp = rng.integers(-10, 3, size=(N, K // 128))
    s = np.exp2(scale_exp).astype(np.float64)
    w = (q * s.repeat(128, axis=1)).astype(np.float32)
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    qw, sc = orc.quantize_pack(bits, K)
    assert np.array_equal(orc.unpack(qw, K).astype(np.int64), q)
    assert np.array_equal(sc.view(np.float16).astype(np.float64), s)
    x = (rng.standard_normal(K).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y, _ = orc.gemv(qw, sc, x, K)
    assert np.allclose(y, w.astype(np.float64) @ bf16_bits_to_f64(x), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- batched grouped experts
def pin_moe_batched(orc):
    """Token m, slot t is the product of expert ids[m][t] with X[m]: against the independent
    numpy dequantise + BLAS path, with repeated experts across tokens, a repeated expert within
    a token, invalid ids (zeros), a padded X stride and a row subset."""
    E, N, K, M, T = 7, 5, 256, 3, 4
    rng = np.random.default_rng(51)
    q = rng.integers(-8, 8, size=(E, N, K))
    words = np.stack([pack_nibbles(q[e]) for e in range(E)])
    scales = rng.uniform(0.001, 0.01, size=(E, N, K // 128)).astype(np.float16).view(np.uint16)
    X = (rng.standard_normal((M, K + 8)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ids = np.array([[1, 4, 6, 1], [4, 0, -2, 6], [7, 3, 1, 2]], np.int32)
    Y, mag = orc.moe_gemv_batched(words, scales, ids, X, K)
    xs = bf16_bits_to_f64(X[:, :K])
    for m in range(M):
        for t in range(T):
            e = ids[m, t]
            if not 0 <= e < E:
                assert np.all(Y[m, t] == 0) and np.all(mag[m, t] == 0)
                continue
            W = numpy_dense_weights(words[e], scales[e], K)
            assert np.allclose(Y[m, t], W @ xs[m], rtol=1e-12, atol=1e-14)
            assert np.allclose(mag[m, t], np.abs(W * xs[m]).sum(1), rtol=1e-12)
    assert np.array_equal(Y[0, 0], Y[0, 3]) and not np.array_equal(Y[0, 1], Y[1, 0])
    Ys, ms = orc.moe_gemv_batched(words, scales, ids, X, K, rows=[4, 0])
    assert np.array_equal(Ys, Y[:, :, [4, 0]]) and np.array_equal(ms, mag[:, :, [4, 0]])


def pin_expert_id_upper_bound(orc):
    """Ids E and E + 1 name no expert in every grouped form, even when the tensors hold more
    experts past the E the oracle is told about (so reading expert E would find real weights):
    their rows are zero, they add nothing to the combine, and the valid slots are unchanged."""
    E, N, K = 3, 4, 256
    rng = np.random.default_rng(61)
    held = E + 2
    q = rng.integers(-8, 8, size=(held, N, K))
    q[E:] = np.where(q[E:] == 0, 5, q[E:])                  # spare experts: no zero codes
    words = np.stack([pack_nibbles(q[e]) for e in range(held)])
    scales = rng.uniform(0.001, 0.01, size=(held, N, K // 128)).astype(np.float16).view(np.uint16)
    x = np.full(K, 0x3F80, np.uint16)                       # x = 1 everywhere
    ids = np.array([1, E, 0, E + 1], np.int32)
    valid = [0, 2]
    y, mag = orc.moe_gemv(words, scales, ids, x, K, num_experts=E)
    yv, mv = orc.moe_gemv(words, scales, ids[valid], x, K, num_experts=E)
    assert np.all(y[[1, 3]] == 0) and np.all(mag[[1, 3]] == 0)
    assert np.array_equal(y[valid], yv) and np.array_equal(mag[valid], mv)
    yall, _ = orc.moe_gemv(words, scales, ids, x, K)         # told all held experts: nonzero
    assert np.all(yall[[1, 3]] != 0)

    X = np.stack([x, x ^ 0x8000])                            # token 1 is -x
    idb = np.array([[E, 2], [0, E + 1]], np.int32)
    Y, magb = orc.moe_gemv_batched(words, scales, idb, X, K, num_experts=E)
    assert np.all(Y[0, 0] == 0) and np.all(Y[1, 1] == 0) and np.all(magb[0, 0] == 0)
    assert np.array_equal(Y[0, 1], orc.gemv(words[2], scales[2], x, K)[0])

    I = N // 2                                              # gate rows [0, I), up rows [I, 2I)
    r = orc.moe_swiglu(words, scales, ids, x, K, num_experts=E)
    for k in ("h", "g", "u", "mag_g", "mag_u"):
        assert np.all(r[k][[1, 3]] == 0)
    assert np.all(r["h_bf16"][[1, 3]] == 0)
    rv = orc.moe_swiglu(words, scales, ids[valid], x, K, num_experts=E)
    assert np.array_equal(r["h"][valid], rv["h"]) and r["h"].shape == (4, I)

    h = np.stack([x] * 4)                                   # each slot's own row: all ones
    w = np.array([0.25, 0.5, 0.75, 1.0], np.float32)
    out, mo = orc.moe_down_combine(words, scales, ids, w, h, num_experts=E)
    ov, mov = orc.moe_down_combine(words, scales, ids[valid], w[valid], h[valid], num_experts=E)
    assert np.array_equal(out, ov) and np.array_equal(mo, mov)
    oall, _ = orc.moe_down_combine(words, scales, ids, w, h)
    assert not np.array_equal(oall, out)


# ---------------------------------------------------------------- three-bit experts
def pack3(q):
    """Independent packer for the three-bit layout, written from its statement: codes [N][K]
    in [-4, 3] to uint32 [N][3K/32]. Block b of a row holds codes 32b..32b+31; code c = 10t + j
    (j < 5) at bits 3j of word t, c = 10t + 5 + j at bits 16 + 3j, and bit i of codes 30 and 31
    at bits 15 and 31 of word i."""
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    f = (q & 7).astype(np.uint64).reshape(N, K // 32, 32)
    words = np.zeros((N, K // 32, 3), np.uint64)
    for t in range(3):
        for j in range(5):
            words[:, :, t] |= f[:, :, 10 * t + j] << np.uint64(3 * j)
            words[:, :, t] |= f[:, :, 10 * t + 5 + j] << np.uint64(16 + 3 * j)
        words[:, :, t] |= ((f[:, :, 30] >> np.uint64(t)) & np.uint64(1)) << np.uint64(15)
        words[:, :, t] |= ((f[:, :, 31] >> np.uint64(t)) & np.uint64(1)) << np.uint64(31)
    return words.reshape(N, 3 * K // 32).astype(np.uint32)


def pin_w5_three_bit_golden(orc):
    """The hand-derived block of tests/golden/w5_three_bit_layout.json: unit probes return the
    codes written there, all ones gives their sum."""
    g = json.load(open(os.path.join(GOLDEN, "w5_three_bit_layout.json")))
    words = np.array(g["words"], np.uint32).reshape(1, 1, 12)
    sc = np.array([[[g["scale_bits"]]]], np.uint16)
    ids = np.array([0], np.int32)
    for k, want in g["probes"].items():
        x = np.zeros(128, np.uint16)
        x[int(k)] = 0x3F80
        y, _ = orc.moe_gemv3(words, sc, ids, x, 128)
        assert y[0, 0] == want, (k, y[0, 0], want)
    y, _ = orc.moe_gemv3(words, sc, ids, np.full(128, 0x3F80, np.uint16), 128)
    assert y[0, 0] == g["all_ones"]


def pin_three_bit_unpack_roundtrip(orc):
    """Random codes packed by the independent packer come back from the oracle's decoder;
    every code value at every position of a block."""
    rng = np.random.default_rng(71)
    q = rng.integers(-4, 4, size=(7, 256))
    assert np.array_equal(orc.unpack3(pack3(q), 256).astype(np.int64), q)
    q = np.array([[(c + p) % 8 - 4 for p in range(32)] for c in range(8)])
    assert np.array_equal(orc.unpack3(pack3(q), 32).astype(np.int64), q)


def pin_three_bit_brute_force(orc):
    """Grouped three-bit product against numpy: dense dequantised weights times x in float64,
    invalid ids (including E and E + 1 with spare experts in memory) give zeros, unit probes
    return q * s exactly."""
    E, held, N, K = 3, 5, 6, 384
    rng = np.random.default_rng(72)
    q = rng.integers(-4, 4, size=(held, N, K))
    words = np.stack([pack3(q[e]) for e in range(held)])
    sc = rng.uniform(0.001, 0.01, size=(held, N, K // 128)).astype(np.float16).view(np.uint16)
    x = (rng.standard_normal(K).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ids = np.array([2, E, 0, -1, E + 1, 2], np.int32)
    y, mag = orc.moe_gemv3(words, sc, ids, x, K, num_experts=E)
    xv = bf16_bits_to_f64(x)
    for t, e in enumerate(ids):
        if not 0 <= e < E:
            assert np.all(y[t] == 0) and np.all(mag[t] == 0)
            continue
        W = q[e] * np.repeat(sc[e].view(np.float16).astype(np.float64), 128, axis=1)
        assert np.allclose(y[t], W @ xv, rtol=1e-12, atol=1e-14)
        assert np.allclose(mag[t], np.abs(W * xv).sum(1), rtol=1e-12)
    for k in (0, 9, 10, 15, 29, 30, 31, 32, 200, 383):
        e1 = np.zeros(K, np.uint16)
        e1[k] = 0x3F80
        yk, _ = orc.moe_gemv3(words, sc, np.array([1], np.int32), e1, K, num_experts=E)
        assert np.array_equal(yk[0], q[1][:, k] * sc[1][:, k // 128].view(np.float16).astype(np.float64))
    ys, ms = orc.moe_gemv3(words, sc, ids, x, K, rows=[5, 0], num_experts=E)
    assert np.array_equal(ys, y[:, [5, 0]]) and np.array_equal(ms, mag[:, [5, 0]])


ALL_PINS = [
    pin_f16_decode, pin_bf16_decode, pin_w1, pin_w2, pin_unpack, pin_unit_probes,
    pin_zero_scale_groups, pin_linearity, pin_negation, pin_constant_rows, pin_brute_force,
    pin_mag_nonnegative, pin_batched, pin_moe, pin_row_subset, pin_bf16_round_brute,
    pin_bf16_round_ties, pin_silu, pin_swiglu_golden, pin_swiglu_brute, pin_down_combine,
    pin_quantize_golden, pin_quantize_brute, pin_quantize_gemv_roundtrip, pin_moe_batched,
    pin_expert_id_upper_bound, pin_w5_three_bit_golden, pin_three_bit_unpack_roundtrip,
    pin_three_bit_brute_force,
]
