"""GPU parity of bf16 -> INT4 quantise-and-pack (w4a16_quantize_pack) against the CPU oracle.

Codes and scales are decided in float32 by the definition, so the packed words and the fp16
scales must be bit-identical to the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
import par_oracle
import weight_only_int4_w4a16_amd as w
from devhelp import host

pytestmark = pytest.mark.gpu


def random_bf16(N, K, seed, spread=20, ld=None):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((N, K)).astype(np.float32)
    a *= np.exp2(rng.integers(-spread, spread + 1, size=(N, K // 128))).repeat(128, axis=1)
    bits = (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    if ld is not None and ld > K:
        pad = rng.integers(0, 1 << 16, size=(N, ld - K), dtype=np.uint16) & 0x7F7F
        bits = np.concatenate([bits, pad], axis=1)
    return bits


def run(bits, K):
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    qw, sc = w.quantize_pack(t, out=(torch.empty((bits.shape[0], K // 8), dtype=torch.int32,
                                                 device="cuda"),
                                     torch.empty((bits.shape[0], K // 128), dtype=torch.float16,
                                                 device="cuda")))
    return host(qw).view(np.uint32), host(sc).view(np.uint16)


@pytest.mark.parametrize("N,K,ld", [(1, 128, None), (3, 256, None), (5, 384, 392), (37, 2304, None),
                                    (300, 4096, 4224), (129, 14336, None), (2, 65536, None)])
@pytest.mark.parametrize("seed", [0, 1])
def test_quantize_bit_exact(N, K, ld, seed):
    bits = random_bf16(N, K, seed, ld=ld)
    print(f"quantize N={N} K={K} ld={ld} seed={seed}", flush=True)
    qw, sc = run(bits, K)
    rq, rs = oracle.quantize_pack(bits, K)
    assert np.array_equal(sc, rs), f"{int((sc != rs).sum())} scales differ"
    assert np.array_equal(qw, rq), f"{int((qw != rq).sum())} words differ"


def test_quantize_special_groups():
    """Ties (w / s = k + 1/2 with s = 1), zero groups, saturating and subnormal scales."""
    K = 1024
    rows = []
    tie = np.zeros(K, np.float32)
    tie[:16] = [7, -7, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, -0.5, -1.5, -2.5, -3.5, -4.5, -5.5, -6.5]
    rows.append(tie)
    rows.append(np.zeros(K, np.float32))
    big = np.full(K, 3.0e38, np.float32)
    big[1::2] = -1.0e37
    rows.append(big)
    tiny = np.full(K, 1.0e-38, np.float32)
    tiny[::3] = -7.0e-40
    rows.append(tiny)
    a = np.stack(rows)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    qw, sc = run(bits, K)
    rq, rs = oracle.quantize_pack(bits, K)
    assert np.array_equal(sc, rs) and np.array_equal(qw, rq)
    assert np.all(sc[1] == 0) and np.all(qw[1] == 0)
    assert np.all(sc[2] == 0x7BFF)
    codes = oracle.unpack(qw[:1, :2], 16)[0]
    assert list(codes) == [7, -7, 0, 2, 2, 4, 4, 6, 6, 0, -2, -2, -4, -4, -6, -6]


def test_quantize_near_ties_bit_exact():
    """Values at and next to w / s = k + 1/2 for scales that are not powers of two: the kernel's
    reciprocal estimate must defer to the exact quotient wherever rounding is close."""
    rng = np.random.default_rng(21)
    K = 128 * 64
    rows = []
    for s16 in rng.integers(0x2800, 0x5000, size=24, dtype=np.uint16):
        s = float(np.array([s16], np.uint16).view(np.float16)[0])
        k = rng.integers(-8, 8, size=K).astype(np.float64)
        jitter = rng.choice([-2, -1, 0, 1, 2], size=K) * 2.0 ** -7
        vals = ((k + 0.5 + jitter * np.abs(k + 0.5) * 2.0 ** -1) * s).astype(np.float32)
        vals.reshape(-1, 128)[:, 0] = np.float32(7.0 * s)         # amax 7 s in every group
        rows.append(vals)
    a = np.stack(rows)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    qw, sc = run(bits, K)
    rq, rs = oracle.quantize_pack(bits, K)
    assert np.array_equal(sc, rs) and np.array_equal(qw, rq)


def test_quantize_then_gemv_matches_oracle():
    """The quantised matrix feeds the GEMV: GPU quantise + GPU GEMV against the oracle's
    quantisation and GEMV (identical operands, so the GEMV tolerance applies)."""
    N, K = 1000, 2304
    bits = random_bf16(N, K, 7, spread=3)
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    qw, sc = w.quantize_pack(t)
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(K).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    xt = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    y = host(w.gemv(qw, sc, xt)).astype(np.float64)
    rq, rs = oracle.quantize_pack(bits, K)
    ref, mag = oracle.gemv(rq, rs, x, K)
    assert np.all(np.abs(y - ref) <= oracle.bound(mag))


def test_quantize_full_size_gate_up():
    """A 28672 x 4096 bf16 matrix (the fused gate+up projection) quantised in one call."""
    N, K = 28672, 4096
    rng = np.random.default_rng(11)
    # finite bf16 patterns of moderate magnitude: exponent field 100..140, random sign/fraction
    expo = rng.integers(100, 141, size=(N, K), dtype=np.uint16)
    bits = (expo << 7) | rng.integers(0, 128, size=(N, K), dtype=np.uint16)
    bits |= (rng.integers(0, 2, size=(N, K), dtype=np.uint16) << 15)
    print(f"quantize full N={N} K={K}", flush=True)
    qw, sc = run(bits, K)
    rq, rs = par_oracle.quantize_pack(bits, K, np.arange(N))
    assert np.array_equal(sc, rs) and np.array_equal(qw, rq)
