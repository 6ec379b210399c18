"""GPU parity of the expert tail: SwiGLU gate+up (w4a16_moe_gemv_swiglu) and the grouped down
projection with the router-weighted sum (w4a16_moe_down_combine), against the CPU oracle.

Tolerances, derived from the arithmetic:
  * h = silu(g) u: the kernel's g and u carry at most the GEMV error dg = 1e-3 mag_g + 1e-5
    (du likewise); |silu'| <= 1.1, so the fp32 h differs from the exact one by at most
    1.1 (|u| + du) dg + (|silu(g)| + 1.1 dg) du, plus fp32 evaluation of silu (1e-6 relative);
    rounding to bfloat16 adds at most half a step, 2^-8 |h| (relative step <= 2^-7).
  * down + combine from the same bf16 h: 1e-3 * sum_t |w_t| sum_k |q s h| + 1e-5 per element.
  * the chained tail (the kernel's own h into the down step): the two h may differ by one
    bfloat16 step (<= 2^-7 |h|) where the rounding decisions fall on either side of a tie
    point, so the allowance is 2^-7 * mag + 1e-3 * mag + 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
import weight_only_int4_w4a16_amd as w
from devhelp import host

pytestmark = pytest.mark.gpu


def dev_tail(d):
    qg = torch.from_numpy(d.gu_qweight.view(np.int32)).cuda()
    sg = torch.from_numpy(d.gu_scales.view(np.float16)).cuda()
    x = torch.from_numpy(d.x.view(np.int16)).cuda().view(torch.bfloat16)
    ids = torch.from_numpy(d.ids).cuda()
    rw = torch.from_numpy(d.route_w).cuda()
    qd = torch.from_numpy(d.down_qweight.view(np.int32)).cuda()
    sd = torch.from_numpy(d.down_scales.view(np.float16)).cuda()
    h = torch.from_numpy(d.h.view(np.int16)).cuda().view(torch.bfloat16)
    return qg, sg, x, ids, rw, qd, sd, h


def gate_up_dev(d):
    """Device copies of grouped operands whose 2I rows per expert are read as gate + up."""
    qg = torch.from_numpy(d.qweight.view(np.int32)).cuda()
    sg = torch.from_numpy(d.scales.view(np.float16)).cuda()
    x = torch.from_numpy(d.x.view(np.int16)).cuda().view(torch.bfloat16)
    return qg, sg, x, torch.from_numpy(d.ids).cuda()


def bf16_to_f64(t):
    bits = host(t.view(torch.int16)).view(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def check_h(h_gpu, r, what):
    got = bf16_to_f64(h_gpu)
    dg, du = oracle.bound(r["mag_g"]), oracle.bound(r["mag_u"])
    sg = r["g"] / (1.0 + np.exp(-r["g"]))
    prop = 1.1 * (np.abs(r["u"]) + du) * dg + (np.abs(sg) + 1.1 * dg) * du
    tol = prop * (1 + 2.0 ** -7) + (2.0 ** -8 + 1e-6) * np.abs(r["h"]) + 1e-30
    err = np.abs(got - r["h"])
    flips = int((host(h_gpu.view(torch.int16)).view(np.uint16) != r["h_bf16"]).sum())
    print(f"{what}: n={err.size} max|err|/tol={float((err / tol).max()):.3f} "
          f"bf16 patterns differing from the oracle's rounding: {flips}", flush=True)
    assert np.all(err <= tol), f"{what}: {int((err > tol).sum())} outside tolerance"
    assert flips <= max(2, err.size // 100)


def check_out(got, ref, mag, what, extra_rel=0.0):
    got = host(got).astype(np.float64)
    tol = oracle.bound(mag) + extra_rel * mag
    err = np.abs(got - ref)
    ratio = float((err / np.maximum(mag, 1e-30)).max())
    print(f"{what}: n={err.size} max|err|={err.max():.3e} max|err|/mag={ratio:.2e}", flush=True)
    assert np.all(err <= tol), f"{what}: {int((err > tol).sum())} outside tolerance"
    assert np.all(np.isfinite(got))


# (E, I, K, topk): K = 2304 takes 8 lanes x 3 chunks, K = 2048 32 lanes (one gate row per
# wave half), K = 128 4 lanes with I below the 8 gate rows of a wave step; I not a multiple of
# the gate rows per step in every case but one.
# The last two: activations longer than two staging passes of 256 threads (K = 8192), and more
# slots than threads (ids staged past the first 256).
SWIGLU_SHAPES = [(6, 64, 384, 3), (4, 3, 128, 2), (5, 37, 2304, 4), (3, 100, 2048, 2),
                 (2, 1000, 4096, 1), (9, 256, 2304, 8), (3, 64, 8192, 2), (300, 8, 256, 300)]


@pytest.mark.parametrize("E,I,K,topk", SWIGLU_SHAPES)
@pytest.mark.parametrize("seed", [0, 1])
def test_swiglu_matches_oracle(E, I, K, topk, seed):
    d = synthetic.moe(E, 2 * I, K, topk, seed, config_id=900)
    print(f"swiglu E={E} I={I} K={K} topk={topk} seed={seed} "
          f"plan={w.describe_tail_plan(0, 0, K, I, topk)}", flush=True)
    qg, sg, x, ids = gate_up_dev(d)
    h = w.moe_gemv_swiglu(qg, sg, ids, x)
    torch.cuda.synchronize()
    r = oracle.moe_swiglu(d.qweight, d.scales, d.ids, d.x, K)
    check_h(h, r, f"swiglu {E}x{2 * I}x{K} top{topk}")


def test_swiglu_invalid_and_repeated_ids():
    d = synthetic.moe(5, 80, 2304, 4, 3, config_id=901)
    ids = np.array([4, -1, 4, 5], np.int32)
    qg, sg, x, _ = gate_up_dev(d)
    h = w.moe_gemv_swiglu(qg, sg, torch.from_numpy(ids).cuda(), x)
    torch.cuda.synchronize()
    r = oracle.moe_swiglu(d.qweight, d.scales, ids, d.x, 2304)
    check_h(h, r, "swiglu invalid/repeated ids")
    hb = host(h.view(torch.int16))
    assert np.all(hb[1] == 0) and np.all(hb[3] == 0)
    assert np.array_equal(hb[0], hb[2])


# (E, I, H, topk): I = 1024 takes 32 lanes per row, I = 384 4 lanes; H below and above the
# rows of one wave step. Then 300 slots (more than the 256 threads that stage ids and router
# weights) over a 38400-long activation, on the staged combine form; and the split-K combine
# forms with 8 chunks per lane (8 lanes: 64 slots of I = 256 and 16 of I = 768; 4 lanes: 64
# slots of I = 128), the instances that hold spilled registers.
DOWN_SHAPES = [(6, 256, 300, 3), (4, 128, 1, 1), (5, 384, 77, 4), (12, 1024, 2304, 8),
               (3, 2048, 129, 2), (40, 512, 1000, 16), (300, 128, 20, 300), (70, 256, 100, 64),
               (20, 768, 100, 16), (70, 128, 100, 64)]


@pytest.mark.parametrize("E,I,H,topk", DOWN_SHAPES)
@pytest.mark.parametrize("seed", [0, 1])
def test_down_combine_matches_oracle(E, I, H, topk, seed):
    d = synthetic.moe_tail(E, I, H, 128, topk, seed, config_id=902)
    print(f"down E={E} H={H} I={I} topk={topk} seed={seed} "
          f"plan={w.describe_tail_plan(1, H, 0, I, topk)}", flush=True)
    _, _, _, ids, rw, qd, sd, h = dev_tail(d)
    out = w.moe_down_combine(qd, sd, ids, rw, h)
    torch.cuda.synchronize()
    ref, mag = oracle.moe_down_combine(d.down_qweight, d.down_scales, d.ids, d.route_w, d.h)
    check_out(out, ref, mag, f"down {E}x{H}x{I} top{topk}")


def test_down_combine_invalid_duplicate_and_signed_weights():
    d = synthetic.moe_tail(6, 256, 200, 128, 5, 4, config_id=903)
    ids = np.array([2, 7, 2, -3, 0], np.int32)
    rw = np.array([0.5, 0.25, -0.75, 1.0, 2.0], np.float32)
    _, _, _, _, _, qd, sd, h = dev_tail(d)
    out = w.moe_down_combine(qd, sd, torch.from_numpy(ids).cuda(), torch.from_numpy(rw).cuda(), h)
    torch.cuda.synchronize()
    ref, mag = oracle.moe_down_combine(d.down_qweight, d.down_scales, ids, rw, d.h)
    check_out(out, ref, mag, "down invalid/duplicate/signed")


def test_down_combine_one_hot_is_the_expert_gemv():
    # A single slot with weight 1.0 is the plain GEMV of that expert's rows with h[0]; the
    # kernel multiplies each group scale by 1.0 exactly, but sums in its own order, so compare
    # with the oracle rather than bit for bit, and check weight 2^-3 scales the result exactly.
    d = synthetic.moe_tail(4, 512, 333, 128, 1, 5, config_id=904)
    _, _, _, ids, _, qd, sd, h = dev_tail(d)
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    o1 = w.moe_down_combine(qd, sd, ids, one, h)
    o8 = w.moe_down_combine(qd, sd, ids, one * 0.125, h)
    torch.cuda.synchronize()
    assert torch.equal(o8, o1 * 0.125)
    e = int(d.ids[0])
    ref, mag = oracle.gemv(d.down_qweight[e], d.down_scales[e], d.h[0], 512)
    check_out(o1, ref, mag, "down one-hot")


@pytest.mark.parametrize("seed", [0, 1])
def test_tail_full_size_chain(seed):
    """The expert tail at its real size (256 experts, 2I = 2048 x K = 2304 gate+up, H = 2304 x
    I = 1024 down, top-8): the kernel's h feeds the down step; every output checked."""
    d = synthetic.tail_config(seed)
    print(f"tail full seed={seed} ids={d.ids.tolist()}", flush=True)
    qg, sg, x, ids, rw, qd, sd, _ = dev_tail(d)
    h = w.moe_gemv_swiglu(qg, sg, ids, x)
    out = w.moe_down_combine(qd, sd, ids, rw, h)
    torch.cuda.synchronize()
    r = oracle.moe_swiglu(d.gu_qweight, d.gu_scales, d.ids, d.x, d.K)
    check_h(h, r, "tail swiglu full")
    ref, mag = oracle.moe_down_combine(d.down_qweight, d.down_scales, d.ids, d.route_w,
                                       r["h_bf16"])
    check_out(out, ref, mag, "tail chain full", extra_rel=2.0 ** -7)


def test_tail_deterministic_and_no_allocation():
    d = synthetic.moe_tail(8, 1024, 2304, 2304, 8, 6, config_id=905)
    qg, sg, x, ids, rw, qd, sd, _ = dev_tail(d)
    h1 = w.moe_gemv_swiglu(qg, sg, ids, x)
    o1 = w.moe_down_combine(qd, sd, ids, rw, h1)
    h2, o2 = torch.empty_like(h1), torch.empty_like(o1)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        w.moe_gemv_swiglu(qg, sg, ids, x, out=h2)
        w.moe_down_combine(qd, sd, ids, rw, h2, out=o2)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16)) and torch.equal(o1, o2)


def test_tail_reads_only_selected_experts_and_skips_invalid_slots():
    """Every expert no slot selects has NaN scales, in both the gate+up and the down weights,
    and expert 0 (the one an invalid slot's loads are pointed at) has infinite down scales; two
    slots carry ids outside [0, E) with nonzero router weights. The SwiGLU rows of the invalid
    slots are zero, everything else is finite, and the combine equals the oracle's, which skips
    the invalid slots altogether."""
    E, I, H, K, topk = 12, 256, 384, 2304, 6
    d = synthetic.moe_tail(E, I, H, K, topk, 7, config_id=906)
    ids = np.array([3, E, 5, -2, 3, 9], np.int32)
    rw = np.array([0.3, 0.5, 0.2, 0.25, 0.1, 0.4], np.float32)
    valid = np.unique(ids[(ids >= 0) & (ids < E)])
    assert 0 not in valid
    gs = np.full_like(d.gu_scales, 0x7E00)
    gs[valid] = d.gu_scales[valid]
    ds = np.full_like(d.down_scales, 0x7E00)
    ds[valid] = d.down_scales[valid]
    ds[0] = 0x7C00                                   # +inf
    qg = torch.from_numpy(d.gu_qweight.view(np.int32)).cuda()
    x = torch.from_numpy(d.x.view(np.int16)).cuda().view(torch.bfloat16)
    tid = torch.from_numpy(ids).cuda()
    h = w.moe_gemv_swiglu(qg, torch.from_numpy(gs.view(np.float16)).cuda(), tid, x)
    r = oracle.moe_swiglu(d.gu_qweight, d.gu_scales, ids, d.x, K)
    check_h(h, r, "swiglu poisoned unselected experts")
    hb = host(h.view(torch.int16)).view(np.uint16)
    assert np.all(hb[[1, 3]] == 0)
    out = w.moe_down_combine(torch.from_numpy(d.down_qweight.view(np.int32)).cuda(),
                             torch.from_numpy(ds.view(np.float16)).cuda(), tid,
                             torch.from_numpy(rw).cuda(), h)
    torch.cuda.synchronize()
    ref, mag = oracle.moe_down_combine(d.down_qweight, d.down_scales, ids, rw, r["h_bf16"])
    check_out(out, ref, mag, "combine, invalid slots over an infinite expert 0",
              extra_rel=2.0 ** -7)
