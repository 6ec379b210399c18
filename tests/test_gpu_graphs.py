"""The entry points inside HIP graphs and on concurrent streams.

Callers capture decode steps in graphs, so every entry point is captured once and replayed
several times with new inputs written between replays (the library issues no memsets or
allocations that a graph could freeze); each replay must equal an eager call on the same
inputs bit for bit. Two streams running different calls at once must each give the eager
result.
"""
import numpy as np
import pytest
import torch

import synthetic
import weight_only_int4_w4a16_amd as w
from devhelp import bf16, f16, words

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_calls():
    d = synthetic.dense(N=3000, K=2304, seed=1, M=16, config_id=960)
    m = synthetic.moe(E=12, N=512, K=2304, topk=4, seed=2, config_id=961)
    m3 = synthetic.moe3(E=12, N=256, K=2304, topk=4, seed=2, config_id=964)
    q3, s3 = words(m3.qweight), f16(m3.scales)
    qd, sd = words(d.qweight), f16(d.scales)
    qm, sm = words(m.qweight), f16(m.scales)
    x1 = bf16(d.x[0]).clone()
    X = bf16(d.x).clone()
    xm = bf16(m.x).clone()
    ids = torch.from_numpy(m.ids).cuda()
    ids2 = torch.from_numpy(np.array([[0, 5], [5, 11], [3, 0]], np.int32)).cuda()
    X3 = X[:3].clone()
    y1 = torch.empty(3000, dtype=torch.float32, device="cuda")
    Y = torch.empty((16, 3000), dtype=torch.float32, device="cuda")
    ym = torch.empty((4, 512), dtype=torch.float32, device="cuda")
    yb = torch.empty((3, 2, 512), dtype=torch.float32, device="cuda")
    y3 = torch.empty((4, 256), dtype=torch.float32, device="cuda")

    def calls():
        w.gemv(qd, sd, x1, out=y1)
        w.gemv_batched(qd, sd, X, out=Y)
        w.moe_gemv(qm, sm, ids, xm, out=ym)
        w.moe_gemv_batched(qm, sm, ids2, X3[:, :2304], out=yb)
        w.moe_gemv3(q3, s3, ids, xm, out=y3)

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    rng = np.random.default_rng(3)
    for rep in range(4):
        # new inputs in place, then replay, then the same calls eagerly
        x1.copy_(bf16(synthetic.draw_acts(rng, (2304,))))
        X.copy_(bf16(synthetic.draw_acts(rng, (16, 2304))))
        xm.copy_(bf16(synthetic.draw_acts(rng, (2304,))))
        X3.copy_(bf16(synthetic.draw_acts(rng, (3, 2304))))
        ids.copy_(torch.from_numpy(rng.choice(12, 4, replace=False).astype(np.int32)).cuda())
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (y1, Y, ym, yb, y3)]
        calls()
        torch.cuda.synchronize()
        for a, b, name in zip(got, (y1, Y, ym, yb, y3),
                              ("gemv", "batched", "moe", "moe_batched", "moe3")):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


def test_graph_replays_of_tail_and_quantise_match_eager_calls():
    """The expert tail (SwiGLU gate+up, then the down projection with the router-weighted sum)
    and quantise-and-pack, captured once and replayed with new inputs between replays."""
    d = synthetic.moe_tail(10, 256, 300, 2304, 4, 5, config_id=962)
    qg = words(d.gu_qweight)
    sg = f16(d.gu_scales)
    qd = words(d.down_qweight)
    sd = f16(d.down_scales)
    x = bf16(d.x).clone()
    ids = torch.from_numpy(d.ids).cuda()
    rw = torch.from_numpy(d.route_w).cuda()
    h = torch.empty((4, 256), dtype=torch.bfloat16, device="cuda")
    out = torch.empty(300, dtype=torch.float32, device="cuda")
    wq = bf16(synthetic.draw_acts(np.random.default_rng(4), (96, 1024))).clone()
    qo = torch.empty((96, 128), dtype=torch.int32, device="cuda")
    so = torch.empty((96, 8), dtype=torch.float16, device="cuda")

    def calls():
        w.moe_gemv_swiglu(qg, sg, ids, x, out=h)
        w.moe_down_combine(qd, sd, ids, rw, h, out=out)
        w.quantize_pack(wq, out=(qo, so))

    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    rng = np.random.default_rng(5)
    for rep in range(4):
        x.copy_(bf16(synthetic.draw_acts(rng, (2304,))))
        ids.copy_(torch.from_numpy(rng.choice(10, 4, replace=False).astype(np.int32)).cuda())
        rw.copy_(torch.from_numpy(rng.uniform(0.05, 1.0, 4).astype(np.float32)).cuda())
        wq.copy_(bf16(synthetic.draw_acts(rng, (96, 1024))))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (h, out, qo, so)]
        calls()
        torch.cuda.synchronize()
        for a, b, name in zip(got, (h, out, qo, so), ("swiglu", "down_combine", "codes", "scales")):
            assert torch.equal(a.view(torch.int16) if a.dtype in (torch.bfloat16, torch.float16)
                               else a, b.view(torch.int16) if b.dtype in (torch.bfloat16,
                                                                          torch.float16) else b), \
                f"replay {rep}: {name} differs from the eager call"


def test_concurrent_streams_give_eager_results():
    a = synthetic.dense(N=8192, K=4096, seed=4, M=1, config_id=962)
    b = synthetic.dense(N=4096, K=14336, seed=5, M=8, config_id=963)
    qa, sa, xa = words(a.qweight), f16(a.scales), bf16(a.x[0])
    qb, sb, xb = words(b.qweight), f16(b.scales), bf16(b.x)
    ya_ref = w.gemv(qa, sa, xa)
    yb_ref = w.gemv_batched(qb, sb, xb)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            ya = w.gemv(qa, sa, xa)
        with torch.cuda.stream(s2):
            yb = w.gemv_batched(qb, sb, xb)
        outs.append((ya, yb))
    torch.cuda.synchronize()
    for ya, yb in outs:
        assert torch.equal(ya, ya_ref) and torch.equal(yb, yb_ref)
