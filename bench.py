"""W4A16 decode GEMV benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]

Workload: the MLP-shaped GEMV pair at M = 1 (one decode token): a 28672 x 4096 fused gate+up
projection followed by a 4096 x 14336 down projection, INT4 weights packed 8 per uint32 along K,
one fp16 scale per 128-wide group, bf16 activations, fp32 outputs; seeded synthetic operands.
One step runs both GEMVs. The weights of a step rotate through enough copies (12 x 91 MB) that
the 256 MB memory-side cache cannot hold them, so every step streams its weights from HBM.
The K timed steps are captured in one HIP graph, replayed once between two HIP events on the
launch stream, with device synchronisation on both sides.

Prints one JSON line. `value` is algorithmic bytes (packed weights + fp16 scales + bf16
activations) per second over the whole step, in GB/s. `roofline` is for the dominant kernel
(the 28672 x 4096 GEMV): the same bytes over its own average duration, timed the same way on a
graph of back-to-back launches; `roofline.launch_floor_us` is the per-launch time of a kernel
that reads 16 bytes, timed the same way (the part of every call that is not memory time).
`cpu_baseline` is the CPU oracle (single thread, float64) timed
on whole steps of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMV achieved HBM GB/s (% of MI355X peak) and µs/call at M=1"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_28672x4096.json")
# The sources that define the GEMV kernels and their template instances (not the validation or
# dispatch layers). A recorded traffic measurement stays valid while these and the launch plan
# of the measured kernel (its describe_plan text) are unchanged.
KERNEL_SOURCES = [os.path.join(ROOT, "weight_only_int4_w4a16_amd", "csrc", f)
                  for f in ("kernels.hip", "plan.h")]


def kernel_source_digest(plan_text: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(plan_text.encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload table (all five shapes) in the JSON line")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time for the oracle baseline (whole steps, at least one)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy 5 times (reference "
                         "kernel of known traffic for scaling FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--profile-workload", default=None,
                    choices=["c1", "c2", "c3a", "c3b", "c4", "c5a", "c5b"],
                    help="only launch this workload's GEMV --steps times on rotated copies "
                         "(for profiler runs; prints a short JSON line, no timing)")
    ap.add_argument("--batch", type=int, default=1, help="tokens M for --profile-workload")
    return ap.parse_args()


def to_dev(d, dev, torch, np):
    qw = torch.from_numpy(np.ascontiguousarray(d.qweight).view(np.int32)).to(dev)
    sc = torch.from_numpy(np.ascontiguousarray(d.scales).view(np.float16)).to(dev)
    x = torch.from_numpy(np.ascontiguousarray(d.x).view(np.int16)).to(dev).view(torch.bfloat16)
    return qw, sc, x


def rotated(torch, t, R):
    """R copies of t in one contiguous allocation (views), so every copy is separate memory."""
    big = torch.empty((R,) + tuple(t.shape), dtype=t.dtype, device=t.device)
    for r in range(R):
        big[r].copy_(t)
    return [big[r] for r in range(R)]


WARM_MS = 50.0


def warm_graph(torch, g, min_ms=WARM_MS):
    """Untimed replays of g until at least min_ms of GPU time has passed (at least 3). On
    MI355X the first ~25 ms of work on freshly set-up buffers run 2-10 % slower than the steady
    state (interleaved repeats of the same graph agree to 0.1-0.3 % after that), so every timed
    replay follows such a warm-up."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(max(2, int(min_ms / one) + 1)):
        g.replay()
    torch.cuda.synchronize()


def graph_avg_us(torch, fn, n):
    """Average µs per fn() call over a HIP graph of n back-to-back calls (events on its stream)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    warm_graph(torch, g)        # untimed replays: graph upload and steady clocks
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n, g


def traffic_for(digest, nbytes_alg):
    """HBM bytes per launch of the dominant kernel from committed counter runs, if current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_digest") != digest:
        return None
    return t.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the GEMV has no multi-GPU path here)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synthetic
    import weight_only_int4_w4a16_amd as w

    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel(), "launches": 5}))
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    if args.profile_workload:
        profile_workload(torch, np, w, synthetic, dev, args.profile_workload, args.batch,
                         args.steps)
        return

    # ---- operands: seed 0 of the gate+up and down shapes, rotated copies on the device
    da = synthetic.config("c3a", 0)
    db = synthetic.config("c3b", 0)
    qa, sa, xa = to_dev(da, dev, torch, np)
    qb, sb, xb = to_dev(db, dev, torch, np)
    bytes_a = synthetic.algorithmic_bytes(da.N, da.K)
    bytes_b = synthetic.algorithmic_bytes(db.N, db.K)
    step_weight_bytes = qa.numel() * 4 + sa.numel() * 2 + qb.numel() * 4 + sb.numel() * 2
    R = max(2, -(-ROTATE_BYTES // step_weight_bytes))
    copies = list(zip(rotated(torch, qa, R), rotated(torch, sa, R), rotated(torch, qb, R),
                      rotated(torch, sb, R)))
    ya = torch.empty(da.N, dtype=torch.float32, device=dev)
    yb = torch.empty(db.N, dtype=torch.float32, device=dev)
    xa1, xb1 = xa[0], xb[0]

    def step(i):
        c = copies[i % R]
        w.gemv(c[0], c[1], xa1, out=ya)
        w.gemv(c[2], c[3], xb1, out=yb)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps in one graph
    step_us, _ = graph_avg_us(torch, step, args.steps)
    ms_per_step = step_us / 1e3
    value = (bytes_a + bytes_b) / (step_us * 1e-6) / 1e9

    # ---- dominant kernel alone (28672 x 4096), same rotation, same timing method
    gate_us, _ = graph_avg_us(torch, lambda i: w.gemv(copies[i % R][0], copies[i % R][1], xa1,
                                                       out=ya), args.steps)
    down_us, _ = graph_avg_us(torch, lambda i: w.gemv(copies[i % R][2], copies[i % R][3], xb1,
                                                       out=yb), args.steps)
    # ---- launch floor: the same graph timing for back-to-back launches of a kernel that reads
    # one 16-byte chunk (the streaming-read kernel, one work-group per CU). Every call above
    # pays this per-launch cost of the command processor (dispatch, completion and the cache
    # operations between dependent kernels) on top of its memory time.
    fbuf = torch.zeros(16, dtype=torch.uint8, device=dev)
    fout = torch.empty(4 * props.multi_processor_count, dtype=torch.int32, device=dev)
    floor_us, _ = graph_avg_us(torch, lambda i: w.stream_read(
        fbuf, 16, fout, props.multi_processor_count, 1), args.steps)
    achieved = bytes_a / (gate_us * 1e-6) / 1e9
    plan_a = w.describe_plan(1, da.N, da.K, 0, props.multi_processor_count)
    digest = kernel_source_digest(plan_a)
    traffic = traffic_for(digest, bytes_a)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded int4 weights uniform in [-8,7], fp16 scales uniform in "
                "[0.001,0.01], bf16 activations ~N(0,1))",
        "config": {
            "workload": "MLP GEMV pair at M=1: 28672x4096 gate+up then 4096x14336 down, "
                        "int4 weights (8 per uint32 along K), fp16 scale per 128-group, bf16 x",
            "M": 1,
            "shapes": [[da.N, da.K], [db.N, db.K]],
            "bytes_per_step": bytes_a + bytes_b,
            "rotated_weight_copies": R,
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "us_per_call": {"gate_up_28672x4096": round(gate_us, 3),
                            "down_4096x14336": round(down_us, 3)},
            "plans": {"gate_up": plan_a,
                      "down": w.describe_plan(1, db.N, db.K, 0, props.multi_processor_count)},
            "device": f"{props.name} {getattr(props, 'gcnArchName', '')} "
                      f"{props.multi_processor_count} CUs",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "w4a16_gemv 28672x4096",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_a,
            "avg_launch_us": round(gate_us, 3),
            "launch_floor_us": round(floor_us, 3),
            "kernel_source_digest": digest,
        },
    }

    if not args.no_configs:
        out["per_workload"] = per_workload(torch, np, w, synthetic, dev,
                                           props.multi_processor_count,
                                           with_oracle=not args.no_cpu_baseline)
        ref = out["per_workload"]["c3a_M1"]
        if "stream_read_us" in ref:
            # the plain streaming read of the same bytes, the practical ceiling of this kernel
            out["roofline"]["stream_read_us_same_bytes"] = ref["stream_read_us"]
            out["roofline"]["frac_of_stream_read"] = round(ref["stream_read_us"] / gate_us, 4)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(da, db, bytes_a + bytes_b, args.cpu_seconds)

    print(json.dumps(out), flush=True)


def graph_replay_stats(torch, fn, n, reps):
    """Per-call µs over `reps` replays of a graph of n back-to-back calls: (median, p10, p90)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    warm_graph(torch, g)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        g.replay()
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[r].elapsed_time(ev[r + 1]) * 1e3 / n for r in range(reps))

    def q(f):
        return per[min(reps - 1, int(round(f * (reps - 1))))]
    return q(0.5), q(0.1), q(0.9)


def stream_ceiling_us(torch, w, dev, nbytes, R, cus):
    """Best median µs of the plain streaming-read kernel over R rotated slices of nbytes."""
    nb = -(-nbytes // 256) * 256
    buf = torch.empty(R * nb, dtype=torch.uint8, device=dev).fill_(1)
    best = None
    for bpc in (1, 2, 4, 8, 16):
        blocks = cus * bpc
        out = torch.empty(blocks * 4, dtype=torch.int32, device=dev)
        for unroll in (2, 4, 8):
            def fn(i, blocks=blocks, unroll=unroll, out=out):
                w.stream_read(buf[(i % R) * nb:], nbytes - nbytes % 16, out, blocks, unroll)
            fn(0)
            med, _, _ = graph_replay_stats(torch, fn, max(2 * R, 64), 5)
            if best is None or med < best[0]:
                best = (med, blocks, unroll)
    del buf
    torch.cuda.empty_cache()
    return best


def rotations(nbytes):
    """Copies of an nbytes operand that together exceed the memory-side cache (>= 1 GiB)."""
    return max(2, -(-ROTATE_BYTES // max(1, nbytes)))


def copy_ceiling_us(torch, dev, nbytes_total):
    """Median µs of the runtime's device-to-device copy that reads and writes nbytes_total / 2
    bytes each (rotated sources, graph-timed): the practical ceiling of a call that moves
    nbytes_total bytes of mixed reads and writes."""
    half = nbytes_total // 2 // 256 * 256
    R = rotations(half)
    src = torch.empty(R * half, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(half, dtype=torch.uint8, device=dev)

    def fn(i):
        j = i % R
        dst.copy_(src[j * half:(j + 1) * half])
    fn(0)
    med, _, _ = graph_replay_stats(torch, fn, max(2 * R, 16), 5)
    del src, dst
    torch.cuda.empty_cache()
    return med


def single_call_us(torch, call, reps=21):
    """Median µs of one eager call between two events, synchronising after each (latency
    context: includes the launch, unlike the graph-timed numbers)."""
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    return sorted(times)[reps // 2]


def per_workload(torch, np, w, synthetic, dev, cus, with_oracle=False):
    """µs per call and GB/s for every workload shape (graph-timed, rotated copies), with the
    same call on one cache-resident copy and the plain streaming-read ceiling over the same
    number of bytes, rotated the same way."""
    res = {}

    def rot(nbytes):
        return max(2, -(-ROTATE_BYTES // nbytes))

    def record(key, N, K, M, b, stats, warm, ceil, plan):
        med, p10, p90 = stats
        e = {"N": N, "K": K, "M": M, "plan": plan, "us_per_call": round(med, 3),
             "us_p10": round(p10, 3), "us_p90": round(p90, 3),
             "GB_s": round(b / med / 1e3, 1),
             "pct_of_peak": round(100 * b / med / 1e3 / HBM_PEAK_GBS, 1),
             "us_cache_warm_same_copy": round(warm, 3)}
        if ceil is not None:
            e["stream_read_us"] = round(ceil[0], 3)
            e["stream_read_launch"] = {"blocks": ceil[1], "unroll": ceil[2]}
            e["pct_of_stream_read"] = round(100 * ceil[0] / med, 1)
        res[key] = e

    ceilings = {}
    for name in ("c1", "c2", "c3a", "c3b", "c5a", "c5b"):
        for M in ((1, 2, 4, 8, 16) if name in ("c5a", "c5b") else (1,)):
            d = synthetic.config(name, 0, M=M)
            qw, sc, x = to_dev(d, dev, torch, np)
            R = rot(qw.numel() * 4 + sc.numel() * 2)
            cp = list(zip(rotated(torch, qw, R), rotated(torch, sc, R)))
            del qw, sc
            y = torch.empty((M, d.N), dtype=torch.float32, device=dev)
            if M == 1:
                def fn(i, cp=cp, x=x, y=y, R=R):
                    w.gemv(cp[i % R][0], cp[i % R][1], x[0], out=y[0])
            else:
                def fn(i, cp=cp, x=x, y=y, R=R):
                    w.gemv_batched(cp[i % R][0], cp[i % R][1], x, out=y)
            fn(0)
            n = max(2 * R, 64)
            stats = graph_replay_stats(torch, fn, n, 10)
            warm, _, _ = graph_replay_stats(torch, lambda i: fn(0), 64, 5)
            single = single_call_us(torch, lambda: fn(0))
            b = synthetic.algorithmic_bytes(d.N, d.K, M)
            del cp
            torch.cuda.empty_cache()
            if b not in ceilings:
                ceilings[b] = stream_ceiling_us(torch, w, dev, b, rot(b), cus)
            record(f"{name}_M{M}", d.N, d.K, M, b, stats, warm, ceilings[b],
                   w.describe_plan(M, d.N, d.K, 0, cus))
            res[f"{name}_M{M}"]["us_single_call_not_graphed"] = round(single, 3)
            if with_oracle:
                ous = oracle_us(d, M, rows=512)
                res[f"{name}_M{M}"]["oracle_us_1_core"] = round(ous, 1)
                res[f"{name}_M{M}"]["oracle_GB_s"] = round(b / ous / 1e3, 4)
    m = synthetic.config("c4", 0)
    qw = torch.from_numpy(m.qweight.view(np.int32)).to(dev)
    sc = torch.from_numpy(m.scales.view(np.float16)).to(dev)
    cp = list(zip(rotated(torch, qw, 2), rotated(torch, sc, 2)))
    del qw, sc
    x = torch.from_numpy(m.x.view(np.int16)).to(dev).view(torch.bfloat16)
    rng = np.random.default_rng([4, 1])
    idsets = [torch.from_numpy(rng.choice(m.E, m.topk, replace=False).astype(np.int32)).to(dev)
              for _ in range(64)]
    y = torch.empty((m.topk, m.N), dtype=torch.float32, device=dev)

    def fn(i):
        w.moe_gemv(cp[i % 2][0], cp[i % 2][1], idsets[i % 64], x, out=y)
    fn(0)
    stats = graph_replay_stats(torch, fn, 128, 10)
    warm, _, _ = graph_replay_stats(torch, lambda i: w.moe_gemv(cp[0][0], cp[0][1], idsets[0], x,
                                                                out=y), 64, 5)
    b = m.topk * (m.N * m.K // 2 + m.N * (m.K // 128) * 2) + m.K * 2
    del cp
    torch.cuda.empty_cache()
    record("c4_moe_top8_of_256", m.N, m.K, 1, b, stats, warm,
           stream_ceiling_us(torch, w, dev, b, rot(b), cus),
           w.describe_plan(1, m.N, m.K, m.topk, cus))
    del m, x, y, idsets
    torch.cuda.empty_cache()
    res["c4_expert_tail_top8_of_256"] = expert_tail(torch, np, w, synthetic, dev, cus)
    res["quantize_pack_28672x4096"] = quantize_rate(torch, np, w, dev)
    res.update(moe_batched(torch, np, w, synthetic, dev, cus))
    return res


def moe_batched(torch, np, w, synthetic, dev, cus):
    """The c4 experts (256 of 2048 x 2304) for M tokens decoded together, each with its own
    top-8: every selected expert is read once. Bytes count each selected expert once (the mean
    over the 64 id sets used) plus the M activation rows."""
    m = synthetic.config("c4", 0)
    qw = torch.from_numpy(m.qweight.view(np.int32)).to(dev)
    sc = torch.from_numpy(m.scales.view(np.float16)).to(dev)
    cp = list(zip(rotated(torch, qw, 2), rotated(torch, sc, 2)))
    del qw, sc
    per_expert = m.N * m.K // 2 + m.N * (m.K // 128) * 2
    out = {}
    for M in (2, 4, 8, 16):
        rng = np.random.default_rng([4, 2, M])
        sets = [np.stack([rng.choice(m.E, m.topk, replace=False) for _ in range(M)])
                .astype(np.int32) for _ in range(64)]
        uniq = float(np.mean([len(np.unique(s_)) for s_ in sets]))
        idsets = [torch.from_numpy(s_).to(dev) for s_ in sets]
        X = torch.from_numpy(synthetic.draw_acts(rng, (M, m.K)).view(np.int16)).to(dev)
        X = X.view(torch.bfloat16)
        Y = torch.empty((M, m.topk, m.N), dtype=torch.float32, device=dev)

        def fn(i, idsets=idsets, X=X, Y=Y):
            w.moe_gemv_batched(cp[i % 2][0], cp[i % 2][1], idsets[i % 64], X, out=Y)
        fn(0)
        med, p10, p90 = graph_replay_stats(torch, fn, 128, 10)
        b = uniq * per_expert + M * m.K * 2
        ceil = stream_ceiling_us(torch, w, dev, int(b), rotations(int(b)), cus)
        out[f"c4_moe_batched_M{M}"] = {
            "experts": m.E, "topk": m.topk, "N": m.N, "K": m.K, "M": M,
            "mean_unique_experts": round(uniq, 2),
            "plan": w.describe_moe_batched_plan(M, m.N, m.K, m.topk, cus),
            "us_per_call": round(med, 3), "us_p10": round(p10, 3), "us_p90": round(p90, 3),
            "GB_s": round(b / med / 1e3, 1), "pct_of_peak": round(100 * b / med / 1e3 / HBM_PEAK_GBS, 1),
            "stream_read_us": round(ceil[0], 3), "pct_of_stream_read": round(100 * ceil[0] / med, 1)}
    del cp
    torch.cuda.empty_cache()
    return out


def quantize_rate(torch, np, w, dev):
    """bf16 -> packed INT4 for the 28672 x 4096 gate+up matrix: reads 2 bytes and writes
    0.5 + 1/64 bytes per weight. Four rotated input copies (940 MB) so reads come from HBM."""
    N, K = 28672, 4096
    g = torch.Generator(device="cpu").manual_seed(0)
    src = (torch.randn((N, K), generator=g) * 0.02).to(torch.bfloat16).to(dev)
    R = 4
    copies = rotated(torch, src, R)
    del src
    qw = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    sc = torch.empty((N, K // 128), dtype=torch.float16, device=dev)
    fn = lambda i: w.quantize_pack(copies[i % R], out=(qw, sc))  # noqa: E731
    fn(0)
    med, p10, p90 = graph_replay_stats(torch, fn, 16, 5)
    b = 2 * N * K + N * K // 2 + N * (K // 128) * 2
    del copies
    torch.cuda.empty_cache()
    copy_us = copy_ceiling_us(torch, dev, b)
    return {"N": N, "K": K, "bytes": b, "us_per_call": round(med, 3), "us_p10": round(p10, 3),
            "us_p90": round(p90, 3), "GB_s": round(b / med / 1e3, 1),
            "pct_of_peak": round(100 * b / med / 1e3 / HBM_PEAK_GBS, 1),
            "copy_us_same_bytes": round(copy_us, 3),
            "pct_of_copy": round(100 * copy_us / med, 1)}


def tail_bytes(d):
    """Algorithmic bytes of the expert tail: the selected gate+up and down experts (packed weights
    and scales), x, and h read by the down step (h written as bf16 is an output)."""
    gu = 2 * d.I * d.K // 2 + 2 * d.I * (d.K // 128) * 2
    dn = d.H * d.I // 2 + d.H * (d.I // 128) * 2
    return d.topk * (gu + dn) + d.K * 2 + d.topk * d.I * 2


def expert_tail(torch, np, w, synthetic, dev, cus):
    """The MoE expert tail for one token: SwiGLU gate+up over the selected experts, then the
    grouped down projection with the router-weighted sum. Two copies of every expert tensor and
    64 id sets drawn from the seeded stream, so consecutive calls read different experts."""
    d = synthetic.tail_config(0)
    qg = torch.from_numpy(d.gu_qweight.view(np.int32)).to(dev)
    sg = torch.from_numpy(d.gu_scales.view(np.float16)).to(dev)
    qd = torch.from_numpy(d.down_qweight.view(np.int32)).to(dev)
    sd = torch.from_numpy(d.down_scales.view(np.float16)).to(dev)
    cp = list(zip(rotated(torch, qg, 2), rotated(torch, sg, 2), rotated(torch, qd, 2),
                  rotated(torch, sd, 2)))
    del qg, sg, qd, sd
    x = torch.from_numpy(d.x.view(np.int16)).to(dev).view(torch.bfloat16)
    rw = torch.from_numpy(d.route_w).to(dev)
    rng = np.random.default_rng([41, 1])
    idsets = [torch.from_numpy(rng.choice(d.E, d.topk, replace=False).astype(np.int32)).to(dev)
              for _ in range(64)]
    h = torch.empty((d.topk, d.I), dtype=torch.bfloat16, device=dev)
    out = torch.empty(d.H, dtype=torch.float32, device=dev)

    def fn(i):
        c, ids = cp[i % 2], idsets[i % 64]
        w.moe_gemv_swiglu(c[0], c[1], ids, x, out=h)
        w.moe_down_combine(c[2], c[3], ids, rw, h, out=out)

    def gate(i):
        c, ids = cp[i % 2], idsets[i % 64]
        w.moe_gemv_swiglu(c[0], c[1], ids, x, out=h)

    def down(i):
        c, ids = cp[i % 2], idsets[i % 64]
        w.moe_down_combine(c[2], c[3], ids, rw, h, out=out)
    fn(0)
    med, p10, p90 = graph_replay_stats(torch, fn, 128, 10)
    g_us, _, _ = graph_replay_stats(torch, gate, 128, 5)
    d_us, _, _ = graph_replay_stats(torch, down, 128, 5)
    b = tail_bytes(d)
    b_gu = d.topk * (2 * d.I * d.K // 2 + 2 * d.I * (d.K // 128) * 2) + d.K * 2
    ceil_us = (stream_ceiling_us(torch, w, dev, b_gu, rotations(b_gu), cus)[0] +
               stream_ceiling_us(torch, w, dev, b - b_gu, rotations(b - b_gu), cus)[0])
    e = {"experts": d.E, "topk": d.topk, "gate_up": [2 * d.I, d.K], "down": [d.H, d.I],
         "plans": {"swiglu": w.describe_tail_plan(0, 0, d.K, d.I, d.topk, cus),
                   "down_combine": w.describe_tail_plan(1, d.H, 0, d.I, d.topk, cus)},
         "bytes": b, "us_per_call": round(med, 3), "us_p10": round(p10, 3),
         "us_p90": round(p90, 3), "us_swiglu": round(g_us, 3), "us_down_combine": round(d_us, 3),
         "GB_s": round(b / med / 1e3, 1),
         "pct_of_peak": round(100 * b / med / 1e3 / HBM_PEAK_GBS, 1),
         "stream_read_us_two_launches": round(ceil_us, 3),
         "pct_of_stream_read": round(100 * ceil_us / med, 1)}
    del cp
    torch.cuda.empty_cache()
    return e


def profile_workload(torch, np, w, synthetic, dev, name, M, steps):
    """Launch one workload's GEMV `steps` times on rotated copies (no timing): a fixed command
    for rocprofv3 counter and trace runs."""
    if name == "c4":
        m = synthetic.config("c4", 0)
        qw = torch.from_numpy(m.qweight.view(np.int32)).to(dev)
        sc = torch.from_numpy(m.scales.view(np.float16)).to(dev)
        cp = list(zip(rotated(torch, qw, 2), rotated(torch, sc, 2)))
        del qw, sc
        if M == 1:
            x = torch.from_numpy(m.x.view(np.int16)).to(dev).view(torch.bfloat16)
            ids = torch.from_numpy(m.ids).to(dev)
            y = torch.empty((m.topk, m.N), dtype=torch.float32, device=dev)
            for i in range(steps):
                w.moe_gemv(cp[i % 2][0], cp[i % 2][1], ids, x, out=y)
            plan = w.describe_plan(1, m.N, m.K, m.topk)
        else:
            # M tokens with their own top-8 (one id set, the same as the bench's first)
            rng = np.random.default_rng([4, 2, M])
            idn = np.stack([rng.choice(m.E, m.topk, replace=False) for _ in range(M)])
            ids = torch.from_numpy(idn.astype(np.int32)).to(dev)
            X = torch.from_numpy(synthetic.draw_acts(rng, (M, m.K)).view(np.int16)).to(dev)
            X = X.view(torch.bfloat16)
            Y = torch.empty((M, m.topk, m.N), dtype=torch.float32, device=dev)
            for i in range(steps):
                w.moe_gemv_batched(cp[i % 2][0], cp[i % 2][1], ids, X, out=Y)
            plan = (w.describe_moe_batched_plan(M, m.N, m.K, m.topk) +
                    f" unique_experts={len(np.unique(idn))}")
    else:
        d = synthetic.config(name, 0, M=M)
        qw, sc, x = to_dev(d, dev, torch, np)
        R = max(2, -(-ROTATE_BYTES // (qw.numel() * 4 + sc.numel() * 2)))
        cp = list(zip(rotated(torch, qw, R), rotated(torch, sc, R)))
        y = torch.empty((M, d.N), dtype=torch.float32, device=dev)
        for i in range(steps):
            if M == 1:
                w.gemv(cp[i % R][0], cp[i % R][1], x[0], out=y[0])
            else:
                w.gemv_batched(cp[i % R][0], cp[i % R][1], x, out=y)
        plan = w.describe_plan(M, d.N, d.K)
    torch.cuda.synchronize()
    print(json.dumps({"profile_workload": name, "M": M, "launches": steps, "plan": plan}))


def cpu_baseline(da, db, bytes_per_step, target_s):
    """The CPU oracle (one thread, float64) on whole steps of the same workload."""
    import oracle
    orc = oracle.default()
    steps, t0 = 0, time.perf_counter()
    while True:
        orc.gemv(da.qweight, da.scales, da.x[0], da.K)
        orc.gemv(db.qweight, db.scales, db.x[0], db.K)
        steps += 1
        el = time.perf_counter() - t0
        if el >= target_s or steps >= 8:
            break
    return {"value": round(bytes_per_step * steps / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{steps} whole steps (28672x4096 + 4096x14336 GEMV, every row), "
                      f"{el:.1f} s, single-threaded C oracle in float64",
            "ms_per_step": round(el / steps * 1e3, 1),
            "host": host_description()}


def host_description():
    """CPU model and the number of cores the process may use (the oracle uses one)."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count()
    return {"cpu": model, "cores_available": avail}


def oracle_us(d, M, rows):
    """µs of the CPU oracle for one call of workload d, timed on a row sample and scaled."""
    import numpy as np
    import oracle
    orc = oracle.default()
    sample = np.arange(0, d.N, max(1, d.N // rows))
    t0 = time.perf_counter()
    if M == 1:
        orc.gemv(d.qweight, d.scales, d.x[0], d.K, rows=sample)
    else:
        orc.gemv_batched(d.qweight, d.scales, d.x, d.K, rows=sample)
    return (time.perf_counter() - t0) * 1e6 * d.N / sample.size


if __name__ == "__main__":
    main()
