"""W4A16 decode GEMV benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]

Workload (the headline): the largest single-GPU configuration, a wide output-head GEMV at M = 1
(one decode token), N = 163840 rows by K = 2304, INT4 weights packed 8 per uint32 along K, one
fp16 scale per 128-wide group, bf16 activations, fp32 output; seeded synthetic operands. One
step is one call. The weights rotate through enough copies (6 x 195 MB) that the 256 MB
memory-side cache cannot hold them, so every call streams its weights from HBM. The K timed
steps are captured in one HIP graph, replayed once between two HIP events on the launch stream,
with device synchronisation on both sides.

Prints one JSON line (last on stdout). `value` is algorithmic bytes (packed weights + fp16
scales + bf16 activations) per second, in GB/s. `roofline` is for the headline kernel: the same
bytes over its own average launch duration, timed on a graph of back-to-back launches, against
8 TB/s, with the plain streaming read of the same bytes as the practical ceiling and the
per-launch time of a kernel that reads 16 bytes (`launch_floor_us`). `config.mlp_pair` is the
MLP-shaped pair at M = 1 (28672 x 4096 gate+up then 4096 x 14336 down). `per_workload` holds,
for every other configuration, [us per call, % of 8 TB/s, % of the streaming-read ceiling] (the
legend is in `per_workload_fields`); the launch plans are printed to stderr. `cpu_baseline` is
the CPU oracle (single thread, float64) timed on whole calls of the headline workload.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_163840x2304.json")
HEADLINE = "c5b"
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
                    choices=["c1", "c2", "c3a", "c3b", "c4", "c4_3bit", "c5a", "c5b"],
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

    cus = props.multi_processor_count

    # ---- headline operands: seed 0 of the 163840 x 2304 head, rotated copies on the device
    dh = synthetic.config(HEADLINE, 0)
    qh, sh, xh = to_dev(dh, dev, torch, np)
    bytes_h = synthetic.algorithmic_bytes(dh.N, dh.K)
    R = max(2, -(-ROTATE_BYTES // (qh.numel() * 4 + sh.numel() * 2)))
    hcopies = list(zip(rotated(torch, qh, R), rotated(torch, sh, R)))
    del qh, sh
    yh = torch.empty(dh.N, dtype=torch.float32, device=dev)
    xh1 = xh[0]

    def step(i):
        c = hcopies[i % R]
        w.gemv(c[0], c[1], xh1, out=yh)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps in one graph
    step_us, _ = graph_avg_us(torch, step, args.steps)
    ms_per_step = step_us / 1e3
    value = bytes_h / (step_us * 1e-6) / 1e9

    # ---- the headline kernel alone: back-to-back launches on the same rotation (a step is one
    # launch, so this repeats the measurement as the kernel's own average duration)
    head_us, _ = graph_avg_us(torch, step, args.steps)
    # ---- launch floor: the same graph timing for back-to-back launches of a kernel that reads
    # one 16-byte chunk (the streaming-read kernel, one work-group per CU). Every call pays this
    # per-launch cost of the command processor (dispatch, completion and the cache operations
    # between dependent kernels) on top of its memory time.
    fbuf = torch.zeros(16, dtype=torch.uint8, device=dev)
    fout = torch.empty(4 * cus, dtype=torch.int32, device=dev)
    floor_us, _ = graph_avg_us(torch, lambda i: w.stream_read(fbuf, 16, fout, cus, 1), args.steps)
    ceil_us = stream_ceiling_us(torch, w, dev, bytes_h, rotations(bytes_h), cus)[0]
    achieved = bytes_h / (head_us * 1e-6) / 1e9
    plan_h = w.describe_plan(1, dh.N, dh.K, 0, cus)
    digest = kernel_source_digest(plan_h)
    traffic = traffic_for(digest, bytes_h)
    del hcopies
    torch.cuda.empty_cache()

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
        "data": "synthetic: seeded int4 codes uniform in [-8,7], fp16 scales in [0.001,0.01], "
                "bf16 x ~N(0,1)",
        "config": {
            "workload": "W4A16 GEMV, M=1, output head 163840x2304 (int4 8 per uint32 along K, "
                        "fp16 scale per 128-group, bf16 x, fp32 y)",
            "M": 1,
            "shape": [dh.N, dh.K],
            "bytes_per_call": bytes_h,
            "us_per_call": round(step_us, 3),
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "device": f"{getattr(props, 'gcnArchName', props.name).split(':')[0]}, {cus} CUs",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "w4a16_gemv 163840x2304",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_h,
            "avg_launch_us": round(head_us, 3),
            "stream_read_us_same_bytes": round(ceil_us, 3),
            "frac_of_stream_read": round(ceil_us / head_us, 4),
            "launch_floor_us": round(floor_us, 3),
            "kernel_source_digest": digest,
        },
    }
    plans = {"c5b_M1": plan_h}
    out["config"]["mlp_pair"] = mlp_pair(torch, np, w, synthetic, dev, cus, args.steps, plans)

    if not args.no_configs:
        out["per_workload_fields"] = ["us_per_call", "pct_of_hbm_peak", "pct_of_stream_read"]
        out["per_workload"] = per_workload(torch, np, w, synthetic, dev, cus, plans)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(dh, bytes_h, args.cpu_seconds)

    for k, v in plans.items():
        print(f"plan {k}: {v}", file=sys.stderr, flush=True)
    print(json.dumps(out, separators=(",", ":")), flush=True)


def mlp_pair(torch, np, w, synthetic, dev, cus, steps, plans):
    """The MLP-shaped GEMV pair at M = 1 (28672 x 4096 gate+up then 4096 x 14336 down), graph-
    timed on rotated copies: µs per pair and per call, and % of 8 TB/s of the pair."""
    da = synthetic.config("c3a", 0)
    db = synthetic.config("c3b", 0)
    qa, sa, xa = to_dev(da, dev, torch, np)
    qb, sb, xb = to_dev(db, dev, torch, np)
    ba = synthetic.algorithmic_bytes(da.N, da.K)
    bb = synthetic.algorithmic_bytes(db.N, db.K)
    wbytes = qa.numel() * 4 + sa.numel() * 2 + qb.numel() * 4 + sb.numel() * 2
    R = max(2, -(-ROTATE_BYTES // wbytes))
    cp = list(zip(rotated(torch, qa, R), rotated(torch, sa, R), rotated(torch, qb, R),
                  rotated(torch, sb, R)))
    del qa, sa, qb, sb
    ya = torch.empty(da.N, dtype=torch.float32, device=dev)
    yb = torch.empty(db.N, dtype=torch.float32, device=dev)

    def pair(i):
        c = cp[i % R]
        w.gemv(c[0], c[1], xa[0], out=ya)
        w.gemv(c[2], c[3], xb[0], out=yb)
    pair(0)
    pair_us, _ = graph_avg_us(torch, pair, steps)
    a_us, _ = graph_avg_us(torch, lambda i: w.gemv(cp[i % R][0], cp[i % R][1], xa[0], out=ya),
                           steps)
    b_us, _ = graph_avg_us(torch, lambda i: w.gemv(cp[i % R][2], cp[i % R][3], xb[0], out=yb),
                           steps)
    plans["c3a_M1"] = w.describe_plan(1, da.N, da.K, 0, cus)
    plans["c3b_M1"] = w.describe_plan(1, db.N, db.K, 0, cus)
    del cp
    torch.cuda.empty_cache()
    return {"us_per_pair": round(pair_us, 3), "us_28672x4096": round(a_us, 3),
            "us_4096x14336": round(b_us, 3),
            "pct_of_hbm_peak": round(100 * (ba + bb) / pair_us / 1e3 / HBM_PEAK_GBS, 2)}


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


def per_workload(torch, np, w, synthetic, dev, cus, plans):
    """[µs per call, % of 8 TB/s, % of the streaming-read ceiling] for every other workload
    (graph-timed median over 10 replays, rotated copies); the streaming read covers the same
    number of bytes, rotated the same way (two reads, one per launch, for the expert tail; a
    device-to-device copy of the same total bytes for quantise)."""
    res = {}

    def rot(nbytes):
        return max(2, -(-ROTATE_BYTES // nbytes))

    def record(key, b, med, ceil_us):
        res[key] = [round(med, 2), round(100 * b / med / 1e3 / HBM_PEAK_GBS, 1),
                    round(100 * ceil_us / med, 1)]

    ceilings = {}
    for name in ("c1", "c2", "c3a", "c3b", "c5a", "c5b"):
        for M in ((1, 2, 4, 8, 16) if name in ("c5a", "c5b") else (1,)):
            if name in ("c3a", "c3b", "c5b") and M == 1:
                continue            # the headline and the MLP pair are timed above
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
            med, _, _ = graph_replay_stats(torch, fn, max(2 * R, 64), 10)
            b = synthetic.algorithmic_bytes(d.N, d.K, M)
            del cp
            torch.cuda.empty_cache()
            if b not in ceilings:
                ceilings[b] = stream_ceiling_us(torch, w, dev, b, rot(b), cus)[0]
            record(f"{name}_M{M}", b, med, ceilings[b])
            plans[f"{name}_M{M}"] = w.describe_plan(M, d.N, d.K, 0, cus)
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
    med, _, _ = graph_replay_stats(torch, fn, 128, 10)
    b = m.topk * (m.N * m.K // 2 + m.N * (m.K // 128) * 2) + m.K * 2
    del cp
    torch.cuda.empty_cache()
    record("c4_moe_top8_of_256", b, med, stream_ceiling_us(torch, w, dev, b, rot(b), cus)[0])
    plans["c4_moe_top8_of_256"] = w.describe_plan(1, m.N, m.K, m.topk, cus)
    del m, x, y, idsets
    torch.cuda.empty_cache()
    b, med, ceil_us, plan = moe_three_bit(torch, np, w, synthetic, dev, cus)
    record("c4_moe3_top8_of_256", b, med, ceil_us)
    plans["c4_moe3_top8_of_256"] = plan
    for k, (b, med, ceil_us, plan) in expert_tail(torch, np, w, synthetic, dev, cus).items():
        record(k, b, med, ceil_us)
        plans[k] = plan
    for k, (b, med, ceil_us, plan) in moe_batched(torch, np, w, synthetic, dev, cus).items():
        record(k, b, med, ceil_us)
        plans[k] = plan
    b, med, copy_us = quantize_rate(torch, np, w, dev)
    record("quantize_pack_28672x4096", b, med, copy_us)
    return res


def moe_three_bit(torch, np, w, synthetic, dev, cus):
    """The c4 experts (256 of 2048 x 2304) as three-bit codes, one token, top-8 (64 id sets
    rotated, two copies of the experts)."""
    cid, N, K = synthetic.SHAPES["c4"]
    m = synthetic.moe3(synthetic.MOE_EXPERTS, N, K, synthetic.MOE_TOPK, 0, config_id=cid)
    qw = torch.from_numpy(m.qweight.view(np.int32)).to(dev)
    sc = torch.from_numpy(m.scales.view(np.float16)).to(dev)
    cp = list(zip(rotated(torch, qw, 2), rotated(torch, sc, 2)))
    del qw, sc
    x = torch.from_numpy(m.x.view(np.int16)).to(dev).view(torch.bfloat16)
    rng = np.random.default_rng([4, 3])
    idsets = [torch.from_numpy(rng.choice(m.E, m.topk, replace=False).astype(np.int32)).to(dev)
              for _ in range(64)]
    y = torch.empty((m.topk, N), dtype=torch.float32, device=dev)

    def fn(i):
        w.moe_gemv3(cp[i % 2][0], cp[i % 2][1], idsets[i % 64], x, out=y)
    fn(0)
    med, _, _ = graph_replay_stats(torch, fn, 128, 10)
    b = synthetic.algorithmic_bytes3(N, K, m.topk)
    del cp
    torch.cuda.empty_cache()
    ceil_us = stream_ceiling_us(torch, w, dev, b, max(2, -(-ROTATE_BYTES // b)), cus)[0]
    return b, med, ceil_us, w.describe_moe3_plan(N, K, m.topk, cus)


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
        out[f"c4_moe_batched_M{M}"] = (
            b, med, ceil[0], w.describe_moe_batched_plan(M, m.N, m.K, m.topk, cus) +
            f" mean_unique_experts={uniq:.2f}")
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
    return b, med, copy_us


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
    plan = (f"swiglu: {w.describe_tail_plan(0, 0, d.K, d.I, d.topk, cus)}; down_combine: "
            f"{w.describe_tail_plan(1, d.H, 0, d.I, d.topk, cus)}; us {g_us:.2f} + {d_us:.2f}")
    del cp
    torch.cuda.empty_cache()
    return {"c4_expert_tail_top8_of_256": (b, med, ceil_us, plan)}


def profile_workload(torch, np, w, synthetic, dev, name, M, steps):
    """Launch one workload's GEMV `steps` times on rotated copies (no timing): a fixed command
    for rocprofv3 counter and trace runs."""
    if name == "c4_3bit":
        cid, N, K = synthetic.SHAPES["c4"]
        m = synthetic.moe3(synthetic.MOE_EXPERTS, N, K, synthetic.MOE_TOPK, 0, config_id=cid)
        qw = torch.from_numpy(m.qweight.view(np.int32)).to(dev)
        sc = torch.from_numpy(m.scales.view(np.float16)).to(dev)
        cp = list(zip(rotated(torch, qw, 2), rotated(torch, sc, 2)))
        del qw, sc
        x = torch.from_numpy(m.x.view(np.int16)).to(dev).view(torch.bfloat16)
        ids = torch.from_numpy(m.ids).to(dev)
        y = torch.empty((m.topk, N), dtype=torch.float32, device=dev)
        for i in range(steps):
            w.moe_gemv3(cp[i % 2][0], cp[i % 2][1], ids, x, out=y)
        plan = w.describe_moe3_plan(N, K, m.topk)
    elif name == "c4":
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


def cpu_baseline(d, bytes_per_call, target_s):
    """The CPU oracle (one thread, float64) on whole calls of the headline workload."""
    import oracle
    orc = oracle.default()
    calls, t0 = 0, time.perf_counter()
    while True:
        orc.gemv(d.qweight, d.scales, d.x[0], d.K)
        calls += 1
        el = time.perf_counter() - t0
        if el >= target_s or calls >= 16:
            break
    return {"value": round(bytes_per_call * calls / el / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{calls} whole calls of the {d.N}x{d.K} GEMV (every row), {el:.1f} s, "
                      f"one-thread C oracle, fp64",
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


if __name__ == "__main__":
    main()
