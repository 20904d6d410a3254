#!/usr/bin/env python3
"""Throughput of the fused-group executor and the tensor-fusion buckets on
one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
input.  The default workload (c5) is a 12-layer Transformer-block stack over
8192 tokens x hidden 1024, bf16 activations: per layer a LayerNorm (three
groups: row mean, row variance, normalise + affine), bias + GELU on
[8192, 4096] and dropout (keep 0.9) + residual on [8192, 1024]; then the
194 fp32 gradient tensors of such a model (151,156,736 elements) are packed
into 25 MiB buckets scaled by 1/8 and unpacked again.  Every layer has its
own buffers (~3 GB in all), so no step re-reads data the 256 MB Infinity
Cache could hold.

value = algorithmic bytes per step / time per step (GB/s), where the
algorithmic bytes count each distinct external input of a group read once
and each output written once, and 2 x payload for pack and for unpack.
The roofline entry is for the dominant kernel (most time per step), timed
with HIP events on the stream the kernels run on: one pair per step around
that kernel's block of back-to-back launches.  The
unfused baseline (one launch per op, intermediates stored) and the
per-tensor bucket baseline run the same data after the timed region.  The
CPU baseline times the oracle on a bounded sample of the same workload.

"groups" breaks the executor down per c5 group: its average launch time
(one event pair around its 12 back-to-back launches, three times), its
algorithmic bytes and GB/s against 8 TB/s, and, from the committed
SQ_INSTS_VALU summary of the same kernel sources, its VALU lane-instruction
rate against the non-packed fp32 issue peak (256 CUs x 4 SIMDs x 16 lanes x
2.4 GHz); "bound" names the larger fraction.

Other workloads (--workload c1..c4) rotate through enough buffer sets to
exceed 1 GiB, so the Infinity Cache cannot serve repeated reads.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused-group HBM GB/s (% of peak) + speedup vs unfused; bucket pack GB/s"
PEAK_GBS = 8000.0
# fp32 VALU issue peak without packed math (the kernels are compiled with
# packed fp32 off): 256 CUs x 4 SIMDs x 16 lanes per cycle x 2.4 GHz lane-instructions/s
VALU_PEAK = 256 * 4 * 16 * 2.4e9
ELEM = {"f32": 4, "bf16": 2, "u8": 1}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5", "joint", "ln", "search", "transpose",
                             "groups", "softmax", "ceiling"])
    ap.add_argument("--layers", type=int, default=12)
    ap.add_argument("--valu-from", metavar="VALU_CSV",
                    help="summarise a rocprofv3 SQ_INSTS_VALU/SQ_WAVES run of --workload groups "
                         "into profiles/valu_c5_groups.txt")
    ap.add_argument("--ln-variant", default="all",
                    choices=["all", "row_resident", "tvm_groups", "unfused", "shared_center",
                             "shared_center_duplicated"],
                    help="--workload ln or softmax: time only this variant (for per-kernel "
                         "profiles)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-baselines", action="store_true",
                    help="skip the unfused and per-tensor baselines")
    ap.add_argument("--trace-from", nargs=3, metavar=("STATS_CSV", "TRACE_CSV", "BENCH_JSON"),
                    help="summarise a rocprofv3 --kernel-trace --stats run of the workload (and the "
                         "bench line it printed) into profiles/<kernel>_<workload>.md and exit (no GPU)")
    ap.add_argument("--ceiling-from", metavar="BENCH_JSON",
                    help="summarise a --workload ceiling run's line into profiles/stream_ceiling.md "
                         "and exit (no GPU)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a c5 run into profiles/traffic_c5.txt and exit (no GPU)")
    return ap.parse_args()


# ------------------------------------------------------------ accounting
def group_bytes(graph, plan):
    """Algorithmic bytes of each group: every tensor the launch reads or
    writes in device memory, once."""
    out = []
    for g in range(plan.num_groups):
        b = 0
        for t in plan.group_tensors(g):
            d = graph.tensors[t]
            n = 1
            for s in d.shape:
                n *= s
            b += n * ELEM[d.dtype]
        out.append(b)
    return out


# ------------------------------------------------------------ device data
def make_tensor(torch, gen, d, kind, a, b):
    shape = tuple(d.shape)
    if d.dtype == "u8":
        u = torch.rand(shape, generator=gen, device="cuda")
        return (u >= a).to(torch.uint8)
    if kind == "normal":
        x = torch.randn(shape, generator=gen, device="cuda") * b + a
    else:
        x = torch.rand(shape, generator=gen, device="cuda") * (b - a) + a
    if d.dtype == "bf16":
        return x.to(torch.bfloat16).view(torch.int16)
    return x.float()


def alloc_graph(torch, gtf, graph, plan, gen, dists):
    bufs = {}
    for t in plan.materialized():
        d = graph.tensors[t]
        if d.role == "in":
            kind, a, b = dists[d.name]
            bufs[t] = make_tensor(torch, gen, d, kind, a, b)
        else:
            dt = {"f32": torch.float32, "bf16": torch.int16}[d.dtype]
            bufs[t] = torch.empty(tuple(d.shape), dtype=dt, device="cuda")
    return bufs


LN_D = {"X": ("normal", 0.0, 1.0), "gamma": ("normal", 1.0, 0.1), "beta": ("normal", 0.0, 0.1)}
GELU_D = {"A": ("normal", 0.0, 1.0), "b1": ("normal", 0.0, 0.1)}
DROP_D = {"h": ("normal", 0.0, 1.0), "mask": ("bernoulli", 0.1, 0.0), "R": ("normal", 0.0, 1.0)}


class Timer:
    """One event pair around a block of consecutive launches of one kernel,
    on the current stream (the stream the kernels are launched on).
    Back-to-back launches run without gaps, so block time / launches is the
    kernel's average duration; a pair around every single launch would add
    the marker and dispatch latency of each.  Events are created up front."""

    def __init__(self, torch, n_blocks):
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n_blocks)]
        self.i = 0
        self.launches = 0

    def block(self, fns):
        e0, e1 = self.ev[self.i]
        self.i += 1
        e0.record()
        for f in fns:
            f()
        e1.record()
        self.launches += len(fns)

    def total_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.ev[: self.i])

    @property
    def count(self):
        return self.launches


# ------------------------------------------------------------ c5 workload
class C5:
    def __init__(self, torch, gtf, configs, layers, fuse=True, seed=5000):
        self.torch, self.gtf = torch, gtf
        self.g_ln = configs.layernorm_graph()
        self.g_ge = configs.gelu_graph()
        self.g_do = configs.dropout_graph()
        self.p = {k: gtf.FusePlan(g, fuse=fuse) for k, g in
                  (("ln", self.g_ln), ("ge", self.g_ge), ("do", self.g_do))}
        gen = torch.Generator(device="cuda")
        self.layers = []
        for l in range(layers):
            gen.manual_seed(seed + l)
            self.layers.append({
                "ln": alloc_graph(torch, gtf, self.g_ln, self.p["ln"], gen, LN_D),
                "ge": alloc_graph(torch, gtf, self.g_ge, self.p["ge"], gen, GELU_D),
                "do": alloc_graph(torch, gtf, self.g_do, self.p["do"], gen, DROP_D)})
        numel = configs.c5_numel()
        self.bp = gtf.BucketPlan(numel, "f32", configs.BUCKET_CAP_BYTES)
        _, _, bn = self.bp.query()
        gen.manual_seed(configs.C5_GRAD_SEED)
        self.grads = [torch.randn(n, generator=gen, device="cuda") * 1e-3 for n in numel]
        self.buckets = [torch.empty(n, dtype=torch.float32, device="cuda") for n in bn]
        self.ws = torch.empty(max(16, self.bp.workspace_bytes), dtype=torch.uint8, device="cuda")
        self.bp.bind(self.ws)
        self.scale = configs.AVG_SCALE
        self.gbytes = {k: group_bytes(g, self.p[k]) for k, g in
                       (("ln", self.g_ln), ("ge", self.g_ge), ("do", self.g_do))}
        self.bucket_bytes = 2 * 4 * sum(numel)  # pack; unpack moves the same
        self.launches = layers * sum(p.num_groups for p in self.p.values()) + 2
        self.bind()

    def bytes_per_step(self):
        per_layer = sum(sum(v) for v in self.gbytes.values())
        return per_layer * len(self.layers) + 2 * self.bucket_bytes

    def exec_bytes_per_step(self):
        return sum(sum(v) for v in self.gbytes.values()) * len(self.layers)

    def bind(self):
        """Marshal every launch of a step once (pointer arrays, stream)."""
        self.exec_calls = []
        for L in self.layers:
            for k in ("ln", "ge", "do"):
                plan = self.p[k]
                self.exec_calls += [plan.launcher(g, L[k]) for g in range(plan.num_groups)]
        self.bucket_calls = [self.bp.launcher(False, self.grads, self.buckets, self.scale),
                             self.bp.launcher(True, self.grads, self.buckets, 1.0)]

    GROUP_NAMES = {"ln": ("ln_mean", "ln_var", "ln_normalise"), "ge": ("bias_gelu",),
                   "do": ("dropout_residual",)}

    def group_calls(self):
        """Per c5 group, its launch in every layer (marshalled once)."""
        out = {}
        for k in ("ln", "ge", "do"):
            plan = self.p[k]
            for g in range(plan.num_groups):
                out[self.GROUP_NAMES[k][g]] = ([plan.launcher(g, L[k]) for L in self.layers],
                                               self.gbytes[k][g])
        return out

    def step(self, exec_t=None, bucket_t=None, per_tensor=False):
        if per_tensor:
            for f in self.exec_calls:
                f()
            self.bp.pack_per_tensor(self.grads, self.buckets, self.scale)
            self.bp.unpack_per_tensor(self.buckets, self.grads, 1.0)
            return
        if exec_t is None:
            for f in self.exec_calls:
                f()
            for f in self.bucket_calls:
                f()
            return
        exec_t.block(self.exec_calls)
        bucket_t.block(self.bucket_calls)


class Timing:
    """Times of `steps` back-to-back steps: the mean (one event before the
    first and one after the last, the figure the whole-job throughput
    uses), the wall time of that timed region, and the distribution of
    per-step times from a second pass with an event between consecutive
    steps (each record puts a small gap in the stream, which matters only
    for launches of tens of microseconds)."""

    def __init__(self, mean, wall, per_step):
        import numpy as np
        self.mean, self.wall = mean, wall
        p = np.asarray(per_step, dtype=np.float64)
        self.median = float(np.median(p))
        self.p10 = float(np.percentile(p, 10))
        self.p90 = float(np.percentile(p, 90))

    def dist(self, scale=1.0, digits=5):
        """median, p10, p90 of the per-step times in ms (times `scale`)."""
        return {"median": round(self.median * scale, digits), "p10": round(self.p10 * scale, digits),
                "p90": round(self.p90 * scale, digits)}


def time_steps(torch, fn, steps, warmup, lead=None):
    """Mean, wall time and per-step times of `steps` calls of fn after
    `warmup` untimed ones.  lead: GPU work queued ahead of the first event
    (not timed), so the host enqueues the steps while the GPU is still busy
    and launches shorter than their host-side cost are not timed as gaps."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if lead is not None:
        lead()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = e0.elapsed_time(e1) / steps
    # the distribution: the same steps again, an event between each two
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    if lead is not None:
        lead()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return Timing(mean, wall, per)


# ------------------------------------------------------------ CPU baseline
def cpu_baseline_c5(target_s=12.0):
    """The oracle, as it is, on a bounded sample of the c5 workload: whole
    layers (LayerNorm, bias+GELU, dropout+residual at 8192 x 1024/4096, each
    layer with its own seed) until about target_s seconds of evaluation have
    passed, then one pack + unpack of all 194 gradient tensors.  Input
    generation is outside the timed spans."""
    import numpy as np
    from oracle import bucket as obucket
    from oracle import evaluate as oev
    from oracle import partition as opart
    from workloads import configs

    gl = [configs.layernorm_graph(), configs.gelu_graph(), configs.dropout_graph()]
    gen_in = [configs.layernorm_inputs, configs.gelu_inputs, configs.dropout_inputs]
    parts = [opart.partition(g) for g in gl]
    stored = [opart.stored_tensors(g, p) for g, p in zip(gl, parts)]
    layer_bytes = 0
    for g, part, st in zip(gl, parts, stored):
        for grp in part:
            produced = {g.ops[i].output for i in grp}
            ext = {t for i in grp for t in g.ops[i].inputs if t not in produced}
            ext |= {t for t in produced if t in st or g.tensors[t].role == "out"}
            layer_bytes += sum(int(np.prod(g.tensors[t].shape)) * ELEM[g.tensors[t].dtype]
                               for t in ext)
    dt, nbytes, layers = 0.0, 0, 0
    while layers < 12 and dt < target_s:
        seed = configs.c5_layer_seed(layers)
        ins = [f(g, seed) for f, g in zip(gen_in, gl)]
        t0 = time.perf_counter()
        for g, i, s, p in zip(gl, ins, stored, parts):
            oev.outputs(g, oev.evaluate(g, i, s, groups=p))
        dt += time.perf_counter() - t0
        nbytes += layer_bytes
        layers += 1
        del ins
    numel = configs.c5_numel()
    grads = configs.gradient_values(numel, configs.C5_GRAD_SEED)
    t0 = time.perf_counter()
    bks = obucket.pack(numel, 4, configs.BUCKET_CAP_BYTES, grads, configs.AVG_SCALE)
    obucket.unpack(numel, 4, configs.BUCKET_CAP_BYTES, bks, 1.0)
    dt += time.perf_counter() - t0
    nbytes += 2 * 2 * 4 * sum(numel)
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count()
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{layers} of 12 layers at full size (LayerNorm, bias+GELU, "
                      f"dropout+residual; 8192 tokens) plus pack+unpack of all 194 gradient "
                      f"tensors; {nbytes} algorithmic bytes in {dt:.1f} s; NumPy/SciPy "
                      f"single-threaded ({ncpu} cores visible)"}


# ------------------------------------------------------------ copy ceiling / lead
class CopyBench:
    """The library's plain dwordx4 copy kernel on 1 GiB: the achievable
    streaming ceiling, the reference for the traffic counters (it moves a
    known 1 GiB in and 1 GiB out), and a lead of queued GPU work that keeps
    the host ahead while launches are timed one by one."""
    NBYTES = 1 << 30

    def __init__(self, torch, gtf):
        self.torch, self.gtf = torch, gtf
        self.src = torch.empty(self.NBYTES, dtype=torch.uint8, device="cuda")
        self.src.random_(0, 256)
        self.dst = torch.empty_like(self.src)

    def run(self):
        self.gtf.device_copy(self.dst, self.src, self.NBYTES)

    def lead(self, n=12):
        for _ in range(n):
            self.run()

    def gbs(self, reps=10):
        self.run()
        ms = time_steps(self.torch, self.run, reps, 1).median
        return 2 * self.NBYTES / (ms * 1e-3) / 1e9, ms


# ------------------------------------------------------------ main
def main():
    args = parse()
    if args.traffic_from:
        print(json.dumps(summarise_traffic(*args.traffic_from, workload=args.workload)))
        return
    if args.valu_from:
        print(json.dumps(summarise_valu(args.valu_from, args.layers, args.workload)))
        return
    if args.trace_from:
        print(summarise_trace(*args.trace_from, workload=args.workload))
        return
    if args.ceiling_from:
        print(summarise_ceiling(args.ceiling_from))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the fused groups shard by rows with no exchange "
              "and the buckets would feed an all-reduce that is not part of this library; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import gradient_tensor_fusion_amd as gtf
    from workloads import configs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.workload == "groups":
        # each c5 group launched once per layer, group after group, nothing
        # else on the GPU: the dispatch order the VALU summary relies on
        w = C5(torch, gtf, configs, args.layers)
        torch.cuda.synchronize()
        for name, (calls, nbytes) in w.group_calls().items():
            for f in calls:
                f()
        torch.cuda.synchronize()
        print(json.dumps({"workload": "groups", "order": list(w.group_calls())}), flush=True)
        return
    if args.workload != "c5":
        print(json.dumps(run_config(torch, gtf, configs, args)), flush=True)
        return
    w = C5(torch, gtf, configs, args.layers)
    # timed region: K whole steps
    tm = time_steps(torch, w.step, args.steps, args.warmup)
    ms, wall = tm.mean, tm.wall
    step_bytes = w.bytes_per_step()
    value = step_bytes / (ms * 1e-3) / 1e9
    # per-kernel timing over a second pass of the same steps: per step, one
    # event pair around the executor launches and one around the bucket
    # launches; queued copies first put the GPU ahead of the host
    cb = CopyBench(torch, gtf)
    et = Timer(torch, args.steps)
    bt = Timer(torch, args.steps)
    torch.cuda.synchronize()
    cb.lead()
    for _ in range(args.steps):
        w.step(exec_t=et, bucket_t=bt)
    torch.cuda.synchronize()
    # per group: one event pair around its 12 back-to-back launches (one
    # per layer), three times, behind a queued lead
    groups = {}
    gt = Timer(torch, 3 * 5)
    torch.cuda.synchronize()
    cb.lead()
    for name, (calls, gbytes) in w.group_calls().items():
        t0 = gt.i
        for _ in range(3):
            gt.block(calls)
        groups[name] = (t0, len(calls), gbytes)
    torch.cuda.synchronize()
    valu = read_valu()
    group_rows = {}
    for name, (t0, n, gbytes) in groups.items():
        gms = sum(gt.ev[i][0].elapsed_time(gt.ev[i][1]) for i in range(t0, t0 + 3)) / (3 * n)
        row = {"avg_launch_us": round(gms * 1e3, 3), "bytes_per_launch": gbytes,
               "gbs": round(gbytes / (gms * 1e-3) / 1e9, 1),
               "hbm_frac": round(gbytes / (gms * 1e-3) / 1e9 / PEAK_GBS, 4)}
        if valu and name in valu:
            rate = valu[name] / (gms * 1e-3)
            row["valu_lane_instr_per_launch"] = valu[name]
            row["valu_frac"] = round(rate / VALU_PEAK, 4)
        row["bound"] = "alu" if row.get("valu_frac", 0) > row["hbm_frac"] else "hbm"
        group_rows[name] = row
    copy_gbs, copy_ms = cb.gbs()
    del cb
    exec_ms = et.total_ms() / args.steps
    bucket_ms = bt.total_ms() / args.steps
    exec_gbs = w.exec_bytes_per_step() / (exec_ms * 1e-3) / 1e9
    bucket_gbs = 2 * w.bucket_bytes / (bucket_ms * 1e-3) / 1e9
    n_exec = et.count // args.steps
    if exec_ms >= bucket_ms:
        dom = {"kernel": "exec_kernel", "launches_per_step": n_exec,
               "avg_launch_us": round(exec_ms * 1e3 / n_exec, 3),
               "bytes_per_launch": w.exec_bytes_per_step() / n_exec, "gbs": exec_gbs}
        # VALU issue fraction of the executor over the step: its lane
        # instructions per step (every group, every layer) over its time
        if valu and all(k in valu for k in group_rows):
            lanes = sum(valu[k] for k in group_rows) * len(w.layers)
            dom["valu_frac"] = lanes / (exec_ms * 1e-3) / VALU_PEAK
    else:
        dom = {"kernel": "bucket_kernel", "launches_per_step": 2,
               "avg_launch_us": round(bucket_ms * 1e3 / 2, 3),
               "bytes_per_launch": w.bucket_bytes, "gbs": bucket_gbs, "valu_frac": 0.0}
    hbm_frac = dom["gbs"] / PEAK_GBS
    # the roofline that binds is the larger of the two fractions (the
    # executor's VALU count comes from the committed counter summary; without
    # one for these sources the bound is not known)
    bound = None if "valu_frac" not in dom else ("alu" if dom["valu_frac"] > hbm_frac else "hbm")
    traffic = None
    tj = read_traffic(dom["kernel"])
    if tj is not None:
        traffic = tj["bytes_per_launch"]
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "c5: 12-layer Transformer-block fused groups (LayerNorm as 3 groups, "
                               "bias+GELU [8192,4096], dropout+residual [8192,1024]) over 8192 tokens "
                               "x hidden 1024, bf16 storage, + pack/unpack of 194 fp32 gradient "
                               "tensors (151,156,736 elements) in 25 MiB buckets, scale 1/8",
                   "layers": args.layers, "tokens": 8192, "hidden": 1024, "ffn": 4096,
                   "storage": "bf16 activations, fp32 gradients; fp32 arithmetic",
                   "bytes_per_step": step_bytes, "launches_per_step": w.launches},
        "step_ms": tm.dist(digits=4),
        "roofline": {"bound": bound, "achieved": round(dom["gbs"], 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(hbm_frac, 4),
                     "traffic": traffic, "kernel": dom["kernel"],
                     "avg_launch_us": dom["avg_launch_us"],
                     "algorithmic_bytes_per_launch": round(dom["bytes_per_launch"]),
                     "valu_frac": round(dom["valu_frac"], 4) if "valu_frac" in dom else None},
        "groups": group_rows,
        "breakdown": {"exec_ms_per_step": round(exec_ms, 4), "exec_gbs": round(exec_gbs, 1),
                      "bucket_ms_per_step": round(bucket_ms, 4), "bucket_gbs": round(bucket_gbs, 1),
                      "wall_s_timed": round(wall, 3),
                      "copy_kernel_gbs": round(copy_gbs, 1),
                      "copy_kernel_note": "library dwordx4 copy of 1 GiB: achievable ceiling"},
    }
    if not args.no_baselines:
        del w
        torch.cuda.empty_cache()
        u = C5(torch, gtf, configs, args.layers, fuse=False)
        ums = time_steps(torch, lambda: u.step(per_tensor=True), max(2, args.steps // 2), 1).mean
        n_grads = len([n for n in configs.c5_numel() if n])
        result["speedup_vs_unfused"] = round(ums / ms, 3)
        result["unfused"] = {"ms_per_step": round(ums, 4), "launches_per_step":
                             len(u.exec_calls) + 2 * n_grads,
                             "note": "one launch per op with bf16/fp32 intermediates stored; "
                                     "one pack and one unpack launch per gradient tensor"}
        del u
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_c5()
    print(json.dumps(result), flush=True)


# ------------------------------------------------------------ c1..c4
def _rotation_sets(set_bytes, floor=1 << 30, cap=64):
    k = 1
    while k * set_bytes < floor and k < cap:
        k += 1
    return k


def run_config(torch, gtf, configs, args):
    """One config on its own, with buffer rotation past the Infinity Cache;
    fused vs unfused (c1-c3) or one launch vs per-tensor launches (c4)."""
    w = args.workload
    res = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic"}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(int(w[1]) if w[1].isdigit() else 7)
    copy_gbs = lead = None
    if w in ("c1", "c2", "c3", "c4"):
        # the 1 GiB copy: the streaming ceiling beside the config, the
        # reference the traffic counters are scaled by, and the lead queued
        # ahead of each timed region
        cb = CopyBench(torch, gtf)
        copy_gbs = round(cb.gbs(5)[0], 1)
        lead = cb.lead
    if w == "c4":
        numel = configs.c4_numel()
        bp = gtf.BucketPlan(numel, "f32", configs.BUCKET_CAP_BYTES)
        _, _, bn = bp.query()
        ws = torch.empty(max(16, bp.workspace_bytes), dtype=torch.uint8, device="cuda")
        bp.bind(ws)
        payload = 4 * sum(numel)
        k = _rotation_sets(2 * payload)
        sets = [([torch.randn(n, generator=gen, device="cuda") * 1e-3 for n in numel],
                 [torch.empty(n, dtype=torch.float32, device="cuda") for n in bn]) for _ in range(k)]
        it = [0]
        # every launch marshalled once (pointer arrays for 161 tensors and
        # the buckets), so the timed loop is not bound by the host
        packs = [bp.launcher(False, g, b, configs.AVG_SCALE) for g, b in sets]
        unpacks = [bp.launcher(True, g, b, 1.0) for g, b in sets]

        def pack():
            packs[it[0] % k]()
            it[0] += 1

        def unpack():
            unpacks[it[0] % k]()
            it[0] += 1

        def pack_pt():
            g, b = sets[it[0] % k]
            it[0] += 1
            bp.pack_per_tensor(g, b, configs.AVG_SCALE)

        def warm_pack():
            packs[0]()
        # every rotation set is touched in the warmup, so none is first used
        # inside the timed region
        wu = max(args.warmup, k)
        tp = time_steps(torch, pack, 5 * args.steps, wu, lead)
        ms_p = tp.mean
        gbs = 2 * payload / (ms_p * 1e-3) / 1e9
        gb = lambda ms: round(2 * payload / (ms * 1e-3) / 1e9, 1)  # noqa: E731
        tj = read_traffic("bucket_kernel", "c4")
        res.update({"value": round(gbs, 2), "ms_per_step": round(ms_p, 4), "steps": 5 * args.steps,
                    "config": {"workload": "c4: pack 161 fp32 gradient tensors (25.6M elements) into "
                                           "25 MiB buckets x 1/8", "rotation_sets": k,
                               "bytes_per_step": 2 * payload},
                    "step_ms": tp.dist(),
                    "step_gbs": {"median": gb(tp.median), "p10_time": gb(tp.p10), "p90_time": gb(tp.p90)},
                    # a copy with one multiply per element: bound by HBM
                    "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                                 "frac": round(gbs / PEAK_GBS, 4), "kernel": "bucket_kernel",
                                 "avg_launch_us": round(ms_p * 1e3, 3),
                                 "algorithmic_bytes_per_launch": 2 * payload,
                                 "traffic": tj["bytes_per_launch"] if tj else None},
                    "copy_kernel_gbs": copy_gbs,
                    "launches": {"one_launch": 1, "per_tensor": len([n for n in numel if n])}})
        if not args.no_baselines:
            tu = time_steps(torch, unpack, args.steps, wu, lead)
            tt = time_steps(torch, pack_pt, args.steps, wu, lead)
            tw = time_steps(torch, warm_pack, args.steps, args.warmup, lead)
            res.update({"unpack_gbs": gb(tu.mean), "unpack_step_ms": tu.dist(),
                        "warm": {"ms_per_step": round(tw.mean, 5), "gbs": gb(tw.mean),
                                 "note": "one buffer set packed again and again (no rotation)"},
                        "per_tensor_pack_ms": round(tt.mean, 4),
                        "speedup_vs_per_tensor": round(tt.mean / ms_p, 3)})
        return res
    if w == "ceiling":
        return run_ceiling(torch, gtf, args, res)
    if w == "joint":
        return run_joint(torch, gtf, configs, args, res, gen)
    if w == "ln":
        return run_ln(torch, gtf, configs, args, res, gen)
    if w == "search":
        return run_search(torch, gtf, configs, args, res, gen)
    if w == "softmax":
        return run_softmax(torch, gtf, configs, args, res, gen)
    if w == "transpose":
        return run_transpose(torch, gtf, configs, args, res, gen)
    if w == "c1":
        g = configs.c1_graph()
        dists = {"x": ("uniform", -1, 1), "a": ("uniform", -1, 1), "b": ("uniform", -1, 1)}
        desc = "c1: y = sigmoid((x*a)*b), f32[64,512]"
    elif w == "c2":
        g = configs.c2_graph()
        dists = {"X": ("normal", 0, 1), "bias": ("normal", 0, 0.1), "R": ("normal", 0, 1)}
        desc = "c2: relu(X + bias) + R, bf16[4096,4096]"
    else:
        g = configs.c3_graph()
        dists = {"P": ("uniform", -2, 2)}
        desc = "c3: rowsum((exp(P) + P/2) + tanh(P)), bf16[8192,4096] -> f32[8192]"
    out = {}
    for fuse in ((True,) if args.no_baselines else (True, False)):
        plan = gtf.FusePlan(g, fuse=fuse)
        nbytes = sum(group_bytes(g, plan))
        k = _rotation_sets(nbytes) if w != "c1" else 1
        sets = [alloc_graph(torch, gtf, g, plan, gen, dists) for _ in range(k)]
        # every launch marshalled once, so the timed loop is not host-bound
        calls = [[plan.launcher(q, st) for q in range(plan.num_groups)] for st in sets]
        it = [0]

        def step():
            for f in calls[it[0] % k]:
                f()
            it[0] += 1

        def warm():
            for f in calls[0]:
                f()
        n = 5 * args.steps  # short launches: more steps for a steadier mean
        tm = time_steps(torch, step, n, max(args.warmup, k), lead)
        # warm: the first set again and again (the Infinity Cache may serve it)
        tw = None if args.no_baselines else time_steps(torch, warm, n, args.warmup, lead)
        out[fuse] = (tm, nbytes, plan.num_groups, k, tw)
        del sets
    tm, nbytes, ng, k, tw = out[True]
    ms = tm.mean
    gbs = nbytes / (ms * 1e-3) / 1e9
    res.update({"value": round(gbs, 2), "ms_per_step": round(ms, 5), "steps": 5 * args.steps,
                "config": {"workload": desc, "rotation_sets": k, "bytes_per_step": nbytes},
                "step_ms": tm.dist(), "launches": ng, "copy_kernel_gbs": copy_gbs})
    if tw is not None:
        res["warm"] = {"ms_per_step": round(tw.mean, 5), "gbs": round(nbytes / (tw.mean * 1e-3) / 1e9, 1),
                       "note": "one buffer set run again and again (no rotation)"}
    if False in out:
        res["speedup_vs_unfused"] = round(out[False][0].mean / ms, 3)
        res["unfused"] = {"ms_per_step": round(out[False][0].mean, 5), "bytes": out[False][1],
                          "launches": out[False][2], "step_ms": out[False][0].dist(),
                          "warm_ms_per_step": round(out[False][4].mean, 5)}
    # the executor's roofline: HBM bytes against 8 TB/s, and VALU
    # lane-instructions (from the committed SQ_INSTS_VALU summary of these
    # kernel sources) against the issue peak; the larger fraction binds
    hbm_frac = gbs / PEAK_GBS
    valu = read_valu(w)
    valu_frac = None
    if valu and "exec_kernel" in valu:
        valu_frac = valu["exec_kernel"] * ng / (ms * 1e-3) / VALU_PEAK
    tj = read_traffic("exec_kernel", w)
    res["roofline"] = {"bound": None if valu_frac is None else ("alu" if valu_frac > hbm_frac else "hbm"),
                       "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                       "frac": round(hbm_frac, 4), "kernel": "exec_kernel",
                       "avg_launch_us": round(ms * 1e3 / ng, 3),
                       "algorithmic_bytes_per_launch": round(nbytes / ng),
                       "traffic": tj["bytes_per_launch"] if tj else None,
                       "valu_frac": None if valu_frac is None else round(valu_frac, 4)}
    return res


def run_ceiling(torch, gtf, args, res):
    """The streaming ceiling of this part: 1 GiB copied, read or written by
    the library's probe kernels (gtf_stream_probe) over every combination of
    16-byte accesses in flight per thread (4, 8, 16), nontemporal or
    ordinary accesses, and grid (one workgroup per span, or 8, 16, 32
    resident workgroups per CU in a grid-stride loop).  Each point is the
    median of `steps` launches; copy counts 2 bytes per byte moved, read and
    write 1.  Ten launches of 1 GiB are far past the Infinity Cache."""
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    src.random_(0, 256)
    dst = torch.empty_like(src)
    kinds = {0: "copy", 1: "read", 2: "write"}
    table = []
    best = {}
    for kind, kname in kinds.items():
        for depth in (4, 8, 16):
            for nt in (False, True):
                for grid in (0, 8, 16, 32):
                    def run():
                        gtf.stream_probe(kind, depth, nt, grid, dst, src, nb)
                    ms = time_steps(torch, run, max(5, args.steps // 2), 2).median
                    gbs = (2 if kind == 0 else 1) * nb / (ms * 1e-3) / 1e9
                    row = {"kind": kname, "depth": depth, "nontemporal": nt, "grid_per_cu": grid,
                           "ms": round(ms, 4), "gbs": round(gbs, 1)}
                    table.append(row)
                    if kname not in best or gbs > best[kname]["gbs"]:
                        best[kname] = row
    # launches the size of one fused group, back to back (the gap between
    # dependent launches and each launch's ramp count, as they do for the
    # groups), rotating through >= 1 GiB of buffers
    small = []
    for kname, kind in (("copy", 0), ("read", 1)):
        bc = best[kname]
        for size in (16 << 20, 32 << 20, 64 << 20, 128 << 20, 256 << 20):
            k = max(1, (1 << 30) // size)
            views = [(dst[i * size:(i + 1) * size], src[i * size:(i + 1) * size]) for i in range(k)]
            calls = [lambda d=d, s_=s_: gtf.stream_probe(kind, bc["depth"], bc["nontemporal"],
                                                         bc["grid_per_cu"], d, s_, size)
                     for d, s_ in views]
            for f in calls:
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for f in calls:
                f()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / len(calls)
            moved = (2 if kind == 0 else 1) * size
            small.append({"kind": kname, "bytes_moved": moved, "us_per_launch": round(us, 2),
                          "gbs": round(moved / (us * 1e-6) / 1e9, 1)})
    cb = CopyBench(torch, gtf)
    lib_copy, _ = cb.gbs(10)
    del cb
    torch.cuda.synchronize()
    t = time_steps(torch, lambda: dst.copy_(src), 10, 2)
    dtod = 2 * nb / (t.median * 1e-3) / 1e9
    res.update({"value": best["copy"]["gbs"], "ms_per_step": best["copy"]["ms"],
                "config": {"workload": "ceiling: 1 GiB streamed by copy, read-only and write-only "
                                       "probe kernels over accesses in flight, nontemporal and grid",
                           "bytes_per_step": 2 * nb},
                "best": best, "back_to_back_launches": small,
                "library_copy_kernel_gbs": round(lib_copy, 1),
                "torch_copy_gbs": round(dtod, 1),
                "frac_of_8tbs": {k: round(v["gbs"] / PEAK_GBS, 4) for k, v in best.items()},
                "table": table})
    return res


def run_ln(torch, gtf, configs, args, res, gen):
    """The c5 LayerNorm, bf16[8192,1024]: one row-resident launch (mean and
    var held in LDS), TVM's three groups (mean and var through HBM), one
    launch per op, and the form with x - mean written once, planned without
    and with duplicate fusion.  Each is captured in a HIP graph
    over its rotation sets and replayed, so host launch cost is not in the
    times."""
    g = configs.layernorm_graph()
    gs = configs.layernorm_shared_graph()
    plans = {"row_resident": (g, lambda: gtf.FusePlan(g, row_resident=True)),
             "tvm_groups": (g, lambda: gtf.FusePlan(g)),
             "unfused": (g, lambda: gtf.FusePlan(g, fuse=False)),
             # x - mean written once: stored and read back by TVM's groups,
             # or recomputed in both readers by duplicate fusion
             "shared_center": (gs, lambda: gtf.FusePlan(gs)),
             "shared_center_duplicated": (gs, lambda: gtf.FusePlan(gs, duplicate=True))}
    if args.ln_variant != "all":
        plans = {args.ln_variant: plans[args.ln_variant]}
    # the 1 GiB copy: the achievable ceiling, and the reference the
    # traffic counters are scaled by
    cb = CopyBench(torch, gtf)
    copy_gbs, _ = cb.gbs(5)
    del cb
    torch.cuda.empty_cache()
    out = {}
    for name, (g, make) in plans.items():
        plan = make()
        nbytes = sum(group_bytes(g, plan))
        k = _rotation_sets(nbytes)
        sets = [alloc_graph(torch, gtf, g, plan, gen, LN_D) for _ in range(k)]
        def rotation():
            # marshalled at each call: the launches go to the current
            # (capturing) stream
            for st in sets:
                plan.run(st)
        # one replay runs the LayerNorm once on each of the k rotation sets
        graph = _captured(torch, rotation)
        ms = time_steps(torch, graph.replay, args.steps, args.warmup).mean
        ms /= k
        out[name] = {"ms_per_step": round(ms, 5), "bytes": nbytes, "launches": plan.num_groups,
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 2)}
    if len(out) == 1:
        name, v = next(iter(out.items()))
        res.update({"value": v["gbs"], "ms_per_step": v["ms_per_step"], "dtype": "bf16",
                    "config": {"workload": f"ln: LayerNorm bf16[8192,1024], {name} only",
                               "bytes_per_step": v["bytes"]},
                    "timing": "graph replays over the rotation sets", "variants": out})
        return res
    rr = out["row_resident"]
    tj = read_traffic("exec_kernel", "ln")
    bound, vf = one_launch_bound("ln", rr["gbs"], rr["ms_per_step"])
    res.update({"value": rr["gbs"], "ms_per_step": rr["ms_per_step"], "dtype": "bf16",
                "config": {"workload": "ln: LayerNorm bf16[8192,1024] with bf16 gamma/beta[1024], "
                                       "one row-resident launch",
                           "bytes_per_step": rr["bytes"]},
                "roofline": {"bound": bound, "achieved": rr["gbs"], "peak": PEAK_GBS, "unit": "GB/s",
                             "frac": round(rr["gbs"] / PEAK_GBS, 4),
                             "traffic": tj["bytes_per_launch"] if tj else None,
                             "kernel": "exec_kernel", "avg_launch_us": round(rr["ms_per_step"] * 1e3, 3),
                             "algorithmic_bytes_per_launch": rr["bytes"], "valu_frac": vf},
                "copy_kernel_gbs": round(copy_gbs, 1),
                "timing": "graph replays over the rotation sets",
                "speedup_vs_tvm_groups": round(out["tvm_groups"]["ms_per_step"] / rr["ms_per_step"], 3),
                "speedup_vs_unfused": round(out["unfused"]["ms_per_step"] / rr["ms_per_step"], 3),
                "duplicate_fusion_speedup": round(out["shared_center"]["ms_per_step"]
                                                  / out["shared_center_duplicated"]["ms_per_step"], 3),
                "variants": out})
    return res


SM_D = {"X": ("normal", 0.0, 2.0)}


def run_softmax(torch, gtf, configs, args, res, gen):
    """Row softmax over bf16[131072,128] (the attention probabilities of 8192
    tokens in 64 sequences of 128, 16 heads): one row-resident launch (max
    and sum held in LDS), TVM's three groups (max, then exp and sum, then
    the output; max and sum through HBM), and one launch per op.  Each is
    captured in a HIP graph over its rotation sets and replayed."""
    g = configs.softmax_graph()
    plans = {"row_resident": lambda: gtf.FusePlan(g, row_resident=True),
             "tvm_groups": lambda: gtf.FusePlan(g),
             "unfused": lambda: gtf.FusePlan(g, fuse=False)}
    if args.ln_variant != "all":
        plans = {args.ln_variant: plans[args.ln_variant]}
    # the 1 GiB copy: the achievable ceiling, and the reference the traffic
    # counters are scaled by
    cb = CopyBench(torch, gtf)
    copy_gbs, _ = cb.gbs(5)
    del cb
    torch.cuda.empty_cache()
    out = {}
    for name, make in plans.items():
        plan = make()
        ms, nbytes = time_plan(torch, gtf, g, plan, gen, SM_D, args.steps, args.warmup)
        out[name] = {"ms_per_step": round(ms, 5), "bytes": nbytes, "launches": plan.num_groups,
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 2)}
    if "row_resident" not in out or len(out) == 1:
        name, v = next(iter(out.items()))
        res.update({"value": v["gbs"], "ms_per_step": v["ms_per_step"], "dtype": "bf16",
                    "config": {"workload": f"softmax: row softmax bf16[131072,128], {name} only",
                               "bytes_per_step": v["bytes"]},
                    "copy_kernel_gbs": round(copy_gbs, 1),
                    "timing": "graph replays over the rotation sets", "variants": out})
        return res
    rr = out["row_resident"]
    tj = read_traffic("exec_kernel", "softmax")
    bound, vf = one_launch_bound("softmax", rr["gbs"], rr["ms_per_step"])
    res.update({"value": rr["gbs"], "ms_per_step": rr["ms_per_step"], "dtype": "bf16",
                "config": {"workload": "softmax: row softmax bf16[131072,128], one row-resident "
                                       "launch", "bytes_per_step": rr["bytes"]},
                "roofline": {"bound": bound, "achieved": rr["gbs"], "peak": PEAK_GBS, "unit": "GB/s",
                             "frac": round(rr["gbs"] / PEAK_GBS, 4),
                             "traffic": tj["bytes_per_launch"] if tj else None,
                             "kernel": "exec_kernel", "avg_launch_us": round(rr["ms_per_step"] * 1e3, 3),
                             "algorithmic_bytes_per_launch": rr["bytes"], "valu_frac": vf},
                "copy_kernel_gbs": round(copy_gbs, 1),
                "timing": "graph replays over the rotation sets",
                "speedup_vs_tvm_groups": round(out["tvm_groups"]["ms_per_step"] / rr["ms_per_step"], 3),
                "speedup_vs_unfused": round(out["unfused"]["ms_per_step"] / rr["ms_per_step"], 3),
                "variants": out})
    return res


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")


def traffic_cmds(workload):
    """The commands that make profiles/traffic_<workload>.txt."""
    extra = ("" if workload == "c5" else f" --workload {workload} --ln-variant row_resident"
             if workload in ("ln", "softmax") else f" --workload {workload}")
    run = f"python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-baselines{extra}"
    return (
        "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE "
        f"-d $OUT/pmc_fetch -o fetch --output-format csv -- {run}",
        "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE "
        f"-d $OUT/pmc_write -o write --output-format csv -- {run}",
        f"python3 bench.py --workload {workload} --traffic-from <fetch>_counter_collection.csv "
        "<write>_counter_collection.csv")


def _counter_per_kernel(path, counter):
    """{kernel short name: [per-dispatch values]} for one counter."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            for k in ("exec_kernel", "bucket_kernel", "copy_kernel"):
                if "gtf::" + k in name:
                    out.setdefault(k, {})[row["Dispatch_Id"]] = float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in out.items()}


def summarise_traffic(fetch_csv, write_csv, workload="c5"):
    fe = _counter_per_kernel(fetch_csv, "FETCH_SIZE")
    wr = _counter_per_kernel(write_csv, "WRITE_SIZE")
    nb = CopyBench.NBYTES
    f_copy = sum(fe["copy_kernel"]) / len(fe["copy_kernel"]) * 1024
    w_copy = sum(wr["copy_kernel"]) / len(wr["copy_kernel"]) * 1024
    kf, kw = nb / f_copy, nb / w_copy
    res = {"source_hash": _kernel_hash(), "copy_bytes_each_way": nb,
           "copy_fetch_bytes_counted": round(f_copy), "copy_write_bytes_counted": round(w_copy),
           "fetch_scale": round(kf, 5), "write_scale": round(kw, 5), "kernels": {}}
    for k in ("exec_kernel", "bucket_kernel"):
        if k not in fe or k not in wr:
            continue
        f = sum(fe[k]) / len(fe[k]) * 1024 * kf
        w = sum(wr[k]) / len(wr[k]) * 1024 * kw
        res["kernels"][k] = {"dispatches": len(fe[k]), "fetch_bytes_per_launch": round(f),
                             "write_bytes_per_launch": round(w),
                             "bytes_per_launch": round(f + w)}
    lines = [f"# HBM traffic per launch of the {workload} workload's kernels: rocprofv3 FETCH_SIZE "
             "and WRITE_SIZE (KiB per dispatch), each scaled so that the 1 GiB copy kernel in "
             "the same run counts exactly 1 GiB read and 1 GiB written.",
             "# commands (R = repository root, OUT = an output directory):"]
    lines += ["#   " + c for c in traffic_cmds(workload)]
    lines.append(json.dumps(res))
    with open(traffic_file(workload), "w") as f:
        f.write("\n".join(lines) + "\n")
    return res


def valu_file(workload):
    return os.path.join(ROOT, "profiles", "valu_c5_groups.txt" if workload == "c5"
                        else f"valu_{workload}.txt")


def valu_cmd(workload):
    run = ("--workload groups" if workload == "c5" else
           f"--workload {workload} --steps 3 --warmup 1 --no-baselines --no-cpu-baseline"
           + (" --ln-variant row_resident" if workload in ("ln", "softmax") else ""))
    return ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc SQ_INSTS_VALU SQ_WAVES "
            f"-d $OUT/pmc_valu -o valu --output-format csv -- python3 $R/bench.py {run}")


def summarise_valu(csv_path, layers, workload="c5"):
    """VALU lane-instructions per launch, from a rocprofv3 SQ_INSTS_VALU run:
    for c5 of each group (--workload groups launches each group's 12
    back-to-back, in C5.group_calls order), otherwise the average over the
    workload's exec_kernel launches.  SQ_INSTS_VALU counts wave
    instructions; every wave of these launches is full, so lane
    instructions are 64x."""
    import csv
    per = {}
    for row in csv.DictReader(open(csv_path, newline="")):
        if "gtf::exec_kernel" not in row["Kernel_Name"]:
            continue
        per.setdefault(int(row["Dispatch_Id"]), {})[row["Counter_Name"]] = float(row["Counter_Value"])
    ids = sorted(per)
    res = {"source_hash": _kernel_hash(), "lanes_per_wave": 64}
    if workload == "c5":
        names = [n for k in ("ln", "ge", "do") for n in C5.GROUP_NAMES[k]]
        assert len(ids) == layers * len(names), (len(ids), layers)
        res["groups"] = {}
        for gi, name in enumerate(names):
            chunk = [per[i] for i in ids[gi * layers:(gi + 1) * layers]]
            res["groups"][name] = {
                "valu_lane_instr_per_launch": round(64 * sum(c["SQ_INSTS_VALU"] for c in chunk) / layers),
                "waves_per_launch": round(sum(c["SQ_WAVES"] for c in chunk) / layers)}
        what = "each c5 group"
    else:
        res["kernels"] = {"exec_kernel": {
            "dispatches": len(ids),
            "valu_lane_instr_per_launch": round(64 * sum(per[i]["SQ_INSTS_VALU"] for i in ids) / len(ids)),
            "waves_per_launch": round(sum(per[i]["SQ_WAVES"] for i in ids) / len(ids))}}
        what = f"the {workload} workload's exec_kernel"
    with open(valu_file(workload), "w") as f:
        f.write(f"# VALU lane-instructions per launch of {what} (rocprofv3 SQ_INSTS_VALU x 64)\n")
        f.write("# command (R = repository root, OUT = an output directory):\n#   " + valu_cmd(workload) + "\n")
        f.write(f"#   python3 bench.py --workload {workload} --valu-from <valu>_counter_collection.csv\n")
        f.write(json.dumps(res) + "\n")
    return res


def _summary_json(path):
    """The last JSON line of a profiles/ summary, or None when absent or
    taken from another version of the kernel sources."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        js = [ln for ln in f if ln.startswith("{")]
    if not js:
        return None
    tj = json.loads(js[-1])
    return tj if tj.get("source_hash") == _kernel_hash() else None


def one_launch_bound(workload, gbs, ms):
    """(bound, VALU fraction) of a workload whose step is one exec_kernel
    launch: the larger of its HBM fraction and its VALU lane-instruction
    rate (committed SQ_INSTS_VALU summary of these sources) against the
    issue peak; (None, None) without a current summary."""
    valu = read_valu(workload)
    if not valu or "exec_kernel" not in valu:
        return None, None
    vf = valu["exec_kernel"] / (ms * 1e-3) / VALU_PEAK
    return ("alu" if vf > gbs / PEAK_GBS else "hbm"), round(vf, 4)


def read_valu(workload="c5"):
    """{group or kernel: VALU lane-instructions per launch}, or None."""
    tj = _summary_json(valu_file(workload))
    if tj is None:
        return None
    return {k: v["valu_lane_instr_per_launch"] for k, v in tj.get("groups", tj.get("kernels", {})).items()}


def summarise_trace(stats_csv, trace_csv, bench_json, workload):
    """profiles/<kernel>_<workload>.md from a rocprofv3 kernel trace of
    `bench.py --workload <workload> --no-baselines --no-cpu-baseline` and
    the bench line that run printed: the library's kernels, and the timed
    kernel's mean duration from the trace beside bench.py's own HIP-event
    figure for the same launches."""
    import csv
    kernel = "bucket_kernel" if workload == "c4" else "exec_kernel"
    rows = list(csv.DictReader(open(stats_csv, newline="")))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    ours = [r for r in rows if "gtf::" in r["Name"]]
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            for r in csv.DictReader(open(trace_csv, newline="")) if "gtf::" + kernel in r["Kernel_Name"]]
    bench = None
    with open(bench_json) as f:
        for ln in f:
            if ln.startswith("{"):
                bench = json.loads(ln)
    # a line with one variant timed (--ln-variant) has no roofline: one launch per step
    rf = bench.get("roofline") or {"avg_launch_us": bench["ms_per_step"] * 1e3,
                                   "algorithmic_bytes_per_launch": bench["config"]["bytes_per_step"],
                                   "achieved": bench["value"]}
    mean_us = sum(durs) / len(durs) / 1e3
    nbytes = rf["algorithmic_bytes_per_launch"]
    lines = [f"# {kernel} on {workload} — rocprofv3 kernel trace", "",
             f"Workload: {bench['config']['workload']}.  MI355X, one GPU.", "",
             "Command (R = repository root, OUT = an output directory):", "", "```",
             "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d $OUT/kt -o kt \\",
             f"    --output-format csv -- python3 $R/bench.py --workload {workload} "
             + ("--ln-variant row_resident" if workload in ("ln", "softmax") else
                "--no-baselines --no-cpu-baseline") + " > $OUT/bench.json",
             f"python3 bench.py --workload {workload} --trace-from $OUT/kt/kt_kernel_stats.csv "
             "$OUT/kt/kt_kernel_trace.csv $OUT/bench.json", "```", "",
             "The library's kernels in that run (warmup and timed launches, and the 1 GiB copy "
             "that gives the streaming ceiling):", "",
             "| Kernel | Calls | Average (ns) | Min (ns) | Max (ns) | Share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in ours:
        name = r["Name"].split("(")[0].replace("void ", "")
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {100 * float(r['TotalDurationNs']) / total:.1f}% |")
    lines += ["", f"`{kernel}`: {len(durs)} dispatches, mean {mean_us:.3f} µs in the trace; bench.py's "
              f"HIP events over its timed launches: {rf['avg_launch_us']:.3f} µs "
              f"({100 * abs(mean_us - rf['avg_launch_us']) / rf['avg_launch_us']:.1f}% apart).",
              f"Algorithmic bytes per launch: {nbytes:,} B, so {nbytes / (mean_us * 1e-6) / 1e9:.0f} GB/s "
              f"by the trace = {nbytes / (mean_us * 1e-6) / 1e9 / PEAK_GBS:.3f} of 8 TB/s "
              f"(bench.py: {rf['achieved']} GB/s; the 1 GiB copy in the same run: "
              f"{bench.get('copy_kernel_gbs', bench.get('breakdown', {}).get('copy_kernel_gbs'))} GB/s).",
              f"Source hash {_kernel_hash()} (kernels.hip, isa.h, plan.cpp)."]
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def summarise_ceiling(bench_json):
    """profiles/stream_ceiling.md from the line of `bench.py --workload
    ceiling`: every probe configuration, the best of each kind, and the
    back-to-back launches the size of one fused group."""
    d = None
    with open(bench_json) as f:
        for ln in f:
            if ln.startswith("{"):
                d = json.loads(ln)
    lines = ["# Streaming ceiling of the part — gtf_stream_probe (copy, read, write of 1 GiB)", "",
             "Command (R = repository root, OUT = an output directory):", "", "```",
             "python3 $R/bench.py --workload ceiling --steps 10 > $OUT/ceiling.json",
             "python3 bench.py --ceiling-from $OUT/ceiling.json", "```", "",
             "Each point is the median of the launches' HIP-event times; copy counts 2 bytes per "
             "byte moved.  Best of each kind:", "",
             "| Kind | 16-byte accesses in flight | Nontemporal | Workgroups per CU (0: one per span) "
             "| ms | GB/s | of 8 TB/s |", "|---|---|---|---|---|---|---|"]
    for k, r in d["best"].items():
        lines.append(f"| {k} | {r['depth']} | {r['nontemporal']} | {r['grid_per_cu']} | {r['ms']} | "
                     f"{r['gbs']} | {r['gbs'] / PEAK_GBS:.3f} |")
    lines += ["", "Back-to-back launches of the best copy and read, each the size of one fused "
              "group, rotating through >= 1 GiB:", "", "| Kind | Bytes moved per launch | µs per launch | GB/s |",
              "|---|---|---|---|"]
    for r in d["back_to_back_launches"]:
        lines.append(f"| {r['kind']} | {r['bytes_moved']:,} | {r['us_per_launch']} | {r['gbs']} |")
    lines += ["", f"The library's dwordx4 copy kernel: {d['library_copy_kernel_gbs']} GB/s; torch's "
              f"device copy: {d['torch_copy_gbs']} GB/s.", "", "Every configuration:", "",
              "| Kind | In flight | Nontemporal | Per CU | ms | GB/s |", "|---|---|---|---|---|---|"]
    for r in d["table"]:
        lines.append(f"| {r['kind']} | {r['depth']} | {r['nontemporal']} | {r['grid_per_cu']} | "
                     f"{r['ms']} | {r['gbs']} |")
    path = os.path.join(ROOT, "profiles", "stream_ceiling.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def read_traffic(kernel, workload="c5"):
    """Traffic record of one kernel, or None when absent or taken from
    another version of the kernel sources."""
    tj = _summary_json(traffic_file(workload))
    return None if tj is None else tj["kernels"].get(kernel)


class MeasuredCost:
    """Cost of a candidate plan for the search: the sum over its groups of
    each group's launch time, measured with HIP events around `reps`
    back-to-back launches on one set of device tensors (every tensor of the
    graph allocated once), cached per group (its ops' origins and the
    tensors it touches)."""

    def __init__(self, torch, graph, gen, dists, reps=10):
        self.torch, self.reps = torch, reps
        self.dev = {}
        for t, d in enumerate(graph.tensors):
            kind, a, b = dists.get(d.name, ("normal", 0.0, 1.0))
            self.dev[t] = make_tensor(torch, gen, d, kind, a, b)
        self.cache = {}
        self.measured = 0

    def __call__(self, plan):
        torch = self.torch
        origin = plan.op_origin()
        total = 0.0
        for k in range(plan.num_groups):
            key = (tuple(sorted(origin[i] for i in plan.group_ops(k))), tuple(plan.group_tensors(k)))
            if key not in self.cache:
                run = plan.launcher(k, self.dev)
                run()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(self.reps):
                    run()
                e1.record()
                torch.cuda.synchronize()
                self.cache[key] = e0.elapsed_time(e1) / self.reps
                self.measured += 1
            total += self.cache[key]
        return total


def time_plan(torch, gtf, graph, plan, gen, dists, steps, warmup):
    """A plan's time per run as HIP-graph replays over rotation sets."""
    nbytes = sum(group_bytes(graph, plan))
    k = _rotation_sets(nbytes)
    sets = [alloc_graph(torch, gtf, graph, plan, gen, dists) for _ in range(k)]

    def rotation():
        for st in sets:
            plan.run(st)
    g = _captured(torch, rotation)
    ms = time_steps(torch, g.replay, steps, warmup).mean
    del sets
    return ms / k, nbytes


def run_search(torch, gtf, configs, args, res, gen):
    """DisCo's backtracking search (alpha 1.05, beta 10, 1000 steps without
    improvement) on the c5 LayerNorm with x - mean written once, costed by
    measured launch times, against the rule-based plans of the same graph.
    Every plan is then timed the same way: HIP-graph replays over rotation
    sets."""
    import time as _time
    g = configs.layernorm_shared_graph()
    cost = MeasuredCost(torch, g, gen, LN_D)
    t0 = _time.perf_counter()
    best, st = gtf.search(g, cost, seed=int(os.environ.get("GTF_SEARCH_SEED", "1")))
    wall = _time.perf_counter() - t0
    del cost
    torch.cuda.empty_cache()
    variants = {"searched": best, "tvm_groups": gtf.FusePlan(g),
                "duplicate": gtf.FusePlan(g, duplicate=True),
                "duplicate_row_resident": gtf.FusePlan(g, duplicate=True, row_resident=True),
                "unfused": gtf.FusePlan(g, fuse=False)}
    out = {}
    for name, plan in variants.items():
        ms, nbytes = time_plan(torch, gtf, g, plan, gen, LN_D, args.steps, args.warmup)
        out[name] = {"ms_per_step": round(ms, 5), "launches": plan.num_groups, "bytes": nbytes,
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 2)}
    s = out["searched"]
    res.update({"value": s["gbs"], "ms_per_step": s["ms_per_step"], "dtype": "bf16",
                "config": {"workload": "search: DisCo backtracking search over fusion plans of the "
                                       "LayerNorm bf16[8192,1024] with x - mean written once, "
                                       "measured launch times as the cost",
                           "alpha": 1.05, "beta": 10, "max_stall": 1000,
                           "bytes_per_step": s["bytes"]},
                "search": {"steps": st["steps"], "evaluations": st["evaluations"],
                           "start_cost_ms": round(st["start_cost"], 5),
                           "best_cost_ms": round(st["best_cost"], 5), "wall_s": round(wall, 2),
                           "groups": best.groups(), "op_origin": best.op_origin()},
                "speedup_vs_tvm_groups": round(out["tvm_groups"]["ms_per_step"] / s["ms_per_step"], 3),
                "timing": "graph replays over the rotation sets", "variants": out})
    return res


def run_transpose(torch, gtf, configs, args, res, gen):
    """y = gelu(transpose(X) + b) with X bf16[4096,8192] -> y bf16[8192,4096]
    (the c5 bias+GELU group's bytes, with its input stored transposed): one
    launch whose transpose is an addressed load, against one launch per op
    and against the same group on an input already in layout."""
    from workloads.graph import Graph
    g = Graph()
    X = g.input("X", "bf16", (4096, 8192))
    b = g.input("b1", "bf16", (4096,))
    t = g.op("transpose", [X], "t", "bf16", (8192, 4096))
    u = g.op("add", [t, b], "u", "bf16", (8192, 4096))
    g.op("gelu", [u], "y", "bf16", (8192, 4096), role="out")
    dists = {"X": ("normal", 0.0, 1.0), "b1": ("normal", 0.0, 0.1)}
    plain = configs.gelu_graph()
    out = {}
    for name, (gg, plan, d) in {"fused": (g, gtf.FusePlan(g), dists),
                                "unfused": (g, gtf.FusePlan(g, fuse=False), dists),
                                "no_transpose": (plain, gtf.FusePlan(plain), GELU_D)}.items():
        ms, nbytes = time_plan(torch, gtf, gg, plan, gen, d, args.steps, args.warmup)
        out[name] = {"ms_per_step": round(ms, 5), "launches": plan.num_groups, "bytes": nbytes,
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 2)}
    f = out["fused"]
    res.update({"value": f["gbs"], "ms_per_step": f["ms_per_step"], "dtype": "bf16",
                "config": {"workload": "transpose: gelu(transpose(X) + b), X bf16[4096,8192] -> "
                                       "y bf16[8192,4096], one launch",
                           "bytes_per_step": f["bytes"]},
                "speedup_vs_unfused": round(out["unfused"]["ms_per_step"] / f["ms_per_step"], 3),
                "timing": "graph replays over the rotation sets", "variants": out})
    return res


def _captured(torch, fn):
    """fn's launches captured once in a HIP graph (on a side stream, which
    the launchers pick up as the current stream) after one eager run."""
    fn()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fn()
    return g


def run_joint(torch, gtf, configs, args, res, gen):
    """Joint op and tensor fusion on c5's 194 parameter gradients.  The
    epilogue g' = g/loss_scale + wd*w ends in *(1/N) and stores into the
    gradient's bucket slot; one fuse_multi launch runs it for all 194
    gradients (value).  Compared with the separate path (the same one-launch
    epilogue into a tensor per gradient, then bucket_pack) and with one
    launch per gradient.  All three are captured once in HIP graphs and
    replayed, so host launch cost is not in the times."""
    numel = configs.c5_numel()
    total = sum(numel)
    bp = gtf.BucketPlan(numel, "f32", configs.BUCKET_CAP_BYTES)
    _, _, bn = bp.query()
    ws = torch.empty(max(16, bp.workspace_bytes), dtype=torch.uint8, device="cuda")
    bp.bind(ws)
    buckets = [torch.empty(n, dtype=torch.float32, device="cuda") for n in bn]
    grads = [torch.randn(n, generator=gen, device="cuda") for n in numel]
    weights = [torch.randn(n, generator=gen, device="cuda") * 0.02 for n in numel]
    outs = [torch.empty(n, dtype=torch.float32, device="cuda") for n in numel]
    gj = configs.grad_epilogue_graph(1024, avg=configs.AVG_SCALE)
    gs = configs.grad_epilogue_graph(1024)
    gi, wi = gj.inputs()
    pj, ps = gtf.FusePlan(gj), gtf.FusePlan(gs)
    mj, ms_ = gtf.FuseMulti(pj, 0, numel), gtf.FuseMulti(ps, 0, numel)
    wsj = torch.empty(max(16, mj.workspace_bytes), dtype=torch.uint8, device="cuda")
    wss = torch.empty(max(16, ms_.workspace_bytes), dtype=torch.uint8, device="cuda")
    mj.bind([{gi: grads[k], wi: weights[k], gj.outputs()[0]: bp.slot_view(buckets, k, (n,))}
             for k, n in enumerate(numel)], wsj)
    ms_.bind([{gi: grads[k], wi: weights[k], gs.outputs()[0]: outs[k]} for k in range(len(numel))], wss)
    per_plans = {}
    for n in set(numel):
        g = configs.grad_epilogue_graph(n, avg=configs.AVG_SCALE)
        per_plans[n] = (g, gtf.FusePlan(g))
    torch.cuda.synchronize()

    def per_tensor():
        for k, n in enumerate(numel):
            g, plan = per_plans[n]
            a, b = g.inputs()
            plan.run_group(0, {a: grads[k], b: weights[k], g.outputs()[0]: bp.slot_view(buckets, k, (n,))})

    captured = lambda fn: _captured(torch, fn)  # noqa: E731
    g_joint = captured(lambda: mj.run())
    g_sep = captured(lambda: (ms_.run(), bp.pack(outs, buckets, configs.AVG_SCALE)))
    g_per = captured(per_tensor)
    ms_j = time_steps(torch, g_joint.replay, args.steps, args.warmup).mean
    ms_s = time_steps(torch, g_sep.replay, args.steps, args.warmup).mean
    ms_p = time_steps(torch, g_per.replay, args.steps, args.warmup).mean
    bytes_j = 12 * total              # read g and w, write the bucket slot
    bytes_s = 12 * total + 8 * total  # ... plus the pack's read and write
    res.update({"value": round(bytes_j / (ms_j * 1e-3) / 1e9, 2), "ms_per_step": round(ms_j, 4),
                "config": {"workload": "joint: epilogue g/1024 + 0.01*w on 194 fp32 gradients "
                                       "(151,156,736 elements) stored x1/8 into 25 MiB bucket slots, "
                                       "one launch",
                           "bytes_per_step": bytes_j},
                "separate": {"ms_per_step": round(ms_s, 4), "bytes_per_step": bytes_s, "launches": 2,
                             "gbs": round(bytes_s / (ms_s * 1e-3) / 1e9, 1),
                             "note": "the same one-launch epilogue into a tensor per gradient, "
                                     "then bucket_pack x1/8"},
                "per_tensor": {"ms_per_step": round(ms_p, 4), "launches": len(numel),
                               "note": "one epilogue launch per gradient, storing into its slot"},
                "speedup_vs_separate": round(ms_s / ms_j, 3),
                "speedup_vs_per_tensor": round(ms_p / ms_j, 3), "launches": 1,
                "timing": "each variant captured once in a HIP graph and replayed"})
    return res


def _kernel_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("kernels.hip", "isa.h", "plan.cpp"):
        with open(os.path.join(ROOT, "gradient_tensor_fusion_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
