"""Benchmark of the DLRMv1 forward hot path on one MI355X.

One step = one call of dlrm_forward (bottom MLP, bag gather + interaction,
top MLP, sigmoid) over one batch of seeded synthetic inputs already resident
in HBM.  Steps cycle through --index-sets independently drawn index sets so
that consecutive steps gather different rows.  By default the steps are
replayed from HIP graphs (captured, and launched once, outside the timed
region) so that host launch overhead does not hide the kernels: the timed run replays graphs
of --graph-steps consecutive steps (one graph launch per 8 forwards, as a
serving loop would; when --steps is not a multiple of it, one more graph holds
the remaining steps, so every timed step is a replay of the same form), the
percentiles and the cold-cache figure time single-step replays, and --eager
times plain calls.

Printed: one JSON line with the contract fields (the page-4 workload: batch
2048, 3 tables), plus
  path              the path dlrm_forward takes for the workload: "fused"
                    (the whole forward in one kernel) or "layered";
  roofline          the dominant kernel of that path against its roofline,
                    from a live HIP-event timing of that kernel;
  layered           the layered path's own dominant kernel and MLP rate, for
                    reference (its kernels also serve as standalone calls);
  roofline_emb_interact  the bag-gather + interaction kernel (dlrm_embbag_interact);
  kernels           per-kernel average durations (HIP events): the
                    single-launch forward and each stage of the layered path;
  nc32              the same figures for the 32-table workload (batch 2048),
                    the metric's second configuration;
  ceilings          the library's own HBM read-stream and random-row gather
                    rates (dlrm_probe_read_stream / dlrm_probe_gather_rows);
  emb_interact_large  dlrm_embbag_interact at batch 16384 with 8, 16 and 32
                    tables: us, algorithmic GB/s and fractions of 8 TB/s and
                    of the ceilings;
  cpu_baseline      the fp64 oracle on the host: the full page-4 and 32-table
                    batches on one thread and on all the cores it may use.
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

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
CSRC = os.path.join(ROOT, "dlrm_embedding_interaction_amd", "csrc")
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--workload", default="page4")
    p.add_argument("--index-sets", type=int, default=8)
    p.add_argument("--eager", action="store_true", help="time plain calls instead of graph replays")
    p.add_argument("--graph-steps", type=int, default=8,
                   help="consecutive steps (cycling the index sets) captured in one HIP graph for the timed run")
    p.add_argument("--path", default="auto", choices=["auto", "fused", "layered"],
                   help="dlrm_forward (auto), dlrm_forward_fused or dlrm_forward_layered")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=2.0,
                   help="least time per CPU-baseline measurement (whole forwards are repeated until it passes)")
    p.add_argument("--no-secondary", action="store_true", help="skip the 32-table workload")
    p.add_argument("--no-large", action="store_true", help="skip the batch-16384 bag + interaction cells")
    p.add_argument("--index-bytes", type=int, default=8, choices=[4, 8],
                   help="width of the indices and offsets handed to the library")
    p.add_argument("--kernel-reps", type=int, default=50)
    p.add_argument("--cold-steps", type=int, default=20,
                   help="forwards timed one by one after a 1 GiB flush of the caches (0: skip)")
    p.add_argument("--sweep", metavar="OUT_JSON", default=None,
                   help="time every batch x tables cell of the sweep grid, write them to OUT_JSON, print no line")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 512 MiB read (the library's probe) and a 512 MiB copy, the reference "
                        "kernels for the HBM byte counters")
    return p.parse_args()


def fused_algorithmic(w, ib=8):
    """Algorithmic flops and HBM bytes of one single-launch forward: every
    Linear layer and the dots; dense rows, gathered rows, indices and offsets
    (ib bytes each), the weights once and the outputs."""
    B, T, D, L = w.batch, w.num_tables, w.dim, w.bag
    flops = 2 * B * w.n_pairs * D
    wbytes = 0
    for ln in (list(w.ln_bot), list(w.ln_top)):
        for K, N in zip(ln[:-1], ln[1:]):
            flops += 2 * B * N * K
            wbytes += 4 * (N * K + N)
    nbytes = 4 * B * w.ln_bot[0] + B * T * L * (D * 4 + ib) + B * T * ib + wbytes + 4 * B
    return dict(name="fused_forward", kind="mfma", flops=flops, bytes=nbytes, M=B)


def algorithmic(w, ib=8):
    """Algorithmic bytes / flops per launch of each stage of the layered path
    (what the method must move or compute; indices and offsets of ib bytes)."""
    B, T, D, L = w.batch, w.num_tables, w.dim, w.bag
    P = w.n_pairs
    stages = []
    ln = list(w.ln_bot)
    for l in range(len(ln) - 1):
        K, N = ln[l], ln[l + 1]
        stages.append(dict(name=f"bot{l}", kind="mfma" if N > 1 else "hbm", flops=2 * B * N * K,
                           bytes=4 * (B * K + N * K + N + B * N), M=B, N=N, K=K))
    # fused gather + interaction: rows, indices, offsets, x read, Z written
    emb_bytes = B * T * L * (D * 4 + ib) + B * T * ib + B * D * 4 + B * P * 4
    stages.append(dict(name="emb_interact", kind="hbm", flops=2 * B * P * D, bytes=emb_bytes))
    ln = list(w.ln_top)
    for l in range(len(ln) - 1):
        K, N = ln[l], ln[l + 1]
        stages.append(dict(name=f"top{l}", kind="mfma" if N > 1 else "hbm", flops=2 * B * N * K,
                           bytes=4 * (B * K + N * K + N + B * N), M=B, N=N, K=K))
    return stages


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only; --gpus must be 1 (the forward shards by batch, with no "
              "exchange between GPUs, so one GPU's share at its real batch is what it times)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dlrm_embedding_interaction_amd as dl
    import dlrm_inputs as di

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dl.load(build_if_missing=False)
    dev = torch.device("cuda", 0)
    if args.sweep:
        run_sweep(torch, dl, di, dev, args)
        return
    if args.copy_calibration:
        copy_calibration(torch, dl, dev)
    w = di.get(args.workload)

    res = run_workload(torch, dl, di, w, dev, args)
    lay = res["layered"]
    G = 1 if args.eager else max(1, min(args.graph_steps, args.steps))
    out = {
        "metric": "DLRMv1 fwd µs @bs2048 nc=3/32; samples/s; emb-bag+interact HBM GB/s",
        "value": res["samples_per_s"],
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "us_per_forward": res["ms_per_step"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": f"synthetic (seeded; dense U[0,1), tables N(0,1/D), {w.dist} indices, bag {w.bag})",
        "config": {"workload": w.name, "batch": w.batch, "num_tables": w.num_tables, "rows_per_table": w.rows,
                   "dim": w.dim, "bag": w.bag, "ln_bot": list(w.ln_bot), "ln_top": list(w.ln_top),
                   "mode": "eager" if args.eager else "hip_graph", "index_sets": args.index_sets,
                   "steps_per_graph": G, "remainder_graph_steps": 0 if args.eager else args.steps % G,
                   "index_bytes": args.index_bytes, "path": res["path"]},
        "path": res["path"],
        "us_per_forward_p10_p50_p90": [res["pct"]["p10"], res["pct"]["p50"], res["pct"]["p90"]],
        "us_per_forward_cold_p50": res["cold_us"],
        "roofline": res["roofline"],
        "layered": lay,
        "roofline_emb_interact": res["roofline_emb"],
        # algorithmic bytes (every gathered row counted) over the stage's time
        "emb_interact_GBps": res["roofline_emb"].get("achieved_algorithmic_GBps", res["roofline_emb"]["achieved"]),
        "mlp_TFLOPs": res["mlp_tflops"],
        "mlp_frac_of_fp32_mfma_peak": res["mlp_tflops"] / FP32_MFMA_PEAK_TFLOPS,
        "kernels": res["kernels"],
    }
    ceil = None
    if not args.copy_calibration:   # counter runs keep the calibration kernels the only probes
        ceil = ceilings(torch, dl, dev)
        out["ceilings"] = ceil
        re = out["roofline_emb_interact"]
        if re["achieved"] is not None:
            re["frac_of_read_ceiling"] = re["achieved"] / ceil["read_stream_GBps"]
        l2_floor(out["roofline"], ceil)
    if not args.no_secondary and w.name != di.MANYTABLE.name:
        w2 = di.MANYTABLE
        r2 = run_workload(torch, dl, di, w2, dev, args)
        out["nc32"] = {"workload": w2.name, "batch": w2.batch, "num_tables": w2.num_tables, "path": r2["path"],
                       "us_per_forward": r2["ms_per_step"] * 1e3, "samples_per_s": r2["samples_per_s"],
                       "us_per_forward_p10_p50_p90": [r2["pct"]["p10"], r2["pct"]["p50"], r2["pct"]["p90"]],
                       "us_per_forward_cold_p50": r2["cold_us"],
                       "mlp_TFLOPs": r2["mlp_tflops"],
                       "emb_interact_GBps": r2["roofline_emb"]["achieved"],
                       "roofline": r2["roofline"], "roofline_emb_interact": r2["roofline_emb"]}
        if ceil:
            l2_floor(out["nc32"]["roofline"], ceil)
    if not args.no_large:
        out["emb_interact_large"] = large_cells(torch, dl, di, dev, args, ceil)
    if not args.no_cpu_baseline:
        extra = [] if args.no_secondary or w.name == di.MANYTABLE.name else [di.MANYTABLE]
        out["cpu_baseline"] = cpu_baseline([w] + extra, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def run_workload(torch, dl, di, w, dev, args):
    torch.cuda.synchronize()
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    inp = di.make_inputs(w, device=dev)
    model = dl.Model.from_inputs(inp)
    B = w.batch
    path = model.path(B) if args.path == "auto" else args.path
    nsets = max(1, args.index_sets)
    idx_sets = [inp.indices]
    for s in range(1, nsets):
        idx_sets.append(di.make_indices(w, device=dev, seed=di.BASE_SEED + 7919 * s))
    itype = torch.int32 if args.index_bytes == 4 else torch.int64
    idx_sets = [[i.to(itype) for i in ix] for ix in idx_sets]
    inp.offsets = [o.to(itype) for o in inp.offsets]
    ws = model.workspace(B)
    out = torch.empty(B, device=dev)
    argsets = [model.forward_args(inp.dense, idx, inp.offsets) for idx in idx_sets]

    def step(i):
        model.forward(inp.dense, idx_sets[i % nsets], inp.offsets, out=out, workspace=ws, args=argsets[i % nsets],
                      path=args.path)

    for i in range(nsets):
        step(i)
    torch.cuda.synchronize()

    run = step
    if not args.eager:
        stream = torch.cuda.Stream()
        graphs = []
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for i in range(nsets):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(i)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()

        def run(i):
            graphs[i % nsets].replay()

        # the timed run replays graphs of G consecutive steps, so that one
        # graph launch covers G forwards (the serving loop's form); the K mod G
        # steps left over run as one more graph of that many steps
        G = max(1, min(args.graph_steps, args.steps))
        rem = args.steps % G

        def capture(n):
            g = torch.cuda.CUDAGraph()
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for i in range(n):
                        step(i)
            torch.cuda.current_stream().wait_stream(stream)
            return g
        multi = capture(G)
        tail = capture(rem) if rem else None
        # a graph's first launch carries one-time setup (its upload to the
        # device); each timed graph is launched once here, untimed
        multi.replay()
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    if args.eager:
        for i in range(args.steps):
            run(i)
    else:
        for _ in range(args.steps // G):
            multi.replay()
        if tail is not None:
            tail.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps

    # per-step distribution: the same replays, each between two events
    n_pct = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_pct)]
    for i, (a, b) in enumerate(evs):
        a.record()
        run(i)
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    pct = {"p10": per[len(per) // 10], "p50": per[len(per) // 2], "p90": per[(len(per) * 9) // 10]}

    # cold caches: a 1 GiB read-modify-write between forwards evicts L2 and the Infinity Cache
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 28, device=dev)
        flush.zero_()
        ct = []
        for i in range(args.cold_steps):
            flush.add_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run(i)
            b.record()
            ct.append((a, b))
        torch.cuda.synchronize()
        cold = sorted(a.elapsed_time(b) * 1e3 for a, b in ct)[len(ct) // 2]
        del flush

    kernels = time_stages(torch, dl, model, inp, idx_sets, ws, w, args.kernel_reps,
                          fused=model.packed is not None and path == "fused", ib=args.index_bytes)
    # the counter summary holds 8-byte-index runs under the workload's name and
    # 4-byte-index runs under name + "_i32"
    traffic = counted_traffic(w.name if args.index_bytes == 8 else w.name + "_i32")
    reuse = w.dist == "zipf"
    stages = [k for k in kernels if k["name"] != "fused_forward"]
    roof_layered = roofline(stages, dominant=True, traffic=traffic, reuse=reuse)
    roof_emb = roofline([k for k in stages if k["name"] == "emb_interact"], dominant=True, traffic=traffic,
                        reuse=reuse)
    if path == "fused":
        fk = next(k for k in kernels if k["name"] == "fused_forward")
        roof = roofline([fk], dominant=True, traffic=traffic)
        roof["weights_streamed_per_block_bytes"] = int(model.packed.numel() * 4)
        mlp_tf = fk["flops"] / (fk["us"] * 1e-6) / 1e12
    else:
        roof = roof_layered
    del inp, model, idx_sets, ws, argsets
    torch.cuda.empty_cache()
    mlp = [k for k in stages if k["name"] != "emb_interact"]
    lay_tf = sum(k["flops"] for k in mlp) / (sum(k["us"] for k in mlp) * 1e-6) / 1e12
    if path != "fused":
        mlp_tf = lay_tf
    layered = {"roofline": roof_layered, "mlp_TFLOPs": lay_tf,
               "stage_us_sum": sum(k["us"] for k in stages)}
    return dict(ms_per_step=ms, samples_per_s=B / (ms * 1e-3), kernels=kernels, roofline=roof, roofline_emb=roof_emb,
                pct=pct, cold_us=cold, mlp_tflops=mlp_tf, path=path, layered=layered)


def time_stages(torch, dl, model, inp, idx_sets, ws, w, reps, fused=False, ib=8):
    """Average duration of each kernel, launched alone on the current stream,
    with HIP events: the single-launch forward (when `fused`) and every stage
    of the layered path."""
    stages = ([fused_algorithmic(w, ib)] if fused else []) + algorithmic(w, ib)
    B, D = w.batch, w.dim
    P = w.n_pairs
    ldR = (D + P + 3) // 4 * 4
    hidden = list(w.ln_bot[1:-1]) + list(w.ln_top[1:-1])
    ldH = (max(hidden) + 3) // 4 * 4 if hidden else 4
    dev = inp.dense.device
    R = torch.zeros((B, ldR), device=dev)
    H = [torch.zeros((B, ldH), device=dev), torch.zeros((B, ldH), device=dev)]
    y = torch.empty((B, 1), device=dev)
    calls = {}
    h, hsel = inp.dense, 0
    for l, (W, b) in enumerate(zip(model.bot_w, model.bot_b)):
        last = l == len(model.bot_w) - 1
        o = R[:, :W.shape[0]] if last else H[hsel][:, :W.shape[0]]
        calls[f"bot{l}"] = (lambda h=h, W=W, b=b, o=o: dl.linear_bias_act(h, W, b, dl.ACT_RELU, out=o))
        if not last:
            hsel ^= 1
        h = o
    nsets = len(idx_sets)
    cnt = [0]

    def emb():
        cnt[0] += 1
        dl.embbag_interact(model.tables, idx_sets[cnt[0] % nsets], inp.offsets, R, concat_dense=False,
                           out=R[:, D:])
    calls["emb_interact"] = emb
    yf = torch.empty(B, device=dev)

    def fused_fwd():
        cnt[0] += 1
        model.forward(inp.dense, idx_sets[cnt[0] % nsets], inp.offsets, out=yf, path="fused")
    calls["fused_forward"] = fused_fwd
    h = R[:, :D + P]
    for l, (W, b) in enumerate(zip(model.top_w, model.top_b)):
        last = l == len(model.top_w) - 1
        o = y if last else H[hsel][:, :W.shape[0]]
        act = dl.ACT_SIGMOID if last else dl.ACT_RELU
        calls[f"top{l}"] = (lambda h=h, W=W, b=b, o=o, act=act: dl.linear_bias_act(h, W, b, act, out=o))
        if not last:
            hsel ^= 1
        h = o
    out = []
    stream = torch.cuda.Stream()
    for st in stages:
        f = calls[st["name"]]
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        # `reps` launches of this stage alone, captured once and replayed, so
        # that the events time the GPU work rather than the host call path
        g = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for _ in range(reps):
                    f()
        torch.cuda.current_stream().wait_stream(stream)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (3 * reps)
        d = dict(st)
        d["us"] = us
        out.append(d)
        del g
    return out


def kernel_source_hash() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counted_traffic(workload: str) -> dict:
    """HBM bytes per dispatch of each stage from the committed counter summary,
    or {} when the kernel sources have changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    text = open(TRAFFIC_FILE).read()
    want = f"kernel-source-sha256: {kernel_source_hash()}"
    if want not in text:
        return {}
    out = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 7 and cells[0] == workload:
            out[cells[1]] = int(cells[6])
    return out


def roofline(kernels, dominant=True, traffic=None, reuse=False):
    """Roofline of the longest of `kernels`.  With `reuse` (Zipf bags, whose
    hot rows are gathered many times per launch) the algorithmic rate counts
    every reuse and passes the HBM peak, so `achieved` and `frac` are taken
    from the counted L2-miss bytes instead (null when no counter summary
    matches the sources), and the algorithmic rate is kept under its own keys."""
    k = max(kernels, key=lambda s: s["us"])
    sec = k["us"] * 1e-6
    tr = (traffic or {}).get(k["name"])
    if k["kind"] == "mfma":
        achieved = k["flops"] / sec / 1e12
        return {"kernel": k["name"], "bound": "mfma", "achieved": achieved, "peak": FP32_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / FP32_MFMA_PEAK_TFLOPS, "traffic": tr,
                "us_per_launch": k["us"], "flops_per_launch": k["flops"],
                "shape": [k.get("M"), k.get("N"), k.get("K")]}
    achieved = k["bytes"] / sec / 1e9
    out = {"kernel": k["name"], "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": achieved / HBM_PEAK_GBPS, "traffic": tr, "us_per_launch": k["us"],
           "bytes_per_launch": k["bytes"]}
    if tr:
        # counted L2-miss bytes (Infinity Cache hits included) over the same time: with reused rows
        # (Zipf bags) the algorithmic rate counts every reuse and can pass the peak; this one cannot
        out["counted_l2_miss_GBps"] = tr / sec / 1e9
        out["frac_counted_l2_miss"] = tr / sec / 1e9 / HBM_PEAK_GBPS
    if reuse:
        out["achieved_algorithmic_GBps"] = achieved
        out["frac_algorithmic"] = achieved / HBM_PEAK_GBPS
        out["achieved"] = out.get("counted_l2_miss_GBps")
        out["frac"] = out.get("frac_counted_l2_miss")
        out["achieved_basis"] = "counted L2-miss bytes per launch" if tr else "no counter summary for these sources"
    return out


def l2_floor(roof, ceil):
    """For the single-launch kernel: every block streams all packed weights
    from L2, so one block's weight bytes over the measured per-CU L2 rate is a
    floor on the kernel's time (one block per CU at batch 2048)."""
    wb = roof.get("weights_streamed_per_block_bytes")
    if wb and ceil.get("l2_stream_GBps_per_cu"):
        fl = wb / (ceil["l2_stream_GBps_per_cu"] * 1e9) * 1e6
        roof["l2_stream_floor_us"] = fl
        roof["frac_of_l2_stream_floor"] = fl / roof["us_per_launch"]


def _time_graph(torch, f, reps, rounds=3):
    """Average microseconds of f() when `reps` calls are captured in one graph
    and the graph is replayed `rounds` times between two events."""
    for _ in range(2):
        f()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for _ in range(reps):
                f()
    torch.cuda.current_stream().wait_stream(stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(rounds):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (rounds * reps)


def ceilings(torch, dl, dev, nbytes=2 << 30, gather_rows=1 << 21, dim=64):
    """The library's own bandwidth ceilings: a sequential float4 read of 2 GiB
    (bigger than every cache), and a gather of 2M random rows of 64 floats
    from a 3.2 GB table (the access pattern of one-index bags; far bigger
    than the 256 MB Infinity Cache)."""
    src = torch.ones(nbytes // 4, device=dev)
    us = _time_graph(torch, lambda: dl.probe_read_stream(src), reps=5)
    read = nbytes / (us * 1e-6) / 1e9
    del src
    rows = (3200 << 20) // (dim * 4)
    table = torch.ones((rows, dim), device=dev)
    gen = torch.Generator(device=dev).manual_seed(11)
    idx = torch.randint(0, rows, (gather_rows,), device=dev, generator=gen)
    us_g = _time_graph(torch, lambda: dl.probe_gather_rows(table, idx), reps=5)
    gbytes = gather_rows * (dim * 4 + 8)
    gather = gbytes / (us_g * 1e-6) / 1e9
    del table, idx
    torch.cuda.empty_cache()
    # L2 -> CU: one block per CU reads the same 1.5 MiB (L2-resident after the
    # first pass), as the single launch streams its packed weights
    l2b = 3 << 19
    l2src = torch.ones(l2b // 4, device=dev)
    us_l2 = _time_graph(torch, lambda: dl.probe_l2_stream(l2src, blocks=256), reps=20)
    l2_cu = l2b / (us_l2 * 1e-6) / 1e9
    del l2src
    torch.cuda.empty_cache()
    return {"read_stream_GBps": read, "read_stream_frac_of_peak": read / HBM_PEAK_GBPS,
            "read_stream_bytes": nbytes, "gather_rows_GBps": gather,
            "gather_rows_frac_of_peak": gather / HBM_PEAK_GBPS,
            "gather_rows": gather_rows, "gather_row_bytes": dim * 4, "gather_bytes_incl_int64_index": gbytes,
            "l2_stream_GBps_per_cu": l2_cu, "l2_stream_B_per_clk_per_cu_at_2p4GHz": l2_cu / 2.4,
            "l2_stream_bytes_per_block": l2b}


LARGE_CELLS = ((16384, 8), (16384, 16), (16384, 32))


def large_cells(torch, dl, di, dev, args, ceil):
    """dlrm_embbag_interact alone at batch 16384 with 8, 16 and 32 tables (the
    sweep cells where the bag + interaction traffic is large enough to judge
    against HBM bandwidth), 8 index sets rotating, replayed from a graph."""
    out = {}
    itype = torch.int32 if args.index_bytes == 4 else torch.int64
    for B, T in LARGE_CELLS:
        w = di.sweep(B, T)
        inp = di.make_inputs(w, device=dev)
        sets = [inp.indices] + [di.make_indices(w, device=dev, seed=di.BASE_SEED + 7919 * s) for s in range(1, 8)]
        sets = [[i.to(itype) for i in ix] for ix in sets]
        offs = [o.to(itype) for o in inp.offsets]
        D, P = w.dim, w.n_pairs
        R = torch.zeros((B, (D + P + 3) // 4 * 4), device=dev)
        cnt = [0]

        def emb():
            cnt[0] += 1
            dl.embbag_interact(inp.tables, sets[cnt[0] % 8], offs, R, concat_dense=False, out=R[:, D:])
        us = _time_graph(torch, emb, reps=24)
        ib = args.index_bytes
        nbytes = B * T * w.bag * (D * 4 + ib) + B * T * ib + B * D * 4 + B * P * 4
        gbps = nbytes / (us * 1e-6) / 1e9
        cell = {"us": us, "bytes": nbytes, "GBps": gbps, "frac_of_peak": gbps / HBM_PEAK_GBPS}
        tr = counted_traffic(w.name if ib == 8 else w.name + "_i32").get("emb_interact")
        if tr:
            cell["traffic"] = tr
            cell["counted_GBps"] = tr / (us * 1e-6) / 1e9
        if ceil:
            cell["frac_of_read_ceiling"] = gbps / ceil["read_stream_GBps"]
            cell["frac_of_gather_ceiling"] = gbps / ceil["gather_rows_GBps"]
        out[f"{B}x{T}"] = cell
        print(f"[bench] emb_interact {B}x{T}: {us:.1f} us, {gbps:.0f} GB/s", file=sys.stderr, flush=True)
        del inp, sets, R
        torch.cuda.empty_cache()
    return out


def copy_calibration(torch, dl, dev, nbytes=512 << 20, reps=5):
    """Kernels of known traffic whose FETCH_SIZE / WRITE_SIZE per dispatch scale
    the counters of the measured kernels to bytes: the library's read-stream
    probe over 512 MiB (read once, nothing written) and a 512 MiB device copy
    (read and written once)."""
    a = torch.ones(nbytes // 4, device=dev)
    for _ in range(reps):
        dl.probe_read_stream(a)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"[bench] counter calibration: {reps} reads and {reps} copies of {nbytes} bytes", file=sys.stderr,
          flush=True)
    del a, b


def run_sweep(torch, dl, di, dev, args):
    rows = []
    for T in di.SWEEP_TABLES:
        for B in di.SWEEP_BATCHES:
            w = di.sweep(B, T)
            a = argparse.Namespace(**vars(args))
            a.steps, a.warmup = max(20, min(args.steps, 200)), 10
            r = run_workload(torch, dl, di, w, dev, a)
            emb = next(k for k in r["kernels"] if k["name"] == "emb_interact")
            row = dict(batch=B, tables=T, path=r["path"], us_per_forward=r["ms_per_step"] * 1e3,
                       samples_per_s=r["samples_per_s"],
                       emb_interact_us=emb["us"], emb_interact_GBps=r["roofline_emb"]["achieved"],
                       kernels={k["name"]: k["us"] for k in r["kernels"]})
            rows.append(row)
            print(f"[sweep] b={B:6d} t={T:2d}  {row['us_per_forward']:9.2f} us/fwd  "
                  f"emb {emb['us']:8.2f} us {row['emb_interact_GBps']:8.1f} GB/s", file=sys.stderr, flush=True)
    with open(args.sweep, "w") as f:
        json.dump(rows, f, indent=1)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(workloads, seconds):
    """The fp64 oracle (as it stands) on the host: each workload's full batch,
    on one thread and on all the threads this process may use (OMP_NUM_THREADS,
    else the CPUs it is allowed to run on), whole forwards repeated until
    `seconds` have passed."""
    import oracle
    import dlrm_inputs as di
    o = oracle.default()
    allowed = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    n_all = int(os.environ.get("OMP_NUM_THREADS", 0)) or allowed

    def rate(inp, threads):
        used = o.set_threads(threads)
        done, t0 = 0, time.perf_counter()
        while True:
            oracle.forward_inputs(inp, oracle=o)
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return inp.workload.batch * done / el, used, done, el

    per = {}
    for w in workloads:
        inp = di.make_inputs(w)
        one, _, n1, t1 = rate(inp, 1)
        many, used, nm, tm = rate(inp, n_all)
        per[w.name] = {"samples_per_s_1thread": one, "samples_per_s_all": many, "threads_all": used,
                       "us_per_forward_1thread": w.batch / one * 1e6, "us_per_forward_all": w.batch / many * 1e6,
                       "forwards_timed": [n1, nm], "seconds": [t1, tm]}
    first = per[workloads[0].name]
    return {"value": first["samples_per_s_all"], "unit": "samples/s", "cores": first["threads_all"],
            "kind": "oracle", "value_1thread": first["samples_per_s_1thread"],
            "sample": f"{workloads[0].name}: the full batch of {workloads[0].batch} samples, whole fp64 forwards "
                      f"(OpenMP over samples) repeated for at least {seconds:.0f} s, on "
                      f"{first['threads_all']} threads and on 1",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "threads_allowed": allowed,
            "workloads": per}


if __name__ == "__main__":
    main()
