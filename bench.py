"""Throughput of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one call of moe_layer_forward (route -> permute -> grouped FFN ->
combine -> aux statistics) over one batch of synthetic inputs already resident
in HBM.  W untimed steps, then exactly K steps bracketed by device
synchronisation and timed with HIP events on the stream the library launches
on; value = tokens per second.  The same step is then timed call by call, warm
and cache-cold (a 512 MB buffer, twice the last-level cache, written before
each call outside the event window), for the median, p10 and p90, and once
more replayed from a HIP graph that captured one step (no host launches; the
replay must give the eager output bit for bit).  Per-stage times come from the stage entry
points timed the same way.  The dominant kernel (the grouped gate/up GEMM with
the fused activation) is timed on its own for the roofline figure.  The CPU
oracle is timed on a bounded sample of the same workload for the CPU baseline
(plus the tiny fp32 layer on one thread and on all threads).  The other four
workloads are then timed the same way (layer step and stages) into the line's
"workloads" object (--only skips them).
Prints one JSON line.  `--train` times a training step instead, `--shard` the
grouped FFN on one GPU's share of the 8-GPU expert/head-parallel layers, and
`--counters` runs each stage a few times for rocprofv3 counter passes.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
# a one-group dense FFN descriptor carries none of the layer's routing options
DENSE = dict(capacity_factor=0.0, gate="topk", n_groups=0, group_limit=0, queue="token", eval=0)
GEMM_SOURCE = os.path.join(ROOT, "mixture_experts_layer_45_amd", "csrc", "gemm.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=None)
    p.add_argument("--set", action="append", default=[], metavar="KEY=VALUE",
                   help="override a workload field, e.g. the routing variants n_groups=8, group_limit=4, "
                        "gate=hash, queue=choice, capacity_factor_eval=1.5, eval=1")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--only", action="store_true",
                   help="time the headline workload only (by default the other workloads are timed too, "
                        "with their stages, into the line's \"workloads\" object)")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the baseline sample")
    p.add_argument("--stage-reps", type=int, default=10)
    p.add_argument("--train", action="store_true",
                   help="time a training step instead: the training forward (it keeps what the backward "
                        "reads) and moe_layer_backward of sum(dy * y) + L_aux")
    p.add_argument("--shard", action="store_true",
                   help="time the grouped FFN on one GPU's share of the expert/head-parallel layers at their "
                        "real shapes (8 GPUs): prints one line")
    p.add_argument("--row-major", action="store_true",
                   help="time the expert weights in their row-major layout (by default the bf16 workloads' "
                        "expert weights are put in fragment order once, before any timing, with moe_pack_weights)")
    p.add_argument("--counters", action="store_true",
                   help="for rocprofv3 --pmc runs: a 1 GiB device copy (counter calibration), then each "
                        "stage (route, gather permute, GEMM1, GEMM2, combine) three times; prints one line")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def per_step(fn, reps, stream, flush=None):
    """Per-call times (ms) from an event pair around each call; with `flush`,
    that buffer is rewritten before every call, outside the event window, so
    each call starts with the last-level cache (256 MB MALL) holding none of
    its inputs."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        if flush is not None:
            flush.fill_(1)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def spread(ms, T):
    import numpy as np
    p10, p50, p90 = (float(v) for v in np.percentile(ms, [10, 50, 90]))
    return {"median_ms": p50, "p10_ms": p10, "p90_ms": p90, "tokens_per_s_median": T / (p50 * 1e-3),
            "calls": len(ms)}


def timed(fn, reps, stream):
    import torch
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps  # ms


def graph_per_step(step, reps, stream, T, out):
    """The same step captured once into a HIP graph (torch.cuda.CUDAGraph on
    the stream the library launches on) and replayed: per-replay spread, and
    whether a replay's output equals the eager step's bit for bit."""
    import torch
    try:
        step()
        torch.cuda.synchronize()
        ref = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                                ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref))
        res = dict(spread(per_step(g.replay, reps, stream), T), bitwise_equal_to_eager=same)
        del g
        return res
    except Exception as e:  # reported, not fatal: the eager figures stand
        return {"error": f"{type(e).__name__}: {e}"[:300]}


def traffic_from_profile(kernel_tag, workload):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current GEMM source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    src_hash = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if fields.get("gemm_source_sha256") != src_hash:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def train_bench(args, cfg, name, inp, desc, ws, y, stream):
    """One training step = moe_layer_forward_train + moe_layer_backward on the
    same batch; prints one JSON line (tokens per second of whole steps)."""
    import numpy as np
    import torch

    import mixture_experts_layer_45_amd as moe
    T, h, H, E, K, f = cfg["T"], cfg["h"], cfg["H"], cfg["E"], cfg["K"], cfg["f"]
    d = h // H
    sv = moe.alloc_saved(desc)
    gr = moe.alloc_grads(desc, inp, inp["x"])
    wsb = moe.workspace(desc, moe.MOE_WS_BACKWARD)
    dy = torch.randn((T, h), generator=torch.Generator(device="cuda").manual_seed(1), device="cuda").to(torch.bfloat16)
    aux = dict(n_kept=torch.empty(1, dtype=torch.int32, device="cuda"))

    def fwd():
        moe.moe_layer_forward_train(desc, inp, inp["x"], y, sv, aux=aux, ws=ws)

    def bwd():
        moe.moe_layer_backward(desc, inp, inp["x"], dy, sv, gr, aux_weight=1.0, ws=wsb)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} training steps")
    ms_step = timed(step, args.steps, stream)
    fwd()
    t_fwd = timed(fwd, args.stage_reps, stream)
    t_bwd = timed(bwd, args.stage_reps, stream)
    n_kept = int(aux["n_kept"].item())
    n_act = 2 if cfg["act"] == "swiglu" else 1
    ffn = 2.0 * (n_act + 1) * n_kept * d * f
    router = 2.0 * T * H * E * d if cfg.get("gate", "topk") != "hash" else 0.0
    fwd_flops = ffn + router
    if cfg.get("n_shared"):
        fwd_flops += 2.0 * (n_act + 1) * T * h * f
    if cfg.get("has_wo"):
        fwd_flops += 2.0 * T * h * h
    # backward: an input-gradient and a weight-gradient product per forward product
    bwd_flops = 2.0 * fwd_flops
    bwd_tfs = bwd_flops / (t_bwd * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu:
        from oracle import oracle as orc

        def to_np(t):
            if t is None:
                return None
            t = t.detach().cpu().contiguous()
            return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

        host = {k: to_np(v) for k, v in inp.items()}
        dyh = dy.float().cpu().numpy().astype(np.float64)
        threads = orc.num_threads()
        Ts, elapsed = 2, 0.0
        while True:
            t0 = time.perf_counter()
            c = dict(cfg, T=Ts)
            orc.layer_forward(c, host, host["x"][:Ts])
            orc.layer_backward(c, host, host["x"][:Ts], dyh[:Ts], c_aux=1.0)
            elapsed = time.perf_counter() - t0
            if elapsed >= args.cpu_seconds * 0.6 or Ts >= T:
                break
            Ts = min(T, Ts * 4, max(Ts + 1, int(Ts * args.cpu_seconds / max(elapsed, 1e-3))))
        log(f"[bench] oracle forward + backward: {Ts} tokens in {elapsed:.2f} s on {threads} threads")
        cpu = {"value": Ts / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"first {Ts} tokens of the {name} batch as their own batch, full weights; fp64 C "
                         f"oracle forward + backward, {elapsed:.1f} s"}
    out = {
        "metric": "MoE-layer fwd+bwd (training step) tokens/sec on 1 GPU",
        "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg["dtype"], "data": "synthetic (seeded inputs, N(0,1) dy)",
        "config": {"workload": name, "tokens": T, "hidden": h, "heads": H, "experts": E, "top_k": K, "ffn": f,
                   "act": cfg["act"], "score": cfg["score"], "capacity_factor": cfg["capacity_factor"],
                   "parallelism": "single GPU"},
        "n_kept": n_kept,
        "stages": {"forward_train_ms": t_fwd, "backward_ms": t_bwd,
                   "forward_tflops": fwd_flops / (t_fwd * 1e-3) / 1e12, "backward_tflops": bwd_tfs},
        "roofline": {"kernel": "whole backward pass (dgrad + wgrad grouped GEMMs on k-major operands, router, dx)",
                     "bound": "mfma", "achieved": bwd_tfs, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": bwd_tfs / MFMA_BF16_PEAK_TFS, "traffic": None, "flops_per_launch": bwd_flops,
                     "launch_ms": t_bwd},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


# One GPU's share of the sharded layers (8 GPUs, each with the workload's T
# tokens): expert parallelism puts E/8 experts on a GPU, which receives every
# GPU's rows routed to them; head parallelism puts one head's 32 experts on a
# GPU, with the d-slices of all 8*T tokens.  (base workload, local groups,
# rows per group)
SHARDS = {
    "ep8_top2_e8_h4096": ("top2_e8_h4096", 1, 16384),        # 8*8192 tokens x K=2 / 8 experts
    "ep8_sigmoid_top8_e256": ("sigmoid_top8_e256_shared", 32, 1024),  # 8*4096 x 8 / 256
    "hp8_multihead_h8_e32": ("multihead_h8_e32_top4", 32, 8192),  # 8*8192 x 4 / 32 per head
}


def shard_bench(args):
    """Grouped FFN (GEMM1 + activation + GEMM2, moe_grouped_ffn) on each
    shard's real shape: uniform rows per local expert, synthetic inputs."""
    import torch

    import mixture_experts_layer_45_amd as moe
    from mixture_experts_layer_45_amd import inputs

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    res = []
    for sname, (base, G, rows) in SHARDS.items():
        b = inputs.CONFIGS[base]
        d = b["h"] // b.get("H", 1)
        N = G * rows
        cfg = dict(b, T=N, h=d, H=1, E=G, K=1, n_shared=0, has_wo=0, logit_bias=None, select_bias=None, **DENSE)
        log(f"[bench] shard {sname}: {G} groups x {rows} rows, d={d}, f={cfg['f']}")
        inp = inputs.make_inputs(cfg, "cuda", seed=0)
        if not args.row_major:  # as the layer is timed: expert weights in fragment order
            inp = moe.pack_weights(inp)
            cfg = dict(cfg, packed=1)
        desc = moe.desc_from_cfg(cfg)
        offsets = torch.arange(0, N + 1, rows, dtype=torch.int32, device="cuda")
        dt = inputs.torch_dtype(cfg)
        h_tmp = torch.empty((N, cfg["f"]), dtype=dt, device="cuda")
        y_perm = torch.empty((N, d), dtype=dt, device="cuda")
        ws = moe.workspace(desc, moe.MOE_WS_FFN)

        def ffn():
            moe.moe_grouped_ffn(desc, inp["x"], offsets, N, inp["w_gate"], inp["w_up"], inp["w_down"], h_tmp,
                                y_perm, 0, ws)

        for _ in range(args.warmup):
            ffn()
        ms = timed(ffn, args.stage_reps, stream)
        n_act = 2 if cfg["act"] == "swiglu" else 1
        flops = 2.0 * N * d * cfg["f"] * (n_act + 1)
        tfs = flops / (ms * 1e-3) / 1e12
        res.append({"shard": sname, "weights": "row-major" if args.row_major else "fragment order",
                    "groups": G, "rows_per_group": rows, "d": d, "f": cfg["f"], "ffn_ms": ms,
                    "tflops": tfs, "mfma_frac": tfs / MFMA_BF16_PEAK_TFS})
        del inp, h_tmp, y_perm, ws
        torch.cuda.empty_cache()
    out = {"metric": "grouped FFN on one GPU's share of the 8-GPU expert/head-parallel layers", "unit": "TFLOP/s",
           "n_gpus": 1, "dtype": "bf16", "data": "synthetic", "shards": res}
    print(json.dumps(out), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measure_layer(args, cfg, over, headline):
    """Times one workload's layer step and its stages; returns a dict.  With
    headline, also the warm / cache-cold / graph-replay spreads, the roofline
    object of the dominant kernel and (unless --no-cpu) the CPU baseline."""
    import numpy as np
    import torch

    import mixture_experts_layer_45_amd as moe
    from mixture_experts_layer_45_amd import inputs

    name = cfg["name"]
    T, h, H, E, K, f = cfg["T"], cfg["h"], cfg["H"], cfg["E"], cfg["K"], cfg["f"]
    d = h // H
    Et, A = H * E, T * H * K
    esz = 2 if cfg["dtype"] == "bf16" else 4
    dev = "cuda"
    stream = torch.cuda.current_stream()
    log(f"[bench] workload {name}: generating inputs on the device")
    inp = inputs.make_inputs(cfg, dev, seed=0)
    # the expert weights in fragment order (a one-time layout change made when
    # the weights are loaded, outside every timed region); the training step
    # reads row-major weights
    inp_rm = desc_rm = None
    packed = cfg["dtype"] == "bf16" and not args.row_major and not args.train
    if packed:
        if headline:
            inp_rm, desc_rm = inp, moe.desc_from_cfg(cfg)
        inp = moe.pack_weights(inp)
        torch.cuda.synchronize()
        cfg = dict(cfg, packed=1)
    desc = moe.desc_from_cfg(cfg)
    ws = moe.workspace(desc)
    y = torch.empty((T, h), dtype=inputs.torch_dtype(cfg), device=dev)
    if args.train:
        return train_bench(args, cfg, name, inp, desc, ws, y, stream)
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    aux = dict(topk_idx=torch.empty((T * H, K), **i32), topk_w=torch.empty((T * H, K), **f32),
               dest_row=torch.empty(A, **i32), counts=torch.empty(Et, **i32), kept=torch.empty(Et, **i32),
               n_kept=torch.empty(1, **i32), n_dropped=torch.empty(1, **i32), f=torch.empty(Et, **f32),
               P=torch.empty(Et, **f32), l_aux=torch.empty(1, **f32))

    def step():
        moe.moe_layer_forward(desc, inp, inp["x"], y, aux, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {name}: timing {args.steps} steps")
    ms_step = timed(step, args.steps, stream)
    tok_s = T / (ms_step * 1e-3)

    res = {"weights": "fragment order (moe_pack_weights)" if packed else "row-major"}
    if inp_rm is not None:
        # the same step on the row-major weights, for reference
        def step_rm():
            moe.moe_layer_forward(desc_rm, inp_rm, inp_rm["x"], y, aux, ws)

        step_rm()
        torch.cuda.synchronize()
        res["row_major_ms_per_step"] = timed(step_rm, args.steps, stream)
        del inp_rm
    if headline:
        # ---- per-step spread, warm and cache-cold (512 MB written before each step)
        res["warm_per_step"] = spread(per_step(step, args.steps, stream), T)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        res["cold_per_step"] = dict(spread(per_step(step, args.steps, stream, flush), T), flush_bytes=512 << 20)
        del flush
        res["graph_per_step"] = graph_per_step(step, args.steps, stream, T, y)

    # ---- routing facts of this batch (N, non-empty experts)
    n_kept = int(aux["n_kept"].item())
    kept = aux["kept"].cpu().numpy()
    nonempty = int((kept > 0).sum())
    l_aux = float(aux["l_aux"].item())

    # ---- stages, each through its own entry point on the same buffers
    cap = moe.moe_capacity(desc)
    max_rows = min(A, Et * cap) if cap < moe.INT32_MAX else A
    topk_idx, topk_w, dest_row = aux["topk_idx"], aux["topk_w"], aux["dest_row"]
    counts, keptb, offsets = torch.empty(Et, **i32), torch.empty(Et, **i32), torch.empty(Et + 1, **i32)
    src = torch.empty(A, **i32)
    x_perm = torch.empty((max_rows, d), dtype=inputs.torch_dtype(cfg), device=dev)
    h_tmp = torch.empty((max_rows, f), dtype=inputs.torch_dtype(cfg), device=dev)
    y_perm = torch.empty((max_rows, d), dtype=inputs.torch_dtype(cfg), device=dev)
    pm = torch.empty(Et, **f32)
    ws_r = moe.workspace(desc, moe.MOE_WS_ROUTE)
    ws_p = moe.workspace(desc, moe.MOE_WS_PERMUTE)
    ws_f = moe.workspace(desc, moe.MOE_WS_FFN)
    R = args.stage_reps

    def route():
        if cfg.get("gate") == "hash":
            moe.moe_route_hash(desc, None, topk_idx, topk_w)
            return
        moe.moe_route(desc, inp["x"], inp["w_router"], inp["logit_bias"], inp["select_bias"], None, 0,
                      topk_idx, topk_w, None, pm, ws_r)

    def permute():
        moe.moe_permute(desc, topk_idx, inp["x"], cap, counts, keptb, offsets, dest_row, src, x_perm, None, ws_p)

    def permute_tables():  # what the layer runs: routing tables only, no row gather
        moe.moe_permute(desc, topk_idx, None, cap, counts, keptb, offsets, dest_row, src, None, None, ws_p)

    def gemm1():  # the layer's gate/up GEMM: rows read from x through src_token
        moe.moe_grouped_ffn_rows(desc, inp["x"], src, offsets, max_rows, inp["w_gate"], inp["w_up"],
                                 inp["w_down"], h_tmp, y_perm, moe.MOE_FFN_GEMM1, ws_f)

    def gemm1_gathered():  # the stage-wise path: the same GEMM on the gathered x_perm
        moe.moe_grouped_ffn(desc, x_perm, offsets, max_rows, inp["w_gate"], inp["w_up"], inp["w_down"], h_tmp,
                            y_perm, moe.MOE_FFN_GEMM1, ws_f)

    def gemm2():
        moe.moe_grouped_ffn(desc, x_perm, offsets, max_rows, inp["w_gate"], inp["w_up"], inp["w_down"], h_tmp,
                            y_perm, moe.MOE_FFN_GEMM2, ws_f)

    y_sh = None
    shared_fn = wo_fn = None
    if cfg.get("n_shared"):
        # the shared expert is one group of all T rows of x: a dense descriptor
        dsh = moe.desc_from_cfg(dict(cfg, H=1, E=1, K=1, n_shared=0, has_wo=0, **DENSE))
        off_sh = torch.tensor([0, T], **i32)
        h_sh = torch.empty((T, f), dtype=inputs.torch_dtype(cfg), device=dev)
        y_sh = torch.empty((T, h), dtype=inputs.torch_dtype(cfg), device=dev)
        ws_sh = moe.workspace(dsh, moe.MOE_WS_FFN)

        def shared_fn():
            moe.moe_grouped_ffn(dsh, inp["x"], off_sh, T, inp["sh_gate"], inp["sh_up"], inp["sh_down"], h_sh,
                                y_sh, 0, ws_sh)
    y_cat = torch.empty((T, h), dtype=inputs.torch_dtype(cfg), device=dev) if cfg.get("has_wo") else None
    if cfg.get("has_wo"):
        # W_o is the second GEMM of a one-group descriptor with f = h
        dwo = moe.desc_from_cfg(dict(cfg, H=1, E=1, K=1, f=h, n_shared=0, has_wo=0, **DENSE))
        off_wo = torch.tensor([0, T], **i32)
        ws_wo = moe.workspace(dwo, moe.MOE_WS_FFN)

        def wo_fn():
            moe.moe_grouped_ffn(dwo, None, off_wo, T, None, None, inp["w_o"], y_cat, y, moe.MOE_FFN_GEMM2, ws_wo)

    def combine():
        moe.moe_combine(desc, dest_row, topk_w, y_perm, y_sh, y_cat if y_cat is not None else y)

    route()
    permute()
    if args.counters:
        torch.cuda.synchronize()
        cp_src = torch.ones(1 << 29, dtype=torch.int16, device=dev)  # 1 GiB
        cp_dst = torch.empty_like(cp_src)
        cp_dst.copy_(cp_src)
        torch.cuda.synchronize()
        # every stage three times, each on its own (the layer's routing tables,
        # the stage-wise gather, both expert GEMMs, the combine)
        for fn in (route, permute, gemm1, gemm2, combine):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
        print(json.dumps({"counters_run": name, "copy_bytes": 1 << 30}), flush=True)
        return None
    gemm1()
    gemm2()
    if shared_fn:
        shared_fn()
    t_route = timed(route, R, stream)
    t_perm = timed(permute, R, stream)
    t_tables = timed(permute_tables, R, stream)
    permute()  # leave x_perm and the tables in place for the gathered-row GEMM
    t_g1_gathered = timed(gemm1_gathered, R, stream)
    t_g1 = timed(gemm1, R, stream)
    t_g2 = timed(gemm2, R, stream)
    t_comb = timed(combine, R, stream)
    t_sh = timed(shared_fn, R, stream) if shared_fn else None
    t_wo = timed(wo_fn, R, stream) if wo_fn else None

    # algorithmic work (bytes moved / flops the method needs), with this batch's N
    n_act = 2 if cfg["act"] == "swiglu" else 1
    gemm1_flops = 2.0 * n_act * n_kept * d * f
    gemm2_flops = 2.0 * n_kept * f * d
    route_bytes = A * 8 if cfg.get("gate") == "hash" else T * h * esz + Et * d * esz + A * 8
    # the gather reads each (sub-)token's slice once (token-major) and writes it to each of its kept rows
    dest = aux["dest_row"].view(T * H, K)
    distinct_rows = int((dest >= 0).any(dim=1).sum().item())
    permute_bytes = distinct_rows * d * esz + n_kept * d * esz + A * 4 * 2
    combine_bytes = n_kept * d * esz + A * 8 + T * h * esz + (T * h * esz if cfg.get("n_shared") else 0)
    w_bytes = nonempty * (n_act + 1) * d * f * esz

    def frac(x, peak):
        return None if x is None else x / peak

    g1_tfs = gemm1_flops / (t_g1 * 1e-3) / 1e12
    g2_tfs = gemm2_flops / (t_g2 * 1e-3) / 1e12
    stages = {
        "route_ms": t_route, "route_hbm_frac": frac(route_bytes / (t_route * 1e-3) / 1e9, HBM_PEAK_GBS),
        "permute_ms": t_perm, "permute_hbm_frac": frac(permute_bytes / (t_perm * 1e-3) / 1e9, HBM_PEAK_GBS),
        "permute_tables_ms": t_tables,
        "gemm1_ms": t_g1, "gemm1_tflops": g1_tfs, "gemm1_mfma_frac": g1_tfs / MFMA_BF16_PEAK_TFS,
        "gemm1_gathered_ms": t_g1_gathered,
        "gemm2_ms": t_g2, "gemm2_tflops": g2_tfs, "gemm2_mfma_frac": g2_tfs / MFMA_BF16_PEAK_TFS,
        "combine_ms": t_comb,
        "combine_hbm_frac": combine_bytes / (t_comb * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "shared_ffn_ms": t_sh,
        "shared_ffn_tflops": None if t_sh is None else 2.0 * (n_act + 1) * T * h * f / (t_sh * 1e-3) / 1e12,
        "w_o_ms": t_wo,
        "w_o_tflops": None if t_wo is None else 2.0 * T * h * h / (t_wo * 1e-3) / 1e12,
        "sum_of_stages_ms": t_route + t_tables + t_g1 + t_g2 + t_comb + (t_sh or 0.0) + (t_wo or 0.0),
        "ffn_mfma_frac": (gemm1_flops + gemm2_flops) / ((t_g1 + t_g2) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
        "ffn_weight_bytes": w_bytes,
    }
    # the FFN against its attainable roofline min(MFMA peak, AI x HBM BW): AI counts
    # the weights of non-empty experts, the x rows read and the y rows written
    # (plus the shared expert's weights and its x/y when there is one)
    ffn_flops = gemm1_flops + gemm2_flops
    ffn_bytes = w_bytes + 2.0 * n_kept * d * esz
    ffn_ms = t_g1 + t_g2
    if cfg.get("n_shared"):
        ffn_flops += 2.0 * (n_act + 1) * T * h * f
        ffn_bytes += (n_act + 1) * h * f * esz + 2.0 * T * h * esz
        ffn_ms += t_sh
    ai = ffn_flops / ffn_bytes
    attain = min(MFMA_BF16_PEAK_TFS, ai * HBM_PEAK_GBS / 1e3)
    ffn_tfs = ffn_flops / (ffn_ms * 1e-3) / 1e12
    stages.update({
        "ffn_flop_per_byte": ai, "ffn_bound": "mfma" if attain >= MFMA_BF16_PEAK_TFS else "hbm",
        "ffn_attainable_tflops": attain, "ffn_tflops": ffn_tfs, "ffn_attainable_frac": ffn_tfs / attain,
    })
    total_flops = gemm1_flops + gemm2_flops + 2.0 * T * H * d * E
    if cfg.get("has_wo"):
        total_flops += 2.0 * T * h * h
    if cfg.get("n_shared"):
        total_flops += 2.0 * (n_act + 1) * T * h * f

    res.update({
        "ms_per_step": ms_step, "tokens_per_s": tok_s, "tflops": total_flops / (ms_step * 1e-3) / 1e12,
        "dtype": cfg["dtype"],
        "config": {"workload": name, "tokens": T, "hidden": h, "heads": H, "experts": E, "top_k": K,
                   "ffn": f, "act": cfg["act"], "score": cfg["score"], "capacity_factor": cfg["capacity_factor"],
                   "parallelism": "single GPU", **({"variant": over} if over else {})},
        "n_kept": n_kept, "n_dropped": A - n_kept, "nonempty_experts": nonempty, "l_aux": l_aux,
        "stages": stages,
    })
    if not headline:
        del inp, ws, ws_r, ws_p, ws_f, x_perm, h_tmp, y_perm
        torch.cuda.empty_cache()
        return res

    res["roofline"] = {
        "kernel": "grouped GEMM1: gate/up projections + SwiGLU" if n_act == 2 else
                  "grouped GEMM1: projection + GELU",
        "bound": "mfma", "achieved": g1_tfs, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
        "frac": g1_tfs / MFMA_BF16_PEAK_TFS, "traffic": traffic_from_profile("gemm1", name),
        "flops_per_launch": gemm1_flops, "launch_ms": t_g1,
    }

    # ---- CPU oracle baseline on a bounded sample: the first Ts tokens as a batch
    cpu = None
    if not args.no_cpu:
        from oracle import oracle as orc

        def to_np(t):
            if t is None:
                return None
            t = t.detach().cpu().contiguous()
            return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

        log("[bench] copying weights to the host for the CPU oracle")
        host = {k: to_np(v) for k, v in inp.items()}
        threads = orc.num_threads()
        Ts = 2
        elapsed = 0.0
        while True:
            t0 = time.perf_counter()
            orc.layer_forward(cfg, host, host["x"][:Ts], T=Ts)
            elapsed = time.perf_counter() - t0
            if elapsed >= args.cpu_seconds * 0.6 or Ts >= T:
                break
            Ts = min(T, Ts * 4, max(Ts + 1, int(Ts * args.cpu_seconds / max(elapsed, 1e-3))))
        log(f"[bench] oracle: {Ts} tokens in {elapsed:.2f} s on {threads} threads")
        cpu = {"value": Ts / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"first {Ts} tokens of the {name} batch as their own batch (capacity for {Ts} "
                         f"tokens), full weights; fp64 C oracle, {elapsed:.1f} s",
               "cpu_model": cpu_model()}
        del host
        # the tiny fp32 layer (all 256 tokens) on one thread and on all of them
        tiny = inputs.CONFIGS["tiny_f32"]
        th = {k: to_np(v) for k, v in inputs.make_inputs(tiny, "cpu", seed=0).items()}
        for n_thr, key in ((1, "tiny_f32_single_thread"), (threads, "tiny_f32_all_threads")):
            orc.set_num_threads(n_thr)
            reps, t0 = 0, time.perf_counter()
            while True:
                orc.layer_forward(tiny, th, th["x"])
                reps += 1
                el = time.perf_counter() - t0
                if el >= 1.0:
                    break
            cpu[key] = {"tokens_per_s": reps * tiny["T"] / el, "ms_per_layer": el / reps * 1e3, "threads": n_thr}
        orc.set_num_threads(threads)
    res["cpu_baseline"] = cpu
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library implements the "
              "one-GPU layer, and its expert/head-parallel sharding exists as a design only.", file=sys.stderr)
        sys.exit(2)
    import torch

    from mixture_experts_layer_45_amd import inputs

    if args.shard:
        return shard_bench(args)
    torch.cuda.set_device(0)
    name = args.workload or inputs.BENCH_WORKLOAD
    over = {}
    for kv in args.set:
        k, v = kv.split("=", 1)
        for conv in (int, float):
            try:
                v = conv(v)
                break
            except ValueError:
                pass
        over[k] = v
    cfg = inputs.variant(name, **over)
    head = measure_layer(args, cfg, over, headline=True)
    if head is None or args.train:
        return
    others = {}
    if not args.only and not over and args.workload is None:
        for wname in inputs.CONFIGS:
            if wname == cfg["name"]:
                continue
            r = measure_layer(args, inputs.variant(wname), {}, headline=False)
            st = r["stages"]
            others[wname] = {
                "ms_per_step": r["ms_per_step"], "tokens_per_s": r["tokens_per_s"], "tflops": r["tflops"],
                "dtype": r["dtype"], "weights": r["weights"], "n_kept": r["n_kept"],
                "nonempty_experts": r["nonempty_experts"],
                "l_aux": r["l_aux"],
                "ffn_mfma_frac": st["ffn_mfma_frac"], "ffn_attainable_frac": st["ffn_attainable_frac"],
                "ffn_bound": st["ffn_bound"], "gemm1_mfma_frac": st["gemm1_mfma_frac"],
                "gemm2_mfma_frac": st["gemm2_mfma_frac"], "route_hbm_frac": st["route_hbm_frac"],
                "permute_hbm_frac": st["permute_hbm_frac"], "combine_hbm_frac": st["combine_hbm_frac"],
                "stages": st,
            }
    out = {
        "metric": "MoE-layer fwd tokens/sec on 1 GPU (grouped-FFN % MFMA peak; route/permute % HBM BW)",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"], "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": head["config"], "tflops": head["tflops"],
        "weights": head["weights"], "row_major_ms_per_step": head.get("row_major_ms_per_step"),
        "n_kept": head["n_kept"], "n_dropped": head["n_dropped"], "nonempty_experts": head["nonempty_experts"],
        "l_aux": head["l_aux"],
        "warm_per_step": head["warm_per_step"], "cold_per_step": head["cold_per_step"],
        "graph_per_step": head["graph_per_step"], "stages": head["stages"], "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "workloads": others or None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
