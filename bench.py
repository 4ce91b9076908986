"""Benchmark of the MoE-layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--prefill-workload NAME|none]
                [--no-cpu-baseline] [--no-flush]
                [--capacity-factor CF --capacity-policy drop|reroute] [--gate-norm] [--noise-std SIGMA]
                [--expert-act gelu|silu|swiglu] [--router-hidden D_R]
python bench.py --import-counters FETCH_CSV WRITE_CSV --workload NAME

One step = the whole layer (router, dispatch, W1 GEMM + activation, W2 GEMM,
combine) over one batch of seeded synthetic input already resident in HBM.
The metric has two halves, measured in one run:
  * decode (default workload: 8 tokens, d = d_ff = 8192, 128 experts), bound
    by HBM bandwidth: the top-level value;
  * prefill (default: 4096 tokens, d = 4096, d_ff = 16384, 16 experts, skewed
    routing), bound by the bf16 matrix cores: the nested "prefill" object.
For each: K timed steps after W warm-ups, each step bracketed by HIP events on
the stream it runs on, with a 512 MB buffer read between steps (outside the
events, a matrix-vector product that writes 256 KB) so the 256 MB Infinity
Cache cannot carry weights from one step to the next; tokens/s from the
median step.  (Reading evicts the cache as writing does; a write touch would
also leave dirty lines whose write-back slows the next step's kernels.)  Then K more steps replay the layer
through the stage entry points (router, permute, W1, W2, combine) with events
between the stages: each stage's average duration, and the roofline of both
expert GEMMs (algorithmic bytes or flops per launch / duration), the longer
one being the dominant kernel.  For a bf16 workload bound by the matrix
cores, `library_dense_gemm` adds context: the vendor library's dense bf16
product (torch.matmul, i.e. hipBLASLt) with the W1 GEMM's flops, timed the
same way outside the layer steps.  The CPU oracle is timed beside it on a
bounded sample of the same workload, on one host core and on all of them.

--import-counters turns two rocprofv3 --pmc runs of this benchmark with
--calibrate-copy (FETCH_SIZE, then WRITE_SIZE) into the HBM traffic per launch
of the W1 and W2 GEMMs, each counter scaled by what it reads for the plain
1 GiB copy, stored in profiles/traffic.json with a hash of the kernel sources
(a changed kernel reads as traffic null).
"""
import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "decode-bf16-T8-d8192-E128"
DEFAULT_PREFILL = "prefill-skewed-bf16-T4096-d4096-E16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector
FLUSH_BYTES = 512 << 20


def make_touch(torch, dev):
    """A read of FLUSH_BYTES between steps: a matrix-vector product over the
    buffer viewed as fp32 rows of 2048 (rocBLAS gemv, bandwidth-bound), whose
    only write is its 256 KB result vector."""
    buf = torch.zeros(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    mat = buf.view(torch.float32).view(-1, 2048)
    vec = torch.zeros(2048, dtype=torch.float32, device=dev)
    res = torch.empty(mat.shape[0], dtype=torch.float32, device=dev)
    return lambda: torch.mv(mat, vec, out=res)
COPY_BYTES = 1 << 30           # the calibration copy


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--prefill-workload", default=DEFAULT_PREFILL,
                    help="second workload measured in the same run ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="oracle seconds per timed leg (about)")
    ap.add_argument("--no-flush", action="store_true", help="do not read a 512 MB buffer between steps")
    ap.add_argument("--capacity-factor", type=float, default=0.0, help="0: dropless dispatch")
    ap.add_argument("--capacity-policy", choices=["drop", "reroute"], default="drop")
    ap.add_argument("--gate-norm", action="store_true", help="gates renormalised over the k chosen experts")
    ap.add_argument("--noise-std", type=float, default=0.0, help="sigma of Gaussian router-logit noise")
    ap.add_argument("--expert-act", choices=["gelu", "silu", "swiglu"], default="gelu",
                    help="expert activation (swiglu: W1 holds 2 d_ff gate/up rows)")
    ap.add_argument("--router-hidden", type=int, default=0,
                    help="width of the two-layer router's hidden layer (0: linear router; the pages use d/4)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy first (reference kernel for HBM byte counters)")
    ap.add_argument("--import-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="counter_collection.csv of two rocprofv3 --pmc runs of this bench with --calibrate-copy "
                         "(FETCH_SIZE, then WRITE_SIZE) -> profiles/traffic.json (no GPU needed)")
    return ap.parse_args(argv)


KERNEL_SOURCES = {"f32": "gemm_f32.hip", "streaming": "gemm_stream.hip", "tiled": "gemm_tiled.hip"}


def gemm_path_name(cfg):
    """The library's automatic expert-GEMM kernel for a workload."""
    import sparse_mixture_experts_03_amd as moe
    if cfg["w"] == moe.F32:
        return "f32"
    if cfg["T"] <= 16 or (cfg["w"] == moe.INT4_G128 and (cfg["d"] % 1024 or cfg["d_ff"] % 1024)):
        return "streaming"
    return "tiled"


# string and character literals (kept) and comments (dropped) of a C/C++/HIP source
_SOURCE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def source_code_only(text):
    """A source's code without its comments, whitespace collapsed: what a
    counter measurement depends on."""
    text = _SOURCE_TOKENS.sub(lambda m: " " if m.group(0).startswith("/") else m.group(0), text)
    return " ".join(text.split())


def kernel_source_hash(kernel, csrc=None):
    """Hash of the code that defines a grouped-GEMM kernel: its own file, the
    shared headers and the launch parameters chosen in moe_api.hip (comments
    and layout left out, so editing a comment keeps the counters valid)."""
    csrc = csrc or os.path.join(ROOT, "sparse_mixture_experts_03_amd", "csrc")
    path = kernel.rsplit("_", 1)[-1]
    h = hashlib.sha256()
    for f in ("common.hpp", "launch.hpp", "moe_api.hip", KERNEL_SOURCES[path]):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + source_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def load_traffic(workload, kernel):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel and
    workload, if the committed measurement was taken on the current sources."""
    if not os.path.exists(TRAFFIC):
        return None
    with open(TRAFFIC) as f:
        table = json.load(f)
    rec = table.get(f"{kernel}|{workload}")
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------ timing

class StreamTimer:
    """HIP events on one stream: elapsed milliseconds between marks."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def mark(self):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record(self.stream)
        return ev


def workload_args(cfg, args, moe):
    act_code = {"gelu": moe.ACT_GELU, "silu": moe.ACT_SILU, "swiglu": moe.ACT_SWIGLU}[args.expert_act]
    cfg["ffn"] = act_code
    cfg["router_hidden"] = args.router_hidden
    policy = moe.CAPACITY_REROUTE if args.capacity_policy == "reroute" else moe.CAPACITY_DROP
    return moe.config(cfg["T"], cfg["d"], cfg["d_ff"], cfg["E"], cfg["k"], cfg["act"], cfg["w"], tau=cfg["tau"],
                      use_gumbel=cfg["gumbel"], seed=0, capacity_factor=args.capacity_factor, capacity_policy=policy,
                      gate_norm=int(args.gate_norm), noise_std=args.noise_std, expert_act=act_code,
                      router_hidden=args.router_hidden)


def measure(name, args, dev, torch, np, moe, moe_synth, with_cpu):
    """One workload: the timed layer steps, the staged per-kernel replay, the
    rooflines and (optionally) the CPU oracle.  Returns the JSON object."""
    cfg = moe_synth.workload(name)
    c = workload_args(cfg, args, moe)
    T, d, d_ff, E, k = cfg["T"], cfg["d"], cfg["d_ff"], cfg["E"], cfg["k"]
    n1 = 2 * d_ff if cfg["ffn"] == moe.ACT_SWIGLU else d_ff  # W1 rows
    print(f"[bench] generating {name} on {dev}", file=sys.stderr, flush=True)
    inp = moe_synth.generate(cfg, device=dev, seed=0)
    torch.cuda.synchronize()
    layer = moe.MoELayerForward(c, device=dev)
    stream = torch.cuda.current_stream()
    tm = StreamTimer(torch, stream)
    flush = None if args.no_flush else make_touch(torch, dev)
    run = lambda: layer(inp["x"], inp["Wg"], inp["bias"], inp["W1"], inp["W2"], inp["S1"], inp["S2"],
                        W_in=inp["W_in"], b_in=inp["b_in"])

    print(f"[bench] {name}: {args.warmup} warm-up + {args.steps} timed steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    marks = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if flush is not None:
            flush()  # reads 512 MB: evicts the previous step's lines from the MALL
        a = tm.mark()
        run()
        marks.append((a, tm.mark()))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in marks]
    med = statistics.median(step_ms)

    counts = layer.counts.cpu().numpy()
    kept = int(counts.sum())
    active = int((counts > 0).sum())
    wbits = {moe.F32: 32, moe.BF16: 16, moe.INT4_G128: 4}[cfg["w"]]
    abytes = 4 if cfg["act"] == moe.F32 else 2
    hbytes = 4 if cfg["w"] == moe.F32 else 2
    w2_bytes = d * d_ff * wbits // 8 + (d * d_ff // 128 * 2 if cfg["w"] == moe.INT4_G128 else 0)
    w1_bytes = w2_bytes * n1 // d_ff
    Tk = kept  # dispatched rows (T k without a capacity)

    # staged replay: the same kernels as the layer step, with events between the stages
    print(f"[bench] {name}: staged replay", file=sys.stderr, flush=True)
    H = torch.empty((Tk, d_ff), dtype=torch.float32 if cfg["w"] == moe.F32 else torch.bfloat16, device=dev)
    Y = torch.empty((Tk, d), dtype=torch.float32, device=dev)
    y2 = torch.empty_like(layer.y)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_token = torch.empty(Tk, dtype=torch.int32, device=dev)
    pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    r_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    r_gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    r_ws = torch.empty(max(256, moe.moe_router_workspace_size(c)), dtype=torch.uint8, device=dev)
    staged = args.capacity_factor == 0  # a capacity adds stages that have no entry point of their own
    stage_ms = {}
    if staged:
        stages = [
            ("router", lambda: moe.moe_router(c, inp["x"], inp["Wg"], inp["bias"], r_ids, r_gates, r_ws,
                                              W_in=inp["W_in"], b_in=inp["b_in"])),
            ("permute", lambda: moe.moe_permute(c, r_ids, cnt, offsets, sorted_token, pos)),
            ("w1", lambda: moe.moe_grouped_gemm(c, 1, inp["x"], sorted_token, offsets, inp["W1"], inp["S1"], H)),
            ("w2", lambda: moe.moe_grouped_gemm(c, 2, H, None, offsets, inp["W2"], inp["S2"], Y)),
            ("combine", lambda: moe.moe_combine(c, Y, pos, r_gates, y2)),
        ]
        for _ in range(2):
            for _, fn in stages:
                fn()
        torch.cuda.synchronize()
        per = {s: [] for s, _ in stages}
        for _ in range(args.steps):
            if flush is not None:
                flush()
            prev = tm.mark()
            for s, fn in stages:
                fn()
                nxt = tm.mark()
                per[s].append((prev, nxt))
                prev = nxt
        torch.cuda.synchronize()
        stage_ms = {s: statistics.mean(a.elapsed_time(b) for a, b in v) for s, v in per.items()}
        assert torch.equal(r_ids, layer.expert_ids), "staged routing differs from the layer's"

    path = gemm_path_name(cfg)
    compute_peak = FP32_PEAK_TFLOPS if cfg["w"] == moe.F32 else BF16_PEAK_TFLOPS
    ridge = compute_peak * 1e12 / (HBM_PEAK_GBS * 1e9)

    def roofline(which):
        if which == 1:
            nbytes = active * w1_bytes + Tk * d * abytes + Tk * d_ff * hbytes
            flops = 2.0 * Tk * d * n1
        else:
            nbytes = active * w2_bytes + Tk * d_ff * hbytes + Tk * d * 4
            flops = 2.0 * Tk * d_ff * d
        kernel = f"moe_grouped_gemm_w{which}_{path}"
        ms = stage_ms.get(f"w{which}")
        if ms is None:
            return None
        if flops / nbytes < ridge:
            achieved = nbytes / (ms * 1e-3) / 1e9
            r = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                     frac=round(achieved / HBM_PEAK_GBS, 4))
        else:
            achieved = flops / (ms * 1e-3) / 1e12
            r = dict(bound="alu" if cfg["w"] == moe.F32 else "mfma", achieved=round(achieved, 1),
                     peak=compute_peak, unit="TFLOP/s", frac=round(achieved / compute_peak, 4))
        r.update(traffic=load_traffic(name, kernel), kernel=kernel, avg_launch_ms=round(ms, 4),
                 algorithmic_bytes=nbytes, algorithmic_flops=flops)
        return r

    roofs = [r for r in (roofline(1), roofline(2)) if r is not None]
    roofs.sort(key=lambda r: -r["avg_launch_ms"])

    d_r = args.router_hidden
    router_w_bytes = (d_r * d * abytes + d_r * E * abytes) if d_r else d * E * abytes
    step_bytes = (T * d * abytes + router_w_bytes + active * (w1_bytes + w2_bytes) + T * d * abytes + T * k * 8
                  + E * 4)
    step_flops = 2.0 * Tk * d * n1 + 2.0 * Tk * d_ff * d
    out = {
        "metric": "MoE-layer tokens/s",
        "value": round(T / (med * 1e-3), 1),
        "unit": "tokens/s",
        "ms_per_step": round(med, 4),
        "ms_per_step_mean": round(statistics.mean(step_ms), 4),
        "ms_per_step_min": round(min(step_ms), 4),
        "timed_wall_s": round(wall, 3),
        "dtype": {moe.F32: "f32", moe.BF16: "bf16", moe.INT4_G128: "bf16 (int4 g128 experts)"}[cfg["w"]],
        "config": {"workload": name, "T": T, "d": d, "d_ff": d_ff, "E": E, "k": k,
                   "router_bias": bool(cfg["bias"]), "tau": cfg["tau"], "gumbel": bool(cfg["gumbel"]),
                   "capacity_factor": args.capacity_factor,
                   "capacity_policy": args.capacity_policy if args.capacity_factor > 0 else None,
                   "gate_norm": int(args.gate_norm), "noise_std": args.noise_std, "expert_act": args.expert_act,
                   "router_hidden": args.router_hidden, "mall_flush_between_steps": "read 512 MB" if flush is not None else None},
        "layer_hbm_frac": round(step_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_mfma_frac": round(step_flops / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "active_experts": active,
        "counts_var": float(np.var(counts)),
        "assignments_kept": kept,
        "stage_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "roofline": roofs[0] if roofs else None,
        "roofline_other": roofs[1] if len(roofs) > 1 else None,
    }
    del layer, H, Y
    torch.cuda.empty_cache()
    if roofs and roofs[0]["bound"] == "mfma" and cfg["w"] == moe.BF16:
        out["library_dense_gemm"] = library_dense_gemm(torch, Tk, n1, d, flush)
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args, np, moe_synth)
    del inp, flush
    torch.cuda.empty_cache()
    return out


def library_dense_gemm(torch, M, N, K, flush, reps=10):
    """Context for the MFMA fraction, outside every timed step: the vendor
    library's dense bf16 product with the W1 GEMM's flops (M dispatched rows,
    N weight rows, K inputs; torch.matmul, i.e. hipBLASLt), no gather and no
    per-expert tiles.  Median of `reps` launches, each after the same MALL
    flush as the layer steps."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(1)
    a = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((K, N), generator=g, device=dev).to(torch.bfloat16)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    torch.matmul(a, b, out=c)
    ms = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(a, b, out=c)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = statistics.median(ms)
    tflops = 2.0 * M * N * K / (med * 1e-3) / 1e12
    del a, b, c
    return {"op": "torch.matmul bf16 (hipBLASLt), dense", "shape_mnk": [M, N, K], "ms": round(med, 4),
            "tflops": round(tflops, 1), "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}


def main():
    args = parse()
    if args.import_counters:
        import_counters(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer runs on a single "
              f"MI355X: no collectives or multi-GPU sharding are built)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import moe_synth
    import sparse_mixture_experts_03_amd as moe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    top = measure(args.workload, args, dev, torch, np, moe, moe_synth, not args.no_cpu_baseline)
    out = {"metric": top.pop("metric"), "value": top.pop("value"), "unit": top.pop("unit"), "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": top.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": top.pop("dtype"),
           "data": "synthetic (seeded N(0,1/fan_in) weights, N(0,1) tokens)", "config": top.pop("config")}
    out.update(top)
    if args.prefill_workload and args.prefill_workload != "none":
        pre = measure(args.prefill_workload, args, dev, torch, np, moe, moe_synth, not args.no_cpu_baseline)
        pre["steps"], pre["warmup"] = args.steps, args.warmup
        out["prefill"] = pre
    print(json.dumps(out))


# ------------------------------------------------------------------ CPU oracle

def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(cfg, inp, args, np, moe_synth):
    """The oracle on a bounded sample of the workload: the routing of every
    token (prorated to the sample) plus the expert FFNs and combine of the
    sampled tokens, timed on one host core and then on all of them (disjoint
    token shards in threads; the oracle call releases the GIL)."""
    import concurrent.futures

    from oracle import oracle as oracle_mod
    orc = oracle_mod.get()
    T, E = cfg["T"], cfg["E"]
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    xb, wgb = moe_synth.to_bits(inp["x"]), moe_synth.to_bits(inp["Wg"])
    enc = None
    if inp["W_in"] is not None:
        enc = (moe_synth.to_bits(inp["W_in"]), inp["b_in"].cpu().numpy())
    limited = args.capacity_factor > 0
    route_kw = dict(bias=bias, tau=float(np.float32(cfg["tau"])), encoder=enc, use_gumbel=cfg["gumbel"], seed=0,
                    want_zp=limited, gate_norm=int(args.gate_norm), noise_std=float(np.float32(args.noise_std)))
    t0 = time.perf_counter()
    ref = orc.route(xb, wgb, cfg["k"], cfg["act"], **route_kw)
    if limited:
        ref = orc.capacity_dispatch(ref, float(np.float32(args.capacity_factor)),
                                    1 if args.capacity_policy == "reroute" else 0)
    t_route = time.perf_counter() - t0
    threads = _threads()
    # rough per-token FFN cost (fp64, about 1.5 ns per multiply-add) sizes the one-core sample
    per_tok = 2.0 * cfg["k"] * cfg["d"] * cfg["d_ff"] * 1.5e-9
    n1 = int(max(1, min(T, args.cpu_seconds // max(per_tok, 1e-9))))
    n_all = int(min(T, max(threads, n1 * threads)))
    all_tokens = np.unique(np.linspace(0, T - 1, n_all).round().astype(np.int64))
    one_tokens = all_tokens[np.unique(np.linspace(0, len(all_tokens) - 1, min(n1, len(all_tokens))).round()
                                      .astype(np.int64))]
    used = sorted(e for e in set(ref["ids"][all_tokens].reshape(-1).tolist()) if e >= 0)
    W1, W2 = [None] * E, [None] * E
    S1 = [None] * E if inp["S1"] is not None else None
    S2 = [None] * E if inp["S2"] is not None else None
    for e in used:
        W1[e] = moe_synth.to_bits(inp["W1"][e])
        W2[e] = moe_synth.to_bits(inp["W2"][e])
        if S1 is not None:
            S1[e] = moe_synth.to_bits(inp["S1"][e])
            S2[e] = moe_synth.to_bits(inp["S2"][e])
    ffn = lambda toks: orc.forward_tokens(xb, ref["ids"], ref["gate_p"], W1, W2, cfg["act"], cfg["w"], cfg["d_ff"],
                                          toks, S1=S1, S2=S2, act=cfg.get("ffn", 0))
    print(f"[bench] oracle: {len(one_tokens)} tokens on 1 core, {len(all_tokens)} on {threads}",
          file=sys.stderr, flush=True)
    # each leg repeats its sample until about cpu_seconds of oracle work has been timed
    reps_one, t0 = 0, time.perf_counter()
    while True:
        ffn(one_tokens)
        reps_one += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    t_one = (time.perf_counter() - t0) / reps_one
    shards = [s for s in np.array_split(all_tokens, threads) if len(s)]
    reps_all = 0
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(shards)) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(ffn, shards))
            reps_all += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        t_all = (time.perf_counter() - t0) / reps_all
    # routing of the whole batch, prorated to the sample (on all cores: the same work split over the threads)
    one = len(one_tokens) / (t_route * len(one_tokens) / T + t_one)
    allc = len(all_tokens) / (t_route * len(all_tokens) / T / threads + t_all)
    return {"value": round(allc, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(),
            "sample": (f"{len(all_tokens)} of {T} tokens on {threads} threads (disjoint token shards, repeated "
                       f"{reps_all}x; routing{' and capacity dispatch' if limited else ''} of all {T} tokens "
                       f"prorated), single-threaded fp64 C oracle per shard; {t_all * reps_all:.1f} s measured"),
            "one_core": {"value": round(one, 3), "unit": "tokens/s", "cores": 1,
                         "sample": (f"{len(one_tokens)} of {T} tokens, repeated {reps_one}x; "
                                    f"{t_one * reps_one + t_route:.1f} s measured")}}


# ------------------------------------------------------------------ counters

# kernel base name -> (path, index of the WHICH template argument)
GEMM_KERNELS = {"gemm_tiled_bf16_kernel": ("tiled", 0), "gemm_tiled_kernel": ("tiled", 1),
                "gemm_stream_kernel": ("streaming", 1), "gemm_f32_kernel": ("f32", 0)}


def gemm_of(kernel_name):
    """(path, which) of a grouped-GEMM kernel's demangled name, or None."""
    for base, (path, idx) in GEMM_KERNELS.items():
        tag = f"::{base}<"
        if tag in kernel_name:
            targs = kernel_name.split(tag, 1)[1].split(">", 1)[0].split(",")
            return path, int(targs[idx].strip())
    return None


def _counter_rows(path, counter):
    with open(path) as f:
        return [r for r in csv.DictReader(f) if r.get("Counter_Name") == counter]


def import_counters(args):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the W1 and W2 GEMM launches
    of one bench run with --calibrate-copy, each scaled by what the same counter
    reads for that run's plain 1 GiB device copy, into profiles/traffic.json."""
    fetch_csv, write_csv = args.import_counters
    fr = _counter_rows(fetch_csv, "FETCH_SIZE")
    wr = _counter_rows(write_csv, "WRITE_SIZE")
    # the runtime's device-to-device copy kernel (torch's elementwise copy kernels of the input generation are
    # not the calibration copy)
    copies = lambda rows: [float(r["Counter_Value"]) for r in rows if "copybuffer" in r["Kernel_Name"].lower()]
    cf, cw = copies(fr), copies(wr)
    if not cf or not cw:
        raise SystemExit("no copy kernel in the counter files: run the bench with --calibrate-copy")
    fetch_scale = COPY_BYTES / (max(cf) * 1024)
    write_scale = COPY_BYTES / (max(cw) * 1024)
    table = {}
    if os.path.exists(TRAFFIC):
        with open(TRAFFIC) as f:
            table = json.load(f)
    for which in (1, 2):
        for kpath in KERNEL_SOURCES:
            sel = lambda rows: [r for r in rows if gemm_of(r["Kernel_Name"]) == (kpath, which)]
            f_rows, w_rows = sel(fr), sel(wr)
            if not f_rows or not w_rows:
                continue
            kname = f"moe_grouped_gemm_w{which}_{kpath}"
            fb = statistics.median(float(r["Counter_Value"]) for r in f_rows) * 1024 * fetch_scale
            wb = statistics.median(float(r["Counter_Value"]) for r in w_rows) * 1024 * write_scale
            table[f"{kname}|{args.workload}"] = {
                "bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb), "write_bytes": int(wb),
                "fetch_scale": round(fetch_scale, 5), "write_scale": round(write_scale, 5),
                "dispatches": len(f_rows), "kernel": f_rows[0]["Kernel_Name"][:96],
                "source_hash": kernel_source_hash(kname)}
    with open(TRAFFIC, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
