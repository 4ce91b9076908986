"""Benchmark of the MoE-layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                [--capacity-factor CF --capacity-policy drop|reroute] [--gate-norm] [--noise-std SIGMA]
                [--expert-act gelu|silu|swiglu] [--router-hidden D_R]

One step = the whole layer (router, dispatch, W1 GEMM + GeLU, W2 GEMM,
combine) over one batch of seeded synthetic input already resident in HBM.
Prints one JSON line: tokens/s over the timed steps, the roofline of the
dominant kernel (the W1 grouped GEMM) measured with HIP events on the stream
it runs on, and the CPU oracle timed on a bounded sample of the same workload.
With a capacity factor the step is the capacity-limited layer (expert
capacity ceil(T k / E * CF), overflow dropped or rerouted).  The line also
carries the router alone and the router with its batch statistics, each timed
with HIP events.
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

DEFAULT_WORKLOAD = "decode-bf16-T8-d8192-E128"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0, help="0: automatic")
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
    return ap.parse_args()


KERNEL_SOURCES = {"f32": "gemm_f32.hip", "streaming": "gemm_stream.hip", "tiled": "gemm_tiled.hip"}


def kernel_source_hash(kernel):
    """Hash of the sources that define a W1 GEMM kernel: its own file, the
    shared headers and the launch parameters chosen in moe_api.hip."""
    csrc = os.path.join(ROOT, "sparse_mixture_experts_03_amd", "csrc")
    path = kernel.rsplit("_", 1)[-1]
    h = hashlib.sha256()
    for f in ("common.hpp", "launch.hpp", "moe_api.hip", KERNEL_SOURCES[path]):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel):
    """HBM traffic measured by rocprofv3 counters for this kernel and workload,
    if the committed measurement was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{kernel}|{workload}")
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
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
    cfg = moe_synth.workload(args.workload)
    act_code = {"gelu": moe.ACT_GELU, "silu": moe.ACT_SILU, "swiglu": moe.ACT_SWIGLU}[args.expert_act]
    cfg["ffn"] = act_code
    cfg["router_hidden"] = args.router_hidden
    T, d, d_ff, E, k = cfg["T"], cfg["d"], cfg["d_ff"], cfg["E"], cfg["k"]
    n1 = 2 * d_ff if act_code == moe.ACT_SWIGLU else d_ff  # W1 rows
    print(f"[bench] generating {args.workload} on {dev}", file=sys.stderr, flush=True)
    inp = moe_synth.generate(cfg, device=dev, seed=0)
    torch.cuda.synchronize()
    policy = moe.CAPACITY_REROUTE if args.capacity_policy == "reroute" else moe.CAPACITY_DROP
    c = moe.config(T, d, d_ff, E, k, cfg["act"], cfg["w"], tau=cfg["tau"], use_gumbel=cfg["gumbel"], seed=0,
                   capacity_factor=args.capacity_factor, capacity_policy=policy, gate_norm=int(args.gate_norm),
                   noise_std=args.noise_std, expert_act=act_code, router_hidden=args.router_hidden)
    layer = moe.MoELayerForward(c, device=dev)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    run = lambda: layer(inp["x"], inp["Wg"], inp["bias"], inp["W1"], inp["W2"], inp["S1"], inp["S2"],
                        W_in=inp["W_in"], b_in=inp["b_in"])

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = T * args.steps / wall

    counts = layer.counts.cpu().numpy()
    kept = int(counts.sum())
    active = int((counts > 0).sum())
    wbits = {moe.F32: 32, moe.BF16: 16, moe.INT4_G128: 4}[cfg["w"]]
    abytes = 4 if cfg["act"] == moe.F32 else 2
    w_bytes = d * d_ff * wbits // 8 + (d * d_ff // 128 * 2 if cfg["w"] == moe.INT4_G128 else 0)  # one W2
    w1_bytes = w_bytes * n1 // d_ff
    Tk = kept  # dispatched rows (T k without a capacity)
    hbytes = 4 if cfg["w"] == moe.F32 else 2

    # dominant kernel: the W1 grouped GEMM (+GeLU), timed alone with HIP events on its stream
    ws = layer.workspace
    stream = torch.cuda.current_stream()
    H = torch.empty((Tk, d_ff), dtype=torch.float32 if cfg["w"] == moe.F32 else torch.bfloat16, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_token = torch.empty(Tk, dtype=torch.int32, device=dev)
    pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    moe.moe_permute(c, layer.expert_ids, cnt, offsets, sorted_token, pos)
    gemm = lambda: moe.moe_grouped_gemm(c, 1, inp["x"], sorted_token, offsets, inp["W1"], inp["S1"], H)
    reps = max(10, args.steps)
    gemm_ms = time_on_stream(torch, stream, gemm, reps)

    # the router alone, and with its batch statistics (expert fractions, mean probabilities, entropy, balance terms)
    r_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    r_gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    r_ws = torch.empty(max(256, moe.moe_router_workspace_size(c)), dtype=torch.uint8, device=dev)
    s_ws = torch.empty(max(256, moe.moe_router_stats_workspace_size(c)), dtype=torch.uint8, device=dev)
    frac = torch.empty(E, dtype=torch.float64, device=dev)
    mprob = torch.empty(E, dtype=torch.float64, device=dev)
    scal = torch.empty(5, dtype=torch.float64, device=dev)
    router_ms = time_on_stream(torch, stream, lambda: moe.moe_router(c, inp["x"], inp["Wg"], inp["bias"], r_ids,
                                                                     r_gates, r_ws, W_in=inp["W_in"],
                                                                     b_in=inp["b_in"]), reps)
    stats_ms = time_on_stream(torch, stream, lambda: moe.moe_router_stats(c, inp["x"], inp["Wg"], inp["bias"], r_ids,
                                                                          r_gates, frac, mprob, scal, s_ws,
                                                                          W_in=inp["W_in"], b_in=inp["b_in"]), reps)
    if cfg["w"] == moe.F32:
        path = "f32"
    elif T <= 16 or (cfg["w"] == moe.INT4_G128 and (d % 1024 or d_ff % 1024)):
        path = "streaming"  # the automatic choice of the library
    else:
        path = "tiled"
    gemm_bytes = active * w1_bytes + Tk * d * abytes + Tk * d_ff * hbytes
    gemm_flops = 2.0 * Tk * d * n1
    kernel_name = f"moe_grouped_gemm_w1_{path}"
    # the binding roof: arithmetic intensity against the ridge point of the compute unit the path uses
    # (bf16 MFMA for bf16/INT4 experts, the fp32 vector ALUs for fp32 experts)
    compute_peak = FP32_PEAK_TFLOPS if cfg["w"] == moe.F32 else BF16_PEAK_TFLOPS
    ridge = compute_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if gemm_flops / gemm_bytes < ridge:
        achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=load_traffic(args.workload, kernel_name))
    else:
        achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
        roof = dict(bound="alu" if cfg["w"] == moe.F32 else "mfma", achieved=round(achieved, 1), peak=compute_peak,
                    unit="TFLOP/s", frac=round(achieved / compute_peak, 4),
                    traffic=load_traffic(args.workload, kernel_name))
    roof.update(kernel=kernel_name, avg_launch_ms=round(gemm_ms, 4),
                algorithmic_bytes=gemm_bytes, algorithmic_flops=gemm_flops)

    d_r = args.router_hidden
    router_w_bytes = (d_r * d * abytes + d_r * E * abytes) if d_r else d * E * abytes
    step_bytes = (T * d * abytes + router_w_bytes + active * (w1_bytes + w_bytes) + T * d * abytes + T * k * 8 + E * 4)
    out = {
        "metric": "MoE-layer tokens/s",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {moe.F32: "f32", moe.BF16: "bf16", moe.INT4_G128: "bf16 (int4 g128 experts)"}[cfg["w"]],
        "data": "synthetic (seeded N(0,1/fan_in) weights, N(0,1) tokens)",
        "config": {"workload": args.workload, "T": T, "d": d, "d_ff": d_ff, "E": E, "k": k,
                   "router_bias": bool(cfg["bias"]), "tau": cfg["tau"], "gumbel": bool(cfg["gumbel"]),
                   "capacity_factor": args.capacity_factor,
                   "capacity_policy": args.capacity_policy if args.capacity_factor > 0 else None,
                   "gate_norm": int(args.gate_norm), "noise_std": args.noise_std, "expert_act": args.expert_act,
                   "router_hidden": args.router_hidden},
        "layer_hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_mfma_frac": round((gemm_flops + 2.0 * Tk * d * d_ff) / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "active_experts": active,
        "counts_var": float(np.var(counts)),
        "assignments_kept": kept,
        "router_ms": round(router_ms, 4),
        "router_stats_ms": round(stats_ms, 4),
        "roofline": roof,
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, layer, args)
    print(json.dumps(out))


def time_on_stream(torch, stream, fn, reps):
    """Average milliseconds of fn() (which enqueues work on `stream`), from HIP events on that stream."""
    for _ in range(3):
        fn()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        fn()
    ev1.record(stream)
    ev1.synchronize()
    return ev0.elapsed_time(ev1) / reps


def cpu_baseline(cfg, inp, layer, args):
    """The oracle, single-threaded on one host core, on a bounded sample: the
    routing of every token plus the expert FFNs and combine of the sampled
    tokens; tokens/s = sampled tokens / (routing share + sampled FFN time)."""
    import numpy as np

    import moe_synth
    from oracle import oracle as oracle_mod
    orc = oracle_mod.get()
    T = cfg["T"]
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    xb, wgb = moe_synth.to_bits(inp["x"]), moe_synth.to_bits(inp["Wg"])
    # rough per-token cost to size the sample to ~10-20 s
    per_tok = 2.0 * cfg["k"] * cfg["d"] * cfg["d_ff"] * 1.5e-9
    n = args.cpu_sample_tokens or int(max(1, min(T, 15.0 // max(per_tok, 1e-9))))
    tokens = np.linspace(0, T - 1, n).round().astype(np.int64)
    tokens = np.unique(tokens)
    t0 = time.perf_counter()
    limited = args.capacity_factor > 0
    enc = None
    if inp["W_in"] is not None:
        enc = (moe_synth.to_bits(inp["W_in"]), inp["b_in"].cpu().numpy())
    ref = orc.route(xb, wgb, cfg["k"], cfg["act"], bias=bias, tau=float(np.float32(cfg["tau"])), encoder=enc,
                    use_gumbel=cfg["gumbel"], seed=0, want_zp=limited, gate_norm=int(args.gate_norm),
                    noise_std=float(np.float32(args.noise_std)))
    if limited:
        ref = orc.capacity_dispatch(ref, float(np.float32(args.capacity_factor)),
                                    1 if args.capacity_policy == "reroute" else 0)
    t_route = time.perf_counter() - t0
    used = sorted(e for e in set(ref["ids"][tokens].reshape(-1).tolist()) if e >= 0)
    E = cfg["E"]
    W1 = [None] * E
    W2 = [None] * E
    S1 = [None] * E if inp["S1"] is not None else None
    S2 = [None] * E if inp["S2"] is not None else None
    for e in used:
        W1[e] = moe_synth.to_bits(inp["W1"][e])
        W2[e] = moe_synth.to_bits(inp["W2"][e])
        if S1 is not None:
            S1[e] = moe_synth.to_bits(inp["S1"][e])
            S2[e] = moe_synth.to_bits(inp["S2"][e])
    t0 = time.perf_counter()
    reps = 0
    while True:  # repeat the sample until ~10 s of oracle work has been timed
        orc.forward_tokens(xb, ref["ids"], ref["gate_p"], W1, W2, cfg["act"], cfg["w"], cfg["d_ff"], tokens,
                           S1=S1, S2=S2, act=cfg.get("ffn", 0))
        reps += 1
        if time.perf_counter() - t0 >= 10.0:
            break
    t_ffn = (time.perf_counter() - t0) / reps
    secs = t_route * len(tokens) / T + t_ffn
    return {"value": round(len(tokens) / secs, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(tokens)} of {T} tokens (routing{' and capacity dispatch' if limited else ''} of all "
                      f"{T} tokens, prorated; expert FFNs and combine "
                      f"of the sample, repeated {reps}x), single-threaded fp64 C oracle; "
                      f"{t_route + t_ffn * reps:.1f} s measured"}


if __name__ == "__main__":
    main()
