"""Benchmark of the predictor-gated activation-sparse FFN step on one MI355X.

A step is one decode step through the whole stack: for every layer predict ->
compact -> sparse up -> sparse down, then one TAM update over all layers.  The
default workload is the OPT-6.7B-shaped ReLU stack (d=4096, f=16384, h=1024, fp16,
32 layers, batch 1) on seeded synthetic layers generated on the device.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C2] [--batch 1]

Prints one JSON line.  `value` = tokens/s per FFN layer = B * layers / step time,
with every input resident in HBM when the timed region starts; the timed region
is one replay of a HIP graph holding exactly K steps.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_HBM_GBPS = 8000.0
METRIC = "sparse-FFN tokens/s per layer + effective HBM GB/s (% of peak) at batch 1"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--config", default="C2")
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--layers", type=int, default=0, help="0 = the workload's layer count")
    p.add_argument("--roofline-steps", type=int, default=8)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-layers", type=int, default=4)
    p.add_argument("--cpu-steps", type=int, default=64)
    p.add_argument("--tam-lambda", type=float, default=0.9)
    p.add_argument("--tam-eps", type=float, default=0.01)
    p.add_argument("--separate", action="store_true", help="time the five separate calls per layer")
    p.add_argument("--fused", action="store_true",
                   help="time sfx_ffn_step where it supports the shape, also from 3 tokens on (by default the "
                        "separate calls are timed there: on the matrix cores they measured faster)")
    p.add_argument("--pipeline", action="store_true",
                   help="time the Live Pipeline step (sfx_ffn_pipeline): each layer's predictor scores the previous "
                        "layer's input (layer 0: the previous token's), inputs of adjacent layers at cosine 0.98")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (5 times): the calibration of HBM byte counters")
    return p.parse_args()


def e_bytes(dt):
    return {"f32": 4, "f16": 2, "bf16": 2}[dt]


def row_bytes(cfg):
    if cfg.wdtype == "q4":
        return cfg.d // 2 + 2 * (cfg.d // 32)
    return cfg.d * e_bytes(cfg.wdtype)


def kernel_bytes(cfg, B, k):
    """Algorithmic bytes of one layer-step, per call (what the method must move)."""
    d, f, h = cfg.d, cfg.f, cfg.h
    ep = e_bytes(cfg.pdtype)
    na = 2 if cfg.act == "reglu" else 1
    er = row_bytes(cfg)
    return {
        "predict": (h * d + f * h) * ep + B * d * ep + B * f * 4,
        "compact": B * f * 4 + (1 + B) * f / 8 + k * 4,
        "up": B * d * ep + k * 4 + na * k * er + k * 4 + B * k * 4,
        "down": k * 4 + B * k * 4 + k * er + B * d * 4,
    }


STEP_SOURCES = ["k_step.hpp", "k_step_host.cpp", "sfx_step.hpp", "sfx_common.hpp", "k_step_f16.hip", "k_step_bf16.hip"]
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "k_step_traffic_opt6.7b_fp16_b1.txt")


def measured_traffic(cfg, B, L):
    """HBM bytes per fused-step launch from the committed rocprofv3 counter summary,
    or None when that summary is for another workload or for other kernel sources."""
    import hashlib
    if not (cfg.name == "C2" and B == 1 and L == cfg.layers) or not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "activation_sparse_ffn_amd", "csrc")
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    if vals.get("source_sha256") != h.hexdigest():
        return None
    return int(vals["traffic_bytes_per_launch"])


def cpu_baseline(cfg, layers_np, xs_np, B, steps):
    """The fp64 oracle, unchanged, on a bounded sample of the same workload."""
    from oracle import sfx_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    n = 0
    t0 = time.perf_counter()
    for li, Lnp in enumerate(layers_np):
        for s in range(steps):
            O.ffn_step(xs_np[li][s], Lnp, cfg.wdtype, cfg.pdtype, cfg.act, Lnp["threshold"])
            n += 1
    dt = time.perf_counter() - t0
    return {"value": B * n / dt, "unit": "tokens/s/layer", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(layers_np)} layers x {steps} decode steps of the benchmark workload "
                      f"(batch {B}), fp64 numpy oracle, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the sharded path is "
              "described, not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}), flush=True)
        return
    import synthetic as S
    from activation_sparse_ffn_amd import StackStep, StepBuffers, TamState, run_layer
    from activation_sparse_ffn_amd import _abi as A

    A.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = S.CONFIGS[args.config]
    B = args.batch
    L = args.layers or cfg.layers
    K, W = args.steps, args.warmup
    G = (cfg.f + 31) // 32
    tam_k = max(1, G // 4) if cfg.tam is None else cfg.tam["K"]

    print(f"[bench] generating {L} layers of {cfg.workload}", file=sys.stderr, flush=True)
    layers = [S.make_layer(cfg, l, device=dev) for l in range(L)]
    if args.pipeline:
        xs = S.make_layer_chain(cfg, L, W + K, B, device=dev)
    else:
        xs = [S.make_tokens(cfg, l, W + K, B, device=dev) for l in range(L)]

    def pred_inputs(s):
        return [xs[0][max(s - 1, 0)]] + [xs[l - 1][s] for l in range(1, L)]
    ubits = torch.zeros(L, G, dtype=torch.int32, device=dev)
    tam = TamState(L, G, tam_k, device=dev)
    tensors = [ly.tensors() for ly in layers]
    # the fused step where it is the faster path (1-2 tokens); from 3 tokens on the
    # separate calls run on the matrix cores and measured faster (--fused forces it)
    fused = (not args.separate) and (args.fused or args.pipeline or B <= 2) and \
        StackStep.supported(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, pipeline=args.pipeline)
    if args.pipeline and not fused:
        print("bench.py: the Live Pipeline kernel does not take this shape", file=sys.stderr)
        sys.exit(2)

    if fused:
        st = StackStep(layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, device=dev, union_bits=ubits,
                       pipeline=args.pipeline)
        descs = [st.descriptors([xs[l][s] for l in range(L)], pred_inputs(s) if args.pipeline else None,
                                tok_bits=False) for s in range(W + K)]

        def step(s):
            st.run(descs[s])
            tam.update(ubits, args.tam_lambda, args.tam_eps)

        def counts_of(s):
            st.run(descs[s])
            return st.counts().cpu().numpy()
    else:
        buf = StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pdtype, device=dev)

        def step(s):
            for l in range(L):
                buf.union_bits = ubits[l]
                run_layer(buf, tensors[l], xs[l][s], layers[l].threshold, cfg.act, tok_bits=False)
            tam.update(ubits, args.tam_lambda, args.tam_eps)

        def counts_of(s):
            cs = []
            for l in range(L):
                buf.union_bits = ubits[l]
                run_layer(buf, tensors[l], xs[l][s], layers[l].threshold, cfg.act, tok_bits=False)
                cs.append(buf.count.clone())
            return torch.cat(cs).cpu().numpy()

    # eager pass (loads code objects), then capture the warmup and timed steps
    step(0)
    torch.cuda.synchronize()
    print(f"[bench] {'fused' if fused else 'separate-call'} path; capturing graphs", file=sys.stderr, flush=True)
    g_warm, g_timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm):
        for s in range(W):
            step(s)
    with torch.cuda.graph(g_timed):
        for s in range(W, W + K):
            step(s)
    torch.cuda.synchronize()

    g_warm.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    g_timed.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / K
    print(f"[bench] timed {K} steps: {ms_total:.3f} ms", file=sys.stderr, flush=True)
    # sticky status words of every workspace the timed steps used: a timed-out wait
    # or an out-of-range hidden value would make the step's outputs undefined
    if fused:
        st.check_status()
    else:
        buf.check_status()

    # Active counts of the timed steps (deterministic: an eager re-run of the same steps).
    counts = np.zeros((K, L), dtype=np.int64)
    for i, s in enumerate(range(W, W + K)):
        counts[i] = counts_of(s)
    kb = [kernel_bytes(cfg, B, int(k)) for k in counts.reshape(-1)]
    tam_bytes = L * G * 16
    step_bytes = sum(sum(v.values()) for v in kb) / K + tam_bytes
    gbps = step_bytes / (ms_step * 1e-3) / 1e9

    # Dominant kernel: per-launch durations from HIP events bracketing each launch on
    # the launch stream; every launch is queued behind a spin kernel so the events
    # time the GPU, not the host.  Fused path: the whole-stack kernel (all layers'
    # bytes per launch).  Separate path: sfx_predict (the largest byte share).
    R = min(args.roofline_steps, K)
    torch.cuda.synchronize()
    if fused:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R)]
        torch.cuda._sleep(int(2e8))
        for i, s in enumerate(range(W, W + R)):
            evs[i][0].record()
            st.run(descs[s])
            evs[i][1].record()
        torch.cuda.synchronize()
        dur_ms = np.array([a.elapsed_time(b) for a, b in evs])
        per_launch = [sum(sum(kernel_bytes(cfg, B, int(k)).values()) for k in counts[i]) for i in range(R)]
        dom_bytes = float(np.mean(per_launch))
        dom_name = ("sfx_ffn_pipeline (k_pipe" if args.pipeline else "sfx_ffn_step (k_step") + \
            ", all layers of one decode step)"
    else:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R * L)]
        torch.cuda._sleep(int(2e8))
        i = 0
        for s in range(W, W + R):
            for l in range(L):
                t = tensors[l]
                evs[i][0].record()
                A.sfx_predict(xs[l][s], t["W1"], t["W2"], buf.scores, buf.ws_pred)
                evs[i][1].record()
                i += 1
        torch.cuda.synchronize()
        dur_ms = np.array([a.elapsed_time(b) for a, b in evs])
        dom_bytes = float(kernel_bytes(cfg, B, 0)["predict"])
        dom_name = "sfx_predict (k_pred_hidden + k_pred_scores)"
    dom_gbps = dom_bytes / (dur_ms.mean() * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(B * L / (ms_step * 1e-3), 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.wdtype,
        "data": "synthetic (seeded, generated on device)",
        "config": {"workload": cfg.workload, "batch": B, "layers": L, "d": cfg.d, "f": cfg.f, "h": cfg.h,
                   "act": cfg.act, "density": cfg.density, "tam": {"lambda": args.tam_lambda,
                                                                  "eps": args.tam_eps, "K": tam_k, "G": G}},
        "us_per_layer_step": round(ms_step * 1e3 / L, 3),
        "effective_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "mean_active": round(float(counts.mean()), 1),
        "bytes_per_layer_step": round(step_bytes / L, 0),
        "path": ("pipeline" if args.pipeline else "fused") if fused else "separate",
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(dom_gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(dom_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(cfg, B, L) if fused and not args.pipeline else None,
                     "avg_launch_us": round(float(dur_ms.mean()) * 1e3, 3),
                     "bytes_per_launch": round(dom_bytes), "launches": int(dur_ms.size)},
    }

    if not args.no_cpu_baseline:
        import synthetic.gen as SG
        nl = min(args.cpu_layers, L)
        ns = min(args.cpu_steps, K)
        lnp, xnp = [], []
        for l in range(nl):
            d = {k: SG.storage_numpy(v) for k, v in tensors[l].items()}
            d["threshold"] = layers[l].threshold
            lnp.append(d)
            xnp.append([SG.storage_numpy(xs[l][s]) for s in range(W, W + ns)])
        result["cpu_baseline"] = cpu_baseline(cfg, lnp, xnp, B, ns)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
