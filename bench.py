"""Benchmark of the predictor-gated activation-sparse FFN step on one MI355X.

A step is one decode step through the whole stack: for every layer predict ->
compact -> sparse up -> sparse down, then one TAM update over all layers.  The
default workload is the OPT-6.7B-shaped ReLU stack (d=4096, f=16384, h=1024, fp16,
32 layers, batch 1) on seeded synthetic layers generated on the device.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C2] [--batch 1]

Prints one JSON line.  `value` = tokens/s per FFN layer = B * layers / step time,
with every input resident in HBM when the timed region starts; the timed region
is one replay of a HIP graph holding exactly K steps.  By default the line also
carries: the LLaMA2-7B ReGLU stack at batch 1 (the 7B-shaped gate workload), the
Live Pipeline step on both stacks with its mask recall, the streaming-read ceiling,
and the fp64 oracle's CPU time (1 thread and all threads) on a sample of the
timed steps together with the parity maxima of that sample.
"""
import argparse
import json
import os
import subprocess
import sys
import tempfile
import time

import numpy as np

PEAK_HBM_GBPS = 8000.0
METRIC = "sparse-FFN tokens/s per layer + effective HBM GB/s (% of peak) at batch 1"
ROOT = os.path.dirname(os.path.abspath(__file__))


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
    p.add_argument("--no-extra", action="store_true",
                   help="only the selected workload (no second stack, Live Pipeline or streaming probe)")
    p.add_argument("--cpu-layers", type=int, default=4)
    p.add_argument("--cpu-steps", type=int, default=24)
    p.add_argument("--tam-lambda", type=float, default=0.9)
    p.add_argument("--tam-eps", type=float, default=0.01)
    p.add_argument("--separate", action="store_true", help="time the five separate calls per layer")
    p.add_argument("--fused", action="store_true",
                   help="time sfx_ffn_step where it supports the shape (the default already does; kept for "
                        "scripts that name the path)")
    p.add_argument("--pipeline", action="store_true",
                   help="time the Live Pipeline step (sfx_ffn_pipeline) as the headline: each layer's predictor "
                        "scores the previous layer's input (layer 0: the previous token's), inputs of adjacent "
                        "layers at cosine 0.98")
    p.add_argument("--pred-q4", action="store_true",
                   help="store the predictor (W1, W2) in int4 g32 with fp16 scales (separate calls)")
    p.add_argument("--stream-probe", type=int, default=0, metavar="MIB",
                   help="only run the streaming-read probe over MIB MiB (5 reads) and print its bandwidth")
    p.add_argument("--no-calib", action="store_true",
                   help="use the generator's hot-first layers and closed-form thresholds instead of "
                        "raw-order layers calibrated on the device")
    p.add_argument("--dense-switch", action="store_true",
                   help="only the sparse/dense study (Falcon-40B-shaped layers, batch 8..64)")
    p.add_argument("--churn", action="store_true",
                   help="only the hot-region churn study (Falcon-40B-shaped layers, TAM vs Top-K)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (5 times): the calibration of HBM byte counters")
    return p.parse_args()


def say(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def e_bytes(dt):
    return {"f32": 4, "f16": 2, "bf16": 2}[dt]


def row_bytes(cfg):
    if cfg.wdtype == "q4":
        return cfg.d // 2 + 2 * (cfg.d // 32)
    return cfg.d * e_bytes(cfg.wdtype)


def pred_weight_bytes(cfg):
    """Bytes per predictor weight: the storage type's, or 1/2 + 2/32 for int4 g32
    (codes and fp16 scales)."""
    return 0.5 + 2.0 / 32 if cfg.pred_q4 else e_bytes(cfg.pdtype)


def kernel_bytes(cfg, B, k):
    """Algorithmic bytes of one layer-step, per call (what the method must move)."""
    d, f, h = cfg.d, cfg.f, cfg.h
    ep = e_bytes(cfg.pdtype)
    epw = pred_weight_bytes(cfg)
    na = 2 if cfg.act == "reglu" else 1
    er = row_bytes(cfg)
    return {
        "predict": (h * d + f * h) * epw + B * d * ep + B * f * 4,
        "compact": B * f * 4 + (1 + B) * f / 8 + k * 4,
        "up": B * d * ep + k * 4 + na * k * er + k * 4 + B * k * 4,
        "down": k * 4 + B * k * 4 + k * er + B * d * 4,
    }


STEP_SOURCES = ["k_step.hpp", "k_step_host.cpp", "sfx_step.hpp", "sfx_common.hpp", "k_step_f16.hip", "k_step_bf16.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_step_traffic_opt6.7b_fp16_b1.txt")


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
    csrc = os.path.join(ROOT, "activation_sparse_ffn_amd", "csrc")
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    if vals.get("source_sha256") != h.hexdigest():
        return None
    return int(vals["traffic_bytes_per_launch"])


def popcount32(t):
    """Set bits per element of an int32 tensor (torch has no popcount)."""
    import torch
    u = t.to(torch.int64) & 0xFFFFFFFF
    sh = torch.arange(32, device=t.device, dtype=torch.int64)
    return ((u.unsqueeze(-1) >> sh) & 1).sum(-1)


N_CAL = 1024


def calibrated_layer(cfg, layer, dev, n_cal=N_CAL, keep_counts=False):
    """The offline calibration pass on a raw-order layer: thresholds at the
    configured density, activation counts and the hot-first table, from n_cal
    calibration tokens (a token stream disjoint from the measured one), then every
    per-neuron row reordered.  Returns (calibrated layer, calibration summary)."""
    import dataclasses
    import synthetic as S
    from activation_sparse_ffn_amd.calib import apply_order, calibrate_layer
    toks = S.make_tokens(cfg, layer.index, n_cal, 1, device=dev, tag="calib")[:, 0]
    r = calibrate_layer(layer.tensors(), toks, cfg.density, group=layer.group)
    t = dict(layer.tensors())
    if layer.group is not None:
        t["group"] = layer.group
    c = apply_order(t, r["perm"])
    perm = r["perm"].cpu().numpy()
    keys = ("W2", "W2_s", "Wa", "Wa_s", "Wl", "Wl_s", "Wd", "Wd_s", "ba", "perm", "group")
    new = dataclasses.replace(layer, threshold=r["threshold"], p=layer.p[perm], **{k: c.get(k) for k in keys})
    out = {"threshold": r["threshold"], "active_share": r["active_share"]}
    if keep_counts:
        out["counts"] = r["counts"]
    return new, out


def make_stack(cfg, L, dev, calibrate=True):
    """L layers of the configuration: raw-order layers calibrated on the device, or
    (calibrate=False) the generator's own hot-first layers with closed-form thresholds."""
    import synthetic as S
    if not calibrate:
        return [S.make_layer(cfg, l, device=dev) for l in range(L)], None
    layers, cal = [], []
    for l in range(L):
        ly, c = calibrated_layer(cfg, S.make_layer(cfg, l, device=dev, order="raw"), dev)
        layers.append(ly)
        cal.append(c)
    th = np.array([c["threshold"] for c in cal])
    sh = np.array([c["active_share"] for c in cal])
    return layers, {"tokens_per_layer": N_CAL, "threshold_mean": round(float(th.mean()), 5),
                    "threshold_min": round(float(th.min()), 5), "threshold_max": round(float(th.max()), 5),
                    "calibration_active_share": round(float(sh.mean()), 5)}


class Workload:
    """One stack of synthetic layers and the step that is timed on it."""

    def __init__(self, args, cfg, B, L, mode, dev):
        import torch
        import synthetic as S
        from activation_sparse_ffn_amd import StackStep, StepBuffers, TamState, run_layer
        self.cfg, self.B, self.L, self.mode = cfg, B, L, mode
        W, K = args.warmup, args.steps
        self.W, self.K = W, K
        G = (cfg.f + 31) // 32
        self.G = G
        self.tam_k = max(1, G // 4) if cfg.tam is None else cfg.tam["K"]
        self.tam_args = (args.tam_lambda, args.tam_eps)
        say(f"generating {L} layers of {cfg.workload} ({mode}, batch {B})")
        self.layers, self.calibration = make_stack(cfg, L, dev, calibrate=not args.no_calib)
        if mode == "pipeline":
            self.xs = S.make_layer_chain(cfg, L, W + K, B, device=dev)
        else:
            self.xs = [S.make_tokens(cfg, l, W + K, B, device=dev) for l in range(L)]
        self.ubits = torch.zeros(L, G, dtype=torch.int32, device=dev)
        self.tam = TamState(L, G, self.tam_k, device=dev)
        self.tensors = [ly.tensors() for ly in self.layers]
        if mode in ("fused", "pipeline"):
            self.st = StackStep(self.layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, device=dev,
                                union_bits=self.ubits, pipeline=(mode == "pipeline"))
            self.descs = [self.st.descriptors([self.xs[l][s] for l in range(L)],
                                              self.pred_inputs(s) if mode == "pipeline" else None,
                                              tok_bits=False) for s in range(W + K)]
        else:
            self.buf = StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pred_storage, device=dev)
            self.run_layer = run_layer

    def pred_inputs(self, s):
        """Live Pipeline predictor inputs of step s: layer l > 0 scores the input of
        layer l - 1, layer 0 the layer-0 input of the previous step."""
        return [self.xs[0][max(s - 1, 0)]] + [self.xs[l - 1][s] for l in range(1, self.L)]

    def launch(self, s):
        """Everything but the TAM update for step s (the dominant kernel's launch on
        the fused paths)."""
        if self.mode in ("fused", "pipeline"):
            self.st.run(self.descs[s])
        else:
            for l in range(self.L):
                self.buf.union_bits = self.ubits[l]
                self.run_layer(self.buf, self.tensors[l], self.xs[l][s], self.layers[l].threshold, self.cfg.act,
                               tok_bits=False)

    def step(self, s):
        self.launch(s)
        self.tam.update(self.ubits, *self.tam_args)

    def counts_of(self, s):
        import torch
        if self.mode in ("fused", "pipeline"):
            self.st.run(self.descs[s])
            return self.st.counts().cpu().numpy()
        cs = []
        for l in range(self.L):
            self.buf.union_bits = self.ubits[l]
            self.run_layer(self.buf, self.tensors[l], self.xs[l][s], self.layers[l].threshold, self.cfg.act,
                           tok_bits=False)
            cs.append(self.buf.count.clone())
        return torch.cat(cs).cpu().numpy()

    def check_status(self):
        if self.mode in ("fused", "pipeline"):
            self.st.check_status()
        else:
            self.buf.check_status()


def time_workload(wl, roofline_steps):
    """Graph-captured timing of K steps, algorithmic bytes from the measured counts,
    and per-launch HIP-event durations of the dominant kernel."""
    import torch
    from activation_sparse_ffn_amd import _abi as A
    cfg, B, L, W, K = wl.cfg, wl.B, wl.L, wl.W, wl.K
    wl.step(0)
    torch.cuda.synchronize()
    say(f"{wl.mode} path; capturing graphs")
    g_warm, g_timed = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm):
        for s in range(W):
            wl.step(s)
    with torch.cuda.graph(g_timed):
        for s in range(W, W + K):
            wl.step(s)
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
    say(f"timed {K} steps: {ms_total:.3f} ms")
    wl.check_status()                 # sticky status words of every workspace the timed steps used

    counts = np.zeros((K, L), dtype=np.int64)
    for i, s in enumerate(range(W, W + K)):
        counts[i] = wl.counts_of(s)
    kb = [kernel_bytes(cfg, B, int(k)) for k in counts.reshape(-1)]
    tam_bytes = L * wl.G * 16
    step_bytes = sum(sum(v.values()) for v in kb) / K + tam_bytes
    gbps = step_bytes / (ms_step * 1e-3) / 1e9

    # Dominant kernel: per-launch durations from HIP events bracketing each launch on
    # the launch stream; every launch is queued behind a spin kernel so the events
    # time the GPU, not the host.  Fused paths: the whole-stack kernel (all layers'
    # bytes per launch).  Separate path: sfx_predict (the largest byte share).
    R = min(roofline_steps, K)
    torch.cuda.synchronize()
    if wl.mode in ("fused", "pipeline"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R)]
        torch.cuda._sleep(int(2e8))
        for i, s in enumerate(range(W, W + R)):
            evs[i][0].record()
            wl.st.run(wl.descs[s])
            evs[i][1].record()
        torch.cuda.synchronize()
        dur_ms = np.array([a.elapsed_time(b) for a, b in evs])
        per_launch = [sum(sum(kernel_bytes(cfg, B, int(k)).values()) for k in counts[i]) for i in range(R)]
        dom_bytes = float(np.mean(per_launch))
        dom_name = ("sfx_ffn_pipeline (k_pipe" if wl.mode == "pipeline" else "sfx_ffn_step (k_step") + \
            ", all layers of one decode step)"
    else:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R * L)]
        torch.cuda._sleep(int(2e8))
        i = 0
        for s in range(W, W + R):
            for l in range(L):
                t = wl.tensors[l]
                evs[i][0].record()
                if t.get("W1_s") is not None:
                    A.sfx_predict_q4(wl.xs[l][s], t["W1"], t["W1_s"], t["W2"], t["W2_s"], wl.buf.scores,
                                     wl.buf.ws_pred)
                else:
                    A.sfx_predict(wl.xs[l][s], t["W1"], t["W2"], wl.buf.scores, wl.buf.ws_pred)
                evs[i][1].record()
                i += 1
        torch.cuda.synchronize()
        dur_ms = np.array([a.elapsed_time(b) for a, b in evs])
        dom_bytes = float(kernel_bytes(cfg, B, 0)["predict"])
        dom_name = ("sfx_predict_q4 (k_pred_hidden_q4 + k_pred_scores_q4)" if cfg.pred_q4 else
                    "sfx_predict (k_pred_hidden + k_pred_scores)")
    dom_gbps = dom_bytes / (dur_ms.mean() * 1e-3) / 1e9
    return {
        "ms_step": ms_step, "counts": counts, "step_bytes": step_bytes, "gbps": gbps,
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(dom_gbps, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(cfg, B, L) if wl.mode == "fused" else None,
                     "avg_launch_us": round(float(dur_ms.mean()) * 1e3, 3), "bytes_per_launch": round(dom_bytes),
                     "launches": int(dur_ms.size)},
    }


def summary(wl, r):
    return {"workload": wl.cfg.workload, "batch": wl.B, "layers": wl.L, "path": wl.mode,
            "calibrated": wl.calibration is not None,
            "us_per_layer_step": round(r["ms_step"] * 1e3 / wl.L, 3),
            "tokens_per_s_per_layer": round(wl.B * wl.L / (r["ms_step"] * 1e-3), 1),
            "effective_GBps": round(r["gbps"], 1), "hbm_frac": round(r["gbps"] / PEAK_HBM_GBPS, 4),
            "mean_active": round(float(r["counts"].mean()), 1), "roofline_frac": r["roofline"]["frac"]}


def mask_recall(wl_pipe, dev, steps):
    """Recall and precision of the Live Pipeline's union masks (predictor on the
    previous layer's input) against the masks of the exact step (predictor on the
    layer's own input), over every layer of `steps` timed steps."""
    import torch
    from activation_sparse_ffn_amd import StackStep
    cfg, L, B = wl_pipe.cfg, wl_pipe.L, wl_pipe.B
    ex_bits = torch.zeros(L, wl_pipe.G, dtype=torch.int32, device=dev)
    ex = StackStep(wl_pipe.layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, device=dev, union_bits=ex_bits)
    hit = exact = pred = 0
    for s in steps:
        wl_pipe.st.run(wl_pipe.descs[s])
        ex.run(ex.descriptors([wl_pipe.xs[l][s] for l in range(L)], tok_bits=False))
        torch.cuda.synchronize()
        hit += int(popcount32(wl_pipe.ubits & ex_bits).sum())
        exact += int(popcount32(ex_bits).sum())
        pred += int(popcount32(wl_pipe.ubits).sum())
    ex.check_status()
    return {"recall": round(hit / max(exact, 1), 4), "precision": round(hit / max(pred, 1), 4),
            "predicted_active": pred, "exact_active": exact, "layer_steps": L * len(steps)}


def stream_probe(dev, mib=2048, reps=5):
    """Bandwidth of the streaming-read helper (sfx_stream_read) over `mib` MiB,
    rotating over two buffers so reads come from HBM, not the 256 MB cache."""
    import torch
    from activation_sparse_ffn_amd import _abi as A
    n = mib << 20
    bufs = [torch.ones(n // 2, dtype=torch.float16, device=dev) for _ in range(2)]
    out = torch.zeros(A.STREAM_READ_OUT_WORDS, dtype=torch.int32, device=dev)
    A.sfx_stream_read(bufs[0], out)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(reps):
        A.sfx_stream_read(bufs[i % 2], out)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / reps
    return {"kernel": "sfx_stream_read (k_stream_read)", "bytes": n, "us": round(us, 2),
            "GBps": round(n / (us * 1e-6) / 1e9, 1)}


def hot_region_churn(dev, L=4, B=1, steps=512):
    """Churn of the hot region on the Falcon-40B-shaped layers (1024 groups of 32,
    K = 256 hot slots, 512 AR(1) decode steps): the layers' own union masks feed
    TAM at each lambda and the Top-K rule on the current step alone; each rule
    keeps its own hot region of W_up, bias and W_down group rows (sfx_hot_update).
    Reports groups and bytes copied per layer-step, the copy kernel's time and
    bandwidth, and how many of a step's active neurons fall in groups the rule
    made hot at the step before."""
    import torch
    import synthetic as S
    from activation_sparse_ffn_amd import HotRegion, StepBuffers, TamState, TopKNowState, run_layer
    cfg = S.CONFIGS["C5"]
    G, K, eps = cfg.groups, cfg.tam["K"], cfg.tam["eps"]
    say(f"hot-region churn: generating {L} layers of {cfg.workload}")
    layers, _ = make_stack(cfg, L, dev)
    xs = [S.make_tokens(cfg, l, steps, B, device=dev) for l in range(L)]
    ubits = torch.zeros(L, G, dtype=torch.int32, device=dev)
    bufs = [StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pred_storage, device=dev, union_bits=ubits[l])
            for l in range(L)]
    mats = [[ly.Wa, ly.ba, ly.Wd] for ly in layers]
    rules = [("tam", lam) for lam in cfg.tam["lambdas"]] + [("topk_now", None)]
    states, regions = [], []
    for kind, lam in rules:
        states.append(TamState(L, G, K, device=dev) if kind == "tam" else TopKNowState(L, G, K, device=dev))
        regions.append(HotRegion(mats, G, K, device=dev))
    group_bytes = sum(regions[0].group_bytes)
    n_rules = len(rules)
    copied = torch.zeros(n_rules, dtype=torch.int64, device=dev)
    covered = torch.zeros(n_rules, dtype=torch.int64, device=dev)
    active = torch.zeros((), dtype=torch.int64, device=dev)
    shifts = torch.arange(32, device=dev, dtype=torch.int64)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
           for _ in range(n_rules)]
    for s in range(steps):
        for l in range(L):
            run_layer(bufs[l], layers[l].tensors(), xs[l][s], layers[l].threshold, cfg.act, tok_bits=False)
        cnt = popcount32(ubits)                                        # [L][G] active neurons per group
        if s > 0:
            active += cnt.sum()
        for r, (kind, lam) in enumerate(rules):
            st, hr = states[r], regions[r]
            if s > 0:                                                  # hot set chosen at the step before
                hot = ((st.hot.to(torch.int64).unsqueeze(-1) >> shifts) & 1).reshape(L, -1)[:, :G]
                covered[r] += (cnt * hot).sum()
            if kind == "tam":
                st.update(ubits, lam, eps)
            else:
                st.update(ubits)
            evs[r][s][0].record()
            hr.update(st.entered, st.left)
            evs[r][s][1].record()
            copied[r] += hr.ncopies.sum()
        if s % 128 == 0:
            say(f"hot-region churn: step {s}")
    torch.cuda.synchronize()
    for b in bufs:
        b.check_status()
    out = {"workload": cfg.workload, "layers": L, "batch": B, "steps": steps, "groups": G, "K": K,
           "group_bytes": group_bytes, "rules": {}}
    tot_active = int(active.item())
    for r, (kind, lam) in enumerate(rules):
        n = int(copied[r].item())
        us = np.array([a.elapsed_time(b) for a, b in evs[r]]) * 1e3
        name = f"tam_lambda_{lam}" if kind == "tam" else "topk_current_step"
        out["rules"][name] = {
            "groups_copied_per_layer_step": round(n / (L * steps), 3),
            "MB_copied_per_layer_step": round(n * group_bytes / (L * steps) / 1e6, 3),
            "next_step_coverage": round(int(covered[r].item()) / max(tot_active, 1), 4),
            "copy_us_per_step": round(float(us.mean()), 2),
            "copy_GBps": round(2 * n * group_bytes / max(float(us.sum()) * 1e-6, 1e-12) / 1e9, 1),
        }
    base = out["rules"]["topk_current_step"]["groups_copied_per_layer_step"]
    for name, v in out["rules"].items():
        if name.startswith("tam"):
            v["topk_copies_over_tam"] = round(base / v["groups_copied_per_layer_step"], 3) \
                if v["groups_copied_per_layer_step"] > 0 else None
    return out


def dense_bytes(cfg, B):
    """Algorithmic bytes of one dense layer-step: every row of W_up (and W_gate),
    the biases and every row of W_down, the tokens, activations and y."""
    d, f = cfg.d, cfg.f
    na = 2 if cfg.act == "reglu" else 1
    er = row_bytes(cfg)
    return B * d * e_bytes(cfg.pdtype) + na * f * er + f * 4 + 2 * B * f * 4 + f * er + B * d * 4


def dense_switch_study(dev, L=4, steps=8, batches=(8, 16, 32, 48, 64)):
    """Sparse step against the dense FFN (sfx_dense_ffn) on calibrated
    Falcon-40B-shaped layers at several batch sizes: time per layer-step of each,
    graph-captured; the bandwidth each path reaches; and the switch's choice from
    the calibration frequencies (expected union) with those bandwidths, against
    the measured faster path."""
    import torch
    import synthetic as S
    from activation_sparse_ffn_amd import StepBuffers, run_layer
    from activation_sparse_ffn_amd import _abi as A
    from activation_sparse_ffn_amd.switch import SparseDenseSwitch, expected_union
    cfg = S.CONFIGS["C5"]
    say(f"dense switch: generating {L} layers of {cfg.workload}")
    layers, cal = [], []
    for l in range(L):
        ly, c = calibrated_layer(cfg, S.make_layer(cfg, l, device=dev, order="raw"), dev, keep_counts=True)
        layers.append(ly)
        cal.append((c["counts"].double() / N_CAL).cpu().numpy())
    # each layer has its own neurons: the expected union is averaged over layers
    tens = [ly.tensors() for ly in layers]
    rows = []

    def timed(fn, n_layers):
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s_ in range(steps):
                fn(s_)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (steps * n_layers)

    for B in batches:
        xs = [S.make_tokens(cfg, l, steps, B, device=dev) for l in range(L)]
        buf = StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pred_storage, device=dev)

        def sparse(s_):
            for l in range(L):
                run_layer(buf, tens[l], xs[l][s_], layers[l].threshold, cfg.act, tok_bits=False)

        hact = torch.empty(cfg.f, B, dtype=torch.float32, device=dev)
        y = torch.empty(B, cfg.d, dtype=torch.float32, device=dev)
        ws = A.workspace(A.sfx_dense_ffn_ws(A.SFX_F16, B, cfg.d, cfg.f), dev)

        def dense(s_):
            for l in range(L):
                t = tens[l]
                A.sfx_dense_ffn(xs[l][s_], t["Wa"], t["ba"], t["Wd"], hact, y, ws, act=cfg.act)

        us_s = timed(sparse, L)
        ks = []
        for s_ in range(steps):
            for l in range(L):
                run_layer(buf, tens[l], xs[l][s_], layers[l].threshold, cfg.act, tok_bits=False)
                ks.append(buf.count.clone())
        k = float(torch.cat(ks).double().mean().item())
        buf.check_status()
        us_d = timed(dense, L)
        kb = kernel_bytes(cfg, B, k)
        eu = float(np.mean([expected_union(pl, B) for pl in cal]))
        rows.append({"batch": B, "mean_union": round(k, 1), "expected_union": round(eu, 1),
                     "sparse_us": round(us_s, 2), "dense_us": round(us_d, 2),
                     "sparse_GBps": round(sum(kb.values()) / (us_s * 1e-6) / 1e9, 1),
                     "dense_GBps": round(dense_bytes(cfg, B) / (us_d * 1e-6) / 1e9, 1),
                     "faster": "dense" if us_d < us_s else "sparse"})
        say(f"dense switch B={B}: sparse {us_s:.1f} us, dense {us_d:.1f} us, union {k:.0f}")
        del buf, hact, y, ws, xs
        torch.cuda.empty_cache()
    # the switch at each batch: the byte model with the bandwidths measured at that
    # batch (both paths slow down as the products grow), on the expected union
    for r in rows:
        sw = SparseDenseSwitch(pred_bytes=(cfg.h * cfg.d + cfg.f * cfg.h) * pred_weight_bytes(cfg),
                               row_bytes=2 * row_bytes(cfg) + 4, f=cfg.f,
                               sparse_gbps=r["sparse_GBps"], dense_gbps=r["dense_GBps"])
        r["switch_choice"] = "dense" if sw.use_dense(r["expected_union"]) else "sparse"
        r["crossover_density"] = round(sw.crossover_k() / cfg.f, 4)
    return {"workload": cfg.workload + ", calibrated", "layers": L, "steps": steps, "by_batch": rows}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_and_parity(wl, nl, ns):
    """The fp64 oracle, unchanged, on a bounded sample of the timed workload (nl
    layers x ns timed steps), in a child process with 1 thread and with every host
    core, thread counts set in its environment before numpy is imported.  The same
    run recomputes the sample's parity maxima against the GPU's outputs for those
    steps (an eager re-run of the timed steps, outside the timed region)."""
    import torch
    import synthetic.gen as SG
    cfg, L = wl.cfg, wl.L
    lsel = sorted(set(int(round(i * (L - 1) / max(nl - 1, 1))) for i in range(nl)))
    arrays = {"wdtype": np.array(cfg.wdtype), "pdtype": np.array(cfg.pdtype), "act": np.array(cfg.act)}
    for j in lsel:
        for k, v in wl.tensors[j].items():
            if k != "perm":
                arrays[f"L{j}/{k}"] = SG.storage_numpy(v)
    layer_of, thr = [], []
    i = 0
    for s in range(wl.W, wl.W + ns):
        wl.launch(s)
        torch.cuda.synchronize()
        for j in lsel:
            b = wl.st.bufs[j] if wl.mode in ("fused", "pipeline") else None
            if b is None:
                raise RuntimeError("the oracle sample needs a fused path")
            kk = int(b["count"].item())
            arrays[f"x{i}"] = SG.storage_numpy(wl.xs[j][s])
            if wl.mode == "pipeline":
                arrays[f"xp{i}"] = SG.storage_numpy(wl.pred_inputs(s)[j])
            arrays[f"scores{i}"] = b["scores"].cpu().numpy()
            arrays[f"idx{i}"] = b["idx"][:kk].cpu().numpy()
            arrays[f"hact{i}"] = b["hact"][:kk].cpu().numpy()
            arrays[f"y{i}"] = b["y"].cpu().numpy()
            layer_of.append(j)
            thr.append(wl.layers[j].threshold)
            i += 1
    arrays["layer_of"] = np.array(layer_of)
    arrays["threshold"] = np.array(thr, dtype=np.float64)
    ncores = len(os.sched_getaffinity(0))
    runs = {}
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "in.npz")
        np.savez(src, **arrays)
        for threads in (1, ncores):
            env = dict(os.environ)
            for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
                env[var] = str(threads)
            say(f"oracle on {len(layer_of)} layer-steps, {threads} thread(s)")
            out = subprocess.run([sys.executable, os.path.join(ROOT, "oracle", "time_oracle.py"), src,
                                  os.path.join(td, "out.npz")], env=env, capture_output=True, text=True,
                                 timeout=900)
            if out.returncode != 0:
                raise RuntimeError(f"oracle timing failed:\n{out.stderr[-2000:]}")
            runs[threads] = json.loads(out.stdout.strip().splitlines()[-1])
    n = len(layer_of)
    rN, r1 = runs[ncores], runs[1]
    sample = (f"{len(lsel)} layers ({', '.join(map(str, lsel))}) x {ns} timed decode steps of the benchmark "
              f"workload (batch {wl.B}), fp64 numpy oracle unchanged: {rN['seconds']:.1f} s on {ncores} threads, "
              f"{r1['seconds']:.1f} s on 1 thread")
    base = {"value": round(wl.B * n / rN["seconds"], 3), "unit": "tokens/s/layer", "cores": ncores,
            "kind": "oracle", "sample": sample, "single_thread_value": round(wl.B * n / r1["seconds"], 3),
            "cpu_model": cpu_model()}
    par = {k: rN[k] for k in ("score_err", "near_threshold", "mask_mismatch", "hact_rel", "y_rel", "y_rel_own_list")}
    par.update({"layer_steps": n, "bar": {"score_err": 1e-5, "y_rel": 1e-3 if cfg.wdtype != "q4" else 2e-3,
                                          "mask_mismatch": 0}})
    return base, par


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
    from activation_sparse_ffn_amd import StackStep
    from activation_sparse_ffn_amd import _abi as A

    A.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.stream_probe:
        print(json.dumps(stream_probe(dev, args.stream_probe)), flush=True)
        return
    if args.churn:
        print(json.dumps(hot_region_churn(dev)), flush=True)
        return
    if args.dense_switch:
        print(json.dumps(dense_switch_study(dev)), flush=True)
        return

    def mode_for(cfg, B, pipeline):
        if pipeline:
            if not StackStep.supported(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, pipeline=True):
                print("bench.py: the Live Pipeline kernel does not take this shape", file=sys.stderr)
                sys.exit(2)
            return "pipeline"
        # the fused step wherever it takes the shape (up to 4 tokens): measured faster
        # than the separate calls at 1-4 tokens on both 7B shapes (at 3 tokens 41.7
        # against 52.4 us per layer-step, OPT-6.7B); --separate forces the calls
        fused = (not args.separate) and not cfg.pred_q4 and \
            StackStep.supported(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act)
        return "fused" if fused else "separate"

    cfg = S.CONFIGS[args.config]
    if args.pred_q4:
        cfg = S.scaled(cfg, name=cfg.name, pred_q4=True,
                       workload=cfg.workload + ", int4 g32 predictor")
    B = args.batch
    L = args.layers or cfg.layers
    wl = Workload(args, cfg, B, L, mode_for(cfg, B, args.pipeline), dev)
    r = time_workload(wl, args.roofline_steps)
    ms_step = r["ms_step"]
    result = {
        "metric": METRIC,
        "value": round(B * L / (ms_step * 1e-3), 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.wdtype,
        "data": "synthetic (seeded, generated on device)" +
                ("; raw-order layers calibrated on the device" if wl.calibration else ""),
        "config": {"workload": cfg.workload, "batch": B, "layers": L, "d": cfg.d, "f": cfg.f, "h": cfg.h,
                   "act": cfg.act, "density": cfg.density, "calibration": wl.calibration,
                   "tam": {"lambda": args.tam_lambda, "eps": args.tam_eps, "K": wl.tam_k, "G": wl.G}},
        "us_per_layer_step": round(ms_step * 1e3 / L, 3),
        "effective_GBps": round(r["gbps"], 1),
        "hbm_frac": round(r["gbps"] / PEAK_HBM_GBPS, 4),
        "mean_active": round(float(r["counts"].mean()), 1),
        "bytes_per_layer_step": round(r["step_bytes"] / L, 0),
        "path": wl.mode,
        "roofline": r["roofline"],
    }
    if not args.no_cpu_baseline and wl.mode in ("fused", "pipeline"):
        base, par = cpu_baseline_and_parity(wl, min(args.cpu_layers, L), min(args.cpu_steps, args.steps))
        result["cpu_baseline"] = base
        result["parity_sample"] = par
    del wl
    torch.cuda.empty_cache()

    if not args.no_extra and args.config == "C2" and B == 1 and not args.pipeline and not args.separate:
        extra = {}
        c3 = S.CONFIGS["C3"]
        w3 = Workload(args, c3, 1, c3.layers, mode_for(c3, 1, False), dev)
        extra["llama2_7b_reglu_b1"] = summary(w3, time_workload(w3, args.roofline_steps))
        del w3
        torch.cuda.empty_cache()
        pipes = {}
        for name, c in (("opt6.7b_b1", S.CONFIGS["C2"]), ("llama2_7b_reglu_b1", c3)):
            wp = Workload(args, c, 1, c.layers, "pipeline", dev)
            s = summary(wp, time_workload(wp, args.roofline_steps))
            s["mask_recall"] = mask_recall(wp, dev, range(args.warmup, args.warmup + min(8, args.steps)))
            pipes[name] = s
            del wp
            torch.cuda.empty_cache()
        extra["live_pipeline"] = pipes
        extra["stream_read_ceiling"] = stream_probe(dev)
        extra["tam_hot_region"] = hot_region_churn(dev)
        torch.cuda.empty_cache()
        extra["dense_switch"] = dense_switch_study(dev)
        torch.cuda.empty_cache()
        result["extra"] = extra

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
