"""Offline calibration of one layer on calibration tokens (PowerInfer page, Method:
offline profiling of activation frequencies and the neuron table; KAIROX page,
Core method, item 1: co-active neurons stored as contiguous groups; Paper vs code,
predictor threshold).  Orchestration only: scores, threshold, counts, order and the
reordered weights all come from libsfx kernels (sfx_predict / sfx_predict_q4,
sfx_select_kth, sfx_compact, sfx_count_active, sfx_hot_first_order,
sfx_gather_rows).

    scores    = the predictor on every calibration token
    threshold = k-th smallest score, k = floor((1 - density) * tokens * f)
    counts[i] = calibration tokens whose mask (score >= threshold) holds neuron i
    perm      = hot-first table (groups by total count, then members by count)
    weights   = every per-neuron row (W2, Wa, Wl, Wd, their scales, ba) in perm order
"""
import torch

from . import _abi as A

ROW_KEYS = ("W2", "W2_s", "Wa", "Wa_s", "Wl", "Wl_s", "Wd", "Wd_s", "ba", "perm", "group")
MAX_CHUNK = 64


def calibration_scores(layer: dict, tokens: torch.Tensor) -> torch.Tensor:
    """Predictor scores [N][f] of N calibration tokens [N][d] (in chunks of 64)."""
    N, d = tokens.shape
    f = layer["W2"].shape[0]
    h = layer["W1"].shape[0]
    q4 = layer.get("W1_s") is not None
    pdt = A.SFX_Q4G32 if q4 else A._wdt_of(tokens)
    scores = torch.empty(N, f, dtype=torch.float32, device=tokens.device)
    ws = A.workspace(A.sfx_predict_ws(pdt, min(N, MAX_CHUNK), d, h, f), tokens.device)
    for b0 in range(0, N, MAX_CHUNK):
        x = tokens[b0:b0 + MAX_CHUNK]
        out = scores[b0:b0 + x.shape[0]]
        if q4:
            A.sfx_predict_q4(x, layer["W1"], layer["W1_s"], layer["W2"], layer["W2_s"], out, ws)
        else:
            A.sfx_predict(x, layer["W1"], layer["W2"], out, ws)
    if int(ws[:4].view(torch.int32).item()) != 0:
        raise RuntimeError("calibration: a predictor hidden value left the fp16 range")
    return scores


def calibrate_layer(layer: dict, tokens: torch.Tensor, density: float, group: torch.Tensor = None):
    """Threshold, per-neuron counts and hot-first table of one layer.

    layer: device tensors W1, W2 (+ W1_s, W2_s for an int4 predictor); tokens [N][d]
    in the predictor's input dtype; group: optional [f] int32 group id per slot.
    Returns {"threshold": float, "counts": [f] int32, "perm": [f] int32,
    "active_share": float (share of calibration scores >= threshold)}."""
    if not 0.0 < density < 1.0:
        raise ValueError("density must lie in (0, 1)")
    dev = tokens.device
    scores = calibration_scores(layer, tokens)
    N, f = scores.shape
    k = min(int((1.0 - density) * N * f), N * f - 1)
    t_dev = torch.empty(1, dtype=torch.float32, device=dev)
    A.sfx_select_kth(scores, k, t_dev)
    threshold = float(t_dev.item())
    W = (f + 31) // 32
    counts = torch.zeros(f, dtype=torch.int32, device=dev)
    B = min(N, MAX_CHUNK)
    tok_bits = torch.zeros(B, W, dtype=torch.int32, device=dev)
    union = torch.zeros(W, dtype=torch.int32, device=dev)
    idx = torch.zeros(f, dtype=torch.int32, device=dev)
    cnt = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = A.workspace(A.sfx_compact_ws(B, f), dev)
    for b0 in range(0, N, B):
        s = scores[b0:b0 + B]
        tb = tok_bits[:s.shape[0]]
        A.sfx_compact(s, threshold, union, idx, cnt, ws, tok_bits=tb)
        A.sfx_count_active(tb, f, counts)
    if int(ws[4:8].view(torch.int32).item()) != 0:
        raise RuntimeError("calibration: compaction reported a timeout")
    perm = torch.empty(f, dtype=torch.int32, device=dev)
    A.sfx_hot_first_order(counts, perm, group=group)
    active = int(counts.sum().item())
    return {"threshold": threshold, "counts": counts, "perm": perm, "active_share": active / (N * f)}


def apply_order(layer: dict, perm: torch.Tensor) -> dict:
    """A copy of the layer's tensors with every per-neuron row in `perm` order (new
    slot r = old slot perm[r]); W1 and W1_s are shared, not copied.  A neuron table
    "perm" in the layer composes (new perm[r] = old perm[perm[r]]), and so does a
    per-slot "group"."""
    out = {}
    for key, t in layer.items():
        if t is None:
            continue
        if key in ROW_KEYS:
            dst = torch.empty_like(t)
            A.sfx_gather_rows(t, perm, dst)
            out[key] = dst
        else:
            out[key] = t
    return out
