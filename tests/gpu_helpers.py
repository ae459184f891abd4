"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI on
seeded synthetic layers, run the fp64 oracle on the same storage, compare."""
import sys

import numpy as np
import torch

import synthetic as S
from activation_sparse_ffn_amd import StepBuffers, run_layer
from oracle import sfx_oracle as O

SCORE_ATOL = 1e-5       # |s_gpu - s64|: well inside the 1e-4 exclusion window
NEAR = 1e-4             # neurons with |s64 - t| < NEAR may legitimately differ
Y_RTOL = {"f32": 1e-3, "f16": 1e-3, "bf16": 1e-3, "q4": 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def layer_np(L: S.Layer) -> dict:
    return {k: S.storage_numpy(v) for k, v in L.tensors().items()}


def gpu_layer_step(cfg, L, x: torch.Tensor, threshold=None, buf=None):
    """Run predict -> compact -> up -> down on the GPU; return host copies."""
    B = x.shape[0]
    if buf is None:
        buf = StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pred_storage)
    t = L.threshold if threshold is None else threshold
    run_layer(buf, L.tensors(), x, t, cfg.act)
    torch.cuda.synchronize()
    buf.check_status()
    k = int(buf.count.item())
    return {
        "scores": buf.scores.cpu().numpy(),
        "tok_bits": buf.tok_bits.cpu().numpy().view(np.uint32),
        "union_bits": buf.union_bits.cpu().numpy().view(np.uint32),
        "idx": buf.idx[:k].cpu().numpy(),
        "count": k,
        "hact": buf.hact[:k].cpu().numpy(),
        "y": buf.y.cpu().numpy(),
    }, buf


def rel_err(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(a - ref)) if ref.size else 0.0
    return num / den if den > 0 else num


def check_step(cfg, Lnp: dict, x_np: np.ndarray, out: dict, t: float, report: dict = None, xp_np=None):
    """Every comparison of one layer-step (the predictor scores `xp_np` when given:
    the Live Pipeline step).  Returns a dict of measured errors."""
    pd, wd = cfg.pdtype, cfg.wdtype
    x64 = O.decode(x_np, pd)
    xp64 = x64 if xp_np is None else O.decode(xp_np, pd)
    s64 = O.predict(xp64, *O.predictor_weights(Lnp, pd))
    r = {}

    # (1) scores against fp64
    r["score_err"] = float(np.max(np.abs(out["scores"].astype(np.float64) - s64)))
    assert r["score_err"] <= SCORE_ATOL, r

    # (2) the gate on the GPU's own fp32 scores: bit-exact
    tok, uni, idx, cnt = O.gate(out["scores"].astype(np.float64), t)
    if out.get("tok_bits") is not None:
        assert np.array_equal(O.pack_bits(tok), out["tok_bits"]), "tok_bits"
    assert np.array_equal(O.pack_bits(uni), out["union_bits"]), "union_bits"
    assert cnt == out["count"] and np.array_equal(idx, out["idx"]), "idx"

    # (3) the gate against fp64 scores, outside the exclusion window
    tok64, _, _, _ = O.gate(s64, t)
    near = np.abs(s64 - t) < NEAR
    assert np.array_equal(tok64[~near], tok[~near]), "mask differs outside the window"
    r["near_threshold"] = int(near.sum())

    # (4) activations and y on the GPU's index list
    gidx = out["idx"]
    Wl = O.rows(Lnp["Wl"], wd, gidx, Lnp.get("Wl_s")) if cfg.act == "reglu" else None
    hact_ref = O.sparse_up(x64, O.rows(Lnp["Wa"], wd, gidx, Lnp.get("Wa_s")),
                           np.asarray(Lnp["ba"], np.float64)[gidx], cfg.act, Wl)
    y_ref = O.sparse_down(O.rows(Lnp["Wd"], wd, gidx, Lnp.get("Wd_s")), hact_ref)
    r["hact_rel"] = rel_err(out["hact"], hact_ref)
    r["y_rel"] = rel_err(out["y"], y_ref)
    assert r["hact_rel"] <= Y_RTOL[wd], r
    assert r["y_rel"] <= Y_RTOL[wd], r
    r["count"] = out["count"]
    if report is not None:
        report.update(r)
    return r
