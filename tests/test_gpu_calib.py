"""GPU parity of the offline calibration (PowerInfer page, Method: offline profiling
and the neuron table; KAIROX page, Core method, item 1; Paper vs code, predictor
threshold).

* the threshold: sfx_select_kth equals the order statistic of the GPU's own scores
  bit for bit, and lies within 1e-5 of the oracle's fp64 quantile of fp64 scores;
* the counts: bit-exact against the masks of the GPU's scores at that threshold;
* the table: bit-exact against the oracle's hot_first_order on the same counts;
* the reordered rows: byte-exact gathers; the step on the calibrated layer maps the
  raw layer's index set through the table and leaves y unchanged."""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic as S
from activation_sparse_ffn_amd import StepBuffers, run_layer
from activation_sparse_ffn_amd import _abi as A
from activation_sparse_ffn_amd.calib import apply_order, calibrate_layer, calibration_scores
from gpu_helpers import check_step, layer_np, rel_err, say
from oracle import sfx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"

CAL = {
    "C1": S.CONFIGS["C1"],
    "C2c": S.scaled(S.CONFIGS["C2"], name="C2c", d=512, f=4096, h=256),
    "C3c": S.scaled(S.CONFIGS["C3"], name="C3c", d=512, f=3104, h=256),
    "C4c": S.scaled(S.CONFIGS["C4"], name="C4c", d=512, f=4096, h=256),
    "C4qc": S.scaled(S.CONFIGS["C4"], name="C4qc", d=512, f=4096, h=256, pred_q4=True),
    "C5c": S.scaled(S.CONFIGS["C5"], name="C5c", d=512, f=4096, h=256),
}


def _kth_ref(v: np.ndarray, k: int) -> np.float32:
    return np.sort(v.astype(np.float32).ravel())[k]


@pytest.mark.parametrize("case", ["normal", "ties", "signed_zero", "one", "extremes"])
def test_select_kth(case):
    rng = np.random.default_rng({"normal": 1, "ties": 2, "signed_zero": 3, "one": 4, "extremes": 5}[case])
    if case == "normal":
        v = rng.standard_normal(1_000_003).astype(np.float32)
    elif case == "ties":
        v = rng.integers(-3, 4, size=200_000).astype(np.float32)
    elif case == "signed_zero":
        v = np.array([0.0, -0.0, 1.0, -1.0, -0.0, 0.0, 2.5], np.float32)
    elif case == "one":
        v = np.array([-7.25], np.float32)
    else:
        v = np.array([np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45, -1e-45, 0.0], np.float32)
    vd = torch.from_numpy(v).to(DEV)
    out = torch.empty(1, dtype=torch.float32, device=DEV)
    ks = sorted({0, v.size // 3, v.size // 2, v.size - 1, max(v.size - 2, 0)})
    for k in ks:
        A.sfx_select_kth(vd, k, out)
        got = np.float32(out.item())
        ref = _kth_ref(v, k)
        say(f"select_kth {case} n={v.size} k={k}: {got} ref {ref}")
        assert got == ref                      # +0 and -0 compare equal: both are the k-th value


def calibrated_layer(cfg, layer: S.Layer, n_cal: int):
    """Calibrate a raw layer on n_cal calibration tokens (a stream disjoint from the
    measured tokens); returns (calibrated Layer, calibration result, tokens)."""
    toks = S.make_tokens(cfg, layer.index, n_cal, 1, device=DEV, tag="calib")[:, 0]
    r = calibrate_layer(layer.tensors(), toks, cfg.density, group=layer.group)
    t = dict(layer.tensors())
    if layer.group is not None:
        t["group"] = layer.group
    c = apply_order(t, r["perm"])
    perm = r["perm"].cpu().numpy()
    new = dataclasses.replace(layer, threshold=r["threshold"], p=layer.p[perm],
                              **{k: c.get(k) for k in ("W2", "W2_s", "Wa", "Wa_s", "Wl", "Wl_s", "Wd", "Wd_s",
                                                        "ba", "perm", "group")})
    return new, r, toks


@pytest.mark.parametrize("name", list(CAL))
def test_calibration_against_oracle(name):
    cfg = CAL[name]
    n_cal = 256
    raw = S.make_layer(cfg, 0, device=DEV, order="raw")
    say(f"calibration {name}: f={cfg.f}, {n_cal} tokens")
    cal, r, toks = calibrated_layer(cfg, raw, n_cal)
    torch.cuda.synchronize()
    # threshold: order statistic of the GPU's scores, and the oracle's fp64 quantile
    s_gpu = calibration_scores(raw.tensors(), toks).cpu().numpy()
    k = min(int((1.0 - cfg.density) * s_gpu.size), s_gpu.size - 1)
    assert np.float32(r["threshold"]) == _kth_ref(s_gpu, k)
    lnp = layer_np(raw)
    s64 = O.predict(O.decode(S.storage_numpy(toks), cfg.pdtype), *O.predictor_weights(lnp, cfg.pdtype))
    t64 = O.calib_threshold(s64, cfg.density)
    say(f"   threshold {r['threshold']:.6f} vs fp64 {t64:.6f}; active share {r['active_share']:.4f}")
    assert abs(r["threshold"] - t64) <= 1e-5
    # counts from the GPU's masks; table from the oracle on the same counts
    counts = r["counts"].cpu().numpy()
    assert np.array_equal(counts, O.neuron_counts(s_gpu >= np.float32(r["threshold"])))
    group = raw.group.cpu().numpy() if raw.group is not None else None
    perm = r["perm"].cpu().numpy()
    assert np.array_equal(perm, O.hot_first_order(counts, group))
    # reordered rows are exact gathers of the raw rows
    pt = r["perm"].long()
    for key in ("W2", "W2_s", "Wa", "Wa_s", "Wl", "Wl_s", "Wd", "Wd_s", "ba"):
        a = getattr(raw, key)
        if a is not None:
            assert torch.equal(getattr(cal, key).view(torch.uint8), a[pt].view(torch.uint8)), key
    if group is not None:                           # planted groups land as aligned blocks of 32
        blocks = cal.group.cpu().numpy().reshape(-1, 32)
        assert np.all(blocks == blocks[:, :1])
    # the hot-first order concentrates activity at the front (power-law predictors)
    if cfg.pred_profile == "zipf":
        head = max(cfg.f // 10, 32)
        assert counts[perm[:head]].sum() > 2.5 * counts.sum() * head / cfg.f

    # one measured token through the raw and the calibrated layer
    x = S.make_tokens(cfg, 0, 1, 2, device=DEV)[0]
    bufs = [StepBuffers(cfg.d, cfg.f, cfg.h, 2, cfg.wdtype, cfg.pred_storage) for _ in range(2)]
    run_layer(bufs[0], raw.tensors(), x, cal.threshold, cfg.act)
    run_layer(bufs[1], cal.tensors(), x, cal.threshold, cfg.act)
    torch.cuda.synchronize()
    inv = np.argsort(perm)
    k0, k1 = int(bufs[0].count.item()), int(bufs[1].count.item())
    idx0, idx1 = bufs[0].idx[:k0].cpu().numpy(), bufs[1].idx[:k1].cpu().numpy()
    assert k0 == k1 and np.array_equal(np.sort(inv[idx0]), idx1)
    y0, y1 = bufs[0].y.cpu().numpy(), bufs[1].y.cpu().numpy()
    assert rel_err(y1, y0) <= 1e-5, rel_err(y1, y0)
    out = {"scores": bufs[1].scores.cpu().numpy(), "tok_bits": bufs[1].tok_bits.cpu().numpy().view(np.uint32),
           "union_bits": bufs[1].union_bits.cpu().numpy().view(np.uint32), "idx": idx1, "count": k1,
           "hact": bufs[1].hact[:k1].cpu().numpy(), "y": y1}
    check_step(cfg, layer_np(cal), S.storage_numpy(x), out, cal.threshold)


def test_calibration_falcon40b_full_size():
    """One Falcon-40B-shaped layer (f = 32768, 1024 planted groups) calibrated on 256
    tokens (8.4M scores): threshold against the fp64 quantile, counts, table and
    group blocks as above."""
    cfg = S.CONFIGS["C5"]
    raw = S.make_layer(cfg, 0, device=DEV, order="raw")
    say("calibration Falcon-40B shape")
    cal, r, toks = calibrated_layer(cfg, raw, 256)
    s_gpu = calibration_scores(raw.tensors(), toks).cpu().numpy()
    k = min(int((1.0 - cfg.density) * s_gpu.size), s_gpu.size - 1)
    assert np.float32(r["threshold"]) == _kth_ref(s_gpu, k)
    lnp = {"W1": S.storage_numpy(raw.W1), "W2": S.storage_numpy(raw.W2)}
    s64 = O.predict(O.decode(S.storage_numpy(toks), cfg.pdtype), *O.predictor_weights(lnp, cfg.pdtype))
    t64 = O.calib_threshold(s64, cfg.density)
    say(f"   threshold {r['threshold']:.6f} vs fp64 {t64:.6f}")
    assert abs(r["threshold"] - t64) <= 1e-5
    counts = r["counts"].cpu().numpy()
    assert np.array_equal(counts, O.neuron_counts(s_gpu >= np.float32(r["threshold"])))
    perm = r["perm"].cpu().numpy()
    assert np.array_equal(perm, O.hot_first_order(counts, raw.group.cpu().numpy()))
    blocks = cal.group.cpu().numpy().reshape(-1, 32)
    assert np.all(blocks == blocks[:, :1])
    for key in ("Wa", "Wd", "ba"):
        idx = torch.tensor([0, 1, 4095, 32767], device=DEV)
        assert torch.equal(getattr(cal, key)[idx], getattr(raw, key)[r["perm"].long()[idx]]), key
