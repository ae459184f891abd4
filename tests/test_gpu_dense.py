"""GPU parity of the dense FFN (sfx_dense_ffn: every neuron, no predictor) against the
fp64 oracle's dense layer, and bit-for-bit against the sparse step whose mask holds
every neuron (threshold -inf: the same kernels on the list 0..f-1).  Bar: hact and y
within 1e-3 relative (2e-3 for int4) of the oracle."""
import numpy as np
import pytest
import torch

import synthetic as S
from activation_sparse_ffn_amd import StepBuffers, run_layer
from activation_sparse_ffn_amd import _abi as A
from gpu_helpers import Y_RTOL, layer_np, rel_err, say
from oracle import sfx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"

SCALED = {
    "C1": S.CONFIGS["C1"],
    "C2s": S.scaled(S.CONFIGS["C2"], name="C2s", d=1032, f=3000, h=136),
    "C3s": S.scaled(S.CONFIGS["C3"], name="C3s", d=1032, f=2080, h=136),
    "C4s": S.scaled(S.CONFIGS["C4"], name="C4s", d=1056, f=2000, h=136),
    "C5s": S.scaled(S.CONFIGS["C5"], name="C5s", d=1032, f=4096, h=264),
    "C2r": S.scaled(S.CONFIGS["C2"], name="C2r", d=1032, f=3000, h=136, act="relu2"),
}


def _dense(cfg, layer, x, act=None):
    t = layer.tensors()
    B = x.shape[0]
    wdt = A.WDT.get(t["Wa"].dtype, A.SFX_Q4G32)
    hact = torch.empty(cfg.f, B, dtype=torch.float32, device=DEV)
    y = torch.empty(B, cfg.d, dtype=torch.float32, device=DEV)
    ws = A.workspace(A.sfx_dense_ffn_ws(wdt, B, cfg.d, cfg.f), DEV)
    A.sfx_dense_ffn(x, t["Wa"], t["ba"], t["Wd"], hact, y, ws, act=act or cfg.act, Wa_scales=t.get("Wa_s"),
                    Wl=t.get("Wl"), Wl_scales=t.get("Wl_s"), Wd_scales=t.get("Wd_s"))
    torch.cuda.synchronize()
    return hact.cpu().numpy(), y.cpu().numpy()


def _oracle_dense(cfg, lnp, x_np):
    wd = cfg.wdtype
    x64 = O.decode(x_np, cfg.pdtype)
    idx = np.arange(cfg.f)
    Wa = O.rows(lnp["Wa"], wd, idx, lnp.get("Wa_s"))
    Wd = O.rows(lnp["Wd"], wd, idx, lnp.get("Wd_s"))
    Wl = O.rows(lnp["Wl"], wd, idx, lnp.get("Wl_s")) if cfg.act == "reglu" else None
    hact = O.sparse_up(x64, Wa, np.asarray(lnp["ba"], np.float64), cfg.act, Wl)
    return hact, O.dense_ffn(x64, Wa, lnp["ba"], Wd, cfg.act, Wl)


@pytest.mark.parametrize("name,B", [("C1", 1), ("C2s", 1), ("C2s", 3), ("C3s", 4), ("C3s", 17), ("C4s", 2),
                                    ("C4s", 16), ("C5s", 32), ("C5s", 64), ("C2r", 5)])
def test_dense_against_oracle(name, B):
    cfg = SCALED[name]
    layer = S.make_layer(cfg, 0, device=DEV)
    x = S.make_tokens(cfg, 0, 1, B, device=DEV)[0]
    say(f"dense {name} B={B}")
    hact, y = _dense(cfg, layer, x)
    hact_ref, y_ref = _oracle_dense(cfg, layer_np(layer), S.storage_numpy(x))
    r_h, r_y = rel_err(hact, hact_ref), rel_err(y, y_ref)
    say(f"   hact_rel {r_h:.2e}  y_rel {r_y:.2e}")
    assert r_h <= Y_RTOL[cfg.wdtype] and r_y <= Y_RTOL[cfg.wdtype]


@pytest.mark.parametrize("name,B", [("C2s", 1), ("C3s", 4), ("C4s", 16), ("C5s", 32)])
def test_dense_equals_all_ones_sparse_step(name, B):
    """The sparse step at threshold -inf lists every neuron: same kernels, same y."""
    cfg = SCALED[name]
    layer = S.make_layer(cfg, 0, device=DEV)
    x = S.make_tokens(cfg, 0, 1, B, device=DEV)[0]
    hact, y = _dense(cfg, layer, x)
    buf = StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pred_storage)
    run_layer(buf, layer.tensors(), x, float("-inf"), cfg.act)
    torch.cuda.synchronize()
    assert int(buf.count.item()) == cfg.f
    assert np.array_equal(buf.y.cpu().numpy(), y)
    assert np.array_equal(buf.hact.cpu().numpy(), hact)


def test_dense_falcon40b_full_size():
    """Falcon-40B-shaped layer (d = 8192, f = 32768) at 32 tokens against the fp64
    dense layer on 8 sampled tokens' outputs."""
    cfg = S.CONFIGS["C5"]
    layer = S.make_layer(cfg, 0, device=DEV)
    x = S.make_tokens(cfg, 0, 1, 32, device=DEV)[0]
    say("dense Falcon-40B shape, 32 tokens")
    hact, y = _dense(cfg, layer, x)
    lnp = {k: S.storage_numpy(getattr(layer, k)) for k in ("Wa", "ba", "Wd")}
    xs = S.storage_numpy(x)
    for b in (0, 7, 19, 31):
        x64 = O.decode(xs[b:b + 1], cfg.pdtype)
        ref = O.dense_ffn(x64, O.decode(lnp["Wa"], "f16"), lnp["ba"], O.decode(lnp["Wd"], "f16"), "relu")
        r = rel_err(y[b:b + 1], ref)
        say(f"   token {b}: y_rel {r:.2e}")
        assert r <= Y_RTOL["f16"]
