"""GPU parity of the Live Pipeline step (sfx_ffn_pipeline): each layer's predictor
scores its predictor input (the previous layer's FFN input; layer 0: the previous
token's), the FFN rows use the layer's own input.  Every layer's outputs against
the fp64 oracle with the bar of the exact step; bitwise reproducibility, graph
replays, the long-list and W2-from-memory paths, empty and full lists."""
import numpy as np
import pytest
import torch

import synthetic as S
from activation_sparse_ffn_amd import StackStep
from gpu_helpers import check_step, layer_np, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

SMALL = {
    "C2s": S.scaled(S.CONFIGS["C2"], name="C2f", d=1032, f=3000, h=136),
    "C3s": S.scaled(S.CONFIGS["C3"], name="C3f", d=1032, f=2080, h=136),
    "C2m": S.scaled(S.CONFIGS["C2"], name="C2m", d=2048, f=8192, h=512),
}
WIDE = S.scaled(S.CONFIGS["C2"], name="C2w", d=4096, f=32768, h=1024)


def _outputs(st, l):
    b = st.bufs[l]
    k = int(b["count"].item())
    return {"scores": b["scores"].cpu().numpy(), "tok_bits": b["tok_bits"].cpu().numpy().view(np.uint32),
            "union_bits": b["union_bits"].cpu().numpy().view(np.uint32), "idx": b["idx"][:k].cpu().numpy(),
            "count": k, "hact": b["hact"][:k].cpu().numpy(), "y": b["y"].cpu().numpy()}


def _pred_inputs(xs, s):
    """Predictor inputs of step s: layer l > 0 scores x_{l-1} of the same step,
    layer 0 the layer-0 input of the previous step (its own at step 0)."""
    L = len(xs)
    return [xs[0][max(s - 1, 0)]] + [xs[l - 1][s] for l in range(1, L)]


def _run_and_check(cfg, L, B, steps, threshold=None, min_k=None):
    layers = [S.make_layer(cfg, l, device=DEV) for l in range(L)]
    if threshold is not None:
        for ly in layers:
            ly.threshold = threshold
    lnp = [layer_np(ly) for ly in layers]
    xs = S.make_layer_chain(cfg, L, steps, B, device=DEV)
    assert StackStep.supported(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, pipeline=True)
    st = StackStep(layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, pipeline=True)
    for s in range(steps):
        xp = _pred_inputs(xs, s)
        descs = st.descriptors([xs[l][s] for l in range(L)], xp, tok_bits=(s % 2 == 0))
        say(f"pipeline {cfg.name} L={L} B={B} step {s}")
        st.run(descs)
        torch.cuda.synchronize()
        st.check_status()
        for l in range(L):
            out = _outputs(st, l)
            if s % 2 == 1:
                out["tok_bits"] = None
            r = check_step(cfg, lnp[l], S.storage_numpy(xs[l][s]), out, layers[l].threshold,
                           xp_np=S.storage_numpy(xp[l]))
            if min_k is not None:
                assert r["count"] > min_k, r
            if l == 0:
                say("   ", {k: (round(v, 8) if isinstance(v, float) else v) for k, v in r.items()})
    return st


@pytest.mark.parametrize("name,B", [("C2s", 1), ("C2s", 3), ("C3s", 1), ("C3s", 2), ("C3s", 4), ("C2m", 1)])
def test_pipeline_scaled(name, B):
    _run_and_check(SMALL[name], 3, B, 3)


@pytest.mark.parametrize("name,B", [("C2", 1), ("C3", 1), ("C3", 4)])
def test_pipeline_full_size(name, B):
    _run_and_check(S.CONFIGS[name], 3, B, 2)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [1, 4])
def test_pipeline_long_list_w2_from_memory(B):
    """k ~ 6.5k / 19k: longer than the LDS list and than one down batch; W2 rows
    of a workgroup (256 KB) read from memory."""
    _run_and_check(WIDE, 2, B, 2, threshold=S.threshold_for_share(WIDE, 0.2), min_k=4920)
    torch.cuda.empty_cache()


def test_pipeline_reglu_list_too_long_for_input_in_lds():
    """LLaMA2-7B shape at one token with about 30% of the neurons active: the list
    (k ~ 3.3k) leaves no room for the input below the hidden in LDS, so the ReGLU
    up rows read it from memory (at the default density they read it from LDS)."""
    cfg = S.CONFIGS["C3"]
    _run_and_check(cfg, 2, 1, 2, threshold=S.threshold_for_share(cfg, 0.3), min_k=1848)
    torch.cuda.empty_cache()


def test_pipeline_threshold_extremes():
    cfg = SMALL["C2s"]
    layers = [S.make_layer(cfg, l, device=DEV) for l in range(2)]
    xs = S.make_layer_chain(cfg, 2, 1, 1, device=DEV)
    x = [xs[l][0] for l in range(2)]
    for t in (float("inf"), float("-inf")):
        for ly in layers:
            ly.threshold = t
        st = StackStep(layers, cfg.d, cfg.f, cfg.h, 1, cfg.wdtype, cfg.act, pipeline=True)
        say(f"pipeline threshold {t}")
        st.run(st.descriptors(x, _pred_inputs(xs, 0)))
        torch.cuda.synchronize()
        st.check_status()
        for l in range(2):
            out = _outputs(st, l)
            if t > 0:
                assert out["count"] == 0 and not out["y"].any()
            else:
                assert out["count"] == cfg.f and np.array_equal(out["idx"], np.arange(cfg.f))
                check_step(cfg, layer_np(layers[l]), S.storage_numpy(x[l]), out, t,
                           xp_np=S.storage_numpy(_pred_inputs(xs, 0)[l]))


def test_pipeline_without_xp_matches_exact_step_masks():
    """With no predictor inputs (xp = x) the pipeline scores exactly what the exact
    step scores: scores, masks and lists bit for bit (the same sums in the same
    order); activations and y agree to fp32 rounding (their sums are grouped
    differently: each up row is split over four waves, the down rows over row
    slices and column bands)."""
    cfg = SMALL["C3s"]
    L, B = 3, 2
    layers = [S.make_layer(cfg, l, device=DEV) for l in range(L)]
    xs = S.make_layer_chain(cfg, L, 1, B, device=DEV)
    x = [xs[l][0] for l in range(L)]
    ex = StackStep(layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act)
    pp = StackStep(layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, pipeline=True)
    ex.run(ex.descriptors(x))
    pp.run(pp.descriptors(x))
    torch.cuda.synchronize()
    for l in range(L):
        a, b = _outputs(ex, l), _outputs(pp, l)
        for key in ("scores", "tok_bits", "union_bits", "idx"):
            assert np.array_equal(a[key], b[key]), (l, key)
        for key in ("hact", "y"):
            assert np.max(np.abs(a[key] - b[key])) <= 1e-5 * np.max(np.abs(a[key])), (l, key)


def test_pipeline_determinism_and_graph_replay():
    cfg = SMALL["C2m"]
    L, B = 4, 1
    layers = [S.make_layer(cfg, l, device=DEV) for l in range(L)]
    xs = S.make_layer_chain(cfg, L, 3, B, device=DEV)
    inputs = [xs[l][0].clone() for l in range(L)]
    preds = [xs[l][0].clone() for l in range(L)]
    st = StackStep(layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, pipeline=True)
    static = st.descriptors(inputs, preds)

    def load(s):
        for l in range(L):
            inputs[l].copy_(xs[l][s])
            preds[l].copy_(_pred_inputs(xs, s)[l])

    eager = []
    for s in range(3):
        load(s)
        st.run(static)
        torch.cuda.synchronize()
        eager.append([_outputs(st, l) for l in range(L)])
    load(2)
    st.run(static)
    torch.cuda.synchronize()
    for l in range(L):
        o = _outputs(st, l)
        for key in ("scores", "union_bits", "idx", "hact", "y"):
            assert np.array_equal(o[key], eager[2][l][key]), key
    say("pipeline graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(static)
    for s in range(3):
        load(s)
        g.replay()
        torch.cuda.synchronize()
        st.check_status()
        for l in range(L):
            o = _outputs(st, l)
            for key in ("idx", "hact", "y"):
                assert np.array_equal(o[key], eager[s][l][key]), (s, l, key)
        _ = torch.randn(1000, device=DEV).sum().item()
