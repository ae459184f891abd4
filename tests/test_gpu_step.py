"""GPU parity of the fused multi-layer step (sfx_ffn_step): every layer's outputs
against the fp64 oracle with the same bar as the separate calls, the barrier error
word stays zero, results are bitwise reproducible, and graph replays match eager
runs."""
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


def _outputs(st: StackStep, l: int):
    b = st.bufs[l]
    k = int(b["count"].item())
    return {"scores": b["scores"].cpu().numpy(), "tok_bits": b["tok_bits"].cpu().numpy().view(np.uint32),
            "union_bits": b["union_bits"].cpu().numpy().view(np.uint32), "idx": b["idx"][:k].cpu().numpy(),
            "count": k, "hact": b["hact"][:k].cpu().numpy(), "y": b["y"].cpu().numpy()}


def _run_and_check(cfg, L, B, steps, layers=None, threshold=None, min_k=None):
    layers = layers or [S.make_layer(cfg, l, device=DEV) for l in range(L)]
    if threshold is not None:
        for ly in layers:
            ly.threshold = threshold
    lnp = [layer_np(ly) for ly in layers]
    xs = [S.make_tokens(cfg, l, steps, B, device=DEV) for l in range(L)]
    assert StackStep.supported(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act)
    st = StackStep(layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act)
    for s in range(steps):
        descs = st.descriptors([xs[l][s] for l in range(L)], tok_bits=(s % 2 == 0))
        say(f"fused {cfg.name} L={L} B={B} step {s}")
        st.run(descs)
        torch.cuda.synchronize()
        assert st.error_word() == 0
        for l in range(L):
            out = _outputs(st, l)
            if s % 2 == 1:                     # tok_bits not requested this step: keep the last ones out
                out["tok_bits"] = None
            r = check_step(cfg, lnp[l], S.storage_numpy(xs[l][s]), out, layers[l].threshold)
            if min_k is not None:
                assert r["count"] > min_k, r
            if l == 0:
                say("   ", {k: (round(v, 8) if isinstance(v, float) else v) for k, v in r.items()})
    return st


@pytest.mark.parametrize("name,B", [("C2s", 1), ("C2s", 3), ("C3s", 1), ("C3s", 2), ("C3s", 4), ("C2m", 1)])
def test_fused_scaled(name, B):
    _run_and_check(SMALL[name], 3, B, 3)


@pytest.mark.parametrize("name,B", [("C2", 1), ("C3", 1), ("C3", 4)])
def test_fused_full_size(name, B):
    cfg = S.CONFIGS[name]
    _run_and_check(cfg, 2, B, 2)
    torch.cuda.empty_cache()


def test_fused_threshold_extremes():
    """+inf: nothing active in any layer, y = 0; -inf: every neuron active."""
    cfg = SMALL["C2s"]
    layers = [S.make_layer(cfg, l, device=DEV) for l in range(2)]
    x = [S.make_tokens(cfg, l, 1, 1, device=DEV)[0].clone() for l in range(2)]
    for t in (float("inf"), float("-inf")):
        for ly in layers:
            ly.threshold = t
        st = StackStep(layers, cfg.d, cfg.f, cfg.h, 1, cfg.wdtype, cfg.act)
        say(f"fused threshold {t}")
        st.run(st.descriptors(x))
        torch.cuda.synchronize()
        assert st.error_word() == 0
        for l in range(2):
            out = _outputs(st, l)
            if t > 0:
                assert out["count"] == 0 and not out["y"].any()
            else:
                assert out["count"] == cfg.f and np.array_equal(out["idx"], np.arange(cfg.f))
                check_step(cfg, layer_np(layers[l]), S.storage_numpy(x[l]), out, t)


def test_fused_determinism_and_graph_replay():
    cfg = SMALL["C3s"]
    L, B = 3, 2
    layers = [S.make_layer(cfg, l, device=DEV) for l in range(L)]
    xs = [S.make_tokens(cfg, l, 3, B, device=DEV) for l in range(L)]
    inputs = [xs[l][0].clone() for l in range(L)]
    st = StackStep(layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act)
    static = st.descriptors(inputs)
    eager = []
    for s in range(3):
        for l in range(L):
            inputs[l].copy_(xs[l][s])
        st.run(static)
        torch.cuda.synchronize()
        eager.append([_outputs(st, l) for l in range(L)])
    # same inputs again: bitwise identical
    for l in range(L):
        inputs[l].copy_(xs[l][2])
    st.run(static)
    torch.cuda.synchronize()
    for l in range(L):
        o = _outputs(st, l)
        for key in ("scores", "union_bits", "idx", "hact", "y"):
            assert np.array_equal(o[key], eager[2][l][key]), key
    say("fused graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(static)
    for s in range(3):
        for l in range(L):
            inputs[l].copy_(xs[l][s])
        g.replay()
        torch.cuda.synchronize()
        assert st.error_word() == 0
        for l in range(L):
            o = _outputs(st, l)
            for key in ("idx", "hact", "y"):
                assert np.array_equal(o[key], eager[s][l][key]), (s, l, key)
        _ = torch.randn(1000, device=DEV).sum().item()


# Active lists longer than the LDS copy of the list (4920 entries: the down phase
# then finds each rank's neuron from the union words) and W2 rows that do not fit
# the 128 KB LDS region (d = 4096, h = 1024, f = 32768: 4 mask words = 256 KB of
# W2 per workgroup, so the scores read W2 from memory).
NID_CAP = 4920
WIDE = S.scaled(S.CONFIGS["C2"], name="C2w", d=4096, f=32768, h=1024)


@pytest.mark.parametrize("B", [1, 4])
def test_fused_long_list_w2_from_memory(B):
    # about 20% of the neurons active per token (k ~ 6.5k at 1 token, more for the
    # union of 4)
    t = S.threshold_for_share(WIDE, 0.2)
    _run_and_check(WIDE, 2, B, 2, threshold=t, min_k=NID_CAP)
    torch.cuda.empty_cache()


def test_fused_outputs_inside_down_loop():
    """Every neuron active at 4 tokens with f = 32768: 8192 list positions per
    workgroup, more than the LDS area that keeps (neuron, activation) pairs for
    outputs written after the grid-barrier flag (5734 pairs at 4 tokens), so the
    rank-order list and activations are written from the down loop itself."""
    _run_and_check(WIDE, 2, 4, 1, threshold=float("-inf"), min_k=NID_CAP)
    torch.cuda.empty_cache()


def test_fused_reglu_input_in_lds_outputs_inside_down_loop():
    """ReGLU at one token with W2 rows in LDS (h = 256) and every neuron active
    (f = 32768: 8192 list positions per workgroup, more than the 6144 pairs the LDS
    save area holds next to the ReGLU up-row slots): the up rows of the own
    neurons read the input from LDS, the overflow rows read it from memory (the
    standard-layout outputs were built over it before the down loop)."""
    cfg = S.scaled(S.CONFIGS["C3"], name="C3w", d=4096, f=32768, h=256)
    _run_and_check(cfg, 2, 1, 1, threshold=float("-inf"), min_k=NID_CAP)
    torch.cuda.empty_cache()


def test_fused_long_list_w2_in_lds():
    """OPT-6.7B shape (W2 rows in LDS) with every neuron active: 16384 > 4920."""
    cfg = S.CONFIGS["C2"]
    _run_and_check(cfg, 2, 1, 1, threshold=float("-inf"), min_k=NID_CAP)
    torch.cuda.empty_cache()


def test_fused_benchmark_launch():
    """The launch the benchmark times: all 32 layers of the OPT-6.7B-shaped stack at
    one token, union words in one [L][W] array, no per-token masks, two steps per
    graph, replayed twice.  Every replay matches an eager run bit for bit, and
    layers 0, 15 and 31 of the last step match the oracle."""
    cfg = S.CONFIGS["C2"]
    L, B, steps = cfg.layers, 1, 4
    W = cfg.groups
    say("benchmark launch: generating 32 layers")
    layers = [S.make_layer(cfg, l, device=DEV) for l in range(L)]
    xs = [S.make_tokens(cfg, l, steps, B, device=DEV) for l in range(L)]
    ubits = torch.zeros(L, W, dtype=torch.int32, device=DEV)
    st = StackStep(layers, cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.act, union_bits=ubits)
    descs = [st.descriptors([xs[l][s] for l in range(L)], tok_bits=False) for s in range(steps)]
    # eager reference of the last step
    st.run(descs[steps - 1])
    torch.cuda.synchronize()
    st.check_status()
    eager = [_outputs(st, l) for l in range(L)]
    say("benchmark launch: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in (steps - 2, steps - 1):
            st.run(descs[s])
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        st.check_status()
        for l in range(L):
            o = _outputs(st, l)
            for key in ("scores", "union_bits", "idx", "hact", "y"):
                assert np.array_equal(o[key], eager[l][key]), (rep, l, key)
        assert np.array_equal(ubits.cpu().numpy()[L - 1], eager[L - 1]["union_bits"].view(np.int32))
        _ = torch.randn(1000, device=DEV).sum().item()
    for l in (0, 15, 31):
        out = _outputs(st, l)
        out["tok_bits"] = None
        r = check_step(cfg, layer_np(layers[l]), S.storage_numpy(xs[l][steps - 1]), out, layers[l].threshold)
        say(f"   layer {l}", {k: (round(v, 8) if isinstance(v, float) else v) for k, v in r.items()})
    del layers, st
    torch.cuda.empty_cache()


def test_fused_hidden_outside_fp16_range():
    """fp16 predictor rows: the fused step splits the hidden into two fp16 pieces
    for its scores; a hidden value past 65504 sends that layer to fp32 sums.  Layer
    0 gets one hidden row of about 8e5 (W1 row 5 = 1000 sign(x)), layer 1 is
    normal: scores within 1e-5 of fp64 relative to max(1, |s|), the gate bit-exact
    on the GPU's scores, activations and y against the oracle on the GPU's list."""
    from oracle import sfx_oracle as O
    from gpu_helpers import Y_RTOL, rel_err
    cfg = SMALL["C2s"]
    layers = [S.make_layer(cfg, l, device=DEV) for l in range(2)]
    x = [S.make_tokens(cfg, l, 1, 1, device=DEV)[0].clone() for l in range(2)]
    layers[0].W1[5] = (1000.0 * torch.sign(x[0][0].float())).to(layers[0].W1.dtype)
    st = StackStep(layers, cfg.d, cfg.f, cfg.h, 1, cfg.wdtype, cfg.act)
    say("fused step, hidden past the fp16 range in layer 0")
    st.run(st.descriptors(x))
    torch.cuda.synchronize()
    assert st.error_word() == 0
    for l in range(2):
        out = _outputs(st, l)
        lnp = layer_np(layers[l])
        x64 = O.decode(S.storage_numpy(x[l]), cfg.pdtype)
        s64 = O.predict(x64, *O.predictor_weights(lnp, cfg.pdtype))
        if l == 0:
            assert np.max(x64 @ O.decode(lnp["W1"], cfg.pdtype).T) > 65504.0
        err = np.max(np.abs(out["scores"].astype(np.float64) - s64) / np.maximum(1.0, np.abs(s64)))
        say(f"   layer {l}: score rel err {err:.2e}, count {out['count']}")
        assert err <= 1e-5, err
        _, uni, idx, cnt = O.gate(out["scores"].astype(np.float64), layers[l].threshold)
        assert np.array_equal(O.pack_bits(uni), out["union_bits"]) and cnt == out["count"]
        assert np.array_equal(idx, out["idx"])
        gidx = out["idx"]
        hact_ref = O.sparse_up(x64, O.rows(lnp["Wa"], cfg.wdtype, gidx), np.asarray(lnp["ba"], np.float64)[gidx],
                               cfg.act)
        y_ref = O.sparse_down(O.rows(lnp["Wd"], cfg.wdtype, gidx), hact_ref)
        assert rel_err(out["hact"], hact_ref) <= Y_RTOL[cfg.wdtype]
        assert rel_err(out["y"], y_ref) <= Y_RTOL[cfg.wdtype]
