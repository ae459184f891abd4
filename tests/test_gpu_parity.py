"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on seeded
synthetic layers.  Bar: scores within 1e-5 of fp64; masks, union bits, index list
and count bit-exact against the oracle's gate on the GPU's fp32 scores, and
against fp64 scores outside the 1e-4 window; hact and y within 1e-3 relative
(2e-3 for int4) of the oracle on the same index list."""
import numpy as np
import pytest
import torch

import synthetic as S
from activation_sparse_ffn_amd import StepBuffers, run_layer
from activation_sparse_ffn_amd import _abi as A
from gpu_helpers import Y_RTOL, check_step, gpu_layer_step, layer_np, rel_err, say
from oracle import sfx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _tokens(cfg, layer, steps, B):
    return S.make_tokens(cfg, layer, steps, B, device=DEV)


# Small shapes that keep every config's recipe but make each tiling ragged:
# d not a multiple of the column tile, f not a multiple of 32 or of the
# compaction block, h not a multiple of 64 chunks.
SCALED = {
    "C2s": S.scaled(S.CONFIGS["C2"], name="C2s", d=1032, f=3000, h=136),
    "C3s": S.scaled(S.CONFIGS["C3"], name="C3s", d=1032, f=2080, h=136),
    "C4s": S.scaled(S.CONFIGS["C4"], name="C4s", d=1056, f=2000, h=136),
    "C5s": S.scaled(S.CONFIGS["C5"], name="C5s", d=1032, f=4096, h=264),
    # predictor layer 1 on the matrix cores with its d walk in 1 part (256 row
    # tiles of 16) and in 3 parts (69 row tiles)
    "C2h1": S.scaled(S.CONFIGS["C2"], name="C2h1", d=264, f=2080, h=4096),
    "C2h3": S.scaled(S.CONFIGS["C2"], name="C2h3", d=1032, f=2080, h=1104),
}


def test_c1_predictor_mask():
    cfg = S.CONFIGS["C1"]
    L = S.make_layer(cfg, 0, device=DEV)
    Lnp = layer_np(L)
    xs = _tokens(cfg, 0, cfg.steps, 1)
    buf = StepBuffers(cfg.d, cfg.f, cfg.h, 1, cfg.wdtype, cfg.pdtype)
    for step in range(cfg.steps):
        say(f"C1 predictor mask step {step}")
        out, _ = gpu_layer_step(cfg, L, xs[step], buf=buf)
        r = check_step(cfg, Lnp, S.storage_numpy(xs[step]), out, L.threshold)
        assert r["y_rel"] <= 1e-5            # fp32 rows: well inside the bar


def test_c1_true_relu_mask():
    """The exact-ReLU index list (from the fp64 oracle) fed to up/down gives the
    dense layer."""
    cfg = S.CONFIGS["C1"]
    L = S.make_layer(cfg, 0, device=DEV)
    Lnp = layer_np(L)
    xs = _tokens(cfg, 0, cfg.steps, 1)
    buf = StepBuffers(cfg.d, cfg.f, cfg.h, 1, cfg.wdtype, cfg.pdtype)
    Wa = O.decode(Lnp["Wa"], "f32")
    Wd = O.decode(Lnp["Wd"], "f32")
    ba = Lnp["ba"].astype(np.float64)
    for step in range(cfg.steps):
        say(f"C1 true-ReLU mask step {step}")
        x = xs[step]
        x64 = O.decode(S.storage_numpy(x), "f32")
        idx = O.true_relu_idx(x64, Wa, ba)
        buf.idx.zero_()
        buf.idx[: idx.size] = torch.from_numpy(idx).to(DEV)
        buf.count.fill_(int(idx.size))
        A.sfx_sparse_up(x, L.Wa, L.ba, buf.idx, buf.count, buf.hact, act="relu")
        A.sfx_sparse_down(L.Wd, buf.idx, buf.count, buf.hact, buf.y, buf.ws_down)
        torch.cuda.synchronize()
        y_dense = O.dense_ffn(x64, Wa, ba, Wd, "relu")
        assert rel_err(buf.y.cpu().numpy(), y_dense) <= 1e-5


@pytest.mark.parametrize("name,B", [("C2s", 1), ("C3s", 1), ("C3s", 3), ("C3s", 4), ("C3s", 8), ("C4s", 1),
                                    ("C4s", 2), ("C2s", 2), ("C2s", 4), ("C5s", 1), ("C5s", 8), ("C5s", 16), ("C5s", 32)])
def test_scaled_configs(name, B):
    cfg = SCALED[name]
    for layer in range(2):
        L = S.make_layer(cfg, layer, device=DEV)
        Lnp = layer_np(L)
        xs = _tokens(cfg, layer, 3, B)
        buf = StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pdtype)
        for step in range(3):
            say(f"{name} B={B} layer {layer} step {step}")
            out, _ = gpu_layer_step(cfg, L, xs[step], buf=buf)
            r = check_step(cfg, Lnp, S.storage_numpy(xs[step]), out, L.threshold)
            say("   ", {k: (round(v, 8) if isinstance(v, float) else v) for k, v in r.items()})


@pytest.mark.parametrize("name,B", [("C2", 1), ("C2", 2), ("C3", 1), ("C3", 4), ("C3", 8), ("C4", 1), ("C4", 2),
                                    ("C5", 1), ("C5", 8), ("C5", 32)])
def test_full_size_layer(name, B):
    """One layer at the workload's full shape, in the launch configuration the
    benchmark times, two decode steps, every output compared."""
    cfg = S.CONFIGS[name]
    L = S.make_layer(cfg, 0, device=DEV)
    Lnp = layer_np(L)
    xs = _tokens(cfg, 0, 2, B)
    buf = StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pdtype)
    for step in range(2):
        say(f"{name} full size B={B} step {step}")
        out, _ = gpu_layer_step(cfg, L, xs[step], buf=buf)
        r = check_step(cfg, Lnp, S.storage_numpy(xs[step]), out, L.threshold)
        say("   ", {k: (round(v, 8) if isinstance(v, float) else v) for k, v in r.items()})
    del L, Lnp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,B", [("C3s", 16), ("C3s", 32), ("C2s", 17), ("C2s", 64), ("C3s", 64),
                                    ("C2h1", 8), ("C2h3", 8), ("C2h3", 33)])
def test_matrix_core_predictor(name, B):
    """B >= 16 runs both predictor layers on the matrix cores (hidden split into
    exact 16-bit pieces): scores must still sit within 1e-5 of fp64."""
    cfg = SCALED[name]
    L = S.make_layer(cfg, 0, device=DEV)
    Lnp = layer_np(L)
    xs = _tokens(cfg, 0, 2, B)
    buf = StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pdtype)
    for step in range(2):
        say(f"matrix-core predictor {name} B={B} step {step}")
        out, _ = gpu_layer_step(cfg, L, xs[step], buf=buf)
        r = check_step(cfg, Lnp, S.storage_numpy(xs[step]), out, L.threshold)
        say("   ", {k: (round(v, 9) if isinstance(v, float) else v) for k, v in r.items()})


def test_threshold_extremes():
    """+inf: nothing active, y = 0.  -inf: every neuron active, y = the dense layer."""
    cfg = SCALED["C2s"]
    L = S.make_layer(cfg, 0, device=DEV)
    Lnp = layer_np(L)
    x = _tokens(cfg, 0, 1, 2)[0]
    buf = StepBuffers(cfg.d, cfg.f, cfg.h, 2, cfg.wdtype, cfg.pdtype)
    buf.hact.fill_(7.0)
    say("threshold +inf")
    out, _ = gpu_layer_step(cfg, L, x, threshold=float("inf"), buf=buf)
    assert out["count"] == 0 and not out["union_bits"].any() and not out["y"].any()
    assert torch.all(buf.hact == 7.0)             # nothing written
    say("threshold -inf")
    out, _ = gpu_layer_step(cfg, L, x, threshold=float("-inf"), buf=buf)
    assert out["count"] == cfg.f and np.array_equal(out["idx"], np.arange(cfg.f))
    x64 = O.decode(S.storage_numpy(x), "f16")
    y_dense = O.dense_ffn(x64, O.decode(Lnp["Wa"], "f16"), Lnp["ba"].astype(np.float64),
                          O.decode(Lnp["Wd"], "f16"), "relu")
    assert rel_err(out["y"], y_dense) <= Y_RTOL["f16"]


def test_compact_crafted_scores():
    """NaN, +-inf and scores exactly at the threshold, B = 3, ragged f."""
    f, B, t = 1000, 3, 0.5
    g = torch.Generator().manual_seed(11)
    s = torch.randn(B, f, generator=g)
    s[0, 3] = t
    s[1, 4] = float("nan")
    s[2, 5] = float("inf")
    s[0, 6] = float("-inf")
    s[1, 999] = t
    s = s.to(DEV)
    W = (f + 31) // 32
    tok = torch.zeros(B, W, dtype=torch.int32, device=DEV)
    uni = torch.zeros(W, dtype=torch.int32, device=DEV)
    idx = torch.full((f,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = A.workspace(A.sfx_compact_ws(B, f))
    for rep in range(2):                                  # the ticket resets itself
        say(f"compact crafted rep {rep}")
        A.sfx_compact(s, t, uni, idx, cnt, ws, tok_bits=tok)
        torch.cuda.synchronize()
        mtok, muni, midx, mcnt = O.gate(s.cpu().double().numpy(), t)
        assert np.array_equal(tok.cpu().numpy().view(np.uint32), O.pack_bits(mtok))
        assert np.array_equal(uni.cpu().numpy().view(np.uint32), O.pack_bits(muni))
        k = int(cnt.item())
        assert k == mcnt and np.array_equal(idx[:k].cpu().numpy(), midx)
        assert torch.all(idx[k:] == -7)
        assert mtok[0, 3] and not mtok[1, 4] and mtok[2, 5] and not mtok[0, 6]


@pytest.mark.parametrize("f,B,t", [(40001, 33, 2.0),       # ~54% union: three list windows, two token batches
                                   (70000, 1, 10.0),       # empty list
                                   (70000, 2, -1e30)])     # every neuron: nine windows, three words per thread
def test_compact_long_lists(f, B, t):
    """Lists longer than one LDS window, the empty list and the full list."""
    g = torch.Generator().manual_seed(f + B)
    s = torch.randn(B, f, generator=g).to(DEV)
    W = (f + 31) // 32
    tok = torch.zeros(B, W, dtype=torch.int32, device=DEV)
    uni = torch.zeros(W, dtype=torch.int32, device=DEV)
    idx = torch.full((f,), -7, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = A.workspace(A.sfx_compact_ws(B, f))
    mtok, muni, midx, mcnt = O.gate(s.cpu().double().numpy(), t)
    for rep in range(2):                       # the second call continues from the first's counter
        say(f"compact long f={f} B={B} t={t} rep {rep}")
        A.sfx_compact(s, t, uni, idx, cnt, ws, tok_bits=tok)
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy().view(np.uint32), O.pack_bits(mtok))
        assert np.array_equal(uni.cpu().numpy().view(np.uint32), O.pack_bits(muni))
        k = int(cnt.item())
        assert k == mcnt and np.array_equal(idx[:k].cpu().numpy(), midx)
        assert torch.all(idx[k:] == -7)
        # workspace after the call: error word clear, call counter advanced by one,
        # every workgroup's count word tagged with this call's counter
        wsw = ws.view(torch.int32).cpu().numpy().view(np.uint32)
        assert wsw[1] == 0 and wsw[0] == rep + 1
        nblk = (f + 1023) // 1024
        assert np.all((wsw[64:64 + nblk] >> 16) == rep + 1)


def test_out_of_range_indices_are_inert():
    cfg = SCALED["C2s"]
    L = S.make_layer(cfg, 0, device=DEV)
    Lnp = layer_np(L)
    x = _tokens(cfg, 0, 1, 1)[0]
    good = np.array([3, 17, 900, 2999], np.int32)
    lst = np.array([3, -1, 17, cfg.f + 5, 900, 2999], np.int32)
    kmax = 16
    idx = torch.zeros(kmax, dtype=torch.int32, device=DEV)
    idx[: lst.size] = torch.from_numpy(lst).to(DEV)
    cnt = torch.tensor([lst.size], dtype=torch.int32, device=DEV)
    hact = torch.full((kmax, 1), 5.0, device=DEV)
    y = torch.empty(1, cfg.d, device=DEV)
    ws = A.workspace(A.sfx_sparse_down_ws(A.SFX_F16, 1, cfg.d, kmax))
    say("out-of-range indices")
    A.sfx_sparse_up(x, L.Wa, L.ba, idx, cnt, hact)
    A.sfx_sparse_down(L.Wd, idx, cnt, hact, y, ws)
    torch.cuda.synchronize()
    h = hact[: lst.size, 0].cpu().numpy()
    assert h[1] == 0.0 and h[3] == 0.0
    x64 = O.decode(S.storage_numpy(x), "f16")
    href = O.sparse_up(x64, O.rows(Lnp["Wa"], "f16", good), Lnp["ba"][good].astype(np.float64), "relu")
    assert rel_err(h[[0, 2, 4, 5]], href[:, 0]) <= 1e-3
    yref = O.sparse_down(O.rows(Lnp["Wd"], "f16", good), href)
    assert rel_err(y.cpu().numpy(), yref) <= 1e-3


def test_max_batch_64():
    cfg = S.scaled(S.CONFIGS["C2"], name="C2b", d=520, f=640, h=72)
    L = S.make_layer(cfg, 0, device=DEV)
    x = _tokens(cfg, 0, 1, 64)[0]
    say("B=64")
    out, _ = gpu_layer_step(cfg, L, x)
    check_step(cfg, layer_np(L), S.storage_numpy(x), out, L.threshold)


def test_bitwise_determinism():
    cfg = SCALED["C3s"]
    L = S.make_layer(cfg, 0, device=DEV)
    x = _tokens(cfg, 0, 1, 4)[0]
    say("determinism")
    a, buf = gpu_layer_step(cfg, L, x)
    b, _ = gpu_layer_step(cfg, L, x, buf=buf)
    c, _ = gpu_layer_step(cfg, L, x)
    for k in ("scores", "union_bits", "idx", "hact", "y"):
        assert np.array_equal(a[k], b[k]) and np.array_equal(a[k], c[k]), k


@pytest.mark.parametrize("B", [2, 8])        # vector kernels; matrix cores (split layer 1, tickets)
def test_graph_replay_matches_eager(B):
    """The layer-step captured in a HIP graph: every replay (new tokens copied into
    the static input between replays, eager work in between) equals eager."""
    cfg = SCALED["C5s"]
    L = S.make_layer(cfg, 0, device=DEV)
    xs = _tokens(cfg, 0, 4, B)
    buf = StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pdtype)
    x_static = xs[0].clone()
    eager = []
    for s in range(4):
        out, _ = gpu_layer_step(cfg, L, xs[s], buf=buf)
        eager.append(out)
    say("graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_layer(buf, L.tensors(), x_static, L.threshold, cfg.act)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_layer(buf, L.tensors(), x_static, L.threshold, cfg.act)
    for s in range(4):
        say(f"graph replay B={B} {s}")
        x_static.copy_(xs[s])
        graph.replay()
        torch.cuda.synchronize()
        k = int(buf.count.item())
        assert k == eager[s]["count"]
        assert np.array_equal(buf.idx[:k].cpu().numpy(), eager[s]["idx"])
        assert np.array_equal(buf.y.cpu().numpy(), eager[s]["y"])
        _ = torch.randn(1000, device=DEV).sum().item()      # eager work between replays


@pytest.mark.parametrize("B", [3, 1])
def test_predict_fp16_range_flag(B):
    """fp16 predictor with one hidden value far past 65504: from 3 tokens (matrix
    cores, fp16 hi + lo pieces) the sticky range flag is set; at one token (vector
    path, fp32 hidden) there is no limit, the flag stays clear and the scores match
    fp64.  A normal input leaves the flag clear on both paths."""
    d, h, f = 512, 64, 1024
    g = torch.Generator(device="cpu").manual_seed(7)
    x = torch.randn(B, d, generator=g, dtype=torch.float64)
    W1 = torch.randn(h, d, generator=g, dtype=torch.float64) / d ** 0.5
    W2 = torch.randn(f, h, generator=g, dtype=torch.float64) / h ** 0.5
    x16, W216 = x.to(torch.float16), W2.to(torch.float16)
    scores = torch.empty(B, f, dtype=torch.float32, device=DEV)
    ws = A.workspace(A.sfx_predict_ws(A.SFX_F16, B, d, h, f))
    for big in (False, True):
        W1b = W1.clone()
        if big:
            # hidden row 5 of token 0 = 1000 * sum|x_0| ~ 4e5
            W1b[5] = 1000.0 * torch.sign(x16[0].to(torch.float64))
        W116 = W1b.to(torch.float16)
        ws.zero_()
        say(f"fp16 range flag B={B} big={big}")
        A.sfx_predict(x16.to(DEV), W116.to(DEV), W216.to(DEV), scores, ws)
        torch.cuda.synchronize()
        flag = int(ws[:4].view(torch.int32).item())
        if big and B >= 3:
            assert flag != 0
            continue
        assert flag == 0
        s64 = O.predict(x16.numpy().astype(np.float64), W116.numpy().astype(np.float64),
                        W216.numpy().astype(np.float64))
        err = np.max(np.abs(scores.cpu().numpy().astype(np.float64) - s64) / np.maximum(1.0, np.abs(s64)))
        assert err <= 1e-5, err


# squared ReLU (activation functions of the PowerInfer page's code notes) on the
# vector kernels (1 token, int4 rows) and the matrix cores (3 tokens)
RELU2 = {
    "C2r": S.scaled(S.CONFIGS["C2"], name="C2r", act="relu2", d=1032, f=3000, h=136),
    "C4r": S.scaled(S.CONFIGS["C4"], name="C4r", act="relu2", d=1056, f=2000, h=136),
}


@pytest.mark.parametrize("name,B", [("C2r", 1), ("C2r", 3), ("C2r", 8), ("C4r", 1)])
def test_squared_relu(name, B):
    cfg = RELU2[name]
    L = S.make_layer(cfg, 0, device=DEV)
    Lnp = layer_np(L)
    xs = _tokens(cfg, 0, 2, B)
    for step in range(2):
        say(f"squared relu {name} B={B} step {step}")
        out, _ = gpu_layer_step(cfg, L, xs[step])
        r = check_step(cfg, Lnp, S.storage_numpy(xs[step]), out, L.threshold)
        assert np.all(out["hact"] >= 0)


# int4 g32 predictor (W1, W2 as codes + fp16 scales) on the OPT-30B recipe
PQ4 = {
    "C4q": S.scaled(S.CONFIGS["C4"], name="C4q", pred_q4=True, d=1056, f=2000, h=160),
    "C2q": S.scaled(S.CONFIGS["C2"], name="C2q", pred_q4=True, d=1024, f=3008, h=128),
}


@pytest.mark.parametrize("name,B", [("C4q", 1), ("C4q", 2), ("C4q", 8), ("C2q", 1), ("C2q", 5)])
def test_int4_predictor(name, B):
    cfg = PQ4[name]
    L = S.make_layer(cfg, 0, device=DEV)
    assert L.W1.dtype == torch.uint8 and L.W1_s is not None
    Lnp = layer_np(L)
    xs = _tokens(cfg, 0, 2, B)
    for step in range(2):
        say(f"int4 predictor {name} B={B} step {step}")
        out, _ = gpu_layer_step(cfg, L, xs[step])
        check_step(cfg, Lnp, S.storage_numpy(xs[step]), out, L.threshold)


def test_int4_predictor_full_size():
    """OPT-30B shape, int4 rows and int4 predictor (30 MB instead of 110 MB of
    predictor per layer-step), batch 1."""
    cfg = S.scaled(S.CONFIGS["C4"], name="C4", pred_q4=True)
    L = S.make_layer(cfg, 0, device=DEV)
    Lnp = layer_np(L)
    xs = _tokens(cfg, 0, 2, 1)
    for step in range(2):
        say(f"int4 predictor full size step {step}")
        out, _ = gpu_layer_step(cfg, L, xs[step])
        r = check_step(cfg, Lnp, S.storage_numpy(xs[step]), out, L.threshold)
        say("   ", r)
    torch.cuda.empty_cache()
