"""sfx_sparse_down_noalloc (the down call that allocates nothing: its workspace is
the library's static device scratch) against sfx_sparse_down with a caller
workspace: the same y bit for bit, within the oracle's bar, on two calls in a row
(the second with a smaller input), and inside a replayed HIP graph."""
import numpy as np
import pytest
import torch

import synthetic as S
from activation_sparse_ffn_amd import _abi as A
from gpu_helpers import Y_RTOL, layer_np, rel_err, say
from oracle import sfx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (workload, tokens, active share) of the first call, then of the smaller second call
CASES = {
    "f16": ((S.scaled(S.CONFIGS["C2"], name="na1", d=4096, f=16384, h=64), 2, 0.08),
            (S.scaled(S.CONFIGS["C2"], name="na2", d=1032, f=3000, h=64), 1, 0.10)),
    "bf16": ((S.scaled(S.CONFIGS["C3"], name="nb1", d=4096, f=11008, h=64), 8, 0.30),
             (S.scaled(S.CONFIGS["C3"], name="nb2", d=1032, f=2080, h=64), 3, 0.20)),
    "q4": ((S.scaled(S.CONFIGS["C4"], name="nq1", d=7168, f=8192, h=64), 1, 0.07),
           (S.scaled(S.CONFIGS["C4"], name="nq2", d=1056, f=2000, h=64), 1, 0.05)),
}


def _inputs(cfg, B, share, seed):
    L = S.make_layer(cfg, 0, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(seed)
    k = max(1, int(share * cfg.f))
    idx = torch.sort(torch.randperm(cfg.f, generator=g)[:k]).values.to(torch.int32)
    hact = torch.rand(cfg.f, B, generator=g, dtype=torch.float32)   # rows past k are never read
    return L, idx.to(DEV), torch.tensor([k], dtype=torch.int32, device=DEV), hact.to(DEV)


def _with_ws(L, idx_full, count, hact, B, d):
    y = torch.full((B, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = A.workspace(A.sfx_sparse_down_ws(A._wdt_of(L.Wd), B, d, idx_full.numel()))
    A.sfx_sparse_down(L.Wd, idx_full, count, hact, y, ws, Wd_scales=L.Wd_s)
    return y


@pytest.mark.parametrize("dt", ["f16", "bf16", "q4"])
def test_down_noalloc_matches_workspace_call(dt):
    for call, (cfg, B, share) in enumerate(CASES[dt]):
        say(f"noalloc {dt} call {call}: d={cfg.d} f={cfg.f} B={B}")
        L, idx, count, hact = _inputs(cfg, B, share, 100 + call)
        # idx holds f entries (kmax = f), the list in its first `count`
        idx_full = torch.zeros(cfg.f, dtype=torch.int32, device=DEV)
        k = int(count.item())
        idx_full[:k] = idx
        y_ws = _with_ws(L, idx_full, count, hact, B, cfg.d)
        y_na = torch.full((B, cfg.d), float("nan"), dtype=torch.float32, device=DEV)
        A.sfx_sparse_down_noalloc(L.Wd, idx_full, count, hact, y_na, Wd_scales=L.Wd_s)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), "noalloc y differs from the workspace call"
        Lnp = layer_np(L)
        gidx = idx.cpu().numpy()
        y_ref = O.sparse_down(O.rows(Lnp["Wd"], cfg.wdtype, gidx, Lnp.get("Wd_s")),
                              hact[:k].cpu().numpy().astype(np.float64))
        r = rel_err(y_na.cpu().numpy(), y_ref)
        say(f"   k={k} y_rel={r:.2e}")
        assert r <= Y_RTOL[cfg.wdtype], r


def test_down_noalloc_graph_replay():
    """Captured in a graph (no allocation inside the capture) and replayed with new
    activations between replays: every replay equals the workspace call."""
    cfg, B, share = CASES["bf16"][0]
    L, idx, count, hact = _inputs(cfg, B, share, 7)
    idx_full = torch.zeros(cfg.f, dtype=torch.int32, device=DEV)
    idx_full[:int(count.item())] = idx
    y = torch.zeros(B, cfg.d, dtype=torch.float32, device=DEV)
    A.sfx_sparse_down_noalloc(L.Wd, idx_full, count, hact, y)      # first call on the device: address lookup
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.sfx_sparse_down_noalloc(L.Wd, idx_full, count, hact, y)
    gen = torch.Generator(device="cpu").manual_seed(3)
    for rep in range(3):
        say(f"noalloc graph replay {rep}")
        hact.copy_(torch.rand(cfg.f, B, generator=gen).to(DEV))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, _with_ws(L, idx_full, count, hact, B, cfg.d)), rep
        _ = torch.randn(1000, device=DEV).sum().item()
