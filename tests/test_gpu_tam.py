"""GPU parity of the TAM update (KAIROX page, Core method, item 4).

The score recurrence is compared with the fp64 oracle (|s_gpu - s64| <= 1e-5).
The integer decisions (top-K list, hot / entered / left bits, count) are compared
bit-exactly with the oracle's selection applied to the GPU's fp32 scores and the
fp32 tau = (1 - lambda) + eps, so both sides decide in the same precision."""
import json
import os

import numpy as np
import pytest
import torch

import synthetic as S
from activation_sparse_ffn_amd import StepBuffers, TamState, run_layer
from gpu_helpers import say
from oracle import sfx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bits_to_bool(words, G):
    w = np.asarray(words).view(np.uint32)
    return np.array([(int(w[g >> 5]) >> (g & 31)) & 1 for g in range(G)], bool)


def _tau32(lam, eps):
    return float(np.float32(np.float32(1.0) - np.float32(lam)) + np.float32(eps))


def _check_layer(st: TamState, l, G, K, prev_hot, score64, tau32):
    s_gpu = st.score[l].cpu().numpy()
    assert np.max(np.abs(s_gpu.astype(np.float64) - score64)) <= 1e-5
    topk, hot, ent, left = O.tam_select(s_gpu.astype(np.float64), prev_hot, tau32, K)
    n = int(st.topk_count[l].item())
    gt = st.topk[l].cpu().numpy()
    assert n == topk.size and np.array_equal(gt[:n], topk)
    assert np.all(gt[n:K] == -1)
    assert np.array_equal(_bits_to_bool(st.hot[l].cpu().numpy(), G), hot)
    assert np.array_equal(_bits_to_bool(st.entered[l].cpu().numpy(), G), ent)
    assert np.array_equal(_bits_to_bool(st.left[l].cpu().numpy(), G), left)
    return hot


def test_tam_hand_fixture():
    with open(os.path.join(GOLD, "tam_tiny.json")) as fh:
        g = json.load(fh)
    st = TamState(1, g["G"], g["K"])
    for i, step in enumerate(g["steps"]):
        say(f"tam fixture step {i}")
        u = torch.tensor([step["union_words"]], dtype=torch.int32, device=DEV)
        st.update(u, g["lambda"], g["eps"])
        torch.cuda.synchronize()
        assert np.array_equal(st.score[0].cpu().numpy().astype(np.float64), np.array(step["score"]))
        n = int(st.topk_count[0].item())
        assert st.topk[0, :n].cpu().tolist() == step["topk"]
        assert np.flatnonzero(_bits_to_bool(st.entered[0].cpu().numpy(), g["G"])).tolist() == step["entered"]
        assert np.flatnonzero(_bits_to_bool(st.left[0].cpu().numpy(), g["G"])).tolist() == step["left"]


def _unpack(words, G):
    """[L][ceil(G/32)] bit words -> bool [L][G] (bit g % 32 of word g / 32)."""
    w = np.asarray(words).view(np.uint32).astype(np.uint64)
    bits = (w[:, :, None] >> np.arange(32, dtype=np.uint64)) & 1
    return bits.reshape(w.shape[0], -1)[:, :G].astype(bool)


@pytest.mark.parametrize("lam", [0.8, 0.9, 0.95])
def test_tam_random_bits_60_layers(lam):
    """The Falcon-40B workload's TAM: 60 layers x 1024 groups, K = 256, 512 steps
    of seeded random group activity with persistence (active groups stay active
    with probability 0.8), every layer of every step against the oracle."""
    L, G, K, eps, steps = 60, 1024, 256, 0.01, 512
    rng = np.random.default_rng(int(lam * 100))
    st = TamState(L, G, K)
    score64 = np.zeros((L, G))
    prev_hot = np.zeros((L, G), bool)
    act = rng.random((L, G)) < 0.2
    tau32 = _tau32(lam, eps)
    worst = 0.0
    for step in range(steps):
        keep = rng.random((L, G)) < 0.8
        act = np.where(act, keep, rng.random((L, G)) < 0.05)
        words = np.where(act, rng.integers(1, 2 ** 32, size=(L, G), dtype=np.uint64), 0).astype(np.uint32)
        u = torch.from_numpy(words.view(np.int32)).to(DEV)
        if step % 64 == 0:
            say(f"tam lambda={lam} step {step}")
        st.update(u, lam, eps)
        torch.cuda.synchronize()
        s_gpu = st.score.cpu().numpy()
        topk_gpu, cnt_gpu = st.topk.cpu().numpy(), st.topk_count.cpu().numpy()
        hot_gpu, ent_gpu, left_gpu = (_unpack(t.cpu().numpy(), G) for t in (st.hot, st.entered, st.left))
        for l in range(L):
            score64[l], _, _, _, _ = O.tam_update(score64[l], prev_hot[l], words[l], lam, eps, K)
            worst = max(worst, float(np.max(np.abs(s_gpu[l].astype(np.float64) - score64[l]))))
            topk, hot, ent, left = O.tam_select(s_gpu[l].astype(np.float64), prev_hot[l], tau32, K)
            n = int(cnt_gpu[l])
            assert n == topk.size and np.array_equal(topk_gpu[l, :n], topk), (step, l)
            assert np.all(topk_gpu[l, n:K] == -1)
            assert np.array_equal(hot_gpu[l], hot) and np.array_equal(ent_gpu[l], ent), (step, l)
            assert np.array_equal(left_gpu[l], left), (step, l)
            prev_hot[l] = hot
    say(f"   max |s_gpu - s64| over {steps} steps: {worst:.2e}")
    assert worst <= 1e-5


def test_tam_on_real_union_bits():
    """TAM fed with the union masks the GPU step produces on a planted-group layer."""
    cfg = S.scaled(S.CONFIGS["C5"], name="C5t", d=1032, f=8192, h=264)
    G, K, lam, eps = cfg.f // 32, 64, 0.9, 0.01
    L = S.make_layer(cfg, 0, device=DEV)
    xs = S.make_tokens(cfg, 0, 24, 8, device=DEV)
    ubits = torch.zeros(1, G, dtype=torch.int32, device=DEV)
    buf = StepBuffers(cfg.d, cfg.f, cfg.h, 8, cfg.wdtype, cfg.pdtype, union_bits=ubits[0])
    st = TamState(1, G, K)
    score64 = np.zeros(G)
    prev = np.zeros(G, bool)
    tau32 = _tau32(lam, eps)
    for step in range(24):
        say(f"tam real bits step {step}")
        run_layer(buf, L.tensors(), xs[step], L.threshold, cfg.act)
        st.update(ubits, lam, eps)
        torch.cuda.synchronize()
        words = ubits[0].cpu().numpy().view(np.uint32)
        score64, _, _, _, _ = O.tam_update(score64, prev, words, lam, eps, K)
        prev = _check_layer(st, 0, G, K, prev, score64, tau32)
    assert int(st.topk_count[0].item()) > 0


def test_tam_resume_is_bitwise():
    """256 steps, copy the state out and back, 256 more == 512 straight."""
    L, G, K, lam, eps = 4, 1024, 256, 0.95, 0.01
    rng = np.random.default_rng(3)
    words = (rng.random((512, L, G)) < 0.3).astype(np.int32)
    wd = torch.from_numpy(words).to(DEV)
    a = TamState(L, G, K)
    for s in range(512):
        a.update(wd[s], lam, eps)
    b = TamState(L, G, K)
    for s in range(256):
        b.update(wd[s], lam, eps)
    torch.cuda.synchronize()
    saved = (b.score.cpu().clone(), b.hot.cpu().clone())
    c = TamState(L, G, K)
    c.score.copy_(saved[0].to(DEV))
    c.hot.copy_(saved[1].to(DEV))
    for s in range(256, 512):
        c.update(wd[s], lam, eps)
    torch.cuda.synchronize()
    say("tam resume")
    assert torch.equal(a.score, c.score) and torch.equal(a.hot, c.hot)
    assert torch.equal(a.topk, c.topk) and torch.equal(a.topk_count, c.topk_count)
