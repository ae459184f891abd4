"""GPU parity of the hot region (KAIROX page, Core method, items 3, 4 and 6) and of
the Top-K reload rule TAM is compared with (Experiments, strategies and ablations).

Decisions and slot tables are integers: compared bit-exactly with the oracle fed the
same entered / left sets.  The region is compared byte for byte with the oracle's
copy of the same source rows."""
import numpy as np
import pytest
import torch

import synthetic as S
from activation_sparse_ffn_amd import HotRegion, StepBuffers, TamState, TopKNowState, run_layer
from activation_sparse_ffn_amd import _abi as A
from gpu_helpers import say
from oracle import sfx_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _unpack(words, G):
    """[L][ceil(G/32)] bit words -> bool [L][G] (bit g % 32 of word g / 32)."""
    w = np.asarray(words).view(np.uint32).astype(np.uint64)
    bits = (w[:, :, None] >> np.arange(32, dtype=np.uint64)) & 1
    return bits.reshape(w.shape[0], -1)[:, :G].astype(bool)


def _activity(rng, act, L, G, p_on=0.05, keep=0.8):
    """Persistent random group activity with random popcounts (1..32 neurons)."""
    stay = rng.random((L, G)) < keep
    act = np.where(act, stay, rng.random((L, G)) < p_on)
    nbits = rng.integers(1, 33, size=(L, G))
    words = np.where(act, (np.left_shift(np.uint64(1), nbits.astype(np.uint64)) - 1).astype(np.uint64), 0)
    words = (words & 0xFFFFFFFF).astype(np.uint32)
    return act, words


def test_topk_now_60_layers():
    """Top-K rule over 128 steps of 60 layers x 1024 groups, K = 256, bit-exact."""
    L, G, K, steps = 60, 1024, 256, 128
    rng = np.random.default_rng(5)
    st = TopKNowState(L, G, K)
    prev = np.zeros((L, G), bool)
    act = rng.random((L, G)) < 0.2
    for step in range(steps):
        act, words = _activity(rng, act, L, G)
        if step % 32 == 0:
            say(f"topk-now step {step}")
        st.update(torch.from_numpy(words.view(np.int32)).to(DEV))
        torch.cuda.synchronize()
        topk_g, cnt_g = st.topk.cpu().numpy(), st.topk_count.cpu().numpy()
        hot_g, ent_g, left_g = (_unpack(t.cpu().numpy(), G) for t in (st.hot, st.entered, st.left))
        for l in range(L):
            topk, hot, ent, left = O.topk_now_update(prev[l], words[l], K)
            n = int(cnt_g[l])
            assert n == topk.size and np.array_equal(topk_g[l, :n], topk), (step, l)
            assert np.all(topk_g[l, n:K] == -1)
            assert np.array_equal(hot_g[l], hot) and np.array_equal(ent_g[l], ent), (step, l)
            assert np.array_equal(left_g[l], left), (step, l)
            prev[l] = hot


def _mats(rng, L, G):
    """Three matrices per layer of different group sizes: fp16 [32G][64] (4 KB per
    group), fp32 [32G] (128 B), uint8 [32G][48] (1.5 KB)."""
    out = []
    for _ in range(L):
        a = torch.from_numpy(rng.standard_normal((32 * G, 64)).astype(np.float16)).to(DEV)
        b = torch.from_numpy(rng.standard_normal(32 * G).astype(np.float32)).to(DEV)
        c = torch.from_numpy(rng.integers(0, 256, (32 * G, 48), dtype=np.uint8)).to(DEV)
        out.append([a, b, c])
    return out


def _check_region(hr: HotRegion, host_regions, slot64, group64, l):
    assert np.array_equal(hr.slot_of[l].cpu().numpy(), slot64[l])
    assert np.array_equal(hr.group_of[l].cpu().numpy(), group64[l])
    for m, ref in enumerate(host_regions[l]):
        got = hr.region[l][m].cpu().numpy()
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), (l, m)


@pytest.mark.parametrize("policy", ["tam", "topk_now"])
def test_hot_region_follows_hot_sets(policy):
    """Slots, copy lists and region bytes over 160 steps of 3 layers with G = 1000
    (ragged last bit word) and K = 200, driven by TAM (lambda = 0.9) or by the
    Top-K rule; every step's slot tables and copy list against hot_assign, the
    region bytes every 16 steps and at the end."""
    L, G, K, steps = 3, 1000, 200, 160
    rng = np.random.default_rng(17 if policy == "tam" else 18)
    mats = _mats(rng, L, G)
    host_src = [[t.cpu().numpy() for t in ms] for ms in mats]
    host_reg = [[np.zeros_like(a[:32 * K]) for a in ms] for ms in host_src]
    hr = HotRegion(mats, G, K)
    st = TamState(L, G, K) if policy == "tam" else TopKNowState(L, G, K)
    slot64 = np.full((L, G), -1)
    group64 = np.full((L, K), -1)
    act = rng.random((L, G)) < 0.2
    total = 0
    for step in range(steps):
        act, words = _activity(rng, act, L, G, p_on=0.08, keep=0.7)
        u = torch.from_numpy(words.view(np.int32)).to(DEV)
        if step % 40 == 0:
            say(f"hot region {policy} step {step}")
        if policy == "tam":
            st.update(u, 0.9, 0.01)
        else:
            st.update(u)
        hr.update(st.entered, st.left)
        torch.cuda.synchronize()
        ent = _unpack(st.entered.cpu().numpy(), G)
        left = _unpack(st.left.cpu().numpy(), G)
        nc = hr.ncopies.cpu().numpy()
        cp = hr.copies.cpu().numpy()
        for l in range(L):
            copies = O.hot_assign(slot64[l], group64[l], ent[l], left[l])
            assert int(nc[l]) == len(copies), (step, l)
            assert [tuple(v) for v in cp[l, :nc[l]].tolist()] == copies, (step, l)
            for m in range(3):
                O.hot_copy(host_reg[l][m], host_src[l][m], copies)
            total += len(copies)
        if step % 16 == 15 or step == steps - 1:
            for l in range(L):
                _check_region(hr, host_reg, slot64, group64, l)
    say(f"   {policy}: {total} group copies over {steps} steps x {L} layers")
    assert total > 0


def test_hot_region_edges():
    """K = G (everything fits: no group ever waits), G = 1 and K = 1, slots only
    (nmat = 0), an all-leave step, and a step that is a no-op."""
    G = 37
    rng = np.random.default_rng(2)
    mats = _mats(rng, 1, G)
    src = [t.cpu().numpy() for t in mats[0]]
    reg = [np.zeros_like(a) for a in src]
    hr = HotRegion(mats, G, G)
    slot64, group64 = np.full(G, -1), np.full(G, -1)
    HW = (G + 31) // 32

    def step(ent_ids, left_ids):
        e = np.zeros(G, bool)
        e[list(ent_ids)] = True
        lf = np.zeros(G, bool)
        lf[list(left_ids)] = True

        def pack(b):
            w = np.zeros(HW, np.uint32)
            for g in np.flatnonzero(b):
                w[g >> 5] |= np.uint32(1 << (g & 31))
            return torch.from_numpy(w.view(np.int32)).to(DEV).view(1, HW)

        hr.update(pack(e), pack(lf))
        torch.cuda.synchronize()
        copies = O.hot_assign(slot64, group64, e, lf)
        for m in range(3):
            O.hot_copy(reg[m], src[m], copies)
        _check_region(hr, [reg], slot64[None], group64[None], 0)

    say("hot region edges: K = G")
    step(range(G), [])                        # every group enters, fills every slot
    step([], [])                              # no-op
    step([], range(0, G, 2))                  # half leave
    step(range(0, G, 2), range(1, G, 2))      # swap halves
    step([], range(G))                        # everything leaves (slot_of of absent groups stays -1)
    assert (hr.group_of.cpu().numpy() == -1).all()

    say("hot region edges: G = K = 1, slots only")
    one = HotRegion([[torch.zeros(32, 8, dtype=torch.float16, device=DEV)]], 1, 1)
    bit = torch.ones(1, 1, dtype=torch.int32, device=DEV)
    zero = torch.zeros(1, 1, dtype=torch.int32, device=DEV)
    A.sfx_hot_update(1, 1, bit, zero, one.slot_of, one.group_of, one.copies, one.ncopies)
    torch.cuda.synchronize()
    assert one.slot_of.item() == 0 and one.group_of.item() == 0 and one.ncopies.item() == 1
    A.sfx_hot_update(1, 1, zero, bit, one.slot_of, one.group_of, one.copies, one.ncopies)
    torch.cuda.synchronize()
    assert one.slot_of.item() == -1 and one.group_of.item() == -1 and one.ncopies.item() == 0


def test_hot_region_falcon40b_shape():
    """The Falcon-40B layer's matrices at full size (d = 8192, f = 32768: 1024
    groups of 512 KB in W_up and in W_down, 128 B of bias), K = 256, two layers,
    16 steps of TAM on the layers' own union masks at batch 8; copied groups
    sampled against the source rows byte for byte, and slot tables against the
    oracle every step."""
    cfg = S.CONFIGS["C5"]
    L, G, K, B = 2, cfg.f // 32, 256, 8
    layers = [S.make_layer(cfg, l, device=DEV) for l in range(L)]
    mats = [[ly.Wa, ly.ba, ly.Wd] for ly in layers]
    hr = HotRegion(mats, G, K)
    ubits = torch.zeros(L, G, dtype=torch.int32, device=DEV)
    bufs = [StepBuffers(cfg.d, cfg.f, cfg.h, B, cfg.wdtype, cfg.pred_storage, union_bits=ubits[l]) for l in range(L)]
    xs = [S.make_tokens(cfg, l, 16, B, device=DEV) for l in range(L)]
    tam = TamState(L, G, K)
    slot64, group64 = np.full((L, G), -1), np.full((L, K), -1)
    rng = np.random.default_rng(4)
    for step in range(16):
        say(f"falcon-40b hot region step {step}")
        for l in range(L):
            run_layer(bufs[l], layers[l].tensors(), xs[l][step], layers[l].threshold, cfg.act)
        tam.update(ubits, 0.9, 0.01)
        hr.update(tam.entered, tam.left)
        torch.cuda.synchronize()
        for b in bufs:
            b.check_status()
        ent = _unpack(tam.entered.cpu().numpy(), G)
        left = _unpack(tam.left.cpu().numpy(), G)
        nc = hr.ncopies.cpu().numpy()
        for l in range(L):
            copies = O.hot_assign(slot64[l], group64[l], ent[l], left[l])
            assert int(nc[l]) == len(copies)
            assert np.array_equal(hr.group_of[l].cpu().numpy(), group64[l])
            for g, s in [copies[i] for i in rng.choice(len(copies), min(3, len(copies)), replace=False)]:
                for m in range(3):
                    a = mats[l][m][32 * g:32 * g + 32]
                    b = hr.region[l][m][32 * s:32 * s + 32]
                    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (step, l, g, s, m)
    assert (hr.group_of.cpu().numpy() >= 0).sum() > 0
