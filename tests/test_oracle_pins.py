"""Pins of the fp64 oracle against values fixed outside it: hand-computed fixtures
(tests/golden), closed forms, special cases and brute force on tiny inputs.

Each test names the oracle function it pins and the kind of mistake it would catch.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import sfx_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as fh:
        return json.load(fh)


# ----------------------------------------------------------------------------- hand fixtures

def test_predict_gate_hand_fixture():
    """predict + gate on the hand-worked example (a dropped ReLU, a transposed
    operand, '>' instead of '>=' or a wrong bit order all change the result)."""
    g = _load("predictor_ffn_tiny.json")
    x = np.array(g["x"], float)
    W1, W2 = np.array(g["W1"], float), np.array(g["W2"], float)
    s = O.predict(x, W1, W2)
    assert np.array_equal(s, np.array(g["scores"], float))
    tok, union, idx, count = O.gate(s, g["threshold"])
    assert np.array_equal(tok, np.array(g["tok_active"]))
    assert np.array_equal(O.pack_bits(tok), np.array(g["tok_bits"], np.uint32)[:, None])
    assert idx.tolist() == g["batch"]["idx"] and count == g["batch"]["count"]
    assert O.pack_bits(union).tolist() == g["batch"]["union_bits"]
    tok1, union1, idx1, count1 = O.gate(s[:1], g["threshold"])
    assert idx1.tolist() == g["single_token"]["idx"] and count1 == 3
    assert O.pack_bits(union1).tolist() == g["single_token"]["union_bits"]


@pytest.mark.parametrize("act", ["relu", "reglu"])
@pytest.mark.parametrize("case", ["single_token", "batch"])
def test_sparse_ffn_hand_fixture(act, case):
    """sparse_up + sparse_down on the hand-worked example, including the union rule
    (a per-token re-mask would give different y for token 0) and the bias."""
    g = _load("predictor_ffn_tiny.json")
    x = np.array(g["x"], float)[: (1 if case == "single_token" else 2)]
    c = g[case]
    idx = np.array(c["idx"])
    Wa, Wl, Wd = (np.array(g[k], float) for k in ("Wa", "Wl", "Wd"))
    ba = np.array(g["ba"], float)
    hact = O.sparse_up(x, Wa[idx], ba[idx], act, Wl[idx] if act == "reglu" else None)
    assert np.array_equal(hact, np.array(c[f"hact_{act}"], float))
    y = O.sparse_down(Wd[idx], hact)
    assert np.array_equal(y, np.array(c[f"y_{act}"], float))


def test_ffn_step_hand_fixture_end_to_end():
    g = _load("predictor_ffn_tiny.json")
    layer = {k: np.array(g[k], np.float32) for k in ("W1", "W2", "Wa", "Wd", "Wl")}
    layer["ba"] = np.array(g["ba"], np.float32)
    out = O.ffn_step(np.array(g["x"], np.float32), layer, "f32", "f32", "relu", g["threshold"])
    assert np.array_equal(out["y"], np.array(g["batch"]["y_relu"], float))
    assert np.array_equal(out["y"], np.array(g["y_dense_relu"], float))


def test_tam_hand_fixture():
    """tam_update over five hand-worked steps: EMA form, strict '>' tau, top-K order,
    entered / left as set differences."""
    g = _load("tam_tiny.json")
    G = g["G"]
    score = np.zeros(G)
    hot = np.zeros(G, bool)
    for st in g["steps"]:
        score, topk, hot_new, ent, left = O.tam_update(score, hot, np.array(st["union_words"], np.uint32),
                                                       g["lambda"], g["eps"], g["K"])
        assert np.array_equal(score, np.array(st["score"], float))
        assert topk.tolist() == st["topk"]
        assert np.flatnonzero(ent).tolist() == st["entered"]
        assert np.flatnonzero(left).tolist() == st["left"]
        hot = hot_new
    t = g["tie"]
    score = np.zeros(t["G"])
    hot = np.zeros(t["G"], bool)
    for st in t["steps"]:
        score, topk, hot, _, _ = O.tam_update(score, hot, np.array(st["union_words"], np.uint32),
                                              g["lambda"], g["eps"], t["K"])
        assert np.array_equal(score, np.array(st["score"], float))
        assert topk.tolist() == st["topk"]


def test_storage_codes():
    """decode (bf16 bit patterns), dequant_q4 (nibble order and sign) and pack_bits."""
    g = _load("storage_codes.json")
    bits = np.array([b for b, _ in g["bf16"]], np.uint16)
    want = np.array([float(v) for _, v in g["bf16"]])
    assert np.array_equal(O.decode(bits, "bf16"), want)
    for byte, lo, hi in g["q4_bytes"]:
        q = np.full((1, 16), byte, np.uint8)
        w = O.dequant_q4(q, np.array([[1.0]], np.float16))
        assert w[0, 0] == lo and w[0, 1] == hi and w[0, 30] == lo and w[0, 31] == hi
    mask = np.zeros(g["bits"]["f"], bool)
    mask[g["bits"]["set"]] = True
    assert O.pack_bits(mask).tolist() == g["bits"]["words"]


def test_q4_scale_broadcast_exactly_32_columns():
    q = np.zeros((1, 32), np.uint8)
    q[0, :] = 0x11                                  # every nibble = +1
    s = np.array([[0.5, -2.0]], np.float16)
    w = O.dequant_q4(q, s)
    assert w.shape == (1, 64)
    assert np.all(w[0, :32] == 0.5) and np.all(w[0, 32:] == -2.0)


# ----------------------------------------------------------------------------- closed forms

def test_predict_identity_special_case():
    """h = d = f and W1 = W2 = I give scores = relu(x)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 7))
    I = np.eye(7)
    assert np.array_equal(O.predict(x, I, I), np.maximum(x, 0.0))


def test_predict_brute_force():
    """predict against explicit per-element loops on a tiny non-square input."""
    rng = np.random.default_rng(2)
    d, h, f, B = 5, 3, 6, 2
    x, W1, W2 = rng.standard_normal((B, d)), rng.standard_normal((h, d)), rng.standard_normal((f, h))
    want = np.zeros((B, f))
    for b in range(B):
        hid = [max(0.0, sum(W1[j][c] * x[b][c] for c in range(d))) for j in range(h)]
        for i in range(f):
            want[b][i] = sum(W2[i][j] * hid[j] for j in range(h))
    assert np.allclose(O.predict(x, W1, W2), want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("B", [1, 3, 4])
def test_gate_brute_force(B):
    """gate against a per-neuron loop: membership, OR-union, ascending idx, bits."""
    rng = np.random.default_rng(10 + B)
    f = 61
    s = rng.standard_normal((B, f))
    s[0, 5] = 0.25                                    # exactly at the threshold: active
    s[B - 1, 7] = np.nan                              # NaN: inactive
    t = 0.25
    tok, union, idx, count = O.gate(s, t)
    want = []
    for i in range(f):
        if any((not math.isnan(s[b][i])) and s[b][i] >= t for b in range(B)):
            want.append(i)
    assert idx.tolist() == want and count == len(want)
    assert tok[0, 5] and not tok[B - 1, 7]
    words = O.pack_bits(union)
    assert sum(bin(int(w)).count("1") for w in words) == count
    for i in range(f):
        assert bool((int(words[i // 32]) >> (i % 32)) & 1) == (i in want)


def _rand_layer(rng, d, f, act):
    Wa = rng.standard_normal((f, d))
    ba = rng.standard_normal(f)
    Wd = rng.standard_normal((f, d))
    Wl = rng.standard_normal((f, d)) if act == "reglu" else None
    return Wa, ba, Wd, Wl


@pytest.mark.parametrize("act", ["relu", "reglu", "relu2"])
def test_all_ones_mask_equals_dense(act):
    """Every neuron active -> sparse up/down equals the dense FFN (np.matmul on the
    whole matrices), rel <= 1e-12."""
    rng = np.random.default_rng(3)
    d, f, B = 24, 40, 3
    Wa, ba, Wd, Wl = _rand_layer(rng, d, f, act)
    x = rng.standard_normal((B, d))
    idx = np.arange(f)
    y = O.sparse_down(Wd[idx], O.sparse_up(x, Wa[idx], ba[idx], act, None if Wl is None else Wl[idx]))
    ref = O.dense_ffn(x, Wa, ba, Wd, act, Wl)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    # through the gate: a threshold of -inf selects every neuron
    _, _, idx2, count = O.gate(rng.standard_normal((B, f)), -np.inf)
    assert count == f and np.array_equal(idx2, idx)


def test_true_relu_mask_equals_dense():
    """The exact ReLU mask gives the dense FFN (inactive neurons contribute zero)."""
    rng = np.random.default_rng(4)
    d, f, B = 32, 80, 2
    Wa, ba, Wd, _ = _rand_layer(rng, d, f, "relu")
    x = rng.standard_normal((B, d))
    idx = O.true_relu_idx(x, Wa, ba)
    assert 0 < idx.size < f
    y = O.sparse_down(Wd[idx], O.sparse_up(x, Wa[idx], ba[idx], "relu"))
    ref = O.dense_ffn(x, Wa, ba, Wd, "relu")
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    # and a strict subset of that mask does not
    y2 = O.sparse_down(Wd[idx[1:]], O.sparse_up(x, Wa[idx[1:]], ba[idx[1:]], "relu"))
    assert np.max(np.abs(y2 - ref)) > 1e-6


def test_permutation_invariance():
    """Reordering neurons (rows of W2, Wa, Wd, ba) permutes the scores and leaves y."""
    rng = np.random.default_rng(5)
    d, h, f = 16, 8, 48
    layer = {"W1": rng.standard_normal((h, d)), "W2": rng.standard_normal((f, h)),
             "Wa": rng.standard_normal((f, d)), "ba": rng.standard_normal(f),
             "Wd": rng.standard_normal((f, d))}
    x = rng.standard_normal((2, d))
    p = rng.permutation(f)
    lp = dict(layer)
    for k in ("W2", "Wa", "ba", "Wd"):
        lp[k] = layer[k][p]
    a = O.ffn_step(x, layer, "f32", "f32", "relu", 0.3)
    b = O.ffn_step(x, lp, "f32", "f32", "relu", 0.3)
    assert np.allclose(b["scores"], a["scores"][:, p], rtol=0, atol=1e-12)
    assert np.allclose(a["y"], b["y"], rtol=1e-12, atol=1e-12)


def test_down_linearity_power_of_two():
    rng = np.random.default_rng(6)
    Wd = rng.standard_normal((9, 11))
    hact = rng.standard_normal((9, 2))
    assert np.array_equal(O.sparse_down(2.0 * Wd, hact), 2.0 * O.sparse_down(Wd, hact))


def test_empty_active_set():
    y = O.sparse_down(np.zeros((0, 5)), np.zeros((0, 3)))
    assert y.shape == (3, 5) and not y.any()


# ----------------------------------------------------------------------------- TAM closed forms

@pytest.mark.parametrize("lam", [0.8, 0.9, 0.95])
def test_tam_closed_forms(lam):
    """n hits from 0 give 1 - lam^n; m misses then give (1 - lam^n) lam^m; an isolated
    hit (1 - lam) is never a candidate; two consecutive hits are a candidate iff
    lam (1 - lam) > eps; always active converges to 1."""
    eps, K = 0.01, 4
    tau = O.tam_tau(lam, eps)
    s = np.zeros(1)
    hot = np.zeros(1, bool)
    for n in range(1, 9):
        s, topk, hot, _, _ = O.tam_update(s, hot, np.array([1], np.uint32), lam, eps, K)
        assert abs(s[0] - (1 - lam ** n)) < 1e-15
        if n == 1:
            assert topk.size == 0                     # isolated hit: 1 - lam < tau
        if n == 2:
            assert (topk.size == 1) == (lam * (1 - lam) > eps) and topk.size == 1
    base = s[0]
    for m in range(1, 6):
        s, _, hot, _, _ = O.tam_update(s, hot, np.array([0], np.uint32), lam, eps, K)
        assert abs(s[0] - base * lam ** m) < 1e-15
    s = np.zeros(1)
    for _ in range(2000):
        s, _, _, _, _ = O.tam_update(s, hot, np.array([7], np.uint32), lam, eps, K)
    assert abs(s[0] - 1.0) < 1e-12
    assert 1 - lam < tau


def test_tam_select_brute_force():
    """Every chosen group beats every unchosen candidate under (score desc, id asc);
    entered / left are the set differences."""
    rng = np.random.default_rng(7)
    G, K = 50, 7
    score = np.round(rng.random(G) * 8) / 8           # many exact ties
    prev = rng.random(G) < 0.2
    tau = 0.3
    topk, hot, ent, left = O.tam_select(score, prev, tau, K)
    cand = [g for g in range(G) if score[g] > tau]
    assert len(topk) == min(K, len(cand))
    chosen = set(topk.tolist())
    for a in chosen:
        for b in cand:
            if b not in chosen:
                assert (score[a] > score[b]) or (score[a] == score[b] and a < b)
    for i in range(len(topk) - 1):
        a, b = topk[i], topk[i + 1]
        assert (score[a] > score[b]) or (score[a] == score[b] and a < b)
    assert set(np.flatnonzero(ent)) == chosen - set(np.flatnonzero(prev))
    assert set(np.flatnonzero(left)) == set(np.flatnonzero(prev)) - chosen


# ----------------------------------------------------------------------------- Live Pipeline

def test_live_step_roles_of_the_two_inputs():
    """ffn_step with a separate predictor input: the mask comes from xp, the
    activations from x.  Identity predictor (h = d = f, W1 = W2 = I) so the scores
    are relu(xp); identity up rows with zero bias so hact = relu(x); Wd rows are
    powers of two so y is exact.  Worked by hand: xp = (1, -1, 2, 0.5), t = 0.75
    -> active {0, 2}; x = (3, 4, -5, 6) -> hact = (3, 0); y = 3 Wd[0] + 0 Wd[2].
    Swapping the roles of x and xp, or scoring x, changes idx and y."""
    I = np.eye(4)
    Wd = np.array([[1, 2, 0, 0], [0, 0, 4, 0], [8, 0, 0, 16], [0, 32, 0, 0]], float)
    layer = {"W1": I, "W2": I, "Wa": I, "ba": np.zeros(4), "Wd": Wd}
    xp = np.array([[1.0, -1.0, 2.0, 0.5]])
    x = np.array([[3.0, 4.0, -5.0, 6.0]])
    r = O.ffn_step(x, layer, "f32", "f32", "relu", 0.75, xp=xp)
    assert r["idx"].tolist() == [0, 2] and r["count"] == 2
    assert r["hact"][:, 0].tolist() == [3.0, 0.0]
    assert r["y"][0].tolist() == [3.0, 6.0, 0.0, 0.0]
    r_same = O.ffn_step(x, layer, "f32", "f32", "relu", 0.75)        # scores of x itself
    assert r_same["idx"].tolist() == [0, 1, 3]
    assert r_same["y"][0].tolist() == [3.0, 6.0 + 192.0, 16.0, 0.0]


def test_mask_recall():
    exact = np.array([1, 1, 0, 1, 0], bool)
    assert O.mask_recall(np.array([1, 0, 1, 1, 0], bool), exact) == 2 / 3
    assert O.mask_recall(exact, exact) == 1.0
    assert O.mask_recall(np.zeros(5, bool), np.zeros(5, bool)) == 1.0


# ----------------------------------------------------------------------------- squared ReLU, int4 predictor

def test_squared_relu_hand_values():
    """sparse_up with 'relu2': z = (2, -1, 0.5) for one token -> (4, 0, 0.25); a
    missing square, a square before the ReLU ((-1)^2 = 1) or a dropped bias fail."""
    x = np.array([[1.0, 2.0]])
    Wa = np.array([[1.0, 0.0], [0.0, -1.0], [0.5, 0.0]])
    ba = np.array([1.0, 1.0, 0.0])
    h = O.sparse_up(x, Wa, ba, "relu2")
    assert h[:, 0].tolist() == [4.0, 0.0, 0.25]


def test_predictor_weights_int4():
    """An int4 predictor is used dequantised: codes 0x8F (-1, -8) and 0x70 (0, 7)
    with scale 0.5 per 32 columns; the scores of a one-hot input pick the column."""
    d, h, f = 32, 32, 32
    W1q = np.zeros((h, d // 2), np.uint8)
    W1q[0, 0] = 0x8F                       # W1[0][0] = -1 * 0.5, W1[0][1] = -8 * 0.5
    W1q[1, 1] = 0x70                       # W1[1][2] = 0, W1[1][3] = 7 * 0.5
    W1s = np.full((h, d // 32), 0.5, np.float16)
    W2q = np.zeros((f, h // 2), np.uint8)
    W2q[5, 0] = 0x10                       # W2[5][1] = 1 * 2
    W2s = np.full((f, h // 32), 2.0, np.float16)
    layer = {"W1": W1q, "W1_s": W1s, "W2": W2q, "W2_s": W2s}
    W1, W2 = O.predictor_weights(layer, "f16")
    assert W1[0, 0] == -0.5 and W1[0, 1] == -4.0 and W1[1, 3] == 3.5 and W1[1, 2] == 0.0
    x = np.zeros((1, d))
    x[0, 3] = 2.0                          # hidden[1] = relu(3.5 * 2) = 7, hidden[0] = 0
    s = O.predict(x, W1, W2)
    assert s[0, 5] == 14.0 and np.count_nonzero(s) == 1


# ----------------------------------------------------------------------------- Top-K rule, hot region

def test_topk_now_hand_case():
    """topk_now_update ranks by the number of active neurons this step (popcount
    of the union word), ties by group id, and needs at least one active neuron.
    Words (1, 0b111, 0, 0b11, 0b101): counts (1, 3, 0, 2, 2) -> K = 3 picks
    (1, 3, 4); a ranking by 'any active' (ids 0, 1, 3) or by word value (1, 4, 3)
    fails.  Previous hot {0, 3} -> entered {1, 4}, left {0}."""
    w = np.array([1, 0b111, 0, 0b11, 0b101], np.uint32)
    prev = np.array([1, 0, 0, 1, 0], bool)
    topk, hot, ent, left = O.topk_now_update(prev, w, 3)
    assert topk.tolist() == [1, 3, 4]
    assert np.flatnonzero(ent).tolist() == [1, 4] and np.flatnonzero(left).tolist() == [0]
    topk, hot, _, _ = O.topk_now_update(prev, np.zeros(5, np.uint32), 3)
    assert topk.size == 0 and not hot.any()
    topk, _, _, _ = O.topk_now_update(prev, np.full(5, 0xFFFFFFFF, np.uint32), 2)
    assert topk.tolist() == [0, 1]


def test_hot_assign_hand_case():
    """hot_assign over three hand-worked steps with K = 3 slots and G = 6:
    step 1 enters {4, 1} -> 1 takes slot 0, 4 slot 1; step 2 enters {0, 5} and
    {1} leaves -> free slots (0, 2) go to 0 and 5; step 3: {4} leaves, {2}
    enters -> slot 1.  A descending fill, a free list that is not ascending, or a
    leaving group that keeps its slot all fail."""
    G, K = 6, 3
    slot_of = np.full(G, -1)
    group_of = np.full(K, -1)

    def bits(ids):
        b = np.zeros(G, bool)
        b[list(ids)] = True
        return b

    c = O.hot_assign(slot_of, group_of, bits([4, 1]), bits([]))
    assert c == [(1, 0), (4, 1)] and group_of.tolist() == [1, 4, -1]
    c = O.hot_assign(slot_of, group_of, bits([0, 5]), bits([1]))
    assert c == [(0, 0), (5, 2)] and group_of.tolist() == [0, 4, 5]
    assert slot_of.tolist() == [0, -1, -1, -1, 1, 2]
    c = O.hot_assign(slot_of, group_of, bits([2]), bits([4]))
    assert c == [(2, 1)] and group_of.tolist() == [0, 2, 5]
    assert slot_of.tolist() == [0, -1, 1, -1, -1, 2]


def test_hot_region_invariants_over_tam_sequence():
    """Over 200 TAM steps on random activity: the region's occupied slots hold
    exactly the hot set, slot_of and group_of are inverse maps, a group that stays
    hot never moves, the copies are exactly the entering groups, and the region
    of a matrix equals the brute-force gather src[group_of[s]] slot by slot."""
    rng = np.random.default_rng(11)
    G, K, lam, eps = 40, 9, 0.8, 0.01
    src = rng.integers(0, 2 ** 16, size=(32 * G, 3))
    region = np.zeros((32 * K, 3), src.dtype)
    score = np.zeros(G)
    hot = np.zeros(G, bool)
    slot_of = np.full(G, -1)
    group_of = np.full(K, -1)
    act = rng.random(G) < 0.3
    for _ in range(200):
        act = np.where(rng.random(G) < 0.8, act, rng.random(G) < 0.3)
        words = np.where(act, rng.integers(1, 2 ** 32, G), 0).astype(np.uint32)
        before = slot_of.copy()
        score, _, hot_new, ent, left = O.tam_update(score, hot, words, lam, eps, K)
        copies = O.hot_assign(slot_of, group_of, ent, left)
        O.hot_copy(region, src, copies)
        assert sorted(g for g, _ in copies) == np.flatnonzero(ent).tolist()
        assert set(group_of[group_of >= 0].tolist()) == set(np.flatnonzero(hot_new).tolist())
        for s in range(K):
            if group_of[s] >= 0:
                assert slot_of[group_of[s]] == s
                assert np.array_equal(region[32 * s:32 * s + 32], src[32 * group_of[s]:32 * group_of[s] + 32])
        stay = hot & hot_new
        assert np.array_equal(slot_of[stay], before[stay])
        assert np.all(slot_of[~hot_new] == -1)
        hot = hot_new


# ----------------------------------------------------------------------------- offline calibration

def test_calib_threshold_hand_case_and_share():
    """calib_threshold: scores (3, 1, 4, 1, 5, 9, 2, 6), density 0.25 -> k = 6 of the
    sorted (1, 1, 2, 3, 4, 5, 6, 9) -> t = 6, and exactly 2 of 8 scores are >= t.
    An off-by-one in k (t = 5 or 9) or a descending sort (t = 1) fails.  On distinct
    random scores the share >= t is exactly (n - k) / n for several densities."""
    s = np.array([[3, 1, 4, 1], [5, 9, 2, 6]], float)
    t = O.calib_threshold(s, 0.25)
    assert t == 6.0 and int((s >= t).sum()) == 2
    rng = np.random.default_rng(9)
    v = rng.standard_normal((37, 53))
    for rho in (0.01, 0.06, 0.12, 0.5):
        t = O.calib_threshold(v, rho)
        k = int((1 - rho) * v.size)
        assert int((v >= t).sum()) == v.size - k


def test_neuron_counts_and_hot_first_order_hand_case():
    """Counts are column sums of the masks.  Without groups the order is count desc,
    slot asc: counts (2, 5, 5, 0, 3) -> (1, 2, 4, 0, 3).  With groups {0: slots 0, 3},
    {1: slots 1, 4}, {2: slot 2}: group totals 2, 8, 5 -> group 1 (slots 1, 4 by
    count), group 2 (slot 2), group 0 (slot 0 then 3) -> (1, 4, 2, 0, 3).  Ranking
    groups ascending, by id, or members by slot first all fail."""
    masks = np.array([[1, 1, 1, 0, 1], [1, 1, 1, 0, 1], [0, 1, 1, 0, 1],
                      [0, 1, 1, 0, 0], [0, 1, 1, 0, 0]], bool)
    c = O.neuron_counts(masks)
    assert c.tolist() == [2, 5, 5, 0, 3]
    assert O.hot_first_order(c).tolist() == [1, 2, 4, 0, 3]
    assert O.hot_first_order(c, np.array([0, 1, 2, 0, 1])).tolist() == [1, 4, 2, 0, 3]


def test_hot_first_order_brute_force_and_blocks():
    """On random counts with tied totals: the table is a permutation, adjacent slots
    respect the four-key order, and groups of exactly 32 come out as aligned blocks."""
    rng = np.random.default_rng(12)
    G = 20
    group = rng.permutation(np.repeat(np.arange(G), 32))
    counts = rng.integers(0, 4, size=32 * G)
    perm = O.hot_first_order(counts, group)
    assert sorted(perm.tolist()) == list(range(32 * G))
    tot = {g: counts[group == g].sum() for g in range(G)}
    key = [(-tot[group[i]], group[i], -counts[i], i) for i in perm]
    assert key == sorted(key)
    blocks = group[perm].reshape(G, 32)
    assert np.all(blocks == blocks[:, :1])


def test_permute_rows_leaves_the_step_unchanged():
    """permute_rows on a ReGLU layer with scale-free rows: the step on the permuted
    layer has the permuted scores, the mapped index set and the same y."""
    rng = np.random.default_rng(15)
    d, h, f = 16, 8, 40
    layer = {"W1": rng.standard_normal((h, d)), "W2": rng.standard_normal((f, h)),
             "Wa": rng.standard_normal((f, d)), "Wl": rng.standard_normal((f, d)),
             "ba": rng.standard_normal(f), "Wd": rng.standard_normal((f, d))}
    x = rng.standard_normal((3, d))
    p = rng.permutation(f)
    a = O.ffn_step(x, layer, "f32", "f32", "reglu", 0.2)
    b = O.ffn_step(x, O.permute_rows(layer, p), "f32", "f32", "reglu", 0.2)
    assert np.array_equal(b["scores"], a["scores"][:, p])
    inv = np.argsort(p)
    assert b["idx"].tolist() == sorted(inv[a["idx"]].tolist())
    assert np.allclose(a["y"], b["y"], rtol=1e-12, atol=1e-12)
