"""Plain fp64 CPU oracle of the predictor-gated activation-sparse FFN step.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path and
imports nothing from it.  Every stored value is first converted exactly to fp64;
all arithmetic is fp64 numpy, with matrix products as the only library primitive.

Functions and the passages they follow:
  predict       PowerInfer page, Method, per-layer predictor pseudocode (§5.1):
                hidden = relu(W1 x), scores = W2 hidden.
  gate          PowerInfer page, Method, hybrid-execution pseudocode (§5.1, §5.3):
                a neuron is active when its score is >= the threshold; Paper vs
                code, predictor threshold (a score below it is skipped).  For a
                batch, the active set is the union of the per-token sets.
  sparse_up     PowerInfer page, Method, neuron-aware operators (§5.4): only the
                rows of active neurons are read; Paper vs code, activation
                functions (ReLU, ReGLU, squared ReLU).
  sparse_down   PowerInfer page, Method, hybrid-execution pseudocode: y is the sum
                of the active neurons' contributions (the partial sums of the two
                executors add up to it).
  dequant_q4    int4 symmetric, group 32, fp16 scale: w = q * s (FFN rows, and the
                predictor's W1 / W2 when they are stored in int4).
  tam_update    KAIROX page, Core method, item 4 (TAM, §6): a group's score
                accumulates when active and decays by lambda when not; candidates
                exceed tau = (1 - lambda) + eps; the highest-scoring candidates fill
                the capacity K.  Item 3 (§5.2): decisions are per group of 32.
                Item 6 (§8): entering / leaving sets are set differences.
  topk_now_update  KAIROX page, Experiments, strategies and ablations: the Top-K
                reload rule TAM is compared with -- the groups most active in this
                step alone (count of active neurons), no memory.
  hot_assign, hot_copy  KAIROX page, Core method, items 3 and 6: a contiguous hot
                region of K group slots; leaving groups free their slots and only
                entering groups are copied in.
  calib_threshold, neuron_counts, hot_first_order, permute_rows
                PowerInfer page, Method, offline profiling (activation counts on
                calibration inputs) and the neuron table; KAIROX page, Core method,
                item 1 (co-active neurons stored as contiguous groups); Paper vs
                code, predictor threshold (one per layer).
  dense_ffn     the dense layer the sparse step reproduces when every neuron with
                a nonzero activation is in the active set (used only by the pins).
  ffn_step      the four steps in order; with a separate predictor input xp it is
                the Live Pipeline step of the KAIROX page (Core method, item 2): the
                predictor of a layer scores an input known one layer earlier, the
                FFN rows then run on the layer's own input.
  mask_recall   share of the active neurons of one mask that another mask also
                holds (KAIROX page, Prediction cost and quality: predictor recall).

Readings where the pages leave a step open: the predictor has no biases; the
hidden layer stays in full precision; a NaN score is inactive; the activated
branch carries a bias and the ReGLU linear branch and the down projection carry
none; for a batch every token computes every neuron of the union; the TAM score is
the exponential moving average s <- lambda*s + (1-lambda)*a, starting from s = 0
and an empty hot set, ranked by score descending then group id ascending.

Pins: every function here is checked in tests/test_oracle_pins.py against hand-
computed fixtures, closed forms and brute force (no function is parity unpinned).
"""
import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------- storage

def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored elements: 'f32' / 'f16' arrays, or 'bf16' given
    as the uint16 bit pattern (the high half of an IEEE single)."""
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(F64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(F64)
    raise ValueError(f"decode: unknown dtype {dtype}")


def dequant_q4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """int4 rows -> fp64.  q uint8 [rows][cols/2]: byte c holds column 2c in its low
    nibble and column 2c+1 in its high nibble, two's complement in [-8, 7].
    s float16 [rows][cols/32]: one scale per 32 consecutive columns.  w = q * s."""
    q = np.asarray(q, dtype=np.uint8)
    rows, half = q.shape
    lo = (q & 0x0F).astype(np.int64)
    hi = (q >> 4).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    vals = np.empty((rows, 2 * half), dtype=F64)
    vals[:, 0::2] = lo
    vals[:, 1::2] = hi
    scale = np.repeat(np.asarray(s).astype(F64), 32, axis=1)
    return vals * scale


def rows(W, dtype: str, idx=None, scales=None) -> np.ndarray:
    """fp64 rows `idx` (all rows when idx is None) of a stored matrix."""
    sel = W if idx is None else np.asarray(W)[np.asarray(idx, dtype=np.int64)]
    if dtype == "q4":
        ssel = scales if idx is None else np.asarray(scales)[np.asarray(idx, dtype=np.int64)]
        return dequant_q4(sel, ssel)
    return decode(sel, dtype)


# ----------------------------------------------------------------------------- predictor

def predict(x: np.ndarray, W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """Scores of every neuron for each token.  x [B][d], W1 [h][d], W2 [f][h] in
    fp64.  Returns scores [B][f]."""
    x = np.atleast_2d(np.asarray(x, dtype=F64))
    scores = np.empty((x.shape[0], W2.shape[0]), dtype=F64)
    for b in range(x.shape[0]):
        hidden = np.maximum(W1 @ x[b], 0.0)      # (h,)
        scores[b] = W2 @ hidden                  # (f,)
    return scores


# ----------------------------------------------------------------------------- gate

def gate(scores: np.ndarray, threshold: float):
    """Active sets.  Returns (tok_mask [B][f] bool, union [f] bool, idx int32
    ascending, count).  A neuron is active for a token when score >= threshold
    (a NaN score compares false and is inactive)."""
    scores = np.atleast_2d(np.asarray(scores, dtype=F64))
    with np.errstate(invalid="ignore"):
        tok_mask = scores >= F64(threshold)
    union = tok_mask.any(axis=0)
    idx = np.flatnonzero(union).astype(np.int32)
    return tok_mask, union, idx, int(idx.size)


def pack_bits(mask: np.ndarray) -> np.ndarray:
    """Bit i of a mask goes to bit (i mod 32) of word i // 32, least significant
    first; the last word is zero-padded.  mask [..., f] -> uint32 [..., ceil(f/32)]."""
    mask = np.asarray(mask, dtype=bool)
    f = mask.shape[-1]
    nw = (f + 31) // 32
    pad = np.zeros(mask.shape[:-1] + (nw * 32,), dtype=np.uint64)
    pad[..., :f] = mask
    pad = pad.reshape(mask.shape[:-1] + (nw, 32))
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (pad * weights).sum(axis=-1).astype(np.uint32)


# ----------------------------------------------------------------------------- sparse FFN

def sparse_up(x: np.ndarray, Wa_rows: np.ndarray, ba_rows, act: str, Wl_rows=None) -> np.ndarray:
    """Activations of the active neurons.  x [B][d]; Wa_rows / Wl_rows [k][d] are the
    active rows (row j <-> neuron idx[j]); ba_rows [k] or None.
    ReLU:  a = max(Wa_i . x + b_i, 0).  ReGLU: a = max(Wa_i . x + b_i, 0) * (Wl_i . x).
    Squared ReLU ('relu2'): a = max(Wa_i . x + b_i, 0)^2.
    Returns hact [k][B]."""
    x = np.atleast_2d(np.asarray(x, dtype=F64))
    z = Wa_rows @ x.T                            # (k, B)
    if ba_rows is not None:
        z = z + np.asarray(ba_rows, dtype=F64)[:, None]
    a = np.maximum(z, 0.0)
    if act == "reglu":
        a = a * (Wl_rows @ x.T)
    elif act == "relu2":
        a = a * a
    elif act != "relu":
        raise ValueError(act)
    return a


def sparse_down(Wd_rows: np.ndarray, hact: np.ndarray) -> np.ndarray:
    """y_b = sum_j hact[j][b] * Wd[idx_j].  Wd_rows [k][d], hact [k][B] -> y [B][d]."""
    hact = np.asarray(hact, dtype=F64)
    if hact.shape[0] == 0:
        return np.zeros((hact.shape[1], Wd_rows.shape[1]), dtype=F64)
    return hact.T @ Wd_rows


def dense_ffn(x, Wa, ba, Wd, act: str, Wl=None) -> np.ndarray:
    """The dense layer: y = Wd^T act(Wa x + b) over every neuron.  x [B][d]."""
    x = np.atleast_2d(np.asarray(x, dtype=F64))
    z = x @ Wa.T
    if ba is not None:
        z = z + np.asarray(ba, dtype=F64)[None, :]
    a = np.maximum(z, 0.0)
    if act == "reglu":
        a = a * (x @ Wl.T)
    elif act == "relu2":
        a = a * a
    return a @ Wd


def true_relu_idx(x, Wa, ba) -> np.ndarray:
    """Neurons whose activated-branch pre-activation is > 0 for some token (the
    exact ReLU mask).  x [B][d], Wa [f][d] fp64."""
    x = np.atleast_2d(np.asarray(x, dtype=F64))
    z = x @ Wa.T
    if ba is not None:
        z = z + np.asarray(ba, dtype=F64)[None, :]
    return np.flatnonzero((z > 0.0).any(axis=0)).astype(np.int32)


def predictor_weights(layer: dict, pdtype: str):
    """fp64 W1, W2 of a layer: decoded from `pdtype` storage, or dequantised when the
    layer carries int4 predictor scales (W1_s, W2_s)."""
    if layer.get("W1_s") is not None:
        return dequant_q4(layer["W1"], layer["W1_s"]), dequant_q4(layer["W2"], layer["W2_s"])
    return decode(layer["W1"], pdtype), decode(layer["W2"], pdtype)


def ffn_step(x, layer: dict, wdtype: str, pdtype: str, act: str, threshold: float, xp=None):
    """One layer-step in the pages' order: predict -> gate -> up -> down.
    `layer` holds storage arrays W1, W2, Wa, ba, Wd (and Wl, *_s scales).  The
    predictor scores `xp` when given (the Live Pipeline's one-layer-ahead input),
    else `x`; the up and down rows always use `x`.
    Returns a dict with scores, tok_mask, union, idx, count, hact, y."""
    x64 = decode(x, pdtype)
    xp64 = x64 if xp is None else decode(xp, pdtype)
    W1, W2 = predictor_weights(layer, pdtype)
    scores = predict(xp64, W1, W2)
    tok_mask, union, idx, count = gate(scores, threshold)
    Wa_r = rows(layer["Wa"], wdtype, idx, layer.get("Wa_s"))
    Wl_r = rows(layer["Wl"], wdtype, idx, layer.get("Wl_s")) if act == "reglu" else None
    ba_r = np.asarray(layer["ba"], dtype=F64)[idx]
    hact = sparse_up(x64, Wa_r, ba_r, act, Wl_r)
    y = sparse_down(rows(layer["Wd"], wdtype, idx, layer.get("Wd_s")), hact)
    return {"scores": scores, "tok_mask": tok_mask, "union": union, "idx": idx,
            "count": count, "hact": hact, "y": y}


def mask_recall(predicted: np.ndarray, exact: np.ndarray) -> float:
    """|predicted AND exact| / |exact| over boolean masks (1.0 when exact is empty)."""
    predicted = np.asarray(predicted, dtype=bool)
    exact = np.asarray(exact, dtype=bool)
    n = int(exact.sum())
    return 1.0 if n == 0 else float((predicted & exact).sum()) / n


# ----------------------------------------------------------------------------- TAM

def tam_tau(lam: float, eps: float) -> float:
    """Candidate threshold tau = (1 - lambda) + eps."""
    return (1.0 - lam) + eps


def tam_select(score: np.ndarray, prev_hot: np.ndarray, tau: float, K: int):
    """Decision part of a TAM step on given scores: candidates have score > tau;
    they are ranked by score descending, then group id ascending; the first
    min(K, #candidates) are hot.  Returns (topk int32, hot, entered, left), the
    three sets as bool [G]."""
    score = np.asarray(score)
    G = score.shape[0]
    cand = np.flatnonzero(score > tau)
    # rank: score descending, then group id ascending (lexsort sorts by its last key first)
    order = cand[np.lexsort((cand, -score[cand]))]
    topk = order[:K].astype(np.int32)
    hot = np.zeros(G, dtype=bool)
    hot[topk] = True
    prev_hot = np.asarray(prev_hot, dtype=bool)
    entered = hot & ~prev_hot
    left = prev_hot & ~hot
    return topk, hot, entered, left


def tam_update(score: np.ndarray, prev_hot: np.ndarray, union_words: np.ndarray,
               lam: float, eps: float, K: int):
    """One TAM step for one layer.  union_words [G] uint32: word g is group g's 32
    neurons in the union mask, and the group is active when any of them is.
    score [G] fp64 is the state before the step.
    Returns (score', topk, hot, entered, left)."""
    a = (np.asarray(union_words) != 0).astype(F64)
    score = lam * np.asarray(score, dtype=F64) + (1.0 - lam) * a
    topk, hot, entered, left = tam_select(score, prev_hot, tam_tau(lam, eps), K)
    return score, topk, hot, entered, left


def topk_now_update(prev_hot: np.ndarray, union_words: np.ndarray, K: int):
    """The Top-K reload rule TAM is compared with (KAIROX page, Experiments:
    strategies and ablations): hot = the K groups with the most active neurons in
    this step's union mask (at least one), ranked by that count descending, then
    group id ascending; no memory of earlier steps.
    Returns (topk int32, hot, entered, left)."""
    w = np.ascontiguousarray(union_words, dtype=np.uint32)
    count = np.unpackbits(w.view(np.uint8)).reshape(-1, 32).sum(axis=1)     # popcount per word
    cand = np.flatnonzero(count > 0)
    order = cand[np.lexsort((cand, -count[cand]))]
    topk = order[:K].astype(np.int32)
    hot = np.zeros(w.shape[0], dtype=bool)
    hot[topk] = True
    prev_hot = np.asarray(prev_hot, dtype=bool)
    return topk, hot, hot & ~prev_hot, prev_hot & ~hot


# ----------------------------------------------------------------------------- hot region

def hot_assign(slot_of: np.ndarray, group_of: np.ndarray, entered: np.ndarray, left: np.ndarray):
    """Slot bookkeeping of the hot region of one layer (KAIROX page, Core method:
    item 3, a group moves as one contiguous block; item 6, only the set difference
    moves).  slot_of [G] / group_of [K] int (-1 = none) are updated in place:
    leaving groups free their slots; then the entering groups in ascending order
    take the free slots in ascending order.  Returns the copies [(group, slot)]."""
    for g in np.flatnonzero(left):
        s = int(slot_of[g])
        if s >= 0:
            group_of[s] = -1
        slot_of[g] = -1
    free = [s for s in range(group_of.shape[0]) if group_of[s] < 0]
    copies = []
    for i, g in enumerate(np.flatnonzero(entered)):
        if i < len(free):
            slot_of[g] = free[i]
            group_of[free[i]] = g
            copies.append((int(g), free[i]))
        else:
            slot_of[g] = -1
    return copies


def hot_copy(region: np.ndarray, src: np.ndarray, copies):
    """Applies the copies to one matrix's hot region: slot s of `region` (32 rows
    per group, any row width) receives group g's 32 rows of `src`."""
    for g, s in copies:
        region[32 * s:32 * s + 32] = src[32 * g:32 * g + 32]
    return region


# ----------------------------------------------------------------------------- offline calibration

def calib_threshold(scores: np.ndarray, density: float) -> float:
    """Per-layer threshold: the k-th smallest calibration score (0-based), with
    k = floor((1 - density) * n) over all n = tokens x f scores, so that the scores
    >= it are a share `density` of the whole (exactly, when the scores are distinct)."""
    v = np.sort(np.asarray(scores, dtype=F64).ravel())
    k = min(int((1.0 - density) * v.size), v.size - 1)
    return float(v[k])


def neuron_counts(masks: np.ndarray) -> np.ndarray:
    """Calibration frequency of each neuron: the number of tokens whose mask holds it.
    masks [N][f] bool."""
    return np.asarray(masks, dtype=bool).sum(axis=0).astype(np.int64)


def hot_first_order(counts: np.ndarray, group: np.ndarray = None) -> np.ndarray:
    """Hot-first neuron table: new slot r holds old slot perm[r].  Groups (group ids
    per slot; None = every neuron alone) are ranked by their members' total count
    descending, then group id ascending; inside a group, members by count descending,
    then slot ascending."""
    counts = np.asarray(counts, dtype=np.int64)
    f = counts.shape[0]
    slot = np.arange(f)
    if group is None:
        gid, gsum = slot, counts
    else:
        gid = np.asarray(group, dtype=np.int64)
        totals = {}
        for i in range(f):
            totals[gid[i]] = totals.get(gid[i], 0) + counts[i]
        gsum = np.array([totals[g] for g in gid])
    # lexsort: last key first -> group count desc, group id asc, count desc, slot asc
    return np.lexsort((slot, -counts, gid, -gsum)).astype(np.int32)


def permute_rows(layer: dict, perm: np.ndarray) -> dict:
    """The layer with every per-neuron row (W2, Wa, Wl, Wd, their scale tables, ba)
    taken in `perm` order; W1 and its scales are unchanged."""
    out = dict(layer)
    for k in ("W2", "W2_s", "Wa", "Wa_s", "Wl", "Wl_s", "Wd", "Wd_s", "ba"):
        if layer.get(k) is not None:
            out[k] = np.asarray(layer[k])[perm]
    return out
