"""Times the fp64 oracle on a sample of a benchmark workload and recomputes its
checks.  TEST INFRASTRUCTURE: run only by the benchmark's CPU-baseline leg, as a
child process whose BLAS thread count is fixed in its environment before numpy is
imported.

    python oracle/time_oracle.py IN.npz OUT.npz

IN holds, for samples i = 0..n-1: the layer's storage arrays (W1, W2, Wa, ba, Wd
and Wl / scales when present, keyed "L{j}/{name}" with j = layer_of[i]), the token
x_i [B][d] and the GPU's outputs for it (scores_i, idx_i, hact_i, y_i); plus the
dtypes, activation and thresholds.  The timed part is `ffn_step` on every sample,
unchanged.  Untimed afterwards: the activations and y on the GPU's index list (the
parity bar), and the comparisons.  Prints one JSON line.
"""
import json
import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from oracle import sfx_oracle as O  # noqa: E402

NEAR = 1e-4


def main():
    src, dst = sys.argv[1], sys.argv[2]
    z = np.load(src)
    wd, pd, act = str(z["wdtype"]), str(z["pdtype"]), str(z["act"])
    layer_of = z["layer_of"]
    thr = z["threshold"]
    layers = {}
    for key in z.files:
        if key.startswith("L"):
            j, name = key[1:].split("/", 1)
            layers.setdefault(int(j), {})[name] = z[key]
    n = len(layer_of)
    xs = [z[f"x{i}"] for i in range(n)]
    xps = [z[f"xp{i}"] if f"xp{i}" in z.files else None for i in range(n)]   # Live Pipeline predictor inputs
    t0 = time.perf_counter()
    refs = [O.ffn_step(xs[i], layers[int(layer_of[i])], wd, pd, act, float(thr[i]), xp=xps[i]) for i in range(n)]
    dt = time.perf_counter() - t0
    r = {"seconds": dt, "layer_steps": n, "score_err": 0.0, "near_threshold": 0, "mask_mismatch": 0,
         "hact_rel": 0.0, "y_rel": 0.0, "y_rel_own_list": 0.0}
    for i in range(n):
        L = layers[int(layer_of[i])]
        ref = refs[i]
        s_gpu = z[f"scores{i}"].astype(np.float64)
        r["score_err"] = max(r["score_err"], float(np.max(np.abs(s_gpu - ref["scores"]))))
        near = np.abs(ref["scores"] - float(thr[i])) < NEAR
        r["near_threshold"] += int(near.sum())
        tok_gpu, _, _, _ = O.gate(s_gpu, float(thr[i]))
        r["mask_mismatch"] += int(np.sum(tok_gpu[~near] != ref["tok_mask"][~near]))
        gidx = z[f"idx{i}"]
        x64 = O.decode(xs[i], pd)
        Wl = O.rows(L["Wl"], wd, gidx, L.get("Wl_s")) if act == "reglu" else None
        hact = O.sparse_up(x64, O.rows(L["Wa"], wd, gidx, L.get("Wa_s")),
                           np.asarray(L["ba"], np.float64)[gidx], act, Wl)
        y = O.sparse_down(O.rows(L["Wd"], wd, gidx, L.get("Wd_s")), hact)
        den = lambda a: float(np.max(np.abs(a))) if a.size else 0.0
        rel = lambda a, b: float(np.max(np.abs(a - b))) / den(b) if den(b) > 0 else float(np.max(np.abs(a - b), initial=0.0))
        r["hact_rel"] = max(r["hact_rel"], rel(z[f"hact{i}"].astype(np.float64), hact))
        r["y_rel"] = max(r["y_rel"], rel(z[f"y{i}"].astype(np.float64), y))
        r["y_rel_own_list"] = max(r["y_rel_own_list"], rel(z[f"y{i}"].astype(np.float64), ref["y"]))
    np.savez(dst, seconds=dt)
    print(json.dumps(r), flush=True)


if __name__ == "__main__":
    main()
