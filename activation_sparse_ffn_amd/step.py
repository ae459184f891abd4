"""Buffers and call order of one layer-step (predict -> compact -> up -> down) and of
the per-step TAM update, on top of the libsfx binding.  Orchestration only: every
number is produced by the library's kernels."""
import torch

from . import _abi as A

TORCH_WDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
WDT_CODE = {"f32": A.SFX_F32, "f16": A.SFX_F16, "bf16": A.SFX_BF16, "q4": A.SFX_Q4G32}
# `pdtype` of StepBuffers is the predictor's storage: "q4" selects the int4 predictor


class StepBuffers:
    """Device buffers for one layer-step at batch B.  `union_bits` may be a row of a
    caller-owned [L][W] array, so the TAM update can read every layer's union."""

    def __init__(self, d: int, f: int, h: int, B: int, wdtype: str, pdtype: str, device="cuda",
                 union_bits: torch.Tensor = None, kmax: int = None):
        self.d, self.f, self.h, self.B = d, f, h, B
        self.wdtype, self.pdtype = wdtype, pdtype
        self.kmax = f if kmax is None else kmax
        W = (f + 31) // 32
        dev = torch.device(device)
        self.scores = torch.empty(B, f, dtype=torch.float32, device=dev)
        self.tok_bits = torch.zeros(B, W, dtype=torch.int32, device=dev)
        self.union_bits = union_bits if union_bits is not None else torch.zeros(W, dtype=torch.int32, device=dev)
        self.idx = torch.zeros(self.kmax, dtype=torch.int32, device=dev)
        self.count = torch.zeros(1, dtype=torch.int32, device=dev)
        self.hact = torch.zeros(self.kmax, B, dtype=torch.float32, device=dev)
        self.y = torch.empty(B, d, dtype=torch.float32, device=dev)
        self.ws_pred = A.workspace(A.sfx_predict_ws(WDT_CODE[pdtype], B, d, h, f), dev)
        self.ws_comp = A.workspace(A.sfx_compact_ws(B, f), dev)
        self.ws_down = A.workspace(A.sfx_sparse_down_ws(WDT_CODE[wdtype], B, d, self.kmax), dev)

    def status(self) -> dict:
        """Sticky status words of the workspaces (synchronises): the predictor's
        fp16-range flag and the compaction's timeout word; nonzero means some call
        since the last `clear_status` produced undefined results."""
        return {"predict_range": int(self.ws_pred[:4].view(torch.int32).item()),
                "compact_timeout": int(self.ws_comp[4:8].view(torch.int32).item())}

    def clear_status(self):
        self.ws_pred[:4].zero_()
        self.ws_comp[4:8].zero_()

    def check_status(self):
        st = self.status()
        if any(st.values()):
            raise RuntimeError(f"libsfx status words set: {st}")


def run_layer(buf: StepBuffers, layer, x: torch.Tensor, threshold: float, act: str,
              tok_bits: bool = True, stream=None):
    """predict -> compact -> up -> down for one layer.  `layer` holds the device
    tensors W1, W2, Wa, ba, Wd (Wl, Wa_s, Wl_s, Wd_s when present)."""
    g = layer.get if isinstance(layer, dict) else (lambda k: getattr(layer, k, None))
    if g("W1_s") is not None:
        A.sfx_predict_q4(x, g("W1"), g("W1_s"), g("W2"), g("W2_s"), buf.scores, buf.ws_pred, stream=stream)
    else:
        A.sfx_predict(x, g("W1"), g("W2"), buf.scores, buf.ws_pred, stream=stream)
    A.sfx_compact(buf.scores, threshold, buf.union_bits, buf.idx, buf.count, buf.ws_comp,
                  tok_bits=buf.tok_bits if tok_bits else None, stream=stream)
    A.sfx_sparse_up(x, g("Wa"), g("ba"), buf.idx, buf.count, buf.hact, act=act, Wa_scales=g("Wa_s"),
                    Wl=g("Wl"), Wl_scales=g("Wl_s"), stream=stream)
    A.sfx_sparse_down(g("Wd"), buf.idx, buf.count, buf.hact, buf.y, buf.ws_down, Wd_scales=g("Wd_s"),
                      stream=stream)


class TamState:
    """TAM state of L layers with G groups each (fp32 scores, hot bits)."""

    def __init__(self, L: int, G: int, K: int, device="cuda"):
        HW = (G + 31) // 32
        self.L, self.G, self.K = L, G, K
        self.score = torch.zeros(L, G, dtype=torch.float32, device=device)
        self.hot = torch.zeros(L, HW, dtype=torch.int32, device=device)
        self.entered = torch.zeros(L, HW, dtype=torch.int32, device=device)
        self.left = torch.zeros(L, HW, dtype=torch.int32, device=device)
        self.topk = torch.full((L, max(K, 1)), -1, dtype=torch.int32, device=device)
        self.topk_count = torch.zeros(L, dtype=torch.int32, device=device)

    def update(self, union_bits: torch.Tensor, lam: float, eps: float, stream=None):
        A.sfx_tam_update(union_bits, lam, eps, self.K, self.score, self.hot, self.entered, self.left,
                         self.topk, self.topk_count, stream=stream)


class TopKNowState:
    """Hot sets of L layers chosen by the Top-K reload rule on each step's activity
    alone (same bit-set layout as TamState, no scores)."""

    def __init__(self, L: int, G: int, K: int, device="cuda"):
        HW = (G + 31) // 32
        self.L, self.G, self.K = L, G, K
        self.hot = torch.zeros(L, HW, dtype=torch.int32, device=device)
        self.entered = torch.zeros(L, HW, dtype=torch.int32, device=device)
        self.left = torch.zeros(L, HW, dtype=torch.int32, device=device)
        self.topk = torch.full((L, max(K, 1)), -1, dtype=torch.int32, device=device)
        self.topk_count = torch.zeros(L, dtype=torch.int32, device=device)

    def update(self, union_bits: torch.Tensor, stream=None):
        A.sfx_topk_now_update(union_bits, self.K, self.hot, self.entered, self.left, self.topk,
                              self.topk_count, stream=stream)


class HotRegion:
    """Contiguous hot region of K group slots per layer for a list of matrices per
    layer (`mats[l][m]`: a device tensor whose first dimension is the f neurons,
    G groups of 32 rows).  `update(entered, left)` frees the slots of leaving
    groups and copies the entering groups' rows into free slots; `region[l][m]`
    holds K groups of matrix m, slot s = group `group_of[l][s]`."""

    def __init__(self, mats, G: int, K: int, device="cuda"):
        L = len(mats)
        self.L, self.G, self.K = L, G, K
        dev = torch.device(device)
        self.slot_of = torch.full((L, G), -1, dtype=torch.int32, device=dev)
        self.group_of = torch.full((L, K), -1, dtype=torch.int32, device=dev)
        self.copies = torch.zeros(L, K, 2, dtype=torch.int32, device=dev)
        self.ncopies = torch.zeros(L, dtype=torch.int32, device=dev)
        nmat = len(mats[0]) if L else 0
        self.group_bytes = []
        self.region = []
        for l, ms in enumerate(mats):
            if len(ms) != nmat:
                raise ValueError("every layer needs the same matrices")
            row = []
            for m, t in enumerate(ms):
                if t.shape[0] != 32 * G or not t.is_contiguous():
                    raise ValueError(f"layer {l} matrix {m}: need a contiguous tensor of {32 * G} rows")
                gb = t.numel() * t.element_size() // G
                if l == 0:
                    self.group_bytes.append(gb)
                elif gb != self.group_bytes[m]:
                    raise ValueError(f"layer {l} matrix {m}: group size differs from layer 0")
                row.append(torch.zeros((32 * K,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev))
            self.region.append(row)
        self.src = torch.tensor([[t.data_ptr() for t in ms] for ms in mats], dtype=torch.int64, device=dev)
        self.dst = torch.tensor([[t.data_ptr() for t in r] for r in self.region], dtype=torch.int64, device=dev)
        self._mats = mats                      # keeps the sources alive

    def update(self, entered: torch.Tensor, left: torch.Tensor, stream=None):
        A.sfx_hot_update(self.G, self.K, entered, left, self.slot_of, self.group_of, self.copies,
                         self.ncopies, self.group_bytes, self.src, self.dst, stream=stream)


class StackStep:
    """All layers of a stack run by one fused multi-layer kernel per step: the exact
    step (sfx_ffn_step) or, with `pipeline=True`, the Live Pipeline step
    (sfx_ffn_pipeline: each layer's predictor scores its own predictor input).
    Each layer keeps its own output buffers.  `descriptors(inputs, pred_inputs)`
    builds the device descriptor array for lists of per-layer tensors [B][d]; a
    step is `run(descs)`."""

    def __init__(self, layers, d: int, f: int, h: int, B: int, wdtype: str, act: str, device="cuda",
                 union_bits: torch.Tensor = None, pipeline: bool = False):
        self.d, self.f, self.h, self.B, self.act = d, f, h, B, act
        self.pipeline = pipeline
        self.wdt = WDT_CODE[wdtype]
        L = len(layers)
        W = (f + 31) // 32
        self.device = torch.device(device)
        dev = self.device
        self.union_bits = union_bits if union_bits is not None else torch.zeros(L, W, dtype=torch.int32, device=dev)
        self.bufs = []
        self.weights = []
        for l, layer in enumerate(layers):
            g = layer.get if isinstance(layer, dict) else (lambda k, _ly=layer: getattr(_ly, k, None))
            self.bufs.append({"scores": torch.empty(B, f, dtype=torch.float32, device=dev),
                              "tok_bits": torch.zeros(B, W, dtype=torch.int32, device=dev),
                              "union_bits": self.union_bits[l],
                              "idx": torch.zeros(f, dtype=torch.int32, device=dev),
                              "count": torch.zeros(1, dtype=torch.int32, device=dev),
                              "hact": torch.zeros(f, B, dtype=torch.float32, device=dev),
                              "y": torch.empty(B, d, dtype=torch.float32, device=dev)})
            self.weights.append({"W1": g("W1"), "W2": g("W2"), "Wa": g("Wa"), "ba": g("ba"), "Wl": g("Wl"),
                                 "Wd": g("Wd"), "threshold": float(g("threshold"))})
        wsq = A.sfx_ffn_pipeline_ws if pipeline else A.sfx_ffn_step_ws
        n = wsq(self.wdt, A.ACTS[act], B, d, h, f)
        if n == 0:
            raise A.SfxError(-7, wsq.__name__)
        self.ws = A.workspace(n, dev)

    @staticmethod
    def supported(d: int, f: int, h: int, B: int, wdtype: str, act: str, pipeline: bool = False) -> bool:
        if wdtype not in ("f16", "bf16"):
            return False
        wsq = A.sfx_ffn_pipeline_ws if pipeline else A.sfx_ffn_step_ws
        return wsq(WDT_CODE[wdtype], A.ACTS[act], B, d, h, f) > 0

    def descriptors(self, inputs, pred_inputs=None, tok_bits: bool = True) -> torch.Tensor:
        """`inputs[l]` is layer l's FFN input; `pred_inputs[l]` its predictor input
        (Live Pipeline only; None = the FFN input)."""
        entries = []
        pred_inputs = pred_inputs if pred_inputs is not None else [None] * len(inputs)
        for b, wt, x, xp in zip(self.bufs, self.weights, inputs, pred_inputs):
            e = dict(b)
            if not tok_bits:
                e["tok_bits"] = None
            e.update(wt)
            e["x"] = x
            e["xp"] = xp
            entries.append(e)
        return A.layer_descriptors(entries, self.B, self.d, self.h, self.f, self.wdt, self.act, self.device)

    def run(self, descs: torch.Tensor, stream=None):
        call = A.sfx_ffn_pipeline if self.pipeline else A.sfx_ffn_step
        call(self.wdt, self.act, self.B, self.d, self.h, self.f, descs, self.ws, stream=stream)

    def counts(self) -> torch.Tensor:
        return torch.cat([b["count"] for b in self.bufs])

    def error_word(self) -> int:
        """The fused kernel's sticky error word (synchronises): nonzero once a wait of
        some launch on this workspace timed out."""
        return int(self.ws[:4].view(torch.int32).item())

    def clear_error(self):
        self.ws[:4].zero_()

    def check_status(self):
        e = self.error_word()
        if e != 0:
            raise RuntimeError(f"sfx_ffn_step: a grid wait timed out (error word {e})")
