"""ctypes binding of libsfx (include/sfx.h).

Argument marshalling only: each function takes torch tensors, checks dtype /
contiguity / device, passes raw pointers and the current HIP stream to the C entry
point of the same name, and raises SfxError on a negative status.  Every step of
the computation runs in the library's kernels; there is no fallback.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsfx.so")

SFX_F32, SFX_F16, SFX_BF16, SFX_Q4G32 = 0, 1, 2, 3
SFX_RELU, SFX_REGLU, SFX_RELU2 = 0, 1, 2
SFX_MAX_B = 64
SFX_MAX_GROUPS = 1024
ACTS = {"relu": SFX_RELU, "reglu": SFX_REGLU, "relu2": SFX_RELU2}
WDT = {torch.float32: SFX_F32, torch.float16: SFX_F16, torch.bfloat16: SFX_BF16}

EXPORTS = ("sfx_status_str", "sfx_abi_version", "sfx_predict_ws", "sfx_predict", "sfx_compact_ws",
           "sfx_compact", "sfx_sparse_up", "sfx_sparse_down_ws", "sfx_sparse_down", "sfx_tam_ws",
           "sfx_tam_update", "sfx_ffn_step_ws", "sfx_ffn_step", "sfx_sparse_down_noalloc",
           "sfx_ffn_pipeline_ws", "sfx_ffn_pipeline", "sfx_stream_read", "sfx_predict_q4",
           "sfx_topk_now_update", "sfx_hot_update", "sfx_count_active", "sfx_select_kth_ws",
           "sfx_select_kth", "sfx_hot_first_order_ws", "sfx_hot_first_order", "sfx_gather_rows",
           "sfx_dense_ffn_ws", "sfx_dense_ffn")
HOT_MAX_MATS = 8
SFX_DOWN_SCRATCH_BYTES = 17 << 20


class SfxLayer(ctypes.Structure):
    """Mirror of `sfx_layer` in include/sfx.h (one layer of a fused step)."""
    _fields_ = [("x", ctypes.c_void_p), ("W1", ctypes.c_void_p), ("W2", ctypes.c_void_p),
                ("Wa", ctypes.c_void_p), ("Wa_scales", ctypes.c_void_p), ("ba", ctypes.c_void_p),
                ("Wl", ctypes.c_void_p), ("Wl_scales", ctypes.c_void_p), ("Wd", ctypes.c_void_p),
                ("Wd_scales", ctypes.c_void_p), ("threshold", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("scores", ctypes.c_void_p), ("tok_bits", ctypes.c_void_p), ("union_bits", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("count", ctypes.c_void_p), ("hact", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("xp", ctypes.c_void_p)]


class SfxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsfx (once).  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libsfx is not built ({path} missing): run "
                           "`python -m activation_sparse_ffn_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.sfx_status_str.restype = ctypes.c_char_p
    lib.sfx_status_str.argtypes = [I]
    lib.sfx_abi_version.restype = I
    lib.sfx_abi_version.argtypes = []
    lib.sfx_predict_ws.restype = Z
    lib.sfx_predict_ws.argtypes = [I, I, I, I, I]
    lib.sfx_predict.restype = I
    lib.sfx_predict.argtypes = [P, I, I, I, I, I, P, P, P, P, P, Z]
    lib.sfx_compact_ws.restype = Z
    lib.sfx_compact_ws.argtypes = [I, I]
    lib.sfx_compact.restype = I
    lib.sfx_compact.argtypes = [P, I, I, P, F, P, P, P, I, P, P, Z]
    lib.sfx_sparse_up.restype = I
    lib.sfx_sparse_up.argtypes = [P, I, I, I, I, I, P, P, P, P, P, P, P, P, I, P]
    lib.sfx_sparse_down_ws.restype = Z
    lib.sfx_sparse_down_ws.argtypes = [I, I, I, I]
    lib.sfx_sparse_down.restype = I
    lib.sfx_sparse_down.argtypes = [P, I, I, I, I, P, P, P, P, I, P, P, P, Z]
    lib.sfx_sparse_down_noalloc.restype = I
    lib.sfx_sparse_down_noalloc.argtypes = [P, I, I, I, I, P, P, P, P, I, P, P]
    lib.sfx_tam_ws.restype = Z
    lib.sfx_tam_ws.argtypes = [I, I]
    lib.sfx_tam_update.restype = I
    lib.sfx_tam_update.argtypes = [P, I, I, P, F, F, I, P, P, P, P, P, P, P, Z]
    lib.sfx_topk_now_update.restype = I
    lib.sfx_topk_now_update.argtypes = [P, I, I, P, I, P, P, P, P, P]
    lib.sfx_hot_update.restype = I
    lib.sfx_hot_update.argtypes = [P, I, I, I, P, P, P, P, P, P, I, P, P, P]
    lib.sfx_count_active.restype = I
    lib.sfx_count_active.argtypes = [P, I, I, P, P]
    lib.sfx_select_kth_ws.restype = Z
    lib.sfx_select_kth_ws.argtypes = []
    lib.sfx_select_kth.restype = I
    lib.sfx_select_kth.argtypes = [P, Z, P, Z, P, P, Z]
    lib.sfx_hot_first_order_ws.restype = Z
    lib.sfx_hot_first_order_ws.argtypes = [I]
    lib.sfx_hot_first_order.restype = I
    lib.sfx_hot_first_order.argtypes = [P, I, P, P, P, P, Z]
    lib.sfx_gather_rows.restype = I
    lib.sfx_gather_rows.argtypes = [P, I, I, Z, P, P, P]
    lib.sfx_dense_ffn_ws.restype = Z
    lib.sfx_dense_ffn_ws.argtypes = [I, I, I, I]
    lib.sfx_dense_ffn.restype = I
    lib.sfx_dense_ffn.argtypes = [P, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, Z]
    lib.sfx_ffn_step_ws.restype = Z
    lib.sfx_ffn_step_ws.argtypes = [I, I, I, I, I, I]
    lib.sfx_ffn_step.restype = I
    lib.sfx_ffn_step.argtypes = [P, I, I, I, I, I, I, I, P, P, Z]
    lib.sfx_predict_q4.restype = I
    lib.sfx_predict_q4.argtypes = [P, I, I, I, I, P, P, P, P, P, P, P, Z]
    lib.sfx_stream_read.restype = I
    lib.sfx_stream_read.argtypes = [P, P, Z, P]
    lib.sfx_ffn_pipeline_ws.restype = Z
    lib.sfx_ffn_pipeline_ws.argtypes = [I, I, I, I, I, I]
    lib.sfx_ffn_pipeline.restype = I
    lib.sfx_ffn_pipeline.argtypes = [P, I, I, I, I, I, I, I, P, P, Z]
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().sfx_status_str(int(status)).decode()


def abi_version() -> int:
    return load().sfx_abi_version()


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != 0:
        raise SfxError(status, where)


def _wdt_of(t: torch.Tensor) -> int:
    if t.dtype == torch.uint8:
        return SFX_Q4G32
    if t.dtype not in WDT:
        raise TypeError(f"unsupported weight dtype {t.dtype}")
    return WDT[t.dtype]


def _need(t, dtype, where):
    if t.dtype != dtype:
        raise TypeError(f"{where}: expected {dtype}, got {t.dtype}")


# ------------------------------------------------------------------------- workspaces

def workspace(nbytes: int, device=None) -> torch.Tensor:
    """Zero-filled device workspace of at least `nbytes` (the library keeps its
    control words at zero between calls)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")


def sfx_predict_ws(wdt: int, B: int, d: int, h: int, f: int) -> int:
    return load().sfx_predict_ws(wdt, B, d, h, f)


def sfx_compact_ws(B: int, f: int) -> int:
    return load().sfx_compact_ws(B, f)


def sfx_sparse_down_ws(wdt: int, B: int, d: int, kmax: int) -> int:
    return load().sfx_sparse_down_ws(wdt, B, d, kmax)


def sfx_tam_ws(G: int, K: int) -> int:
    return load().sfx_tam_ws(G, K)


# ------------------------------------------------------------------------- entry points

def sfx_predict(x, W1, W2, scores, ws, stream=None):
    """scores[B][f] = W2 relu(W1 x_b).  x [B][d], W1 [h][d], W2 [f][h] (same dtype)."""
    B, d = x.shape
    h, f = W1.shape[0], W2.shape[0]
    if W1.shape[1] != d or W2.shape[1] != h or tuple(scores.shape) != (B, f):
        raise ValueError("sfx_predict: shape mismatch")
    if W1.dtype != x.dtype or W2.dtype != x.dtype:
        raise TypeError("sfx_predict: x, W1, W2 must share a dtype")
    _need(scores, torch.float32, "scores")
    ptrs = (_ptr(x), _ptr(W1), _ptr(W2), _ptr(scores), _ptr(ws))
    st = load().sfx_predict(_stream(stream), _wdt_of(x), B, d, h, f, *ptrs, ws.numel() if ws is not None else 0)
    _check(st, "sfx_predict")


def sfx_predict_q4(x, W1, W1_scales, W2, W2_scales, scores, ws, stream=None):
    """scores[B][f] = W2 relu(W1 x_b) with int4 W1 [h][d/2] / W2 [f][h/2] codes and
    fp16 scales; x [B][d] fp16."""
    B, d = x.shape
    h, f = W1.shape[0], W2.shape[0]
    if W1.shape[1] * 2 != d or W2.shape[1] * 2 != h or tuple(scores.shape) != (B, f):
        raise ValueError("sfx_predict_q4: shape mismatch")
    _need(x, torch.float16, "x")
    _need(scores, torch.float32, "scores")
    for t, n in ((W1, "W1"), (W2, "W2")):
        _need(t, torch.uint8, n)
    for t, n in ((W1_scales, "W1_scales"), (W2_scales, "W2_scales")):
        _need(t, torch.float16, n)
    p = (_ptr(x), _ptr(W1), _ptr(W1_scales), _ptr(W2), _ptr(W2_scales), _ptr(scores), _ptr(ws))
    st = load().sfx_predict_q4(_stream(stream), B, d, h, f, *p, ws.numel() if ws is not None else 0)
    _check(st, "sfx_predict_q4")


def sfx_compact(scores, threshold, union_bits, idx, count, ws, tok_bits=None, stream=None):
    """Union of {score >= threshold} over tokens -> ascending idx, device count."""
    B, f = scores.shape
    _need(scores, torch.float32, "scores")
    for t, n in ((union_bits, "union_bits"), (count, "count"), (idx, "idx")):
        if t.dtype not in (torch.int32, torch.uint32):
            raise TypeError(f"{n} must be int32/uint32")
    p = (_ptr(scores), _ptr(tok_bits), _ptr(union_bits), _ptr(idx), _ptr(count), _ptr(ws))
    st = load().sfx_compact(_stream(stream), B, f, p[0], float(threshold), p[1], p[2], p[3], idx.numel(), p[4],
                            p[5], ws.numel() if ws is not None else 0)
    _check(st, "sfx_compact")


def sfx_sparse_up(x, Wa, ba, idx, count, hact, act="relu", Wa_scales=None, Wl=None, Wl_scales=None,
                  stream=None):
    """hact[kmax][B] for the listed neurons (rows < count written)."""
    B, d = x.shape
    f = Wa.shape[0]
    wdt = _wdt_of(Wa)
    kmax = idx.numel()
    if hact.numel() < kmax * B:
        raise ValueError("hact too small")
    _need(hact, torch.float32, "hact")
    if ba is not None:
        _need(ba, torch.float32, "ba")
    p = (_ptr(x), _ptr(Wa), _ptr(Wa_scales), _ptr(ba), _ptr(Wl), _ptr(Wl_scales), _ptr(idx), _ptr(count))
    st = load().sfx_sparse_up(_stream(stream), wdt, ACTS[act], B, d, f, *p, kmax, _ptr(hact))
    _check(st, "sfx_sparse_up")


def sfx_sparse_down(Wd, idx, count, hact, y, ws, Wd_scales=None, stream=None):
    """y[B][d] = sum_j hact[j][b] Wd[idx_j] (overwritten)."""
    B, d = y.shape
    f = Wd.shape[0]
    wdt = _wdt_of(Wd)
    kmax = idx.numel()
    _need(y, torch.float32, "y")
    _need(hact, torch.float32, "hact")
    p = (_ptr(Wd), _ptr(Wd_scales), _ptr(idx), _ptr(count))
    q = (_ptr(hact), _ptr(y), _ptr(ws))
    st = load().sfx_sparse_down(_stream(stream), wdt, B, d, f, *p, kmax, *q, ws.numel() if ws is not None else 0)
    _check(st, "sfx_sparse_down")


def sfx_dense_ffn_ws(wdt: int, B: int, d: int, f: int) -> int:
    return load().sfx_dense_ffn_ws(wdt, B, d, f)


def sfx_dense_ffn(x, Wa, ba, Wd, hact, y, ws, act="relu", Wa_scales=None, Wl=None, Wl_scales=None,
                  Wd_scales=None, stream=None):
    """The FFN over every neuron: hact[f][B] and y[B][d] (both overwritten)."""
    B, d = x.shape
    f = Wa.shape[0]
    wdt = _wdt_of(Wa)
    if hact.numel() < f * B or tuple(y.shape) != (B, d):
        raise ValueError("sfx_dense_ffn: hact [f][B] and y [B][d] expected")
    _need(hact, torch.float32, "hact")
    _need(y, torch.float32, "y")
    if ba is not None:
        _need(ba, torch.float32, "ba")
    p = (_ptr(x), _ptr(Wa), _ptr(Wa_scales), _ptr(ba), _ptr(Wl), _ptr(Wl_scales), _ptr(Wd), _ptr(Wd_scales),
         _ptr(hact), _ptr(y), _ptr(ws))
    st = load().sfx_dense_ffn(_stream(stream), wdt, ACTS[act], B, d, f, *p, ws.numel() if ws is not None else 0)
    _check(st, "sfx_dense_ffn")


def sfx_sparse_down_noalloc(Wd, idx, count, hact, y, Wd_scales=None, stream=None):
    """sfx_sparse_down without a workspace: the library's static scratch is used
    (shared by every call on the GPU, so calls must not overlap)."""
    B, d = y.shape
    f = Wd.shape[0]
    wdt = _wdt_of(Wd)
    kmax = idx.numel()
    _need(y, torch.float32, "y")
    _need(hact, torch.float32, "hact")
    p = (_ptr(Wd), _ptr(Wd_scales), _ptr(idx), _ptr(count))
    st = load().sfx_sparse_down_noalloc(_stream(stream), wdt, B, d, f, *p, kmax, _ptr(hact), _ptr(y))
    _check(st, "sfx_sparse_down_noalloc")


def sfx_tam_update(union_bits, lam, eps, K, score, hot_bits, entered_bits, left_bits, topk, topk_count,
                   ws=None, stream=None):
    """One TAM step for L layers.  union_bits [L][G], score [L][G] fp32, bit sets [L][ceil(G/32)]."""
    L, G = union_bits.shape
    _need(score, torch.float32, "score")
    p = (_ptr(score), _ptr(hot_bits), _ptr(entered_bits), _ptr(left_bits), _ptr(topk) if K > 0 else None,
         _ptr(topk_count), _ptr(ws))
    st = load().sfx_tam_update(_stream(stream), L, G, _ptr(union_bits), float(lam), float(eps), int(K), *p,
                               ws.numel() if ws is not None else 0)
    _check(st, "sfx_tam_update")


def sfx_topk_now_update(union_bits, K, hot_bits, entered_bits, left_bits, topk, topk_count, stream=None):
    """The Top-K reload rule on this step's activity alone (no score state).
    union_bits [L][G], bit sets [L][ceil(G/32)], topk [L][K], topk_count [L]."""
    L, G = union_bits.shape
    st = load().sfx_topk_now_update(_stream(stream), L, G, _ptr(union_bits), int(K), _ptr(hot_bits),
                                    _ptr(entered_bits), _ptr(left_bits), _ptr(topk) if K > 0 else None,
                                    _ptr(topk_count))
    _check(st, "sfx_topk_now_update")


def sfx_hot_update(G, K, entered_bits, left_bits, slot_of, group_of, copies, ncopies, group_bytes=(),
                   src=None, dst=None, stream=None):
    """Hot-region slots and the copy of entering groups for L layers.
    entered_bits / left_bits [L][ceil(G/32)], slot_of [L][G], group_of [L][K],
    copies [L][K][2], ncopies [L] (int32 device tensors); group_bytes: host sizes
    of one group per matrix; src / dst: device int64 tensors [L][nmat] of
    matrix addresses (None when group_bytes is empty)."""
    L = entered_bits.shape[0]
    nmat = len(group_bytes)
    gb = (ctypes.c_size_t * max(nmat, 1))(*[int(v) for v in group_bytes])
    st = load().sfx_hot_update(_stream(stream), L, int(G), int(K), _ptr(entered_bits), _ptr(left_bits),
                               _ptr(slot_of), _ptr(group_of), _ptr(copies), _ptr(ncopies), nmat,
                               gb if nmat > 0 else None, _ptr(src) if nmat > 0 else None,
                               _ptr(dst) if nmat > 0 else None)
    _check(st, "sfx_hot_update")


# ------------------------------------------------------------------------- calibration

def sfx_count_active(tok_bits, f, counts, stream=None):
    """counts [f] int32 += active tokens per neuron; tok_bits [B][ceil(f/32)]."""
    B = tok_bits.shape[0]
    _check(load().sfx_count_active(_stream(stream), B, int(f), _ptr(tok_bits), _ptr(counts)), "sfx_count_active")


def sfx_select_kth(values, k, out, ws=None, stream=None):
    """out[0] = k-th smallest (0-based) of the fp32 values, exact."""
    _need(values, torch.float32, "values")
    if ws is None:
        ws = workspace(load().sfx_select_kth_ws(), values.device)
    st = load().sfx_select_kth(_stream(stream), values.numel(), _ptr(values), int(k), _ptr(out), _ptr(ws),
                               ws.numel())
    _check(st, "sfx_select_kth")


def sfx_hot_first_order(counts, perm, group=None, ws=None, stream=None):
    """perm [f] int32 = hot-first neuron table from counts [f] (and group ids)."""
    f = counts.numel()
    if group is not None and ws is None:
        ws = workspace(load().sfx_hot_first_order_ws(f), counts.device)
    st = load().sfx_hot_first_order(_stream(stream), f, _ptr(counts), _ptr(group), _ptr(perm), _ptr(ws),
                                    ws.numel() if ws is not None else 0)
    _check(st, "sfx_hot_first_order")


def sfx_gather_rows(src, idx, dst, stream=None):
    """dst row r = src row idx[r]; rows along the first dimension."""
    if src.dtype != dst.dtype or src.shape[1:] != dst.shape[1:] or dst.shape[0] != idx.numel():
        raise ValueError("dst must be [len(idx)] + src row shape, same dtype")
    row_bytes = src[0].numel() * src.element_size()
    st = load().sfx_gather_rows(_stream(stream), dst.shape[0], src.shape[0], row_bytes, _ptr(src), _ptr(idx),
                                _ptr(dst))
    _check(st, "sfx_gather_rows")


# ------------------------------------------------------------------------- fused step

def sfx_ffn_step_ws(wdt: int, act: int, B: int, d: int, h: int, f: int) -> int:
    """Workspace bytes of the fused step, 0 when the shape is not built for it."""
    return load().sfx_ffn_step_ws(wdt, act, B, d, h, f)


TORCH_OF = {SFX_F16: torch.float16, SFX_BF16: torch.bfloat16}


def _check_layer(i: int, e: dict, B: int, d: int, h: int, f: int, wdt: int, act: int):
    """Raise unless layer entry `e` holds what the fused kernel reads and writes:
    the kernel cannot check device-resident descriptors, so a missing, short or
    misaligned buffer must be caught here."""
    W = (f + 31) // 32
    wt = TORCH_OF.get(wdt)
    if wt is None:
        raise TypeError("fused step: weights must be fp16 or bf16")
    need = ["x", "W1", "W2", "Wa", "Wd", "scores", "union_bits", "idx", "count", "hact", "y"]
    if act == SFX_REGLU:
        need.append("Wl")
    for n in need:
        if e.get(n) is None:
            raise ValueError(f"layer {i}: '{n}' is required")
    shapes = {"x": (B, d), "xp": (B, d), "W1": (h, d), "W2": (f, h), "Wa": (f, d), "Wl": (f, d), "Wd": (f, d)}
    for n, shp in shapes.items():
        t = e.get(n)
        if t is None:
            continue
        if t.dtype != wt:
            raise TypeError(f"layer {i}: '{n}' is {t.dtype}, expected {wt}")
        if tuple(t.shape) != shp:
            raise ValueError(f"layer {i}: '{n}' has shape {tuple(t.shape)}, expected {shp}")
    # outputs and the bias: dtype and at least the elements the kernel touches
    sizes = {"ba": (torch.float32, f), "scores": (torch.float32, B * f), "hact": (torch.float32, f * B),
             "y": (torch.float32, B * d), "tok_bits": ((torch.int32, torch.uint32), B * W),
             "union_bits": ((torch.int32, torch.uint32), W), "idx": ((torch.int32,), f),
             "count": ((torch.int32,), 1)}
    for n, (dt, numel) in sizes.items():
        t = e.get(n)
        if t is None:
            continue
        dts = dt if isinstance(dt, tuple) else (dt,)
        if t.dtype not in dts:
            raise TypeError(f"layer {i}: '{n}' is {t.dtype}, expected {dts}")
        if t.numel() < numel:
            raise ValueError(f"layer {i}: '{n}' holds {t.numel()} elements, needs >= {numel}")
    for n, t in e.items():
        if not isinstance(t, torch.Tensor):
            continue
        align = 4 if n in ("tok_bits", "union_bits", "idx", "count", "ba") else 16
        if t.data_ptr() % align != 0:
            raise ValueError(f"layer {i}: '{n}' is not {align}-byte aligned")


def layer_descriptors(layers, B: int, d: int, h: int, f: int, wdt: int, act, device=None) -> torch.Tensor:
    """Device array of `sfx_layer` descriptors.  `layers` is a list of dicts of
    tensors (x, W1, W2, Wa, ba, Wl, Wd, scores, tok_bits, union_bits, idx, count,
    hact, y) plus a float `threshold`; missing optional entries (ba, Wl for ReLU,
    tok_bits) are NULL.  Every entry is checked against the shape (B, d, h, f) first."""
    a = ACTS[act] if isinstance(act, str) else int(act)
    arr = (SfxLayer * len(layers))()
    for i, e in enumerate(layers):
        _check_layer(i, e, B, d, h, f, wdt, a)
        for name, _ in SfxLayer._fields_:
            if name in ("threshold", "reserved"):
                continue
            t = e.get(name)
            setattr(arr[i], name, _ptr(t).value if t is not None else None)
        arr[i].threshold = float(e["threshold"])
    raw = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
    return raw.to(device or "cuda")


def sfx_ffn_step(wdt: int, act, B: int, d: int, h: int, f: int, descs: torch.Tensor, ws, stream=None):
    """Every layer's predict -> compact -> up -> down in one launch."""
    L = descs.numel() // ctypes.sizeof(SfxLayer)
    a = ACTS[act] if isinstance(act, str) else int(act)
    p = (_ptr(descs), _ptr(ws))
    st = load().sfx_ffn_step(_stream(stream), wdt, a, B, d, h, f, L, p[0], p[1], ws.numel())
    _check(st, "sfx_ffn_step")


def sfx_ffn_pipeline_ws(wdt: int, act: int, B: int, d: int, h: int, f: int) -> int:
    """Workspace bytes of the Live Pipeline step, 0 when the shape is not built for it."""
    return load().sfx_ffn_pipeline_ws(wdt, act, B, d, h, f)


def sfx_ffn_pipeline(wdt: int, act, B: int, d: int, h: int, f: int, descs: torch.Tensor, ws, stream=None):
    """Every layer's step with layer l+1's predictor (on its input xp) overlapped with
    layer l's FFN, in one launch."""
    L = descs.numel() // ctypes.sizeof(SfxLayer)
    a = ACTS[act] if isinstance(act, str) else int(act)
    p = (_ptr(descs), _ptr(ws))
    st = load().sfx_ffn_pipeline(_stream(stream), wdt, a, B, d, h, f, L, p[0], p[1], ws.numel())
    _check(st, "sfx_ffn_pipeline")


STREAM_READ_OUT_WORDS = 16384


def sfx_stream_read(buf: torch.Tensor, out: torch.Tensor, stream=None):
    """Measurement helper: read `buf` once (the streaming-read ceiling)."""
    if out.numel() < STREAM_READ_OUT_WORDS or out.element_size() != 4:
        raise ValueError("out must hold 16384 32-bit words")
    st = load().sfx_stream_read(_stream(stream), _ptr(buf), buf.numel() * buf.element_size(), _ptr(out))
    _check(st, "sfx_stream_read")
