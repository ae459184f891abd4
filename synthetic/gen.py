"""Seeded generators for one FFN layer and its token stream.

The recipe reproduces the structure the pages measure, on seeded random data:

* power-law activation (PowerInfer, Method, Insight 1): the activated branch gets
  a bias b_i = Phi^-1(p_i) where p_i follows a clipped Zipf(1.1) profile scaled to
  the configured mean density; rows are unit-norm Gaussian, so for x ~ N(0, I)
  the pre-activation is N(b_i, 1) and neuron i fires with probability p_i;
* temporal locality of successive tokens (KAIROX, Key observations, observation 3):
  AR(1) tokens x_t = 0.9 x_{t-1} + sqrt(0.19) xi_t with unit stationary variance;
* co-activated groups of 32 (KAIROX, Core method, items 1 and 3): the predictor's
  output rows of one group share a common direction, r_i = sqrt(0.9) u_grp +
  sqrt(0.1) v_i, so the group's scores move together;
* a predictor that fires with the same power law (PowerInfer, Method, Insight 1:
  the predictor predicts that activation).  With W1 ~ N(0, 1/d) and unit-variance
  tokens every hidden unit is relu of a standard normal: mean mu = 1/sqrt(2 pi),
  standard deviation sd = sqrt(1/2 - 1/(2 pi)).  Row i of W2 is its random part r_i
  (N(0, 1/h) entries, row mean removed) plus m_i / (mu h) on every entry, so its
  score is about N(m_i, sd^2); m_i = sd Phi^-1(p_i) and the threshold 0 give
  P(score_i >= 0) = p_i.  Configuration C1 keeps a plain N(0, 1/h) W2 (its
  recipe states one): scores N(0, 1/2), threshold Phi^-1(1 - density) / sqrt(2);
* storage order.  `order="hot_first"` (the default) stores slot i = the neuron of
  Zipf rank i+1, planted groups as aligned blocks of 32: the layer as offline
  placement would leave it (PowerInfer, Method, neuron table; KAIROX, Core method,
  item 3).  `order="raw"` stores the same neurons in a seeded random order, as a
  model ships before calibration: `perm` of the hot-first layer maps its slots to
  the raw layer's (hot_first row r = raw row perm[r]), and `group` gives each raw
  slot's planted group, the output of the offline grouping step.

The thresholds here are closed forms; a calibration pass replaces them with the
(1 - density)-quantile of measured scores.  Nothing here evaluates the predictor,
the gate or the FFN.
"""
import hashlib
import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch
from scipy.special import ndtr, ndtri

from .configs import FFNConfig

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
CHUNK_ROWS = 2048          # rows drawn per generator call (fixed: part of the recipe)
AR1_RHO = 0.9
PLANT_RHO = 0.9
ZIPF_S = 1.1
ZIPF_PMAX = 0.99


def seed_for(cfg_name: str, layer: int, tag: str) -> int:
    """63-bit seed of tensor `tag` of layer `layer` in configuration `cfg_name`."""
    dig = hashlib.sha256(f"sfx/{cfg_name}/{layer}/{tag}".encode()).digest()
    return int.from_bytes(dig[:8], "little") & ((1 << 63) - 1)


def _rng(cfg_name: str, layer: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(cfg_name, layer, tag))
    return g


def zipf_profile(f: int, density: float, s: float = ZIPF_S, pmax: float = ZIPF_PMAX) -> np.ndarray:
    """p_r = min(pmax, c * r^-s) for ranks r = 1..f, c chosen so that mean(p) = density."""
    r = np.arange(1, f + 1, dtype=np.float64)
    base = r ** (-s)

    def mean_p(c):
        return np.minimum(pmax, c * base).mean()

    if density >= pmax:
        raise ValueError("density must be below the clip level")
    lo, hi = 0.0, 1.0
    while mean_p(hi) < density:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mean_p(mid) < density:
            lo = mid
        else:
            hi = mid
    return np.minimum(pmax, hi * base)


RELU_MEAN = 1.0 / math.sqrt(2.0 * math.pi)                 # E relu(z), z ~ N(0, 1)
RELU_SD = math.sqrt(0.5 - 1.0 / (2.0 * math.pi))           # sd of relu(z)


def threshold_for(density: float) -> float:
    """Closed-form threshold of the plain N(0, 1/h) predictor (scores N(0, 1/2))."""
    return float(np.float32(ndtri(1.0 - density) / math.sqrt(2.0)))


def layer_threshold(cfg: FFNConfig) -> float:
    """Closed-form per-layer threshold of the configuration's predictor."""
    return 0.0 if cfg.pred_profile == "zipf" else threshold_for(cfg.density)


def threshold_for_share(cfg: FFNConfig, share: float) -> float:
    """Closed-form threshold at which about `share` of the neurons are active per
    token (tests that need long or short active lists): for the power-law predictor
    the t with mean_i Phi(Phi^-1(p_i) - t / sd) = share (bisection); for the plain
    predictor Phi^-1(1 - share) / sqrt(2)."""
    if cfg.pred_profile != "zipf":
        return threshold_for(share)
    z = ndtri(zipf_profile(cfg.f, cfg.density))
    lo, hi = -20.0, 20.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if ndtr(z - mid / RELU_SD).mean() > share:
            lo = mid
        else:
            hi = mid
    return float(np.float32(0.5 * (lo + hi)))


def _randn(g: torch.Generator, rows: int, cols: int, device) -> torch.Tensor:
    """fp64 N(0,1) matrix drawn in fixed row chunks."""
    out = torch.empty(rows, cols, dtype=torch.float64, device=device)
    for r0 in range(0, rows, CHUNK_ROWS):
        r1 = min(rows, r0 + CHUNK_ROWS)
        out[r0:r1] = torch.randn(r1 - r0, cols, generator=g, dtype=torch.float64, device=device)
    return out


def _unit_rows(g, rows, cols, device) -> torch.Tensor:
    w = _randn(g, rows, cols, device)
    return w / w.norm(dim=1, keepdim=True)


def quantize_q4(w: torch.Tensor):
    """Symmetric int4, group 32 along a row, fp16 scales.

    Per group: s = fp16(max|w| / 7); q = clamp(round_half_even(w / s), -8, 7), q = 0
    where s = 0.  Packed two's-complement nibbles, column 2c in the low nibble of
    byte c.  Returns (q uint8 [rows][cols/2], s float16 [rows][cols/32]).
    """
    rows, cols = w.shape
    assert cols % 32 == 0
    wg = w.reshape(rows, cols // 32, 32)
    s16 = (wg.abs().amax(dim=2) / 7.0).to(torch.float16)
    s = s16.to(torch.float64).unsqueeze(2)
    q = torch.where(s > 0, torch.round(wg / torch.where(s > 0, s, torch.ones_like(s))),
                    torch.zeros_like(wg))
    q = q.clamp(-8, 7).to(torch.int16).reshape(rows, cols)
    nib = (q & 0xF).to(torch.uint8)
    packed = nib[:, 0::2] | (nib[:, 1::2] << 4)
    return packed.contiguous(), s16.contiguous()


@dataclass
class Layer:
    cfg: FFNConfig
    index: int
    W1: torch.Tensor               # [h][d]  predictor layer 1 (pdtype; int4: uint8 [h][d/2])
    W2: torch.Tensor               # [f][h]  predictor layer 2 (pdtype; int4: uint8 [f][h/2])
    Wa: torch.Tensor               # [f][d]  activated branch (row = neuron); q4: uint8 [f][d/2]
    ba: torch.Tensor               # [f]     fp32 bias of the activated branch
    Wd: torch.Tensor               # [f][d]  down projection, neuron-major; q4: uint8 [f][d/2]
    threshold: float
    perm: torch.Tensor             # [f]     int32 neuron table: slot -> raw-order slot
    p: np.ndarray                  # [f]     Zipf activation probability per slot
    group: Optional[torch.Tensor] = None   # [f] int32 planted group of each slot (planted configs)
    Wl: Optional[torch.Tensor] = None      # [f][d] ReGLU linear branch
    Wa_s: Optional[torch.Tensor] = None    # q4 scales [f][d/32] fp16
    Wl_s: Optional[torch.Tensor] = None
    Wd_s: Optional[torch.Tensor] = None
    W1_s: Optional[torch.Tensor] = None    # int4 predictor scales [h][d/32], [f][h/32] fp16
    W2_s: Optional[torch.Tensor] = None

    def tensors(self) -> Dict[str, torch.Tensor]:
        out = {}
        for k in ("W1", "W2", "Wa", "ba", "Wd", "perm", "Wl", "Wa_s", "Wl_s", "Wd_s", "W1_s", "W2_s"):
            v = getattr(self, k)
            if v is not None:
                out[k] = v
        return out


def make_layer(cfg: FFNConfig, layer: int, device="cpu", order: str = "hot_first") -> Layer:
    if order not in ("hot_first", "raw"):
        raise ValueError("order is 'hot_first' or 'raw'")
    d, f, h = cfg.d, cfg.f, cfg.h
    pdt = TORCH_DTYPE[cfg.pdtype]
    name = cfg.name
    p = zipf_profile(f, cfg.density)

    W1 = _randn(_rng(name, layer, "W1", device), h, d, device) / math.sqrt(d)
    if cfg.planted:
        groups = (f + 31) // 32
        u = _randn(_rng(name, layer, "blk", device), groups, h, device)
        v = _randn(_rng(name, layer, "W2", device), f, h, device)
        grp = torch.arange(f, device=device) // 32
        W2 = (math.sqrt(PLANT_RHO) * u[grp] + math.sqrt(1.0 - PLANT_RHO) * v) / math.sqrt(h)
        del u, v
    else:
        W2 = _randn(_rng(name, layer, "W2", device), f, h, device) / math.sqrt(h)
    if cfg.pred_profile == "zipf":
        m = torch.from_numpy(RELU_SD * ndtri(p)).to(device)
        W2 = W2 - W2.mean(dim=1, keepdim=True) + (m / (RELU_MEAN * h)).unsqueeze(1)
    W1_s = W2_s = None
    if cfg.pred_q4:
        W1, W1_s = quantize_q4(W1)
        W2, W2_s = quantize_q4(W2)
    else:
        W1, W2 = W1.to(pdt), W2.to(pdt)

    ba = torch.from_numpy(ndtri(p)).to(torch.float32).to(device)

    Wa64 = _unit_rows(_rng(name, layer, "Wa", device), f, d, device)
    Wd64 = _randn(_rng(name, layer, "Wd", device), f, d, device) / math.sqrt(f)
    Wl64 = _unit_rows(_rng(name, layer, "Wl", device), f, d, device) if cfg.act == "reglu" else None

    Wa_s = Wl_s = Wd_s = None
    if cfg.wdtype == "q4":
        Wa, Wa_s = quantize_q4(Wa64)
        Wd, Wd_s = quantize_q4(Wd64)
        Wl = None
        if Wl64 is not None:
            Wl, Wl_s = quantize_q4(Wl64)
    else:
        wdt = TORCH_DTYPE[cfg.wdtype]
        Wa, Wd = Wa64.to(wdt), Wd64.to(wdt)
        Wl = Wl64.to(wdt) if Wl64 is not None else None
    del Wa64, Wd64, Wl64

    # raw order: raw slot j holds hot-first slot sigma[j]; so hot-first slot r is raw
    # slot perm[r] with perm = sigma^-1
    sigma = torch.randperm(f, generator=_rng(name, layer, "perm", "cpu"))
    group = (torch.arange(f, dtype=torch.int32) // 32) if cfg.planted else None
    if order == "hot_first":
        perm = torch.argsort(sigma).to(torch.int32).to(device)
        return Layer(cfg=cfg, index=layer, W1=W1, W2=W2, Wa=Wa, ba=ba, Wd=Wd,
                     threshold=layer_threshold(cfg), perm=perm, p=p,
                     group=group.to(device) if group is not None else None,
                     Wl=Wl, Wa_s=Wa_s, Wl_s=Wl_s, Wd_s=Wd_s, W1_s=W1_s, W2_s=W2_s)
    sd = sigma.to(device)

    def shuf(t):
        return None if t is None else t.index_select(0, sd).contiguous()

    return Layer(cfg=cfg, index=layer, W1=W1, W2=shuf(W2), Wa=shuf(Wa), ba=shuf(ba), Wd=shuf(Wd),
                 threshold=layer_threshold(cfg), perm=torch.arange(f, dtype=torch.int32, device=device),
                 p=p[sigma.numpy()], group=shuf(group.to(device)) if group is not None else None,
                 Wl=shuf(Wl), Wa_s=shuf(Wa_s), Wl_s=shuf(Wl_s), Wd_s=shuf(Wd_s), W1_s=W1_s, W2_s=shuf(W2_s))


def make_tokens(cfg: FFNConfig, layer: int, steps: int, B: int, device="cpu", tag: str = "x") -> torch.Tensor:
    """Token stream [steps][B][d] in the predictor dtype: B independent streams,
    i.i.d. N(0, I) or AR(1) with lag-1 correlation 0.9 and unit variance."""
    g = _rng(cfg.name, layer, f"{tag}/B{B}", device)
    xi = torch.randn(steps, B, cfg.d, generator=g, dtype=torch.float64, device=device)
    if cfg.x_process == "ar1":
        x = torch.empty_like(xi)
        x[0] = xi[0]
        c = math.sqrt(1.0 - AR1_RHO * AR1_RHO)
        for t in range(1, steps):
            x[t] = AR1_RHO * x[t - 1] + c * xi[t]
    else:
        x = xi
    return x.to(TORCH_DTYPE[cfg.pdtype]).contiguous()


LAYER_COS = 0.98


def make_layer_chain(cfg: FFNConfig, layers: int, steps: int, B: int, device="cpu", cos: float = LAYER_COS,
                     tag: str = "chain"):
    """FFN inputs of consecutive layers within each decode step, for the Live
    Pipeline: layer 0 follows the configuration's token process (AR(1) over steps),
    and x_{l+1} = cos x_l + sqrt(1 - cos^2) xi_l with fresh N(0, I) noise, so
    adjacent layers' inputs have cosine similarity ~cos (KAIROX, Key observations,
    observation 1: about 0.98) and unit variance.  Returns a list of `layers`
    tensors [steps][B][d] in the predictor dtype."""
    x = make_tokens(cfg, 0, steps, B, device=device, tag=f"{tag}/x0").to(torch.float64)
    out = [x.to(TORCH_DTYPE[cfg.pdtype]).contiguous()]
    c = math.sqrt(1.0 - cos * cos)
    for l in range(1, layers):
        g = _rng(cfg.name, l, f"{tag}/B{B}", device)
        xi = torch.randn(steps, B, cfg.d, generator=g, dtype=torch.float64, device=device)
        x = cos * x + c * xi
        out.append(x.to(TORCH_DTYPE[cfg.pdtype]).contiguous())
    return out


def storage_numpy(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a tensor as a host numpy array (bf16 as its uint16 bit pattern)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
