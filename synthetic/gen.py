"""Seeded generators for one FFN layer and its token stream.

The recipe reproduces the structure the pages measure, on seeded random data:

* power-law activation (PowerInfer, Method, Insight 1): the activated branch gets
  a bias b_i = Phi^-1(p_i) where p_i follows a clipped Zipf(1.1) profile scaled to
  the configured mean density; rows are unit-norm Gaussian, so for x ~ N(0, I)
  the pre-activation is N(b_i, 1) and neuron i fires with probability p_i;
* temporal locality of successive tokens (KAIROX, Key observations, observation 3):
  AR(1) tokens x_t = 0.9 x_{t-1} + sqrt(0.19) xi_t with unit stationary variance;
* co-activated groups of 32 (KAIROX, Core method, items 1 and 3): the predictor's
  output rows of one group share a common direction, W2_i = sqrt(0.9) u_grp +
  sqrt(0.1) v_i, so the group's scores move together;
* hot-first storage (PowerInfer, Method, neuron table; KAIROX, Core method, item 3):
  slot i holds the neuron of Zipf rank i+1, so groups of 32 consecutive slots are
  contiguous and ordered by frequency.  `perm` is the neuron table (slot -> id).

The per-layer threshold is set for the configured density from the score
distribution in closed form: with W1 ~ N(0, 1/d), W2 ~ N(0, 1/h) and unit-variance
tokens, a score is N(0, 1/2), so t = Phi^-1(1 - density) / sqrt(2).

Nothing here evaluates the predictor, the gate or the FFN.
"""
import hashlib
import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch
from scipy.special import ndtri

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


def threshold_for(density: float) -> float:
    """Per-layer threshold for the configured density (closed form, see module doc)."""
    return float(np.float32(ndtri(1.0 - density) / math.sqrt(2.0)))


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
    perm: torch.Tensor             # [f]     int32 neuron table: slot -> original neuron id
    p: np.ndarray                  # [f]     Zipf activation probability per slot
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


def make_layer(cfg: FFNConfig, layer: int, device="cpu") -> Layer:
    d, f, h = cfg.d, cfg.f, cfg.h
    pdt = TORCH_DTYPE[cfg.pdtype]
    name = cfg.name

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
    W1_s = W2_s = None
    if cfg.pred_q4:
        W1, W1_s = quantize_q4(W1)
        W2, W2_s = quantize_q4(W2)
    else:
        W1, W2 = W1.to(pdt), W2.to(pdt)

    p = zipf_profile(f, cfg.density)
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

    g = _rng(name, layer, "perm", "cpu")
    perm = torch.randperm(f, generator=g).to(torch.int32).to(device)
    return Layer(cfg=cfg, index=layer, W1=W1, W2=W2, Wa=Wa, ba=ba, Wd=Wd,
                 threshold=threshold_for(cfg.density), perm=perm, p=p,
                 Wl=Wl, Wa_s=Wa_s, Wl_s=Wl_s, Wd_s=Wd_s, W1_s=W1_s, W2_s=W2_s)


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
