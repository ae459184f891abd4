"""Checks of the seeded input recipe (the generator holds none of the step's
arithmetic; the oracle is used here only to measure what the data produces)."""
import math

import numpy as np
import pytest
import torch

import synthetic as S
from oracle import sfx_oracle as O


def test_seed_is_stable_and_distinct():
    a = S.seed_for("C2", 3, "W1")
    assert a == S.seed_for("C2", 3, "W1")
    assert a != S.seed_for("C2", 4, "W1") and a != S.seed_for("C2", 3, "W2")
    assert 0 <= a < 2 ** 63


@pytest.mark.parametrize("f,rho", [(1024, 0.10), (16384, 0.08), (11008, 0.12), (28672, 0.07), (32768, 0.06)])
def test_zipf_profile_mean_and_clip(f, rho):
    p = S.zipf_profile(f, rho)
    assert abs(p.mean() - rho) < 1e-9
    assert p.max() == pytest.approx(0.99)
    assert np.all(np.diff(p) <= 0)                    # hot-first: rank order
    clipped = np.mean(p >= 0.99)
    assert 0.0 < clipped < 0.05


def test_threshold_closed_form():
    # Phi^-1(0.9) / sqrt(2) for 10% density
    assert S.threshold_for(0.10) == pytest.approx(1.2815515655446004 / math.sqrt(2), rel=1e-6)


def _small(name, **kw):
    return S.scaled(S.CONFIGS[name], **kw)


def test_layer_shapes_and_dtypes():
    cfg = _small("C3", d=256, f=320, h=64)
    L = S.make_layer(cfg, 0)
    assert L.W1.shape == (64, 256) and L.W1.dtype == torch.bfloat16
    assert L.W2.shape == (320, 64) and L.Wa.shape == (320, 256) and L.Wl.shape == (320, 256)
    assert L.Wd.shape == (320, 256) and L.ba.dtype == torch.float32
    assert sorted(L.perm.tolist()) == list(range(320))
    cfg4 = _small("C4", d=256, f=128, h=64)
    L4 = S.make_layer(cfg4, 0)
    assert L4.Wa.dtype == torch.uint8 and L4.Wa.shape == (128, 128) and L4.Wa_s.shape == (128, 8)
    assert L4.W1.dtype == torch.float16


def test_rows_unit_norm_and_down_scale():
    cfg = _small("C1", f=512)
    L = S.make_layer(cfg, 0)
    n = L.Wa.double().norm(dim=1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-6)
    sd = L.Wd.double().std().item()
    assert sd == pytest.approx(1 / math.sqrt(512), rel=0.05)


def test_layers_are_deterministic():
    cfg = _small("C2", d=64, f=128, h=32)
    a, b = S.make_layer(cfg, 1), S.make_layer(cfg, 1)
    assert torch.equal(a.W2, b.W2) and torch.equal(a.Wa, b.Wa)
    c = S.make_layer(cfg, 2)
    assert not torch.equal(a.W2, c.W2)


def test_ar1_lag1_correlation_and_variance():
    cfg = _small("C2", d=512)
    x = S.make_tokens(cfg, 0, 400, 2).double()
    a, b = x[:-1].reshape(-1), x[1:].reshape(-1)
    r = torch.corrcoef(torch.stack([a, b]))[0, 1].item()
    assert r == pytest.approx(0.9, abs=0.02)
    assert x.var().item() == pytest.approx(1.0, abs=0.05)


def test_q4_roundtrip_within_half_step():
    """The quantiser's codes, decoded by the oracle, are within s/2 of the source."""
    g = torch.Generator().manual_seed(5)
    w = torch.randn(16, 256, generator=g, dtype=torch.float64) * 0.03
    q, s = S.quantize_q4(w)
    back = O.dequant_q4(q.numpy(), s.numpy())
    step = np.repeat(s.numpy().astype(np.float64), 32, axis=1)
    assert np.all(np.abs(back - w.numpy()) <= step / 2 + 1e-12)
    assert q.shape == (16, 128) and s.shape == (16, 8)


def test_true_relu_density_follows_zipf():
    """P(z_i > 0) = p_i: with unit-norm rows and N(0, I) tokens the exact-ReLU density
    matches the configured mean."""
    cfg = _small("C1", f=2048, steps=64)
    L = S.make_layer(cfg, 0)
    x = S.make_tokens(cfg, 0, 64, 1)[:, 0].double().numpy()
    z = x @ L.Wa.double().numpy().T + L.ba.double().numpy()[None, :]
    dens = (z > 0).mean()
    assert dens == pytest.approx(cfg.density, abs=0.01)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C5"])
def test_predictor_density_near_target(name):
    """The closed-form threshold gives a mean per-token active share near the target
    (measured with the oracle's predictor on generated data; planted groups make a
    single layer's share noisy, so it is averaged over layers)."""
    cfg = _small(name, d=512, f=4096, h=256) if name != "C1" else S.CONFIGS["C1"]
    layers = 6 if cfg.planted else 2
    dens = []
    for li in range(layers):
        L = S.make_layer(cfg, li)
        x = S.make_tokens(cfg, li, 32, 1)[:, 0]
        sc = O.predict(O.decode(S.storage_numpy(x), cfg.pdtype),
                       O.decode(S.storage_numpy(L.W1), cfg.pdtype), O.decode(S.storage_numpy(L.W2), cfg.pdtype))
        dens.append((sc >= L.threshold).mean())
    assert np.mean(dens) == pytest.approx(cfg.density, rel=0.2)


def test_planted_groups_coactivate():
    """With planted groups, active neurons cluster in groups of 32: far fewer groups
    are touched than for independent neurons at the same density."""
    cfg = _small("C5", d=512, f=4096, h=256)
    L = S.make_layer(cfg, 0)
    x = S.make_tokens(cfg, 0, 16, 1)[:, 0]
    sc = O.predict(S.storage_numpy(x).astype(np.float64), O.decode(S.storage_numpy(L.W1), "f16"),
                   O.decode(S.storage_numpy(L.W2), "f16"))
    m = sc >= L.threshold
    grp_active = m.reshape(m.shape[0], -1, 32).any(axis=2).mean()
    indep = 1 - (1 - m.mean()) ** 32
    assert grp_active < 0.6 * indep


def test_layer_chain_cosine_and_variance():
    """Adjacent layers' inputs have cosine ~0.98 and unit variance; layer 0 keeps
    the AR(1) lag-1 correlation of the token process."""
    cfg = S.scaled(S.CONFIGS["C2"], name="chain", d=4096, f=64, h=16)
    xs = S.make_layer_chain(cfg, 3, 6, 2)
    assert len(xs) == 3 and tuple(xs[1].shape) == (6, 2, 4096)
    a, b = xs[0].double(), xs[1].double()
    cos = (a * b).sum(-1) / (a.norm(dim=-1) * b.norm(dim=-1))
    assert abs(float(cos.mean()) - S.LAYER_COS) < 0.005
    assert abs(float(xs[2].double().var()) - 1.0) < 0.03
    lag = (xs[0][1:].double() * xs[0][:-1].double()).mean()
    assert abs(float(lag) - 0.9) < 0.03
    again = S.make_layer_chain(cfg, 3, 6, 2)
    assert all(torch.equal(u, v) for u, v in zip(xs, again))


@pytest.mark.parametrize("name,share", [("C2", 0.2), ("C5", 0.3), ("C1", 0.2)])
def test_threshold_for_share(name, share):
    """The closed-form threshold for a target per-token share gives about that share
    with the oracle's predictor on generated data."""
    cfg = _small(name, d=512, f=4096, h=256) if name != "C1" else S.CONFIGS["C1"]
    t = S.threshold_for_share(cfg, share)
    dens = []
    for li in range(4):
        L = S.make_layer(cfg, li)
        x = S.make_tokens(cfg, li, 32, 1)[:, 0]
        sc = O.predict(O.decode(S.storage_numpy(x), cfg.pdtype),
                       O.decode(S.storage_numpy(L.W1), cfg.pdtype), O.decode(S.storage_numpy(L.W2), cfg.pdtype))
        dens.append((sc >= t).mean())
    assert np.mean(dens) == pytest.approx(share, rel=0.2)
    assert S.threshold_for_share(cfg, cfg.density) == pytest.approx(S.layer_threshold(cfg), abs=1e-3)


def test_raw_order_is_a_shuffle_of_hot_first():
    """order='raw' stores the hot-first layer's rows in a seeded random order, and
    the hot-first layer's perm maps its slots to the raw slots."""
    cfg = _small("C3", d=256, f=320, h=64)
    hf = S.make_layer(cfg, 0)
    raw = S.make_layer(cfg, 0, order="raw")
    perm = hf.perm.long()
    assert sorted(perm.tolist()) == list(range(320)) and not torch.equal(perm, torch.arange(320))
    for k in ("W2", "Wa", "Wl", "Wd", "ba"):
        assert torch.equal(getattr(raw, k)[perm], getattr(hf, k)), k
    assert torch.equal(raw.group[perm], hf.group) and torch.equal(hf.group, torch.arange(320) // 32)
    assert np.array_equal(raw.p[perm.numpy()], hf.p)
    assert torch.equal(hf.W1, raw.W1) and raw.threshold == hf.threshold
