"""The synthetic workloads hit the retention targets their recipes name,
and no unit sits so close to the threshold that float64 rounding could
flip it (no GPU)."""
import numpy as np
import pytest

import oracle
import workloads as W


def _frac(cfg, w):
    p = oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, w)
    return sum(L.r for L in p.layers) / sum(L.n for L in p.layers)


@pytest.mark.parametrize("name,target", [("gdn", 0.45), ("kda", 0.38)])
def test_w_max_is_integer_nearest_target(name, target):
    cfg = W.CONFIGS[name]()
    errs = {w: abs(_frac(cfg, w) - target) for w in range(2, 64)}
    assert min(errs, key=errs.get) == cfg.w_max


def test_mixed_layers_retain_exactly_their_slow_units():
    cfg = W.mixed()
    p = oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    fr = [L.r / L.n for L in p.layers]
    assert fr == pytest.approx(cfg.extra["slow_fraction"], abs=0)
    assert 0.18 <= min(fr) and max(fr) <= 0.82
    assert [L.kind for L in p.layers] == [W.GDN if l % 2 == 0 else W.KDA for l in range(27)]


@pytest.mark.parametrize("name", ["tiny_kda", "gdn", "kda", "mixed"])
def test_no_near_ties(name):
    cfg = W.CONFIGS[name]()
    p = oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    gap = min(np.min(np.abs(L.H_s - cfg.w_max)) / cfg.w_max for L in p.layers)
    assert gap > 1e-9


def test_kda_static_decay_median_near_pages():
    # Median one-step static decay 0.471 for Kimi-Linear (dasc §3.3).
    cfg = W.kda()
    g = np.concatenate([oracle.gate_log_decay(L.A_log, L.dt_bias, cfg.a_s) for L in cfg.layers])
    assert abs(float(np.median(np.exp(g))) - 0.471) < 0.01


def test_refresh_inputs_shapes_and_norms():
    cfg = W.tiny_kda()
    Wn = W.windows(cfg)
    x = W.refresh_inputs(cfg, Wn)
    T = int(Wn.sum())
    assert x.k.shape == (T, 64) and x.v.shape == (T, 64) and x.a.shape == (T, 64)
    assert x.beta.shape == (T, 4) and x.tok_off.tolist() == [0, 8, 16]
    n = np.linalg.norm(x.k.float().reshape(T, 4, 16).numpy(), axis=-1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert float(x.beta.min()) > 0 and float(x.beta.max()) < 1


def test_mixed_windows_range():
    w = W.windows(W.mixed())
    assert w.min() >= 64 and w.max() <= 1024 and len(w) == 64
