"""The seeded input generator (synth/): determinism, random access, formats
and the workload table.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

import synth
from synth import configs

HERE = os.path.dirname(os.path.abspath(__file__))


def test_deterministic_and_random_access():
    a = synth.normal_f32(0, 4, 10000, 0.02)
    assert (a == synth.normal_f32(0, 4, 10000, 0.02)).all()
    part = synth.normal_f32(0, 4, 1000, 0.02, start=3000)
    assert (part == a[3000:4000]).all()
    assert not (a == synth.normal_f32(1, 4, 10000, 0.02)).all()
    assert not (a == synth.normal_f32(0, 5, 10000, 0.02)).all()


def test_normal_moments():
    a = synth.normal_f32(0, 1, 1 << 20, 1.0).astype(np.float64)
    assert abs(a.mean()) < 5e-3
    assert abs(a.std() - 1.0) < 5e-3
    k = ((a - a.mean()) ** 4).mean() / a.var() ** 2
    assert abs(k - 2.9) < 0.05          # Irwin-Hall(12)
    assert np.abs(a).max() <= 6.0


def test_bf16_is_rounded_f32():
    f = synth.normal_f32(0, 7, 50000, 0.5)
    b = synth.normal_bf16(0, 7, 50000, 0.5)
    u = f.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert (b == rne).all()


def test_q8b32_blocks():
    q, s = synth.q8b32(0, 4, 64, 256, 0.02)
    assert q.dtype == np.int8 and s.shape == (64, 8)
    w = synth.normal_f32(0, 4, 64 * 256, 0.02).astype(np.float64).reshape(64, 8, 32)
    sc = s.view(np.float16).astype(np.float64)
    assert (np.abs(q) <= 127).all()
    amax = np.abs(w).max(-1)
    assert np.allclose(sc, amax / 127, rtol=2 ** -10)
    deq = q.reshape(64, 8, 32) * sc[..., None]
    assert (np.abs(deq - w) <= 0.5 * sc[..., None] * (1 + 1e-6) + 1e-7).all()
    # rows are independent of how they are batched
    q2, s2 = synth.q8b32(0, 4, 10, 256, 0.02, row0=20)
    assert (q2 == q[20:30]).all() and (s2 == s[20:30]).all()


def test_zipf_bias():
    b, r = synth.zipf_bias(0, 3, 256, 0.5)
    assert sorted(r.tolist()) == list(range(1, 257))
    assert np.allclose(b, -0.5 * np.log(r.astype(np.float64)), rtol=1e-6, atol=1e-7)


def test_skew_beta_matches_calibration():
    with open(os.path.join(HERE, "golden", "skew_beta.json")) as f:
        cal = json.load(f)
    assert configs.C5_BETA == cal["beta"]
    assert abs(cal["achieved_share"] - 0.30) <= 0.01


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_layer_shapes(name):
    cfg = configs.get(name)
    L = configs.make_layer(cfg)
    T, d, E, F = cfg["T"], cfg["d"], cfg["E"], cfg["F"]
    assert L["x"].shape == (T, d) and L["w_router"].shape == (E, d)
    g = L["gate"][0] if isinstance(L["gate"], tuple) else L["gate"]
    dn = L["down"][0] if isinstance(L["down"], tuple) else L["down"]
    assert g.shape == (E, F, d) and dn.shape == (E, d, F)
    if cfg["bias"] == "none":
        assert L["bias"] is None


def test_partial_experts_match_full():
    cfg = configs.get("c1")
    full = configs.make_layer(cfg)
    part = configs.make_layer(cfg, experts=[3, 17])
    for w in ("gate", "up", "down"):
        assert (part[w][[3, 17]] == full[w][[3, 17]]).all()
        assert (part[w][0] == 0).all()


def test_smaller_T_is_prefix():
    cfg = configs.get("c3")
    assert (configs.gen_x(cfg, 2)[:1] == configs.gen_x(cfg, 1)).all()


def test_lookahead_walk_statistics(orc):
    """The look-ahead workload's tokens: each row keeps the spread of the
    layer's activations, consecutive rows have correlation LOOKAHEAD_RHO, and
    the oracle's router on one token picks about three quarters of the next
    token's experts (the prediction rate the look-ahead stands in for)."""
    import numpy as np
    from synth import configs
    cfg = configs.get("c2")
    T = 160
    x = configs.gen_x_walk(cfg, T, configs.LOOKAHEAD_RHO)
    assert x.dtype == np.uint16 and x.shape == (T, cfg["d"])
    f = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(f.std(axis=1) / cfg["x_sigma"] - 1.0) < 0.05)
    corr = [np.corrcoef(f[t], f[t + 1])[0, 1] for t in range(T - 1)]
    assert abs(np.mean(corr) - configs.LOOKAHEAD_RHO) < 0.005
    _, idx, _ = orc.route(cfg, x, configs.gen_router(cfg), configs.gen_bias(cfg))
    hit = np.mean([len(set(idx[t]) & set(idx[t + 1])) / cfg["k"] for t in range(T - 1)])
    assert 0.65 < hit < 0.85, hit
    # the f32 form is the same walk before rounding
    xf = configs.gen_x_walk(configs.get("c1"), 8, 0.5)
    assert xf.dtype == np.float32 and xf.shape == (8, 512)
