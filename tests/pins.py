"""The oracle's pins: checks that tie each oracle function to something other
than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` when
the oracle disagrees with the pinned fact.  ``tests/test_oracle_pins.py``
runs them on the real oracle; ``tests/test_oracle_mutants.py`` runs them on
builds with a planted mistake and requires every mistake to trip one.

Sources of the facts (none of them the oracle's own formula):
* brute-force enumeration of every k-subset (selection and tie-break);
* 50-digit ``decimal`` evaluation of the scores, rounded exactly to fp32;
* exact rational arithmetic and integer bit manipulation for the formats;
* numpy float16 decoding, numpy fp64 matmul, Python's sort;
* closed forms and invariants of the layer (weights sum to the scale, one
  expert with top-1 is a dense SwiGLU, identity weights, exact doublings).

The formulas pinned are those of the pages: the router scores with sigmoid
(GLM-5.2, Hy3) or sqrt(softplus) and the 1.5 scale (DeepSeek Flash), top-8 /
top-6 ("256 experts, 512 lines", sections "Why GLM-5.2 in an engine built
for DeepSeek" and "The constant that always said 256"); the per-expert bias
(NeutronStar README, main branch, Hy3 paragraph); an always-on shared
expert; gate/up and down projections (NeutronStar README, "GLM-5.2 CUDA port"
and the batch expert-tile bug note).
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np

import exact


def _cfg(**kw):
    base = dict(T=1, d=32, E=4, k=2, F=32, Fs=32, n_shared=0, score="sigmoid", scale=1.0,
                act="f32", w="f32")
    base.update(kw)
    return base


# ---------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------

def pin_f16_decode_all_patterns(orc):
    """fp16 scale decoding equals numpy's float16 for all 65536 bit patterns."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([orc.f16_to_f32(int(b)) for b in bits], np.float32)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), "fp16 decode differs at %s" % bits[~same][:8]


def pin_bf16_rounding(orc):
    """bf16 round-to-nearest-even from fp64 equals exact integer rounding."""
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000)))
    # halfway cases (ties to even), values just off halfway, subnormals, overflow, zeros
    for m in range(128, 256):
        base = float(m) / 128.0
        vals += [base + 1.0 / 256.0, base + 1.0 / 256.0 + 2.0 ** -40, base + 1.0 / 256.0 - 2.0 ** -40]
    vals += [2.0 ** -130 * 1.5, 2.0 ** -133 * 0.5, 2.0 ** -133 * 0.75, 2.0 ** -134, 2.0 ** -140,
             3.0e38, 3.3895313892515355e38, 3.39e38, 1e300, -1e300, 0.0, -0.0, -2.0 ** -133 * 1.5]
    for v in vals:
        want = exact.bf16_round_bits(v)
        got = orc.bf16_from_f64(v)
        assert got == want, "bf16(%r): oracle %#06x, exact %#06x" % (v, got, want)


# ---------------------------------------------------------------------------
# Scores
# ---------------------------------------------------------------------------

def pin_score_closed_forms(orc):
    assert orc.score("sigmoid", 0.0) == np.float32(0.5)
    assert orc.score("sigmoid", -104.0) == 0.0  # 1/(1+e^104) < 2^-150
    assert orc.score("sigmoid", 30.0) == np.float32(1.0)
    # sqrt(softplus(0)) = sqrt(ln 2) = 0.83255461115769...
    assert orc.score("sqrt_softplus", 0.0) == exact.round_f32(Fraction("0.83255461115769775635"))
    assert orc.score("sqrt_softplus", -210.0) == 0.0  # e^-105 < 2^-150
    assert orc.score("sqrt_softplus", 100.0) == exact.round_f32(Fraction(10))  # sqrt(100 + 4e-44)


def pin_score_correctly_rounded(orc):
    """Scores equal the 50-digit value rounded to fp32 on >= 1 - 1e-6 of a sweep."""
    rng = np.random.default_rng(2)
    logits = np.concatenate([rng.standard_normal(3000), rng.standard_normal(1500) * 8.0,
                             rng.uniform(-120, 60, 500), np.linspace(-3, 3, 1000)]).astype(np.float32)
    bad = 0
    for kind in ("sigmoid", "sqrt_softplus"):
        for l in logits:
            got = np.float32(orc.score(kind, float(l)))
            want = exact.score_f32(kind, float(l))
            bad += exact.f32_bits(got) != exact.f32_bits(want)
    assert bad <= 0, "%d of %d scores not correctly rounded" % (bad, 2 * len(logits))


def pin_score_monotone(orc):
    xs = np.linspace(-60, 60, 4001).astype(np.float32)
    for kind in ("sigmoid", "sqrt_softplus"):
        s = np.array([orc.score(kind, float(v)) for v in xs])
        assert (np.diff(s) >= 0).all(), kind
        assert s[-1] > s[0]


# ---------------------------------------------------------------------------
# Selection (top-k with the tie-break)
# ---------------------------------------------------------------------------

def _brute_select(keys, k):
    """The unique k-subset every member of which precedes every non-member, in
    rank order; precedence: larger key, then lower index (exact fp32 compare)."""
    E = len(keys)

    def prec(a, b):
        return keys[a] > keys[b] or (keys[a] == keys[b] and a < b)

    found = []
    for sub in itertools.combinations(range(E), k):
        rest = [b for b in range(E) if b not in sub]
        if all(prec(a, b) for a in sub for b in rest):
            found.append(sub)
    assert len(found) == 1, "dominance subset not unique: %s" % found
    return sorted(found[0], key=lambda a: (-float(keys[a]), a))


def _keys(kind, logits, bias):
    s = [exact.score_f32(kind, float(l)) for l in logits]
    if bias is None:
        return s
    return [np.float32(si + np.float32(b)) for si, b in zip(s, bias)]


def pin_topk_bruteforce(orc):
    """Every logit vector in {-1,0,1}^E (E <= 6; a sample for E = 7, 8), every k."""
    rng = np.random.default_rng(3)
    for E in range(1, 9):
        vecs = np.array(list(itertools.product([-1.0, 0.0, 1.0], repeat=E)), np.float32)
        if E >= 7:
            vecs = vecs[rng.choice(len(vecs), 150, replace=False)]
        for kind in ("sigmoid", "sqrt_softplus"):
            biases = [None]
            if kind == "sigmoid" and E <= 6:
                biases.append(np.array([0.25 * ((e * 7 + 3) % 2) for e in range(E)], np.float32))
            for bias in biases:
                key_rows = [_keys(kind, v, bias) for v in vecs]
                for k in range(1, E + 1):
                    cfg = _cfg(T=len(vecs), E=E, k=k, score=kind)
                    idx, _ = orc.select(cfg, np.ascontiguousarray(vecs), bias)
                    for t in range(len(vecs)):
                        want = _brute_select(key_rows[t], k)
                        assert list(idx[t]) == want, (E, k, kind, vecs[t], bias, idx[t], want)


def pin_topk_special_orders(orc):
    """All-equal logits pick [0..k-1]; a falling ramp picks [0..k-1]; a rising
    ramp picks [E-1, E-2, ...], for E up to 1024 and both scores."""
    for E in (1, 5, 32, 192, 256, 1024):
        ramp = np.arange(E) * (4.0 / E)  # steps far above an fp32 ulp of the scores
        lg = np.stack([np.zeros(E), -ramp, ramp - 2.0]).astype(np.float32)
        for k in sorted({1, min(E, 6), min(E, 8), min(E, 32)}):
            for kind in ("sigmoid", "sqrt_softplus"):
                idx, _ = orc.select(_cfg(T=3, E=E, k=k, score=kind), lg)
                assert list(idx[0]) == list(range(k)), "all-equal"
                assert list(idx[1]) == list(range(k)), "descending"
                assert list(idx[2]) == list(range(E - 1, E - 1 - k, -1)), "ascending"


def pin_topk_nan_and_signed_zero(orc):
    E, k = 6, 4
    cfg = _cfg(T=2, E=E, k=k, score="sigmoid")
    lg = np.array([[np.nan, 0.0, np.nan, -1.0, 1.0, 0.0],
                   [0.0, -0.0, 0.0, -0.0, np.nan, np.nan]], np.float32)
    idx, _ = orc.select(cfg, lg)
    assert list(idx[0]) == [4, 1, 5, 3], idx[0]       # NaN keys after every number
    assert list(idx[1]) == [0, 1, 2, 3], idx[1]       # equal keys: lower index first
    cfg = _cfg(T=1, E=E, k=6, score="sigmoid")
    idx, _ = orc.select(cfg, lg[:1].copy())
    assert list(idx[0]) == [4, 1, 5, 3, 0, 2], idx[0]  # NaNs last, by index


def pin_selection_invariants(orc):
    rng = np.random.default_rng(4)
    for E, k in ((32, 4), (192, 8), (256, 6), (256, 8), (1024, 32), (7, 7)):
        lg = (rng.standard_normal((64, E)) * rng.choice([0.01, 1.0, 10.0])).astype(np.float32)
        lg[:8] = np.round(lg[:8])  # many exact ties
        for kind in ("sigmoid", "sqrt_softplus"):
            idx, w = orc.select(_cfg(T=64, E=E, k=k, score=kind), lg)
            assert ((idx >= 0) & (idx < E)).all()
            for row in idx:
                assert len(set(row.tolist())) == k


# ---------------------------------------------------------------------------
# Row top-k over long candidate rows (indexer-style selection)
# ---------------------------------------------------------------------------

def _py_topk_rows(row, k):
    """Python's own sort as the definition: NaN after every number, larger value
    first (-0 equals +0), then lower index; the first k, listed by index."""
    order = sorted(range(len(row)), key=lambda i: (1, 0.0, i) if math.isnan(row[i])
                   else (0, -float(row[i]), i))
    return sorted(order[:k])


def pin_topk_rows_python_sort(orc):
    """Against Python's sort on rows with heavy ties, NaN and signed zeros."""
    rng = np.random.default_rng(21)
    for n, k in ((1, 1), (7, 3), (64, 64), (300, 17), (1000, 512), (4099, 1024)):
        rows = rng.standard_normal((6, n)).astype(np.float32)
        rows[1] = np.round(rows[1] * 2) / 2                   # few distinct values
        rows[2] = np.where(rng.random(n) < 0.3, np.nan, rows[2])
        rows[3] = np.where(rng.random(n) < 0.5, -0.0, 0.0)    # only signed zeros
        rows[4] = np.maximum(rows[4], 0)                      # ReLU-like: many exact zeros
        rows[5] = np.float32(7.0)
        rows = np.ascontiguousarray(rows, np.float32)
        idx, vals = orc.topk_rows(rows, k)
        for r in range(rows.shape[0]):
            want = _py_topk_rows(rows[r].tolist(), k)
            assert idx[r].tolist() == want, (n, k, r)
            assert np.array_equal(vals[r].view(np.uint32), rows[r][want].view(np.uint32))


def pin_topk_rows_bruteforce(orc):
    """Every row over {-1, -0, +0, 1, NaN}^n for n <= 4, every k: the chosen set
    is the unique k-subset whose members each precede every non-member."""
    alphabet = [-1.0, -0.0, 0.0, 1.0, float("nan")]

    def prec(r, a, b):
        na, nb = math.isnan(r[a]), math.isnan(r[b])
        if na != nb:
            return nb
        if not na and r[a] != r[b]:
            return r[a] > r[b]
        return a < b

    for n in range(1, 5):
        rows = np.array(list(itertools.product(alphabet, repeat=n)), np.float32)
        for k in range(1, n + 1):
            idx, _ = orc.topk_rows(rows, k)
            for t, r in enumerate(rows.tolist()):
                found = [sub for sub in itertools.combinations(range(n), k)
                         if all(prec(r, a, b) for a in sub for b in range(n) if b not in sub)]
                assert len(found) == 1
                assert idx[t].tolist() == list(found[0]), (r, k, idx[t])


def pin_topk_rows_special_cases(orc):
    """Closed forms: all equal -> [0, k); rising -> [n-k, n); falling -> [0, k);
    k == n -> everything; only m < k numbers -> those plus the first NaNs."""
    for n in (1, 2, 33, 1000, 65536):
        rise = np.arange(n, dtype=np.float32)
        rows = np.stack([np.full(n, 3.0), rise, -rise]).astype(np.float32)
        for k in sorted({1, min(n, 2), min(n, 512), min(n, 2048), n}):
            idx, _ = orc.topk_rows(rows, k)
            assert idx[0].tolist() == list(range(k))
            assert idx[1].tolist() == list(range(n - k, n))
            assert idx[2].tolist() == list(range(k))
    n, k = 100, 10
    row = np.full((1, n), np.nan, np.float32)
    row[0, [90, 5, 50]] = [1.0, -2.0, 0.5]
    idx, _ = orc.topk_rows(row, k)
    assert idx[0].tolist() == sorted([5, 50, 90] + [i for i in range(n) if i not in (5, 50, 90)][:7])


def pin_topk_rows_threshold_invariants(orc):
    """At indexer scale (n = 65536, k = 2048): indices ascending and in range,
    values copied exactly, every chosen value >= every unchosen one, and the
    count strictly above the k-th largest value is < k."""
    rng = np.random.default_rng(22)
    n, k = 65536, 2048
    rows = np.maximum(rng.standard_normal((2, n)), 0).astype(np.float32)
    rows[1] = np.round(rows[1] * 8) / 8
    idx, vals = orc.topk_rows(rows, k)
    for r in range(2):
        ix = idx[r]
        assert (np.diff(ix) > 0).all() and ix[0] >= 0 and ix[-1] < n
        assert np.array_equal(vals[r], rows[r][ix])
        mask = np.zeros(n, bool)
        mask[ix] = True
        assert vals[r].min() >= rows[r][~mask].max()
        kth = np.sort(rows[r])[::-1][k - 1]
        assert (rows[r] > kth).sum() < k and vals[r].min() == kth
        tied = np.flatnonzero(rows[r] == kth)          # the tie at the cut goes by index
        taken = np.flatnonzero(mask & (rows[r] == kth))
        assert np.array_equal(taken, tied[:len(taken)])


# ---------------------------------------------------------------------------
# Weights (renormalisation and scale)
# ---------------------------------------------------------------------------

def pin_weight_invariants(orc):
    """w >= 0, sum w = scale within (k+1) ulps, w proportional to the unbiased
    scores (so the bias selects but never weights)."""
    rng = np.random.default_rng(5)
    for kind, scale, E, k in (("sigmoid", 1.0, 192, 8), ("sqrt_softplus", 1.5, 256, 6),
                              ("sigmoid", 2.5, 32, 4), ("sqrt_softplus", 1.0, 64, 1)):
        lg = rng.standard_normal((40, E)).astype(np.float32)
        bias = (rng.uniform(-0.5, 0.5, E)).astype(np.float32)
        idx, w = orc.select(_cfg(T=40, E=E, k=k, score=kind, scale=scale), lg, bias)
        assert (w >= 0).all()
        tol = (k + 1) * 2.0 ** -24 * scale
        assert np.all(np.abs(w.astype(np.float64).sum(1) - scale) <= tol), w.sum(1)
        for t in range(40):
            s = [Fraction(float(exact.score_f32(kind, float(lg[t, e])))) for e in idx[t]]
            S = sum(s)
            for j in range(k):
                ratio = Fraction(float(w[t, j])) / (s[j] / S * Fraction(scale))
                assert abs(ratio - 1) <= Fraction(1, 2 ** 23), (t, j)


def pin_weight_special_cases(orc):
    for kind, scale in (("sigmoid", 1.0), ("sqrt_softplus", 1.5)):
        for k in (1, 3, 6, 8):
            _, w = orc.select(_cfg(T=1, E=8, k=k, score=kind, scale=scale), np.zeros((1, 8), np.float32))
            assert (w == exact.round_f32(Fraction(scale) / k)).all(), (kind, k, w)
        _, w = orc.select(_cfg(T=1, E=1, k=1, score=kind, scale=scale), np.array([[0.3]], np.float32))
        assert w[0, 0] == np.float32(scale)
    # every selected score underflows to 0 -> weights 0 (no NaN)
    _, w = orc.select(_cfg(T=1, E=4, k=2, score="sigmoid"), np.full((1, 4), -200.0, np.float32))
    assert (w == 0).all()
    _, w = orc.select(_cfg(T=1, E=4, k=2, score="sqrt_softplus", scale=1.5),
                      np.full((1, 4), -300.0, np.float32))
    assert (w == 0).all()


def pin_golden_routing(orc):
    """Closed-form worked examples stored in tests/golden/routing_examples.json."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "routing_examples.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        lg = np.array(c["logits"], np.float32)
        bias = None if c.get("bias") is None else np.array(c["bias"], np.float32)
        cfg = _cfg(T=lg.shape[0], E=lg.shape[1], k=c["k"], score=c["score"], scale=c["scale"])
        idx, w = orc.select(cfg, lg, bias)
        assert idx.tolist() == c["topk_idx"], (c["name"], idx.tolist())
        want = np.array([[exact.round_f32(Fraction(v)) for v in row] for row in c["topk_w"]],
                        np.float32)
        assert (w == want).all(), (c["name"], w.tolist())


# ---------------------------------------------------------------------------
# Logits
# ---------------------------------------------------------------------------

def pin_logits_exact_integers(orc):
    """Small-integer inputs make every partial sum exact: logits equal numpy's."""
    rng = np.random.default_rng(6)
    T, d, E = 5, 96, 12
    x = rng.integers(-8, 9, (T, d)).astype(np.float32)
    wr = rng.integers(-8, 9, (E, d)).astype(np.float32) / 4
    logits, _, _ = orc.route(_cfg(T=T, d=d, E=E, k=3), x, wr)
    assert (logits == (x.astype(np.float64) @ wr.T.astype(np.float64)).astype(np.float32)).all()


def pin_logits_fp64_accuracy(orc):
    """Random inputs: logits equal the exactly-rounded rational dot product
    (fp64 sums of exact products err far below half an fp32 ulp here)."""
    import synth
    rng = np.random.default_rng(7)
    T, d, E = 3, 512, 16
    xb = synth.normal_bf16(0, 99, T * d, 1.0).reshape(T, d)
    wr = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    cfg = _cfg(T=T, d=d, E=E, k=2, act="bf16", w="bf16")
    logits, _, _ = orc.route(cfg, xb, wr)
    xf = exact.widen_bf16(xb)
    mism = 0
    for t in range(T):
        for e in range(E):
            fr = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(xf[t], wr[e]))
            mism += exact.f32_bits(exact.round_f32(fr)) != exact.f32_bits(logits[t, e])
    assert mism == 0, mism


def pin_logit_stride(orc):
    """Row t of the logits holds token t against every expert (stride n_expert)."""
    T, d, E = 3, 8, 5
    x = np.zeros((T, d), np.float32)
    for t in range(T):
        x[t, t] = 1.0
    wr = np.arange(E * d, dtype=np.float32).reshape(E, d)
    logits, _, _ = orc.route(_cfg(T=T, d=d, E=E, k=1), x, wr)
    assert (logits == wr[:, :T].T).all()


# ---------------------------------------------------------------------------
# Permutation
# ---------------------------------------------------------------------------

def pin_permutation(orc):
    rng = np.random.default_rng(8)
    for T, E, k in ((1, 256, 6), (2, 192, 8), (37, 8, 3), (300, 256, 8), (64, 1, 1)):
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        off, perm, inv = orc.permute(_cfg(T=T, E=E, k=k), idx)
        flat = idx.reshape(-1)
        assert perm.tolist() == sorted(range(T * k), key=lambda f: (flat[f], f))
        assert off.tolist() == [0] + np.cumsum(np.bincount(flat, minlength=E)).tolist()
        assert (inv[perm] == np.arange(T * k)).all()


def pin_permutation_invalid_and_duplicates(orc):
    idx = np.array([[3, 3], [9, 0], [-1, 2]], np.int32)   # E = 4: 9 and -1 are out of range
    off, perm, inv = orc.permute(_cfg(T=3, E=4, k=2), idx)
    assert off.tolist() == [0, 1, 1, 2, 4]
    assert perm.tolist() == [3, 5, 0, 1, -1, -1]
    assert inv.tolist() == [2, 3, -1, 0, -1, 1]


# ---------------------------------------------------------------------------
# Expert FFN and combine
# ---------------------------------------------------------------------------

def _rand_layer(rng, cfg, T, x_sigma=1.0, w_sigma=0.2):
    E, d, F, Fs = cfg["E"], cfg["d"], cfg["F"], cfg["Fs"]

    def mat(n, r, c):
        v = rng.standard_normal((n, r, c)) * w_sigma
        if cfg["w"] == "f32":
            return v.astype(np.float32)
        if cfg["w"] == "bf16":
            return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        q = rng.integers(-127, 128, (n, r, c)).astype(np.int8)
        s = (rng.uniform(0.5, 2.0, (n, r, c // 32)) * w_sigma / 64).astype(np.float16).view(np.uint16)
        return (q, s)

    xv = rng.standard_normal((T, d)) * x_sigma
    x = xv.astype(np.float32) if cfg["act"] == "f32" else \
        (xv.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    L = dict(x=x, w_router=(rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32),
             bias=(rng.uniform(-0.1, 0.1, E)).astype(np.float32) if cfg["score"] == "sigmoid" else None,
             gate=mat(E, F, d), up=mat(E, F, d), down=mat(E, d, F))
    if cfg["n_shared"]:
        L.update(s_gate=mat(1, Fs, d), s_up=mat(1, Fs, d), s_down=mat(1, d, Fs))
    return L


def _numpy_ffn(cfg, L, which, e, x64, F):
    """SwiGLU of all tokens through one expert with numpy fp64 matmuls; h rounded
    by exact integer arithmetic (bf16) or by numpy's float32 cast."""
    g, u, dn = (exact.as_f64(L[key], cfg["w"]) for key in which)
    G = x64 @ g[e].T
    U = x64 @ u[e].T
    A = G / (1.0 + np.exp(-G)) * U
    H = A.astype(np.float32).astype(np.float64) if cfg["act"] == "f32" else exact.bf16_round_array(A)
    return H @ dn[e].T


def pin_layer_vs_numpy(orc):
    """The whole layer against numpy fp64 matmuls for every supported format."""
    rng = np.random.default_rng(9)
    for act, w in (("f32", "f32"), ("bf16", "bf16"), ("bf16", "q8b32")):
        for kind, scale in (("sigmoid", 1.0), ("sqrt_softplus", 1.5)):
            cfg = _cfg(T=6, d=64, E=8, k=3, F=32, Fs=64, n_shared=1, score=kind, scale=scale,
                       act=act, w=w)
            L = _rand_layer(rng, cfg, 6)
            out = orc.layer_forward(cfg, L)
            x64 = exact.as_f64(L["x"], act)
            y = _numpy_ffn(cfg, L, ("s_gate", "s_up", "s_down"), 0, x64, cfg["Fs"])
            idx, wt = out["topk_idx"], out["topk_w"]
            for t in range(6):
                for j in range(3):
                    y[t] += float(wt[t, j]) * _numpy_ffn(cfg, L, ("gate", "up", "down"), idx[t, j],
                                                         x64[t:t + 1], cfg["F"])[0]
            err = np.abs(out["y"] - y).max(1) / np.abs(y).max(1)
            assert err.max() < 1e-6, (act, w, kind, err.max())


def pin_one_expert_is_dense(orc):
    """E = 1, top-1, no shared expert: y is the dense SwiGLU (sigmoid weight 1),
    and exactly 1.5 times it under sqrt(softplus) with scale 1.5."""
    rng = np.random.default_rng(10)
    for act, w in (("f32", "f32"), ("bf16", "bf16"), ("bf16", "q8b32")):
        for kind, scale in (("sigmoid", 1.0), ("sqrt_softplus", 1.5)):
            cfg = _cfg(T=5, d=64, E=1, k=1, F=96, Fs=32, n_shared=0, score=kind, scale=scale,
                       act=act, w=w)
            L = _rand_layer(rng, cfg, 5)
            y = orc.layer_forward(cfg, L)["y"]
            dense = orc.dense_swiglu(cfg, L["x"], L["gate"], L["up"], L["down"])
            assert (y == (dense * scale).astype(np.float32)).all(), (act, w, kind)


def pin_identity_weights(orc):
    """d = F, Wg = Wu = Wd = I, one expert: y_i = round_h(silu(x_i) * x_i)."""
    d = 64
    rng = np.random.default_rng(11)
    for act in ("f32", "bf16"):
        cfg = _cfg(T=4, d=d, E=1, k=1, F=d, Fs=d, n_shared=0, act=act, w=act)
        eye = np.eye(d, dtype=np.float32)[None]
        if act == "bf16":
            eye = (eye.view(np.uint32) >> 16).astype(np.uint16)
        xv = (rng.standard_normal((4, d)) * 3).astype(np.float32)
        x = xv if act == "f32" else (xv.view(np.uint32) >> 16).astype(np.uint16)
        x64 = exact.as_f64(x, act)
        L = dict(x=x, w_router=np.ones((1, d), np.float32), bias=None, gate=eye, up=eye, down=eye)
        y = orc.layer_forward(cfg, L)["y"]
        a = np.array([[xv_ / (1 + math.exp(-xv_)) * xv_ for xv_ in row] for row in x64])
        want = a.astype(np.float32) if act == "f32" else exact.bf16_round_array(a).astype(np.float32)
        assert (y == want).all(), act


def pin_down_doubling_and_zero(orc):
    """Doubling every down matrix doubles y exactly; zero routed down matrices
    leave exactly the shared expert's dense output."""
    rng = np.random.default_rng(12)
    cfg = _cfg(T=4, d=64, E=6, k=2, F=32, Fs=32, n_shared=1, act="bf16", w="bf16")
    L = _rand_layer(rng, cfg, 4)
    y1 = orc.layer_forward(cfg, L)["y"]
    L2 = dict(L)
    for key in ("down", "s_down"):
        f = exact.widen_bf16(L[key]) * 2
        L2[key] = (f.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y2 = orc.layer_forward(cfg, L2)["y"]
    assert (y2 == 2 * y1).all()
    L3 = dict(L)
    L3["down"] = np.zeros_like(L["down"])
    y3 = orc.layer_forward(cfg, L3)["y"]
    dense = orc.dense_swiglu(cfg, L["x"], L["s_gate"], L["s_up"], L["s_down"], F=cfg["Fs"])
    assert (y3 == dense.astype(np.float32)).all()


def pin_identical_experts(orc):
    """When every routed expert is the same, y = shared + scale * FFN, whatever
    the routing (up to the fp32 rounding of the weights)."""
    rng = np.random.default_rng(13)
    cfg = _cfg(T=6, d=64, E=8, k=3, F=32, Fs=32, n_shared=1, score="sqrt_softplus", scale=1.5,
               act="bf16", w="bf16")
    L = _rand_layer(rng, cfg, 6)
    for key in ("gate", "up", "down"):
        L[key] = np.ascontiguousarray(np.repeat(L[key][:1], 8, axis=0))
    y = orc.layer_forward(cfg, L)["y"].astype(np.float64)
    ex = orc.dense_swiglu(cfg, L["x"], L["gate"], L["up"], L["down"])
    sh = orc.dense_swiglu(cfg, L["x"], L["s_gate"], L["s_up"], L["s_down"], F=cfg["Fs"])
    want = sh + 1.5 * ex
    assert (np.abs(y - want).max(1) / np.abs(want).max(1)).max() < 1e-6


def pin_q8_bf16_bridge(orc):
    """int8 quants with power-of-two scales are exactly bf16 values: the Q8B32
    layer equals the bf16 layer with the dequantised weights, bit for bit."""
    rng = np.random.default_rng(14)
    cfg = _cfg(T=3, d=64, E=4, k=2, F=64, Fs=32, n_shared=1, score="sigmoid", act="bf16", w="q8b32")
    L = _rand_layer(rng, cfg, 3)
    Lb = dict(L)
    for key in ("gate", "up", "down", "s_gate", "s_up", "s_down"):
        q, _ = L[key]
        s = (2.0 ** rng.integers(-12, -4, (q.shape[0], q.shape[1], q.shape[2] // 32))).astype(np.float16)
        L[key] = (q, s.view(np.uint16))
        deq = exact.dequant_q8(q, s.view(np.uint16)).astype(np.float32)
        assert ((deq.view(np.uint32) & 0xFFFF) == 0).all()
        Lb[key] = (deq.view(np.uint32) >> 16).astype(np.uint16)
    cb = dict(cfg, w="bf16")
    assert (orc.layer_forward(cfg, L)["y"] == orc.layer_forward(cb, Lb)["y"]).all()


def pin_split_api_matches_layer(orc):
    """route -> permute -> expert_ffn -> combine reproduces the whole-layer call:
    identical routing and permutation, y within the fp32 rounding of the slots."""
    rng = np.random.default_rng(15)
    cfg = _cfg(T=9, d=64, E=8, k=3, F=32, Fs=32, n_shared=1, act="bf16", w="bf16")
    L = _rand_layer(rng, cfg, 9)
    full = orc.layer_forward(cfg, L)
    lg, idx, w = orc.route(cfg, L["x"], L["w_router"], L["bias"])
    assert (idx == full["topk_idx"]).all() and (w == full["topk_w"]).all()
    assert (lg == full["logits"]).all()
    off, perm, inv = orc.permute(cfg, idx)
    assert (off == full["offsets"]).all() and (perm == full["perm_rows"]).all()
    slot, shared = orc.expert_ffn(cfg, L, off, perm, w)
    y = orc.combine(cfg, slot, shared)
    assert (np.abs(y - full["y"]).max(1) / np.abs(full["y"]).max(1)).max() < 1e-6


def pin_combine_definition(orc):
    """Combine adds the shared row and the token's k slot rows."""
    rng = np.random.default_rng(16)
    T, k, d = 5, 3, 16
    cfg = _cfg(T=T, d=d, k=k)
    slot = rng.integers(-50, 50, (T * k, d)).astype(np.float32)
    shared = rng.integers(-50, 50, (T, d)).astype(np.float32)
    y = orc.combine(cfg, slot, shared)
    assert (y == shared + slot.reshape(T, k, d).sum(1)).all()
    assert (orc.combine(cfg, slot, None) == slot.reshape(T, k, d).sum(1)).all()


def _exact_weights(cfg, m):
    """Integer weights [n, rows, cols] (int64) of an exact_layer tensor."""
    if cfg["w"] == "q8b32":
        q, sc = m
        shift = (0x3C00 - sc.astype(np.int64)) // 0x0400
        assert np.all(sc.astype(np.int64) == 0x3C00 - 0x0400 * shift) and np.all((shift >= 0) & (shift <= 2))
        q = q.astype(np.int64)
        mult = np.repeat(2 ** shift, 32, axis=2)
        assert np.all(q % mult == 0)
        return q // mult
    if cfg["w"] == "bf16":
        return (m.astype(np.uint32) << 16).view(np.float32).astype(np.int64)
    return m.astype(np.int64)


def pin_exact_layers_integer_evaluation(orc):
    """On the exact-arithmetic layers the GPU tests use (synth.configs.
    exact_layer) the oracle's y equals an evaluation in exact integers: the
    selected experts are the token's indicator set, each weight is 1/k, and
    silu(g) = g for the integer gate sums g >= 20 at fp32 precision (e^-20 <
    2^-25).  Pins the premise of the GPU's bit-exact tests, for bf16, int8 and
    fp32 weights and for the decode and prefill shapes."""
    from synth import configs
    for spec in (dict(T=3, d=256, E=32, k=4, F=128), dict(T=40, d=256, E=16, k=4, F=128, w="q8b32"),
                 dict(T=5, d=128, E=8, k=2, F=64, act="f32", w="f32"),
                 dict(T=30, d=192, E=4, k=1, F=64, Fs=128, n_shared=0)):
        L = configs.exact_layer(**spec, seed=11)
        cfg = L["cfg"]
        E, k = cfg["E"], cfg["k"]
        x = L["x"]
        xi = (x.astype(np.uint32) << 16).view(np.float32) if cfg["act"] == "bf16" else x
        xi = xi.astype(np.int64)
        ref = orc.layer_forward(cfg, L)
        G, U, D = (_exact_weights(cfg, L[w]) for w in ("gate", "up", "down"))
        want = np.zeros((cfg["T"], cfg["d"]), dtype=object)
        for t in range(cfg["T"]):
            sel = np.flatnonzero(xi[t, :E])
            assert ref["topk_idx"][t].tolist() == sel.tolist()
            acc = np.zeros(cfg["d"], dtype=object)
            for e in sel:
                g, u = G[e] @ xi[t], U[e] @ xi[t]
                assert g.min() >= 20
                acc = acc + (D[e] @ (g * u)).astype(object) * Fraction(1, k)
            if cfg["n_shared"]:
                g = _exact_weights(cfg, L["s_gate"])[0] @ xi[t]
                u = _exact_weights(cfg, L["s_up"])[0] @ xi[t]
                acc = acc + (_exact_weights(cfg, L["s_down"])[0] @ (g * u)).astype(object)
            want[t] = acc
        assert np.all(ref["topk_w"] == np.float32(1.0 / k))
        assert np.array_equal(ref["y"].astype(np.float64), want.astype(np.float64)), spec


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
