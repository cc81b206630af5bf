"""The five MoE-layer workloads, as data.

Each workload stands in for one MoE layer of a model the pages discuss:

* ``c1`` tiny fp32 layer, sigmoid + bias top-4 (the smallest parity case);
* ``c2`` DeepSeek-Flash-style decode: 256 experts, sqrt(softplus) top-6 x1.5,
  int8 blocks of 32 with an fp16 scale (the pages keep "decision" tensors at
  Q8_0/F32: NeutronStar README, "The model");
* ``c3`` Hy3-style decode/verify: 192 experts, sigmoid + per-expert bias top-8
  (NeutronStar README, main branch, Hy3 paragraph), T in {1, 2};
* ``c4`` prefill chunk, 512 tokens, near-uniform routing;
* ``c5`` long prefill, 4096 tokens, expert bias skewed so that the ten most
  popular experts (3.9% of 256) take 30% of the selections (the popularity skew the pages
  report for the host expert cache: NeutronStar README, "SSD streaming
  optimizations").

Stream ids under the master seed: x 1, router weights 2, bias 3, gate 4, up 5,
down 6, shared gate/up/down 7/8/9, distinct decode tokens 10, skew
calibration batch 11.  Row t of x is elements [t*d, (t+1)*d) of its stream,
so a smaller T is a prefix of a larger one.
"""
from __future__ import annotations

import copy
import math

import numpy as np

from . import normal_bf16, normal_f32, q8b32, uniform_f32, zipf_bias

S_X, S_WR, S_BIAS, S_GATE, S_UP, S_DOWN, S_SGATE, S_SUP, S_SDOWN, S_DECODE, S_CALIB = range(1, 12)

# Skew strength of the c5 bias, b_e = -beta * ln(rank_e).  Found by bisection
# with the oracle router on the 4096-token calibration batch (stream 11) so that
# the 10 hottest experts (3.9%) receive 30% of the top-8 selections; the script
# that finds it is tests/golden/calibrate_skew.py and its output is
# tests/golden/skew_beta.json.
C5_BETA = 0.07193540781736374

CONFIGS = {
    "c1": dict(T=4, d=512, E=32, k=4, F=256, Fs=256, n_shared=1, score="sigmoid", scale=1.0,
               act="f32", w="f32", x_sigma=0.02, wr_sigma=0.02, w_sigma=0.02,
               bias="uniform", bias_lo=-0.1, bias_hi=0.1, path="decode"),
    "c2": dict(T=1, d=4096, E=256, k=6, F=2048, Fs=2048, n_shared=1, score="sqrt_softplus",
               scale=1.5, act="bf16", w="q8b32", x_sigma=0.02, wr_sigma=0.02, w_sigma=0.02,
               bias="none", path="decode"),
    "c3": dict(T=1, d=4096, E=192, k=8, F=1536, Fs=1536, n_shared=1, score="sigmoid", scale=1.0,
               act="bf16", w="bf16", x_sigma=1.0, wr_sigma=1.0 / 64.0, w_sigma=0.02,
               bias="uniform", bias_lo=-0.01, bias_hi=0.01, path="decode"),
    "c4": dict(T=512, d=6144, E=256, k=8, F=2048, Fs=2048, n_shared=1, score="sigmoid",
               scale=1.0, act="bf16", w="bf16", x_sigma=1.0, wr_sigma=1.0 / math.sqrt(6144.0),
               w_sigma=0.02, bias="uniform", bias_lo=-0.01, bias_hi=0.01, path="prefill"),
    "c5": dict(T=4096, d=6144, E=256, k=8, F=2048, Fs=2048, n_shared=1, score="sigmoid",
               scale=1.0, act="bf16", w="bf16", x_sigma=1.0, wr_sigma=1.0 / math.sqrt(6144.0),
               w_sigma=0.02, bias="zipf", beta=C5_BETA, path="prefill"),
}


def get(name: str, label: str | None = None, **over) -> dict:
    """A copy of workload ``name`` with fields overridden (e.g. ``T=2``),
    named ``label`` if given."""
    cfg = copy.deepcopy(CONFIGS[name])
    cfg.update(over)
    cfg["name"] = label or name
    cfg.setdefault("seed", 0)
    return cfg


def custom(**fields) -> dict:
    """A workload from explicit fields (defaults: c1's distributions)."""
    cfg = copy.deepcopy(CONFIGS["c1"])
    cfg.update(fields)
    cfg.setdefault("name", "custom")
    cfg.setdefault("seed", 0)
    return cfg


def _normal(cfg, stream, n, sigma, start=0, dtype=None):
    dtype = dtype or cfg["act"]
    if dtype == "f32":
        return normal_f32(cfg["seed"], stream, n, sigma, start=start)
    return normal_bf16(cfg["seed"], stream, n, sigma, start=start)


def gen_x(cfg, T=None, stream=S_X, token0=0):
    """Activations [T, d] (fp32, or bf16 bits as uint16)."""
    T = cfg["T"] if T is None else T
    d = cfg["d"]
    return _normal(cfg, stream, T * d, cfg["x_sigma"], start=token0 * d).reshape(T, d)


# Correlation of consecutive tokens in the look-ahead workload: with 256
# experts and top-6 selection, logits of correlation 0.97 share about 74% of
# their top-6 sets, the prediction rate the NeutronStar fork page reports for
# its router look-ahead.
LOOKAHEAD_RHO = 0.97


def gen_x_walk(cfg, T, rho, stream=S_DECODE):
    """T tokens [T, d] whose consecutive rows have correlation ``rho``: x_0 = z_0,
    x_t = rho x_{t-1} + sqrt(1 - rho^2) z_t with z ~ N(0, x_sigma^2) (fp32 walk;
    bf16 workloads get each row rounded to bf16, as uint16 bits).  A stand-in
    for a layer's input and the next layer's, which share the residual stream."""
    d = cfg["d"]
    z = normal_f32(cfg["seed"], stream, T * d, cfg["x_sigma"]).reshape(T, d).astype(np.float64)
    x = np.empty_like(z)
    x[0] = z[0]
    c = math.sqrt(1.0 - rho * rho)
    for t in range(1, T):
        x[t] = rho * x[t - 1] + c * z[t]
    x = x.astype(np.float32)
    if cfg["act"] == "f32":
        return x
    return (round_to_bf16(x).view(np.uint32) >> 16).astype(np.uint16)


def gen_router(cfg):
    E, d = cfg["E"], cfg["d"]
    return normal_f32(cfg["seed"], S_WR, E * d, cfg["wr_sigma"]).reshape(E, d)


def gen_bias(cfg):
    kind = cfg.get("bias", "none")
    if kind == "none":
        return None
    if kind == "uniform":
        return uniform_f32(cfg["seed"], S_BIAS, cfg["E"], cfg["bias_lo"], cfg["bias_hi"])
    if kind == "zipf":
        return zipf_bias(cfg["seed"], S_BIAS, cfg["E"], cfg["beta"])[0]
    raise ValueError(kind)


def skew_ranks(cfg):
    """1-based popularity ranks behind a ``zipf`` bias (rank 1 = hottest)."""
    return zipf_bias(cfg["seed"], S_BIAS, cfg["E"], cfg.get("beta", 0.0))[1]


_MAT_STREAM = {"gate": S_GATE, "up": S_UP, "down": S_DOWN,
               "s_gate": S_SGATE, "s_up": S_SUP, "s_down": S_SDOWN}


def mat_shape(cfg, which):
    """(n_experts, rows, cols) of an expert weight tensor; cols is the reduction dim."""
    d = cfg["d"]
    if which in ("gate", "up"):
        return cfg["E"], cfg["F"], d
    if which == "down":
        return cfg["E"], d, cfg["F"]
    if which in ("s_gate", "s_up"):
        return cfg["n_shared"], cfg["Fs"], d
    if which == "s_down":
        return cfg["n_shared"], d, cfg["Fs"]
    raise ValueError(which)


def gen_mat(cfg, which, e0=0, e1=None):
    """Experts [e0, e1) of one expert weight tensor.

    fp32 -> float32 [n, rows, cols]; bf16 -> uint16 bits; q8b32 ->
    (int8 [n, rows, cols], uint16 fp16-bits [n, rows, cols/32]).
    """
    n_e, rows, cols = mat_shape(cfg, which)
    e1 = n_e if e1 is None else e1
    n = e1 - e0
    st, sig = _MAT_STREAM[which], cfg["w_sigma"]
    if cfg["w"] == "q8b32":
        q, s = q8b32(cfg["seed"], st, n * rows, cols, sig, row0=e0 * rows)
        return q.reshape(n, rows, cols), s.reshape(n, rows, cols // 32)
    start = e0 * rows * cols
    if cfg["w"] == "f32":
        a = normal_f32(cfg["seed"], st, n * rows * cols, sig, start=start)
    else:
        a = normal_bf16(cfg["seed"], st, n * rows * cols, sig, start=start)
    return a.reshape(n, rows, cols)


def empty_mat(cfg, which):
    """Zero-filled host tensor of the full shape (pages are only touched when written)."""
    n_e, rows, cols = mat_shape(cfg, which)
    if cfg["w"] == "q8b32":
        return (np.zeros((n_e, rows, cols), np.int8), np.zeros((n_e, rows, cols // 32), np.uint16))
    return np.zeros((n_e, rows, cols), np.float32 if cfg["w"] == "f32" else np.uint16)


def fill_experts(cfg, which, mat, experts):
    """Write the listed experts' weights into a tensor from :func:`empty_mat`."""
    for e in sorted(set(int(e) for e in experts)):
        part = gen_mat(cfg, which, e, e + 1)
        if isinstance(mat, tuple):
            mat[0][e] = part[0][0]
            mat[1][e] = part[1][0]
        else:
            mat[e] = part[0]
    return mat


def make_layer(cfg, T=None, experts=None):
    """All inputs of one layer call as numpy arrays.

    ``experts`` (optional) restricts the routed expert weights that are filled;
    the others stay zero.  Used where only a sample of tokens is evaluated.
    """
    L = dict(cfg=cfg, x=gen_x(cfg, T), w_router=gen_router(cfg), bias=gen_bias(cfg))
    for which in ("gate", "up", "down"):
        if experts is None:
            L[which] = gen_mat(cfg, which)
        else:
            L[which] = fill_experts(cfg, which, empty_mat(cfg, which), experts)
    for which in ("s_gate", "s_up", "s_down"):
        L[which] = gen_mat(cfg, which) if cfg["n_shared"] else None
    return L


def algorithmic_bytes_per_expert(cfg) -> int:
    """HBM bytes of one routed expert's three matrices in the stored format."""
    n = 3 * cfg["F"] * cfg["d"]
    return {"f32": 4 * n, "bf16": 2 * n, "q8b32": n + n // 16}[cfg["w"]]


# ---------------------------------------------------------------------------
# Row top-k workloads: the sparse attention indexer's selection (its top-512
# and top-1024 over a long row of scores: "256 experts, 512 lines" blog post,
# section "The constant that always said 256").  A row is one query token's
# scores against n candidate key rows.
#   i1  small parity case: 8 rows x 5000 candidates, top-512
#   i2  a 512-token prefill chunk against 32768 candidates, top-1024
#   i3  one decode token against 65536 candidates, top-1024
# Streams: normals 12, head weights 13.
# ---------------------------------------------------------------------------
S_IDX_Z, S_IDX_W = 12, 13

TOPK_ROWS = {
    "i1": dict(rows=8, n=5000, k=512, heads=4, fmt="f32"),
    "i2": dict(rows=512, n=32768, k=1024, heads=4, fmt="f32"),
    "i3": dict(rows=1, n=65536, k=1024, heads=4, fmt="f32"),
}


def topk_rows_spec(name: str, **over) -> dict:
    spec = copy.deepcopy(TOPK_ROWS[name])
    spec.update(over)
    spec.setdefault("name", name)
    spec.setdefault("seed", 0)
    return spec


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), kept as fp32."""
    b = a.astype(np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return (b & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def gen_indexer_scores(spec, row0=0, rows=None):
    """Scores [rows, n] fp32 shaped like an indexer's output: a weighted sum
    over heads of ReLU'd dot products, score[r, s] = sum_h w[r, h] *
    max(z[r, s, h], 0) with z ~ N(0, 1) and per-row head weights w ~ U(0, 1).
    They are nonnegative with about one exact zero in 2^heads.  fmt "bf16"
    rounds them to bf16 precision, which makes exact ties common."""
    rows = spec["rows"] if rows is None else rows
    n, H, seed = spec["n"], spec["heads"], spec["seed"]
    z = normal_f32(seed, S_IDX_Z, rows * n * H, 1.0, start=row0 * n * H).reshape(rows, n, H)
    w = uniform_f32(seed, S_IDX_W, rows * H, 0.0, 1.0, start=row0 * H).reshape(rows, H)
    s = np.zeros((rows, n), np.float32)
    for h in range(H):
        s += w[:, h:h + 1] * np.maximum(z[:, :, h], np.float32(0))
    if spec.get("fmt", "f32") == "bf16":
        s = round_to_bf16(s)
    return np.ascontiguousarray(s, np.float32)


# ---------------------------------------------------------------------------
# Exact-arithmetic layers: small-integer inputs for which every product and
# every partial sum of the layer is an exactly representable number, so any
# correct evaluation order gives the same bits.  Built from a numpy seeded
# generator; no step of the method is computed here.
#
# x[t] holds, in its first E columns, the 0/1 indicator of a k-subset S_t of
# the experts; column E ("lift") holds 32 and column E+1 ("one") holds 1; the
# remaining columns are integers in [-2, 2].  The router gives expert e weight
# 24 on column e plus three +-1 entries in the free columns, so a logit is
# 24 + n (e in S_t) or n (otherwise) with |n| <= 6: the selected experts'
# sigmoid scores round to exactly 1.0 (logit >= 18), every other score stays
# below 1, and the renormalised weights are exactly 1/k.  Every gate row has 1
# on the lift column plus six +-1 entries, so g is an integer in [20, 44],
# where silu(g) rounds to g in fp32; every up row has 1 on the one column plus
# two +-1 entries, so u is an integer in [-3, 5] and g*u an integer of at most
# 220 in magnitude (exact in bf16); every down row has eight +-1 entries.  int8
# layers store each weight as q * scale with a per-block scale of 1, 1/2 or
# 1/4 (fp16) and q = weight / scale.
# ---------------------------------------------------------------------------

def _sparse_pm1(rng, n, rows, cols, per_row, forbid=()):
    """[n, rows, cols] float64 with ``per_row`` entries of +-1 per row, at
    distinct columns outside ``forbid``."""
    allowed = np.setdiff1d(np.arange(cols), np.asarray(forbid, dtype=np.int64))
    assert allowed.size >= per_row
    pick = rng.integers(0, allowed.size, (n, rows, per_row))
    while True:  # draw again the rows that hit a column twice
        srt = np.sort(pick, axis=2)
        dup = (srt[:, :, 1:] == srt[:, :, :-1]).any(axis=2)
        if not dup.any():
            break
        pick[dup] = rng.integers(0, allowed.size, (int(dup.sum()), per_row))
    out = np.zeros((n, rows, cols))
    sign = rng.choice(np.array([-1.0, 1.0]), size=(n, rows, per_row))
    np.put_along_axis(out, allowed[pick], sign, axis=2)
    return out


def _store(cfg, w, rng):
    """Integer-valued float64 weights [n, rows, cols] in the workload's format."""
    if cfg["w"] == "f32":
        return np.ascontiguousarray(w.astype(np.float32))
    if cfg["w"] == "bf16":
        return np.ascontiguousarray((w.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    n, rows, cols = w.shape
    shift = rng.integers(0, 3, (n, rows, cols // 32))            # scale 2^-shift
    scale_bits = (0x3C00 - 0x0400 * shift).astype(np.uint16)      # fp16 1.0, 0.5, 0.25
    q = w * np.repeat(2.0 ** shift, 32, axis=2)
    return (np.ascontiguousarray(q.astype(np.int8)), np.ascontiguousarray(scale_bits))


def exact_layer(T, d, E, k, F, Fs=None, n_shared=1, act="bf16", w="bf16", seed=0, skew=0.0):
    """A layer (dict as :func:`make_layer`, with its workload dict under
    ``cfg``) on which the method's arithmetic is exact (see above).  Sigmoid
    router, no bias, scale 1; k must be 1, 2, 4 or 8 and d >= E + 2.  With
    ``skew`` > 0 each token's expert subset is drawn with probabilities
    proportional to (e + 1)^-skew, so low-numbered experts get many rows."""
    assert k in (1, 2, 4, 8) and k <= E and d >= E + 2 and d % 64 == 0
    Fs = F if Fs is None else Fs
    cfg = custom(T=T, d=d, E=E, k=k, F=F, Fs=Fs, n_shared=n_shared, score="sigmoid", scale=1.0, act=act,
                 w=w, bias="none", name="exact")
    rng = np.random.default_rng(seed)
    lift, one = E, E + 1
    x = np.zeros((T, d))
    prob = (np.arange(E) + 1.0) ** -skew
    prob /= prob.sum()
    for t in range(T):
        x[t, rng.choice(E, k, replace=False, p=prob)] = 1.0
    x[:, lift] = 32.0
    x[:, one] = 1.0
    x[:, E + 2:] = rng.integers(-2, 3, (T, d - E - 2))
    wr = np.zeros((E, d))
    wr[np.arange(E), np.arange(E)] = 24.0
    wr += _sparse_pm1(rng, 1, E, d, 3, forbid=range(E + 2))[0]
    L = dict(cfg=cfg, w_router=np.ascontiguousarray(wr.astype(np.float32)), bias=None)
    if act == "f32":
        L["x"] = np.ascontiguousarray(x.astype(np.float32))
    else:
        L["x"] = np.ascontiguousarray((x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))

    def gate_up(n, rows):
        g = _sparse_pm1(rng, n, rows, d, 6, forbid=(lift, one))
        g[:, :, lift] = 1.0
        u = _sparse_pm1(rng, n, rows, d, 2, forbid=(lift, one))
        u[:, :, one] = 1.0
        return g, u

    g, u = gate_up(E, F)
    L["gate"], L["up"] = _store(cfg, g, rng), _store(cfg, u, rng)
    L["down"] = _store(cfg, _sparse_pm1(rng, E, d, F, 8), rng)
    if n_shared:
        g, u = gate_up(1, Fs)
        L["s_gate"], L["s_up"] = _store(cfg, g, rng), _store(cfg, u, rng)
        L["s_down"] = _store(cfg, _sparse_pm1(rng, 1, d, Fs, 8), rng)
    else:
        L["s_gate"] = L["s_up"] = L["s_down"] = None
    return L
