"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on
the same seeded inputs.

Bar: expert indices, offsets and permutation exact; logits and routing weights
within one ulp; y within 2e-3 (bf16 / int8 layers) or 1e-5 (fp32 layers),
row-normwise (see gpu_harness).  Decode workloads run 32-64 steps of the
benchmark's token stream, every token checked.  The full-size prefill
workloads check routing and the permutation on every token and y on every
token (c4, c2 with 512 tokens) or on a sample that reaches every row tile of
the most and least loaded experts (c5, and the matrix-core supplements s1 and
s2).  Bit-exact checks on exact-arithmetic layers are in test_gpu_exact.py.
"""
import math
import sys

import numpy as np
import pytest

from synth import configs
import gpu_harness as H

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sparse_moe_layer_02_amd as moe
    moe.load()
    return torch


def oracle_full(orc, cfg, L):
    return orc.layer_forward(cfg, L)


def run_and_check(orc, cfg, L, path="auto", label=""):
    say("case", label, "T=%d" % L["x"].shape[0], "path", path)
    dev = H.upload_layer(L)
    got = H.layer_outputs(cfg, dev["x"], dev, path=path)
    ref = oracle_full(orc, cfg, L)
    stats = H.check_routing(got, ref, label)
    err = H.check_y(got["y"], ref["y"], cfg, label)
    say("   ok: y err %.2e, logit ulp hist %s" % (err, stats["logit_ulp_hist"][:3]))
    return got, ref


# ---------------------------------------------------------------------------
# Workloads c1-c3 (decode sizes): many decode steps of the benchmark's token
# stream, the oracle on every token of every step
# ---------------------------------------------------------------------------

def _host_layer_on_device(cfg, T=None):
    """The whole layer on the host (for the oracle) and its weights on the GPU."""
    L = configs.make_layer(cfg, T=T)
    return L, H.upload_layer(L)


DECODE_STEPS = {"c1": ("c1", 4, 1), "c2": ("c2", 1, 64), "c3": ("c3", 1, 32), "c3t2": ("c3", 2, 32)}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", sorted(DECODE_STEPS))
def test_decode_workloads(torch_cuda, orc, name):
    """c2: 64 distinct tokens, c3: 32 one-token and 32 two-token (verify)
    steps, all from the benchmark's decode token stream; c1 its own 4 tokens.
    Every step through the decode path, the first two also through the
    prefill path; routing exact and y within tolerance on every token."""
    base, T, steps = DECODE_STEPS[name]
    cfg = configs.get(base, T=T)
    say("case", name, "T", T, "steps", steps, "(generating the layer)")
    L, W = _host_layer_on_device(cfg)
    if name == "c1":
        xs = [L["x"]]
    else:
        xs = [configs.gen_x(cfg, T, stream=configs.S_DECODE, token0=i * T) for i in range(steps)]
    got = [H.layer_outputs(cfg, H.to_dev(x), W) for x in xs]
    say("   %d GPU steps done; oracle on %d tokens" % (len(xs), len(xs) * T))
    Lr = dict(L)
    Lr["x"] = np.ascontiguousarray(np.concatenate(xs))
    ref = orc.layer_forward(cfg, Lr)
    errs, unions = [], []
    for i, g in enumerate(got):
        sl = slice(i * T, (i + 1) * T)
        r = dict(logits=ref["logits"][sl], topk_idx=ref["topk_idx"][sl], topk_w=ref["topk_w"][sl])
        ro, rp, ri = orc.permute(cfg, r["topk_idx"])
        r.update(offsets=ro, perm_rows=rp, inv_perm=ri)
        H.check_routing(g, r, "%s step %d" % (name, i))
        errs.append(H.check_y(g["y"], ref["y"][sl], cfg, "%s step %d" % (name, i)))
        unions.append(len(np.unique(r["topk_idx"])))
        if i < 2:
            gp = H.layer_outputs(cfg, H.to_dev(xs[i]), W, path="prefill")
            H.check_routing(gp, r, "%s step %d / prefill" % (name, i))
            H.check_y(gp["y"], ref["y"][sl], cfg, "%s step %d / prefill" % (name, i))
    say("   ok %s: %d steps, y err max %.2e median %.2e, expert union mean %.2f"
        % (name, len(xs), max(errs), float(np.median(errs)), float(np.mean(unions))))
    del W
    torch_cuda.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Full-size prefill workloads: c4 / c5, c2's int8 layer with a 512-token
# batch, and the two matrix-core supplements (s1: one dense expert over 4096
# tokens at d = 6144, s2: c4's layer with 16384 tokens), all on the 256-,
# 128- or 64-row tiles the library picks for them
# ---------------------------------------------------------------------------

PREFILL = {
    "c4": dict(base="c4", sample="all"),
    "c5": dict(base="c5", sample=512),
    "c2p": dict(base="c2", T=512, sample="all"),
    "s1": dict(base="c5", over=dict(E=1, k=1, n_shared=0, bias="none"), sample=96),
    "s2": dict(base="c4", T=16384, sample=256),
}


def _tile_sample(off, perm, k, experts, step):
    """One token from every ``step`` rows of each listed expert's segment of the
    grouped order, plus the token of its last row (the ragged tail)."""
    out = []
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = list(range(lo, hi, step)) + ([hi - 1] if hi > lo else [])
        out += [int(perm[r]) // k for r in rows]
    return out


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", sorted(PREFILL))
def test_prefill_workloads(torch_cuda, orc, name):
    """Routing and permutation exact on every token; y within tolerance on every
    token of c4 and c2p, and on a seeded sample of c5, s1 and s2 that holds a
    token from every 64 rows of the three most loaded experts (so every M tile
    of every tile size and every slot of the XCD work order that serves them)
    and of the shared expert, the last rows of the least loaded experts, and
    seeded random tokens."""
    spec = PREFILL[name]
    cfg = configs.get(spec["base"], label=name, **({"T": spec["T"]} if "T" in spec else {}),
                      **spec.get("over", {}))
    T, k = cfg["T"], cfg["k"]
    say("case", name, "T", T, "(generating the layer)")
    L, W = _host_layer_on_device(cfg)
    say("   running the layer on the GPU")
    got = H.layer_outputs(cfg, W["x"], W)
    say("   oracle routing of all %d tokens" % T)
    lg, idx, wts = orc.route(cfg, L["x"], L["w_router"], L["bias"])
    off, perm, inv = orc.permute(cfg, idx)
    ref = dict(logits=lg, topk_idx=idx, topk_w=wts, offsets=off, perm_rows=perm, inv_perm=inv)
    stats = H.check_routing(got, ref, name)
    say("   routing exact; logit ulp histogram", stats["logit_ulp_hist"])
    counts = np.diff(off)
    say("   expert rows: min %d max %d mean %.1f, active %d" % (counts.min(), counts.max(), counts.mean(),
                                                              (counts > 0).sum()))
    if name == "c5":
        ranks = configs.skew_ranks(cfg)
        share = np.isin(idx, np.where(ranks <= 10)[0]).mean()
        say("   hottest 10 experts receive %.1f%% of selections" % (100 * share))
        assert 0.26 <= share <= 0.34
    assert np.isfinite(got["y"]).all()
    if spec["sample"] == "all":
        sample = np.arange(T)
    else:
        hot = np.argsort(-counts, kind="stable")[:3]
        cold = [int(e) for e in np.argsort(counts, kind="stable") if counts[e] > 0][:3]
        chosen = set(_tile_sample(off, perm, k, hot, 64) + _tile_sample(off, perm, k, cold, 64))
        if cfg["n_shared"]:
            chosen |= set(range(0, T, 64)) | {T - 1}
        rng = np.random.default_rng(12345)
        rest = rng.permutation(np.setdiff1d(np.arange(T), sorted(chosen)))
        n_more = max(0, spec["sample"] - len(chosen))
        sample = np.array(sorted(chosen | set(rest[:n_more].tolist())))
        say("   sample: %d tokens (%d from the tiles of experts %s and %s and the shared expert)"
            % (len(sample), len(chosen), hot.tolist(), cold))
    Ls = dict(L)
    Ls["x"] = np.ascontiguousarray(L["x"][sample])
    say("   oracle y on %d tokens" % len(sample))
    ref_s = orc.layer_forward(cfg, Ls)
    assert np.array_equal(ref_s["topk_idx"], idx[sample])
    err = H.check_y(got["y"][sample], ref_s["y"], cfg, name)
    say("   ok %s: y err %.2e over %d tokens" % (name, err, len(sample)))
    del W, L
    torch_cuda.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Edge cases on small shapes (full oracle)
# ---------------------------------------------------------------------------

def _custom(**kw):
    base = dict(x_sigma=1.0, w_sigma=0.05, bias="uniform", bias_lo=-0.05, bias_hi=0.05, n_shared=1,
                score="sigmoid", scale=1.0, act="bf16", w="bf16")
    base.update(kw)
    base.setdefault("Fs", base["F"])
    base.setdefault("wr_sigma", 1.0 / math.sqrt(base["d"]))
    return configs.custom(**base)


EDGE = {
    "one_expert_top1": dict(T=5, d=64, E=1, k=1, F=64),
    "one_expert_no_shared": dict(T=3, d=64, E=1, k=1, F=128, n_shared=0),
    "E63_k7_ragged": dict(T=9, d=192, E=63, k=7, F=128),
    "E1024_k32_softplus": dict(T=3, d=128, E=1024, k=32, F=64, score="sqrt_softplus", scale=1.5,
                               bias="none"),
    "E384_T70_ragged_tiles": dict(T=70, d=576, E=384, k=8, F=192, Fs=128),
    "E16_T300_multiblock_perm": dict(T=300, d=128, E=16, k=8, F=64),
    "q8_prefill_small": dict(T=37, d=256, E=16, k=4, F=128, w="q8b32", score="sqrt_softplus",
                            scale=1.5, bias="none"),
    "q8_decode_T8": dict(T=8, d=256, E=32, k=6, F=128, w="q8b32", score="sqrt_softplus", scale=1.5,
                         bias="none"),
    # int8 grouped GEMMs: several 64-row tiles per expert, a partial last
    # 128-column tile of down (d = 320), a shared expert wider than the routed
    # ones, odd numbers of 64-wide K chunks (d = 320 -> 5, F = 192 -> 3)
    "q8_prefill_tiles": dict(T=300, d=320, E=4, k=2, F=192, Fs=256, w="q8b32", score="sqrt_softplus",
                             scale=1.5, bias="none"),
    "q8_prefill_no_shared": dict(T=65, d=128, E=8, k=3, F=64, n_shared=0, w="q8b32"),
    "f32_prefill": dict(T=40, d=128, E=8, k=2, F=64, act="f32", w="f32", x_sigma=0.5, w_sigma=0.1),
    "f32_decode_T3": dict(T=3, d=512, E=32, k=4, F=256, act="f32", w="f32", x_sigma=0.5, w_sigma=0.1),
    "no_shared_prefill": dict(T=33, d=128, E=8, k=3, F=64, n_shared=0),
    "shared_wider_than_routed": dict(T=12, d=128, E=8, k=2, F=64, Fs=192),
    # 256-row LDS-copy tiles whose last tile is short (experts average
    # 96-255 rows): odd numbers of 32-wide K stages (d = 192, F = 320), short
    # tiles with 1 to 7 live 32-row blocks, shared expert wider than the
    # routed ones, experts of one full and one short tile
    "bm256_short_odd_stages": dict(T=300, d=192, E=4, k=2, F=320, Fs=448),
    "bm256_short_single_stage_pair": dict(T=200, d=64, E=2, k=1, F=64, Fs=64),
    "bm256_short_many_tiles": dict(T=700, d=256, E=6, k=3, F=128, Fs=128),
    # 256-row tiles fed through LDS copies (experts average >= 256 rows):
    # 32-wide K stages in groups of four with a tail (d = 320 -> 10 stages,
    # Fs = 448 -> 14), a partial last N tile of gate/up (F = 320) and of down
    # (d = 320), ragged last M tiles, fewer stages than the pipeline depth
    # (d = F = 64 -> 2), exact multiples, three experts with two stage tails
    "bm256_ragged": dict(T=700, d=320, E=2, k=2, F=320, Fs=448),
    "bm256_short_k": dict(T=600, d=64, E=1, k=1, F=64, Fs=64),
    "bm256_one_expert": dict(T=1000, d=256, E=1, k=1, F=256, n_shared=0),
    "bm256_three_experts": dict(T=520, d=192, E=3, k=3, F=192, Fs=128),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_cases(torch_cuda, orc, case):
    cfg = _custom(**EDGE[case])
    L = configs.make_layer(cfg)
    run_and_check(orc, cfg, L, label=case)
    if cfg["T"] <= 8:
        run_and_check(orc, cfg, L, path="prefill", label=case + "/prefill")


def test_skewed_all_to_few_experts(torch_cuda, orc):
    """A dominant bias sends every token to the same k experts: one expert gets
    300 rows (five GEMM tiles) and the rest none."""
    cfg = _custom(T=300, d=128, E=32, k=4, F=64)
    L = configs.make_layer(cfg)
    L["bias"] = np.zeros(32, np.float32)
    L["bias"][[3, 5, 17, 30]] = 10.0
    got, ref = run_and_check(orc, cfg, L, label="all_to_four")
    assert sorted(set(got["topk_idx"].reshape(-1).tolist())) == [3, 5, 17, 30]


def test_decode_path_identity(torch_cuda, orc):
    """T = 1..8 through the decode and the prefill paths: identical routing and
    permutation, y within tolerance of each other and of the oracle."""
    for T in range(1, 9):
        cfg = _custom(T=T, d=256, E=48, k=6, F=128)
        L = configs.make_layer(cfg)
        a, ref = run_and_check(orc, cfg, L, path="decode", label="decode T=%d" % T)
        b, _ = run_and_check(orc, cfg, L, path="prefill", label="prefill T=%d" % T)
        for key in ("topk_idx", "offsets", "perm_rows", "inv_perm"):
            assert np.array_equal(a[key], b[key])


def test_uninitialised_workspace(torch_cuda, orc):
    """The library writes every workspace word before reading it: a workspace
    full of 0xFF bytes gives the same bits as a zeroed one, with the routing
    kept in the workspace (no debug outputs) and with it exported."""
    for path, spec in (("decode", dict(T=3, d=256, E=40, k=5, F=128)),
                       ("prefill", dict(T=300, d=256, E=40, k=5, F=128)),
                       ("prefill", dict(T=40, d=256, E=24, k=4, F=128, w="q8b32"))):
        cfg = _custom(**spec)
        L = configs.make_layer(cfg)
        dev = H.upload_layer(L)
        ref = oracle_full(orc, cfg, L)
        for debug in (False, True):
            a = H.layer_outputs(cfg, dev["x"], dev, path=path, ws_fill=0, debug=debug)
            b = H.layer_outputs(cfg, dev["x"], dev, path=path, ws_fill=0xFF, debug=debug)
            for key in a:
                assert np.array_equal(a[key], b[key]), (path, spec, debug, key)
            H.check_y(b["y"], ref["y"], cfg, "ws 0xFF %s T=%d" % (path, spec["T"]))
        say("   ok: %s T=%d" % (path, spec["T"]))


def test_deterministic(torch_cuda, orc):
    cfg = _custom(T=70, d=256, E=32, k=4, F=128)
    L = configs.make_layer(cfg)
    dev = H.upload_layer(L)
    a = H.layer_outputs(cfg, dev["x"], dev)
    b = H.layer_outputs(cfg, dev["x"], dev)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


# ---------------------------------------------------------------------------
# The separate entry points
# ---------------------------------------------------------------------------

def test_split_entry_points(torch_cuda, orc):
    import torch
    import sparse_moe_layer_02_amd as moe
    for spec in (dict(T=6, d=128, E=16, k=4, F=64), dict(T=90, d=128, E=16, k=4, F=64),
                 dict(T=20, d=256, E=16, k=4, F=128, w="q8b32")):
        cfg = _custom(**spec)
        L = configs.make_layer(cfg)
        T, k, d = cfg["T"], cfg["k"], cfg["d"]
        say("case split", spec)
        dev = H.upload_layer(L)
        c = moe.config_from(cfg)
        ws = moe.workspace(c)
        logits = torch.empty((T, cfg["E"]), dtype=torch.float32, device="cuda")
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        moe.moe_route(c, dev["x"], dev["w_router"], dev["bias"], logits, idx, w, ws)
        off = torch.empty(cfg["E"] + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
        inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
        moe.moe_permute(c, idx, off, perm, inv, ws)
        slot = torch.empty((T * k, d), dtype=torch.float32, device="cuda")
        shared = torch.empty((T, d), dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn(c, dev["x"], moe.make_weights(dev), off, perm, w, slot, shared, ws)
        y = torch.empty((T, d), dtype=torch.float32, device="cuda")
        moe.moe_combine(c, slot, shared, y)
        torch.cuda.synchronize()
        r_lg, r_idx, r_w = orc.route(cfg, L["x"], L["w_router"], L["bias"])
        H.check_routing(dict(logits=logits.cpu().numpy(), topk_idx=idx.cpu().numpy(),
                             topk_w=w.cpu().numpy()), dict(logits=r_lg, topk_idx=r_idx, topk_w=r_w))
        r_off, r_perm, r_inv = orc.permute(cfg, r_idx)
        assert np.array_equal(off.cpu().numpy(), r_off)
        assert np.array_equal(perm.cpu().numpy(), r_perm)
        assert np.array_equal(inv.cpu().numpy(), r_inv)
        r_slot, r_shared = orc.expert_ffn(cfg, L, r_off, r_perm, r_w)
        H.check_y(slot.cpu().numpy(), r_slot, cfg, "slot_out")
        H.check_y(shared.cpu().numpy(), r_shared, cfg, "shared_out")
        r_y = orc.combine(cfg, r_slot, r_shared)
        H.check_y(y.cpu().numpy(), r_y, cfg, "y")
        # combine of identical inputs: both sides add the same fp32 values
        y2 = torch.empty_like(y)
        moe.moe_combine(c, torch.from_numpy(r_slot).cuda(), torch.from_numpy(r_shared).cuda(), y2)
        torch.cuda.synchronize()
        assert H.rownorm_err(y2.cpu().numpy(), orc.combine(cfg, r_slot, r_shared)) < 1e-6


def test_expert_ffn_masked_to_hot_experts(torch_cuda, orc):
    """moe_expert_ffn over a routing masked to its most-loaded experts (every
    other assignment replaced by -1, as the c5hot benchmark does), on the
    256-row LDS-copy tiles (T*k >= 96 E): experts of two and three tiles whose
    last tiles run through the cold loop (5, 13 and 41 rows) or the hot one
    (232 and 253 rows), with and without the shared expert.  The grouping is
    exact, every listed slot row (and shared_out) matches the oracle's, and no
    other slot row is written."""
    import torch
    import sparse_moe_layer_02_amd as moe
    for n_shared, hot in ((0, 3), (1, 5)):
        cfg = _custom(T=1800, d=256, E=16, k=4, F=128, n_shared=n_shared)
        T, E, k, d = cfg["T"], cfg["E"], cfg["k"], cfg["d"]
        assert T * k >= 96 * E
        say("case masked", dict(n_shared=n_shared, hot=hot))
        L = configs.make_layer(cfg)
        r_lg, r_idx, r_w = orc.route(cfg, L["x"], L["w_router"], L["bias"])
        counts = np.bincount(r_idx.reshape(-1), minlength=E)
        keep = np.argsort(-counts, kind="stable")[:hot]
        idx = np.where(np.isin(r_idx, keep), r_idx, -1).astype(np.int32)
        r_off, r_perm, r_inv = orc.permute(cfg, idx)
        rows = np.diff(r_off)
        assert rows.max() > 512 and (rows[keep] % 256).min() > 0  # three-tile experts, ragged tails
        dev = H.upload_layer(L)
        c = moe.config_from(cfg)
        ws = moe.workspace(c)
        off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
        inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
        moe.moe_permute(c, H.to_dev(idx), off, perm, inv, ws)
        slot = torch.full((T * k, d), float("nan"), dtype=torch.float32, device="cuda")
        shared = torch.empty((T, d), dtype=torch.float32, device="cuda") if n_shared else None
        moe.moe_expert_ffn(c, dev["x"], moe.make_weights(dev), off, perm, H.to_dev(r_w), slot, shared, ws)
        torch.cuda.synchronize()
        assert np.array_equal(off.cpu().numpy(), r_off)
        assert np.array_equal(perm.cpu().numpy(), r_perm)
        assert np.array_equal(inv.cpu().numpy(), r_inv)
        r_slot, r_shared = orc.expert_ffn(cfg, L, r_off, r_perm, r_w)
        listed = r_perm[r_perm >= 0]
        got = slot.cpu().numpy()
        H.check_y(got[listed], r_slot[listed], cfg, "slot_out of the kept experts")
        unlisted = np.setdiff1d(np.arange(T * k), listed)
        assert np.isnan(got[unlisted]).all(), "a slot row outside the kept experts was written"
        if n_shared:
            H.check_y(shared.cpu().numpy(), r_shared, cfg, "shared_out")


@pytest.mark.parametrize("spec", [dict(T=4100, d=128, E=192, k=8, F=64, act="bf16", w="bf16"),
                                  dict(T=2100, d=192, E=250, k=6, F=64, act="f32", w="f32",
                                       score="sqrt_softplus", scale=1.5, bias="none"),
                                  dict(T=1000, d=320, E=72, k=4, F=64, act="bf16", w="bf16"),
                                  dict(T=1100, d=128, E=64, k=8, F=64, act="f32", w="f32"),
                                  dict(T=4100, d=128, E=250, k=8, F=64, act="bf16", w="bf16"),
                                  dict(T=4200, d=192, E=255, k=6, F=64, act="f32", w="f32",
                                       score="sqrt_softplus", scale=1.5, bias="none")],
                         ids=["bf16_T4100_E192", "f32_T2100_E250", "split_bf16_T1000_E72_d320",
                              "split_f32_T1100_E64_d128", "bf16_T4100_E250", "f32_T4200_E255_d192"])
def test_router_matrix_cores(torch_cuda, orc, spec):
    """Router shapes on the fp64 matrix-core kernels (at least 128 tiles of
    64 x 64, or of 16 x 32 with K split over four groups of wavefronts, five
    and two 64-column chunks for the split cases), with ragged token and expert
    tails: logits within one ulp, indices and weights as the oracle's."""
    import torch
    import sparse_moe_layer_02_amd as moe
    cfg = _custom(**spec)
    T, E, k, d = cfg["T"], cfg["E"], cfg["k"], cfg["d"]
    assert (((T + 63) // 64) * ((E + 63) // 64) >= 128 or ((T + 15) // 16) * ((E + 31) // 32) >= 128) \
        and (T % 64, E % 64) != (0, 0)
    say("router", spec)
    x = configs.gen_x(cfg)
    wr = configs.gen_router(cfg)
    bias = configs.gen_bias(cfg)
    c = moe.config_from(cfg, path="prefill")
    ws = moe.workspace(c)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(c, H.to_dev(x), H.to_dev(wr), H.to_dev(bias), logits, idx, w, ws)
    torch.cuda.synchronize()
    r_lg, r_idx, r_w = orc.route(cfg, x, wr, bias)
    hist = H.check_routing(dict(logits=logits.cpu().numpy(), topk_idx=idx.cpu().numpy(),
                                topk_w=w.cpu().numpy()), dict(logits=r_lg, topk_idx=r_idx, topk_w=r_w))
    say("  ulp histograms", hist)


def test_select_special_values(torch_cuda, orc):
    """NaN logits rank last, integer logits tie, and the compile-time
    256-expert top-k gives the same bits as the runtime-E kernel."""
    import torch
    import sparse_moe_layer_02_amd as moe
    rng = np.random.default_rng(0)
    for E, k, kind, scale in ((256, 6, "sqrt_softplus", 1.5), (256, 8, "sigmoid", 1.0),
                              (192, 8, "sigmoid", 1.0), (7, 7, "sigmoid", 1.0), (1024, 32, "sigmoid", 1.0)):
        T = 64
        lg = rng.standard_normal((T, E)).astype(np.float32)
        lg[:16] = np.round(lg[:16])            # exact ties
        lg[16:20, ::3] = np.nan                 # NaN experts
        lg[20:24] = -300.0                      # every score underflows
        bias = rng.uniform(-0.1, 0.1, E).astype(np.float32) if kind == "sigmoid" else None
        cfg = dict(T=T, d=64, E=E, k=k, F=64, Fs=64, n_shared=0, score=kind, scale=scale, act="bf16",
                   w="bf16")
        r_idx, r_w = orc.select(cfg, lg, bias)
        outs = []
        for path in ("auto", "prefill"):
            c = moe.config_from(cfg, path=path)
            idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
            w = torch.empty((T, k), dtype=torch.float32, device="cuda")
            moe.moe_select(c, H.to_dev(lg), H.to_dev(bias), idx, w)
            torch.cuda.synchronize()
            outs.append((idx.cpu().numpy(), w.cpu().numpy()))
            assert np.array_equal(outs[-1][0], r_idx), (E, k, path)
            same = (outs[-1][1].view(np.uint32) == r_w.view(np.uint32)) | (np.isnan(outs[-1][1]) & np.isnan(r_w))
            assert same.all(), (E, k, path)
        assert np.array_equal(outs[0][0], outs[1][0])
        assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


def test_permute_caller_indices(torch_cuda, orc):
    """Caller-supplied indices, including out-of-range and repeated experts."""
    import torch
    import sparse_moe_layer_02_amd as moe
    rng = np.random.default_rng(1)
    for T, k, E in ((3, 2, 4), (200, 8, 37), (1000, 6, 256)):
        idx = rng.integers(-2, E + 2, (T, k)).astype(np.int32)
        cfg = dict(T=T, d=64, E=E, k=k, F=64, Fs=64, n_shared=1, score="sigmoid", scale=1.0, act="bf16",
                   w="bf16")
        c = moe.config_from(cfg)
        ws = moe.workspace(c)
        off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
        inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
        moe.moe_permute(c, H.to_dev(idx), off, perm, inv, ws)
        torch.cuda.synchronize()
        r_off, r_perm, r_inv = orc.permute(cfg, idx)
        assert np.array_equal(off.cpu().numpy(), r_off)
        assert np.array_equal(perm.cpu().numpy(), r_perm)
        assert np.array_equal(inv.cpu().numpy(), r_inv)


def test_graph_capture_replay(torch_cuda, orc):
    """The decode and prefill paths captured in a HIP graph: every replay (with
    eager work and synchronisations in between) reproduces the eager result."""
    import torch
    import sparse_moe_layer_02_amd as moe
    for spec in (dict(T=1, d=256, E=64, k=6, F=128, w="q8b32", score="sqrt_softplus", scale=1.5, bias="none"),
                 dict(T=2, d=256, E=48, k=8, F=128), dict(T=70, d=256, E=32, k=4, F=128)):
        cfg = _custom(**spec)
        say("case graph", spec)
        L = configs.make_layer(cfg)
        dev = H.upload_layer(L)
        c = moe.config_from(cfg)
        ws = moe.workspace(c)
        W = moe.make_weights(dev)
        xs = [H.to_dev(configs.gen_x(cfg, cfg["T"], stream=configs.S_DECODE, token0=i * cfg["T"])) for i in range(3)]
        ys = [torch.empty((cfg["T"], cfg["d"]), dtype=torch.float32, device="cuda") for _ in range(3)]
        eager = []
        for x, y in zip(xs, ys):
            moe.moe_layer_forward(c, x, W, y, ws)
            torch.cuda.synchronize()
            eager.append(y.clone())
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            moe.moe_layer_forward(c, xs[0], W, ys[0], ws, stream=side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream().cuda_stream
            for x, y in zip(xs, ys):
                moe.moe_layer_forward(c, x, W, y, ws, stream=cap)
        for rep in range(4):
            for y in ys:
                y.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            for y, ref in zip(ys, eager):
                assert torch.equal(y, ref), "replay %d differs" % rep
            # eager work between replays
            moe.moe_layer_forward(c, xs[1], W, ys[1], ws)
            torch.cuda.synchronize()
