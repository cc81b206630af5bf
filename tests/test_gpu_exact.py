"""Exact-arithmetic parity: on layers whose every product and partial sum is
exactly representable (small-integer activations and weights, power-of-two
int8 block scales; synth.configs.exact_layer), any correct evaluation order
gives the same bits, so the GPU must equal the oracle bit for bit - logits,
routing, permutation, y, and on the split entry points slot_out and
shared_out - not merely to a tolerance.

The gate pre-activations g are integers in [20, 44], where silu(g) rounds to g
in fp32, so h = g * u is an exact integer: a wrong gate or up sum (a K chunk
dropped, repeated or taken from the wrong rows) changes h, and with it y, by
a whole number.  Every expert kernel family is reached: the decode GEMVs
(bf16, int8, fp32), the grouped MFMA GEMMs with 64- and 256-row tiles (the
latter through LDS copies, with short tiles, also at d = 6144), the int8
grouped GEMMs (K loops of whole and partial register rings), and the
prefill GEMVs (int8 with few rows per expert, fp32).
"""
import sys

import numpy as np
import pytest

from synth import configs
import gpu_harness as H

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # decode path (T <= 8): router / selection / GEMV kernels
    "decode_bf16_T1": dict(T=1, d=256, E=32, k=8, F=128),
    "decode_bf16_T2": dict(T=2, d=320, E=48, k=8, F=192, Fs=128),
    "decode_bf16_T8": dict(T=8, d=256, E=32, k=4, F=128),
    "decode_q8_T1": dict(T=1, d=512, E=64, k=4, F=256, w="q8b32"),
    "decode_q8_T5": dict(T=5, d=256, E=32, k=2, F=128, w="q8b32"),
    "decode_f32_T3": dict(T=3, d=512, E=32, k=4, F=256, act="f32", w="f32"),
    # prefill: 64-row tiles (fewer than 96 rows per expert)
    "prefill_bm64": dict(T=40, d=256, E=16, k=4, F=128),
    "prefill_bm64_no_shared": dict(T=70, d=192, E=8, k=2, F=64, n_shared=0),
    # 256-row tiles through LDS copies (96 rows per expert or more on
    # average): odd 32-wide K stages, experts of 140-160 rows (one full and
    # one short tile each), skewed loads from 17 to 506 rows (tiles with 1 to
    # 8 live 32-row blocks, one or two live A-row copies)
    "prefill_bm256_short_tiles": dict(T=300, d=192, E=4, k=2, F=320, Fs=448),
    "prefill_bm256_skewed": dict(T=800, d=256, E=16, k=2, F=192, skew=1.2),
    "prefill_bm256_skewed_no_shared": dict(T=700, d=192, E=12, k=2, F=128, n_shared=0, skew=1.0),
    "prefill_bm256": dict(T=700, d=320, E=2, k=2, F=320, Fs=448),
    "prefill_bm256_d6144": dict(T=600, d=6144, E=2, k=1, F=2048),
    # int8: grouped GEMMs for both products (1.5 rows per expert or more),
    # GEMV gate/up beside the GEMM down (0.5 to 1.5 rows), GEMVs for both
    "prefill_q8_mfma": dict(T=64, d=320, E=16, k=4, F=192, Fs=256, w="q8b32"),
    "prefill_q8_gemv": dict(T=9, d=256, E=32, k=2, F=128, w="q8b32"),
    "prefill_q8_gemv_only": dict(T=9, d=256, E=64, k=2, F=128, w="q8b32"),
    # int8 LDS-copy grouped GEMMs (up to 8 rows per expert on average, K a
    # multiple of 256): 32-row passes, a 40-row shared tile in two passes,
    # skewed experts of up to 37 rows, partial and whole eight-stage rounds
    "prefill_q8_dma": dict(T=40, d=256, E=16, k=2, F=256, Fs=512, w="q8b32"),
    "prefill_q8_dma_skewed": dict(T=60, d=768, E=16, k=2, F=256, w="q8b32", skew=1.2),
    # int8 grouped GEMMs with K a multiple of the register ring (4 chunks of
    # 64): full and partial 64-row tiles, skewed loads from 4 to 108 rows
    "prefill_q8_ring": dict(T=96, d=512, E=8, k=2, F=256, Fs=512, w="q8b32"),
    "prefill_q8_ring_skewed": dict(T=200, d=256, E=16, k=2, F=512, w="q8b32", skew=1.0),
    # fp32 prefill (GEMVs over the grouped rows)
    "prefill_f32": dict(T=40, d=128, E=8, k=2, F=64, act="f32", w="f32"),
}


def _bits_equal(a, b):
    return a.shape == b.shape and np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                                                 np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("case", sorted(CASES))
def test_exact_layer_bitwise(orc, case):
    import torch
    import sparse_moe_layer_02_amd as moe
    assert torch.cuda.is_available()
    moe.load()
    L = configs.exact_layer(**CASES[case], seed=len(case))
    cfg = L["cfg"]
    say("case", case, "T=%d d=%d E=%d k=%d F=%d %s/%s" % (cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["F"],
                                                         cfg["act"], cfg["w"]))
    ref = orc.layer_forward(cfg, L)
    assert np.all(ref["topk_w"] == np.float32(1.0 / cfg["k"]))    # the construction's premise
    dev = H.upload_layer(L)
    got = H.layer_outputs(cfg, dev["x"], dev)
    for key in ("logits", "topk_idx", "topk_w", "offsets", "perm_rows", "inv_perm", "y"):
        assert _bits_equal(got[key], ref[key]), (case, key, np.argwhere(got[key] != ref[key])[:5])
    say("   y bit-identical (max |y| %.0f)" % np.abs(ref["y"]).max())
    if cfg["T"] <= moe.DECODE_MAX_TOKENS:   # the same inputs through the prefill kernels
        got_p = H.layer_outputs(cfg, dev["x"], dev, path="prefill")
        for key in ("topk_idx", "y"):
            assert _bits_equal(got_p[key], ref[key]), (case, "prefill", key)


@pytest.mark.parametrize("case", ["prefill_bm64", "prefill_bm256_skewed", "prefill_bm256", "prefill_q8_mfma",
                                  "prefill_q8_ring", "prefill_q8_dma", "decode_q8_T5"])
def test_exact_split_entry_points(orc, case):
    """moe_expert_ffn and moe_combine alone, with caller routing weights that
    are powers of two: slot_out, shared_out and y bit for bit."""
    import torch
    import sparse_moe_layer_02_amd as moe
    L = configs.exact_layer(**CASES[case], seed=7 + len(case))
    cfg = L["cfg"]
    T, k, d = cfg["T"], cfg["k"], cfg["d"]
    _, idx, _ = orc.route(cfg, L["x"], L["w_router"], None)
    off, perm, _ = orc.permute(cfg, idx)
    rng = np.random.default_rng(3)
    wts = (2.0 ** rng.integers(-3, 2, (T, k))).astype(np.float32)
    r_slot, r_shared = orc.expert_ffn(cfg, L, off, perm, wts)
    r_y = orc.combine(cfg, r_slot, r_shared)
    dev = H.upload_layer(L)
    c = moe.config_from(cfg)
    ws = moe.workspace(c)
    slot = torch.full((T * k, d), float("nan"), dtype=torch.float32, device="cuda")
    shared = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda") if cfg["n_shared"] else None
    moe.moe_expert_ffn(c, dev["x"], moe.make_weights(dev), H.to_dev(off), H.to_dev(perm), H.to_dev(wts), slot,
                       shared, ws)
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    moe.moe_combine(c, slot, shared, y)
    torch.cuda.synchronize()
    assert _bits_equal(slot.cpu().numpy(), r_slot), case
    if shared is not None:
        assert _bits_equal(shared.cpu().numpy(), r_shared), case
    assert _bits_equal(y.cpu().numpy(), r_y), case
    say("   %s: slot_out, shared_out, y bit-identical" % case)
