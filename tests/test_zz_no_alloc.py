"""moe_layer_forward_noalloc (the library's static device scratch instead of a
caller workspace) against moe_layer_forward with a workspace, through the C
ABI: the same kernels on the same inputs, so every output must be the same
bits.  Two calls in a row on one layer, the second with fewer tokens, so the
second call runs over scratch the first call left behind; each is also
checked against the oracle (indices exact, y within tolerance).
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


def _layer(T, **kw):
    base = dict(T=T, x_sigma=1.0, w_sigma=0.05, bias="uniform", bias_lo=-0.05, bias_hi=0.05, n_shared=1,
                score="sigmoid", scale=1.0, act="bf16", w="bf16")
    base.update(kw)
    base.setdefault("Fs", base["F"])
    base.setdefault("wr_sigma", 1.0 / math.sqrt(base["d"]))
    return configs.custom(**base)


def _outputs(moe, torch, cfg, x, W, noalloc):
    T, E, k = x.shape[0], cfg["E"], cfg["k"]
    c = moe.config_from(cfg, T=T)
    out = dict(y=torch.full((T, cfg["d"]), float("nan"), dtype=torch.float32, device="cuda"),
               logits=torch.empty((T, E), dtype=torch.float32, device="cuda"),
               topk_idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
               topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda"),
               offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
               perm_rows=torch.empty(T * k, dtype=torch.int32, device="cuda"),
               inv_perm=torch.empty(T * k, dtype=torch.int32, device="cuda"))
    dbg = {key: v for key, v in out.items() if key != "y"}
    if noalloc:
        moe.moe_layer_forward_noalloc(c, x, moe.make_weights(W), out["y"], debug=dbg)
    else:
        ws = moe.workspace(c)
        ws.fill_(0xA5)
        moe.moe_layer_forward(c, x, moe.make_weights(W), out["y"], ws, debug=dbg)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in out.items()}


# (layer, token counts of the two calls in a row): prefill then a smaller
# prefill batch, prefill then decode, int8 prefill then int8 decode
CASES = {
    "bf16_prefill_300_then_70": (dict(d=256, E=40, k=5, F=128), (300, 70)),
    "bf16_prefill_200_then_decode_3": (dict(d=320, E=24, k=4, F=192, Fs=128), (200, 3)),
    "q8_prefill_120_then_decode_1": (dict(d=256, E=32, k=6, F=128, w="q8b32", score="sqrt_softplus",
                                          scale=1.5, bias="none"), (120, 1)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_workspace_entry(orc, case):
    import torch
    import sparse_moe_layer_02_amd as moe
    assert torch.cuda.is_available()
    moe.load()
    spec, counts = CASES[case]
    cfg = _layer(max(counts), **spec)
    L = configs.make_layer(cfg)
    W = H.upload_layer(L)
    for T in counts:
        say("case", case, "T", T)
        x = H.to_dev(np.ascontiguousarray(L["x"][:T]))
        a = _outputs(moe, torch, cfg, x, W, noalloc=True)
        b = _outputs(moe, torch, cfg, x, W, noalloc=False)
        for key in a:
            assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (case, T, key)
        Ls = dict(L)
        Ls["x"] = np.ascontiguousarray(L["x"][:T])
        ref = orc.layer_forward(dict(cfg, T=T), Ls)
        H.check_routing(a, ref, "%s T=%d" % (case, T))
        err = H.check_y(a["y"], ref["y"], cfg, "%s T=%d" % (case, T))
        say("   ok: bit-identical to the workspace entry point; y err %.2e" % err)


def test_noalloc_refuses_oversize_config():
    """A layer whose workspace exceeds the static scratch is refused before
    anything is enqueued."""
    import ctypes
    import sparse_moe_layer_02_amd as moe
    lib = moe.load()
    c = moe.make_config(T=4096, d=6144, E=256, k=8, F=2048)
    assert lib.moe_workspace_bytes(ctypes.byref(c)) > moe.binding.STATIC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)
    m = moe.binding.moe_mat(fake.value, None)
    w = moe.binding.moe_weights(fake.value, None, m, m, m, m, m, m)
    assert lib.moe_layer_forward_noalloc(ctypes.byref(c), fake, ctypes.byref(w), fake, None, None) == 3
