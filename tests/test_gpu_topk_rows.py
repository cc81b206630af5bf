"""GPU parity of the row top-k (moe_topk_rows) against the CPU oracle.

Bar: the chosen indices (ascending) equal the oracle's exactly, and the values
equal the scores at those indices bit for bit (NaN payloads and the sign of
zero included).  Cases span every launch shape (512 threads with 1..32 keys
each, 1024 threads with 32 or 64), a ragged tail in the last chunk, the
degenerate rows of the selection order (all equal, NaN, signed zeros,
infinities, subnormals, heavy ties at the cut), one row per branch of the
sampled pass (topk_branch_rows) and the full-size indexer workloads.
"""
import ctypes
import sys

import numpy as np
import pytest

from synth import configs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sparse_moe_layer_02_amd as moe
    moe.load()
    return torch, moe


def special_rows(n, rng):
    """Rows that exercise the selection order's corner cases."""
    rows = [
        np.full(n, 0.25, np.float32),                                               # all equal
        np.where(rng.random(n) < 0.6, np.nan, rng.standard_normal(n)).astype(np.float32),
        np.where(rng.random(n) < 0.5, -0.0, 0.0).astype(np.float32),                # signed zeros only
        rng.choice(np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 1.0, -1.0], np.float32), n),
        (rng.integers(-3, 4, n) * np.float32(1e-45)).astype(np.float32),            # subnormals
        np.arange(n, dtype=np.float32)[::-1].copy(),                                 # falling ramp
        np.round(rng.standard_normal(n) * 4).astype(np.float32),                     # few values
    ]
    return np.stack(rows).astype(np.float32)


def check(dev, orc, scores, k, label, with_vals=True):
    torch, moe = dev
    rows, n = scores.shape
    say("topk_rows %s: rows=%d n=%d k=%d" % (label, rows, n, k))
    want_idx, want_vals = orc.topk_rows(np.ascontiguousarray(scores), k)
    s_dev = torch.from_numpy(np.ascontiguousarray(scores)).cuda()
    idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    vals = torch.full((rows, k), 12345.0, dtype=torch.float32, device="cuda") if with_vals else None
    moe.moe_topk_rows(s_dev, k, idx, vals)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    bad = np.nonzero((got != want_idx).any(1))[0]
    assert len(bad) == 0, "%s: %d rows differ, first row %d: got %s want %s" % (
        label, len(bad), bad[0], got[bad[0]][:12], want_idx[bad[0]][:12])
    if with_vals:
        gv = vals.cpu().numpy()
        assert np.array_equal(gv.view(np.uint32), want_vals.view(np.uint32)), label


# (n, k): every launch shape, tails, k at both ends; the long rows with small k
# take the sampled pass when their sample is good (random and ramp rows) and
# the full radix path otherwise (constant, signed-zero and few-valued rows)
SHAPES = [(1, 1), (7, 7), (64, 5), (300, 17), (512, 512), (513, 100), (1000, 999), (2048, 64),
          (3000, 300), (4097, 1024), (8192, 8192), (16384, 2048), (16385, 1024), (20000, 512), (32768, 1),
          (32769, 4096), (50000, 2048), (65536, 65536),
          # rows of more than 32768 keys with k small enough for the sampled pass
          (40000, 512), (65536, 700), (65536, 1200)]


@pytest.mark.parametrize("n,k", SHAPES, ids=["n%d_k%d" % s for s in SHAPES])
def test_topk_rows_shapes(dev, orc, n, k):
    rng = np.random.default_rng(n * 7 + k)
    scores = np.concatenate([rng.standard_normal((3, n)).astype(np.float32), special_rows(n, rng)])
    check(dev, orc, scores, k, "n%d_k%d" % (n, k))


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_topk_rows_indexer_small(dev, orc, fmt):
    spec = configs.topk_rows_spec("i1", fmt=fmt)
    check(dev, orc, configs.gen_indexer_scores(spec), spec["k"], "i1_" + fmt)


def test_topk_rows_without_values(dev, orc):
    spec = configs.topk_rows_spec("i1", fmt="bf16")
    check(dev, orc, configs.gen_indexer_scores(spec), 700, "i1_idx_only", with_vals=False)


@pytest.mark.parametrize("name,fmt", [("i2", "f32"), ("i2", "bf16"), ("i3", "f32")])
def test_topk_rows_indexer_full(dev, orc, name, fmt):
    """The full-size workloads, every row against the oracle."""
    spec = configs.topk_rows_spec(name, fmt=fmt)
    check(dev, orc, configs.gen_indexer_scores(spec), spec["k"], "%s_%s" % (name, fmt))


def test_topk_rows_events_and_empty(dev):
    """The dispatch events are recorded, and rows = 0 enqueues nothing."""
    torch, moe = dev
    lib = moe.load()
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    arr = (ctypes.c_void_p * 2)(ev[0].value, ev[1].value)
    s = torch.rand((64, 4096), device="cuda")
    idx = torch.empty((64, 256), dtype=torch.int32, device="cuda")
    moe.moe_topk_rows(s, 256, idx, None, events=arr)
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    assert 0.0 < ms.value < 100.0
    for e in ev:
        hip.hipEventDestroy(e)
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.moe_topk_rows(None, 0, 4096, 8, None, None, None, ctypes.c_void_p(stream)) == 0


@pytest.mark.parametrize("n,k", [(32768, 1024), (65536, 1024), (20000, 512)])
def test_topk_rows_clustered(dev, orc, n, k):
    """High scores gathered in a few wavefronts' ranges (recent positions of an
    attention row, a block of equal scores at the cut): the sampled pass's
    compaction takes candidates from anywhere in the row."""
    rng = np.random.default_rng(n + 3 * k)
    rows = rng.standard_normal((4, n)).astype(np.float32)
    rows[0, -2000:] += 6.0                                 # the last 2000 positions score high
    rows[1, 100:1100] += 6.0                               # one block early in the row
    rows[2, -3 * k:] = np.float32(5.0)                     # 3k equal scores at the end: ties at the cut
    rows[3, ::97] += 8.0                                   # spread thinly over every wavefront
    check(dev, orc, rows, k, "clustered_n%d_k%d" % (n, k))


@pytest.mark.parametrize("name", ["all candidates equal", "bin whole", "one-wavefront pick",
                                  "radix on candidates", "full radix"])
def test_topk_rows_branches(dev, orc, name):
    """One row per branch of the sampled pass (rows built in topk_branch_rows,
    whose host-side check confirms the branch each takes), against the oracle."""
    from topk_branch_rows import branch_rows
    row, k = branch_rows()[name]
    check(dev, orc, row[None, :].copy(), k, "branch " + name)
