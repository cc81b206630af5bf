"""Rows of 32768 scores built to take each branch of the row top-k's sampled
pass, and a host-side restatement of the decision that picks the branch.

The sampled pass (rows of 16 or more keys per thread) takes as threshold T
the 16-bit prefix of the sample_rank-th largest of 256 sampled keys (the
middle chunk of every wavefront, every fourth lane), selects among the keys
>= T when there are between k and 8 * threads of them, and otherwise runs the
full radix passes.  Among the candidates it counts 4096 bins over [T, max
key]; the bin where the count from the top reaches k is then taken whole,
searched by one wavefront (at most 64 keys) or by radix passes on the
candidates (dense ties).  sampled_branch() restates that decision for
n = 32768 (1024 threads x 32 keys), so a CPU test can check that each row
takes the branch it is named after, and the GPU test runs the same rows
against the oracle.
"""
import numpy as np

N_BR, K_BR = 32768, 512


def _keys(row):
    u = row.view(np.uint32).astype(np.uint64)
    return np.where(u >> 31, (~u) & 0xFFFFFFFF, u | 0x80000000).astype(np.uint64)


def sampled_branch(row, k):
    threads, npt, waves = 1024, 32, 16
    key = _keys(row)
    kf = k * 256.0 / (threads * npt)
    r = int(np.ceil(kf + 4.0 * np.sqrt(kf) + 3.0))
    pos = np.array([w * npt * 64 + (npt // 2) * 64 + 4 * m for w in range(waves) for m in range(16)])
    samples = np.sort(key[pos])[::-1]
    T = int(samples[r - 1]) >> 16 << 16
    kmax = int(key.max())
    C = int((key >= T).sum())
    if T == 0 or C < k or C > 8 * threads:
        return "full radix"
    if T == kmax:
        return "all candidates equal"
    span = kmax - T
    sh = max(0, span.bit_length() - 12)
    bins = np.bincount(((key[key >= T] - T) >> sh).astype(np.int64), minlength=4096)
    above = 0
    for b in range(4095, -1, -1):
        if above + bins[b] >= k:
            rem, cbin = k - above, int(bins[b])
            return "bin whole" if rem == cbin else "one-wavefront pick" if cbin <= 64 else "radix on candidates"
        above += int(bins[b])
    raise AssertionError("k beyond the candidates")


def branch_rows():
    rng = np.random.default_rng(2024)
    base = lambda: rng.uniform(0.0, 0.5, N_BR).astype(np.float32)
    rows = {}
    r = base()
    r[::8] = 1.0                                   # half the samples and 4096 keys at the row's maximum
    rows["all candidates equal"] = (r, K_BR)
    r = base()
    r[64 * np.arange(K_BR) + 1] = 10.0 + 0.001 * np.arange(K_BR)  # exactly k keys far above the rest, none sampled
    rows["bin whole"] = (r, K_BR)
    rows["one-wavefront pick"] = (r.copy(), K_BR - 12)  # the same row, the cut inside a bin of about 16 keys
    r = base()
    r[64 * np.arange(300) + 1] = 20.0 + 0.001 * np.arange(300)
    r[64 * np.arange(400) + 3] = 5.0               # 400 equal keys at the cut: 212 of them needed
    rows["radix on candidates"] = (r, K_BR)
    r = base()
    pos = np.array([w * 2048 + 1024 + 4 * m for w in range(16) for m in range(16)])
    r[pos] = 10.0 + 0.01 * np.arange(256)          # every sample high: fewer than k keys reach T
    r[64 * np.arange(300) + 2] = 5.0 + 0.001 * np.arange(300)
    rows["full radix"] = (r, K_BR)
    return rows


