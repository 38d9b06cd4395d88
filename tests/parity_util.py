"""Helpers shared by the GPU parity tests: host copies, oracle states, sampling.

The oracle is only ever fed the same bytes the GPU path received (copied
device -> host); no expected value comes from the GPU path.
"""

import numpy as np
import torch

from oracle.reduce import chunk_mean, owned_chunk, shard_segments, widen
from oracle.ring import chunk_bounds
from workloads import to_bits


def host(t):
    return to_bits(t)


def oracle_states(master_host, buckets, n, uneven=False):
    """Each rank's shard-compact (master, m, v) at t = 0."""
    out = []
    for r in range(n):
        segs = shard_segments(buckets, n, owned_chunk(r, n), uneven)
        w = np.concatenate([master_host[g:g + l] for g, l, _ in segs]) if segs else \
            np.zeros(0, np.float32)
        out.append((w, np.zeros_like(w), np.zeros_like(w)))
    return out


def assert_bits(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    if got.dtype.kind == "f":
        same = (got.view(np.uint32 if got.itemsize == 4 else np.uint64) ==
                want.view(np.uint32 if want.itemsize == 4 else np.uint64))
        both_nan = np.isnan(got) & np.isnan(want)
        bad = ~(same | both_nan)
    else:
        bad = got != want
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; first at {i}: "
                             f"{got[i]!r} vs {want[i]!r}")


def max_rel(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.maximum(np.abs(want), 1e-30)
    return float(np.max(np.abs(got - want) / den)) if got.size else 0.0


def chunk_of_index(buckets, n, idx):
    """(bucket b, chunk c, arena start of chunk) of arena indices ``idx``."""
    out_b = np.empty(idx.size, np.int64)
    out_c = np.empty(idx.size, np.int64)
    for b, (off, length) in enumerate(buckets):
        for c, (lo, hi) in enumerate(chunk_bounds(length, n)):
            sel = (idx >= off + lo) & (idx < off + hi)
            out_b[sel] = b
            out_c[sel] = c
    return out_b, out_c


def sample_indices(length, count, seed, extra=()):
    """Sorted unique sample of [0, length): random picks, both ends, and ``extra``."""
    rng = np.random.default_rng(seed)
    pick = rng.integers(0, max(length, 1), size=min(count, max(length, 1)))
    edges = [0, 1, 7, 8, length // 2, length - 9, length - 8, length - 1]
    s = np.concatenate([pick, np.array([e for e in list(edges) + list(extra)
                                        if 0 <= e < length], np.int64)])
    return np.unique(s)


def gather_host(t, idx):
    """Values of a device tensor at host indices ``idx`` (bf16 as uint16 bits)."""
    sel = torch.from_numpy(idx).to(t.device)
    return to_bits(t.index_select(0, sel))


def oracle_mean_at(contribs_at, chunk_ids, kind, average=True):
    """Oracle mean of sampled elements: ``contribs_at[j]`` = rank j's values there."""
    acc_dtype = np.float64 if kind == "f64" else np.float32
    out = np.empty(chunk_ids.size, acc_dtype)
    for c in np.unique(chunk_ids):
        sel = chunk_ids == c
        out[sel] = chunk_mean([widen(a[sel], kind) for a in contribs_at], int(c), average)
    return out


def _fan_blocks(x):
    """The library's block fold of each 4096 consecutive values of ``x``: lane l
    of 256 adds values l, l + 256, ..., l + 3840 of the block in that order
    (from +0.0, skipping values past the end), the lanes of each 64-wide wave
    combine by an xor butterfly (every lane ends with the same bits), and the
    four waves' sums combine as (w0 + w1) + (w2 + w3)."""
    x = np.asarray(x, np.float64)
    n = x.size
    nl = max(1, -(-n // 4096))
    pad = np.zeros(nl * 4096)
    pad[:n] = x
    mask = np.zeros(nl * 4096, bool)
    mask[:n] = True
    v = pad.reshape(nl, 16, 256)
    m = mask.reshape(nl, 16, 256)
    s = np.zeros((nl, 256))
    for k in range(16):
        s = np.where(m[:, k], s + v[:, k], s)
    w = s.reshape(nl, 4, 64)
    for step in (1, 2, 4, 8, 16, 32):
        w = w + w[:, :, np.arange(64) ^ step]
    return (w[:, 0, 0] + w[:, 1, 0]) + (w[:, 2, 0] + w[:, 3, 0])


def fixed_tree_sum(x):
    """The norm's fixed combine order, emulated on the host: block folds level
    by level until at most 4096 values are left, then one last block fold.  A
    test of the kernels' tree shape (not of the method: the oracle sums the
    squares exactly)."""
    x = np.asarray(x, np.float64)
    while x.size > 4096:
        x = _fan_blocks(x)
    return float(_fan_blocks(x)[0])
