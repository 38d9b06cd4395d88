"""Least-squares gradients for the equal-shard identity (oracle; test infrastructure).

"Lab 09 -- Parallelism, simulated", s.2 "Data parallelism: why averaging is
exact": for a loss that is a mean over examples, the full-batch gradient is
the mean of the N equal shards' gradients, each shard's gradient being the
mean over its own examples.  For least squares, the gradient of
1/2 * mean((X w - y)^2) over n rows is X^T (X w - y) / n.
"""

import numpy as np


def lsq_grad(X, y, w):
    """X^T (X w - y) / n for the rows given."""
    X = np.asarray(X, dtype=np.float64)
    r = X @ np.asarray(w, dtype=np.float64) - np.asarray(y, dtype=np.float64)
    return (X.T @ r) / X.shape[0]


def shard_grads(X, y, w, nshards):
    """Each of ``nshards`` equal row blocks' own mean-loss gradient."""
    n = X.shape[0]
    assert n % nshards == 0
    rows = n // nshards
    return [lsq_grad(X[k * rows:(k + 1) * rows], y[k * rows:(k + 1) * rows], w)
            for k in range(nshards)]


def shard_sum_grads(X, y, w, sizes):
    """Per-shard gradients summed over the shard's rows, for row blocks of ``sizes``
    (unequal shards; "Lab 09", s.2: with unequal shards weight by tokens --
    sum the per-example losses and divide by the global count)."""
    X = np.asarray(X, dtype=np.float64)
    out, start = [], 0
    for s in sizes:
        Xs, ys = X[start:start + s], np.asarray(y, dtype=np.float64)[start:start + s]
        out.append(Xs.T @ (Xs @ np.asarray(w, dtype=np.float64) - ys))
        start += s
    return out


def shard_mean_grads(X, y, w, sizes):
    """Each shard's own mean-loss gradient for row blocks of ``sizes``."""
    return [g / s for g, s in zip(shard_sum_grads(X, y, w, sizes), sizes)]
