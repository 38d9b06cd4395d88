"""The ring-order fold against the simulator, closed forms and library routines."""

import numpy as np
import pytest
import torch

from oracle.lsq import lsq_grad, shard_grads
from oracle.reduce import (chunk_mean, chunk_owner, owned_chunk, reduce_scatter_mean,
                           ring_fold, shard_segments, widen)
from oracle.ring import chunk_bounds, ring_all_reduce, ring_reduce_scatter


@pytest.mark.parametrize("n", [2, 3, 4, 5, 8, 13, 16])
@pytest.mark.parametrize("dtype", [np.float32, np.float64])
@pytest.mark.parametrize("length", [64, 67])
def test_fold_equals_simulated_ring(n, dtype, length):
    # Gaussian data: float addition is not associative, so only the exact
    # order the ring uses reproduces the simulator's bits.
    rng = np.random.default_rng(7 * n + length)
    arrays = [rng.standard_normal(length).astype(dtype) * dtype(10.0 ** rng.integers(-3, 3))
              for _ in range(n)]
    owned, _ = ring_reduce_scatter(arrays)
    bounds = chunk_bounds(length, n)
    for r in range(n):
        c, vals = owned[r]
        assert c == owned_chunk(r, n) and chunk_owner(c, n) == r
        lo, hi = bounds[c]
        folded = ring_fold([a[lo:hi] for a in arrays], c)
        assert folded.dtype == dtype
        assert np.array_equal(folded, vals)
    full, _, _ = ring_all_reduce(arrays)
    summed = reduce_scatter_mean(arrays, "f64" if dtype == np.float64 else "f32",
                                 [(0, length)], -1, average=False)
    for r in range(n):
        assert np.array_equal(full[r].astype(summed.dtype), summed)


def test_fold_order_is_observable():
    # The test above bites: a fold that starts at rank 0 instead of rank c
    # disagrees with the ring on this data.
    rng = np.random.default_rng(3)
    n = 8
    arrays = [rng.standard_normal(4096).astype(np.float32) for _ in range(n)]
    c = 5
    ring = ring_fold(arrays, c)
    plain = arrays[0].copy()
    for j in range(1, n):
        plain = arrays[j] + plain
    assert not np.array_equal(ring, plain)


@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_integer_data_mean_is_sum_over_n(n):
    rng = np.random.default_rng(n)
    arrays = [rng.integers(-50, 50, size=96).astype(np.float64) for _ in range(n)]
    got = reduce_scatter_mean(arrays, "f64", [(0, 96)], -1)
    assert np.array_equal(got, np.sum(np.stack(arrays), axis=0) / n)


def test_bf16_widening_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("integer", [True, False])
def test_equal_shard_identity_least_squares(integer):
    # "Lab 09", s.2 and "What to implement" item 7: the mean of 8 equal-shard
    # gradients equals X^T (X w - y) / 64; X is 64 x 32 as in the page's demo.
    rng = np.random.default_rng(11)
    if integer:
        X = rng.integers(-3, 4, size=(64, 32)).astype(np.float64)
        y = rng.integers(-3, 4, size=64).astype(np.float64)
        w = rng.integers(-3, 4, size=32).astype(np.float64)
    else:
        X, y, w = rng.standard_normal((64, 32)), rng.standard_normal(64), rng.standard_normal(32)
    full = lsq_grad(X, y, w)
    shards = shard_grads(X, y, w, 8)
    mean = reduce_scatter_mean(shards, "f64", [(0, 32)], -1)
    if integer:
        assert np.array_equal(mean, full)
    else:
        np.testing.assert_allclose(mean, full, rtol=1e-13, atol=1e-14 * np.abs(full).max())
    # "Common bugs": summing is N times too large, dividing twice N times too small.
    summed = reduce_scatter_mean(shards, "f64", [(0, 32)], -1, average=False)
    np.testing.assert_allclose(summed, 8 * full, rtol=1e-12, atol=1e-12)
    assert not np.allclose(summed, full)
    twice = mean / 8
    assert not np.allclose(twice, full)


def test_shard_compact_layout_and_divisibility():
    n = 4
    buckets = [(40, 24), (0, 40)]  # processing order: the later arena range first
    rng = np.random.default_rng(5)
    arrays = [rng.standard_normal(64).astype(np.float32) for _ in range(n)]
    full = reduce_scatter_mean(arrays, "f32", buckets, -1)
    for r in range(n):
        c = owned_chunk(r, n)
        shard = reduce_scatter_mean(arrays, "f32", buckets, c)
        segs = shard_segments(buckets, n, c)
        assert [s[2] for s in segs] == [0, 6]
        for g, length, cstart in segs:
            assert np.array_equal(shard[cstart:cstart + length], full[g:g + length])
        compact_in = [np.concatenate([a[g:g + l] for g, l, _ in segs]) for a in arrays]
        again = reduce_scatter_mean(compact_in, "f32", buckets, c, compact_inputs=True)
        assert np.array_equal(again, shard)
    with pytest.raises(ValueError):
        reduce_scatter_mean(arrays, "f32", [(0, 62)], 1)  # "Part 2": an uneven split is an error
    uneven = reduce_scatter_mean(arrays, "f32", [(0, 62)], 1, uneven=True)
    assert uneven.shape == (16,)


def test_single_rank_is_identity():
    x = np.random.default_rng(1).standard_normal(33).astype(np.float32)
    assert np.array_equal(chunk_mean([x], 0), x)


# --- the bf16 wire ("13.5 Multi-GPU from First Principles", exercise 8) -----

from oracle.bf16 import bf16_round  # noqa: E402
from oracle.reduce import wire_round  # noqa: E402


def _bf16_vectors(rng, n, length, scale=1e-3):
    return [bf16_round((rng.standard_normal(length) * scale).astype(np.float32))
            for _ in range(n)]


@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_bf16_wire_fold_equals_simulated_bf16_ring(n):
    rng = np.random.default_rng(70 + n)
    bits = _bf16_vectors(rng, n, 67)
    vals = [widen(b, "bf16") for b in bits]
    full, _, _ = ring_all_reduce(vals, wire_round=lambda x: wire_round(x, "bf16"))
    for c, (lo, hi) in enumerate(chunk_bounds(67, n)):
        folded = ring_fold([v[lo:hi] for v in vals], c, wire="bf16")
        for r in range(n):
            assert np.array_equal(full[r][lo:hi], folded)
    assert np.all(full[0].view(np.uint32) & np.uint32(0xFFFF) == 0)  # bf16 on the wire
    got = reduce_scatter_mean(bits, "bf16", [(0, 67)], -1, average=False, wire="bf16")
    assert np.array_equal(got, full[0])


def test_bf16_wire_exact_when_partial_sums_are_bf16_exact():
    # Integers |x| < 16 summed over 8 ranks stay below 128: every partial sum
    # is a bf16 value, so rounding per hop changes nothing.
    rng = np.random.default_rng(71)
    ints = [rng.integers(-15, 16, 512).astype(np.float32) for _ in range(8)]
    bits = [bf16_round(x) for x in ints]
    wire = reduce_scatter_mean(bits, "bf16", [(0, 512)], -1, average=False, wire="bf16")
    assert np.array_equal(wire, np.sum(np.stack(ints), axis=0))


def test_bf16_wire_differs_from_fp32_accumulation_on_gaussian_data():
    rng = np.random.default_rng(72)
    bits = _bf16_vectors(rng, 8, 4096)
    wire = reduce_scatter_mean(bits, "bf16", [(0, 4096)], 3, wire="bf16")
    fp32 = reduce_scatter_mean(bits, "bf16", [(0, 4096)], 3)
    assert not np.array_equal(wire, fp32)
    with pytest.raises(ValueError):
        reduce_scatter_mean([np.zeros(8, np.float32)] * 2, "f32", [(0, 8)], 0, wire="bf16")


def bf16_wire_error_study(ks=(2, 8, 64), length=1 << 16, seed=73):
    """Relative error (2-norm) against the exact sum of fp32 gradients for
    (a) bf16 inputs summed with a bf16 wire (rounded every hop) and (b) bf16
    inputs summed in fp32 (rounded once, on the way in)."""
    rng = np.random.default_rng(seed)
    out = {}
    for k in ks:
        xs = [(rng.standard_normal(length) * 1e-3).astype(np.float32) for _ in range(k)]
        exact = np.sum(np.stack(xs).astype(np.float64), axis=0)
        bits = [bf16_round(x) for x in xs]
        per_hop = reduce_scatter_mean(bits, "bf16", [(0, length)], -1, average=False,
                                      wire="bf16")
        once = reduce_scatter_mean(bits, "bf16", [(0, length)], -1, average=False)
        nrm = np.linalg.norm(exact)
        out[k] = (float(np.linalg.norm(per_hop - exact) / nrm),
                  float(np.linalg.norm(once - exact) / nrm))
    return out


def test_bf16_wire_error_grows_with_k_and_fp32_accumulation_does_not():
    err = bf16_wire_error_study()
    hop = [err[k][0] for k in (2, 8, 64)]
    once = [err[k][1] for k in (2, 8, 64)]
    assert hop[0] < hop[1] < hop[2]                # per-hop rounding accumulates
    assert max(once) < 2 * min(once)               # one rounding per input: flat in k
    assert hop[2] > 3 * once[2]                    # at k = 64 the wire dominates
    # Both are within bf16's unit roundoff scale: 2^-8 relative per rounding.
    assert once[0] < 2 ** -8 and hop[2] < 2 ** -8 * 64


# --- token-weighted mean for unequal shards -----------------------------------

from oracle.lsq import shard_mean_grads, shard_sum_grads  # noqa: E402


@pytest.mark.parametrize("integer", [True, False])
def test_token_weighted_mean_is_the_full_batch_gradient(integer):
    # "Lab 09", s.2: 65 rows over 8 ranks; the plain average of the shards'
    # means misses the full-batch gradient, weighting by tokens does not.
    rng = np.random.default_rng(80)
    sizes = [9, 8, 8, 8, 8, 8, 8, 8]
    if integer:
        X = rng.integers(-3, 4, size=(65, 32)).astype(np.float64)
        y = rng.integers(-3, 4, size=65).astype(np.float64)
        w = rng.integers(-3, 4, size=32).astype(np.float64)
    else:
        X, y, w = rng.standard_normal((65, 32)), rng.standard_normal(65), rng.standard_normal(32)
    full = lsq_grad(X, y, w)
    sums = shard_sum_grads(X, y, w, sizes)
    weighted = reduce_scatter_mean(sums, "f64", [(0, 32)], -1, token_counts=sizes)
    if integer:
        assert np.array_equal(weighted, full)
    else:
        np.testing.assert_allclose(weighted, full, rtol=1e-12, atol=1e-13 * np.abs(full).max())
    plain = reduce_scatter_mean(shard_mean_grads(X, y, w, sizes), "f64", [(0, 32)], -1)
    miss = np.abs(plain - full).max() / np.abs(full).max()
    assert miss > 1e-3  # the page's draw missed by 1.4% of the largest component


def test_token_weights_of_the_two_recipes():
    # "13.5 Multi-GPU from First Principles", exercise 2b: shards of 3000 and
    # 1000 tokens.  Averaging the shards' means gives a token on the first
    # shard 2/3 and one on the second 2 times its full-batch weight; the
    # token-weighted mean gives every token weight exactly 1.
    counts = [3000, 1000]
    for shard in (0, 1):
        # one unit of gradient on every token of `shard`, none on the other
        sums = [np.array([float(counts[r] if r == shard else 0)]) for r in range(2)]
        means = [s / c for s, c in zip(sums, counts)]
        full = counts[shard] / sum(counts)
        recipe_b = reduce_scatter_mean(means, "f64", [(0, 1)], -1)[0]
        exact = reduce_scatter_mean(sums, "f64", [(0, 1)], -1, token_counts=counts)[0]
        assert recipe_b / full == pytest.approx([2 / 3, 2.0][shard], rel=1e-15)
        assert exact == full


def test_least_squares_gradient_against_autograd():
    # The closed form X^T (X w - y) / n against torch's autograd of
    # 1/2 * mean((X w - y)^2) ("Lab 09", s.2).
    rng = np.random.default_rng(82)
    X, y, w = rng.standard_normal((64, 32)), rng.standard_normal(64), rng.standard_normal(32)
    wt = torch.tensor(w, requires_grad=True)
    loss = 0.5 * torch.mean((torch.from_numpy(X) @ wt - torch.from_numpy(y)) ** 2)
    loss.backward()
    np.testing.assert_allclose(lsq_grad(X, y, w), wt.grad.numpy(), rtol=1e-12, atol=1e-14)
    sizes = [9, 8, 8, 8, 8, 8, 8, 7]
    sums = shard_sum_grads(X, y, w, sizes)
    np.testing.assert_allclose(np.sum(sums, axis=0) / 64, lsq_grad(X, y, w), rtol=1e-12)


@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_ring_fold_is_within_the_recursive_summation_bound(n):
    # The fp32 fold in ring order against the exact sum (fp64 fsum of the
    # widened values): recursive summation of n terms errs by at most
    # (n - 1) u * sum|x_i| with u = 2^-24 (Higham, "Accuracy and Stability of
    # Numerical Algorithms", s.4.2), plus the final division's half ulp.
    import math
    rng = np.random.default_rng(100 + n)
    contribs = [(rng.standard_normal(4096) * 10.0 ** rng.integers(-3, 3)).astype(np.float32)
                for _ in range(n)]
    for chunk in (0, n - 1):
        got = chunk_mean(contribs, chunk).astype(np.float64)
        exact = np.array([math.fsum(float(c[i]) for c in contribs)
                          for i in range(4096)]) / n
        absum = np.sum(np.abs(np.stack(contribs).astype(np.float64)), axis=0) / n
        u = 2.0 ** -24
        bound = (n - 1) * u * absum * (1 + u) + u * np.abs(exact) + 1e-300
        assert np.all(np.abs(got - exact) <= bound)
        if n == 2:  # one rounding (the division by 2 is exact): the correctly rounded mean
            assert np.array_equal(got, exact.astype(np.float32).astype(np.float64))
        else:  # several roundings: the order shows
            assert np.any(got != exact.astype(np.float32))
