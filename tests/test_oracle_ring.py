"""The ring simulator against what "Lab 09 -- Parallelism, simulated" prints."""

import numpy as np
import pytest

from oracle.ring import (chunk_bounds, naive_gather_receive_bytes,
                         ring_all_reduce, ring_reduce_scatter)

LETTER = {"a": 0, "b": 1, "c": 2}


def _contributors(value):
    """Ranks whose contribution 2^r is inside an exact float64 partial sum."""
    v = int(value)
    assert v == value
    return {r for r in range(8) if v >> r & 1}


def test_n3_schedule_table(golden):
    # One element per chunk; rank r contributes 2^r to every chunk, so a
    # partial sum names its contributors exactly.
    arrays = [np.full(3, 2.0 ** r) for r in range(3)]
    results, sent, log = ring_all_reduce(arrays)
    rs = {(t, dst): (src, c, p) for ph, t, src, dst, c, p in log if ph == "RS"}
    ag = {(t, dst): (src, c, p) for ph, t, src, dst, c, p in log if ph == "AG"}
    owned, _ = ring_reduce_scatter(arrays)
    rows = golden("ring_n3_schedule.txt")
    assert len(rows) == 15
    for phase, step, rank, chunk, extra in rows:
        rank = int(rank)
        if phase == "RS":
            src, c, payload = rs[(int(step), rank)]
            assert src == (rank - 1) % 3
            assert c == LETTER[chunk]
            assert _contributors(payload[0]) == {int(x) for x in extra.split(",")}
        elif phase == "OWN":
            c, vals = owned[rank]
            assert c == LETTER[chunk]
            assert _contributors(vals[0]) == {0, 1, 2}
        else:
            src, c, payload = ag[(int(step), rank)]
            assert c == LETTER[chunk]
            assert src == int(extra.split("=")[1])
            assert _contributors(payload[0]) == {0, 1, 2}
    for r in range(3):
        assert np.all(results[r] == 7.0)


@pytest.mark.parametrize("row", [0, 1, 2])
def test_bytes_per_rank_64_float64(golden, row):
    n, ring_bytes, naive = (int(x) for x in golden("ring_bytes.txt")[row])
    rng = np.random.default_rng(n)
    arrays = [rng.standard_normal(64) for _ in range(n)]
    _, sent, _ = ring_all_reduce(arrays)
    assert sent == [ring_bytes] * n
    assert naive_gather_receive_bytes(64 * 8, n) == naive


@pytest.mark.parametrize("k", [2, 3, 4, 5, 8, 16])
def test_eq_13_5_1_bytes(k):
    # "13.5 Multi-GPU from First Principles", Eq. (13.5.1): 2(k-1)/k * N bytes
    # per device for an N-byte vector split into k equal chunks.
    length = 12 * k
    arrays = [np.zeros(length, dtype=np.float32) for _ in range(k)]
    _, sent, _ = ring_all_reduce(arrays)
    nbytes = length * 4
    assert all(s * k == 2 * (k - 1) * nbytes for s in sent)


@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_integer_data_equals_numpy_sum(n):
    rng = np.random.default_rng(100 + n)
    arrays = [rng.integers(-1000, 1000, size=64).astype(np.float64) for _ in range(n)]
    results, _, _ = ring_all_reduce(arrays)
    expect = np.sum(np.stack(arrays), axis=0)
    for r in range(n):
        assert np.array_equal(results[r], expect)


@pytest.mark.parametrize("n", [3, 4, 8])
def test_allgather_from_wrong_chunk_corrupts(n):
    # "Common bugs": starting the all-gather from chunk r instead of the
    # finished chunk (r + 1) mod N overwrites correct sums with partial ones.
    arrays = [np.full(8 * n, 2.0 ** r) for r in range(n)]
    good, _, _ = ring_all_reduce(arrays)
    bad, _, _ = ring_all_reduce(arrays, ag_start_offset=0)
    full = float(2 ** n - 1)
    assert all(np.all(g == full) for g in good)
    assert any(np.any(b != full) for b in bad)


def test_star_example(golden):
    rows = golden("star_allreduce.txt")
    before = [np.array([float(x) for x in r[1:r.index("|")]]) for r in rows]
    after = [np.array([float(x) for x in r[r.index("|") + 1:]]) for r in rows]
    results, _, _ = ring_all_reduce(before)
    for got, want in zip(results, after):
        assert np.array_equal(got, want)


@pytest.mark.parametrize("length,n", [(64, 3), (10, 4), (7, 8), (0, 2), (5, 5), (100, 7)])
def test_chunk_bounds_match_array_split(length, n):
    parts = np.array_split(np.arange(length), n)
    bounds = chunk_bounds(length, n)
    assert [hi - lo for lo, hi in bounds] == [len(p) for p in parts]
    assert [lo for lo, _ in bounds] == [int(p[0]) if len(p) else lo for p, (lo, _) in zip(parts, bounds)]
