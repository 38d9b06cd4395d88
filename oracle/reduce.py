"""Reduce-scatter-mean in the ring's fold order (oracle; test infrastructure).

What is computed, with its sources:

* Chunk c of a bucket is the c-th ``array_split`` piece of it ("Lab 09 --
  Parallelism, simulated", s.1: each vector is split into N chunks).
* The finished sum of chunk c is built around the ring: it starts as rank c's
  values (rank c sends chunk c in reduce-scatter step 0), then ranks c + 1,
  c + 2, ..., c + N - 1 (mod N) each add their own values to the partial sum
  they received ("Tips": in step t rank r sends chunk (r - t) mod N).  The
  last rank to add, (c - 1) mod N, owns the chunk; equivalently rank r owns
  chunk (r + 1) mod N (the "owns sum(b) / sum(c) / sum(a)" row of the N = 3
  table in s.1).
* The average is the full sum divided by N exactly once: s.2 of "Lab 09"
  (one all-reduce, sum then divide by N) and "Part 3 -- Gradient Reduction"
  of "A4 -- Multi-GPU with NCCL and ZeRO-1" (ncclAvg divides by N; "Common
  Mistakes": dividing twice is a bug).
* A flat arena is split into buckets, each bucket into N chunks; the ZeRO-1
  shard of rank r is chunk (r + 1) mod N of every bucket, concatenated in
  plan order ("A4", "Common Mistakes": offset into the layer first, then into
  the shard).  Sharding requires every bucket length to be divisible by N
  ("Part 2 -- Tensor Sharding" makes an uneven split an error).

Precision (a reading, the pages do not fix it): bf16 and fp32 gradients are
widened to fp32 and accumulated in fp32, rounding after every addition;
float64 inputs stay in float64.  bf16 is the top half of an IEEE binary32, so
widening is exact.

Wire precision (the bf16-wire mode): "13.5 Multi-GPU from First Principles",
exercise 8 ("Gradients in bf16"): a ring that sends bf16 rounds the partial sum
to bf16 once per hop -- each reduce-scatter hop adds the incoming partial sum
to the local chunk.  With ``wire="bf16"`` every addition of the fold is done in
fp32 and its result rounded to bf16 (round to nearest even) before the next
hop; the last hop's sum is rounded too, as the owner keeps it in bf16; the
mean is then that bf16 sum divided by N in fp32.

Pins (tests/test_oracle_reduce.py): the fold equals the message-passing ring
simulator of ``oracle.ring`` bit for bit for N in {2, 3, 4, 8}; on integer
valued data it equals ``numpy.sum``; the star example of "13.5 Multi-GPU from
First Principles" (1 + 2 = 3); the equal-shard identity of s.2 of "Lab 09" on
least squares; the bf16 widening against torch's CPU conversion for all 2^16
patterns; and the "Common bugs" (summing, or dividing twice, misses the
full-batch gradient by a factor N).
"""

import numpy as np

from .bf16 import bf16_round
from .ring import chunk_bounds


def owned_chunk(rank, nranks):
    """Chunk that rank ``rank`` holds fully reduced after the reduce-scatter."""
    return (rank + 1) % nranks


def chunk_owner(chunk, nranks):
    """Rank that owns chunk ``chunk`` after the reduce-scatter."""
    return (chunk - 1) % nranks


def widen(values, kind):
    """Gradient values as the accumulation type.

    ``kind`` is ``"bf16"`` (``values`` holds the uint16 bit patterns),
    ``"f32"`` or ``"f64"``.  A bf16 value is the binary32 whose upper 16 bits
    are its pattern and whose lower 16 bits are zero.
    """
    if kind == "bf16":
        bits = np.asarray(values, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32)
    if kind == "f32":
        return np.array(values, dtype=np.float32, copy=True)
    if kind == "f64":
        return np.array(values, dtype=np.float64, copy=True)
    raise ValueError(f"unknown gradient kind {kind!r}")


def wire_round(values, wire):
    """What one hop of a ring sends: the partial sum as is, or rounded to bf16."""
    if wire is None:
        return values
    if wire == "bf16":
        return widen(bf16_round(values), "bf16")
    raise ValueError(f"unknown wire precision {wire!r}")


def ring_fold(contribs, chunk, wire=None):
    """Sum of chunk ``chunk`` in ring order.

    ``contribs[j]`` holds rank j's (widened) values of that chunk.  The sum
    starts with rank ``chunk``'s values and adds ranks chunk+1, chunk+2, ...
    (mod N) one at a time, rounding after each addition (to the accumulation
    type, then to the wire precision if one is given).
    """
    n = len(contribs)
    acc = np.array(contribs[chunk % n], copy=True)
    for j in range(1, n):
        acc = wire_round(contribs[(chunk + j) % n] + acc, wire)
    return acc


def chunk_mean(contribs, chunk, average=True, wire=None, divisor=None):
    """Ring-order sum of one chunk, divided once by N -- or by ``divisor``, the
    global token count of a token-weighted mean -- unless ``average`` is False."""
    acc = ring_fold(contribs, chunk, wire)
    if average:
        d = len(contribs) if divisor is None else divisor
        acc = acc / acc.dtype.type(d)
    return acc


def shard_segments(buckets, nranks, chunk, uneven=False):
    """Where the ZeRO-1 shard of chunk ``chunk`` lives.

    Returns ``[(global_start, length, compact_start)]``, one entry per bucket
    in plan order.  Raises ``ValueError`` when a bucket length is not
    divisible by N and ``uneven`` is False.
    """
    out = []
    compact = 0
    for off, length in buckets:
        if not uneven and length % nranks != 0:
            raise ValueError(
                f"bucket of {length} elements cannot be split evenly over {nranks} ranks")
        lo, hi = chunk_bounds(length, nranks)[chunk]
        out.append((off + lo, hi - lo, compact))
        compact += hi - lo
    return out


def reduce_scatter_mean(rank_arenas, kind, buckets, chunk, average=True,
                        uneven=False, compact_inputs=False, arena_len=None, wire=None,
                        token_counts=None):
    """Reduce-scatter-mean of N rank arenas over a bucket plan.

    * ``rank_arenas[j]`` -- rank j's flat gradient arena (global layout), or,
      with ``compact_inputs``, only rank j's values of the chunks being
      reduced, concatenated in plan order (shard-compact).
    * ``buckets`` -- ``[(offset, length)]`` in processing order.
    * ``chunk >= 0`` -- reduce that chunk of every bucket (ZeRO-1
      reduce-scatter); returns the shard-compact result.
    * ``chunk == -1`` -- reduce every chunk of every bucket (all-reduce, plain
      data parallelism); returns a globally indexed array of ``arena_len``
      elements, NaN where no bucket covers it.  Chunks may be uneven here.
    * ``wire`` -- None (sum in the accumulation type) or ``"bf16"`` (each hop's
      partial sum rounded to bf16; bf16 inputs only).
    * ``token_counts`` -- per-rank token counts when each rank holds the sum of
      its per-token gradients: the result is the sum over ranks divided by the
      total count ("Lab 09", s.2, weight by tokens; "13.5 Multi-GPU from First
      Principles", exercise 2).
    """
    divisor = None if token_counts is None else int(sum(int(c) for c in token_counts))
    if wire is not None and kind != "bf16":
        raise ValueError("the bf16 wire applies to bf16 gradients")
    n = len(rank_arenas)
    acc_dtype = np.float64 if kind == "f64" else np.float32
    if chunk >= 0:
        segs = shard_segments(buckets, n, chunk, uneven=uneven)
        total = sum(s[1] for s in segs)
        out = np.empty(total, dtype=acc_dtype)
        for gstart, length, cstart in segs:
            src = cstart if compact_inputs else gstart
            contribs = [widen(a[src:src + length], kind) for a in rank_arenas]
            out[cstart:cstart + length] = chunk_mean(contribs, chunk, average, wire, divisor)
        return out
    if compact_inputs:
        raise ValueError("compact inputs only exist for a single chunk")
    if arena_len is None:
        arena_len = max(off + length for off, length in buckets) if buckets else 0
    out = np.full(arena_len, np.nan, dtype=acc_dtype)
    for off, length in buckets:
        for c, (lo, hi) in enumerate(chunk_bounds(length, n)):
            contribs = [widen(a[off + lo:off + hi], kind) for a in rank_arenas]
            out[off + lo:off + hi] = chunk_mean(contribs, c, average, wire, divisor)
    return out
