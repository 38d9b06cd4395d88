"""The reduce on seeded random plans, against the oracle.

Each case draws N (1..16), the gradient type, even or array_split chunks, a
few buckets whose arena order differs from their processing order, a chunk to
reduce and the output layout (shard-compact, arena offsets, or every chunk).
The mean is compared bit for bit; each piece sum (GRZ_PIECE values of one
chunk, numbered bucket by bucket, chunk 0..N-1, piece by piece) against the
exact sum of the squares of the oracle's mean over the same elements.
"""

import math

import numpy as np
import pytest
import torch

import gradient_reduce_zero_amd as grz
from oracle.bf16 import bf16_round
from oracle.reduce import reduce_scatter_mean, shard_segments
from oracle.ring import chunk_bounds
from oracle.step import held_gradient
from parity_util import assert_bits, host
from workloads import rank_grad

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
PIECE = grz.GRZ_PIECE


def _draw(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 17))
    kind = ["bf16", "f32", "f64"][int(rng.integers(0, 3))]
    even = bool(rng.integers(0, 2))
    lengths = [int(x) for x in rng.integers(0, 3 * PIECE + 60, size=int(rng.integers(1, 5)))]
    if even:
        lengths = [l - l % n for l in lengths]
    if sum(lengths) == 0:
        lengths[0] = 8 * n
    order = rng.permutation(len(lengths))
    offs, pos = [0] * len(lengths), 0
    for i in order:
        offs[i] = pos
        pos += lengths[i]
    mode = ["compact", "global", "all"][int(rng.integers(0, 3))]
    chunk = -1 if mode == "all" else int(rng.integers(0, n))
    return n, kind, even, list(zip(offs, lengths)), pos, chunk, mode


def _pieces_of(mean_global, buckets, n, chunks, bucket_ids=None):
    """Exact sum of squares per piece, in the plan's piece numbering; None for
    pieces of chunks not reduced (and of buckets outside ``bucket_ids``)."""
    out = []
    for b, (off, length) in enumerate(buckets):
        for c, (lo, hi) in enumerate(chunk_bounds(length, n)):
            for p0 in range(lo, hi, PIECE):
                p1 = min(p0 + PIECE, hi)
                if c in chunks and (bucket_ids is None or b in bucket_ids):
                    vals = mean_global[off + p0:off + p1].astype(np.float64)
                    out.append(math.fsum((vals * vals).tolist()))
                else:
                    out.append(None)
    return out


@pytest.mark.parametrize("seed", range(24))
def test_reduce_on_a_random_plan(seed):
    n, kind, even, buckets, p, chunk, mode = _draw(1000 + seed)
    flags = 0 if even else grz.GRZ_UNEVEN
    if mode == "global":
        flags |= grz.GRZ_OUT_GLOBAL
    grads = [rank_grad(p, 1e-2, kind, 7000 + 31 * seed + r, device=DEV) for r in range(n)]
    acc = np.float64 if kind == "f64" else np.float32
    out_t = torch.float64 if kind == "f64" else torch.float32
    npieces = grz.dp_piece_count(buckets, n, flags)
    parts = torch.full((max(npieces, 1),), -1.0, dtype=torch.float64, device=DEV)
    shard = grz.dp_shard_numel(buckets, n, chunk, flags) if chunk >= 0 else p
    out = torch.full((max(shard if mode == "compact" else p, 1),), float("nan"), dtype=out_t,
                     device=DEV)
    grz.dp_reduce_scatter_mean(grads, buckets, chunk, out, parts, flags=flags)
    torch.cuda.synchronize()
    hg = [host(g) for g in grads]
    mean_global = np.full(p, np.nan, acc)
    chunks = range(n) if chunk < 0 else [chunk]
    for c in chunks:
        comp = reduce_scatter_mean(hg, kind, buckets, c, uneven=not even)
        for g0, length, c0 in shard_segments(buckets, n, c, uneven=not even):
            mean_global[g0:g0 + length] = comp[c0:c0 + length]
    if mode == "compact":
        want = reduce_scatter_mean(hg, kind, buckets, chunk, uneven=not even)
        assert_bits(host(out)[:shard], want, f"seed {seed}: shard-compact mean")
    else:
        assert_bits(host(out)[:p], mean_global, f"seed {seed}: mean at arena offsets")
    got = host(parts)
    for i, want_i in enumerate(_pieces_of(mean_global, buckets, n, set(chunks))):
        if want_i is None:
            assert got[i] == -1.0, f"seed {seed}: piece {i} of a chunk not reduced was written"
        else:
            assert math.isclose(got[i], want_i, rel_tol=1e-13, abs_tol=0.0), (seed, i)


@pytest.mark.parametrize("held", ["f32", "bf16"])
@pytest.mark.parametrize("seed", range(16))
def test_update_on_a_random_plan(seed, held):
    # Clipped AdamW on the shard of a random chunk (or the whole plan) with the
    # bf16 write into 1-3 replicas: state bit-exact against the oracle's AdamW
    # on the same inputs, the replicas equal to the oracle's rounding at the
    # shard's arena offsets and untouched elsewhere.  held="bf16": the mean
    # gradient is a shard held in bf16 (GRZ_MEAN_BF16), widened exactly.
    from oracle.step import Hyper as OHyper
    from oracle.step import adamw

    rng = np.random.default_rng(5000 + seed)
    n, _, even, buckets, p, chunk, _ = _draw(2000 + seed)
    if rng.integers(0, 4) == 0:
        chunk = -1
    flags = 0 if even else grz.GRZ_UNEVEN
    t = int(rng.integers(1, 4))
    warmup = int(rng.integers(0, 3))
    scale = np.float32(rng.uniform(0.05, 1.0)) if rng.integers(0, 2) else np.float32(1.0)
    nrep = int(rng.integers(1, 4))
    if chunk >= 0:
        segs = shard_segments(buckets, n, chunk, uneven=not even)
        numel = sum(s[1] for s in segs)
    else:
        segs = [(off, length, off) for off, length in buckets]
        numel = p
    w = rng.standard_normal(numel).astype(np.float32) * np.float32(0.02)
    m = rng.standard_normal(numel).astype(np.float32) * np.float32(1e-3)
    v = np.abs(rng.standard_normal(numel)).astype(np.float32) * np.float32(1e-6)
    g = rng.standard_normal(numel).astype(np.float32) * np.float32(1e-2)
    hyper = grz.Hyper(lr=1e-3, warmup=warmup)
    dev = [torch.from_numpy(a.copy()).to(DEV) for a in (w, m, v, g)]
    if numel == 0:
        dev = [torch.zeros(1, device=DEV) for _ in range(4)]
    if held == "bf16":
        gb = bf16_round(g)
        g = held_gradient(g, "bf16")
        dev[3] = torch.from_numpy(gb.view(np.int16).copy()).to(DEV).view(torch.bfloat16) \
            if numel else torch.zeros(1, dtype=torch.bfloat16, device=DEV)
    sentinel = 0x7A5C  # a bf16 bit pattern no update writes here
    reps = [torch.full((p,), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
            for _ in range(nrep)]
    grz.zero1_adamw_gather(dev[0], dev[1], dev[2], dev[3], buckets, n, chunk,
                           torch.tensor([scale], device=DEV),
                           grz.adamw_args(**grz.step_scalars(hyper, t)), reps, flags=flags)
    torch.cuda.synchronize()
    s = OHyper(lr=1e-3, warmup=warmup).scalars(t)
    w1, m1, v1 = adamw(w, m, v, g * scale, **s)
    for k, want in enumerate((w1, m1, v1)):
        assert_bits(host(dev[k])[:numel], want, f"seed {seed}: state {k}")
    want_rep = np.full(p, sentinel, np.uint16)
    b = bf16_round(w1)
    for g0, length, c0 in segs:
        want_rep[g0:g0 + length] = b[c0:c0 + length]
    for r in reps:
        assert_bits(host(r), want_rep, f"seed {seed}: replica")


def test_a_plan_of_many_buckets_spans_several_launches():
    # 150 buckets at N = 5 with array_split chunks: one shard has 150
    # segments and the whole plan 750, more than one launch takes (64), so
    # every entry point splits the plan into several launches.  The mean and
    # the piece sums of one chunk and of every chunk, the update of one shard
    # into two replicas, and both all-gathers, each against the oracle.
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(0, 900, size=150)]
    lengths[::37] = [2 * PIECE + 3] * len(lengths[::37])  # a few multi-piece chunks
    lengths[5] = 0
    _every_entry_point_on(5, lengths, rng, 9100)


@pytest.mark.parametrize("nb", [2, 7, 8, 9, 16, 17, 63, 64, 65, 130])
def test_segment_lookup_at_group_and_launch_edges(nb):
    # Each kernel finds a tile's segment among up to 64 per launch by groups
    # of 8: plans whose shards have segment counts at the edges of a group
    # and of a launch, segments of one tile and of several, at N = 2 (a
    # shard of nb segments, the whole plan 2 * nb), every entry point against
    # the oracle.
    rng = np.random.default_rng(500 + nb)
    choices = [2, 96, 514, 2048, 2 * PIECE + 6, 3 * PIECE - 2]
    lengths = [int(choices[i]) for i in rng.integers(0, len(choices), size=nb)]
    _every_entry_point_on(2, lengths, rng, 9400 + nb)


def _every_entry_point_on(n, lengths, rng, seed):
    from oracle.bf16 import bf16_round
    from oracle.reduce import owned_chunk
    from oracle.step import Hyper as OHyper
    from oracle.step import adamw, all_gather

    nb = len(lengths)
    order = rng.permutation(nb)
    offs, pos = [0] * nb, 0
    for i in order:
        offs[i] = pos
        pos += lengths[i]
    buckets, p = list(zip(offs, lengths)), pos
    flags = grz.GRZ_UNEVEN
    grads = [rank_grad(p, 1e-2, "bf16", seed + r, device=DEV) for r in range(n)]
    hg = [host(g) for g in grads]
    npieces = grz.dp_piece_count(buckets, n, flags)

    mean_global = np.full(p, np.nan, np.float32)
    for c in range(n):
        comp = reduce_scatter_mean(hg, "bf16", buckets, c, uneven=True)
        for g0, length, c0 in shard_segments(buckets, n, c, uneven=True):
            mean_global[g0:g0 + length] = comp[c0:c0 + length]
    for chunk in (2 % n, -1):
        size = grz.dp_shard_numel(buckets, n, chunk, flags) if chunk >= 0 else p
        out = torch.full((size,), float("nan"), device=DEV)
        parts = torch.full((npieces,), -1.0, dtype=torch.float64, device=DEV)
        grz.dp_reduce_scatter_mean(grads, buckets, chunk, out, parts, flags=flags)
        torch.cuda.synchronize()
        if chunk >= 0:
            want = reduce_scatter_mean(hg, "bf16", buckets, chunk, uneven=True)
        else:
            want = mean_global
        assert_bits(host(out), want, f"mean, chunk {chunk}")
        got = host(parts)
        chunks = set(range(n)) if chunk < 0 else {chunk}
        for i, want_i in enumerate(_pieces_of(mean_global, buckets, n, chunks)):
            if want_i is None:
                assert got[i] == -1.0, f"chunk {chunk}: piece {i} written"
            else:
                assert math.isclose(got[i], want_i, rel_tol=1e-13, abs_tol=0.0), (chunk, i)

    # Clipped AdamW on one chunk's shard, written into two replicas.
    chunk = 2 % n
    segs = shard_segments(buckets, n, chunk, uneven=True)
    k = sum(s[1] for s in segs)
    w = rng.standard_normal(k).astype(np.float32) * np.float32(0.02)
    m = rng.standard_normal(k).astype(np.float32) * np.float32(1e-3)
    v = np.abs(rng.standard_normal(k)).astype(np.float32) * np.float32(1e-6)
    g = reduce_scatter_mean(hg, "bf16", buckets, chunk, uneven=True)
    scale = np.float32(0.375)
    dev = [torch.from_numpy(a.copy()).to(DEV) for a in (w, m, v, g)]
    sentinel = 0x7A5C
    reps = [torch.full((p,), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
            for _ in range(2)]
    hyper = grz.Hyper(lr=1e-3)
    grz.zero1_adamw_gather(dev[0], dev[1], dev[2], dev[3], buckets, n, chunk,
                           torch.tensor([scale], device=DEV),
                           grz.adamw_args(**grz.step_scalars(hyper, 2)), reps, flags=flags)
    torch.cuda.synchronize()
    w1, m1, v1 = adamw(w, m, v, g * scale, **OHyper(lr=1e-3).scalars(2))
    for i, want in enumerate((w1, m1, v1)):
        assert_bits(host(dev[i]), want, f"state {i}")
    want_rep = np.full(p, sentinel, np.uint16)
    b = bf16_round(w1)
    for g0, length, c0 in segs:
        want_rep[g0:g0 + length] = b[c0:c0 + length]
    for r in reps:
        assert_bits(host(r), want_rep, "replica after the update")

    # Both all-gathers: every rank's shard (rank 1's already in place).
    sizes = [grz.dp_shard_numel(buckets, n, owned_chunk(r, n), flags) for r in range(n)]
    bf = [rng.integers(0, 1 << 16, size=max(s, 1), dtype=np.uint16) for s in sizes]
    f32 = [rng.standard_normal(max(s, 1)).astype(np.float32) for s in sizes]
    bf_t = [torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16) for a in bf]
    f32_t = [torch.from_numpy(a.copy()).to(DEV) for a in f32]
    rep_bf = torch.full((p,), sentinel, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    rep_f32 = torch.full((p,), float("nan"), device=DEV)
    grz.zero1_all_gather([None if r == 1 else bf_t[r] for r in range(n)], buckets, [rep_bf],
                         flags=flags)
    grz.dp_all_gather([None if r == 1 else f32_t[r] for r in range(n)], buckets, [rep_f32],
                      flags=flags)
    torch.cuda.synchronize()
    want_bf = all_gather([None if r == 1 else bf[r][:sizes[r]] for r in range(n)], buckets, n,
                         p, uneven=True)
    rank1 = [(g0, length) for g0, length, _ in shard_segments(buckets, n, owned_chunk(1, n),
                                                              uneven=True)]
    for g0, length in rank1:
        want_bf[g0:g0 + length] = sentinel
    assert_bits(host(rep_bf), want_bf, "bf16 all-gather")
    want_f32 = np.full(p, np.nan, np.float32)
    for r in range(n):
        if r == 1:
            continue
        for g0, length, c0 in shard_segments(buckets, n, owned_chunk(r, n), uneven=True):
            want_f32[g0:g0 + length] = f32[r][c0:c0 + length]
    assert_bits(host(rep_f32), want_f32, "fp32 all-gather")


@pytest.mark.parametrize("held", ["f32", "bf16"])
@pytest.mark.parametrize("seed", range(24))
def test_reduce_modes_on_a_random_plan(seed, held):
    # The reduce's other modes on random plans: the sum instead of the mean,
    # the bf16 wire (bf16 gradients), the token-weighted mean (totals that are
    # and are not powers of two), shard-compact inputs, and a bucket range
    # whose inputs hold only that range (GRZ_IN_RANGE, how a ZeRO-2 backward
    # feeds the reduce from a staging buffer), alone and together.  Output
    # bit-exact against the oracle's reduce of the whole arenas at the range's
    # positions and untouched elsewhere; the piece sums against the exact sum
    # of squares of the oracle's output, other pieces untouched.  With
    # held="bf16" the output is the gradient shard held in bf16
    # (GRZ_MEAN_BF16): the oracle's mean rounded once, piece sums of the
    # rounded values (fp64 gradients, which have no such mode, become fp32).
    rng = np.random.default_rng(8000 + seed)
    n, kind, even, buckets, p, chunk, mode = _draw(3000 + seed)
    if held == "bf16" and kind == "f64":
        kind = "f32"
    flags = 0 if even else grz.GRZ_UNEVEN
    if held == "bf16":
        flags |= grz.GRZ_MEAN_BF16
    if mode == "global":
        flags |= grz.GRZ_OUT_GLOBAL
    wire = "bf16" if kind == "bf16" and rng.integers(0, 2) else None
    if wire:
        flags |= grz.GRZ_BF16_WIRE
    counts = None
    if rng.integers(0, 3) == 0:
        counts = [int(c) for c in rng.integers(0, 4000, size=n)]
        if rng.integers(0, 2):
            counts[-1] += (1 << 12) * (1 + n) - sum(counts)  # a power-of-two total
        counts[0] = max(counts[0], 1) if sum(counts) == 0 else counts[0]
    elif rng.integers(0, 4) == 0:
        flags |= grz.GRZ_SUM
    compact = chunk >= 0 and mode == "compact" and bool(rng.integers(0, 2))
    grads = [rank_grad(p, 1e-2, kind, 9300 + 17 * seed + r, device=DEV) for r in range(n)]
    hg = [host(g) for g in grads]
    if compact:
        flags |= grz.GRZ_IN_COMPACT
        segs = shard_segments(buckets, n, chunk, uneven=not even)
        idx = torch.tensor([i for g0, l, _ in segs for i in range(g0, g0 + l)] or [0],
                           dtype=torch.int64, device=DEV)
        inputs = [g[idx].contiguous() for g in grads]
        hin = [host(g) for g in inputs]
    else:
        inputs, hin = grads, hg
    nb = len(buckets)
    brange, in_range = None, set(range(nb))
    if not compact and rng.integers(0, 2):
        first = int(rng.integers(0, nb))
        brange = (first, int(rng.integers(1, nb - first + 1)))
        in_range = set(range(first, first + brange[1]))
        sel = [buckets[b] for b in sorted(in_range) if buckets[b][1] > 0]
        lo = min((o for o, _ in sel), default=0)
        hi = max((o + l for o, l in sel), default=0)
        inputs = [g[lo:max(hi, lo + 1)].contiguous() for g in grads]  # the range only
        flags |= grz.GRZ_IN_RANGE
    acc = np.float64 if kind == "f64" else np.float32
    out_t = torch.float64 if kind == "f64" else torch.float32
    if held == "bf16":
        out_t = torch.bfloat16
    npieces = grz.dp_piece_count(buckets, n, flags)
    parts = torch.full((max(npieces, 1),), -1.0, dtype=torch.float64, device=DEV)
    shard = grz.dp_shard_numel(buckets, n, chunk, flags) if chunk >= 0 else p
    out = torch.full((max(shard if mode == "compact" else p, 1),), float("nan"), dtype=out_t,
                     device=DEV)
    grz.dp_reduce_scatter_mean(inputs, buckets, chunk, out, parts, flags=flags,
                               token_counts=counts, bucket_range=brange)
    torch.cuda.synchronize()
    kw = dict(average=not flags & grz.GRZ_SUM, uneven=not even, wire=wire, token_counts=counts)
    out_global = np.full(p, np.nan, acc)
    chunks = range(n) if chunk < 0 else [chunk]
    for c in chunks:
        comp = reduce_scatter_mean(hg, kind, buckets, c, **kw)
        for b, (g0, length, c0) in enumerate(shard_segments(buckets, n, c, uneven=not even)):
            if b in in_range:
                out_global[g0:g0 + length] = comp[c0:c0 + length]
    what = (f"seed {seed} (n {n}, {kind}, wire {wire}, counts {counts}, flags {flags}, "
            f"range {brange}, held {held})")
    as_held = (lambda x: bf16_round(x)) if held == "bf16" else (lambda x: x)
    if mode == "compact":
        want = reduce_scatter_mean(hin, kind, buckets, chunk, compact_inputs=compact, **kw)
        for b, (_, length, c0) in enumerate(shard_segments(buckets, n, chunk, uneven=not even)):
            if b not in in_range:
                want[c0:c0 + length] = np.nan  # not reduced: left as it was
        assert_bits(host(out)[:shard], as_held(want), what)
    else:
        assert_bits(host(out)[:p], as_held(out_global), what)
    if held == "bf16":
        out_global = held_gradient(out_global, "bf16")
    got = host(parts)
    for i, want_i in enumerate(_pieces_of(out_global, buckets, n, set(chunks), in_range)):
        if want_i is None:
            assert got[i] == -1.0, f"{what}: piece {i} of a chunk not reduced was written"
        else:
            assert math.isclose(got[i], want_i, rel_tol=1e-13, abs_tol=0.0), (what, i)


def _nan_fill(kind):
    return {"bf16": np.uint16(0x7FC0), "f32": np.float32("nan"), "f64": np.float64("nan")}[kind]


@pytest.mark.parametrize("held", ["f32", "bf16"])
@pytest.mark.parametrize("seed", range(48))
def test_tiled_receive_on_a_random_plan(seed, held):
    # The reduce reading the N ranks' values of its chunk from one tiled
    # receive buffer (GRZ_IN_TILED), built here from the oracle's chunk
    # bounds with NaN wherever no value belongs (the rest of a short piece's
    # slot), on random plans with the reduce's modes (sum, bf16 wire, token
    # weights, arena-indexed output, a bucket range): bit for bit against the
    # oracle and against the same call on N separate shard-compact tensors;
    # the piece sums against the exact sums of squares; `tiled_receive` packs
    # the same buffer.  held="bf16": the mean written as a bf16 gradient shard
    # (GRZ_MEAN_BF16; fp64 gradients, which have no such mode, become fp32).
    rng = np.random.default_rng(12000 + seed)
    n, kind, even, buckets, p, chunk, mode = _draw(5000 + seed)
    if held == "bf16" and kind == "f64":
        kind = "f32"
    if chunk < 0:
        chunk = int(rng.integers(0, n))
    flags = 0 if even else grz.GRZ_UNEVEN
    if held == "bf16":
        flags |= grz.GRZ_MEAN_BF16
    out_global = bool(rng.integers(0, 3) == 0)
    if out_global:
        flags |= grz.GRZ_OUT_GLOBAL
    wire = "bf16" if kind == "bf16" and rng.integers(0, 2) else None
    if wire:
        flags |= grz.GRZ_BF16_WIRE
    counts = None
    if rng.integers(0, 3) == 0:
        counts = [int(c) + 1 for c in rng.integers(0, 4000, size=n)]
    elif rng.integers(0, 4) == 0:
        flags |= grz.GRZ_SUM
    nb = len(buckets)
    brange, in_range = None, set(range(nb))
    if rng.integers(0, 2):
        first = int(rng.integers(0, nb))
        brange = (first, int(rng.integers(1, nb - first + 1)))
        in_range = set(range(first, first + brange[1]))
    grads = [rank_grad(p, 1e-2, kind, 15000 + 17 * seed + r, device=DEV) for r in range(n)]
    hg = [host(g) for g in grads]
    segs = shard_segments(buckets, n, chunk, uneven=not even)
    hin = [np.concatenate([h[g0:g0 + length] for g0, length, _ in segs]) for h in hg]
    npc = sum(-(-length // PIECE) for _, length, _ in segs)
    buf = np.full((max(npc, 1), n, PIECE), _nan_fill(kind), dtype=hg[0].dtype)
    filled = np.zeros(buf.shape, bool)
    k = 0
    for g0, length, _ in segs:
        for a in range(0, length, PIECE):
            e = min(length, a + PIECE)
            for j in range(n):
                buf[k, j, :e - a] = hg[j][g0 + a:g0 + e]
            filled[k, :, :e - a] = True
            k += 1
    assert npc * n * PIECE == grz.dp_tiled_numel(buckets, n, chunk, flags & grz.GRZ_UNEVEN)
    dev_t = {"bf16": torch.int16, "f32": torch.float32, "f64": torch.float64}[kind]
    flat = buf.reshape(-1)
    recv = torch.from_numpy(flat.view(np.int16) if kind == "bf16" else flat).to(DEV)
    compact = [torch.from_numpy(h.view(np.int16) if kind == "bf16" else h).to(DEV) for h in hin]
    packed = grz.tiled_receive(compact, buckets, n, chunk)
    got_buf = host(packed.buffer).view(buf.dtype).reshape(buf.shape)
    assert np.array_equal(got_buf[filled], buf[filled])
    out_t = torch.float64 if kind == "f64" else torch.float32
    if held == "bf16":
        out_t = torch.bfloat16
    shard = grz.dp_shard_numel(buckets, n, chunk, flags & grz.GRZ_UNEVEN)
    npieces = grz.dp_piece_count(buckets, n, flags & grz.GRZ_UNEVEN)
    outs, parts = [], []
    for inputs, extra in ((grz.Tiled(recv, n), 0), (compact, grz.GRZ_IN_COMPACT)):
        o = torch.full((max(p if out_global else shard, 1),), float("nan"), dtype=out_t,
                       device=DEV)
        q = torch.full((max(npieces, 1),), -1.0, dtype=torch.float64, device=DEV)
        grz.dp_reduce_scatter_mean(inputs, buckets, chunk, o, q, flags=flags | extra,
                                   token_counts=counts, bucket_range=brange)
        outs.append(o)
        parts.append(q)
    torch.cuda.synchronize()
    what = (f"seed {seed} (n {n}, {kind}, chunk {chunk}, wire {wire}, counts {counts}, "
            f"flags {flags}, range {brange}, held {held})")
    assert_bits(host(outs[0]), host(outs[1]), f"{what}: tiled against separate tensors")
    assert_bits(host(parts[0]), host(parts[1]), f"{what}: piece sums, tiled against separate")
    acc = np.float64 if kind == "f64" else np.float32
    kw = dict(average=not flags & grz.GRZ_SUM, uneven=not even, wire=wire, token_counts=counts)
    comp = reduce_scatter_mean(hin, kind, buckets, chunk, compact_inputs=True, **kw)
    full = np.full(p, np.nan, acc)
    for b, (g0, length, c0) in enumerate(segs):
        if b in in_range:
            full[g0:g0 + length] = comp[c0:c0 + length]
        else:
            comp[c0:c0 + length] = np.nan  # not reduced: left as it was
    as_held = (lambda x: bf16_round(x)) if held == "bf16" else (lambda x: x)
    if out_global:
        assert_bits(host(outs[0])[:p], as_held(full), what)
    else:
        assert_bits(host(outs[0])[:shard], as_held(comp), what)
    if held == "bf16":
        full = held_gradient(full, "bf16")
    got = host(parts[0])
    for i, want_i in enumerate(_pieces_of(full, buckets, n, {chunk}, in_range)):
        if want_i is None:
            assert got[i] == -1.0, f"{what}: piece {i} of a chunk not reduced was written"
        else:
            assert math.isclose(got[i], want_i, rel_tol=1e-13, abs_tol=0.0), (what, i)
