"""The smaller one-rank shares the bench records, in the launch configuration
it times them: set up by the bench's own helper (the same seeded inputs, the
reduce reading them from the tiled receive buffer), the step captured once in
a HIP graph and replayed, against the oracle over two replays.  Char GPT and GPT-2 124M are checked on every element; GPT-2 1.5B
(389 M owned parameters at N = 4) on sampled elements, with the norm over the
whole shard in streamed tiles."""

import math

import numpy as np
import pytest
import torch

import bench
import gradient_reduce_zero_amd as grz
from oracle.reduce import chunk_mean, shard_segments, widen
from oracle.step import Hyper as OHyper
from oracle.step import adamw, bf16_round, clip_scale, grad_sqnorm
from parity_util import assert_bits, gather_host, host, sample_indices

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _peer_mask(one):
    """Piece slots that hold the peers' pieces (not this rank's own)."""
    mask = np.ones(one.norm.npieces, bool)
    for first, cnt in one.own_piece_slots():
        mask[first:first + cnt] = False
    return mask


def _arena_positions(segs, idx):
    """Arena offsets of shard-compact indices ``idx`` of a shard laid out as
    ``segs`` ([(arena start, length, compact start)])."""
    c0 = np.array([c for _, _, c in segs], np.int64)
    g0 = np.array([g for g, _, _ in segs], np.int64)
    k = np.searchsorted(c0, idx, side="right") - 1
    return g0[k] + (idx - c0[k])


def _tiled_own_sqnorm(incoming, chunk, length, tile=1 << 25):
    parts = []
    for lo in range(0, length, tile):
        hi = min(length, lo + tile)
        mean = chunk_mean([widen(host(t[lo:hi]), "bf16") for t in incoming], chunk)
        parts.append(np.sum(np.square(mean.astype(np.float64))))
    return float(np.sum(parts))


@pytest.mark.parametrize("config,n", [("char_gpt", 8), ("gpt2_124m", 8), ("gpt2_1p5b", 4)])
def test_bench_one_rank_share_as_a_graph_matches_oracle(config, n):
    setup = bench.onerank_setup(config, n, 0, DEV)
    one, inp = setup["pipe"], setup["inp"]
    assert isinstance(inp["recv"], grz.Tiled)
    chunk, shard, buckets = setup["chunk"], setup["shard"], setup["buckets"]
    whole = shard <= 1 << 25
    idx = np.arange(shard) if whole else sample_indices(shard, 100_000, 3)
    w = gather_host(one.state[0], idx)
    m, v = np.zeros_like(w), np.zeros_like(w)
    # The oracle's mean at the checked elements and the norm over the whole
    # shard plus the peers' pieces as received.
    if whole:
        mean = chunk_mean([widen(host(t), "bf16") for t in inp["incoming"]], chunk)
        peers = host(inp["partials"])[_peer_mask(one)]
        sq = grad_sqnorm(mean, extra=peers)
    else:
        mean = chunk_mean([widen(gather_host(t, idx), "bf16") for t in inp["incoming"]], chunk)
        peers = host(inp["partials"])[_peer_mask(one)]
        sq = _tiled_own_sqnorm(inp["incoming"], chunk, shard) + float(np.sum(peers))
    scale = clip_scale(sq, 1.0)
    cap = grz.CapturedStep(lambda a, s: (one.reduce(inp["recv"], s),
                                         one.update(None, s, args=a),
                                         one.gather(inp["peer_shards"], s)),
                           one.hyper, 1, 2)
    h = OHyper()
    segs = shard_segments(buckets, n, chunk)
    for t in (1, 2):
        cap.replay()
        torch.cuda.synchronize()
        what = f"{config} N={n} replay {t}"
        assert_bits(gather_host(one.mean, idx), mean, f"{what}: mean")
        assert math.isclose(one.norm.sqnorm.item(), sq, rel_tol=1e-12), what
        assert np.float32(one.norm.scale.item()) == scale, what
        w, m, v = adamw(w, m, v, mean * scale, **h.scalars(t))
        for k, want in enumerate((w, m, v)):
            assert_bits(gather_host(one.state[k], idx), want, f"{what}: state {k}")
        # The arena: the own shard's elements are the master rounded to bf16,
        # at their arena offsets; every peer's shard lands at its own.
        assert_bits(gather_host(one.arena, _arena_positions(segs, idx)), bf16_round(w),
                    f"{what}: own shard in the arena")
        for j in (1, n - 1):
            psegs = shard_segments(buckets, n, (j + 1) % n)
            assert_bits(gather_host(one.arena, _arena_positions(psegs, idx)),
                        gather_host(inp["peer_shards"][j], idx), f"{what}: peer {j}'s shard")
    assert scale < 1


def test_bench_ddp_one_rank_gpt2_124m_matches_oracle():
    # The bench's GPT-2 124M DDP rank (9 reverse-layer buckets, N = 8, rank 0,
    # set up by the bench's own helper, the tiled receive buffer), one step,
    # every element against the oracle: the own chunk's mean (ring fold), the
    # peers' mean chunks as received, the norm over the own chunk plus the
    # peers' pieces as received, clipped AdamW over the whole arena and its
    # bf16 rounding.
    d = bench.ddp_setup("gpt2_124m", 8, 0, DEV)
    one, n, buckets, chunk, p = d["one"], d["n"], d["buckets"], d["chunk"], d["p"]
    assert isinstance(d["recv"], grz.Tiled)
    w0 = host(one.state[0])
    one.step(d["recv"], d["peer_means"], 1)
    torch.cuda.synchronize()
    own = chunk_mean([widen(host(t), "bf16") for t in d["incoming"]], chunk)
    want = np.empty(p, np.float32)
    for g0, length, c0 in shard_segments(buckets, n, chunk):
        want[g0:g0 + length] = own[c0:c0 + length]
    for j in range(n):
        if j != d["rank"]:
            peer = host(d["peer_means"][j])
            for g0, length, c0 in shard_segments(buckets, n, (j + 1) % n):
                want[g0:g0 + length] = peer[c0:c0 + length]
    assert_bits(host(one.mean), want, "DDP 124M mean")
    sq = grad_sqnorm(own, extra=host(d["partials"])[_peer_mask(one)])
    assert math.isclose(one.norm.sqnorm.item(), sq, rel_tol=1e-12)
    scale = clip_scale(sq, 1.0)
    assert scale < 1 and np.float32(one.norm.scale.item()) == scale
    z = np.zeros_like(w0)
    w, m, v = adamw(w0, z, z, want * scale, **OHyper().scalars(1))
    for k, x in enumerate((w, m, v)):
        assert_bits(host(one.state[k]), x, f"DDP 124M state {k}")
    assert_bits(host(one.arena), bf16_round(w), "DDP 124M bf16 arena")


def test_bench_char_gpt_share_100_steps_matches_oracle():
    # The char GPT workload runs 100 steps.  The bench's char GPT one-rank
    # share (N = 8, rank 0, the tiled receive buffer), captured and replayed
    # 100 times, as three kernels and as one launch (zero1_fused_step_args):
    # master, m, v and the own shard in the arena against the oracle's AdamW
    # after every 10th step, bit for bit (the same received gradients every
    # step, so the oracle's mean and norm are computed once).
    setup = bench.onerank_setup("char_gpt", 8, 0, DEV)
    one, inp = setup["pipe"], setup["inp"]
    chunk, shard, buckets, n = setup["chunk"], setup["shard"], setup["buckets"], setup["n"]
    fused = grz.Zero1OneRank(buckets, n, 0, inp["shard_master"].clone(), device=DEV,
                             arena_numel=setup["p"], fused=True)
    fused.norm.partials.copy_(inp["partials"])
    mean = chunk_mean([widen(host(t), "bf16") for t in inp["incoming"]], chunk)
    scale = clip_scale(grad_sqnorm(mean, extra=host(inp["partials"])[_peer_mask(one)]), 1.0)
    assert scale < 1
    steps = 100
    three_cap = grz.CapturedStep(lambda a, s: (one.reduce(inp["recv"], s),
                                               one.update(None, s, args=a),
                                               one.gather(inp["peer_shards"], s)),
                                 one.hyper, 1, steps)
    fused_cap = grz.CapturedStep(lambda a, s: (fused.fused_update(inp["incoming"], a, s),
                                               fused.gather(inp["peer_shards"], s)),
                                 fused.hyper, 1, steps)
    w = host(one.state[0])
    m, v = np.zeros_like(w), np.zeros_like(w)
    g = mean * scale
    h = OHyper()
    own = _arena_positions(shard_segments(buckets, n, chunk), np.arange(shard))
    for t in range(1, steps + 1):
        three_cap.replay()
        fused_cap.replay()
        w, m, v = adamw(w, m, v, g, **h.scalars(t))
        if t % 10 == 0:
            torch.cuda.synchronize()
            fused.check_fused()
            for pipe, name in ((one, "three kernels"), (fused, "one launch")):
                for k, want in enumerate((w, m, v)):
                    assert_bits(host(pipe.state[k]), want, f"{name} t={t}: state {k}")
                assert_bits(host(pipe.arena)[own], bf16_round(w), f"{name} t={t}: own shard")
