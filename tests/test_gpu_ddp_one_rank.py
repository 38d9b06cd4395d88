"""One rank's plain data-parallel (ZeRO stage 0) step, against the oracle.

The all-reduce of the mean is its two halves ("Lab 09", s.1: reduce-scatter,
then all-gather): the reduce of the rank's own chunk written at its arena
offsets (GRZ_OUT_GLOBAL), the all-gather of the peers' fp32 mean chunks
(dp_all_gather, also for fp64 and bf16), then clip + AdamW over the rank's
full copy of the state.  Bars as for the rest of the GPU path: reduced values
and copies bit-exact, norm within 1e-13, state and bf16 weights bit-exact when
the clip factors agree.
"""

import io
import math

import numpy as np
import pytest
import torch

import gradient_reduce_zero_amd as grz
from oracle.reduce import owned_chunk, reduce_scatter_mean, shard_segments
from oracle.step import Hyper as OHyper
from oracle.step import ddp_step
from parity_util import assert_bits, host, max_rel
from workloads import grad_seed, master_init, rank_grad

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _place(compact, segs, out):
    """The oracle's placement of a shard-compact chunk at its arena offsets."""
    for g0, length, c0 in segs:
        out[g0:g0 + length] = compact[c0:c0 + length]
    return out


def _chunk_index(buckets, n, c, uneven=False):
    return torch.cat([torch.arange(g0, g0 + length, device=DEV)
                      for g0, length, _ in shard_segments(buckets, n, c, uneven)])


@pytest.mark.parametrize("n,kind,uneven", [(3, "bf16", False), (5, "f32", False),
                                           (8, "bf16", False), (3, "f32", True)])
def test_reduce_out_global_writes_the_chunk_at_arena_offsets(n, kind, uneven):
    # Two buckets in reverse order, several pieces and a ragged tail each; with
    # `uneven` the lengths do not divide by N (array_split chunks).
    a, b = n * (2 * 4096 + 40), n * (4096 + 24) + (2 if uneven else 0)
    buckets = [(a, b), (0, a)]
    p = a + b
    flags = grz.GRZ_UNEVEN if uneven else 0
    grads = [rank_grad(p, 1e-2, kind, grad_seed(3, r), device=DEV) for r in range(n)]
    hg = [host(g) for g in grads]
    npieces = grz.dp_piece_count(buckets, n, flags)
    for c in range(n):
        segs = shard_segments(buckets, n, c, uneven)
        shard = sum(s[1] for s in segs)
        out = torch.full((p,), float("nan"), device=DEV)
        parts = torch.full((npieces,), -1.0, dtype=torch.float64, device=DEV)
        grz.dp_reduce_scatter_mean(grads, buckets, c, out, parts,
                                   flags=flags | grz.GRZ_OUT_GLOBAL)
        # The same chunk from compact inputs, and the plain shard-compact call.
        idx = _chunk_index(buckets, n, c, uneven)
        out_c = torch.full((p,), float("nan"), device=DEV)
        grz.dp_reduce_scatter_mean([g.index_select(0, idx).contiguous() for g in grads],
                                   buckets, c, out_c, None,
                                   flags=flags | grz.GRZ_OUT_GLOBAL | grz.GRZ_IN_COMPACT)
        compact = torch.empty(shard, device=DEV)
        parts_c = torch.full((npieces,), -1.0, dtype=torch.float64, device=DEV)
        grz.dp_reduce_scatter_mean(grads, buckets, c, compact, parts_c, flags=flags)
        torch.cuda.synchronize()
        want_c = reduce_scatter_mean(hg, kind, buckets, c, uneven=uneven)
        want = _place(want_c, segs, np.full(p, np.nan, np.float32))
        assert_bits(host(out), want, f"chunk {c} at arena offsets")
        assert_bits(host(out_c), want, f"chunk {c} from compact inputs")
        assert_bits(host(compact), want_c, f"chunk {c} shard-compact")
        assert_bits(host(parts), host(parts_c), f"chunk {c} pieces")


@pytest.mark.parametrize("dtype", [torch.float32, torch.float64, torch.bfloat16])
def test_all_gather_of_any_element_size(dtype):
    # Shards straight from the seeded generator; rank 1's is already in place.
    # Every other element keeps the replica's previous bytes.
    n = 4
    a, b = n * (4096 + 8) + n * 8 * 3, n * 8 * 7 + n  # the second ends off a 16-byte line
    buckets = [(a, b), (0, a)]
    p = a + b
    shards = []
    for r in range(n):
        numel = sum(s[1] for s in shard_segments(buckets, n, (r + 1) % n))
        shards.append(master_init(numel, seed=400 + r, device=DEV).to(dtype))
    shards[1] = None
    fill = -7.25
    reps = [torch.full((p,), fill, dtype=dtype, device=DEV) for _ in range(2)]
    grz.dp_all_gather(shards, buckets, reps)
    torch.cuda.synchronize()
    want = host(torch.full((p,), fill, dtype=dtype))
    for r, s in enumerate(shards):
        if s is not None:
            _place(host(s), shard_segments(buckets, n, (r + 1) % n), want)
    for rep in reps:
        assert_bits(host(rep), want, f"{dtype} all-gather")


@pytest.mark.parametrize("recv", ["ranks", "tiled"])
def test_ddp_one_rank_matches_the_oracle_and_the_all_ranks_replica(recv):
    # Rank r fed what its peers deliver -- its chunk of every rank's gradient
    # (as N tensors, or in one tiled receive buffer), the peers' mean chunks
    # (the oracle's, as inputs) and every rank's norm pieces -- reproduces the
    # oracle's ddp_step and, over two steps, the replica DDPStep computes from
    # the full arenas, bit for bit.
    n, p = 8, 8 * (3 * 4096 + 136)
    buckets = [(8 * 4096, p - 8 * 4096), (0, 8 * 4096)]
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(max_norm=0.5)
    full = grz.DDPStep(buckets, n, master, hyper, device=DEV)
    ones = {r: grz.DDPOneRank(buckets, n, r, master, hyper, DEV) for r in (0, 5)}
    w0 = host(master)
    for t in (1, 2):
        grads = [rank_grad(p, 1e-2, "bf16", grad_seed(5 + t, r), device=DEV) for r in range(n)]
        hg = [host(g) for g in grads]
        full.step(grads, t)
        torch.cuda.synchronize()
        assert full.norm.scale.item() < 1
        peer_mean = {j: _dev(reduce_scatter_mean(hg, "bf16", buckets, owned_chunk(j, n)))
                     for j in range(n)}
        if t == 1:
            z = np.zeros_like(w0)
            want = ddp_step(hg, "bf16", buckets, (w0, z, z), OHyper(max_norm=0.5), 1)
        for r, one in ones.items():
            c = owned_chunk(r, n)
            idx = _chunk_index(buckets, n, c)
            one.norm.partials.copy_(full.norm.partials)  # every rank's pieces, as received
            mine = [g.index_select(0, idx).contiguous() for g in grads]
            if recv == "tiled":
                mine = grz.tiled_receive(mine, buckets, n, c)
            one.step(mine, [None if j == r else peer_mean[j] for j in range(n)], t)
            torch.cuda.synchronize()
            assert_bits(host(one.mean), host(full.mean), f"rank {r} step {t} mean")
            assert_bits(host(one.norm.sqnorm), host(full.norm.sqnorm), f"rank {r} sqnorm")
            for k in range(3):
                assert_bits(host(one.state[k]), host(full.state[k]), f"rank {r} state {k}")
            assert_bits(host(one.arena), host(full.replica), f"rank {r} bf16 arena")
            if t == 1:
                assert_bits(host(one.mean), want["mean"], f"rank {r} mean vs oracle")
                assert math.isclose(one.norm.sqnorm.item(), want["sqnorm"], rel_tol=1e-13)
                # The fp32 clip factors agree bit for bit (the norms differ by
                # ~1e-15 relative), so the state is compared bit for bit.
                assert np.float32(one.norm.scale.item()) == want["scale"]
                for k in range(3):
                    assert max_rel(host(one.state[k]), want["state"][k]) <= 1e-6
                    assert_bits(host(one.state[k]), want["state"][k], f"state {k} vs oracle")
                assert_bits(host(one.arena), want["arena"], "bf16 arena vs oracle")


def test_ddp_one_rank_with_uneven_chunks():
    # Plain data parallelism is what runs when bucket lengths do not divide by
    # N: the chunks follow array_split, and each rank's step still equals the
    # oracle's ddp_step and the all-ranks DDPStep replica.
    n = 3
    a, b = 3 * (4096 + 5) + 1, 3 * 4096 + 2
    buckets = [(a, b), (0, a)]
    p = a + b
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(max_norm=0.5)
    full = grz.DDPStep(buckets, n, master, hyper, device=DEV)
    grads = [rank_grad(p, 1e-2, "bf16", grad_seed(9, r), device=DEV) for r in range(n)]
    hg = [host(g) for g in grads]
    full.step(grads, 1)
    torch.cuda.synchronize()
    w0 = host(master)
    z = np.zeros_like(w0)
    want = ddp_step(hg, "bf16", buckets, (w0, z, z), OHyper(max_norm=0.5), 1)
    assert want["scale"] < 1
    for r in range(n):
        said = io.StringIO()
        one = grz.one_rank_step(buckets, n, r, master, hyper, DEV, log=said)
        assert isinstance(one, grz.DDPOneRank) and one.flags == grz.GRZ_UNEVEN
        assert "stage 0" in said.getvalue()
        idx = _chunk_index(buckets, n, owned_chunk(r, n), uneven=True)
        one.norm.partials.copy_(full.norm.partials)
        peers = [None if j == r else
                 _dev(reduce_scatter_mean(hg, "bf16", buckets, owned_chunk(j, n), uneven=True))
                 for j in range(n)]
        one.step([g.index_select(0, idx).contiguous() for g in grads], peers, 1)
        torch.cuda.synchronize()
        assert_bits(host(one.mean), want["mean"], f"rank {r} mean vs oracle")
        assert_bits(host(one.mean), host(full.mean), f"rank {r} mean vs DDPStep")
        assert np.float32(one.norm.scale.item()) == want["scale"]
        for k in range(3):
            assert_bits(host(one.state[k]), host(full.state[k]), f"rank {r} state {k}")
            assert max_rel(host(one.state[k]), want["state"][k]) <= 1e-6
            assert_bits(host(one.state[k]), want["state"][k], f"rank {r} state {k} vs oracle")
        assert_bits(host(one.arena), want["arena"], f"rank {r} bf16 arena vs oracle")


def test_captured_ddp_one_rank_replays_match_eager():
    # Graph replays of one rank's plain data-parallel step, with eager work and
    # host synchronisations in between, each equal to the eager step of the
    # same number; one replay past the scalar table raises and changes nothing.
    n, rank = 8, 3
    p = 8 * (2 * 4096 + 72)
    buckets = [(8 * 4096, p - 8 * 4096), (0, 8 * 4096)]
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(lr=1e-3, warmup=2, max_norm=0.05)
    c = owned_chunk(rank, n)
    idx = _chunk_index(buckets, n, c)
    grads = [rank_grad(p, 1e-2, "bf16", grad_seed(3, r), device=DEV) for r in range(n)]
    incoming = [g.index_select(0, idx).contiguous() for g in grads]
    hg = [host(g) for g in grads]
    peers = [None if j == rank else
             _dev(reduce_scatter_mean(hg, "bf16", buckets, owned_chunk(j, n)))
             for j in range(n)]
    full = grz.DDPStep(buckets, n, master, hyper, device=DEV)
    full.step(grads, 1)
    eager = grz.DDPOneRank(buckets, n, rank, master, hyper, DEV)
    graphed = grz.DDPOneRank(buckets, n, rank, master, hyper, DEV)
    for d in (eager, graphed):
        d.norm.partials.copy_(full.norm.partials)
    cap = grz.CapturedStep(lambda args, s: graphed.enqueue(incoming, peers, args, s), hyper, 1,
                           4)
    junk = torch.randn(1 << 20, device=DEV)
    for t in range(1, 5):
        eager.step(incoming, peers, t)
        cap.replay()
        junk.mul_(0.5).add_(1.0)
        torch.cuda.synchronize()
        for a, b, what in ((eager.mean, graphed.mean, "mean"),
                           (eager.state[0], graphed.state[0], "master"),
                           (eager.state[2], graphed.state[2], "v"),
                           (eager.arena, graphed.arena, "arena"),
                           (eager.norm.scale, graphed.norm.scale, "scale")):
            assert_bits(host(b), host(a), f"replay {t}: {what}")
    assert int(cap.counter.item()) == 4
    before = host(graphed.state[0])
    with pytest.raises(RuntimeError, match="4 steps"):
        cap.replay()
    torch.cuda.synchronize()
    assert int(cap.counter.item()) == 4
    assert_bits(host(graphed.state[0]), before, "master after the refused replay")
