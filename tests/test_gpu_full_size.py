"""Parity at the full model sizes, in the launch configuration the bench times.

Where the oracle can redo everything in seconds (char GPT, GPT-2 124M) it
does; at 1.5B and 7B it recomputes sampled elements one by one from the same
input bytes (random picks, both ends, piece and chunk boundaries) and the
norm over the whole reduced gradient in streamed tiles.
"""

import math

import numpy as np
import pytest
import torch

import gradient_reduce_zero_amd as grz
from oracle.plan import plan_buckets as oracle_plan
from oracle.reduce import chunk_mean, owned_chunk, shard_segments, widen
from oracle.step import Hyper as OHyper
from oracle.step import adamw, bf16_round, clip_scale, ddp_step, zero1_step
from parity_util import (assert_bits, chunk_of_index, gather_host, host, max_rel,
                         oracle_mean_at, oracle_states, sample_indices)
from workloads import arena, grad_seed, master_init, onerank_inputs, rank_grad

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _layer_spans(a, sigma=1e-3):
    """Char GPT: sigma_l = 1e-3 * 2^(l - (L-1)/2) for block l, 1e-3 elsewhere."""
    nl = max(layer for _, _, layer in a.tensors)
    spans = []
    for off, n, layer in a.spans():
        s = sigma * 2.0 ** (layer - (nl - 1) / 2) if 0 <= layer < nl else sigma
        spans.append((off, n, s))
    return spans


def test_char_gpt_all_ranks_10_steps():
    a = arena("char_gpt")
    p, n = a.numel, 8
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV)
    d = grz.DDPStep(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV)
    states = oracle_states(host(master), buckets, n)
    spans = _layer_spans(a)
    for t in range(1, 11):
        grads = [rank_grad(p, 1e-3, "bf16", grad_seed(t, r), DEV, spans) for r in range(n)]
        z.step(grads, t)
        d.step(grads, t)
        torch.cuda.synchronize()
        ref = zero1_step([host(g) for g in grads], "bf16", buckets, states, OHyper(), t)
        states = ref["states"]
        for r in range(n):
            assert_bits(host(z.means[r]), ref["means"][r], f"t={t} mean rank {r}")
        assert math.isclose(z.norm.sqnorm.item(), ref["sqnorm"], rel_tol=1e-13)
        assert ref["scale"] < 1  # the char GPT's norm is above 1: the clip is active
        assert_bits(host(z.norm.scale), np.array([ref["scale"]], np.float32), f"t={t} scale")
        for r in range(n):
            for k in range(3):
                got, want = host(z.state[r][k]), ref["states"][r][k]
                assert max_rel(got, want) <= 1e-6
                assert_bits(got, want, f"t={t} state {k} rank {r}")
        assert_bits(host(z.replicas[n - 1]), ref["arena"], f"t={t} replica")
        assert_bits(host(d.replica), ref["arena"], f"t={t} DDP replica")


def _arena_state(states, buckets, n, p):
    """The ranks' shard-compact (master, m, v) placed at their arena offsets."""
    out = [np.empty(p, np.float32) for _ in range(3)]
    for r in range(n):
        for g0, length, c0 in shard_segments(buckets, n, owned_chunk(r, n)):
            for k in range(3):
                out[k][g0:g0 + length] = states[r][k][c0:c0 + length]
    return tuple(out)


def test_gpt2_124m_reverse_layer_buckets_10_steps():
    # GPT-2 124M with its 9 reverse-layer buckets, N = 8, ZeRO-1 (every rank)
    # and plain data parallelism, 10 steps: every array, every step, against
    # the oracle's zero1_step (means, norm, clip factor, master/m/v, all
    # replicas).  DDP's state and weights equal the ranks' shards placed at
    # their arena offsets every step, and at steps 1 and 10 the oracle's own
    # ddp_step (from the oracle's state of the step before) is checked too.
    a = arena("gpt2_124m")
    p, n = a.numel, 8
    buckets = grz.plan_buckets(a.numels, 25 * 2 ** 20, 2)
    assert buckets == oracle_plan(a.numels, 25 * 2 ** 20, 2) and len(buckets) == 9
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV)
    d = grz.DDPStep(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV)
    states = oracle_states(host(master), buckets, n)
    dstate = (host(master), np.zeros(p, np.float32), np.zeros(p, np.float32))
    del master
    for t in range(1, 11):
        grads = [rank_grad(p, 1e-3, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]
        z.step(grads, t)
        d.step(grads, t)
        torch.cuda.synchronize()
        hg = [host(g) for g in grads]
        del grads
        ref = zero1_step(hg, "bf16", buckets, states, OHyper(), t)
        if t in (1, 10):
            dref = ddp_step(hg, "bf16", buckets, dstate, OHyper(), t)
            assert_bits(host(d.mean), dref["mean"], f"t={t} DDP mean over 9 buckets")
            # Above 2e7 terms both oracle steps sum the squares with numpy, in
            # different orders (shard by shard, arena order): equal to ~1e-15.
            assert math.isclose(dref["sqnorm"], ref["sqnorm"], rel_tol=1e-13)
            assert dref["scale"] == ref["scale"]
            for k in range(3):
                assert_bits(host(d.state[k]), dref["state"][k], f"t={t} DDP state {k}")
            assert_bits(host(d.replica), dref["arena"], f"t={t} DDP bf16 arena")
        del hg
        states = ref["states"]
        for r in range(n):
            assert_bits(host(z.means[r]), ref["means"][r], f"t={t} ZeRO-1 shard of rank {r}")
            for k in range(3):
                got, want = host(z.state[r][k]), ref["states"][r][k]
                assert max_rel(got, want) <= 1e-6, (t, r, k)
                assert_bits(got, want, f"t={t} state {k} of rank {r}")
        assert math.isclose(z.norm.sqnorm.item(), ref["sqnorm"], rel_tol=1e-13)
        assert_bits(host(z.norm.sqnorm), host(d.norm.sqnorm), f"t={t} ZeRO-1 vs DDP sqnorm")
        assert_bits(host(z.norm.scale), np.array([ref["scale"]], np.float32), f"t={t} scale")
        for r in range(n):
            assert_bits(host(z.replicas[r]), ref["arena"], f"t={t} ZeRO-1 replica {r}")
        assert_bits(host(d.replica), ref["arena"], f"t={t} DDP replica")
        dstate = _arena_state(states, buckets, n, p)
        for k in range(3):
            assert_bits(host(d.state[k]), dstate[k], f"t={t} DDP state {k} vs the ranks' shards")
    assert ref["scale"] < 1


def _tiled_sqnorm(tensors_for, chunk, kind, length, wire=None, divisor=None, tile=1 << 24,
                  workers=8):
    """Oracle norm of the mean (with a wire precision or a divisor, if given)
    over [0, length) of a shard: tiles folded by the oracle in worker threads
    (NumPy releases the interpreter lock inside its loops), the tile sums
    added in tile order."""
    from concurrent.futures import ThreadPoolExecutor

    def part(lo):
        hi = min(length, lo + tile)
        m = chunk_mean([widen(host(t[lo:hi]), kind) for t in tensors_for], chunk, True, wire,
                       divisor)
        return float(np.sum(np.square(m.astype(np.float64))))

    with ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(part, range(0, length, tile)))
    return float(np.sum(parts))


def _clip_factor_bits_agree(got_scale, scale, what):
    """The GPU's clip factor has the oracle's bits.  The two norms differ by
    ~1e-15 relative (fixed tree against exact or pairwise sums), so their fp32
    factors could only differ if the norm sat that close to a rounding
    boundary of the factor; the assertion says these inputs do not.  Every
    state comparison is then bit for bit, against the oracle's own factor."""
    assert np.float32(got_scale) == np.float32(scale), \
        f"{what}: clip factor {float(got_scale)!r} vs the oracle's {float(scale)!r}"


@pytest.mark.parametrize("n", [8, 2, 16])
def test_llama_7b_one_rank_share_sampled(n):
    # The bench's configuration: rank 0 of N = 8 owns chunk 1 of the whole
    # 6.74e9-element arena; 842,301,952 owned parameters, 10 steps.  The
    # incoming gradients alternate between two seeded sets (steps 1, 3, ...
    # and 2, 4, ...), so that the oracle's norm over the whole shard is
    # computed once per set; the oracle carries master, m and v on 200 k
    # sampled elements through all 10 steps.  At N = 2 (one step) the shard
    # holds 3.37e9 elements (indices beyond 2^31 in every shard-compact
    # array); N = 16 (one step) folds each tile's loads in two batches.  At
    # N = 8 and 16 the reduce reads the tiled receive buffer, as the bench
    # does; at N = 2 the N separate tensors.
    a = arena("llama_7b")
    p, rank = a.numel, 0
    steps = 10 if n == 8 else 1
    buckets = grz.whole_arena(p)
    chunk = owned_chunk(rank, n)
    shard = grz.dp_shard_numel(buckets, n, chunk)
    assert shard == p // n
    npieces = grz.dp_piece_count(buckets, n)
    inp = onerank_inputs(shard, n, rank, npieces, grz.GRZ_PIECE, device=DEV)
    pipe = grz.Zero1OneRank(buckets, n, rank, inp["shard_master"], device=DEV, arena_numel=p)
    idx = sample_indices(shard, 200_000, 7, extra=[4095, 4096, 4097, shard - 4096 * 2,
                                                   (1 << 31) - 1, 1 << 31, (1 << 31) + 1])
    w = gather_host(pipe.state[0], idx)
    m, v = np.zeros_like(w), np.zeros_like(w)
    peers = host(inp["partials"])
    own = pipe.own_piece_slots()
    mask = np.ones(npieces, bool)
    for first, cnt in own:
        mask[first:first + cnt] = False
    sets = [inp["incoming"]]
    if steps > 1:
        sets.append([rank_grad(shard, 1e-3, "bf16", grad_seed(2, j), device=DEV)
                     for j in range(n)])
    recvs = sets if n == 2 else [grz.tiled_receive(x, buckets, n, chunk) for x in sets]
    # Per set: the oracle's mean at the samples and its norm (own part
    # recomputed in tiles from the inputs, the peers' pieces as received).
    want_means, sqs = [], []
    for incoming in sets:
        want_means.append(oracle_mean_at([gather_host(t, idx) for t in incoming],
                                         np.full(idx.size, chunk), "bf16"))
        sqs.append(_tiled_sqnorm(incoming, chunk, "bf16", shard) + float(np.sum(peers[mask])))
    pipe.norm.partials.copy_(inp["partials"])
    h = OHyper()
    lo = chunk * shard
    for t in range(1, steps + 1):
        k = (t - 1) % len(sets)
        pipe.step(recvs[k], inp["peer_shards"], t)
        torch.cuda.synchronize()
        what = f"7B N={n} t={t}"
        assert_bits(gather_host(pipe.mean, idx), want_means[k], f"{what} mean (sampled)")
        assert math.isclose(pipe.norm.sqnorm.item(), sqs[k], rel_tol=1e-10), what
        scale = clip_scale(sqs[k], 1.0)
        assert scale < 1
        _clip_factor_bits_agree(pipe.norm.scale.item(), scale, what)
        w, m, v = adamw(w, m, v, want_means[k] * scale, **h.scalars(t))
        for j, want in enumerate((w, m, v)):
            got = gather_host(pipe.state[j], idx)
            assert max_rel(got, want) <= 1e-6, (what, j)
            assert_bits(got, want, f"{what} state {j} (sampled)")
        # The rank's bf16 arena: own chunk = RNE(oracle master); peers' chunks
        # as received.
        assert_bits(gather_host(pipe.arena, idx + lo), bf16_round(w), f"{what} own chunk")
        for j in sorted({1, n // 2, n - 1} - {rank}):
            c = owned_chunk(j, n)
            assert_bits(gather_host(pipe.arena, idx + c * shard),
                        gather_host(inp["peer_shards"][j], idx), f"{what} peer {j}'s chunk")
        if t == 1:
            # Properties over every element (every tile edge of every kernel):
            # after step 1 from m = v = 0 the moments are m = (1 - b1) * g' and
            # v = (1 - b2) * (g' * g'), g' = mean * clip factor, each product
            # rounded once in fp32.
            f32 = dict(dtype=torch.float32, device=DEV)
            g = pipe.mean * pipe.norm.scale
            omb1 = torch.tensor(np.float32(1) - np.float32(h.beta1), **f32)
            omb2 = torch.tensor(np.float32(1) - np.float32(h.beta2), **f32)
            assert torch.equal(pipe.state[1], omb1 * g)
            assert torch.equal(pipe.state[2], omb2 * (g * g))
            del g
    # Every element after the last step: each peer's chunk of the arena is its
    # shard byte for byte and the own chunk is the master rounded to bf16.
    for j in range(n):
        if j == rank:
            continue
        c = owned_chunk(j, n)
        assert torch.equal(pipe.arena[c * shard:(c + 1) * shard], inp["peer_shards"][j]), j
    assert torch.equal(pipe.arena[lo:lo + shard], pipe.state[0].to(torch.bfloat16))


@pytest.mark.parametrize("mode", ["bf16_wire", "token_weighted"])
def test_llama_7b_one_rank_share_modes_sampled(mode):
    # The 7B share (N = 8, rank 0, one bucket, the tiled receive buffer) as
    # `bench.py --wire bf16` and `--token-weighted` run it, one step: the mean
    # at 200 k samples against the
    # oracle's fold (each hop's partial sum rounded to bf16, or the sum divided
    # by the global token count), the norm against the oracle's over the whole
    # shard in tiles, AdamW on the samples and the own chunk of the arena bit
    # for bit.
    a = arena("llama_7b")
    p, n, rank = a.numel, 8, 0
    buckets = grz.whole_arena(p)
    chunk = owned_chunk(rank, n)
    shard = p // n
    npieces = grz.dp_piece_count(buckets, n)
    inp = onerank_inputs(shard, n, rank, npieces, grz.GRZ_PIECE, device=DEV)
    wire, counts = None, None
    if mode == "bf16_wire":
        wire = "bf16"
    else:  # the bench's counts: unequal, their sum not a power of two
        counts = [4096 + 1000 * (j % 3) - 1000 for j in range(n)]
        counts[0] += 123
    divisor = None if counts is None else sum(counts)
    pipe = grz.Zero1OneRank(buckets, n, rank, inp["shard_master"], device=DEV, arena_numel=p,
                            reduce_flags=grz.GRZ_BF16_WIRE if wire else 0)
    idx = sample_indices(shard, 200_000, 11, extra=[4095, 4096, 4097, (1 << 31) - 1, 1 << 31])
    w = gather_host(pipe.state[0], idx)
    peers = host(inp["partials"])
    mask = np.ones(npieces, bool)
    for first, cnt in pipe.own_piece_slots():
        mask[first:first + cnt] = False
    pipe.norm.partials.copy_(inp["partials"])
    pipe.reduce(grz.tiled_receive(inp["incoming"], buckets, n, chunk), token_counts=counts)
    pipe.update(1)
    pipe.gather(inp["peer_shards"])
    torch.cuda.synchronize()
    want = chunk_mean([widen(gather_host(t, idx), "bf16") for t in inp["incoming"]], chunk,
                      True, wire, divisor)
    assert_bits(gather_host(pipe.mean, idx), want, f"7B {mode} mean (sampled)")
    sq = _tiled_sqnorm(inp["incoming"], chunk, "bf16", shard, wire, divisor)
    sq += float(np.sum(peers[mask]))
    assert math.isclose(pipe.norm.sqnorm.item(), sq, rel_tol=1e-10), mode
    scale = clip_scale(sq, 1.0)
    assert scale < 1
    _clip_factor_bits_agree(pipe.norm.scale.item(), scale, f"7B {mode}")
    z = np.zeros_like(w)
    w1, m1, v1 = adamw(w, z, z, want * scale, **OHyper().scalars(1))
    for j, x in enumerate((w1, m1, v1)):
        assert_bits(gather_host(pipe.state[j], idx), x, f"7B {mode} state {j} (sampled)")
    assert_bits(gather_host(pipe.arena, idx + chunk * shard), bf16_round(w1),
                f"7B {mode} own chunk")


def test_llama_7b_ddp_one_rank_sampled():
    # One rank of plain data parallelism at 7B, as the bench runs it (its
    # chunk's inputs in the tiled receive buffer): its full fp32 state holds
    # 6.74e9 elements (beyond 2^32), its own chunk is reduced at arena offsets
    # and the peers' fp32 mean chunks land around it.
    a = arena("llama_7b")
    p, n, rank = a.numel, 8, 0
    buckets = grz.whole_arena(p)
    chunk = owned_chunk(rank, n)
    shard = p // n
    npieces = grz.dp_piece_count(buckets, n)
    inp = onerank_inputs(shard, n, rank, npieces, grz.GRZ_PIECE, device=DEV)
    incoming, partials = inp["incoming"], inp["partials"]
    del inp
    master = master_init(p, device=DEV)
    idx = sample_indices(p, 200_000, 13, extra=[shard - 1, shard, 2 * shard - 1, 2 * shard,
                                                (1 << 32) - 1, 1 << 32, (1 << 32) + 1, p - 1])
    w0 = gather_host(master, idx)
    one = grz.DDPOneRank(buckets, n, rank, master, device=DEV)
    del master
    one.norm.partials.copy_(partials)
    peer_means = [None if j == rank else
                  rank_grad(shard, 1e-3 / n ** 0.5, "f32", grad_seed(1, 100 + j), device=DEV)
                  for j in range(n)]
    peers = host(partials)
    own = one.own_piece_slots()
    one.step(grz.tiled_receive(incoming, buckets, n, chunk), peer_means, 1)
    torch.cuda.synchronize()

    # The mean: the own chunk bit-exact against the oracle's fold, every peer
    # chunk byte for byte what that peer delivered (all of it, chunk by chunk).
    lo = chunk * shard
    mine = (idx >= lo) & (idx < lo + shard)
    want_own = oracle_mean_at([gather_host(g, idx[mine] - lo) for g in incoming],
                              np.full(int(mine.sum()), chunk), "bf16")
    assert_bits(gather_host(one.mean, idx[mine]), want_own, "7B DDP own chunk (sampled)")
    for j in range(n):
        if j != rank:
            c = owned_chunk(j, n)
            assert torch.equal(one.mean[c * shard:(c + 1) * shard], peer_means[j]), j
    # Norm: the own pieces recomputed from the inputs, the peers' as received.
    mask = np.ones(npieces, bool)
    for first, cnt in own:
        mask[first:first + cnt] = False
    sq = _tiled_sqnorm(incoming, chunk, "bf16", shard) + float(np.sum(peers[mask]))
    assert math.isclose(one.norm.sqnorm.item(), sq, rel_tol=1e-10)
    scale = clip_scale(sq, 1.0)
    _clip_factor_bits_agree(one.norm.scale.item(), scale, "7B DDP")
    # AdamW over the whole arena, sampled, on the oracle's mean of each element.
    g_at = np.empty(idx.size, np.float32)
    g_at[mine] = want_own
    for j in range(n):  # the peers' chunks: the values they delivered
        c = owned_chunk(j, n)
        sel = (idx >= c * shard) & (idx < (c + 1) * shard)
        if j != rank:
            g_at[sel] = gather_host(peer_means[j], idx[sel] - c * shard)
    z = np.zeros_like(w0)
    w1, m1, v1 = adamw(w0, z, z, g_at * scale, **OHyper().scalars(1))
    for k, want in enumerate((w1, m1, v1)):
        got = gather_host(one.state[k], idx)
        assert max_rel(got, want) <= 1e-6
        assert_bits(got, want, f"7B DDP state {k} (sampled)")
    assert_bits(gather_host(one.arena, idx), bf16_round(w1), "7B DDP arena (sampled)")
    # Every element, one chunk at a time: the arena is the master rounded to
    # bf16 and the step-1 moments are (1 - b1) * g' and (1 - b2) * (g' * g').
    h = OHyper()
    f32 = dict(dtype=torch.float32, device=DEV)
    omb1 = torch.tensor(np.float32(1) - np.float32(h.beta1), **f32)
    omb2 = torch.tensor(np.float32(1) - np.float32(h.beta2), **f32)
    for c in range(n):
        sl = slice(c * shard, (c + 1) * shard)
        assert torch.equal(one.arena[sl], one.state[0][sl].to(torch.bfloat16)), c
        g = one.mean[sl] * one.norm.scale
        assert torch.equal(one.state[1][sl], omb1 * g), c
        assert torch.equal(one.state[2][sl], omb2 * (g * g)), c


def test_gpt2_1p5b_all_ranks_11_steps_sampled():
    # GPT-2 1.5B, all 4 ranks, 11 steps: the learning rate warms up linearly
    # over 10 steps (1e-5, 2e-5, ..., 1e-4) and stays at 1e-4 at step 11.  The
    # same seeded gradients every step, so that the oracle's norm over the
    # 1.56e9-element mean is computed once (in tiles); the mean is reduced
    # again every step and checked on 100 k sampled elements, and the oracle
    # carries master, m and v on the samples through all 11 steps.
    a = arena("gpt2_1p5b")
    p, n = a.numel, 4
    buckets = [(0, p)]
    hyper = grz.Hyper(lr=1e-4, warmup=10, max_norm=1.0)
    h = OHyper(lr=1e-4, warmup=10)
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    idx = sample_indices(p, 100_000, 11, extra=[p // 4 - 1, p // 4, p // 2, 3 * p // 4])
    w = gather_host(master, idx)
    m, v = np.zeros_like(w), np.zeros_like(w)
    del master
    grads = [rank_grad(p, 1e-3, "bf16", grad_seed(1, r), device=DEV) for r in range(n)]
    _, chunks = chunk_of_index(buckets, n, idx)
    want_mean = oracle_mean_at([gather_host(g, idx) for g in grads], chunks, "bf16")
    shard = p // n
    sq = 0.0
    for r in range(n):
        c = owned_chunk(r, n)
        sq += _tiled_sqnorm([g[c * shard:(c + 1) * shard] for g in grads], c, "bf16", shard)
    scale = clip_scale(sq, 1.0)
    assert scale < 1
    for t in range(1, 12):
        z.step(grads, t)
        torch.cuda.synchronize()
        what = f"1.5B t={t}"
        s = h.scalars(t)
        assert s["lr"] == np.float32(1e-4 * min(t, 10) / 10), what
        assert float(np.float32(grz.step_scalars(hyper, t)["lr"])) == float(s["lr"]), what
        for r in range(n):
            c = owned_chunk(r, n)
            sel = chunks == c
            assert_bits(gather_host(z.means[r], idx[sel] - c * shard), want_mean[sel],
                        f"{what} mean rank {r}")
        assert math.isclose(z.norm.sqnorm.item(), sq, rel_tol=1e-10), what
        _clip_factor_bits_agree(z.norm.scale.item(), scale, what)
        w, m, v = adamw(w, m, v, want_mean * scale, **s)
        for r in range(n):
            c = owned_chunk(r, n)
            sel = chunks == c
            for k, want in enumerate((w, m, v)):
                got = gather_host(z.state[r][k], idx[sel] - c * shard)
                assert max_rel(got, want[sel]) <= 1e-6, (what, r, k)
                assert_bits(got, want[sel], f"{what} state {k} rank {r}")
        for rep in (z.replicas[0], z.replicas[3]):
            assert_bits(gather_host(rep, idx), bf16_round(w), f"{what} replicas")
        if t == 1:
            # Every element: the step-1 moments are (1 - b1) * g' and
            # (1 - b2) * (g' * g') with g' = mean * clip factor.
            f32 = dict(dtype=torch.float32, device=DEV)
            omb1 = torch.tensor(np.float32(1) - np.float32(s["beta1"]), **f32)
            omb2 = torch.tensor(np.float32(1) - np.float32(s["beta2"]), **f32)
            for r in range(n):
                g = z.means[r] * z.norm.scale
                assert torch.equal(z.state[r][1], omb1 * g), r
                assert torch.equal(z.state[r][2], omb2 * (g * g)), r
                del g
    # Every element after the last step: all replicas hold the same bytes and
    # chunk c of each is rank r's master rounded to bf16.
    for rep in z.replicas[1:]:
        assert torch.equal(rep, z.replicas[0])
    for r in range(n):
        c = owned_chunk(r, n)
        assert torch.equal(z.replicas[0][c * shard:(c + 1) * shard],
                           z.state[r][0].to(torch.bfloat16)), r


def test_char_gpt_100_steps_zero1_equals_ddp_every_step():
    # The char GPT workload runs 100 steps.  The oracle checks the first ten
    # (test_char_gpt_all_ranks_10_steps); over all 100, ZeRO-1 and plain data
    # parallelism must stay bit-identical (same pieces, same norm, same update)
    # and finite.
    a = arena("char_gpt")
    p, n = a.numel, 8
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV)
    d = grz.DDPStep(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV)
    spans = _layer_spans(a)
    for t in range(1, 101):
        grads = [rank_grad(p, 1e-3, "bf16", grad_seed(t, r), DEV, spans) for r in range(n)]
        z.step(grads, t)
        d.step(grads, t)
        if t % 10 == 0 or t == 1:
            torch.cuda.synchronize()
            assert torch.equal(z.norm.sqnorm, d.norm.sqnorm), t
            assert torch.equal(z.replicas[t % n].view(torch.int16), d.replica.view(torch.int16)), t
    torch.cuda.synchronize()
    assert torch.isfinite(d.state[0]).all()
    assert z.norm.scale.item() < 1
