"""Host planning of the product against the oracle's independent versions."""

import io

import numpy as np
import pytest

from gradient_reduce_zero_amd.plan import Hyper, plan_buckets, step_scalars, zero_stage
from oracle.plan import plan_buckets as oracle_plan
from oracle.step import Hyper as OHyper
from workloads import arena


@pytest.mark.parametrize("name", ["tiny", "char_gpt", "gpt2_124m", "gpt2_1p5b", "llama_7b"])
@pytest.mark.parametrize("cap", [25 * 2 ** 20, 25 * 10 ** 6, 1 << 16])
def test_plan_buckets_matches_oracle(name, cap):
    a = arena(name)
    assert plan_buckets(a.numels, cap, 2) == oracle_plan(a.numels, cap, 2)


def test_plan_small_cases_match_oracle():
    rng = np.random.default_rng(0)
    for _ in range(200):
        numels = rng.integers(0, 50, size=rng.integers(0, 12)).tolist()
        cap = int(rng.integers(1, 120))
        assert plan_buckets(numels, cap, 1) == oracle_plan(numels, cap, 1)


@pytest.mark.parametrize("t", [1, 2, 5, 10, 11, 100, 1000])
def test_step_scalars_match_oracle(t):
    ours = step_scalars(Hyper(lr=1e-4, warmup=10), t)
    ref = OHyper(lr=1e-4, warmup=10).scalars(t)
    assert np.float32(ours["lr"]) == ref["lr"]
    assert np.float32(ours["bias_corr1"]) == ref["bc1"]
    assert np.float32(ours["bias_corr2"]) == ref["bc2"]
    assert np.float32(ours["beta1"]) == np.float32(ref["beta1"])
    with pytest.raises(ValueError):
        step_scalars(Hyper(), 0)


def test_zero_stage_fallback_message():
    log = io.StringIO()
    assert zero_stage([(0, 64), (64, 63)], 4, 1, log) == 0
    assert "split evenly over 4 ranks" in log.getvalue() and "stage 0" in log.getvalue()
    assert zero_stage([(0, 64)], 4, 1, io.StringIO()) == 1
    assert zero_stage([(0, 64)], 4, 0, io.StringIO()) == 0


def test_resident_bytes_against_the_zero_table():
    from gradient_reduce_zero_amd.plan import resident_bytes
    from oracle.memory import zero_memory_bytes
    p, n = 7e9, 8
    # Stage 0 and 1 differ from the page's model only by the fp32 reduced
    # gradient this pipeline keeps for the optimizer (4 bytes per kept param).
    assert resident_bytes(p, n, 0) == zero_memory_bytes(p, n, 0) + 4 * p
    assert resident_bytes(p, n, 1) == zero_memory_bytes(p, n, 1) + 4 * p / n
    # Stage 2: bf16 shards of the page become fp32 shards, plus the staging.
    longest = 25 * 2 ** 20 // 2
    assert resident_bytes(p, n, 2, longest_bucket=longest) == \
        zero_memory_bytes(p, n, 2) + 2 * p / n + 4 * longest
    # With the gradient shard held in bf16 the stage-2 state is the page's
    # 2 + 14/N bytes per parameter (26.25 GB for 7e9 on 8), the staging on top.
    assert resident_bytes(p, n, 2, shard_bytes=2) == zero_memory_bytes(p, n, 2) == 26.25e9
    assert resident_bytes(p, n, 2, longest_bucket=longest, shard_bytes=2) == \
        zero_memory_bytes(p, n, 2) + 4 * longest
    with pytest.raises(ValueError):
        resident_bytes(p, n, 2, shard_bytes=1)


def test_one_rank_step_falls_back_to_plain_data_parallelism(capsys):
    # Built on the host (no kernel runs): an even plan gives the rank its ZeRO-1
    # shard; a bucket N does not divide gives it the whole arena, with the
    # fallback said on stderr.
    import torch

    import gradient_reduce_zero_amd as grz

    master = torch.arange(8 * 40, dtype=torch.float32)
    z = grz.one_rank_step([(0, 8 * 40)], 8, 3, master, device="cpu")
    assert isinstance(z, grz.Zero1OneRank) and capsys.readouterr().err == ""
    lo = grz.owned_chunk(3, 8) * 40
    assert torch.equal(z.state[0], master[lo:lo + 40]) and z.arena.numel() == 320
    d = grz.one_rank_step([(0, 8 * 40 - 3), (8 * 40 - 3, 3)], 8, 3, master, device="cpu")
    assert isinstance(d, grz.DDPOneRank) and d.flags == grz.GRZ_UNEVEN
    assert torch.equal(d.state[0], master)
    assert "running ZeRO stage 0" in capsys.readouterr().err
    s0 = grz.one_rank_step([(0, 8 * 40)], 8, 3, master, device="cpu", stage=0)
    assert isinstance(s0, grz.DDPOneRank) and s0.flags == 0


def test_shard_state_sits_at_the_phase_of_its_arena_position():
    # GPT-2 1.5B at N = 4: chunks 1 and 3 start 16 elements past a 32-element
    # boundary of the arena, so their fp32 state goes 16 elements (64 bytes)
    # into a 128-byte line; chunks 0 and 2 and the DDP layout stay at 0.
    import torch

    import gradient_reduce_zero_amd as grz

    p = arena("gpt2_1p5b").numel
    assert [grz.state_phase(grz.whole_arena(p), 4, c) for c in range(4)] == [0, 16, 0, 16]
    assert grz.state_phase(grz.whole_arena(p), 4, -1) == 0
    # Two buckets at N = 4, chunk 1: the first has d = 64 - 0 = 0 (mod 32) over
    # 64 elements, the second d = 256 + 1008 - 64 = 16 over 1008: the longer wins.
    assert grz.state_phase([(0, 256), (256, 4032)], 4, 1) == 16
    assert grz.state_phase([(0, 4 * 2048), (4 * 2048, 4032)], 4, 1) == 0  # 2048 at d = 0
    assert grz.state_phase([(0, 256), (256, 4000)], 4, 1) == 8  # d = 8 over 1000
    # d = 9 would leave the arrays off their 16-byte alignment: phase 0.
    assert grz.state_phase([(0, 256), (256, 4004)], 4, 1) == 0
    for phase in (0, 4, 16, 28):
        t = grz.placed_zeros(1000, phase, "cpu")
        assert t.numel() == 1000 and (t.data_ptr() // 4) % 32 == phase
        assert not t.any()
    master = torch.arange(4 * 48, dtype=torch.float32)
    shard = master[48:96]
    z = grz.Zero1OneRank(grz.whole_arena(4 * 48), 4, 0, shard, device="cpu")
    for x in (*z.state, z.mean):
        assert (x.data_ptr() // 4) % 32 == 16 and x.numel() == 48
    assert torch.equal(z.state[0], shard) and not z.state[1].any()
    assert z.state[0].data_ptr() != shard.data_ptr()  # the step holds a copy
    zf = grz.Zero1OneRank(grz.whole_arena(4 * 48), 4, 0, shard, device="cpu", fused=True)
    assert zf.mean is None
    za = grz.Zero1AllRanks(grz.whole_arena(4 * 48), 4, master, device="cpu")
    for c, (w, m, v), mean in zip(za.chunks, za.state, za.means):
        want = 16 if c % 2 else 0
        assert all((x.data_ptr() // 4) % 32 == want for x in (w, m, v, mean))
        assert torch.equal(w, master[c * 48:(c + 1) * 48])


def test_steps_over_every_chunk_refuse_a_tiled_receive_buffer():
    # A tiled receive buffer holds one rank's chunk: the all-ranks steps, which
    # read every rank's full arena, refuse it before any call into the library.
    import torch

    import gradient_reduce_zero_amd as grz

    master = torch.zeros(4 * 64)
    tiled = grz.Tiled(torch.zeros(4 * 4 * grz.GRZ_PIECE), 4)
    z = grz.Zero1AllRanks([(0, 4 * 64)], 4, master, device="cpu")
    d = grz.DDPStep([(0, 4 * 64)], 4, master, device="cpu", nreplicas=4)
    for step in (z, d):
        with pytest.raises(TypeError, match="tiled receive buffer"):
            step.enqueue(tiled, grz.adamw_args(1e-3, 0.9, 0.95, 1e-8, 0.1, 0.1, 0.05))
    with pytest.raises(TypeError, match="tiled receive buffer"):
        grz.OverlappedZero1.bucket_ready(type("P", (), {"pipe": z})(), 0, tiled)


@pytest.mark.parametrize("n,lengths", [(8, [8 * 5000, 8 * 4096]), (3, [64, 3 * 4096 + 2, 0]),
                                       (16, [16 * 4096 * 3])])
def test_tiled_receive_layout(n, lengths):
    # On the host (no kernel runs): piece k of the chunk (in plan order, the
    # array_split chunk rule) lands in slot k with rank j's values at j * 4096;
    # the rest of a short piece's slot stays zero.
    import torch

    import gradient_reduce_zero_amd as grz
    from oracle.reduce import shard_segments

    T = grz.GRZ_PIECE
    offs, pos = [], 0
    for length in lengths:
        offs.append(pos)
        pos += length
    buckets = list(zip(offs, lengths))
    uneven = any(length % n for length in lengths)
    for chunk in (0, n - 1):
        segs = shard_segments(buckets, n, chunk, uneven=uneven)
        shard = sum(length for _, length, _ in segs)
        rng = np.random.default_rng(chunk)
        incoming = [torch.from_numpy(rng.standard_normal(shard).astype(np.float32) + 1)
                    for _ in range(n)]
        t = grz.tiled_receive(incoming, buckets, n, chunk)
        got = t.buffer.numpy().reshape(-1, n, T)
        want = np.zeros_like(got)
        k = 0
        for _, length, c0 in segs:
            for a in range(0, length, T):
                e = min(length, a + T)
                for j in range(n):
                    want[k, j, :e - a] = incoming[j].numpy()[c0 + a:c0 + e]
                k += 1
        assert k * n * T == t.buffer.numel() and t.nranks == n
        assert np.array_equal(got, want)
