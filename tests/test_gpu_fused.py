"""The one-launch step (zero1_fused_step) against the three-kernel path and the
oracle.

The fused kernel holds the mean in registers and passes the piece sums
between its workgroups through self-flagging workspace slots (no grid
barrier), so that every workgroup can clip once the norm is known; every
value it produces must have the bits of dp_reduce_scatter_mean ->
dp_grad_sqnorm -> zero1_adamw_gather on the same inputs, which the oracle
pins independently.
"""

import math

import numpy as np
import pytest
import torch

import gradient_reduce_zero_amd as grz
from oracle.reduce import owned_chunk, reduce_scatter_mean, shard_segments
from oracle.step import Hyper as OHyper
from oracle.step import ddp_step
from parity_util import assert_bits, host
from workloads import arena, grad_seed, master_init, onerank_inputs, rank_grad

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _same(a, b, what):
    assert_bits(host(a), host(b), what)


# --- plain data parallelism in one launch, against the oracle -------------------

@pytest.mark.parametrize("max_norm", [1.0, 0.1])
def test_fused_ddp_tiny_10_steps_matches_oracle(max_norm):
    p, n = 4096, 2
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    d = grz.DDPStep(buckets, n, master, grz.Hyper(max_norm=max_norm), device=DEV, fused=True)
    dstate = (host(master), np.zeros(p, np.float32), np.zeros(p, np.float32))
    for t in range(1, 11):
        grads = [rank_grad(p, 0.01, "f32", grad_seed(t, r), device=DEV) for r in range(n)]
        d.step(grads, t)
        torch.cuda.synchronize()
        ref = ddp_step([host(g) for g in grads], "f32", buckets, dstate, OHyper(max_norm=max_norm),
                       t)
        dstate = ref["state"]
        assert math.isclose(d.norm.sqnorm.item(), ref["sqnorm"], rel_tol=1e-13)
        assert_bits(host(d.norm.scale), np.array([ref["scale"]], np.float32), f"t={t} scale")
        for k, name in enumerate(("master", "m", "v")):
            assert_bits(host(d.state[k]), ref["state"][k], f"t={t} {name}")
        assert_bits(host(d.replica), ref["arena"], f"t={t} bf16 weights")
    assert not grz.fused_timed_out(d.workspace)
    assert (ref["scale"] < 1) == (max_norm == 0.1)


def test_fused_ddp_char_gpt_equals_zero1_all_ranks():
    # 10.77 M parameters, N = 8: 2632 pieces in 8 segments, one launch.
    a = arena("char_gpt")
    p, n = a.numel, 8
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV)
    d = grz.DDPStep(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV, fused=True)
    for t in range(1, 6):
        grads = [rank_grad(p, 1e-3, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]
        z.step(grads, t)
        d.step(grads, t)
        torch.cuda.synchronize()
        _same(d.norm.partials, z.norm.partials, f"t={t} pieces")
        _same(d.norm.sqnorm, z.norm.sqnorm, f"t={t} sqnorm")
        _same(d.norm.scale, z.norm.scale, f"t={t} scale")
        _same(d.replica, z.replicas[t % n], f"t={t} weights")
    assert z.norm.scale.item() < 1
    # The master of every shard against the fused DDP master.
    for r in range(n):
        c = owned_chunk(r, n)
        lo, cnt = grz.dp_chunk_range(p, n, c)
        _same(d.state[0][lo:lo + cnt], z.state[r][0], f"master of rank {r}")
        _same(d.state[2][lo:lo + cnt], z.state[r][2], f"v of rank {r}")
    assert not grz.fused_timed_out(d.workspace)


# --- one rank's ZeRO-1 share in one launch ------------------------------------

def _one_rank_pair(buckets, p, n, rank):
    chunk = owned_chunk(rank, n)
    shard = grz.dp_shard_numel(buckets, n, chunk)
    npieces = grz.dp_piece_count(buckets, n)
    inp = onerank_inputs(shard, n, rank, npieces, grz.GRZ_PIECE, device=DEV)
    three = grz.Zero1OneRank(buckets, n, rank, inp["shard_master"].clone(), device=DEV,
                             arena_numel=p)
    one = grz.Zero1OneRank(buckets, n, rank, inp["shard_master"].clone(), device=DEV,
                           arena_numel=p, fused=True)
    for z in (three, one):
        z.norm.partials.copy_(inp["partials"])
    return inp, three, one


@pytest.mark.parametrize("config", ["char_gpt", "gpt2_124m"])
def test_fused_one_rank_equals_three_kernels(config):
    a = arena(config)
    p, n, rank = a.numel, 8, 3
    buckets = grz.plan_buckets(a.numels, 25 * 2 ** 20, 2) if config == "gpt2_124m" \
        else [(0, p)]
    inp, three, one = _one_rank_pair(buckets, p, n, rank)
    if config == "gpt2_124m":
        assert one.norm.npieces > 4096  # the norm tree has a level below the final fold
    mean_copy = torch.full_like(three.mean, float("nan"))
    for t in (1, 2, 3):
        three.step(inp["incoming"], inp["peer_shards"], t)
        if t == 1:  # once with the optional copy of the mean, launched cooperatively
            w, m, v = one.state
            grz.zero1_fused_step(inp["incoming"], buckets, one.chunk, w, m, v,
                                 grz.adamw_args(**grz.step_scalars(one.hyper, t)),
                                 one.hyper.max_norm, [one.arena], one.norm.partials,
                                 one.workspace, one.norm.sqnorm, one.norm.scale,
                                 mean_out=mean_copy,
                                 flags=grz.GRZ_IN_COMPACT | grz.GRZ_COOPERATIVE)
            one.gather(inp["peer_shards"])
        else:
            one.step(inp["incoming"], inp["peer_shards"], t)
        torch.cuda.synchronize()
        if t == 1:
            _same(mean_copy, three.mean, "mean")
        for x, y, what in ((one.norm.partials, three.norm.partials, "pieces"),
                           (one.norm.sqnorm, three.norm.sqnorm, "sqnorm"),
                           (one.norm.scale, three.norm.scale, "scale"),
                           (one.state[0], three.state[0], "master"),
                           (one.state[1], three.state[1], "m"),
                           (one.state[2], three.state[2], "v"),
                           (one.arena, three.arena, "arena")):
            _same(x, y, f"{config} t={t} {what}")
    assert three.norm.scale.item() < 1
    assert not grz.fused_timed_out(one.workspace)


def test_fused_one_rank_mean_matches_oracle():
    # Shard-compact inputs of rank 0 (chunk 1) with three buckets, one ragged:
    # the fused mean copy against the oracle's fold of the same bytes.
    n, rank = 8, 0
    buckets = [(8 * 5000, 8 * 4096 * 2), (0, 8 * 5000), (8 * 5000 + 8 * 8192, 8 * 17)]
    p = 8 * (5000 + 8192 + 17)
    chunk = owned_chunk(rank, n)
    shard = grz.dp_shard_numel(buckets, n, chunk)
    npieces = grz.dp_piece_count(buckets, n)
    inp = onerank_inputs(shard, n, rank, npieces, grz.GRZ_PIECE, device=DEV)
    one = grz.Zero1OneRank(buckets, n, rank, inp["shard_master"].clone(), device=DEV,
                           arena_numel=p, fused=True)
    one.norm.partials.copy_(inp["partials"])
    mean = torch.empty(shard, dtype=torch.float32, device=DEV)
    w, m, v = one.state
    grz.zero1_fused_step(inp["incoming"], buckets, chunk, w, m, v,
                         grz.adamw_args(**grz.step_scalars(one.hyper, 1)), 1.0, [one.arena],
                         one.norm.partials, one.workspace, one.norm.sqnorm, one.norm.scale,
                         mean_out=mean, flags=grz.GRZ_IN_COMPACT)
    torch.cuda.synchronize()
    want = reduce_scatter_mean([host(g) for g in inp["incoming"]], "bf16", buckets, chunk,
                               compact_inputs=True)
    assert_bits(host(mean), want, "fused mean vs oracle")


# --- ragged, unaligned and N = 3 ---------------------------------------------

@pytest.mark.parametrize("n,kind", [(1, "f32"), (1, "bf16"), (2, "f32"), (2, "bf16"),
                                    (3, "f32"), (3, "bf16"), (4, "f32"), (4, "bf16"),
                                    (5, "bf16"), (8, "f32"), (8, "bf16")])
def test_fused_ragged_unaligned_matches_three_kernels_and_oracle(n, kind):
    # Uneven chunks (GRZ_UNEVEN), a bucket shorter than N, pieces with ragged
    # tails, and every base one element past a 16-byte boundary (element-wise
    # accesses throughout).  N = 1, 2, 4 and 8 have their own kernel instances
    # (a fold unrolled for that N), the others share the one that loops.
    buckets = [(3 * 4096 + 11, 2 * 4096 + 7), (0, 3 * 4096 + 11), (5 * 4096 + 18, 2)]
    p = 5 * 4096 + 20
    flags = grz.GRZ_UNEVEN

    def off(t):  # the same values, one element further along
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        buf[1:] = t
        return buf[1:]

    master = master_init(p, device=DEV)
    grads = [off(rank_grad(p, 1e-2, kind, grad_seed(1, r), device=DEV)) for r in range(n)]
    hyper = grz.Hyper(max_norm=0.05)
    three = grz.DDPStep(buckets, n, master, hyper, device=DEV, reduce_flags=flags)
    one = grz.DDPStep(buckets, n, master, hyper, device=DEV, reduce_flags=flags, fused=True)
    one.state = tuple(off(x) for x in one.state)
    one.replicas = [off(one.replica)]
    one.replica = one.replicas[0]
    dstate = (host(master), np.zeros(p, np.float32), np.zeros(p, np.float32))
    for t in (1, 2):
        three.step(grads, t)
        one.step(grads, t)
        torch.cuda.synchronize()
        ref = ddp_step([host(g) for g in grads], kind, buckets, dstate, OHyper(max_norm=0.05), t)
        dstate = ref["state"]
        for k in range(3):
            _same(one.state[k], three.state[k], f"N={n} t={t} state {k}")
            assert_bits(host(one.state[k]), ref["state"][k], f"N={n} t={t} state {k} vs oracle")
        _same(one.replica, three.replica, f"N={n} t={t} weights")
        assert_bits(host(one.replica), ref["arena"], f"N={n} t={t} weights vs oracle")
        _same(one.norm.sqnorm, three.norm.sqnorm, f"N={n} t={t} sqnorm")
    assert ref["scale"] < 1


# --- device-side step scalars --------------------------------------------------

def test_fused_device_args_equal_host_args():
    p, n = 8 * 4096 + 64, 4
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    grads = [rank_grad(p, 1e-2, "bf16", grad_seed(2, r), device=DEV) for r in range(n)]
    hyper = grz.Hyper(max_norm=0.3, warmup=4)
    host_args = grz.DDPStep(buckets, n, master, hyper, device=DEV, fused=True)
    dev_args = grz.DDPStep(buckets, n, master, hyper, device=DEV, fused=True)
    for t in (1, 2, 3):
        host_args.step(grads, t)
        s = grz.step_scalars(hyper, t)
        row = torch.tensor([s[k] for k in ("lr", "beta1", "beta2", "eps", "weight_decay",
                                           "bias_corr1", "bias_corr2")],
                           dtype=torch.float32, device=DEV)
        w, m, v = dev_args.state
        grz.zero1_fused_step(grads, buckets, -1, w, m, v, row, hyper.max_norm,
                             [dev_args.replica], dev_args.norm.partials, dev_args.workspace)
        torch.cuda.synchronize()
        for k in range(3):
            _same(dev_args.state[k], host_args.state[k], f"t={t} state {k}")
        _same(dev_args.replica, host_args.replica, f"t={t} weights")


# --- refusals and the bounded wait --------------------------------------------

def test_fused_refuses_what_it_cannot_hold():
    cap = grz.zero1_fused_capacity(1, torch.float32)
    # 4 pieces per resident workgroup but the one that folds the norm: 1023 on
    # a 256-CU MI355X.
    assert cap >= 4092
    p = (cap + 1) * grz.GRZ_PIECE
    g = torch.zeros(p, device=DEV)
    st = [torch.zeros(p, device=DEV) for _ in range(3)]
    rep = torch.zeros(p, dtype=torch.bfloat16, device=DEV)
    parts = torch.zeros(cap + 1, dtype=torch.float64, device=DEV)
    ws = torch.zeros(grz.zero1_fused_workspace(cap + 1), dtype=torch.uint8, device=DEV)
    args = grz.adamw_args(**grz.step_scalars(grz.Hyper(), 1))
    with pytest.raises(grz.GrzError, match="out of range"):
        grz.zero1_fused_step([g], [(0, p)], -1, *st, args, 1.0, [rep], parts, ws)
    # More than 32 (bucket, chunk) segments.
    buckets = [(8 * i, 8) for i in range(5)]  # 5 buckets x 8 chunks = 40 segments
    small = [torch.zeros(40, device=DEV) for _ in range(8)]
    st = [torch.zeros(40, device=DEV) for _ in range(3)]
    rep = torch.zeros(40, dtype=torch.bfloat16, device=DEV)
    parts = torch.zeros(40, dtype=torch.float64, device=DEV)
    with pytest.raises(grz.GrzError, match="out of range"):
        grz.zero1_fused_step(small, buckets, -1, *st, args, 1.0, [rep], parts, ws)
    # The bf16-wire fold and the sum mode are the separate entry points' only.
    for flag in (grz.GRZ_BF16_WIRE, grz.GRZ_SUM):
        with pytest.raises(grz.GrzError, match="invalid"):
            grz.zero1_fused_step([x.to(torch.bfloat16) for x in small], buckets[:1], -1, *st,
                                 args, 1.0, [rep], parts, ws, flags=flag)
    torch.cuda.synchronize()
    assert not grz.fused_timed_out(ws)


@pytest.mark.parametrize("config", ["char_gpt", "gpt2_124m"])
def test_fused_wait_that_gives_up_writes_nothing_and_is_reported(config):
    # A poll limit of one makes every workgroup that has to wait give up at
    # once.  The call still ends (every wait is bounded) and the flag is up.
    # A workgroup that gave up writes nothing after its wait, so every piece
    # of the shard holds either its old state or the correct update (the
    # three-kernel path's), never anything else; the step's check reports the
    # give-up and clears the workspace, keeping its poll limit.  Restarted
    # from the same state with the default limit, the next call is exact
    # again.  The char GPT's plan (fewer than 4096 pieces) has one level of
    # waits (workgroup 0 for the pieces, everyone for the norm); GPT-2 124M's
    # (30,416 pieces, 9 buckets) two, any of which can give up.
    a = arena(config)
    p, n, rank = a.numel, 8, 5
    buckets = grz.plan_buckets(a.numels) if config == "gpt2_124m" else [(0, p)]
    inp, three, one = _one_rank_pair(buckets, p, n, rank)
    three.step(inp["incoming"], inp["peer_shards"], 1)
    old = [host(x) for x in one.state]
    old_arena = host(one.arena)
    grz.fused_set_spin_limit(one.workspace, 1)
    one.step(inp["incoming"], inp["peer_shards"], 1)
    torch.cuda.synchronize()
    assert grz.fused_timed_out(one.workspace)
    with pytest.raises(RuntimeError, match="gave up"):
        one.check_fused()
    assert not grz.fused_timed_out(one.workspace)
    words = one.workspace.view(torch.int32)
    assert int(words[3].item()) == 1 and int(words.abs().sum().item()) == 1
    new = [host(x) for x in three.state]
    got = [host(x) for x in one.state]
    got_arena, new_arena = host(one.arena), host(three.arena)
    updated = pieces = 0
    for g0, length, c0 in shard_segments(buckets, n, one.chunk):
        for k0 in range(0, length, grz.GRZ_PIECE):  # the pieces (tiles) of this segment
            k1 = min(k0 + grz.GRZ_PIECE, length)
            sl, asl = slice(c0 + k0, c0 + k1), slice(g0 + k0, g0 + k1)
            same_old = all(np.array_equal(x[sl].view(np.uint32), o[sl].view(np.uint32))
                           for x, o in zip(got, old))
            same_new = all(np.array_equal(x[sl].view(np.uint32), w[sl].view(np.uint32))
                           for x, w in zip(got, new))
            assert same_old or same_new, f"piece at {c0 + k0}: neither old state nor update"
            want = new_arena[asl] if same_new else old_arena[asl]
            assert np.array_equal(got_arena[asl], want), f"arena piece at {g0 + k0}"
            updated += same_new and not same_old
            pieces += 1
    print(f"{updated} of {pieces} pieces updated before the give-up")
    # Start again from the same state with the default poll limit.
    grz.fused_set_spin_limit(one.workspace, 0)
    one.state[0].copy_(inp["shard_master"])
    one.state[1].zero_()
    one.state[2].zero_()
    one.norm.partials.copy_(inp["partials"])
    one.step(inp["incoming"], inp["peer_shards"], 1)
    torch.cuda.synchronize()
    one.check_fused()
    for k in range(3):
        _same(one.state[k], three.state[k], f"after the restart: state {k}")
    _same(one.arena, three.arena, "after the restart: arena")


@pytest.mark.parametrize("bad", ["nan", "inf", "peer_nan"])
def test_fused_non_finite_gradient_equals_three_kernels(bad):
    # A NaN or an infinity in one rank's gradient (or a NaN among the peers'
    # piece sums): the norm is NaN or +Inf, the clip factor 1 (NaN) or 0
    # (Inf, max_norm / Inf), and the update propagates it.  The published slot
    # carries a NaN as the one quiet NaN, so only the NaN's payload in the
    # norm may differ; master, m, v and the arena equal the three kernels'
    # bit for bit (NaN where the three kernels have NaN).
    a = arena("char_gpt")
    p, n, rank = a.numel, 8, 4
    buckets = [(0, p)]
    inp, three, one = _one_rank_pair(buckets, p, n, rank)
    if bad == "peer_nan":
        slot = next(i for i in range(one.norm.npieces)
                    if all(not (f <= i < f + c) for f, c in one.own_piece_slots()))
        for z in (three, one):
            z.norm.partials[slot] = float("nan")
    else:
        g = inp["incoming"][5].view(torch.int16)
        g[1234] = 0x7FC0 if bad == "nan" else 0x7F80  # bf16 NaN / +Inf
    three.step(inp["incoming"], inp["peer_shards"], 1)
    one.step(inp["incoming"], inp["peer_shards"], 1)
    torch.cuda.synchronize()
    one.check_fused()
    s3, s1 = three.norm.sqnorm.item(), one.norm.sqnorm.item()
    if bad == "inf":
        assert s3 == s1 == float("inf")
    else:
        assert math.isnan(s3) and math.isnan(s1)
    _same(one.norm.scale, three.norm.scale, "clip factor")
    for k in range(3):
        _same(one.state[k], three.state[k], f"{bad}: state {k}")
    _same(one.arena, three.arena, f"{bad}: arena")


def test_fused_workspace_refuses_a_plan_of_another_piece_count():
    # A workspace's published piece sums carry the parity of the launch that
    # wrote them; they alternate launch by launch only while every launch
    # rewrites all of them.  A call whose plan has another piece count than
    # the last call's raises the flag and writes nothing; once the workspace
    # is cleared the same call equals the three-kernel step.
    n = 4
    small, big = [(0, n * 4096 * 3)], [(0, n * 4096 * 5)]
    p = big[0][1]
    master = master_init(p, device=DEV)
    grads = [rank_grad(p, 1e-2, "bf16", grad_seed(5, r), device=DEV) for r in range(n)]
    hyper = grz.Hyper(max_norm=0.5)
    args = grz.adamw_args(**grz.step_scalars(hyper, 1))
    ws = torch.zeros(grz.zero1_fused_workspace(grz.dp_piece_count(big, n)), dtype=torch.uint8,
                     device=DEV)
    q = small[0][1]
    s1 = [master[:q].clone(), torch.zeros(q, device=DEV), torch.zeros(q, device=DEV)]
    r1 = torch.zeros(q, dtype=torch.bfloat16, device=DEV)
    parts1 = torch.zeros(grz.dp_piece_count(small, n), dtype=torch.float64, device=DEV)
    grz.zero1_fused_step([g[:q] for g in grads], small, -1, *s1, args, hyper.max_norm, [r1],
                         parts1, ws)
    torch.cuda.synchronize()
    assert not grz.fused_timed_out(ws)
    s2 = [master.clone(), torch.zeros(p, device=DEV), torch.zeros(p, device=DEV)]
    r2 = torch.zeros(p, dtype=torch.bfloat16, device=DEV)
    parts2 = torch.zeros(grz.dp_piece_count(big, n), dtype=torch.float64, device=DEV)
    grz.zero1_fused_step(grads, big, -1, *s2, args, hyper.max_norm, [r2], parts2, ws)
    torch.cuda.synchronize()
    assert grz.fused_timed_out(ws)
    _same(s2[0], master, "refused call: master untouched")
    assert not s2[1].any() and not s2[2].any() and not r2.view(torch.int16).any()
    assert not parts2.any()
    grz.fused_clear(ws)
    grz.zero1_fused_step(grads, big, -1, *s2, args, hyper.max_norm, [r2], parts2, ws)
    three = grz.DDPStep(big, n, master, hyper, device=DEV)
    three.step(grads, 1)
    torch.cuda.synchronize()
    assert not grz.fused_timed_out(ws)
    for k in range(3):
        _same(s2[k], three.state[k], f"after the clear: state {k}")
    _same(r2, three.replica, "after the clear: weights")


def test_fused_sixteen_ranks_equals_three_kernels():
    # The largest N (a runtime-N fold) with two buckets and ragged chunks.
    n = 16
    buckets = [(16 * 300, 16 * 4096 + 16 * 7), (0, 16 * 300)]
    p = 16 * (300 + 4096 + 7)
    master = master_init(p, device=DEV)
    grads = [rank_grad(p, 1e-2, "bf16", grad_seed(4, r), device=DEV) for r in range(n)]
    hyper = grz.Hyper(max_norm=0.05)
    three = grz.DDPStep(buckets, n, master, hyper, device=DEV)
    one = grz.DDPStep(buckets, n, master, hyper, device=DEV, fused=True)
    inp, three_r, one_r = _one_rank_pair(buckets, p, n, 11)
    for t in (1, 2):
        three.step(grads, t)
        one.step(grads, t)
        three_r.step(inp["incoming"], inp["peer_shards"], t)
        one_r.step(inp["incoming"], inp["peer_shards"], t)
        torch.cuda.synchronize()
        for k in range(3):
            _same(one.state[k], three.state[k], f"N=16 DDP t={t} state {k}")
            _same(one_r.state[k], three_r.state[k], f"N=16 rank 11 t={t} state {k}")
        _same(one.replica, three.replica, f"N=16 DDP t={t} weights")
        _same(one_r.arena, three_r.arena, f"N=16 rank 11 t={t} arena")
        _same(one_r.norm.sqnorm, three_r.norm.sqnorm, f"N=16 rank 11 t={t} sqnorm")
    assert three.norm.scale.item() < 1


def test_captured_fused_step_replays_match_eager_fused_steps():
    # The one-launch step captured in a HIP graph: it has no norm launch of its
    # own, so each replay advances the step scalars with grz_step_args_next
    # ahead of the fused launch (GRZ_ARGS_DEVICE); every replay equals the
    # eager fused step of the same number, which equals the three kernels.
    a = arena("char_gpt")
    p, n, rank = a.numel, 8, 2
    inp, three, eager = _one_rank_pair([(0, p)], p, n, rank)
    graphed = grz.Zero1OneRank([(0, p)], n, rank, inp["shard_master"].clone(), device=DEV,
                               arena_numel=p, fused=True)
    graphed.norm.partials.copy_(inp["partials"])
    cap = grz.CapturedStep(lambda args, s: graphed.enqueue(inp["incoming"], inp["peer_shards"],
                                                            args, s), graphed.hyper, 1, 3)
    for t in (1, 2, 3):
        three.step(inp["incoming"], inp["peer_shards"], t)
        eager.step(inp["incoming"], inp["peer_shards"], t)
        cap.replay()
        torch.cuda.synchronize()
        eager.check_fused()
        graphed.check_fused()
        for k in range(3):
            _same(graphed.state[k], eager.state[k], f"replay {t}: state {k}")
            _same(eager.state[k], three.state[k], f"eager fused t={t}: state {k}")
        _same(graphed.arena, eager.arena, f"replay {t}: arena")
        _same(graphed.norm.sqnorm, three.norm.sqnorm, f"replay {t}: sqnorm")
    assert int(cap.counter.item()) == 3
