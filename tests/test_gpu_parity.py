"""GPU path (C ABI -> HIP kernels) against the CPU oracle, element by element.

Bars: the reduced gradient, ownership and indexing bit-exact; the norm within
1e-13 relative (the GPU sums fixed pieces in a fixed tree, the oracle sums
exactly); fp32 master, m and v within 1e-6 relative after 10 steps (and in
fact bit-exact whenever the clip factor agrees, which it does here); the
bf16 weights bit-exact against the oracle's rounding of the same masters.
"""

import math

import numpy as np
import pytest
import torch

import gradient_reduce_zero_amd as grz
from oracle.reduce import owned_chunk, reduce_scatter_mean, shard_segments
from oracle.ring import ring_all_reduce, ring_reduce_scatter
from oracle.step import Hyper as OHyper
from oracle.step import all_gather, bf16_round, clip_scale, ddp_step, grad_sqnorm, zero1_step
from parity_util import assert_bits, host, max_rel, oracle_states
from workloads import arena, grad_seed, master_init, rank_grad

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# --- the float64 ring check: 64 values at N = 2, 3, 4, 8 ----------------------

@pytest.mark.parametrize("n", [2, 3, 4, 8])
@pytest.mark.parametrize("integer", [False, True])
def test_f64_ring_64_values(n, integer):
    rng = np.random.default_rng(40 + n)
    if integer:
        arrays = [rng.integers(-100, 100, 64).astype(np.float64) for _ in range(n)]
    else:
        arrays = [rng.standard_normal(64) for _ in range(n)]
    grads = [_dev(a) for a in arrays]
    full, _, _ = ring_all_reduce(arrays)
    out = torch.full((64,), float("nan"), dtype=torch.float64, device=DEV)
    grz.dp_reduce_scatter_mean(grads, [(0, 64)], -1, out, flags=grz.GRZ_SUM)
    assert_bits(host(out), full[0], "ring sum (all-reduce)")
    if integer:
        assert_bits(host(out), np.sum(np.stack(arrays), axis=0), "integer sum")
    owned, _ = ring_reduce_scatter(arrays)
    for r in range(n):
        c, vals = owned[r]
        assert c == grz.dp_ring_owned_chunk(r, n)
        shard = torch.empty(vals.size, dtype=torch.float64, device=DEV)
        grz.dp_reduce_scatter_mean(grads, [(0, 64)], c, shard,
                                   flags=grz.GRZ_SUM | grz.GRZ_UNEVEN)
        assert_bits(host(shard), vals, f"owned chunk of rank {r}")
    mean = torch.empty(64, dtype=torch.float64, device=DEV)
    grz.dp_reduce_scatter_mean(grads, [(0, 64)], -1, mean)
    assert_bits(host(mean), reduce_scatter_mean(arrays, "f64", [(0, 64)], -1), "f64 mean")


# --- Tiny: 4096 fp32 parameters, N = 2, 10 steps, ZeRO-1 and DDP --------------

def _tiny_run(max_norm, steps=10, p=4096, n=2, sigma=0.01):
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(max_norm=max_norm)
    ohyper = OHyper(max_norm=max_norm)
    z = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    d = grz.DDPStep(buckets, n, master, hyper, device=DEV)
    states = oracle_states(host(master), buckets, n)
    dstate = (host(master), np.zeros(p, np.float32), np.zeros(p, np.float32))
    for t in range(1, steps + 1):
        grads = [rank_grad(p, sigma, "f32", grad_seed(t, r), device=DEV) for r in range(n)]
        z.step(grads, t)
        d.step(grads, t)
        torch.cuda.synchronize()
        hg = [host(g) for g in grads]
        ref = zero1_step(hg, "f32", buckets, states, ohyper, t)
        dref = ddp_step(hg, "f32", buckets, dstate, ohyper, t)
        states, dstate = ref["states"], dref["state"]
        for r in range(n):
            assert_bits(host(z.means[r]), ref["means"][r], f"t={t} mean of rank {r}")
        assert math.isclose(z.norm.sqnorm.item(), ref["sqnorm"], rel_tol=1e-13)
        assert_bits(host(z.norm.scale), np.array([ref["scale"]], np.float32), f"t={t} scale")
        for r in range(n):
            for k, name in enumerate(("master", "m", "v")):
                got, want = host(z.state[r][k]), ref["states"][r][k]
                assert max_rel(got, want) <= 1e-6, f"t={t} {name} rank {r}"
                assert_bits(got, want, f"t={t} {name} of rank {r}")
        for rep in z.replicas:
            assert_bits(host(rep), ref["arena"], f"t={t} bf16 replica")
        # DDP: same reduced gradient, same norm bits, same weights.
        assert_bits(host(d.mean), dref["mean"], f"t={t} DDP mean")
        assert_bits(host(d.norm.sqnorm), host(z.norm.sqnorm), f"t={t} DDP vs ZeRO-1 sqnorm")
        assert_bits(host(d.replica), host(z.replicas[0]), f"t={t} DDP vs ZeRO-1 weights")
        assert_bits(host(d.state[0]), dref["state"][0], f"t={t} DDP master")
    return z, ref


@pytest.mark.parametrize("max_norm", [1.0, 0.1])
def test_tiny_zero1_and_ddp_10_steps(max_norm):
    z, ref = _tiny_run(max_norm)
    if max_norm == 0.1:
        assert ref["scale"] < 1  # clipping is active in this case
    else:
        assert ref["scale"] == 1


def test_tiny_bf16_weights_are_rne_of_the_masters():
    # bf16 weights bit-exact given matching fp32 masters: the GPU masters equal
    # the oracle's, and each rank's chunk of every replica is the oracle's
    # rounding of them.
    z, ref = _tiny_run(1.0, steps=2)
    for r in range(2):
        assert_bits(host(z.state[r][0]), ref["states"][r][0], "masters match")
        c = grz.dp_ring_owned_chunk(r, 2)
        lo, cnt = grz.dp_chunk_range(4096, 2, c)
        for rep in z.replicas:
            assert_bits(host(rep)[lo:lo + cnt], bf16_round(ref["states"][r][0]), "RNE(master)")


# --- odd shapes: ragged tails, misaligned buckets, runtime N, empty buckets ---

@pytest.mark.parametrize("n,kind,buckets,p", [
    (3, "f32", [(0, 64)], 64),                                   # uneven chunks (DDP)
    (5, "bf16", [(9000, 1003), (4003, 4997), (0, 4003)], 10003),  # odd sizes, misaligned
    (6, "f32", [(0, 6 * 4097 + 5)], 6 * 4097 + 5),                # ragged pieces
    (7, "bf16", [(0, 0), (0, 70007)], 70007),                     # empty bucket, N = 7
    (16, "bf16", [(16 * 8 * 300, 16 * 8 * 300), (0, 16 * 8 * 300)], 16 * 8 * 600),
    (1, "f32", [(0, 12345)], 12345),                              # one rank: identity
    (8, "f64", [(0, 8 * 4096 * 3 + 8 * 5)], 8 * 4096 * 3 + 40),
])
def test_ddp_reduce_odd_shapes(n, kind, buckets, p):
    rng_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f64": torch.float64}[kind]
    grads = [rank_grad(p, 1e-2, kind, grad_seed(3, r), device=DEV) for r in range(n)]
    assert grads[0].dtype == rng_dt
    out_dt = torch.float64 if kind == "f64" else torch.float32
    out = torch.full((p,), float("nan"), dtype=out_dt, device=DEV)
    parts = torch.full((max(grz.dp_piece_count(buckets, n), 1),), -1.0, dtype=torch.float64,
                       device=DEV)
    grz.dp_reduce_scatter_mean(grads, buckets, -1, out, parts)
    hg = [host(g) for g in grads]
    ref = reduce_scatter_mean(hg, kind, buckets, -1, arena_len=p)
    assert_bits(host(out), ref, "DDP mean")
    npieces = grz.dp_piece_count(buckets, n)
    sq = float(np.sum(host(parts)[:npieces]))
    assert math.isclose(sq, grad_sqnorm(ref[~np.isnan(ref)]), rel_tol=1e-12)
    # ZeRO-1 (uneven allowed) per chunk, shard-compact.
    flags = grz.GRZ_UNEVEN
    for c in range(n):
        cnt = grz.dp_shard_numel(buckets, n, c, flags)
        shard = torch.empty(max(cnt, 1), dtype=out_dt, device=DEV)
        grz.dp_reduce_scatter_mean(grads, buckets, c, shard, flags=flags)
        want = reduce_scatter_mean(hg, kind, buckets, c, uneven=True)
        assert_bits(host(shard)[:cnt], want, f"shard of chunk {c}")


@pytest.mark.parametrize("npieces", [1, 3000, 4096, 4097, 8 * 4096, 8 * 4096 + 5, 16 * 4096,
                                     16 * 4096 + 1, 403 * 4096 + 7, 4096 * 4097 + 3])
def test_norm_tree_is_the_fixed_tree_bit_for_bit(npieces):
    # The norm's combine order is a fixed tree that depends only on the piece
    # count: a single final block, or level-by-level launches (one or two
    # levels) and then the final block, give the bits of the tree emulated on
    # the host, and leave the first level's sums in the workspace.
    from parity_util import fixed_tree_sum
    g = torch.Generator(device=DEV).manual_seed(npieces)
    parts = torch.rand(npieces, dtype=torch.float64, device=DEV, generator=g) * 1e-3
    ws = torch.empty(max(grz.dp_grad_sqnorm_workspace(npieces) // 8, 1), dtype=torch.float64,
                     device=DEV)
    sq = torch.zeros(1, dtype=torch.float64, device=DEV)
    sc = torch.zeros(1, dtype=torch.float32, device=DEV)
    max_norm = 0.5
    grz.dp_grad_sqnorm(parts, max_norm, ws, sq, sc)
    torch.cuda.synchronize()
    want = fixed_tree_sum(host(parts))
    assert_bits(host(sq), np.array([want]), f"{npieces} pieces")
    assert math.isclose(want, math.fsum(host(parts).tolist()), rel_tol=1e-13)
    norm = math.sqrt(want)
    factor = np.float32(max_norm / norm) if norm > max_norm else np.float32(1.0)
    assert_bits(host(sc), np.array([factor], np.float32), f"{npieces} pieces: clip factor")
    if npieces > 4096:  # the first level's sums are left in the workspace
        from parity_util import _fan_blocks
        nl = -(-npieces // 4096)
        assert_bits(host(ws)[:nl], _fan_blocks(host(parts)), f"{npieces} pieces: level sums")


@pytest.mark.parametrize("npieces", [3000, 30416])
def test_norm_that_also_advances_the_step_scalars(npieces):
    # dp_grad_sqnorm_step_args, through the C ABI: the norm and clip factor of
    # dp_grad_sqnorm bit for bit, and the work of grz_step_args_next in the
    # same launch (the row at the counter, clamped to the table, copied to
    # `current`; the counter advanced) -- with one tree level and with none.
    import ctypes
    from gradient_reduce_zero_amd import _native as N

    def ptr(t):
        return ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    g = torch.Generator(device=DEV).manual_seed(npieces)
    parts = torch.rand(npieces, dtype=torch.float64, device=DEV, generator=g) * 1e-3
    ws = torch.empty(max(grz.dp_grad_sqnorm_workspace(npieces) // 8, 1), dtype=torch.float64,
                     device=DEV)
    table = torch.arange(3 * 7, dtype=torch.float32, device=DEV) + 0.5
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    current = torch.zeros(7, dtype=torch.float32, device=DEV)
    want_sq = torch.zeros(1, dtype=torch.float64, device=DEV)
    want_sc = torch.zeros(1, dtype=torch.float32, device=DEV)
    assert grz.lib().dp_grad_sqnorm(ptr(parts), npieces, 0.25, ptr(ws), ptr(want_sq),
                                    ptr(want_sc), stream) == N.GRZ_OK
    for step in range(4):  # rows 0, 1, 2, then the last row again
        sq = torch.zeros(1, dtype=torch.float64, device=DEV)
        sc = torch.zeros(1, dtype=torch.float32, device=DEV)
        assert grz.lib().dp_grad_sqnorm_step_args(
            ptr(parts), npieces, 0.25, ptr(ws), ptr(sq), ptr(sc), ptr(table), 3, ptr(counter),
            ptr(current), stream) == N.GRZ_OK
        torch.cuda.synchronize()
        assert_bits(host(sq), host(want_sq), f"step {step}: sqnorm")
        assert_bits(host(sc), host(want_sc), f"step {step}: clip factor")
        assert_bits(host(current), host(table.view(3, 7)[min(step, 2)]), f"step {step}: row")
        assert int(counter.item()) == step + 1
    assert grz.lib().dp_grad_sqnorm_step_args(ptr(parts), npieces, 0.25, ptr(ws), ptr(sq),
                                              ptr(sc), None, 3, ptr(counter), ptr(current),
                                              stream) == N.GRZ_EINVAL


def test_empty_plan_is_a_no_op():
    g = [torch.zeros(8, device=DEV) for _ in range(2)]
    out = torch.full((8,), 3.0, device=DEV)
    grz.dp_reduce_scatter_mean(g, [], -1, out)
    grz.dp_reduce_scatter_mean(g, [(0, 0)], 0, out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    sq = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    sc = torch.zeros(1, device=DEV)
    grz.dp_grad_sqnorm(torch.zeros(1, dtype=torch.float64, device=DEV), 1.0, None, sq, sc,
                       npieces=0)
    torch.cuda.synchronize()
    assert sq.item() == 0.0 and sc.item() == 1.0


# --- invariants: grid width, repeat runs, cross-N on grid-exact data ---------

def test_results_do_not_depend_on_grid_width():
    p, n = 3 * 4096 * 8 + 8 * 77, 8
    buckets = [(4096 * 8, p - 4096 * 8), (0, 4096 * 8)]
    grads = [rank_grad(p, 1e-3, "bf16", grad_seed(9, r), device=DEV) for r in range(n)]
    master = master_init(p, device=DEV)
    outs = []
    # The norm of an fp32 array with more pieces than one tree level holds
    # (4096 * 4096 + 5 elements: 4097 pieces, two levels), and a copy of fp32
    # shards, under the same widths.
    flat = rank_grad(4096 * 4096 + 5, 1e-2, "f32", 77, device=DEV)
    ws = torch.empty(grz.dp_grad_sqnorm_of_workspace(flat.numel()) // 8, dtype=torch.float64,
                     device=DEV)
    try:
        for blocks in (1 << 30, 1, 7, 64):
            grz.grz_set_max_blocks(blocks)
            z = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=0.01), device=DEV)
            z.step(grads, 1)
            z.step(grads, 2)
            sq = torch.zeros(1, dtype=torch.float64, device=DEV)
            grz.dp_grad_sqnorm_of(flat, 1.0, ws, sq, None)
            mean = torch.zeros(p, device=DEV)
            grz.dp_all_gather([m for m in z.means], buckets, [mean])
            torch.cuda.synchronize()
            outs.append((host(z.norm.partials), host(z.replicas[3]),
                         [host(s[0]) for s in z.state], host(ws), host(sq), host(mean)))
    finally:
        grz.grz_set_max_blocks(1 << 30)
    for o in outs[1:]:
        assert_bits(o[0], outs[0][0], "piece sums")
        assert_bits(o[1], outs[0][1], "replica")
        for a, b in zip(o[2], outs[0][2]):
            assert_bits(a, b, "master")
        assert_bits(o[3], outs[0][3], "pieces and level sums of an fp32 array")
        assert_bits(o[4], outs[0][4], "its squared norm")
        assert_bits(o[5], outs[0][5], "fp32 all-gather")


@pytest.mark.parametrize("max_norm", [1e-4, 0.0])
def test_cross_n_identity_grid_exact(max_norm):
    # Values k * 2^-24 with |k| < 2^13: every sum is exact, so the mean, the
    # norm and the weights cannot depend on N -- with the clip active and
    # with it switched off.  The N = 1 run is also the oracle's, bit for bit.
    p, steps = 1 << 16, 3
    rng = np.random.default_rng(21)
    micro = [[(rng.integers(-(1 << 13), 1 << 13, p) * 2.0 ** -24).astype(np.float32)
              for _ in range(8)] for _ in range(steps)]
    master = master_init(p, device=DEV)
    arenas = {}
    for n in (1, 2, 4, 8):
        z = grz.Zero1AllRanks([(0, p)], n, master, grz.Hyper(max_norm=max_norm), device=DEV)
        d = grz.DDPStep([(0, p)], n, master, grz.Hyper(max_norm=max_norm), device=DEV)
        states = oracle_states(host(master), [(0, p)], n)
        for t in range(1, steps + 1):
            per = 8 // n
            hg = [np.sum(np.stack(micro[t - 1][r * per:(r + 1) * per]), axis=0)
                  * np.float32(n / 8) for r in range(n)]
            grads = [_dev(g) for g in hg]
            z.step(grads, t)
            d.step(grads, t)
            if n in (1, 8):
                ref = zero1_step(hg, "f32", [(0, p)], states, OHyper(max_norm=max_norm), t)
                states = ref["states"]
        torch.cuda.synchronize()
        if max_norm > 0:
            assert z.norm.scale.item() < 1
        else:
            assert z.norm.scale.item() == 1.0
        arenas[n] = host(z.replicas[0])
        assert_bits(host(d.replica), arenas[n], f"DDP vs ZeRO-1 at N={n}")
        if n in (1, 8):
            assert_bits(arenas[n], ref["arena"], f"weights at N={n} vs the oracle")
    for n in (2, 4, 8):
        assert_bits(arenas[n], arenas[1], f"weights at N={n} vs N=1")


def test_nan_in_one_rank_propagates_like_the_oracle():
    p, n = 4096, 2
    grads = [rank_grad(p, 0.01, "f32", grad_seed(1, r), device=DEV) for r in range(n)]
    grads[1][100] = float("nan")
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks([(0, p)], n, master, grz.Hyper(max_norm=1.0), device=DEV)
    z.step(grads, 1)
    torch.cuda.synchronize()
    ref = zero1_step([host(g) for g in grads], "f32", [(0, p)],
                     oracle_states(host(master), [(0, p)], n), OHyper(max_norm=1.0), 1)
    assert math.isnan(z.norm.sqnorm.item()) and math.isnan(ref["sqnorm"])
    assert_bits(host(z.norm.scale), np.array([ref["scale"]], np.float32), "scale")
    for r in range(n):
        assert_bits(host(z.state[r][0]), ref["states"][r][0], "master with a NaN")
    # The sign of a NaN produced by arithmetic is not fixed by IEEE 754: compare
    # the NaN element by class and every other element bit for bit.
    got, want = host(z.replicas[0]), ref["arena"]
    nan = (want & 0x7F80) == 0x7F80
    nan &= (want & 0x7F) != 0
    assert nan.sum() == 1 and ((got[nan] & 0x7F80) == 0x7F80).all() and (got[nan] & 0x7F).all()
    assert_bits(got[~nan], want[~nan], "replica with a NaN")


@pytest.mark.parametrize("other", [None, "-inf", "overflow"])
def test_infinite_gradient_clips_like_the_oracle(other):
    # +inf in one rank: the norm is infinite, the clip factor max_norm / inf is
    # 0, finite elements take a zero gradient and the inf element turns NaN.
    # With -inf at the same element of the other rank, the mean itself is NaN
    # and so is the norm: the factor is then 1 (a NaN norm fails the test
    # norm > max_norm), as in the oracle.
    # "overflow": finite 3e38 in both ranks, whose fp32 sum overflows to inf.
    p, n = 4096, 2
    grads = [rank_grad(p, 0.01, "f32", grad_seed(2, r), device=DEV) for r in range(n)]
    if other == "overflow":
        grads[0][100] = grads[1][100] = 3e38
    else:
        grads[1][100] = float("inf")
        if other is not None:
            grads[0][100] = float(other)
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks([(0, p)], n, master, grz.Hyper(max_norm=1.0), device=DEV)
    z.step(grads, 1)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):  # the infinities are the point
        ref = zero1_step([host(g) for g in grads], "f32", [(0, p)],
                         oracle_states(host(master), [(0, p)], n), OHyper(max_norm=1.0), 1)
    sq = z.norm.sqnorm.item()
    assert (math.isnan(sq) and math.isnan(ref["sqnorm"])) if other == "-inf" else (
        math.isinf(sq) and math.isinf(ref["sqnorm"]))
    assert_bits(host(z.norm.scale), np.array([ref["scale"]], np.float32), "scale")
    assert float(ref["scale"]) == (1.0 if other == "-inf" else 0.0)
    for r in range(n):
        assert_bits(host(z.means[r]), ref["means"][r], "mean with an infinity")
        for k in range(3):
            assert_bits(host(z.state[r][k]), ref["states"][r][k], f"state {k} with an infinity")
    got, want = host(z.replicas[0]), ref["arena"]
    nan = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    assert nan.sum() == 1 and ((got[nan] & 0x7F80) == 0x7F80).all() and (got[nan] & 0x7F).all()
    assert_bits(got[~nan], want[~nan], "replica with an infinity")


@pytest.mark.parametrize("case", ["subnormal", "zero"])
def test_subnormal_and_zero_gradients_match_the_oracle(case):
    # Subnormal bf16 gradients (k * 2^-133, |k| < 128, beside a few normal
    # values) must be summed and divided without flushing to zero; all-zero
    # gradients give a zero norm, factor 1 and a pure weight-decay update.
    p, n = 4096 * 2 + 36, 4
    rng = np.random.default_rng(17)
    grads = []
    for r in range(n):
        if case == "zero":
            x = np.zeros(p, np.float32)
        else:
            x = (rng.integers(-127, 128, size=p) * 2.0 ** -133).astype(np.float32)
            x[::97] = rng.standard_normal(x[::97].size).astype(np.float32) * np.float32(1e-30)
        grads.append(torch.from_numpy(x).to(DEV).to(torch.bfloat16))
    hg = [host(g) for g in grads]
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks([(0, p)], n, master, grz.Hyper(max_norm=1.0), device=DEV)
    z.step(grads, 1)
    torch.cuda.synchronize()
    ref = zero1_step(hg, "bf16", [(0, p)], oracle_states(host(master), [(0, p)], n),
                     OHyper(max_norm=1.0), 1)
    if case == "subnormal":
        assert any(np.count_nonzero((m != 0) & (np.abs(m) < np.finfo(np.float32).tiny))
                   for m in ref["means"]), "the case must hold subnormal means"
    else:
        assert ref["sqnorm"] == 0.0 and z.norm.sqnorm.item() == 0.0
    assert math.isclose(z.norm.sqnorm.item(), ref["sqnorm"], rel_tol=1e-13, abs_tol=0.0)
    assert_bits(host(z.norm.scale), np.array([ref["scale"]], np.float32), "scale")
    for r in range(n):
        assert_bits(host(z.means[r]), ref["means"][r], f"{case} mean rank {r}")
        for k in range(3):
            assert_bits(host(z.state[r][k]), ref["states"][r][k], f"{case} state {k} rank {r}")
    assert_bits(host(z.replicas[2]), ref["arena"], f"{case} replica")


def test_bf16_rounding_on_every_upper_half():
    # With lr = 0 and a zero gradient AdamW leaves every finite master as it
    # is, so the kernel's bf16 output is its rounding of chosen fp32 patterns:
    # every finite upper half (sign, exponent, top mantissa bits) with the
    # lower halves that decide round-to-nearest-even (the tie, its
    # neighbours, 0, 1, 0xFFFF) and a random one, against the oracle.
    rng = np.random.default_rng(3)
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = [np.full(1 << 16, low, np.uint32) for low in (0x0000, 0x0001, 0x7FFF, 0x8000,
                                                          0x8001, 0xFFFF)]
    lows.append(rng.integers(0, 1 << 16, size=1 << 16, dtype=np.uint32))
    bits = np.concatenate([hi | low for low in lows])
    bits = bits[(bits & 0x7F800000) != 0x7F800000]  # finite only: 0 * inf is NaN
    x = bits.view(np.float32)
    w = _dev(x.copy())
    zeros = torch.zeros_like(w)
    m, v, g = zeros.clone(), zeros.clone(), zeros.clone()
    out = torch.empty(x.size, dtype=torch.bfloat16, device=DEV)
    args = grz.adamw_args(lr=0.0, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                          bias_corr1=0.1, bias_corr2=0.05)
    grz.zero1_adamw_step(w, m, v, g, None, args, out)
    torch.cuda.synchronize()
    assert_bits(host(w), x, "masters unchanged at lr = 0")
    assert_bits(host(out), bf16_round(x), "bf16 rounding of every upper half")


# --- the unfused optimizer and the standalone all-gather ----------------------

def test_unfused_adamw_and_all_gather_match_fused_and_oracle():
    p, n = 8 * 4096 + 8 * 13, 4
    buckets = [(8 * 4096, 8 * 13), (0, 8 * 4096)]
    grads = [rank_grad(p, 1e-3, "bf16", grad_seed(5, r), device=DEV) for r in range(n)]
    master = master_init(p, device=DEV)
    fused = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=0.02), device=DEV)
    fused.step(grads, 1)
    # Same step with the optimizer writing compact bf16 shards, then all-gather.
    plain = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=0.02), device=DEV)
    for c, mean in zip(plain.chunks, plain.means):
        grz.dp_reduce_scatter_mean(grads, buckets, c, mean, plain.norm.partials)
    plain.norm.run(0.02)
    args = grz.adamw_args(**grz.step_scalars(plain.hyper, 1))
    shards = []
    for (w, m, v), mean in zip(plain.state, plain.means):
        out = torch.empty(w.numel(), dtype=torch.bfloat16, device=DEV)
        grz.zero1_adamw_step(w, m, v, mean, plain.norm.scale, args, out)
        shards.append(out)
    reps = [torch.zeros(p, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    grz.zero1_all_gather(shards, buckets, reps)
    torch.cuda.synchronize()
    ref = zero1_step([host(g) for g in grads], "bf16", buckets,
                     oracle_states(host(master), buckets, n), OHyper(max_norm=0.02), 1)
    for r in range(n):
        assert_bits(host(shards[r]), ref["shards"][r], f"compact bf16 shard of rank {r}")
    for rep in reps:
        assert_bits(host(rep), ref["arena"], "unfused all-gather vs oracle")
        assert_bits(host(rep), host(fused.replicas[0]), "unfused vs fused")


def test_standalone_all_gather_of_synthetic_shards():
    # Shards straight from the seeded generator (not from a GPU step): every
    # replica must hold each rank's shard at its chunks' arena offsets.
    p, n = 4 * (4096 * 2 + 24) + 4 * 8 * 7, 4
    buckets = [(4 * (4096 * 2 + 24), 4 * 8 * 7), (0, 4 * (4096 * 2 + 24))]
    shards = [master_init(grz.dp_shard_numel(buckets, n, (r + 1) % n), seed=300 + r,
                          device=DEV).to(torch.bfloat16) for r in range(n)]
    shards[2] = None  # already in place on its owner: not copied
    reps = [torch.zeros(p, dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    grz.zero1_all_gather(shards, buckets, reps)
    torch.cuda.synchronize()
    want = all_gather([None if s is None else host(s) for s in shards], buckets, n, p)
    for rep in reps:
        assert_bits(host(rep), want, "all-gather")


def test_negative_controls_bite():
    # Planted mistakes, in the oracle: each must disagree with the GPU result.
    p, n = 4096, 4
    grads = [rank_grad(p, 0.01, "f32", grad_seed(2, r), device=DEV) for r in range(n)]
    out = torch.empty(p // n, device=DEV)
    c = grz.dp_ring_owned_chunk(0, n)
    grz.dp_reduce_scatter_mean(grads, [(0, p)], c, out)
    hg = [host(g) for g in grads]
    got = host(out)
    good = reduce_scatter_mean(hg, "f32", [(0, p)], c)
    assert_bits(got, good, "mean")
    summed = reduce_scatter_mean(hg, "f32", [(0, p)], c, average=False)
    assert not np.allclose(got, summed)                       # sum instead of mean
    assert not np.allclose(got, good / n)                      # divided twice
    wrong_chunk = reduce_scatter_mean(hg, "f32", [(0, p)], (c + 1) % n)
    assert not np.allclose(got, wrong_chunk)                   # wrong ownership
    lo, cnt = grz.dp_chunk_range(p, n, c)
    start0 = [a[lo:lo + cnt] for a in hg]
    plain = start0[0].copy()
    for j in range(1, n):
        plain = start0[j] + plain
    assert not np.array_equal(got, plain / np.float32(n))       # fold not in ring order
    # An unordered reduction (what float atomics give): each element's ranks
    # added in an order of their own.
    rng = np.random.default_rng(11)
    order = np.argsort(rng.random((n, cnt)), axis=0)
    vals = np.stack(start0)
    shuffled = vals[order, np.arange(cnt)]
    unordered = shuffled[0].copy()
    for j in range(1, n):
        unordered = shuffled[j] + unordered
    assert not np.array_equal(got, unordered / np.float32(n))


def test_negative_control_shard_offset_without_bucket_offset():
    # "A4", "Common Mistakes": the ZeRO-1 offset is the bucket's (layer's)
    # offset plus the chunk's; dropping the first reads the wrong elements.
    n = 4
    buckets = [(4096, 8192), (0, 4096)]
    p = 12288
    grads = [rank_grad(p, 0.01, "f32", grad_seed(3, r), device=DEV) for r in range(n)]
    c = grz.dp_ring_owned_chunk(1, n)
    out = torch.empty(grz.dp_shard_numel(buckets, n, c), device=DEV)
    grz.dp_reduce_scatter_mean(grads, buckets, c, out)
    hg = [host(g) for g in grads]
    got = host(out)
    assert_bits(got, reduce_scatter_mean(hg, "f32", buckets, c), "shard")
    no_bucket_offset = [(0, length) for _, length in buckets]  # planted in the oracle
    assert not np.array_equal(got, reduce_scatter_mean(hg, "f32", no_bucket_offset, c))


# --- the bf16 wire: every partial sum rounded to bf16 --------------------------

@pytest.mark.parametrize("n", [2, 3, 8, 16])
def test_bf16_wire_mode_matches_oracle(n):
    p = 3 * 4096 * n + 8 * 13 * n
    buckets = [(4096 * n, p - 4096 * n), (0, 4096 * n)]
    grads = [rank_grad(p, 1e-3, "bf16", grad_seed(7, r), device=DEV) for r in range(n)]
    hg = [host(g) for g in grads]
    out = torch.full((p,), float("nan"), device=DEV)
    grz.dp_reduce_scatter_mean(grads, buckets, -1, out, flags=grz.GRZ_BF16_WIRE)
    want = reduce_scatter_mean(hg, "bf16", buckets, -1, arena_len=p, wire="bf16")
    assert_bits(host(out), want, "bf16-wire all-reduce mean")
    plain = reduce_scatter_mean(hg, "bf16", buckets, -1, arena_len=p)
    assert not np.array_equal(host(out), plain)  # the mode is not a no-op
    for c in range(n):
        shard = torch.empty(grz.dp_shard_numel(buckets, n, c), device=DEV)
        grz.dp_reduce_scatter_mean(grads, buckets, c, shard,
                                   flags=grz.GRZ_BF16_WIRE | grz.GRZ_SUM)
        want = reduce_scatter_mean(hg, "bf16", buckets, c, average=False, wire="bf16")
        assert_bits(host(shard), want, f"bf16-wire sum of chunk {c}")
        assert np.all(host(shard).view(np.uint32) & 0xFFFF == 0)  # bf16 values


def test_bf16_wire_zero1_step_matches_oracle():
    p, n = 8 * 4096 * 2, 8
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV,
                          reduce_flags=grz.GRZ_BF16_WIRE)
    states = oracle_states(host(master), buckets, n)
    for t in (1, 2):
        grads = [rank_grad(p, 1e-3, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]
        z.step(grads, t)
        torch.cuda.synchronize()
        ref = zero1_step([host(g) for g in grads], "bf16", buckets, states, OHyper(), t,
                         wire="bf16")
        states = ref["states"]
        for r in range(n):
            assert_bits(host(z.means[r]), ref["means"][r], "wire mean")
            assert_bits(host(z.state[r][0]), ref["states"][r][0], "wire master")
        assert_bits(host(z.replicas[0]), ref["arena"], "wire replica")


def test_bf16_wire_needs_bf16_gradients():
    g = [torch.zeros(64, device=DEV) for _ in range(2)]
    with pytest.raises(grz.GrzError):
        grz.dp_reduce_scatter_mean(g, [(0, 64)], 0, torch.empty(32, device=DEV),
                                   flags=grz.GRZ_BF16_WIRE)


# --- bucket-by-bucket reduction and its overlap with a backward --------------

def test_bucket_range_calls_equal_one_call():
    a = arena("char_gpt")
    p, n = a.numel, 8
    buckets = grz.plan_buckets(a.numels, 1 << 20, 2)  # 1 MiB cap: many buckets
    assert len(buckets) > 5
    grads = [rank_grad(p, 1e-3, "bf16", grad_seed(4, r), device=DEV) for r in range(n)]
    npieces = grz.dp_piece_count(buckets, n)
    for chunk in (-1, 3):
        size = p if chunk < 0 else grz.dp_shard_numel(buckets, n, chunk)
        one = torch.full((size,), float("nan"), device=DEV)
        many = torch.full((size,), float("nan"), device=DEV)
        p1 = torch.full((npieces,), -1.0, dtype=torch.float64, device=DEV)
        p2 = torch.full((npieces,), -1.0, dtype=torch.float64, device=DEV)
        grz.dp_reduce_scatter_mean(grads, buckets, chunk, one, p1)
        for b in reversed(range(len(buckets))):  # any order
            grz.dp_reduce_scatter_mean(grads, buckets, chunk, many, p2, bucket_range=(b, 1))
        assert_bits(host(many), host(one), f"bucket by bucket, chunk {chunk}")
        assert_bits(host(p2), host(p1), f"piece sums, chunk {chunk}")
    with pytest.raises(grz.GrzError):
        grz.dp_reduce_scatter_mean(grads, buckets, 0, many, bucket_range=(len(buckets), 1))


def _check_all_ranks_against_oracle(pipe, ref, what):
    """Every rank's mean, norm, clip factor, master/m/v and every replica of an
    all-ranks step against the oracle's zero1_step."""
    for r in range(pipe.n):
        mean, state = pipe.rank_view(r) if hasattr(pipe, "rank_view") else \
            (pipe.means[r], pipe.state[r])
        want = ref["means"][r]
        if mean.dtype == torch.bfloat16:  # a gradient shard held in bf16
            want = bf16_round(want)
        assert_bits(host(mean), want, f"{what}: mean of rank {r}")
        for k, name in enumerate(("master", "m", "v")):
            assert_bits(host(state[k]), ref["states"][r][k], f"{what}: {name} of rank {r}")
    assert math.isclose(pipe.norm.sqnorm.item(), ref["sqnorm"], rel_tol=1e-13), what
    assert_bits(host(pipe.norm.scale), np.array([ref["scale"]], np.float32), f"{what}: scale")
    for i, rep in enumerate(pipe.replicas):
        assert_bits(host(rep), ref["arena"], f"{what}: replica {i}")


def test_overlapped_step_matches_oracle():
    # Many buckets, each reduced on the communication stream as the backward
    # (a GEMM per bucket on the compute stream, then the bucket's gradient
    # write) produces it, last layer first; norm, clip, AdamW and the
    # all-gather after the last bucket.  Every output against the oracle's
    # ZeRO-1 step over the same plan, bit for bit, over two steps.
    a = arena("char_gpt")
    p, n = a.numel, 4
    buckets = grz.plan_buckets(a.numels, 2 << 20, 2)
    assert len(buckets) > 4
    master = master_init(p, device=DEV)
    ov = grz.OverlappedZero1(grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=0.5),
                                               device=DEV))
    states = oracle_states(host(master), buckets, n)
    x = torch.randn(1024, 1024, device=DEV)
    for t in (1, 2):
        src = [rank_grad(p, 1e-3, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]
        grads = [torch.zeros_like(s) for s in src]
        for b, (off, length) in enumerate(buckets):  # the backward, last layer first
            x = torch.tanh(x @ x.T * 1e-3)            # the bucket's compute
            for g, s in zip(grads, src):
                g[off:off + length].copy_(s[off:off + length])
            ov.bucket_ready(b, grads)
        ov.finish(t)
        torch.cuda.synchronize()
        ref = zero1_step([host(s) for s in src], "bf16", buckets, states, OHyper(max_norm=0.5),
                         t)
        states = ref["states"]
        _check_all_ranks_against_oracle(ov.pipe, ref, f"overlapped t={t}")
    assert ref["scale"] < 1


def test_dropped_wait_reads_gradients_not_yet_written():
    # "A4", "Common Mistakes": without the event wait the reduction can start
    # before the backward has written the gradients.  The compute stream runs
    # milliseconds of GEMMs before it writes them; the ordered step reduces
    # the written values, the one with the wait dropped reduces what was there
    # before (zeros).  When the two streams share a hardware queue (HIP maps
    # streams onto a few queues, so this depends on the streams made before)
    # they run one after the other and the race cannot show: then that half
    # is skipped, not failed; tests/test_overlap_schedule.py checks the
    # ordering itself deterministically.
    n, p = 2, 2 * 4096 * 16
    buckets = [(0, p)]
    src = [rank_grad(p, 1e-2, "bf16", grad_seed(4, r), device=DEV) for r in range(n)]
    want = reduce_scatter_mean([host(s) for s in src], "bf16", buckets, owned_chunk(0, n))
    master = master_init(p, device=DEV)
    x = torch.randn(4096, 4096, device=DEV) / 64

    class NoWait(grz.OverlappedZero1):
        def bucket_ready(self, b, rank_grads, compute_stream=None):
            q = self.pipe
            for c, mean in zip(q.chunks, q.means):  # no record, no wait
                grz.dp_reduce_scatter_mean(rank_grads, q.buckets, c, mean, q.norm.partials,
                                           stream=self.comm, bucket_range=(b, 1))

    def run(cls):
        ov = cls(grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=0.0), device=DEV))
        grads = [torch.zeros_like(s) for s in src]
        torch.cuda.synchronize()
        y = x
        for _ in range(8):  # the backward's compute ahead of the write
            y = y @ x
        for g, s in zip(grads, src):
            g.copy_(s)
        ov.bucket_ready(0, grads)
        ov.finish(1)
        torch.cuda.synchronize()
        return host(ov.pipe.means[0])

    assert_bits(run(grz.OverlappedZero1), want, "with the wait: the written gradients")
    raced = run(NoWait)
    if np.array_equal(raced.view(np.uint32), want.view(np.uint32)):
        pytest.skip("the streams ran in order here: the dropped wait could not show")
    assert np.count_nonzero(raced.view(np.uint32) != want.view(np.uint32)) > 0


@pytest.mark.parametrize("grad_shard", ["f32", "bf16"])
@pytest.mark.parametrize("layout", ["shards", "arena"])
def test_zero2_staged_step_matches_oracle(layout, grad_shard):
    # ZeRO-2 at GPT-2 124M (9 reverse-layer buckets, N = 8): each bucket's
    # gradients arrive in a staging buffer the size of the longest bucket and
    # are reduce-scattered from it at once (GRZ_IN_RANGE); no full gradient
    # arena is kept.  Gradient shards, norm, clip factor, master/m/v and every
    # replica against the oracle's ZeRO-1 step (the update is the same), bit
    # for bit, over two steps -- with the ranks' shards held shard-compact, and
    # at their arena offsets (one reduce launch per bucket for all ranks); the
    # gradient shards held in fp32, and in bf16 ("Lab 09", s.4's 2 bytes per
    # owned parameter: the oracle's step with grad_shard="bf16").
    a = arena("gpt2_124m")
    p, n = a.numel, 8
    buckets = grz.plan_buckets(a.numels)  # 9 buckets, reverse layer order
    master = master_init(p, device=DEV)
    z2 = grz.Zero2AllRanks(buckets, n, master, grz.Hyper(max_norm=1.0), device=DEV,
                           layout=layout, grad_shard=grad_shard)
    shard_t = torch.float32 if grad_shard == "f32" else torch.bfloat16
    assert all(mu.dtype == shard_t for mu in ([z2.mean] if layout == "arena" else z2.means))
    longest = max(length for _, length in buckets)
    assert len(buckets) == 9 and z2.staging[0][0].numel() == longest < p
    states = oracle_states(host(master), buckets, n)
    del master
    for t in (1, 2):
        grads = [rank_grad(p, 1e-3, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]

        def produce(b, bufs):
            off, length = buckets[b]
            for buf, g in zip(bufs, grads):
                buf[:length].copy_(g[off:off + length])
        z2.step(produce, t)
        torch.cuda.synchronize()
        hg = [host(g) for g in grads]
        del grads
        ref = zero1_step(hg, "bf16", buckets, states, OHyper(max_norm=1.0), t,
                         grad_shard=None if grad_shard == "f32" else "bf16")
        del hg
        states = ref["states"]
        _check_all_ranks_against_oracle(z2, ref, f"ZeRO-2 ({grad_shard} shards) t={t}")
    assert ref["scale"] < 1


# --- token-weighted mean for shards of unequal size ---------------------------

def test_token_weighted_reduce_matches_oracle():
    n, p = 5, 3 * 4096 * 5 + 40
    counts = [1000, 2500, 17, 4096, 300]
    buckets = [(4096 * 5, p - 4096 * 5), (0, 4096 * 5)]
    sums = [rank_grad(p, 1e-3 * c, "bf16", grad_seed(8, r), device=DEV)
            for r, c in enumerate(counts)]
    hs = [host(g) for g in sums]
    out = torch.full((p,), float("nan"), device=DEV)
    grz.dp_reduce_scatter_mean(sums, buckets, -1, out, token_counts=counts)
    want = reduce_scatter_mean(hs, "bf16", buckets, -1, arena_len=p, token_counts=counts)
    assert_bits(host(out), want, "token-weighted all-reduce")
    for c in range(n):
        shard = torch.empty(grz.dp_shard_numel(buckets, n, c), device=DEV)
        grz.dp_reduce_scatter_mean(sums, buckets, c, shard, token_counts=counts)
        assert_bits(host(shard), reduce_scatter_mean(hs, "bf16", buckets, c,
                                                     token_counts=counts), f"chunk {c}")
    with pytest.raises(grz.GrzError):
        grz.dp_reduce_scatter_mean(sums, buckets, -1, out, token_counts=[1 << 23] * 5)
    with pytest.raises(grz.GrzError):
        grz.dp_reduce_scatter_mean(sums, buckets, -1, out, token_counts=[0] * 5)
    with pytest.raises(grz.GrzError):
        grz.dp_reduce_scatter_mean(sums, buckets, -1, out, flags=grz.GRZ_SUM,
                                   token_counts=counts)


def test_token_weighted_least_squares_65_rows_on_8_ranks():
    from oracle.lsq import lsq_grad, shard_sum_grads
    rng = np.random.default_rng(81)
    sizes = [9, 8, 8, 8, 8, 8, 8, 8]
    X = rng.integers(-3, 4, size=(65, 32)).astype(np.float64)
    y = rng.integers(-3, 4, size=65).astype(np.float64)
    w = rng.integers(-3, 4, size=32).astype(np.float64)
    sums = [_dev(g) for g in shard_sum_grads(X, y, w, sizes)]
    out = torch.empty(32, dtype=torch.float64, device=DEV)
    grz.dp_reduce_scatter_mean(sums, [(0, 32)], -1, out, token_counts=sizes)
    assert_bits(host(out), lsq_grad(X, y, w), "full-batch gradient")


def test_token_weighted_zero1_step_matches_oracle():
    p, n = 4096 * 4, 4
    counts = [512, 2048, 1024, 100]
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks([(0, p)], n, master, grz.Hyper(max_norm=1.0), device=DEV)
    sums = [rank_grad(p, 1e-3 * c ** 0.5, "f32", grad_seed(1, r), device=DEV)
            for r, c in enumerate(counts)]
    z.step(sums, 1, token_counts=counts)
    torch.cuda.synchronize()
    hs = [host(g) for g in sums]
    states = oracle_states(host(master), [(0, p)], n)
    ref = zero1_step(hs, "f32", [(0, p)], states, OHyper(max_norm=1.0), 1, token_counts=counts)
    for r in range(n):
        assert_bits(host(z.means[r]), ref["means"][r], f"weighted shard of rank {r}")
        assert_bits(host(z.state[r][0]), ref["states"][r][0], f"weighted master of rank {r}")
    assert_bits(host(z.replicas[2]), ref["arena"], "weighted replica")


# --- gates: N = 1 equals a plain optimizer step; checkpoint / resume ---------

def test_single_rank_ddp_equals_plain_adamw():
    # "Distributed training", "Gates": at N = 1 data parallelism is the plain
    # training loop.  One rank's DDP step == the optimizer alone on its gradient.
    p = 4096 * 3 + 100
    master = master_init(p, device=DEV)
    d = grz.DDPStep([(0, p)], 1, master, grz.Hyper(max_norm=0.0), device=DEV)
    w = master.clone()
    m, v = torch.zeros_like(w), torch.zeros_like(w)
    out = torch.empty(p, dtype=torch.bfloat16, device=DEV)
    for t in (1, 2, 3):
        g = rank_grad(p, 1e-2, "f32", grad_seed(t, 0), device=DEV)
        d.step([g], t)
        grz.zero1_adamw_step(w, m, v, g, None, grz.adamw_args(**grz.step_scalars(d.hyper, t)),
                             out)
    torch.cuda.synchronize()
    assert_bits(host(d.state[0]), host(w), "N = 1 DDP master vs plain AdamW")
    assert_bits(host(d.replica), host(out), "N = 1 DDP weights vs plain AdamW")


def test_checkpoint_resume_is_bit_identical():
    # All state is caller-owned tensors plus the step counter: saving them after
    # k steps and resuming gives the uninterrupted run's bits.
    p, n = 8 * 4096 + 64, 4
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(max_norm=0.5)
    grads = [[rank_grad(p, 1e-2, "f32", grad_seed(t, r), device=DEV) for r in range(n)]
             for t in range(1, 6)]
    full = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    for t in range(1, 6):
        full.step(grads[t - 1], t)
    first = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    for t in range(1, 4):
        first.step(grads[t - 1], t)
    torch.cuda.synchronize()
    saved = {"t": 3, "state": [[x.cpu().clone() for x in s] for s in first.state],
             "replicas": [r.cpu().clone() for r in first.replicas]}
    resumed = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    for dst, src in zip(resumed.state, saved["state"]):
        for x, y in zip(dst, src):
            x.copy_(y)
    for dst, src in zip(resumed.replicas, saved["replicas"]):
        dst.copy_(src)
    for t in range(saved["t"] + 1, 6):
        resumed.step(grads[t - 1], t)
    torch.cuda.synchronize()
    for a, b in zip(resumed.state, full.state):
        for x, y in zip(a, b):
            assert_bits(host(x), host(y), "resumed state")
    assert_bits(host(resumed.replicas[0]), host(full.replicas[0]), "resumed weights")


# --- a captured step, replayed ---------------------------------------------------

def test_captured_one_rank_step_replays_match_eager():
    # Graph replays, with eager work and host synchronisations in between, each
    # compared with the eager step of the same number.
    n, rank = 8, 0
    p = 8 * (3 * 4096 + 520)
    buckets = [(0, p)]
    chunk = grz.dp_ring_owned_chunk(rank, n)
    shard = grz.dp_shard_numel(buckets, n, chunk)
    npieces = grz.dp_piece_count(buckets, n)
    from workloads import onerank_inputs
    inp = onerank_inputs(shard, n, rank, npieces, grz.GRZ_PIECE, device=DEV)
    hyper = grz.Hyper(lr=1e-3, warmup=3, max_norm=0.05)
    eager = grz.Zero1OneRank(buckets, n, rank, inp["shard_master"].clone(), hyper, DEV, p)
    graphed = grz.Zero1OneRank(buckets, n, rank, inp["shard_master"].clone(), hyper, DEV, p)
    for z in (eager, graphed):
        z.norm.partials.copy_(inp["partials"])
    cap = grz.CapturedStep(lambda args, s: graphed.enqueue(inp["incoming"], inp["peer_shards"],
                                                            args, s), hyper, 1, 5)
    junk = torch.randn(1 << 20, device=DEV)
    for t in range(1, 6):
        eager.reduce(inp["incoming"])
        eager.update(t)
        eager.gather(inp["peer_shards"])
        cap.replay()
        junk.mul_(0.5).add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        for a, b, what in ((eager.mean, graphed.mean, "mean"), (eager.state[0], graphed.state[0],
                           "master"), (eager.state[2], graphed.state[2], "v"),
                           (eager.arena, graphed.arena, "arena"),
                           (eager.norm.scale, graphed.norm.scale, "scale")):
            assert_bits(host(b), host(a), f"replay {t}: {what}")
    assert int(cap.counter.item()) == 5
    # The table holds steps 1..5: a sixth replay would run with step 5's
    # scalars again, so it is refused before anything is enqueued.
    before = host(graphed.state[0])
    with pytest.raises(RuntimeError, match="5 steps"):
        cap.replay()
    torch.cuda.synchronize()
    assert int(cap.counter.item()) == 5
    assert_bits(host(graphed.state[0]), before, "master after the refused replay")


def test_captured_all_ranks_step_replays_match_eager():
    p, n = 4 * 4096 * 3, 4
    buckets = [(8192, p - 8192), (0, 8192)]
    master = master_init(p, device=DEV)
    grads = [rank_grad(p, 1e-2, "f32", grad_seed(1, r), device=DEV) for r in range(n)]
    eager = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=0.2), device=DEV)
    graphed = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=0.2), device=DEV)
    cap = grz.CapturedStep(lambda args, s: graphed.enqueue(grads, args, s), graphed.hyper, 1, 4)
    for t in range(1, 5):
        eager.step(grads, t)
        cap.replay()
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits(host(graphed.state[r][0]), host(eager.state[r][0]), f"replay {t} master")
        assert_bits(host(graphed.replicas[3]), host(eager.replicas[3]), f"replay {t} replica")


def test_device_step_scalars_advance_once_per_eager_step():
    # Eager steps fed from a device table: each step's StepScalars object
    # advances the row once (the norm's last launch), next() gives the
    # following step's; the same bits as host scalars step by step.
    p, n = 4 * 4096 * 2 + 4 * 40, 4
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(max_norm=0.05, warmup=3)
    host_args = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    dev_args = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    rows = [[s["lr"], s["beta1"], s["beta2"], s["eps"], s["weight_decay"], s["bias_corr1"],
             s["bias_corr2"]] for s in (grz.step_scalars(hyper, t) for t in range(1, 4))]
    sc = grz.StepScalars(torch.tensor(rows, dtype=torch.float32, device=DEV),
                         torch.zeros(1, dtype=torch.int64, device=DEV),
                         torch.zeros(7, dtype=torch.float32, device=DEV))
    for t in range(1, 4):
        grads = [rank_grad(p, 1e-2, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]
        host_args.step(grads, t)
        dev_args.enqueue(grads, sc)
        assert sc.advanced
        sc = sc.next()
        torch.cuda.synchronize()
        assert int(sc.counter.item()) == t
        for r in range(n):
            for j in range(3):
                assert_bits(host(dev_args.state[r][j]), host(host_args.state[r][j]),
                            f"step {t} rank {r} state {j}")


def test_captured_arena_layout_step_replays_match_eager():
    # Every rank in arena layout (DDPStep with N replicas: one reduce, the norm,
    # one optimizer launch) captured once and replayed; each replay against the
    # eager step of the same number, and the eager steps against the oracle.
    p, n = 8 * (4096 + 40) + 8 * 300, 8
    buckets = [(8 * (4096 + 40), 8 * 300), (0, 8 * (4096 + 40))]
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(max_norm=0.05)
    eager = grz.DDPStep(buckets, n, master, hyper, device=DEV, nreplicas=n)
    graphed = grz.DDPStep(buckets, n, master, hyper, device=DEV, nreplicas=n)
    grads = [rank_grad(p, 1e-2, "bf16", grad_seed(1, r), device=DEV) for r in range(n)]
    cap = grz.CapturedStep(lambda args, s: graphed.enqueue(grads, args, s), hyper, 1, 3)
    states = oracle_states(host(master), buckets, n)
    for t in range(1, 4):
        eager.step(grads, t)
        cap.replay()
        torch.cuda.synchronize()
        ref = zero1_step([host(g) for g in grads], "bf16", buckets, states, OHyper(max_norm=0.05),
                         t)
        states = ref["states"]
        for j in range(3):
            assert_bits(host(graphed.state[j]), host(eager.state[j]), f"replay {t} state {j}")
        for r in (0, 5):
            assert_bits(host(graphed.replicas[r]), host(eager.replicas[r]), f"replay {t} rep {r}")
        assert_bits(host(eager.replicas[7]), ref["arena"], f"step {t} arena vs oracle")
        w = host(eager.state[0])
        for r in range(n):
            segs = shard_segments(buckets, n, owned_chunk(r, n))
            mine = np.concatenate([w[g:g + length] for g, length, _ in segs])
            assert_bits(mine, ref["states"][r][0], f"step {t} rank {r} master vs oracle")


def test_zero1_state_placed_at_each_arena_phase_matches_oracle():
    # Chunks of the long bucket land d = 24, 28, 0, 4 elements past a
    # 32-element arena boundary (shard offset 8, chunk length 8196): each
    # rank's state sits at that phase of its lines, so the optimizer's head
    # brings its bf16 stores and its fp32 streams onto whole blocks together.
    n = 4
    buckets = [(0, 4 * 8), (4 * 8, 4 * 8196)]
    p = 4 * 8 + 4 * 8196
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=0.05), device=DEV)
    phases = [grz.state_phase(buckets, n, c) for c in z.chunks]
    assert phases == [28, 0, 4, 24]  # chunks 1, 2, 3, 0
    for ph, (w, m, v), mean in zip(phases, z.state, z.means):
        assert all((x.data_ptr() // 4) % 32 == ph for x in (w, m, v, mean))
    states = oracle_states(host(master), buckets, n)
    for t in (1, 2):
        grads = [rank_grad(p, 1e-2, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]
        z.step(grads, t)
        torch.cuda.synchronize()
        ref = zero1_step([host(g) for g in grads], "bf16", buckets, states, OHyper(max_norm=0.05),
                         t)
        states = ref["states"]
        assert ref["scale"] < 1
        for r in range(n):
            assert_bits(host(z.means[r]), ref["means"][r], f"phase test mean rank {r}")
            for j in range(3):
                assert_bits(host(z.state[r][j]), ref["states"][r][j],
                            f"phase test state {j} rank {r}")
        for r in range(n):
            assert_bits(host(z.replicas[r]), ref["arena"], f"phase test replica {r}")


def test_sixteen_ranks_zero1_step_matches_oracle():
    # The largest N the library takes, with two buckets and a ragged tail.
    p, n = 16 * (4096 + 40) + 16 * 8 * 100, 16
    buckets = [(16 * (4096 + 40), 16 * 8 * 100), (0, 16 * (4096 + 40))]
    master = master_init(p, device=DEV)
    z = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(max_norm=0.05), device=DEV)
    states = oracle_states(host(master), buckets, n)
    for t in (1, 2):
        grads = [rank_grad(p, 1e-2, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]
        z.step(grads, t)
        torch.cuda.synchronize()
        ref = zero1_step([host(g) for g in grads], "bf16", buckets, states, OHyper(max_norm=0.05),
                         t)
        states = ref["states"]
        assert ref["scale"] < 1
        for r in (0, 7, 15):
            assert_bits(host(z.means[r]), ref["means"][r], f"N=16 mean rank {r}")
            assert_bits(host(z.state[r][0]), ref["states"][r][0], f"N=16 master rank {r}")
        assert_bits(host(z.replicas[11]), ref["arena"], "N=16 replica")


# --- dp_grad_sqnorm_of: the norm straight from an fp32 gradient array ---------

@pytest.mark.parametrize("n,offset", [(1, 0), (4095, 0), (4096, 0), (4097, 1),
                                      (3 * 4096 + 5, 0), (3 * 4096 + 5, 3),
                                      (4096 * 4096 + 77, 0)])
def test_grad_sqnorm_of_equals_reduce_path_and_oracle(n, offset):
    gen = torch.Generator(device=DEV).manual_seed(900 + n)
    buf = torch.randn(n + offset, generator=gen, device=DEV) * 1e-3
    g = buf[offset:]  # offset 1 or 3 leaves the base 4 or 12 bytes past a 16-byte line
    max_norm = 0.5 * math.sqrt(n) * 1e-3  # clips
    ws = torch.empty(grz.dp_grad_sqnorm_of_workspace(n), dtype=torch.uint8, device=DEV)
    sq, sc = (torch.empty(1, dtype=torch.float64, device=DEV),
              torch.empty(1, dtype=torch.float32, device=DEV))
    grz.dp_grad_sqnorm_of(g, max_norm, ws, sq, sc)
    # The same pieces and tree as reducing one rank's single-bucket arena.
    mean = torch.empty(n, dtype=torch.float32, device=DEV)
    parts = torch.empty(grz.dp_piece_count([(0, n)], 1), dtype=torch.float64, device=DEV)
    grz.dp_reduce_scatter_mean([g.clone()], [(0, n)], -1, mean, parts)
    sq2, sc2 = torch.empty_like(sq), torch.empty_like(sc)
    wsn = torch.empty(max(grz.dp_grad_sqnorm_workspace(parts.numel()), 8), dtype=torch.uint8,
                      device=DEV)
    grz.dp_grad_sqnorm(parts, max_norm, wsn, sq2, sc2)
    torch.cuda.synchronize()
    assert_bits(host(sq), host(sq2), "sqnorm: array vs reduce path")
    assert_bits(host(sc), host(sc2), "clip factor: array vs reduce path")
    assert_bits(host(ws.view(torch.float64)[:parts.numel()]), host(parts), "piece sums")
    want = grad_sqnorm(host(g))
    assert math.isclose(sq.item(), want, rel_tol=1e-13)
    assert abs(sc.item() - clip_scale(want, max_norm)) <= 2 ** -23 * abs(sc.item())


def test_grad_sqnorm_of_errors():
    g = torch.zeros(10, device=DEV)
    sq = torch.empty(1, dtype=torch.float64, device=DEV)
    with pytest.raises(ValueError):
        grz.dp_grad_sqnorm_of(g, 1.0, None, sq, None)
    ws = torch.empty(grz.dp_grad_sqnorm_of_workspace(10), dtype=torch.uint8, device=DEV)
    with pytest.raises(grz.GrzError):
        grz.dp_grad_sqnorm_of(g, 1.0, ws, None, None)
    grz.dp_grad_sqnorm_of(g, 1.0, ws, sq, None)
    assert sq.item() == 0.0


# --- the one-rank share is one rank of the whole job -------------------------

def test_one_rank_share_equals_that_rank_of_the_all_ranks_step():
    # Rank r's share fed what the other ranks of the same job deliver -- the
    # chunk of every rank's gradient, every rank's norm pieces and the peers'
    # new bf16 shards -- reproduces rank r of the all-ranks step bit for bit.
    n, p = 8, 8 * (3 * 4096 + 136)
    buckets = [(8 * 4096, p - 8 * 4096), (0, 8 * 4096)]
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(max_norm=0.5)
    full = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    grads = [rank_grad(p, 1e-2, "bf16", grad_seed(5, r), device=DEV) for r in range(n)]
    full.step(grads, 1)
    torch.cuda.synchronize()
    assert full.norm.scale.item() < 1
    for r in (0, 5):
        c = grz.dp_ring_owned_chunk(r, n)
        idx = torch.cat([torch.arange(o + grz.dp_chunk_range(l, n, c)[0],
                                      o + sum(grz.dp_chunk_range(l, n, c)), device=DEV)
                         for o, l in buckets])
        incoming = [g.index_select(0, idx).contiguous() for g in grads]
        one = grz.Zero1OneRank(buckets, n, r, master.index_select(0, idx), hyper, DEV, p)
        one.norm.partials.copy_(full.norm.partials)  # every rank's pieces, as received
        peers = []
        for j in range(n):
            cj = grz.dp_ring_owned_chunk(j, n)
            ij = torch.cat([torch.arange(o + grz.dp_chunk_range(l, n, cj)[0],
                                         o + sum(grz.dp_chunk_range(l, n, cj)), device=DEV)
                            for o, l in buckets])
            peers.append(None if j == r else full.replicas[0].index_select(0, ij).contiguous())
        one.step(incoming, peers, 1)
        torch.cuda.synchronize()
        assert_bits(host(one.mean), host(full.means[r]), f"rank {r} mean")
        assert_bits(host(one.norm.sqnorm), host(full.norm.sqnorm), f"rank {r} sqnorm")
        for k in range(3):
            assert_bits(host(one.state[k]), host(full.state[r][k]), f"rank {r} state {k}")
        assert_bits(host(one.arena), host(full.replicas[r]), f"rank {r} bf16 arena")


def test_two_ranks_every_strategy_gives_the_same_weights():
    # The noeira "Gates" at N = 2: data parallelism, ZeRO-1, ZeRO-2 and the
    # one-launch forms give the same weights -- here bit for bit even with the
    # clip on, since every strategy sums the same norm pieces in the same tree.
    n, p = 2, 2 * (2 * 4096 + 96)
    buckets = [(2 * 4096, p - 2 * 4096), (0, 2 * 4096)]
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(max_norm=0.05)
    ddp = grz.DDPStep(buckets, n, master, hyper, device=DEV)
    ddp_fused = grz.DDPStep(buckets, n, master, hyper, device=DEV, fused=True)
    z1 = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    z2 = grz.Zero2AllRanks(buckets, n, master, hyper, device=DEV)
    z2a = grz.Zero2AllRanks(buckets, n, master, hyper, device=DEV, layout="arena")
    for t in (1, 2, 3):
        grads = [rank_grad(p, 1e-2, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]
        ddp.step(grads, t)
        ddp_fused.step(grads, t)
        z1.step(grads, t)

        def produce(b, bufs):
            off, length = buckets[b]
            for buf, g in zip(bufs, grads):
                buf[:length].copy_(g[off:off + length])
        z2.step(produce, t)
        z2a.step(produce, t)
        torch.cuda.synchronize()
        want = host(ddp.replica)
        for what, rep in (("fused DDP", ddp_fused.replica), ("ZeRO-1", z1.replicas[0]),
                          ("ZeRO-1 rank 1", z1.replicas[1]), ("ZeRO-2", z2.replicas[1]),
                          ("ZeRO-2 in arena layout", z2a.replicas[1])):
            assert_bits(host(rep), want, f"t={t} {what} weights")
        for what, sq in (("fused DDP", ddp_fused.norm.sqnorm), ("ZeRO-1", z1.norm.sqnorm),
                         ("ZeRO-2", z2.norm.sqnorm), ("ZeRO-2 in arena layout", z2a.norm.sqnorm)):
            assert_bits(host(sq), host(ddp.norm.sqnorm), f"t={t} {what} sqnorm")
    assert ddp.norm.scale.item() < 1


@pytest.mark.parametrize("max_norm", [0.0, -1.0])
def test_clipping_switched_off(max_norm):
    # max_norm <= 0 disables the clip: factor exactly 1, the step the oracle
    # takes without clipping, although the norm here is far above 1.
    p, n = 4 * 4096 + 12, 4
    buckets = [(0, p)]
    master = master_init(p, device=DEV)
    d = grz.DDPStep(buckets, n, master, grz.Hyper(max_norm=max_norm), device=DEV)
    grads = [rank_grad(p, 1.0, "f32", grad_seed(1, r), device=DEV) for r in range(n)]
    d.step(grads, 1)
    torch.cuda.synchronize()
    dstate = (host(master), np.zeros(p, np.float32), np.zeros(p, np.float32))
    ref = ddp_step([host(g) for g in grads], "f32", buckets, dstate, OHyper(max_norm=max_norm), 1)
    assert ref["sqnorm"] > 1 and ref["scale"] == 1
    assert_bits(host(d.norm.scale), np.array([1.0], np.float32), "clip factor")
    assert math.isclose(d.norm.sqnorm.item(), ref["sqnorm"], rel_tol=1e-13)
    for k in range(3):
        assert_bits(host(d.state[k]), ref["state"][k], f"state {k}")
    assert_bits(host(d.replica), ref["arena"], "weights")


def test_all_ranks_in_arena_layout_equal_the_shard_compact_ranks():
    # Every simulated rank's ZeRO-1 step at once as one data-parallel step
    # writing all N replicas: each rank's master, m and v, read at its arena
    # offsets, equal the shard-compact ranks' bit for bit.
    n, p = 4, 4 * (2 * 4096 + 20)
    buckets = [(4 * 4096, p - 4 * 4096), (0, 4 * 4096)]
    master = master_init(p, device=DEV)
    hyper = grz.Hyper(max_norm=0.1)
    z = grz.Zero1AllRanks(buckets, n, master, hyper, device=DEV)
    d = grz.DDPStep(buckets, n, master, hyper, device=DEV, nreplicas=n)
    for t in (1, 2):
        grads = [rank_grad(p, 1e-2, "bf16", grad_seed(t, r), device=DEV) for r in range(n)]
        z.step(grads, t)
        d.step(grads, t)
    torch.cuda.synchronize()
    for r in range(n):
        c = grz.dp_ring_owned_chunk(r, n)
        idx = torch.cat([torch.arange(o + grz.dp_chunk_range(l, n, c)[0],
                                      o + sum(grz.dp_chunk_range(l, n, c)), device=DEV)
                         for o, l in buckets])
        for k in range(3):
            assert_bits(host(d.state[k].index_select(0, idx)), host(z.state[r][k]),
                        f"rank {r} state {k}")
        assert_bits(host(d.replicas[r]), host(z.replicas[r]), f"replica {r}")
