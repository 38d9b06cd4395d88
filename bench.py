"""Throughput of the ZeRO-1 gradient pipeline on one MI355X.

Default workload: one rank's ZeRO-1 share of a Llama-shaped 7B arena
(6,738,415,616 parameters) at N = 8 -- rank 0 owns chunk 1, 842,301,952
parameters.  One step:

  K1 dp_reduce_scatter_mean  sum the 8 incoming bf16 chunks of the shard in
                             ring order (read from one tiled receive buffer,
                             ``--recv ranks``: 8 tensors), fp32 mean, fp64
                             norm pieces
  K2 dp_grad_sqnorm          global norm over this rank's and the received
                             peers' pieces -> clip factor (device scalar)
  K3 zero1_adamw_gather      clip + AdamW on fp32 master/m/v, bf16 weights
                             written into this rank's full arena
  AG zero1_all_gather        the 7 received peer bf16 shards into the arena

Everything is resident in HBM before timing starts; every input is seeded
and synthetic.  Prints one JSON line.  ``--gpus`` above 1 is refused: the
pipeline runs on one GPU (the ranks are simulated as resident buffers).
Other modes (``--all-ranks``, ``--ddp``, ``--overlap``, ``--zero2``, ``--fused``,
``--graph``, ``--cold``, ``--torch-ref``) are described in their --help lines.
"""

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E peak
COUNTERS = os.path.join(ROOT, "profiles", "llama7b_onerank_step_counters.txt")
KERNEL_SRC = os.path.join(ROOT, "gradient_reduce_zero_amd", "csrc", "grz.hip")
KERNEL_NAMES = {"reduce": "rs_mean_kernel", "adamw": "adamw_kernel", "gather": "gather_kernel"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def settle():
    """Collect once and freeze the objects made so far: a full collection of
    torch's many long-lived objects takes tens of ms and, landing inside a
    timed loop whose steps are host-bound (the small arenas), would be timed
    as GPU time."""
    gc.collect()
    gc.freeze()


def onerank_setup(name, n, rank, device, reduce_flags=0, bucket_plan="default", recv="tiled"):
    import torch  # noqa: F401

    import gradient_reduce_zero_amd as grz
    from workloads import arena, onerank_inputs

    a = arena(name)
    p = a.numel
    if bucket_plan == "25mb" or (bucket_plan == "default" and name == "gpt2_124m"):
        buckets = grz.plan_buckets(a.numels)  # reverse layer order, 25 MiB of gradient
    else:
        buckets = grz.whole_arena(p)
    chunk = grz.owned_chunk(rank, n)
    shard = grz.dp_shard_numel(buckets, n, chunk)
    npieces = grz.dp_piece_count(buckets, n)
    inp = onerank_inputs(shard, n, rank, npieces, grz.GRZ_PIECE, device=device)
    pipe = grz.Zero1OneRank(buckets, n, rank, inp["shard_master"], device=device, arena_numel=p,
                            reduce_flags=reduce_flags)
    pipe.norm.partials.copy_(inp["partials"])
    # What the reduce reads: the N ranks' chunks in one tiled receive buffer,
    # or as N separate tensors.
    inp["recv"] = (grz.tiled_receive(inp["incoming"], buckets, n, chunk) if recv == "tiled"
                   else inp["incoming"])
    return dict(arena=a, p=p, n=n, rank=rank, chunk=chunk, shard=shard, buckets=buckets,
                npieces=npieces, inp=inp, pipe=pipe, recv=recv)


def bytes_per_owned(n, grad_bytes=2):
    """Algorithmic HBM bytes per owned parameter, per kernel of one step."""
    return {
        "reduce": n * grad_bytes + 4,        # N incoming chunks read, fp32 mean written
        "adamw": 4 * 4 + 3 * 4 + 2,          # mean+master+m+v read; master+m+v+bf16 written
        "gather": 2 * (n - 1) * grad_bytes,  # N-1 peer bf16 shards read and written
    }


def kernel_digest():
    """sha256 of the kernel source with comments and white space removed, and of
    the build flags: what decides the compiled kernels."""
    import hashlib
    import re

    from gradient_reduce_zero_amd.build import FLAGS

    src = open(KERNEL_SRC).read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = re.sub(r"\s+", " ", src).strip()
    return hashlib.sha256((src + "\n" + " ".join(FLAGS)).encode()).hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a copy of known size), or None
    when the kernel code has changed since the counters were taken."""
    try:
        text = open(COUNTERS).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if "=" in line:
            k, _, v = line.partition("=")
            vals[k.strip()] = v.strip()
    if vals.get("kernel_code_digest") != kernel_digest() or KERNEL_NAMES[kernel] not in vals:
        return None
    return int(vals[KERNEL_NAMES[kernel]])


def _oracle_onerank(g, w, peers, partials, n, chunk, wire=None, divisor=None):
    """The oracle's one-rank step on host arrays (bf16 bits of the N incoming
    chunks, fp32 master, peers' bf16 shards, peers' norm pieces): fold,
    norm, clip, AdamW from zero moments, bf16 rounding, arena assembly."""
    import math

    import numpy as np

    from oracle.reduce import chunk_mean, widen
    from oracle.step import Hyper, adamw, bf16_round, clip_scale, grad_sqnorm

    npieces = math.ceil(w.size / 4096)
    z = np.zeros_like(w)
    mean = chunk_mean([widen(x, "bf16") for x in g], chunk, wire=wire, divisor=divisor)
    sq = grad_sqnorm(mean, extra=partials[:npieces * (n - 1)])
    scale = clip_scale(sq, 1.0)
    w1, m1, v1 = adamw(w, z, z, mean * scale, **Hyper().scalars(1))
    arena = np.empty((n, w.size), np.uint16)
    arena[chunk] = bf16_round(w1)
    for j, s in enumerate(peers):
        if s is not None:
            arena[(j + 1) % n] = s
    return arena


def cpu_baseline(setup, sample, wire=None, token_counts=None):
    """The CPU oracle on a bounded sample of the same step (reported, not a target)."""
    from workloads import to_bits

    inp = setup["inp"]
    n, shard, chunk = setup["n"], setup["shard"], setup["chunk"]
    lo = (shard // 2) & ~7
    hi = min(shard, lo + sample)
    g = [to_bits(t[lo:hi]) for t in inp["incoming"]]
    w = to_bits(inp["shard_master"][lo:hi])
    peers = [None if s is None else to_bits(s[lo:hi]) for s in inp["peer_shards"]]
    partials = to_bits(inp["partials"])
    divisor = None if token_counts is None else sum(token_counts)
    t0 = time.perf_counter()
    _oracle_onerank(g, w, peers, partials, n, chunk, wire, divisor)
    dt = time.perf_counter() - t0
    return dict(value=(hi - lo) / dt, unit="params/s", cores=1, kind="oracle",
                sample=f"{hi - lo} of the {shard} owned parameters (contiguous, mid-shard): "
                       f"fold of {n} bf16 chunks, float64 norm with the matching share of peer "
                       f"pieces, clip, fp32 AdamW, bf16 rounding, arena assembly; "
                       f"single-threaded NumPy, {dt:.2f} s",
                seconds=dt, count=hi - lo)


def _oracle_worker(i, count, n, rank, chunk, wire, divisor, barrier, results):
    """One worker of the multi-process oracle timing: make a tile of the same
    synthetic inputs (its own seeds), wait for every worker, time the step."""
    try:
        import torch

        torch.set_num_threads(1)
        from workloads import GRAD_SEED, onerank_inputs, to_bits

        npieces = -(-count // 4096) * n
        inp = onerank_inputs(count, n, rank, npieces, 4096, base=GRAD_SEED + 7919 * (i + 1))
        g = [to_bits(t) for t in inp["incoming"]]
        w = to_bits(inp["shard_master"])
        peers = [None if s is None else to_bits(s) for s in inp["peer_shards"]]
        partials = to_bits(inp["partials"])
        del inp
        barrier.wait(timeout=240)
        t0 = time.perf_counter()
        _oracle_onerank(g, w, peers, partials, n, chunk, wire, divisor)
        results.put(("ok", i, count, t0, time.perf_counter()))
    except BaseException as e:  # reported to the parent, which gives up
        barrier.abort()
        results.put(("error", i, repr(e), 0.0, 0.0))


def cpu_baseline_parallel(count, n, rank, chunk, workers, wire=None, divisor=None):
    """The same oracle step over ``count`` parameters split into ``workers``
    disjoint tiles, one forked process each, all started together.  Runs
    before the process touches the GPU (nothing is forked afterwards).
    Throughput = count / (last end - first start), clocks being the system's
    monotonic one."""
    import multiprocessing as mp
    import queue

    ctx = mp.get_context("fork")
    barrier, results = ctx.Barrier(workers), ctx.Queue()
    sizes = [count // workers + (1 if i < count % workers else 0) for i in range(workers)]
    procs = [ctx.Process(target=_oracle_worker,
                         args=(i, sizes[i], n, rank, chunk, wire, divisor, barrier, results),
                         daemon=True) for i in range(workers)]
    for pr in procs:
        pr.start()
    got, ok = [], False
    deadline = time.monotonic() + 300
    try:
        while len(got) < workers:
            try:
                got.append(results.get(timeout=2))
            except queue.Empty:
                dead = [pr.exitcode for pr in procs if pr.exitcode not in (None, 0)]
                if dead or time.monotonic() > deadline:
                    raise RuntimeError("oracle workers " + ("exited with " + str(dead) if dead
                                                            else "timed out"))
        ok = True
    finally:
        for pr in procs:
            if not ok and pr.is_alive():
                pr.kill()  # our own children, by handle
            pr.join(timeout=60)
    bad = [r for r in got if r[0] != "ok"]
    if bad:
        raise RuntimeError(f"oracle worker {bad[0][1]} failed: {bad[0][2]}")
    t0, t1 = min(r[3] for r in got), max(r[4] for r in got)
    return dict(value=count / (t1 - t0), unit="params/s", cores=workers, kind="oracle",
                seconds=t1 - t0,
                sample=f"{count} owned parameters in {workers} tiles of the same synthetic "
                       f"recipe (own seeds), one forked NumPy process per tile, "
                       f"{t1 - t0:.2f} s from the first start to the last end")


def cpu_baseline_all_ranks(grads, buckets, n, hyper, sample):
    """The oracle's ZeRO-1 step of all N ranks on host copies of the same
    gradients: the whole arena when it has at most ``sample`` parameters,
    else its first ``sample`` (a multiple of N) as one bucket."""
    import numpy as np

    from oracle.reduce import shard_segments
    from oracle.step import Hyper, zero1_step
    from workloads import master_init, to_bits

    p = grads[0].numel()
    if p <= sample:
        count, plan = p, [tuple(b) for b in buckets]
    else:
        count = sample - sample % n
        plan = [(0, count)]
    host = [to_bits(g[:count]) for g in grads]
    shard = count // n
    master = to_bits(master_init(count))
    states = []
    for r in range(n):
        w = np.concatenate([master[g0:g0 + ln]
                            for g0, ln, _ in shard_segments(plan, n, (r + 1) % n)])
        states.append((w, np.zeros(shard, np.float32), np.zeros(shard, np.float32)))
    h = Hyper(lr=hyper.lr, warmup=hyper.warmup, max_norm=hyper.max_norm)
    t0 = time.perf_counter()
    zero1_step(host, "bf16", plan, states, h, 1)
    dt = time.perf_counter() - t0
    what = "the whole arena" if count == p else f"the first {count} of {p} parameters"
    return dict(value=count / dt, unit="params/s", cores=1, kind="oracle",
                sample=f"{what}, {len(plan)} bucket(s), all {n} ranks: ring folds, float64 "
                       f"norm, clip, fp32 AdamW of every shard, bf16 all-gather; "
                       f"single-threaded NumPy, {dt:.2f} s")


def overlap_bench(args, dev):
    """Bucket overlap: one JSON line with serial vs overlapped step times."""
    import torch

    import gradient_reduce_zero_amd as grz
    from workloads import arena, master_init

    a = arena("gpt2_124m")
    p, n = a.numel, 8
    buckets = grz.plan_buckets(a.numels)
    d = 768
    log(f"overlap: GPT-2 124M, N={n}, {len(buckets)} buckets")
    master = master_init(p, device=dev)
    pipe = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(), device=dev)
    ov = grz.OverlappedZero1(pipe)
    # The backward of each bucket, per simulated rank: the weight-gradient GEMM
    # (d x T) @ (T x len/d) with T = 1024 tokens, written straight into that
    # rank's gradient arena -- compute-bound, as a real backward is.
    tokens = 1024
    act_t = [torch.randn(d, tokens, device=dev, dtype=torch.bfloat16) * 0.03 for _ in range(n)]
    dout = [[torch.randn(tokens, length // d, device=dev, dtype=torch.bfloat16) * 0.03
             for _, length in buckets] for _ in range(n)]
    grads = [torch.empty(p, dtype=torch.bfloat16, device=dev) for _ in range(n)]

    def produce(b):
        off, length = buckets[b]
        for r in range(n):
            torch.mm(act_t[r], dout[r][b], out=grads[r][off:off + length].view(d, length // d))

    def producer_only(t):
        for b in range(len(buckets)):
            produce(b)

    def serial(t):
        producer_only(t)
        pipe.step(grads, t)

    def overlapped(t):
        for b in range(len(buckets)):
            produce(b)
            ov.bucket_ready(b, grads)
        ov.finish(t)

    def pipeline_only(t):
        pipe.step(grads, t)

    def reduce_only(t):
        for c, mean in zip(pipe.chunks, pipe.means):
            grz.dp_reduce_scatter_mean(grads, buckets, c, mean, pipe.norm.partials)

    def timed(fn):
        settle()
        for t in range(1, args.warmup + 1):
            fn(t)
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for t in range(1, args.steps + 1):
            fn(t)
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    res = {k: timed(f) for k, f in (("producer_ms", producer_only), ("pipeline_ms", pipeline_only),
                                    ("reduce_ms", reduce_only), ("serial_ms", serial),
                                    ("overlapped_ms", overlapped))}
    last = buckets[-1][1] / p  # the last bucket's reduce cannot overlap anything
    hidden = (res["serial_ms"] - res["overlapped_ms"]) / res["reduce_ms"]
    log(", ".join(f"{k} {v:.3f}" for k, v in res.items()) + f"; reduce hidden {hidden:.2f} "
        f"(at most {1 - last:.2f}: the last bucket holds {last:.0%} of the arena)")
    print(json.dumps({"mode": "bucket_overlap", "workload": "gpt2_124m all 8 ranks ZeRO-1",
                      "buckets": len(buckets), "steps": args.steps, **res,
                      "fraction_of_reduce_hidden": hidden,
                      "max_fraction_hideable": 1 - last,
                      "model_params_per_s_overlapped": p / (res["overlapped_ms"] * 1e-3)}),
          flush=True)


def stage_bench(args, dev):
    """ZeRO-1 against ZeRO-2 on GPT-2 124M (all 8 ranks): step time and the
    gradient bytes each keeps resident.  The same synthetic backward feeds both:
    each bucket's gradients are copied in (to the full arenas for ZeRO-1, to
    the one-bucket staging buffers for ZeRO-2)."""
    import torch

    import gradient_reduce_zero_amd as grz
    from workloads import arena, grad_seed, master_init, rank_grad

    a = arena("gpt2_124m")
    p, n = a.numel, 8
    buckets = grz.plan_buckets(a.numels)
    master = master_init(p, device=dev)
    src = [rank_grad(p, 1e-3, "bf16", grad_seed(1, r), device=dev) for r in range(n)]
    z1 = grz.Zero1AllRanks(buckets, n, master, grz.Hyper(), device=dev)
    grads = [torch.empty_like(s) for s in src]
    z2 = grz.Zero2AllRanks(buckets, n, master, grz.Hyper(), device=dev)
    # Every rank at once, each rank's shard at its arena offsets: one reduce
    # (ZeRO-1) or one per bucket (ZeRO-2) and one optimizer launch for all.
    z1a = grz.DDPStep(buckets, n, master, grz.Hyper(), device=dev, nreplicas=n)
    z2a = grz.Zero2AllRanks(buckets, n, master, grz.Hyper(), device=dev, layout="arena")
    # The gradient shards held in bf16 (2 bytes per owned parameter).
    z2b = grz.Zero2AllRanks(buckets, n, master, grz.Hyper(), device=dev, grad_shard="bf16")
    z2ab = grz.Zero2AllRanks(buckets, n, master, grz.Hyper(), device=dev, layout="arena",
                             grad_shard="bf16")

    def copy_in():
        for off, length in buckets:
            for g, s in zip(grads, src):
                g[off:off + length].copy_(s[off:off + length])

    def step1(t):
        copy_in()
        z1.step(grads, t)

    def step1a(t):
        copy_in()
        z1a.step(grads, t)

    def produce(b, bufs):
        off, length = buckets[b]
        for buf, s in zip(bufs, src):
            buf[:length].copy_(s[off:off + length])

    def step2(t):
        z2.step(produce, t)

    def step2a(t):
        z2a.step(produce, t)

    def step2b(t):
        z2b.step(produce, t)

    def step2ab(t):
        z2ab.step(produce, t)

    def timed(fn):
        settle()
        for t in range(1, args.warmup + 1):
            fn(t)
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for t in range(1, args.steps + 1):
            fn(t)
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    t1, t2 = timed(step1), timed(step2)
    t1a, t2a = timed(step1a), timed(step2a)
    t2b, t2ab = timed(step2b), timed(step2ab)
    g1 = sum(g.numel() * g.element_size() for g in grads)
    g2 = sum(b.numel() * b.element_size() for bufs in z2.staging for b in bufs)
    s32 = sum(mu.numel() * mu.element_size() for mu in z2.means)
    s16 = sum(mu.numel() * mu.element_size() for mu in z2b.means)
    log(f"ZeRO-1 {t1:.3f} ms, ZeRO-2 {t2:.3f} ms (ranks shard-compact); ZeRO-1 {t1a:.3f} ms, "
        f"ZeRO-2 {t2a:.3f} ms (ranks in arena layout); gradient bytes resident "
        f"{g1 / 1e6:.0f} MB vs {g2 / 1e6:.0f} MB")
    log(f"ZeRO-2, gradient shards held in bf16: {t2b:.3f} ms (ranks shard-compact), "
        f"{t2ab:.3f} ms (arena layout); the 8 ranks' gradient shards {s16 / 1e6:.0f} MB "
        f"against {s32 / 1e6:.0f} MB in fp32")
    longest = max(l for _, l in buckets)
    print(json.dumps({"mode": "zero2_vs_zero1", "workload": "gpt2_124m all 8 ranks",
                      "buckets": len(buckets), "steps": args.steps, "zero1_ms": t1,
                      "zero2_ms": t2, "zero1_arena_layout_ms": t1a,
                      "zero2_arena_layout_ms": t2a,
                      "zero2_bf16_shard_ms": t2b, "zero2_bf16_shard_arena_layout_ms": t2ab,
                      "zero1_grad_bytes": g1, "zero2_grad_bytes": g2,
                      "zero2_grad_shard_bytes": {"f32": s32, "bf16": s16},
                      "resident_bytes_per_rank": {
                          "zero1": grz.resident_bytes(p, n, 1),
                          "zero2": grz.resident_bytes(p, n, 2, longest_bucket=longest),
                          "zero2_bf16_shard": grz.resident_bytes(p, n, 2, longest_bucket=longest,
                                                                 shard_bytes=2),
                          "zero2_bf16_shard_without_staging": grz.resident_bytes(
                              p, n, 2, shard_bytes=2)}}),
          flush=True)


def all_ranks_bench(args, dev, emit=True):
    """ZeRO-1 step of all N simulated ranks: one JSON line (time, bytes, GB/s),
    also returned as a dict."""
    import torch

    import gradient_reduce_zero_amd as grz
    from workloads import arena, grad_seed, master_init, rank_grad

    a = arena(args.config)
    p, n = a.numel, args.nranks
    buckets = grz.plan_buckets(a.numels) if args.config == "gpt2_124m" else grz.whole_arena(p)
    hyper = grz.Hyper(lr=1e-4, warmup=10) if args.config == "gpt2_1p5b" else grz.Hyper()
    log(f"all ranks: {args.config}, N={n}, {len(buckets)} buckets")
    master = master_init(p, device=dev)
    pipe = grz.Zero1AllRanks(buckets, n, master, hyper, device=dev)
    del master
    grads = [rank_grad(p, 1e-3, "bf16", grad_seed(1, r), device=dev) for r in range(n)]
    torch.cuda.synchronize()
    settle()
    for t in range(1, args.warmup + 1):
        pipe.step(grads, t)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for t in range(args.warmup + 1, args.warmup + args.steps + 1):
        pipe.step(grads, t)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # The same steps again with events between the three phases.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for k, t in enumerate(range(args.warmup + args.steps + 1, args.warmup + 2 * args.steps + 1)):
        ev[k][0].record(s)
        for c, mean in zip(pipe.chunks, pipe.means):
            grz.dp_reduce_scatter_mean(grads, pipe.buckets, c, mean, pipe.norm.partials)
        ev[k][1].record(s)
        pipe.norm.run(pipe.hyper.max_norm, s)
        ev[k][2].record(s)
        args_t = grz.adamw_args(**grz.step_scalars(pipe.hyper, t))
        for c, (w, m, v), mean in zip(pipe.chunks, pipe.state, pipe.means):
            grz.zero1_adamw_gather(w, m, v, mean, pipe.buckets, n, c, pipe.norm.scale, args_t,
                                   pipe.replicas)
        ev[k][3].record(s)
    torch.cuda.synchronize()
    phase = {nm: sum(e[i].elapsed_time(e[i + 1]) for e in ev) / args.steps
             for i, nm in enumerate(("reduce", "sqnorm", "adamw"))}
    pbytes = {"reduce": p * (2 * n + 4), "adamw": p * (16 + 12 + 2 * n)}
    step_bytes = p * (n * 2 + 4 + 28 + 2 * n)  # reduce N*s + mean 4; AdamW 28; N bf16 replicas
    log(f"{ms:.3f} ms/step, {step_bytes / (ms * 1e-3) / 1e9:.0f} GB/s; "
        + ", ".join(f"{k} {v:.3f} ms" for k, v in phase.items()))
    # The same N ranks with their shards held at arena offsets: one reduce and
    # one optimizer launch writing all N replicas (bit-identical per element).
    arena_pipe = grz.DDPStep(buckets, n, master_init(p, device=dev), hyper, device=dev,
                             nreplicas=n)
    for t in range(1, args.warmup + 1):
        arena_pipe.step(grads, t)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(s)
    for t in range(args.warmup + 1, args.warmup + args.steps + 1):
        arena_pipe.step(grads, t)
    a1.record(s)
    torch.cuda.synchronize()
    arena_ms = a0.elapsed_time(a1) / args.steps
    log(f"arena layout (2 launches + norm): {arena_ms:.3f} ms/step")
    out = {"mode": "all_ranks_zero1", "workload": f"{a.name} all {n} ranks",
           "arena_params": p, "buckets": len(buckets), "steps": args.steps,
           "ms_per_step": ms, "step_bytes": step_bytes,
           "achieved_GBps": step_bytes / (ms * 1e-3) / 1e9,
           "model_params_per_s": p / (ms * 1e-3), "phases_ms": phase,
           "phases_GBps": {k: pbytes[k] / (phase[k] * 1e-3) / 1e9 for k in pbytes},
           "arena_layout_ms_per_step": arena_ms,
           "arena_layout_frac_of_peak": step_bytes / (arena_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
           "ms_at_70pct_of_peak": step_bytes / (0.7 * PEAK_HBM_GBPS * 1e9) * 1e3}
    if args.graph:
        first = args.warmup + 2 * args.steps + 1
        cap = grz.CapturedStep(lambda a_, s_: pipe.enqueue(grads, a_, s_), pipe.hyper, first,
                               args.warmup + args.steps)
        for _ in range(args.warmup):
            cap.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(s)
        for _ in range(args.steps):
            cap.replay()
        g1.record(s)
        torch.cuda.synchronize()
        out["graph_ms_per_step"] = g0.elapsed_time(g1) / args.steps
        log(f"graph replay: {out['graph_ms_per_step']:.3f} ms/step")
        # The arena layout captured too: its three launches back to back.
        reps = max(args.steps, 100)
        acap = grz.CapturedStep(lambda a_, s_: arena_pipe.enqueue(grads, a_, s_), hyper,
                                args.warmup + args.steps + 1, args.warmup + reps)
        for _ in range(args.warmup):
            acap.replay()
        torch.cuda.synchronize()
        g0.record(s)
        for _ in range(reps):
            acap.replay()
        g1.record(s)
        torch.cuda.synchronize()
        ams = g0.elapsed_time(g1) / reps
        out["arena_layout_graph_ms_per_step"] = ams
        out["arena_layout_graph_frac_of_peak"] = step_bytes / (ams * 1e-3) / 1e9 / PEAK_HBM_GBPS
        log(f"arena layout as a graph: {ams:.4f} ms/step over {reps} replays")
        # The arena layout as one launch (reduce + norm + clip + AdamW with the
        # bf16 write into all N replicas) where the whole plan fits one.
        npieces = grz.dp_piece_count(buckets, n)
        nl = -(-npieces // 4096) if npieces > 4096 else 0
        fit = grz.zero1_fused_capacity(n, torch.bfloat16) - 4 * (max(nl, 1) - 1)
        if npieces <= fit and len(buckets) * n <= 32:
            fpipe = grz.DDPStep(buckets, n, master_init(p, device=dev), hyper, device=dev,
                                nreplicas=n, fused=True)
            fcap = grz.CapturedStep(lambda a_, s_: fpipe.enqueue(grads, a_, s_), hyper,
                                    args.warmup + args.steps + 1, args.warmup + reps)
            for _ in range(args.warmup):
                fcap.replay()
            torch.cuda.synchronize()
            g0.record(s)
            for _ in range(reps):
                fcap.replay()
            g1.record(s)
            torch.cuda.synchronize()
            fpipe.check_fused()
            fms = g0.elapsed_time(g1) / reps
            fbytes = p * (n * 2 + 28 + 2 * n)  # no mean written or read
            out["arena_layout_one_launch_graph_ms_per_step"] = fms
            out["arena_layout_one_launch_graph_frac_of_peak"] = (
                fbytes / (fms * 1e-3) / 1e9 / PEAK_HBM_GBPS)
            log(f"arena layout as one launch, as a graph: {fms:.4f} ms/step over {reps} replays")
    if not args.no_cpu:
        log("timing the CPU oracle's all-ranks step")
        out["cpu_baseline"] = cpu_baseline_all_ranks(grads, buckets, n, hyper,
                                                     min(args.cpu_sample, 1 << 28))
    if emit:
        print(json.dumps(out), flush=True)
    return out


def torch_reference(args, setup, stream):
    """The same one-rank step written with PyTorch ops on the same resident
    inputs -- the fold as an fp32 copy plus in-place adds in ring order, the
    division, the fp64 norm with the peers' pieces, the clip, fused AdamW, the
    bf16 copy into the arena and the peers' shard copies.  A timing reference
    (the norm is not summed in the library's tree), not part of the product."""
    import torch

    inp, n, c, shard = setup["inp"], setup["n"], setup["chunk"], setup["shard"]
    rows, peers = inp["incoming"], inp["peer_shards"]
    if len(setup["buckets"]) != 1:
        return None  # one whole-arena bucket only: each chunk is one arena range
    arena = torch.zeros(setup["p"], dtype=torch.bfloat16, device=rows[0].device)
    acc = torch.empty(shard, device=rows[0].device)
    peer_sq = inp["partials"].sum()
    param = torch.nn.Parameter(inp["shard_master"].clone())
    opt = torch.optim.AdamW([param], lr=1e-3, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1,
                            fused=True)

    def step():
        acc.copy_(rows[c])
        for j in range(1, n):
            acc.add_(rows[(c + j) % n])
        acc.div_(n)
        sq = torch.linalg.vector_norm(acc, dtype=torch.float64) ** 2 + peer_sq
        scale = torch.clamp(1.0 / torch.sqrt(sq), max=1.0).to(torch.float32)
        param.grad = acc.mul_(scale)
        opt.step()
        arena[c * shard:(c + 1) * shard].copy_(param.detach())
        for j, s in enumerate(peers):
            if s is not None:
                cj = (j + 1) % n
                arena[cj * shard:(cj + 1) * shard].copy_(s)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"the same step in PyTorch ops: {ms:.3f} ms/step")
    return {"ms_per_step": ms, "value": shard / (ms * 1e-3),
            "what": "PyTorch ops: fp32 fold by in-place adds, vector_norm, clip, "
                    "AdamW(fused=True), bf16 and peer copies"}


def ddp_bytes(p, n, grad_bytes=2):
    """Algorithmic HBM bytes of one rank's plain data-parallel step, per phase:
    the reduce of its chunk (N chunks of P/N read, fp32 mean chunk written),
    the peers' fp32 mean chunks copied in (read: simulation only; written),
    and AdamW over the full arena with the bf16 write (30 B per parameter)."""
    peers = 4 * p * (n - 1) // n
    return {"reduce": grad_bytes * p + 4 * p // n, "gather": 2 * peers, "adamw": 30 * p}


def ddp_setup(name, n, rank, device, recv="tiled"):
    """One rank's plain data-parallel step over a workload arena with seeded
    inputs resident: the rank's chunk of every rank's gradient (``recv``: one
    tiled receive buffer, or N tensors), the peers' fp32 mean chunks and the
    peers' norm pieces (standing in for what the collectives deliver)."""
    import gradient_reduce_zero_amd as grz
    from workloads import arena, grad_seed, master_init, onerank_inputs, rank_grad

    a = arena(name)
    p = a.numel
    buckets = grz.plan_buckets(a.numels) if name == "gpt2_124m" else grz.whole_arena(p)
    hyper = grz.Hyper(lr=1e-4, warmup=10) if name == "gpt2_1p5b" else grz.Hyper()
    chunk = grz.owned_chunk(rank, n)
    shard = grz.dp_shard_numel(buckets, n, chunk)
    npieces = grz.dp_piece_count(buckets, n)
    inp = onerank_inputs(shard, n, rank, npieces, grz.GRZ_PIECE, device=device)
    incoming, partials = inp["incoming"], inp["partials"]
    del inp
    one = grz.DDPOneRank(buckets, n, rank, master_init(p, device=device), hyper, device)
    one.norm.partials.copy_(partials)
    peer_means = [None if j == rank else
                  rank_grad(shard, 1e-3 / n ** 0.5, "f32", grad_seed(1, 100 + j), device=device)
                  for j in range(n)]
    return dict(arena=a, p=p, n=n, rank=rank, chunk=chunk, shard=shard, buckets=buckets,
                hyper=hyper, incoming=incoming, partials=partials, one=one,
                peer_means=peer_means,
                recv=(grz.tiled_receive(incoming, buckets, n, chunk) if recv == "tiled"
                      else incoming))


def ddp_bench(args, dev, emit=True):
    """One rank's plain data-parallel (ZeRO stage 0) step: one JSON line, also
    returned as a dict."""
    import torch

    import gradient_reduce_zero_amd as grz

    log(f"DDP one rank: {args.config}, N={args.nranks}")
    d = ddp_setup(args.config, args.nranks, 0, dev, args.recv)
    a, p, n, rank, buckets, hyper = d["arena"], d["p"], d["n"], d["rank"], d["buckets"], d["hyper"]
    incoming, recv, one, peer_means = d["incoming"], d["recv"], d["one"], d["peer_means"]
    log(f"{len(buckets)} buckets")
    torch.cuda.synchronize()
    log(f"inputs resident: P={p}, {torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")
    settle()
    s = torch.cuda.current_stream()
    t = 1
    for _ in range(args.warmup):
        one.step(recv, peer_means, t, s)
        t += 1
    torch.cuda.synchronize()
    names = ("reduce", "gather", "sqnorm", "adamw")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(s)
    for k in range(args.steps):
        e = ev[k]
        e[0].record(s)
        one.reduce(recv, s)
        e[1].record(s)
        one.receive_means(peer_means, s)
        e[2].record(s)
        one.norm.run(one.hyper.max_norm, s)
        e[3].record(s)
        w, m, v = one.state
        grz.zero1_adamw_gather(w, m, v, one.mean, one.buckets, n, -1, one.norm.scale,
                               grz.adamw_args(**grz.step_scalars(one.hyper, t)), [one.arena],
                               stream=s)
        e[4].record(s)
        t += 1
    stop.record(s)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    phase = {nm: sum(e[i].elapsed_time(e[i + 1]) for e in ev) / args.steps
             for i, nm in enumerate(names)}
    pb = ddp_bytes(p, n)
    step_bytes = sum(pb.values())
    simulated = 4 * p * (n - 1) // n
    gbps = {k: pb[k] / (phase[k] * 1e-3) / 1e9 for k in pb}
    log(f"{ms:.3f} ms/step, {step_bytes / (ms * 1e-3) / 1e9:.0f} GB/s; "
        + ", ".join(f"{k} {v:.3f} ms" for k, v in phase.items()))
    out = {"mode": "ddp_one_rank", "workload": f"{a.name} one-rank plain data parallelism",
           "arena_params": p, "nranks_simulated": n, "rank": rank, "buckets": len(buckets),
           "recv_layout": args.recv,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "params_updated_per_s": p / (ms * 1e-3), "step_bytes": step_bytes,
           "achieved_GBps": step_bytes / (ms * 1e-3) / 1e9,
           "pct_of_peak_hbm": 100.0 * step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
           "step_bytes_without_simulated_reads": step_bytes - simulated,
           "ms_at_70pct_of_peak": step_bytes / (0.7 * PEAK_HBM_GBPS * 1e9) * 1e3,
           "phases_ms": phase, "phases_GBps": gbps}
    if args.graph:
        cap = grz.CapturedStep(lambda a_, s_: one.enqueue(recv, peer_means, a_, s_),
                               one.hyper, t, args.warmup + args.steps)
        for _ in range(args.warmup):
            cap.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(s)
        for _ in range(args.steps):
            cap.replay()
        g1.record(s)
        torch.cuda.synchronize()
        out["graph_ms_per_step"] = g0.elapsed_time(g1) / args.steps
        log(f"graph replay: {out['graph_ms_per_step']:.3f} ms/step")
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_ddp(incoming, n, hyper, min(args.cpu_sample, 1 << 27))
    if emit:
        print(json.dumps(out), flush=True)
    return out


def cpu_baseline_ddp(incoming, n, hyper, sample):
    """The oracle's plain data-parallel step (``oracle.step.ddp_step``: the
    all-reduce of every chunk, clip, AdamW over the whole arena) on an arena
    of ``sample`` parameters (a multiple of N) made of the first values of the
    ranks' incoming gradients."""
    import numpy as np

    from oracle.step import Hyper, ddp_step
    from workloads import master_init, to_bits

    count = min(sample, incoming[0].numel())
    count -= count % n
    g = [to_bits(x[:count]) for x in incoming]
    w = to_bits(master_init(count))
    z = np.zeros_like(w)
    h = Hyper(lr=hyper.lr, warmup=hyper.warmup, max_norm=hyper.max_norm)
    t0 = time.perf_counter()
    ddp_step(g, "bf16", [(0, count)], (w, z, z), h, 1)
    dt = time.perf_counter() - t0
    return dict(value=count / dt, unit="params/s", cores=1, kind="oracle",
                sample=f"an arena of {count} parameters (the first values of the {n} ranks' "
                       f"incoming gradients), one bucket: ring folds of every chunk, float64 "
                       f"norm, clip, fp32 AdamW, bf16 rounding; single-threaded NumPy, "
                       f"{dt:.2f} s")


def cold_bench(args, pipe, inp, stream, dev, t, step_bytes):
    """Each step preceded by a 512 MB scrub (outside the timed events)."""
    import torch

    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.warmup + args.steps):
        scrub.fill_(k & 255)
        if k >= args.warmup:
            ev[k - args.warmup][0].record(stream)
        pipe.step(inp["recv"], inp["peer_shards"], t, stream)
        if k >= args.warmup:
            ev[k - args.warmup][1].record(stream)
        t += 1
    torch.cuda.synchronize()
    times = sorted(e[0].elapsed_time(e[1]) for e in ev)
    ms = sum(times) / len(times)
    log(f"cold steps: {ms:.4f} ms/step (median {times[len(times) // 2]:.4f})")
    return {"ms_per_step": ms, "median_ms": times[len(times) // 2],
            "value": pipe.state[0].numel() / (ms * 1e-3),
            "achieved_GBps": step_bytes / (ms * 1e-3) / 1e9}


# The smaller one-rank shares the default run also times, each as the
# workload names it: (arena, simulated ranks).
OTHER_CONFIGS = (("char_gpt", 8), ("gpt2_124m", 8), ("gpt2_1p5b", 4))


def other_configs_bench(args, dev):
    """The char GPT, GPT-2 124M and GPT-2 1.5B one-rank ZeRO-1 shares, each
    step captured once in a HIP graph and replayed: warm (back to back) and
    cold (each replay after a 512 MB write that evicts the Infinity Cache and
    the L2s; the replay alone is timed).  Each against the time 70 % of the
    8 TB/s peak would take for its analytic bytes."""
    import torch

    import gradient_reduce_zero_amd as grz

    stream = torch.cuda.current_stream()
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = {}
    steps = max(args.steps, 100)  # replays of a few µs to ms: time enough of them
    for name, n in OTHER_CONFIGS:
        setup = onerank_setup(name, n, 0, dev)
        pipe, inp = setup["pipe"], setup["inp"]
        owned = setup["shard"]
        step_bytes = owned * sum(bytes_per_owned(n).values())
        count = 2 * (args.warmup + steps)
        cap = grz.CapturedStep(lambda a, s: (pipe.reduce(inp["recv"], s),
                                             pipe.update(None, s, args=a),
                                             pipe.gather(inp["peer_shards"], s)),
                               pipe.hyper, 1, count)
        settle()
        for _ in range(args.warmup):
            cap.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(steps):
            cap.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        warm = g0.elapsed_time(g1) / steps
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for k in range(args.warmup + steps):
            scrub.fill_(k & 255)
            if k >= args.warmup:
                ev[k - args.warmup][0].record(stream)
            cap.replay()
            if k >= args.warmup:
                ev[k - args.warmup][1].record(stream)
        torch.cuda.synchronize()
        cold = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
        target = step_bytes / (0.7 * PEAK_HBM_GBPS * 1e9) * 1e3
        out[name] = {
            "workload": f"{setup['arena'].name} one-rank ZeRO-1 share",
            "arena_params": setup["p"], "owned_params": owned, "nranks_simulated": n,
            "buckets": len(setup["buckets"]), "recv_layout": setup["recv"],
            "step_bytes": step_bytes, "replays": steps,
            "graph_ms_per_step": warm, "cold_graph_ms_per_step": cold,
            "params_per_s": owned / (warm * 1e-3),
            "achieved_GBps": step_bytes / (warm * 1e-3) / 1e9,
            "frac_of_peak": step_bytes / (warm * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "cold_frac_of_peak": step_bytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "ms_at_70pct_of_peak": target,
        }
        log(f"{name} one-rank share as a graph: warm {warm:.4f} ms, cold {cold:.4f} ms "
            f"(70 % of peak: {target:.4f} ms)")
        own_pieces, fcap = fused_fit(setup)
        if own_pieces <= fcap and len(setup["buckets"]) <= 32:
            # The same step as one launch (reduce + norm + clip + AdamW) and the
            # peers' copy, captured and replayed the same way.
            fpipe = grz.Zero1OneRank(setup["buckets"], n, 0, inp["shard_master"].clone(),
                                     device=dev, arena_numel=setup["p"], fused=True)
            fpipe.norm.partials.copy_(inp["partials"])
            fcapt = grz.CapturedStep(lambda a, s: (fpipe.fused_update(inp["incoming"], a, s),
                                                   fpipe.gather(inp["peer_shards"], s)),
                                     fpipe.hyper, 1, count)
            settle()
            for _ in range(args.warmup):
                fcapt.replay()
            torch.cuda.synchronize()
            g0.record(stream)
            for _ in range(steps):
                fcapt.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            fwarm = g0.elapsed_time(g1) / steps
            for k in range(args.warmup + steps):
                scrub.fill_(k & 255)
                if k >= args.warmup:
                    ev[k - args.warmup][0].record(stream)
                fcapt.replay()
                if k >= args.warmup:
                    ev[k - args.warmup][1].record(stream)
            torch.cuda.synchronize()
            fpipe.check_fused()  # raises if a wait of any replay gave up
            fcold = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
            fbytes = owned * (n * 2 + 12 + 14 + bytes_per_owned(n)["gather"])
            out[name].update({
                "fused_graph_ms_per_step": fwarm, "fused_cold_graph_ms_per_step": fcold,
                "fused_step_bytes": fbytes,
                "fused_params_per_s": owned / (fwarm * 1e-3),
                "fused_frac_of_peak": fbytes / (fwarm * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            })
            log(f"{name} one-rank share, one launch + copy as a graph: warm {fwarm:.4f} ms, "
                f"cold {fcold:.4f} ms")
            del fpipe, fcapt
        del setup, pipe, inp, cap
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def other_modes_bench(args, dev):
    """The step in its other modes, as ``--all-ranks`` and ``--ddp`` run them
    (without the CPU oracle): every simulated rank of the char GPT, GPT-2 124M
    (each also as a graph) and GPT-2 1.5B, and one rank's plain data-parallel
    step at GPT-2 124M (also as a graph) and at 7B (10 steps)."""
    import torch

    out = {}
    runs = [("all_ranks", "char_gpt", 8, True), ("all_ranks", "gpt2_124m", 8, True),
            ("all_ranks", "gpt2_1p5b", 4, False), ("ddp_one_rank", "gpt2_124m", 8, True),
            ("ddp_one_rank", "llama_7b", 8, False)]
    for mode, cfg, n, graph in runs:
        sub = argparse.Namespace(**vars(args))
        sub.config, sub.nranks, sub.graph, sub.no_cpu = cfg, n, graph, True
        if cfg == "llama_7b":
            sub.steps, sub.warmup = min(args.steps, 10), min(args.warmup, 2)
        fn = all_ranks_bench if mode == "all_ranks" else ddp_bench
        out[f"{cfg}_{mode}"] = fn(sub, dev, emit=False)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def fused_fit(setup):
    """(own pieces, pieces one launch holds for this plan): the launch's
    resident workgroups hold 4 pieces each, less one folding workgroup per
    4096 pieces of the plan (at least one)."""
    import torch

    import gradient_reduce_zero_amd as grz

    n = setup["n"]
    own = sum(-(-grz.dp_chunk_range(l, n, setup["chunk"])[1] // grz.GRZ_PIECE)
              for _, l in setup["buckets"])
    cap = grz.zero1_fused_capacity(n, torch.bfloat16)  # with one folding workgroup
    nl = -(-setup["npieces"] // 4096) if setup["npieces"] > 4096 else 0
    return own, cap - 4 * (max(nl, 1) - 1)


def fused_bench(args, setup, stream, dev):
    """The same one-rank step with reduce + norm + clip + AdamW as one launch."""
    import torch

    import gradient_reduce_zero_amd as grz

    n, inp = setup["n"], setup["inp"]
    own_pieces, cap = fused_fit(setup)
    if own_pieces > cap or len(setup["buckets"]) > 32:
        log(f"fused step: {own_pieces} pieces do not fit the {cap} one launch holds")
        return {"fits": False, "pieces": own_pieces, "capacity": cap}
    pipe = grz.Zero1OneRank(setup["buckets"], n, setup["rank"], inp["shard_master"].clone(),
                            device=dev, arena_numel=setup["p"], fused=True)
    pipe.norm.partials.copy_(inp["partials"])
    settle()
    t = 1
    for _ in range(args.warmup):
        pipe.step(inp["incoming"], inp["peer_shards"], t, stream)
        t += 1
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(args.steps):
        ev[k][0].record(stream)
        pipe.fused_update(inp["incoming"], grz.adamw_args(**grz.step_scalars(pipe.hyper, t)),
                          stream)
        ev[k][1].record(stream)
        pipe.gather(inp["peer_shards"], stream)
        ev[k][2].record(stream)
        t += 1
    stop.record(stream)
    torch.cuda.synchronize()
    pipe.check_fused()  # raises if a wait of a launch gave up
    ms = start.elapsed_time(stop) / args.steps
    fused_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    gather_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    owned = setup["shard"]
    fused_bpo = n * 2 + 12 + 14  # N bf16 chunks + master/m/v read; master/m/v + bf16 written
    step_bytes = owned * (fused_bpo + bytes_per_owned(n)["gather"])
    log(f"fused step: {ms:.4f} ms/step (fused launch {fused_ms:.4f} ms, gather "
        f"{gather_ms:.4f} ms), {step_bytes / (ms * 1e-3) / 1e9:.0f} GB/s")
    return {"fits": True, "pieces": own_pieces, "capacity": cap, "ms_per_step": ms,
            "value": owned / (ms * 1e-3), "fused_kernel_ms": fused_ms, "gather_ms": gather_ms,
            "bytes_per_owned_param": fused_bpo,
            "fused_kernel_GBps": owned * fused_bpo / (fused_ms * 1e-3) / 1e9,
            "step_GBps": step_bytes / (ms * 1e-3) / 1e9}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama_7b",
                    choices=["llama_7b", "gpt2_1p5b", "gpt2_124m", "char_gpt"])
    ap.add_argument("--nranks", type=int, default=8)
    ap.add_argument("--cpu-sample", type=int, default=1 << 29)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--wire", choices=["fp32", "bf16"], default="fp32",
                    help="precision of the ring's partial sums: fp32 accumulation (default) "
                         "or a bf16 wire that rounds every hop")
    ap.add_argument("--all-ranks", action="store_true",
                    help="instead of one rank's share: the ZeRO-1 step of all N simulated "
                         "ranks of --config (every rank's reduce, AdamW and bf16 write to all "
                         "N replicas)")
    ap.add_argument("--ddp", action="store_true",
                    help="instead of the ZeRO-1 share: one rank's plain data-parallel step "
                         "(its chunk reduced at arena offsets, the peers' fp32 mean chunks "
                         "copied in, clip + AdamW over the full arena)")
    ap.add_argument("--torch-ref", action="store_true",
                    help="also time the same one-rank step written with PyTorch ops "
                         "(fused AdamW) on the same inputs, as a reference")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed")
    ap.add_argument("--token-weighted", action="store_true",
                    help="ranks hold gradient sums over unequal token counts; the reduce "
                         "divides by the global count instead of N")
    ap.add_argument("--zero2", action="store_true",
                    help="instead of the default workload: GPT-2 124M, all 8 simulated ranks, "
                         "ZeRO-1 (full gradient arenas) against ZeRO-2 (one-bucket staging)")
    ap.add_argument("--overlap", action="store_true",
                    help="instead of the default workload: GPT-2 124M, all 8 simulated ranks, "
                         "9 reverse-layer buckets, reduce-scatter overlapped with a synthetic "
                         "backward (a bf16 GEMM per bucket) on a second stream")
    ap.add_argument("--fused", action="store_true",
                    help="also time the one-launch step (zero1_fused_step: reduce, norm, clip "
                         "and AdamW with the mean kept in registers) when the shard fits")
    ap.add_argument("--cold", action="store_true",
                    help="also time each step after a 512 MB write that evicts the 256 MB "
                         "Infinity Cache and the L2s (steps whose bytes fit those caches "
                         "otherwise run warm); the step's kernels alone are timed")
    ap.add_argument("--bucket-plan", choices=["default", "whole", "25mb"], default="default",
                    help="the one-rank share's bucket plan: the workload's own (one bucket "
                         "for the whole arena, GPT-2 124M's nine 25 MiB buckets), the whole "
                         "arena, or reverse-layer buckets of 25 MiB of gradient")
    ap.add_argument("--recv", choices=["tiled", "ranks"], default="tiled",
                    help="how the one-rank share's reduce reads the N ranks' chunks: one "
                         "receive buffer with each piece's N values side by side (the "
                         "default), or N separate shard-compact tensors")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip what the default run times after the headline workload: the "
                         "smaller one-rank shares (char GPT, GPT-2 124M and 1.5B, as graph "
                         "replays, warm and cold), every simulated rank of those three "
                         "arenas, and one rank's plain data-parallel step at GPT-2 124M "
                         "and 7B")
    ap.add_argument("--calibrate", action="store_true",
                    help="first run a plain 2 GiB bf16 copy (the library's all-gather "
                         "kernel with one rank and one replica) as the reference of known "
                         "size for hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the N ranks are "
              "simulated as resident buffers on that GPU, and no multi-GPU run is "
              "implemented", file=sys.stderr)
        sys.exit(2)

    # Unequal token counts (sum 8 * 4096 + 123, not a power of two: the
    # division is a true IEEE division, not a multiply).
    counts = ([4096 + 1000 * (j % 3) - 1000 for j in range(args.nranks)]
              if args.token_weighted else None)
    if counts is not None:
        counts[0] += 123
    wire = "bf16" if args.wire == "bf16" else None

    # The oracle over several processes, forked before this process touches
    # the GPU: the same parameter count as the single-core sample below.
    parallel = None
    if not (args.no_cpu or args.overlap or args.zero2 or args.all_ranks or args.ddp):
        from workloads import arena

        shard = arena(args.config).numel // args.nranks
        count = min(shard - ((shard // 2) & ~7), args.cpu_sample)
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        log(f"timing the CPU oracle on {count} parameters over {workers} processes")
        try:
            parallel = cpu_baseline_parallel(count, args.nranks, 0, 1 % args.nranks, workers,
                                             wire, None if counts is None else sum(counts))
        except Exception as e:  # reported, never fatal: it is a baseline
            log(f"multi-process oracle timing failed: {e}")

    import torch

    import gradient_reduce_zero_amd as grz

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate:
        numel = 1 << 30  # 2 GiB of bf16 read, 2 GiB written
        src = torch.ones(numel, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            grz.zero1_all_gather([src], [(0, numel)], [dst])
        torch.cuda.synchronize()
        assert bool(torch.equal(src, dst))
        log(f"calibration copy: 3 launches of {2 * numel} bytes read + {2 * numel} written")
        del src, dst
    if args.overlap:
        overlap_bench(args, dev)
        return
    if args.zero2:
        stage_bench(args, dev)
        return
    if args.all_ranks:
        all_ranks_bench(args, dev)
        return
    if args.ddp:
        ddp_bench(args, dev)
        return
    log(f"setting up {args.config} one-rank share, N={args.nranks}")
    flags = grz.GRZ_BF16_WIRE if args.wire == "bf16" else 0
    setup = onerank_setup(args.config, args.nranks, 0, dev, reduce_flags=flags,
                          bucket_plan=args.bucket_plan, recv=args.recv)
    pipe, inp = setup["pipe"], setup["inp"]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    settle()
    log(f"inputs resident: P={setup['p']}, owned={setup['shard']}, "
        f"{torch.cuda.memory_allocated() / 1e9:.1f} GB allocated")

    def reduce():
        pipe.reduce(inp["recv"], stream, token_counts=counts)

    t = 1
    for _ in range(args.warmup):
        reduce()
        pipe.update(t, stream)
        pipe.gather(inp["peer_shards"], stream)
        t += 1
    torch.cuda.synchronize()
    log("warmup done")

    names = ("reduce", "sqnorm", "adamw", "gather")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        e = ev[k]
        e[0].record(stream)
        reduce()
        e[1].record(stream)
        pipe.norm.run(pipe.hyper.max_norm, stream)
        e[2].record(stream)
        args_t = grz.adamw_args(**grz.step_scalars(pipe.hyper, t))
        grz.zero1_adamw_gather(*pipe.state, pipe.mean, pipe.buckets, pipe.n, pipe.chunk,
                               pipe.norm.scale, args_t, [pipe.arena], stream=stream)
        e[3].record(stream)
        pipe.gather(inp["peer_shards"], stream)
        e[4].record(stream)
        t += 1
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)
    per = {nm: sum(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)) / args.steps
           for i, nm in enumerate(names)}
    ms = total_ms / args.steps
    per_step = sorted(ev[k][0].elapsed_time(ev[k][len(names)]) for k in range(args.steps))
    median_ms = per_step[len(per_step) // 2]
    log(f"timed {args.steps} steps: {ms:.3f} ms/step (wall {wall:.2f} s); per kernel "
        + ", ".join(f"{k} {v:.3f} ms" for k, v in per.items()))

    owned, n = setup["shard"], setup["n"]
    bpo = bytes_per_owned(n)
    kbytes = {k: owned * v for k, v in bpo.items()}
    step_bytes = sum(kbytes.values())
    gbps = {k: kbytes[k] / (per[k] * 1e-3) / 1e9 for k in kbytes}
    dominant = max(kbytes, key=lambda k: per[k])
    step_gbps = step_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "params updated/sec + achieved HBM GB/s (% of peak), fused reduce+AdamW step",
        "value": owned / (ms * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": median_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{setup['arena'].name} one-rank ZeRO-1 share",
            "arena_params": setup["p"], "owned_params": owned, "nranks_simulated": n,
            "rank": 0, "owned_chunk": setup["chunk"], "buckets": len(setup["buckets"]),
            "grad_dtype": "bf16", "state_dtype": "fp32", "weights_dtype": "bf16",
            "clip": 1.0, "wire": args.wire, "token_counts": counts,
            "recv_layout": setup["recv"],
        },
        "achieved_GBps": step_gbps,
        "pct_of_peak_hbm": 100.0 * step_gbps / PEAK_HBM_GBPS,
        "model_params_per_s": setup["p"] / (ms * 1e-3),
        "step_bytes": step_bytes,
        # The peers' bf16 shards are read only because the ranks are simulated
        # here (on N GPUs they arrive over the links): the step's bytes without
        # those reads, and the rate they give over the same time.
        "step_bytes_without_simulated_reads": step_bytes - owned * (n - 1) * 2,
        "achieved_GBps_without_simulated_reads":
            (step_bytes - owned * (n - 1) * 2) / (ms * 1e-3) / 1e9,
        "kernels_ms": per,
        "kernels_GBps": gbps,
        "roofline": {
            "bound": "hbm",
            "kernel": dominant,
            "achieved": gbps[dominant],
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": gbps[dominant] / PEAK_HBM_GBPS,
            "traffic": measured_traffic(dominant) if args.config == "llama_7b" and n == 8
            else None,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "copy-calibrated; profiles/llama7b_onerank_step_counters.txt)",
            "bytes_per_owned_param": bpo[dominant],
        },
    }
    if args.graph:
        cap = grz.CapturedStep(lambda a, s: (pipe.reduce(inp["recv"], s, token_counts=counts),
                                             pipe.update(None, s, args=a),
                                             pipe.gather(inp["peer_shards"], s)),
                               pipe.hyper, t, args.warmup + args.steps)
        for _ in range(args.warmup):
            cap.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            cap.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        out["graph_ms_per_step"] = g0.elapsed_time(g1) / args.steps
        log(f"graph replay: {out['graph_ms_per_step']:.3f} ms/step")
    if args.cold:
        out["cold"] = cold_bench(args, pipe, inp, stream, dev, t, step_bytes)
    if args.fused:
        out["fused"] = fused_bench(args, setup, stream, dev)
    if args.torch_ref:
        out["torch_reference"] = torch_reference(args, setup, stream)
    if not args.no_cpu:
        log(f"timing the CPU oracle on {args.cpu_sample} parameters")
        cb = cpu_baseline(setup, args.cpu_sample, wire=wire, token_counts=counts)
        out["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        out["cpu_baseline"]["host_cpus"] = os.cpu_count()
        out["cpu_baseline"]["affinity_cpus"] = len(os.sched_getaffinity(0))
        out["cpu_baseline"]["parallel"] = parallel
        # The same analytic bytes per owned parameter as the GPU line, and the
        # time the oracle would take for the whole step at its sampled rate.
        per_param = step_bytes / setup["shard"]
        out["cpu_baseline"]["seconds_per_step"] = setup["shard"] / cb["value"]
        out["cpu_baseline"]["GBps"] = cb["value"] * per_param / 1e9
        if isinstance(parallel, dict) and parallel.get("value"):
            parallel["GBps"] = parallel["value"] * per_param / 1e9
    if not args.no_other_configs and args.config == "llama_7b" and args.nranks == 8 \
            and args.wire == "fp32" and counts is None and args.bucket_plan == "default":
        del setup, pipe, inp
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["other_configs"] = other_configs_bench(args, dev)
        out["other_modes"] = other_modes_bench(args, dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
