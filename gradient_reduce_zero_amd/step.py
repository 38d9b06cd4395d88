"""One training step of the gradient pipeline, driven through the C ABI.

Views of the same step, all on one GPU with the ranks simulated as
resident buffers ("Distributed training" (noeira), "The process group": the
simulator runs every rank on one device with the collectives as local
kernels):

* ``Zero1AllRanks`` -- all N ranks of a ZeRO-1 step: each rank reduces the
  chunk it owns, the norm is taken over every rank's pieces, each rank runs
  AdamW on its shard and writes the new bf16 weights into all N replicas.
* ``DDPStep``       -- plain data parallelism (ZeRO stage 0) as one replica
  sees it: all-reduce-mean of every chunk, norm, AdamW over the whole arena,
  bf16 weights into the replica.  Every replica runs the same computation.
* ``Zero1OneRank``  -- what a single GPU of an N-GPU ZeRO-1 job does: sum the
  N incoming chunks of its shard, combine its norm pieces with the peers'
  (received), AdamW on its shard, then assemble its full bf16 arena from its
  own shard and the peers' received shards.
* ``DDPOneRank``    -- a single GPU of an N-GPU plain data-parallel job: the
  all-reduce of the mean as reduce-scatter (its chunk, at arena offsets) plus
  all-gather (the peers' mean chunks), then AdamW over its whole copy.
  ``one_rank_step`` picks this or ``Zero1OneRank`` from the plan.

``Zero1OneRank`` and ``DDPStep`` take ``fused=True`` to run reduce, norm,
clip and AdamW as one launch (``zero1_fused_step``) when the shard fits.

The step order is "A4 -- Multi-GPU with NCCL and ZeRO-1", "Part 4":
reduce-scatter, AdamW on the shard, all-gather; with the clip in between as in
"Distributed training", "Four strategies, one interface".  The host only
enqueues kernels and fills the per-step scalars; there is no host
synchronisation inside a step.
"""

import sys

import torch

from . import binding as B
from ._native import GRZ_IN_COMPACT, GRZ_IN_RANGE, GRZ_OUT_GLOBAL, GRZ_PIECE, GRZ_UNEVEN
from .plan import Hyper, owned_chunk, step_scalars, zero_stage


def _shard_index(buckets, nranks, chunk, device):
    """Arena indices of the shard of ``chunk``, in shard-compact order (setup only)."""
    parts = []
    for b, (off, length) in enumerate(buckets):
        lo, cnt = B.dp_chunk_range(length, nranks, chunk)
        parts.append(torch.arange(off + lo, off + lo + cnt, device=device, dtype=torch.int64))
    return torch.cat(parts) if parts else torch.empty(0, dtype=torch.int64, device=device)


def state_phase(buckets, nranks, chunk):
    """Element offset, modulo 32, at which the fp32 shard arrays of ``chunk``
    (master, m, v, mean) are placed on their 128-byte lines.

    Shard element j of bucket b lands at arena element j + d_b.  The optimizer
    splits off a short head so that its bf16 stores into the arena cover whole
    64-byte blocks; with the fp32 arrays at phase d_b mod 32 the same head also
    brings their reads onto whole 128-byte lines.  (GPT-2 1.5B at N = 4, chunk
    1, d = 16: the optimizer 1.97-2.07 ms at phase 0 against 1.87-1.89 ms at
    phase 16 on MI355X.)  Of the buckets' d_b mod 32 the one covering the most
    owned elements is taken, and only a multiple of 4, so that the arrays keep
    the 16-byte alignment of the kernels' vector accesses; 0 for the DDP
    layout (``chunk`` -1), whose arrays are arena-indexed."""
    if chunk < 0:
        return 0
    cover, shard = {}, 0
    for off, length in buckets:
        lo, cnt = B.dp_chunk_range(length, nranks, chunk)
        d = (off + lo - shard) % 32
        cover[d] = cover.get(d, 0) + cnt
        shard += cnt
    best = max(sorted(cover), key=lambda d: cover[d], default=0)
    return best if best % 4 == 0 else 0


def placed_zeros(numel, phase, device, dtype=torch.float32):
    """Zeroed array of ``numel`` whose element 0 sits ``phase`` elements (mod 32)
    past a 128-byte boundary (a view into an allocation 32 elements longer)."""
    buf = torch.zeros(numel + 32, dtype=dtype, device=device)
    esz = buf.element_size()
    off = (phase - buf.data_ptr() // esz) % 32 if buf.data_ptr() % esz == 0 else 0
    return buf[off:off + numel]


def _shard_state(src, phase, with_mean=True):
    """(master, m, v) and the mean buffer (None without ``with_mean``) of one
    shard, placed at ``phase``; the master a copy of ``src``."""
    n, dev = src.numel(), src.device
    w = placed_zeros(n, phase, dev)
    w.copy_(src)
    state = (w, placed_zeros(n, phase, dev), placed_zeros(n, phase, dev))
    return state, (placed_zeros(n, phase, dev) if with_mean else None)


def tiled_receive(incoming, buckets, nranks, chunk):
    """The ranks' shard-compact values of chunk ``chunk`` (``incoming[j]``, rank
    j's) laid out as one ``GRZ_IN_TILED`` receive buffer: piece k of the chunk
    (in plan order) in slot k, its N ranks' values side by side.  Device
    copies only; on N GPUs each peer writes its pieces into the owner's slots
    itself, here the simulation packs them once."""
    buckets = [(int(o), int(l)) for o, l in buckets]
    n = nranks
    flags = GRZ_UNEVEN if any(length % n for _, length in buckets) else 0
    x0 = incoming[0]
    buf = torch.zeros(B.dp_tiled_numel(buckets, n, chunk, flags), dtype=x0.dtype,
                      device=x0.device)
    slots = buf.view(-1, n, GRZ_PIECE)
    comp = piece = 0
    for _, length in buckets:
        _, cnt = B.dp_chunk_range(length, n, chunk)
        full, tail = divmod(cnt, GRZ_PIECE)
        for j, x in enumerate(incoming):
            if full:
                slots[piece:piece + full, j].copy_(x[comp:comp + full * GRZ_PIECE]
                                                   .view(full, GRZ_PIECE))
            if tail:
                slots[piece + full, j, :tail].copy_(x[comp + full * GRZ_PIECE:comp + cnt])
        comp += cnt
        piece += -(-cnt // GRZ_PIECE)
    return B.Tiled(buf, n)


class _Norm:
    """Piece sums, workspace and the two device scalars of the clip."""

    def __init__(self, npieces, device):
        self.npieces = npieces
        self.partials = torch.zeros(max(npieces, 1), dtype=torch.float64, device=device)
        ws = B.dp_grad_sqnorm_workspace(npieces)
        self.workspace = torch.empty(max(ws // 8, 1), dtype=torch.float64, device=device)
        self.sqnorm = torch.zeros(1, dtype=torch.float64, device=device)
        self.scale = torch.ones(1, dtype=torch.float32, device=device)

    def run(self, max_norm, stream=None, args=None):
        """The norm and the clip factor; ``args`` (the step's scalars, as handed to
        an ``enqueue``) are advanced in the same launch when they are a
        captured step's ``StepScalars``."""
        B.dp_grad_sqnorm(self.partials, max_norm, self.workspace, self.sqnorm, self.scale,
                         npieces=self.npieces, stream=stream,
                         step_args=args if isinstance(args, B.StepScalars) else None)


def _fused_workspace(npieces, device):
    """Zeroed workspace of the one-launch step (control words and the slots
    its workgroups publish the norm's sums in)."""
    return torch.zeros(B.zero1_fused_workspace(npieces), dtype=torch.uint8, device=device)


def _arenas(rank_grads):
    """The N ranks' full gradient arenas a step over every chunk reads; a tiled
    receive buffer holds one chunk only."""
    if isinstance(rank_grads, B.Tiled):
        raise TypeError("this step reads every rank's full gradient arena; a tiled receive "
                        "buffer holds one rank's chunk (Zero1OneRank, DDPOneRank)")
    return rank_grads


def _check_fused(workspace):
    """Raise if a wait of the last one-launch step gave up (or the workspace
    last served a plan of another piece count), after clearing the workspace
    so that the next step can run.  Reads a device word, so it waits for the
    stream's work."""
    if workspace is not None and B.fused_timed_out(workspace):
        B.fused_clear(workspace)
        raise RuntimeError("a wait of the one-launch step gave up, or its workspace served a "
                           "plan of another piece count: the tiles of the workgroups that gave "
                           "up kept their previous state (the others were updated); the "
                           "workspace has been cleared")


class Zero1AllRanks:
    """ZeRO-1 step of N simulated ranks over a bucket plan."""

    def __init__(self, buckets, nranks, master, hyper=None, device="cuda", reduce_flags=0):
        self.buckets = [(int(o), int(l)) for o, l in buckets]
        self.n = nranks
        self.hyper = hyper or Hyper()
        self.reduce_flags = reduce_flags
        self.numel = master.numel()
        master = master.to(device=device, dtype=torch.float32)
        self.chunks = [owned_chunk(r, nranks) for r in range(nranks)]
        self.state, self.means = [], []
        for c in self.chunks:
            idx = _shard_index(self.buckets, nranks, c, device)
            state, mean = _shard_state(master.index_select(0, idx),
                                       state_phase(self.buckets, nranks, c))
            self.state.append(state)
            self.means.append(mean)
        self.norm = _Norm(B.dp_piece_count(self.buckets, nranks), device)
        self.replicas = [master.to(torch.bfloat16) for _ in range(nranks)]

    def step(self, rank_grads, t, stream=None, token_counts=None):
        """One step; ``token_counts`` (one per rank) when each rank's gradient is a
        sum over its own tokens (token-weighted mean)."""
        self.enqueue(rank_grads, B.adamw_args(**step_scalars(self.hyper, t)), stream,
                     token_counts)

    def enqueue(self, rank_grads, args, stream=None, token_counts=None):
        """The step's kernels; ``args`` host ``AdamWArgs`` or a device tensor."""
        rank_grads = _arenas(rank_grads)
        for c, mean in zip(self.chunks, self.means):
            B.dp_reduce_scatter_mean(rank_grads, self.buckets, c, mean, self.norm.partials,
                                     flags=self.reduce_flags, stream=stream,
                                     token_counts=token_counts)
        self.norm.run(self.hyper.max_norm, stream, args)
        for c, (w, m, v), mean in zip(self.chunks, self.state, self.means):
            B.zero1_adamw_gather(w, m, v, mean, self.buckets, self.n, c, self.norm.scale, args,
                                 self.replicas, stream=stream)


class DDPStep:
    """Plain data-parallel step as one replica computes it.

    ``fused=True`` runs the step as one ``zero1_fused_step`` launch (the mean
    stays in registers; the arena must fit ``zero1_fused_capacity``).

    ``nreplicas=N`` writes the new weights into N replica arenas: then the
    step is also every simulated rank's ZeRO-1 step at once, with each rank's
    shard (chunk (r + 1) mod N of every bucket) held at its arena offsets in
    the one master/m/v -- the same arithmetic per element, bit for bit, in one
    reduce and one optimizer launch instead of N of each."""

    def __init__(self, buckets, nranks, master, hyper=None, device="cuda", reduce_flags=0,
                 fused=False, nreplicas=1):
        self.buckets = [(int(o), int(l)) for o, l in buckets]
        self.n = nranks
        self.hyper = hyper or Hyper()
        self.reduce_flags = reduce_flags
        self.fused = fused
        w = master.to(device=device, dtype=torch.float32).clone()
        self.state = (w, torch.zeros_like(w), torch.zeros_like(w))
        self.norm = _Norm(B.dp_piece_count(self.buckets, nranks), device)
        self.mean = None if fused else torch.zeros_like(w)
        self.workspace = _fused_workspace(self.norm.npieces, device) if fused else None
        self.replicas = [w.to(torch.bfloat16) for _ in range(nreplicas)]
        self.replica = self.replicas[0]

    def check_fused(self):
        """After the stream's work, with ``fused=True``: raise if a wait of the
        last step gave up (see ``zero1_fused_step``)."""
        _check_fused(self.workspace)

    def step(self, rank_grads, t, stream=None, token_counts=None):
        self.enqueue(rank_grads, B.adamw_args(**step_scalars(self.hyper, t)), stream,
                     token_counts)

    def enqueue(self, rank_grads, args, stream=None, token_counts=None):
        """The step's kernels; ``args`` host ``AdamWArgs``, a device tensor or a
        captured step's ``StepScalars``."""
        rank_grads = _arenas(rank_grads)
        w, m, v = self.state
        if self.fused:
            if token_counts is not None:
                raise ValueError("the fused step takes the plain mean")
            B.zero1_fused_step(rank_grads, self.buckets, -1, w, m, v, args,
                               self.hyper.max_norm, self.replicas, self.norm.partials,
                               self.workspace, self.norm.sqnorm, self.norm.scale,
                               flags=self.reduce_flags, stream=stream)
            return
        B.dp_reduce_scatter_mean(rank_grads, self.buckets, -1, self.mean, self.norm.partials,
                                 flags=self.reduce_flags, stream=stream,
                                 token_counts=token_counts)
        self.norm.run(self.hyper.max_norm, stream, args)
        B.zero1_adamw_gather(w, m, v, self.mean, self.buckets, self.n, -1, self.norm.scale,
                             args, self.replicas, stream=stream)


class Zero1OneRank:
    """ZeRO-1 step of one rank; its peers' contributions arrive as inputs.

    Per step the caller provides (all resident on the device):

    * ``incoming[j]`` -- rank j's gradient values of this rank's chunk,
      shard-compact (what a reduce-scatter delivers to the owner), or all N
      ranks' values in one ``Tiled`` receive buffer (``tiled_receive``);
    * the peers' norm pieces, written into ``self.norm.partials`` outside this
      rank's slots (what an all-gather of the piece sums delivers);
    * ``peer_shards[j]`` -- rank j's updated bf16 shard (``None`` at this rank),
      what the all-gather of the weights delivers.

    ``shard_master`` is copied into the step's own state (``self.state``), held
    at ``state_phase`` on its 128-byte lines.
    """

    def __init__(self, buckets, nranks, rank, shard_master, hyper=None, device="cuda",
                 arena_numel=None, reduce_flags=0, fused=False):
        self.buckets = [(int(o), int(l)) for o, l in buckets]
        self.reduce_flags = reduce_flags
        self.fused = fused
        self.n, self.rank = nranks, rank
        self.chunk = owned_chunk(rank, nranks)
        self.hyper = hyper or Hyper()
        w = shard_master.to(device=device, dtype=torch.float32)
        if w.numel() != B.dp_shard_numel(self.buckets, nranks, self.chunk):
            raise ValueError("shard_master does not match the plan's shard")
        self.state, self.mean = _shard_state(w.reshape(-1),
                                             state_phase(self.buckets, nranks, self.chunk),
                                             with_mean=not fused)
        self.norm = _Norm(B.dp_piece_count(self.buckets, nranks), device)
        self.workspace = _fused_workspace(self.norm.npieces, device) if fused else None
        ext = arena_numel or max(o + l for o, l in self.buckets)
        self.arena = torch.zeros(ext, dtype=torch.bfloat16, device=device)

    def own_piece_slots(self):
        """(first, count) ranges of this rank's pieces in the norm-piece array."""
        out = []
        for b, (_, length) in enumerate(self.buckets):
            first = B.dp_piece_offset(self.buckets, self.n, b, self.chunk)
            _, cnt = B.dp_chunk_range(length, self.n, self.chunk)
            out.append((first, -(-cnt // GRZ_PIECE)))
        return out

    def reduce(self, incoming, stream=None, token_counts=None):
        B.dp_reduce_scatter_mean(incoming, self.buckets, self.chunk, self.mean,
                                 self.norm.partials, flags=GRZ_IN_COMPACT | self.reduce_flags,
                                 stream=stream, token_counts=token_counts)

    def update(self, t, stream=None, args=None):
        """Norm, clip and AdamW with the bf16 write; ``args`` (host ``AdamWArgs`` or
        device tensor) overrides the scalars of step ``t``."""
        self.norm.run(self.hyper.max_norm, stream, args)
        if args is None:
            args = B.adamw_args(**step_scalars(self.hyper, t))
        w, m, v = self.state
        B.zero1_adamw_gather(w, m, v, self.mean, self.buckets, self.n, self.chunk,
                             self.norm.scale, args, [self.arena], stream=stream)

    def gather(self, peer_shards, stream=None):
        B.zero1_all_gather(peer_shards, self.buckets, [self.arena], stream=stream)

    def check_fused(self):
        """After the stream's work, with ``fused=True``: raise if a wait of the
        last step gave up (see ``zero1_fused_step``)."""
        _check_fused(self.workspace)

    def fused_update(self, incoming, args, stream=None):
        """reduce + update as one launch (the mean never leaves the registers)."""
        w, m, v = self.state
        B.zero1_fused_step(incoming, self.buckets, self.chunk, w, m, v, args,
                           self.hyper.max_norm, [self.arena], self.norm.partials,
                           self.workspace, self.norm.sqnorm, self.norm.scale,
                           flags=GRZ_IN_COMPACT | self.reduce_flags, stream=stream)

    def step(self, incoming, peer_shards, t, stream=None):
        if self.fused:
            self.fused_update(incoming, B.adamw_args(**step_scalars(self.hyper, t)), stream)
        else:
            self.reduce(incoming, stream)
            self.update(t, stream)
        self.gather(peer_shards, stream)

    def enqueue(self, incoming, peer_shards, args, stream=None):
        if self.fused:
            self.fused_update(incoming, args, stream)
        else:
            self.reduce(incoming, stream)
            self.update(None, stream, args=args)
        self.gather(peer_shards, stream)


class DDPOneRank:
    """Plain data-parallel (ZeRO stage 0) step of one rank; its peers'
    contributions arrive as inputs.

    The all-reduce of the mean is a reduce-scatter followed by an all-gather:
    this rank reduces its chunk ((rank + 1) mod N of every bucket) in ring
    order straight into its arena positions of the full fp32 mean, the peers'
    mean chunks land around it, and the rank runs clip + AdamW over its full
    copy of the state and writes its bf16 arena.  Per step the caller
    provides (all resident on the device):

    * ``incoming[j]`` -- rank j's gradient values of this rank's chunk,
      shard-compact;
    * ``peer_means[j]`` -- rank j's mean of its own chunk, shard-compact (what
      the all-gather half delivers; ``None`` at this rank);
    * the peers' norm pieces, written into ``self.norm.partials`` outside this
      rank's slots.

    Bucket lengths need not divide by N (plain data parallelism is what runs
    when they do not): the chunks then follow the array_split rule.
    """

    def __init__(self, buckets, nranks, rank, master, hyper=None, device="cuda"):
        self.buckets = [(int(o), int(l)) for o, l in buckets]
        self.n, self.rank = nranks, rank
        self.flags = GRZ_UNEVEN if any(l % nranks for _, l in self.buckets) else 0
        self.chunk = owned_chunk(rank, nranks)
        self.hyper = hyper or Hyper()
        w = master.to(device=device, dtype=torch.float32).contiguous().clone()
        self.state = (w, torch.zeros_like(w), torch.zeros_like(w))
        self.mean = torch.zeros_like(w)
        self.norm = _Norm(B.dp_piece_count(self.buckets, nranks, self.flags), device)
        self.arena = w.to(torch.bfloat16)

    own_piece_slots = Zero1OneRank.own_piece_slots

    def reduce(self, incoming, stream=None):
        B.dp_reduce_scatter_mean(incoming, self.buckets, self.chunk, self.mean,
                                 self.norm.partials,
                                 flags=GRZ_IN_COMPACT | GRZ_OUT_GLOBAL | self.flags,
                                 stream=stream)

    def receive_means(self, peer_means, stream=None):
        B.dp_all_gather(peer_means, self.buckets, [self.mean], flags=self.flags, stream=stream)

    def update(self, t, stream=None, args=None):
        self.norm.run(self.hyper.max_norm, stream, args)
        if args is None:
            args = B.adamw_args(**step_scalars(self.hyper, t))
        w, m, v = self.state
        B.zero1_adamw_gather(w, m, v, self.mean, self.buckets, self.n, -1, self.norm.scale,
                             args, [self.arena], stream=stream)

    def step(self, incoming, peer_means, t, stream=None):
        self.reduce(incoming, stream)
        self.receive_means(peer_means, stream)
        self.update(t, stream)

    def enqueue(self, incoming, peer_means, args, stream=None):
        """The step's kernels; ``args`` host ``AdamWArgs`` or a device tensor."""
        self.reduce(incoming, stream)
        self.receive_means(peer_means, stream)
        self.update(None, stream, args=args)


def one_rank_step(buckets, nranks, rank, master, hyper=None, device="cuda", stage=1,
                  log=None):
    """The step rank ``rank`` runs over ``master`` (the whole fp32 arena): ZeRO-1
    on its shard when ``stage`` is 1 and every bucket splits evenly over N,
    otherwise plain data parallelism on the whole arena, saying so ("A4",
    "Part 2 -- Tensor Sharding": an uneven split is an error for the sharding,
    and the caller falls back to stage 0)."""
    buckets = [(int(o), int(l)) for o, l in buckets]
    if zero_stage(buckets, nranks, stage, sys.stderr if log is None else log) == 1:
        idx = _shard_index(buckets, nranks, owned_chunk(rank, nranks), master.device)
        return Zero1OneRank(buckets, nranks, rank, master.index_select(0, idx), hyper, device,
                            arena_numel=master.numel())
    return DDPOneRank(buckets, nranks, rank, master, hyper, device)


class OverlappedZero1:
    """A ``Zero1AllRanks`` step whose reduce-scatter overlaps the backward.

    As each bucket's gradients become ready on the compute stream (the
    backward produces the last layer's bucket first), ``bucket_ready`` records
    an event there, makes the communication stream wait for it and enqueues
    that bucket's reduce-scatter on the communication stream ("A4 -- Multi-GPU
    with NCCL and ZeRO-1", "Part 3 -- Gradient Reduction": event record + stream
    wait, never a host synchronisation; "Distributed training" (noeira),
    "Overlap and graphs": buckets reduced on a second stream while the
    backward runs).  ``finish`` runs the norm, AdamW and the all-gather on the
    communication stream once every bucket is in, and makes the compute stream
    wait for them.  Both streams have the default priority.  The bytes
    produced are those of ``Zero1AllRanks.step`` (piece numbering and offsets
    are those of the whole plan).
    """

    def __init__(self, pipe, comm_stream=None):
        self.pipe = pipe
        self.comm = comm_stream if comm_stream is not None else torch.cuda.Stream()
        self.ready = [torch.cuda.Event() for _ in pipe.buckets]
        self.done = torch.cuda.Event()

    def bucket_ready(self, b, rank_grads, compute_stream=None):
        rank_grads = _arenas(rank_grads)
        p = self.pipe
        cs = compute_stream if compute_stream is not None else torch.cuda.current_stream()
        self.ready[b].record(cs)
        self.comm.wait_event(self.ready[b])
        for c, mean in zip(p.chunks, p.means):
            B.dp_reduce_scatter_mean(rank_grads, p.buckets, c, mean, p.norm.partials,
                                     flags=p.reduce_flags, stream=self.comm,
                                     bucket_range=(b, 1))

    def finish(self, t, compute_stream=None):
        p = self.pipe
        cs = compute_stream if compute_stream is not None else torch.cuda.current_stream()
        p.norm.run(p.hyper.max_norm, self.comm)
        args = B.adamw_args(**step_scalars(p.hyper, t))
        for c, (w, m, v), mean in zip(p.chunks, p.state, p.means):
            B.zero1_adamw_gather(w, m, v, mean, p.buckets, p.n, c, p.norm.scale, args,
                                 p.replicas, stream=self.comm)
        self.done.record(self.comm)
        cs.wait_event(self.done)


class Zero2AllRanks(Zero1AllRanks):
    """ZeRO stage 2 of N simulated ranks: gradients are sharded as well.

    No rank ever holds a full gradient arena: the backward hands each bucket's
    gradients to ``step`` through a staging buffer the size of the largest
    bucket (two of them, alternating), the bucket is reduce-scattered at once
    into the ranks' gradient shards, and the buffer is reused ("Lab 09 --
    Parallelism, simulated", s.4: stage 2 shards the gradients, 2 + 14/N bytes
    per parameter with bf16 gradient shards; "Distributed training" (noeira),
    ZeroSharded[2]).  With ``grad_shard="f32"`` the shards hold the fp32 mean
    and the update is the ZeRO-1 one, so the results are the same bits (as
    the noeira gates have every stage match plain data parallelism); with
    ``grad_shard="bf16"`` each shard holds the mean rounded once to bf16
    (``GRZ_MEAN_BF16``), 2 bytes per owned parameter as the page counts them,
    and the norm, the clip and AdamW take the rounded values.

    ``layout="shards"`` keeps each rank's gradient shard and state
    shard-compact (N reduce launches per bucket, N optimizer launches);
    ``layout="arena"`` holds every rank's shard at its arena offsets in one
    fp32 gradient array and one master/m/v (each rank still owns only its
    chunk of every bucket), so that each bucket is one reduce launch over all
    N chunks and the update one optimizer launch writing all N replicas --
    the same arithmetic per element, as ``DDPStep(nreplicas=N)`` is for ZeRO-1.
    """

    def __init__(self, buckets, nranks, master, hyper=None, device="cuda", reduce_flags=0,
                 grad_dtype=torch.bfloat16, layout="shards", grad_shard="f32"):
        if layout not in ("shards", "arena"):
            raise ValueError("layout is 'shards' or 'arena'")
        if grad_shard not in ("f32", "bf16"):
            raise ValueError("grad_shard is 'f32' or 'bf16'")
        self.layout = layout
        self.grad_shard = grad_shard
        shard_dtype = torch.float32 if grad_shard == "f32" else torch.bfloat16
        if layout == "shards":
            super().__init__(buckets, nranks, master, hyper, device, reduce_flags)
            if grad_shard == "bf16":
                self.means = [placed_zeros(mu.numel(), state_phase(self.buckets, nranks, c),
                                           mu.device, dtype=shard_dtype)
                              for c, mu in zip(self.chunks, self.means)]
        else:
            self.buckets = [(int(o), int(l)) for o, l in buckets]
            self.n = nranks
            self.hyper = hyper or Hyper()
            self.reduce_flags = reduce_flags
            self.numel = master.numel()
            w = master.to(device=device, dtype=torch.float32).clone()
            self.chunks = [owned_chunk(r, nranks) for r in range(nranks)]
            self.state = (w, torch.zeros_like(w), torch.zeros_like(w))
            # rank r's gradient shard at its arena offsets, every r
            self.mean = torch.zeros(w.numel(), dtype=shard_dtype, device=w.device)
            self.norm = _Norm(B.dp_piece_count(self.buckets, nranks), device)
            self.replicas = [w.to(torch.bfloat16) for _ in range(nranks)]
        longest = max((length for _, length in self.buckets), default=0)
        self.staging = [[torch.empty(max(longest, 1), dtype=grad_dtype, device=device)
                         for _ in range(nranks)] for _ in range(2)]

    def step(self, produce, t, stream=None):
        """``produce(b, bufs)`` writes rank r's gradients of bucket b (processing
        order) into ``bufs[r][:length_b]`` on ``stream``."""
        arena = self.layout == "arena"
        for b in range(len(self.buckets)):
            bufs = self.staging[b % 2]
            produce(b, bufs)
            flags = self.reduce_flags | GRZ_IN_RANGE
            if arena:
                B.dp_reduce_scatter_mean(bufs, self.buckets, -1, self.mean, self.norm.partials,
                                         flags=flags, stream=stream, bucket_range=(b, 1))
            else:
                for c, mean in zip(self.chunks, self.means):
                    B.dp_reduce_scatter_mean(bufs, self.buckets, c, mean, self.norm.partials,
                                             flags=flags, stream=stream, bucket_range=(b, 1))
        self.norm.run(self.hyper.max_norm, stream)
        args = B.adamw_args(**step_scalars(self.hyper, t))
        if arena:
            w, m, v = self.state
            B.zero1_adamw_gather(w, m, v, self.mean, self.buckets, self.n, -1, self.norm.scale,
                                 args, self.replicas, stream=stream)
            return
        for c, (w, m, v), mean in zip(self.chunks, self.state, self.means):
            B.zero1_adamw_gather(w, m, v, mean, self.buckets, self.n, c, self.norm.scale, args,
                                 self.replicas, stream=stream)

    def rank_view(self, rank):
        """Rank ``rank``'s gradient shard and (master, m, v), shard-compact (a copy
        gathered from the arena layout, or the held tensors)."""
        if self.layout == "shards":
            return self.means[rank], self.state[rank]
        idx = _shard_index(self.buckets, self.n, self.chunks[rank], self.mean.device)
        return (self.mean.index_select(0, idx),
                tuple(x.index_select(0, idx) for x in self.state))


class CapturedStep:
    """A whole step captured once in a HIP graph and replayed step after step.

    "Distributed training" (noeira), "Overlap and graphs": RankGraphs captures
    one graph per GPU and replays it.  The step's AdamW scalars change every
    step, so they live in a device table (rows for steps ``first_t`` ..
    ``first_t + count - 1``, filled once on the host with ``step_scalars``);
    each replay copies its row to the slot the optimizer reads
    (``GRZ_ARGS_DEVICE``) in the norm's last launch (``StepScalars``; the
    one-launch step, which has no norm launch of its own, does it in its
    launch).  ``enqueue(args, stream)`` must enqueue
    the step's kernels with ``args`` as their scalars;
    every buffer it touches keeps its address for the graph's lifetime.
    ``replay`` counts replays on the host and raises once the table's
    ``count`` steps are used (a further replay would repeat the last row's
    learning rate and bias corrections); capture again with a larger
    ``count`` to run longer.  Replays produce the bits of the eager steps.
    """

    def __init__(self, enqueue, hyper, first_t, count, device="cuda"):
        rows = []
        for t in range(first_t, first_t + count):
            s = step_scalars(hyper, t)
            rows.append([s["lr"], s["beta1"], s["beta2"], s["eps"], s["weight_decay"],
                         s["bias_corr1"], s["bias_corr2"]])
        self.table = torch.tensor(rows, dtype=torch.float32, device=device)
        self.count = count
        self.replays = 0
        self.counter = torch.zeros(1, dtype=torch.int64, device=device)
        self.current = torch.zeros(B.ARGS_FIELDS, dtype=torch.float32, device=device)
        self.scalars = B.StepScalars(self.table, self.counter, self.current)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            enqueue(self.scalars, torch.cuda.current_stream())

    def replay(self):
        """Run the next step; RuntimeError (nothing enqueued) past the table."""
        if self.replays >= self.count:
            raise RuntimeError(f"the captured step holds the scalars of {self.count} steps, "
                               "all replayed; capture it again with a larger count")
        self.graph.replay()
        self.replays += 1
