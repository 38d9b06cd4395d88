"""Norm, clip, AdamW, bf16 rounding and all-gather (oracle; test infrastructure).

The step order is the one every page gives: reduce the gradients, clip by the
global norm, run AdamW only on the owned shard, all-gather the new weights
("A4 -- Multi-GPU with NCCL and ZeRO-1", "Part 4 -- Multi-GPU Backward and
Update", gpt2_update; "Distributed training" (noeira), "Four strategies, one
interface": set_lr, forward_backward, clip_grads_device(max_norm), step).
The optimizer state is fp32 master weights, m and v ("A4", "Overview",
ZeRO-1 in one picture; "Lab 09", s.4: 12 bytes of fp32 state per parameter).

Readings (the pages name these steps but do not print their formulas):

* Norm: Euclidean norm of the mean gradient over the whole arena.  Every
  square of an fp32 value is exact in float64; the oracle sums them with
  ``math.fsum`` (the correctly rounded exact sum) up to ``FSUM_LIMIT`` terms
  and with float64 ``numpy.sum`` above.
* Clip: scale = max_norm / norm rounded to fp32 when norm > max_norm, else 1;
  a non-positive max_norm disables clipping.  No epsilon.
* AdamW (decoupled weight decay, Loshchilov & Hutter), every operation in
  fp32 and rounded on its own (no fused multiply-add), t starting at 1,
  m = v = 0 before the first step, weight decay on every element:
      g = mean * scale
      m = b1*m + (1 - b1)*g
      v = b2*v + (1 - b2)*(g*g)
      u = (m / bc1) / (sqrt(v / bc2) + eps)
      master = master - lr*(u + wd*master)
  with bc1 = fp32(1 - b1^t), bc2 = fp32(1 - b2^t) evaluated in float64.
* bf16: round to nearest, ties to even mantissa; a value beyond the largest
  bf16 by half an ulp or more becomes an infinity; NaN stays a (quiet) NaN.
* The gradient shard an owner keeps between the reduce-scatter and the
  update: by default in fp32, the type the ring accumulates in, so that every
  ZeRO stage sees the same values as plain data parallelism ("Distributed
  training", "Gates": the stages agree bit for bit with DDP when nothing is
  clipped).  With ``grad_shard="bf16"`` it is held in bf16 as "Lab 09", s.4
  counts it (2 bytes of bf16 gradients per parameter, divided by N from
  stage 2 on): each mean value is rounded once to bf16 (nearest even), and
  the norm, the clip and AdamW all take the rounded value, widened exactly.

Pins (tests/test_oracle_step.py): the norm against a closed form (constant
gradient a over P elements has norm |a|*sqrt(P)) and against
``torch.nn.utils.clip_grad_norm_``; its numpy branch (above FSUM_LIMIT terms)
against ``math.fsum`` with the limit lowered, and above the limit against the
closed-form sum of squares of a grid gradient whose every partial sum is exact; AdamW against ``torch.optim.AdamW``
(``foreach=False``, float64, CPU) over 10 steps and against two closed forms
(all-zero gradients decay the weights by (1 - lr*wd) per step; at t = 1 the
update is g / (|g| + eps) up to rounding); bf16 rounding against torch's CPU
``.to(torch.bfloat16)`` on a dense sample of binary32 patterns (ties, subnormals,
the overflow boundary, infinities, NaN).  The bf16 gradient shard: on means
that are bf16 values already the step is the fp32-shard step bit for bit; on
means just off bf16 values (below, above and exactly at half a bf16 ulp) it
is the fp32-shard step on the hand-rounded means, and the norm is the closed
form of those rounded values.
"""

import math

import numpy as np

from .bf16 import bf16_round  # noqa: F401  (re-exported)
from .reduce import owned_chunk, reduce_scatter_mean, shard_segments, widen

FSUM_LIMIT = 20_000_000


def grad_sqnorm(values, extra=()):
    """Sum of squares of ``values`` (fp32 or fp64) plus ``extra`` float64 terms.

    ``extra`` carries partial sums of squares that another rank computed (a
    rank that only holds its own shard needs its peers' parts to form the
    global norm).
    """
    sq = np.square(np.asarray(values, dtype=np.float64))
    extra = np.asarray(extra, dtype=np.float64)
    if sq.size + extra.size <= FSUM_LIMIT:
        return math.fsum(np.concatenate([sq.ravel(), extra.ravel()]).tolist())
    return float(np.sum(sq, dtype=np.float64) + np.sum(extra, dtype=np.float64))


def clip_scale(sqnorm, max_norm):
    """fp32 factor that brings the gradient norm down to ``max_norm``."""
    if max_norm <= 0:
        return np.float32(1.0)
    norm = math.sqrt(sqnorm)
    if norm > max_norm:
        return np.float32(max_norm / norm)
    return np.float32(1.0)


def bias_corrections(t, beta1, beta2):
    """fp32(1 - beta1^t), fp32(1 - beta2^t), evaluated in float64."""
    return np.float32(1.0 - float(beta1) ** t), np.float32(1.0 - float(beta2) ** t)


def lr_at(t, base_lr, warmup=0):
    """Learning rate of step t: linear warmup over ``warmup`` steps, then flat."""
    if warmup > 0 and t <= warmup:
        return np.float32(float(base_lr) * t / warmup)
    return np.float32(base_lr)


def adamw(master, m, v, g, lr, beta1, beta2, eps, wd, bc1, bc2):
    """One AdamW update in fp32; returns new (master, m, v).  Inputs are not modified."""
    f = np.float32
    master = np.asarray(master, dtype=np.float32)
    m = np.asarray(m, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    b1, b2, one = f(beta1), f(beta2), f(1.0)
    m_new = b1 * m + (one - b1) * g
    v_new = b2 * v + (one - b2) * (g * g)
    m_hat = m_new / f(bc1)
    v_hat = v_new / f(bc2)
    upd = m_hat / (np.sqrt(v_hat) + f(eps))
    master_new = master - f(lr) * (upd + f(wd) * master)
    return master_new, m_new, v_new


def all_gather(shards, buckets, nranks, arena_len, uneven=False):
    """Every replica's bf16 arena after the all-gather.

    ``shards[r]`` is rank r's shard-compact bf16 shard (chunk (r + 1) mod N of
    every bucket) or None for a rank that sends nothing.  Each replica ends
    with every shard at its global offsets ("Lab 09", s.1, the all-gather
    rows of the N = 3 table; "A4", gpt2_update).  Returns one arena; all N
    replicas are equal to it.
    """
    out = np.zeros(arena_len, dtype=np.uint16)
    for r, shard in enumerate(shards):
        if shard is None:
            continue
        for gstart, length, cstart in shard_segments(buckets, nranks, owned_chunk(r, nranks), uneven):
            out[gstart:gstart + length] = shard[cstart:cstart + length]
    return out


class Hyper:
    """Optimizer settings of one run."""

    def __init__(self, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                 max_norm=1.0, warmup=0):
        self.lr, self.beta1, self.beta2 = lr, beta1, beta2
        self.eps, self.weight_decay = eps, weight_decay
        self.max_norm, self.warmup = max_norm, warmup

    def scalars(self, t):
        bc1, bc2 = bias_corrections(t, self.beta1, self.beta2)
        return dict(lr=lr_at(t, self.lr, self.warmup), beta1=self.beta1, beta2=self.beta2,
                    eps=self.eps, wd=self.weight_decay, bc1=bc1, bc2=bc2)


def _check_cover(buckets, arena_len):
    spans = sorted(buckets)
    pos = 0
    for off, length in spans:
        if off != pos:
            raise ValueError("buckets must tile the arena")
        pos += length
    if pos != arena_len:
        raise ValueError("buckets must tile the arena")


def held_gradient(mean, grad_shard=None):
    """The gradient shard as its owner holds it until the update.

    ``None``: the fp32 mean itself.  ``"bf16"``: the mean rounded once to bf16
    (nearest even) and widened back to fp32, which is exact ("Lab 09", s.4:
    2 bytes of bf16 gradients per parameter).
    """
    if grad_shard is None:
        return mean
    if grad_shard == "bf16":
        if mean.dtype != np.float32:
            raise ValueError("a bf16 gradient shard holds the mean of fp32 or bf16 gradients")
        return widen(bf16_round(mean), "bf16")
    raise ValueError(f"unknown gradient shard type {grad_shard!r}")


def zero1_step(rank_grads, kind, buckets, states, hyper, t, wire=None, token_counts=None,
               grad_shard=None):
    """One ZeRO-1 step of all N simulated ranks.

    ``states[r] = (master, m, v)``: rank r's shard-compact fp32 state for
    chunk (r + 1) mod N of every bucket.  Returns a dict with the per-rank
    mean shards (as held, see ``held_gradient``), the global sqnorm and clip
    scale, the new states, the per-rank bf16 shards and the gathered bf16
    arena (equal on all ranks).  With ``grad_shard="bf16"`` it is the step of
    ZeRO-2 as "Lab 09", s.4 counts its bytes.
    """
    n = len(rank_grads)
    arena_len = rank_grads[0].shape[0]
    _check_cover(buckets, arena_len)
    means = [held_gradient(reduce_scatter_mean(rank_grads, kind, buckets, owned_chunk(r, n),
                                               wire=wire, token_counts=token_counts),
                           grad_shard)
             for r in range(n)]
    sq = grad_sqnorm(np.concatenate(means))
    scale = clip_scale(sq, hyper.max_norm)
    s = hyper.scalars(t)
    new_states, shards = [], []
    for r in range(n):
        g = means[r] * scale
        master, m, v = adamw(*states[r], g, **s)
        new_states.append((master, m, v))
        shards.append(bf16_round(master))
    arena = all_gather(shards, buckets, n, arena_len)
    return dict(means=means, sqnorm=sq, scale=scale, states=new_states,
                shards=shards, arena=arena)


def ddp_step(rank_grads, kind, buckets, state, hyper, t, wire=None, token_counts=None):
    """One plain data-parallel step (ZeRO stage 0).

    Every replica all-reduces the full gradient and runs the identical AdamW
    on its full copy of the state, so one replica's computation stands for
    all of them.  ``state = (master, m, v)`` over the whole arena.
    """
    arena_len = rank_grads[0].shape[0]
    _check_cover(buckets, arena_len)
    mean = reduce_scatter_mean(rank_grads, kind, buckets, -1, arena_len=arena_len, wire=wire,
                               token_counts=token_counts)
    sq = grad_sqnorm(mean)
    scale = clip_scale(sq, hyper.max_norm)
    master, m, v = adamw(*state, mean * scale, **hyper.scalars(t))
    return dict(mean=mean, sqnorm=sq, scale=scale, state=(master, m, v),
                arena=bf16_round(master))
