"""Seeded synthetic gradients, weights and peer partial norms.

Recipe: rank r's gradient at step t is sigma * z with z ~ N(0, 1) in fp32,
drawn from a torch generator seeded with 1_000_003 * t + 1_009 * r + base, on
the device the caller names; bf16 gradients are that fp32 draw rounded to
bf16 by torch.  Master weights are fp32 N(0, 0.02) from seed base + 7
("Distributed training" (noeira), "Training a GPT": Normal(0.0, 0.02)).
The same bytes are copied to the host for the oracle.
"""

import torch

GRAD_SEED = 0


def grad_seed(step, rank, base=GRAD_SEED):
    return 1_000_003 * int(step) + 1_009 * int(rank) + int(base)


_TORCH = {"bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}


def rank_grad(numel, sigma, kind, seed, device="cpu", spans=None):
    """One rank's flat gradient as a torch tensor of ``kind``'s dtype.

    ``spans`` (optional) is ``[(offset, numel, sigma)]``: a per-range standard
    deviation that replaces ``sigma`` there.
    """
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    draw_dtype = torch.float64 if kind == "f64" else torch.float32
    z = torch.randn(int(numel), generator=g, device=device, dtype=draw_dtype)
    if spans is None:
        z.mul_(sigma)
    else:
        for off, n, s in spans:
            z[off:off + n].mul_(s)
    return z.to(_TORCH[kind]) if kind == "bf16" else z


def master_init(numel, seed=GRAD_SEED + 7, device="cpu", std=0.02):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(int(numel), generator=g, device=device, dtype=torch.float32).mul_(std)


def peer_partials(count, piece, sigma_mean, seed, device="cpu"):
    """Plausible fp64 sums of squares of ``piece`` mean-gradient values each.

    A rank that holds only its own shard receives its peers' partial norms
    over the wire; these stand in for them: piece * sigma_mean^2 * (1 + 0.05 z).
    """
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    z = torch.randn(int(count), generator=g, device=device, dtype=torch.float64)
    return (z.mul_(0.05).add_(1.0)).mul_(float(piece) * float(sigma_mean) ** 2)


def to_bits(t):
    """Host NumPy view of a tensor: bf16 as uint16 patterns, others as is."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def onerank_inputs(shard_numel, nranks, rank, npieces, piece, step=1, sigma=1e-3,
                   device="cpu", base=GRAD_SEED):
    """Everything one ZeRO-1 rank receives in a step, resident on ``device``.

    * ``incoming[j]``: rank j's bf16 gradient values of this rank's shard;
    * ``peer_shards[j]``: rank j's updated bf16 weight shard (None for ``rank``);
    * ``partials``: fp64 norm pieces of the whole plan (``npieces``), standing in
      for the peers' pieces (this rank's own slots are overwritten by its reduce);
    * ``shard_master``: fp32 N(0, 0.02) master weights of this rank's shard.
    """
    incoming = [rank_grad(shard_numel, sigma, "bf16", grad_seed(step, j, base), device)
                for j in range(nranks)]
    peer_shards = [None if j == rank else
                   master_init(shard_numel, seed=base + 100 + j, device=device).to(torch.bfloat16)
                   for j in range(nranks)]
    partials = peer_partials(npieces, piece, sigma / nranks ** 0.5, seed=base + 99,
                             device=device)
    shard_master = master_init(shard_numel, seed=base + 7 + rank, device=device)
    return dict(incoming=incoming, peer_shards=peer_shards, partials=partials,
                shard_master=shard_master)
