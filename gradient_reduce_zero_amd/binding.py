"""Python binding of libgrz: the C entry points under the same names.

Argument marshalling only.  Every function takes torch tensors for device
memory (PyTorch provides allocation and the current HIP stream), checks that
each buffer is on the GPU, contiguous and large enough for the plan (the C
library sees raw pointers and cannot check extents), and calls the C entry
point, raising ``GrzError`` on a non-zero status.  All arithmetic runs in the
library's kernels.
"""

import ctypes
import functools

import torch

from . import _native as N
from ._native import AdamWArgs, Bucket, check, lib

_KIND = {torch.bfloat16: N.GRZ_BF16, torch.int16: N.GRZ_BF16, torch.uint16: N.GRZ_BF16,
         torch.float32: N.GRZ_F32, torch.float64: N.GRZ_F64}
_OUT = {N.GRZ_BF16: torch.float32, N.GRZ_F32: torch.float32, N.GRZ_F64: torch.float64}
_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtypes=None, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the plan needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _key(buckets):
    return tuple((int(o), int(l)) for o, l in buckets)


@functools.lru_cache(maxsize=256)
def _bucket_array_of(key):
    # Read-only during each call, so one ctypes array per plan is reused.
    return (Bucket * max(len(key), 1))(*key), len(key)


def _bucket_array(buckets):
    return _bucket_array_of(_key(buckets))


def _extent(buckets):
    return max((o + l for o, l in buckets), default=0)


# -- plan helpers ------------------------------------------------------------

def dp_ring_owned_chunk(rank, nranks):
    return lib().dp_ring_owned_chunk(rank, nranks)


def dp_ring_chunk_owner(chunk, nranks):
    return lib().dp_ring_chunk_owner(chunk, nranks)


def dp_chunk_range(length, nranks, chunk):
    off, cnt = ctypes.c_int64(), ctypes.c_int64()
    check("dp_chunk_range", lib().dp_chunk_range(length, nranks, chunk, ctypes.byref(off),
                                                 ctypes.byref(cnt)))
    return off.value, cnt.value


def _neg_check(fn, value):
    if value < 0:
        check(fn, -value)
    return value


@functools.lru_cache(maxsize=1024)
def _piece_count(key, nranks, flags):
    arr, nb = _bucket_array_of(key)
    return _neg_check("dp_piece_count", lib().dp_piece_count(arr, nb, nranks, flags))


def dp_piece_count(buckets, nranks, flags=0):
    return _piece_count(_key(buckets), int(nranks), int(flags))


def dp_piece_offset(buckets, nranks, bucket, chunk, flags=0):
    arr, nb = _bucket_array(buckets)
    return _neg_check("dp_piece_offset",
                      lib().dp_piece_offset(arr, nb, nranks, flags, bucket, chunk))


@functools.lru_cache(maxsize=1024)
def _shard_numel(key, nranks, chunk, flags):
    arr, nb = _bucket_array_of(key)
    return _neg_check("dp_shard_numel", lib().dp_shard_numel(arr, nb, nranks, chunk, flags))


def dp_shard_numel(buckets, nranks, chunk, flags=0):
    return _shard_numel(_key(buckets), int(nranks), int(chunk), int(flags))


@functools.lru_cache(maxsize=1024)
def _tiled_numel(key, nranks, chunk, flags):
    arr, nb = _bucket_array_of(key)
    return _neg_check("dp_tiled_numel", lib().dp_tiled_numel(arr, nb, nranks, chunk, flags))


def dp_tiled_numel(buckets, nranks, chunk, flags=0):
    """Elements of chunk ``chunk``'s ``GRZ_IN_TILED`` receive buffer."""
    return _tiled_numel(_key(buckets), int(nranks), int(chunk), int(flags))


class Tiled:
    """The N ranks' values of one chunk in one receive buffer (``GRZ_IN_TILED``):
    the chunk's pieces in plan order, each piece's slot holding the N ranks'
    values side by side, ``GRZ_PIECE`` elements apiece (``dp_tiled_numel``
    elements).  Passed to ``dp_reduce_scatter_mean`` in place of the list of
    N rank tensors; the call then adds ``GRZ_IN_COMPACT | GRZ_IN_TILED``."""

    def __init__(self, buffer, nranks):
        self.buffer, self.nranks = buffer, int(nranks)


def dp_grad_sqnorm_workspace(npieces):
    return int(lib().dp_grad_sqnorm_workspace(int(npieces)))


# -- the pipeline --------------------------------------------------------------

def dp_reduce_scatter_mean(rank_grads, buckets, chunk, mean_out, piece_sqnorm=None, flags=0,
                           stream=None, bucket_range=None, token_counts=None):
    """Ring-order reduce-scatter-mean of ``rank_grads`` (one tensor per rank, or
    a ``Tiled`` receive buffer).

    ``bucket_range = (first, count)`` restricts the call to those buckets of
    the plan (``dp_reduce_scatter_mean_range``).  ``token_counts`` (one int per
    rank) makes it the token-weighted mean of per-rank gradient sums
    (``dp_reduce_scatter_weighted``).  A bf16 ``mean_out`` holds the mean
    rounded to bf16 (``GRZ_MEAN_BF16``)."""
    tiled = isinstance(rank_grads, Tiled)
    n = rank_grads.nranks if tiled else len(rank_grads)
    if not 1 <= n <= N.GRZ_MAX_RANKS:
        raise ValueError(f"{n} ranks; 1..{N.GRZ_MAX_RANKS} supported")
    dt = rank_grads.buffer.dtype if tiled else rank_grads[0].dtype
    if dt not in _KIND:
        raise TypeError(f"gradient dtype {dt} not supported")
    kind = _KIND[dt]
    buckets = list(buckets)
    if tiled:
        if chunk < 0 or flags & N.GRZ_IN_RANGE:
            raise ValueError("a tiled receive buffer holds one chunk (chunk >= 0, no GRZ_IN_RANGE)")
        flags |= N.GRZ_IN_COMPACT | N.GRZ_IN_TILED
    if chunk >= 0:
        shard = dp_shard_numel(buckets, n, chunk, flags & N.GRZ_UNEVEN)
        need_in = shard if flags & N.GRZ_IN_COMPACT else _extent(buckets)
        need_out = _extent(buckets) if flags & N.GRZ_OUT_GLOBAL else shard
    else:
        need_in = need_out = _extent(buckets)
    if flags & N.GRZ_IN_RANGE:
        if bucket_range is None:
            bucket_range = (0, len(buckets))
        sel = [b for b in buckets[bucket_range[0]:bucket_range[0] + bucket_range[1]] if b[1] > 0]
        need_in = _extent(sel) - min((o for o, _ in sel), default=0)
    same = _BF16_LIKE if kind == N.GRZ_BF16 else (dt,)
    if tiled:
        buf = rank_grads.buffer
        base = _dev(buf, "receive buffer", same,
                    dp_tiled_numel(buckets, n, chunk, flags & N.GRZ_UNEVEN)).value
        step = N.GRZ_PIECE * buf.element_size()
        ptrs = (ctypes.c_void_p * n)(*[base + j * step for j in range(n)])
    else:
        ptrs = (ctypes.c_void_p * n)(*[_dev(g, f"rank_grads[{j}]", same, need_in).value
                                       for j, g in enumerate(rank_grads)])
    if isinstance(mean_out, torch.Tensor) and mean_out.dtype in _BF16_LIKE:
        flags |= N.GRZ_MEAN_BF16
    out = _dev(mean_out, "mean_out",
               _BF16_LIKE if flags & N.GRZ_MEAN_BF16 else (_OUT[kind],), need_out)
    part = None
    if piece_sqnorm is not None:
        part = _dev(piece_sqnorm, "piece_sqnorm", (torch.float64,),
                    dp_piece_count(buckets, n, flags & N.GRZ_UNEVEN))
    arr, nb = _bucket_array(buckets)
    if token_counts is not None:
        if len(token_counts) != n:
            raise ValueError("one token count per rank")
        counts = (ctypes.c_int64 * n)(*[int(c) for c in token_counts])
        first, count = bucket_range if bucket_range is not None else (0, nb)
        check("dp_reduce_scatter_weighted",
              lib().dp_reduce_scatter_weighted(ptrs, counts, n, kind, arr, nb, int(first),
                                               int(count), chunk, flags, out, part,
                                               _stream(stream)))
    elif bucket_range is None:
        check("dp_reduce_scatter_mean",
              lib().dp_reduce_scatter_mean(ptrs, n, kind, arr, nb, chunk, flags, out, part,
                                           _stream(stream)))
    else:
        first, count = (int(x) for x in bucket_range)
        check("dp_reduce_scatter_mean_range",
              lib().dp_reduce_scatter_mean_range(ptrs, n, kind, arr, nb, first, count, chunk,
                                                 flags, out, part, _stream(stream)))


class StepScalars:
    """The AdamW scalars of a step in device memory: ``table`` (rows of 7
    float32 values, one per step), ``counter`` (int64, the next row) and
    ``current`` (the row the optimizer reads).  The first call of a step that
    needs ``current`` advances it -- the norm in its own last launch
    (``dp_grad_sqnorm_step_args``), the one-launch step in its launch
    (``zero1_fused_step_args``), else the optimizer's entry point with a
    ``grz_step_args_next`` launch before its own; ``advanced`` records that it
    was done for the step being enqueued.

    One object stands for one enqueued step: a captured step enqueues once and
    each replay advances the scalars again; eager steps take ``next()`` (the
    same tensors, not yet advanced) for each further step."""

    def __init__(self, table, counter, current):
        self.table, self.counter, self.current = table, counter, current
        self.advanced = False

    def next(self):
        """The scalars of the following step (same device tensors)."""
        return StepScalars(self.table, self.counter, self.current)


def dp_grad_sqnorm(piece_sqnorm, max_norm, workspace, sqnorm_out, clip_scale_out,
                   npieces=None, stream=None, step_args=None):
    """Fixed-order global squared norm of the piece sums and the clip factor;
    with ``step_args`` (a ``StepScalars`` not yet advanced for this step) the
    same launch advances the step's scalars."""
    npieces = piece_sqnorm.numel() if npieces is None else int(npieces)
    part = _dev(piece_sqnorm, "piece_sqnorm", (torch.float64,), npieces)
    need = dp_grad_sqnorm_workspace(npieces)
    ws = None
    if need:
        if workspace is None:
            raise ValueError(f"dp_grad_sqnorm needs {need} bytes of workspace")
        ws = _dev(workspace, "workspace")
        if workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                             f"bytes, {need} needed")
    sq = None if sqnorm_out is None else _dev(sqnorm_out, "sqnorm_out", (torch.float64,), 1)
    sc = None if clip_scale_out is None else _dev(clip_scale_out, "clip_scale_out",
                                                   (torch.float32,), 1)
    if step_args is not None and not step_args.advanced:
        rows = step_args.table.numel() // ARGS_FIELDS
        check("dp_grad_sqnorm_step_args",
              lib().dp_grad_sqnorm_step_args(
                  part, npieces, float(max_norm), ws, sq, sc,
                  _dev(step_args.table, "table", (torch.float32,), ARGS_FIELDS),
                  rows, _dev(step_args.counter, "counter", (torch.int64,), 1),
                  _dev(step_args.current, "current", (torch.float32,), ARGS_FIELDS),
                  _stream(stream)))
        step_args.advanced = True
        return
    check("dp_grad_sqnorm", lib().dp_grad_sqnorm(part, npieces, float(max_norm), ws, sq, sc,
                                                 _stream(stream)))


def dp_grad_sqnorm_noalloc(piece_sqnorm, max_norm, sqnorm_out, clip_scale_out, npieces=None,
                           stream=None):
    """``dp_grad_sqnorm`` with the library's static per-device scratch instead of
    a workspace (allocates nothing); calls that overlap on one device race."""
    npieces = piece_sqnorm.numel() if npieces is None else int(npieces)
    part = _dev(piece_sqnorm, "piece_sqnorm", (torch.float64,), npieces)
    sq = None if sqnorm_out is None else _dev(sqnorm_out, "sqnorm_out", (torch.float64,), 1)
    sc = None if clip_scale_out is None else _dev(clip_scale_out, "clip_scale_out",
                                                   (torch.float32,), 1)
    check("dp_grad_sqnorm_noalloc",
          lib().dp_grad_sqnorm_noalloc(part, npieces, float(max_norm), sq, sc, _stream(stream)))


def dp_grad_sqnorm_of_workspace(n):
    return int(lib().dp_grad_sqnorm_of_workspace(int(n)))


def dp_grad_sqnorm_of(grad, max_norm, workspace, sqnorm_out, clip_scale_out, stream=None):
    """Global squared norm and clip factor of an fp32 gradient array."""
    n = grad.numel()
    g = _dev(grad, "grad", (torch.float32,))
    need = dp_grad_sqnorm_of_workspace(n)
    ws = None
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"dp_grad_sqnorm_of needs {need} bytes of workspace")
        ws = _dev(workspace, "workspace")
    sq = None if sqnorm_out is None else _dev(sqnorm_out, "sqnorm_out", (torch.float64,), 1)
    sc = None if clip_scale_out is None else _dev(clip_scale_out, "clip_scale_out",
                                                   (torch.float32,), 1)
    check("dp_grad_sqnorm_of", lib().dp_grad_sqnorm_of(g, n, float(max_norm), ws, sq, sc,
                                                       _stream(stream)))


def adamw_args(lr, beta1, beta2, eps, weight_decay, bias_corr1, bias_corr2):
    return AdamWArgs(lr, beta1, beta2, eps, weight_decay, bias_corr1, bias_corr2)


def _state(master, m, v, mean_grad, n, grad_types=(torch.float32,)):
    f32 = (torch.float32,)
    return (_dev(master, "master", f32, n), _dev(m, "m", f32, n), _dev(v, "v", f32, n),
            _dev(mean_grad, "mean_grad", grad_types, n))


def zero1_adamw_step(master, m, v, mean_grad, clip_scale, args, bf16_out=None, n=None,
                     stream=None):
    """Clipped AdamW over ``n`` (default: all) shard-compact elements."""
    n = master.numel() if n is None else int(n)
    w, mm, vv, g = _state(master, m, v, mean_grad, n)
    sc = None if clip_scale is None else _dev(clip_scale, "clip_scale", (torch.float32,), 1)
    out = None if bf16_out is None else _dev(bf16_out, "bf16_out", _BF16_LIKE, n)
    check("zero1_adamw_step", lib().zero1_adamw_step(w, mm, vv, g, n, sc, ctypes.byref(args),
                                                     out, _stream(stream)))


ARGS_FIELDS = 7  # floats in grz_adamw_args


def _device_args(args, stream):
    """(pointer, True) for step scalars in device memory (a float32 tensor of
    7 values, or a ``StepScalars``, advanced first if nothing did it yet for
    this step), (byref, False) for host ``AdamWArgs``."""
    if isinstance(args, StepScalars):
        if not args.advanced:
            grz_step_args_next(args.table, args.counter, args.current, stream=stream)
            args.advanced = True
        args = args.current
    if isinstance(args, torch.Tensor):
        return ctypes.cast(_dev(args, "args", (torch.float32,), ARGS_FIELDS),
                           ctypes.POINTER(AdamWArgs)), True
    return ctypes.byref(args), False


def zero1_adamw_gather(master, m, v, mean_grad, buckets, nranks, chunk, clip_scale, args,
                       replicas, flags=0, stream=None):
    """Clipped AdamW on the shard of ``chunk`` with the bf16 all-gather write fused in.

    ``args`` is an ``AdamWArgs`` (host, read now) or a float32 device tensor of
    7 values in ``grz_adamw_args`` order, read when the kernel runs
    (``GRZ_ARGS_DEVICE``).  A bf16 ``mean_grad`` is a gradient shard held in
    bf16 (``GRZ_MEAN_BF16``)."""
    buckets = list(buckets)
    if isinstance(mean_grad, torch.Tensor) and mean_grad.dtype in _BF16_LIKE:
        flags |= N.GRZ_MEAN_BF16
    plan_flags = flags & ~N.GRZ_MEAN_BF16
    n = dp_shard_numel(buckets, nranks, chunk, plan_flags) if chunk >= 0 else _extent(buckets)
    w, mm, vv, g = _state(master, m, v, mean_grad, n,
                          _BF16_LIKE if flags & N.GRZ_MEAN_BF16 else (torch.float32,))
    sc = None if clip_scale is None else _dev(clip_scale, "clip_scale", (torch.float32,), 1)
    ext = _extent(buckets)
    reps = (ctypes.c_void_p * max(len(replicas), 1))(
        *[_dev(r, f"replicas[{i}]", _BF16_LIKE, ext).value for i, r in enumerate(replicas)])
    arr, nb = _bucket_array(buckets)
    a, on_device = _device_args(args, stream)
    if on_device:
        flags |= N.GRZ_ARGS_DEVICE
    check("zero1_adamw_gather",
          lib().zero1_adamw_gather(w, mm, vv, g, arr, nb, nranks, chunk, flags, sc, a, reps,
                                   len(replicas), _stream(stream)))


def grz_step_args_next(table, counter, current, stream=None):
    """Enqueue current = table[min(counter, rows - 1)]; counter += 1 (all on the device)."""
    rows = table.numel() // ARGS_FIELDS
    t = _dev(table, "table", (torch.float32,), ARGS_FIELDS)
    c = _dev(counter, "counter", (torch.int64,), 1)
    cur = _dev(current, "current", (torch.float32,), ARGS_FIELDS)
    check("grz_step_args_next", lib().grz_step_args_next(t, rows, c, cur, _stream(stream)))


def zero1_all_gather(shards, buckets, replicas, flags=0, stream=None):
    """Copy every rank's bf16 shard (``None`` = already in place) into every replica."""
    buckets = list(buckets)
    n = len(shards)
    ext = _extent(buckets)
    ptrs = []
    for r, s in enumerate(shards):
        if s is None:
            ptrs.append(None)
        else:
            need = dp_shard_numel(buckets, n, (r + 1) % n, flags)
            ptrs.append(_dev(s, f"shards[{r}]", _BF16_LIKE, need).value)
    sp = (ctypes.c_void_p * max(n, 1))(*ptrs)
    reps = (ctypes.c_void_p * max(len(replicas), 1))(
        *[_dev(r, f"replicas[{i}]", _BF16_LIKE, ext).value for i, r in enumerate(replicas)])
    arr, nb = _bucket_array(buckets)
    check("zero1_all_gather", lib().zero1_all_gather(sp, n, arr, nb, flags, reps, len(replicas),
                                                     _stream(stream)))


def dp_all_gather(shards, buckets, replicas, flags=0, stream=None):
    """``zero1_all_gather`` for bf16, fp32 or fp64 shards (all of one dtype, that of
    the replicas): rank r's shard-compact chunk (r + 1) mod N lands at its arena
    offsets in every replica (``None`` = already in place)."""
    buckets = list(buckets)
    n = len(shards)
    given = [s for s in shards if s is not None] + list(replicas)
    if not given:
        raise ValueError("no shard and no replica")
    dt = given[0].dtype
    kind = _KIND.get(dt)
    if kind is None:
        raise TypeError(f"dtype {dt} not supported")
    same = _BF16_LIKE if kind == N.GRZ_BF16 else (dt,)
    ext = _extent(buckets)
    ptrs = []
    for r, s in enumerate(shards):
        if s is None:
            ptrs.append(None)
        else:
            need = dp_shard_numel(buckets, n, (r + 1) % n, flags)
            ptrs.append(_dev(s, f"shards[{r}]", same, need).value)
    sp = (ctypes.c_void_p * max(n, 1))(*ptrs)
    reps = (ctypes.c_void_p * max(len(replicas), 1))(
        *[_dev(r, f"replicas[{i}]", same, ext).value for i, r in enumerate(replicas)])
    arr, nb = _bucket_array(buckets)
    check("dp_all_gather", lib().dp_all_gather(sp, n, kind, arr, nb, flags, reps, len(replicas),
                                               _stream(stream)))


def fused_set_spin_limit(workspace, polls):
    """Polls a wait of ``zero1_fused_step`` on ``workspace`` makes before it
    gives up (the workspace's 32-bit word at byte 12; 0 restores the library's
    default).  Enqueued on the current stream like any write."""
    if not 0 <= int(polls) < 2 ** 31:
        raise ValueError("polls must be in [0, 2^31)")
    workspace.view(torch.int32)[3].fill_(int(polls))


def zero1_fused_workspace(npieces):
    return int(lib().zero1_fused_workspace(int(npieces)))


def zero1_fused_capacity(nranks, dtype):
    """Pieces one fused launch holds for ``nranks`` ranks of ``dtype`` gradients."""
    kind = _KIND[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return _neg_check("zero1_fused_capacity", lib().zero1_fused_capacity(int(nranks), kind))


def zero1_fused_step(rank_grads, buckets, chunk, master, m, v, args, max_norm, replicas,
                     piece_sqnorm, workspace, sqnorm_out=None, clip_scale_out=None,
                     mean_out=None, flags=0, stream=None):
    """Reduce-scatter-mean, norm, clip, AdamW and the bf16 write of one shard
    (``chunk >= 0``) or of every chunk (``chunk = -1``) in one launch.

    ``workspace`` (``zero1_fused_workspace`` bytes) must be zeroed before its
    first use; ``args`` is an ``AdamWArgs``, a device float32 tensor of 7
    values (``GRZ_ARGS_DEVICE``), or a ``StepScalars`` whose row the launch
    takes and advances itself (``zero1_fused_step_args``)."""
    n = len(rank_grads)
    if not 1 <= n <= N.GRZ_MAX_RANKS:
        raise ValueError(f"{n} ranks; 1..{N.GRZ_MAX_RANKS} supported")
    dt = rank_grads[0].dtype
    if dt not in (torch.float32,) + _BF16_LIKE:
        raise TypeError(f"gradient dtype {dt} not supported by the fused step")
    kind = _KIND[dt]
    buckets = list(buckets)
    ext = _extent(buckets)
    shard = dp_shard_numel(buckets, n, chunk, flags & N.GRZ_UNEVEN) if chunk >= 0 else ext
    need_in = shard if flags & N.GRZ_IN_COMPACT else ext
    same = _BF16_LIKE if kind == N.GRZ_BF16 else (dt,)
    ptrs = (ctypes.c_void_p * n)(*[_dev(g, f"rank_grads[{j}]", same, need_in).value
                                   for j, g in enumerate(rank_grads)])
    f32 = (torch.float32,)
    w, mm, vv = (_dev(master, "master", f32, shard), _dev(m, "m", f32, shard),
                 _dev(v, "v", f32, shard))
    npieces = dp_piece_count(buckets, n, flags & N.GRZ_UNEVEN)
    part = _dev(piece_sqnorm, "piece_sqnorm", (torch.float64,), npieces)
    need_ws = zero1_fused_workspace(npieces)
    if workspace.numel() * workspace.element_size() < need_ws:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                         f"bytes, {need_ws} needed")
    ws = _dev(workspace, "workspace")
    sq = None if sqnorm_out is None else _dev(sqnorm_out, "sqnorm_out", (torch.float64,), 1)
    sc = None if clip_scale_out is None else _dev(clip_scale_out, "clip_scale_out", f32, 1)
    mo = None if mean_out is None else _dev(mean_out, "mean_out", f32, shard)
    reps = (ctypes.c_void_p * max(len(replicas), 1))(
        *[_dev(r, f"replicas[{i}]", _BF16_LIKE, ext).value for i, r in enumerate(replicas)])
    arr, nb = _bucket_array(buckets)
    if isinstance(args, StepScalars) and not args.advanced:
        # One launch takes the step's row of the table and advances it.
        check("zero1_fused_step_args",
              lib().zero1_fused_step_args(
                  ptrs, n, kind, arr, nb, chunk, flags, w, mm, vv,
                  _dev(args.table, "table", (torch.float32,)), args.table.shape[0],
                  _dev(args.counter, "counter", (torch.int64,), 1),
                  _dev(args.current, "current", (torch.float32,), ARGS_FIELDS),
                  float(max_norm), reps, len(replicas), part, ws, sq, sc, mo, _stream(stream)))
        args.advanced = True
        return
    a, on_device = _device_args(args, stream)
    if on_device:
        flags |= N.GRZ_ARGS_DEVICE
    check("zero1_fused_step",
          lib().zero1_fused_step(ptrs, n, kind, arr, nb, chunk, flags, w, mm, vv, a,
                                 float(max_norm), reps, len(replicas), part, ws, sq, sc, mo,
                                 _stream(stream)))


def fused_timed_out(workspace):
    """True if a wait of a fused step on ``workspace`` gave up, or a step with
    another piece count was refused (reads the device word: synchronises with
    the stream's work)."""
    return int(workspace.view(torch.int32)[2].item()) != 0


def fused_clear(workspace):
    """Zero a fused-step workspace after a wait gave up (the flag, the launch
    counter and the published piece sums), keeping its poll limit."""
    words = workspace.view(torch.int32)
    limit = words[3].clone()
    workspace.zero_()
    words[3].copy_(limit)


def grz_set_max_blocks(blocks):
    """Grid width of the grid-stride kernels (speed only; results do not change)."""
    check("grz_set_max_blocks", lib().grz_set_max_blocks(int(blocks)))
