"""The overlapped step's stream schedule, checked on the CPU with stand-ins for
streams, events and the library calls: every bucket's reduce is enqueued on
the communication stream only after that stream waits for an event recorded
on the compute stream after the bucket was produced ("A4 -- Multi-GPU with
NCCL and ZeRO-1", "Part 3" and "Common Mistakes": without the event the
collective can start before the gradients exist)."""

import types

import gradient_reduce_zero_amd.step as S


class FakeEvent:
    log = None

    def __init__(self):
        self.id = len(FakeEvent.all)
        FakeEvent.all.append(self)

    def record(self, stream):
        FakeEvent.log.append(("record", stream.name, self.id))


class FakeStream:
    def __init__(self, name):
        self.name = name

    def wait_event(self, ev):
        FakeEvent.log.append(("wait", self.name, ev.id))


def _run_schedule(monkeypatch, overlapped_cls):
    """Run two buckets through ``overlapped_cls`` with stand-ins; return (calls, ov)."""
    FakeEvent.all, FakeEvent.log = [], []
    monkeypatch.setattr(S.torch.cuda, "Event", FakeEvent)
    calls = FakeEvent.log

    def rs(grads, buckets, c, mean, partials, flags=0, stream=None, bucket_range=None):
        calls.append(("reduce", stream.name, bucket_range, c))

    def norm_run(max_norm, stream):
        calls.append(("norm", stream.name))

    def adamw(*a, stream=None, **k):
        calls.append(("adamw", stream.name))

    monkeypatch.setattr(S.B, "dp_reduce_scatter_mean", rs)
    monkeypatch.setattr(S.B, "zero1_adamw_gather", adamw)
    monkeypatch.setattr(S.B, "adamw_args", lambda **k: None)
    pipe = types.SimpleNamespace(
        buckets=[(8, 8), (0, 8)], chunks=[1, 0], means=[None, None], n=2, reduce_flags=0,
        norm=types.SimpleNamespace(partials=None, scale=None, run=norm_run),
        hyper=S.Hyper(), state=[(0, 0, 0), (0, 0, 0)], replicas=[])
    comm, compute = FakeStream("comm"), FakeStream("compute")
    ov = overlapped_cls(pipe, comm_stream=comm)
    for b in range(2):
        calls.append(("produce", "compute", b))
        ov.bucket_ready(b, [None, None], compute_stream=compute)
    ov.finish(1, compute_stream=compute)
    return calls, ov


def schedule_violations(calls, ov):
    """What is out of order in a recorded schedule (empty when it is right)."""
    bad = []
    for b in range(2):
        produced = calls.index(("produce", "compute", b))
        recorded = calls.index(("record", "compute", ov.ready[b].id))
        waits = [i for i, c in enumerate(calls) if c == ("wait", "comm", ov.ready[b].id)]
        reduces = [i for i, c in enumerate(calls) if c[0] == "reduce" and c[2] == (b, 1)]
        if len(reduces) != 2 or any(calls[i][1] != "comm" for i in reduces):
            bad.append(f"bucket {b}: reduces not on the communication stream")
        if not waits or not produced < recorded < waits[0] < min(reduces):
            bad.append(f"bucket {b}: reduce not ordered after its gradients")
    last_reduce = max(i for i, c in enumerate(calls) if c[0] == "reduce")
    norm = calls.index(("norm", "comm"))
    adam = [i for i, c in enumerate(calls) if c[0] == "adamw"]
    done = calls.index(("record", "comm", ov.done.id))
    if not (last_reduce < norm < min(adam) and max(adam) < done):
        bad.append("update not after every reduce")
    if calls[-1] != ("wait", "compute", ov.done.id):
        bad.append("compute stream does not wait for the update")
    return bad


def test_overlap_orders_each_bucket_reduce_after_its_event(monkeypatch):
    calls, ov = _run_schedule(monkeypatch, S.OverlappedZero1)
    assert schedule_violations(calls, ov) == []


def test_a_dropped_wait_is_caught(monkeypatch):
    # Planted on the CPU: the communication stream never waits for the
    # compute stream's event, so its reduce could read gradients that are not
    # there yet ("A4", "Common Mistakes"; noeira's unordered naive streams).
    class NoWait(S.OverlappedZero1):
        def bucket_ready(self, b, rank_grads, compute_stream=None):
            comm = self.comm
            self.comm = types.SimpleNamespace(name=comm.name, wait_event=lambda ev: None)
            try:
                super().bucket_ready(b, rank_grads, compute_stream)
            finally:
                self.comm = comm

    calls, ov = _run_schedule(monkeypatch, NoWait)
    bad = schedule_violations(calls, ov)
    assert any("not ordered after its gradients" in v for v in bad)
