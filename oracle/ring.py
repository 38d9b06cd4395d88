"""Ring all-reduce, simulated by explicit messages (oracle; test infrastructure).

Follows "Lab 09 -- Parallelism, simulated":

* s.1 "Ring all-reduce": N ranks each hold a vector split into N chunks; two
  phases of N - 1 steps; in every step each rank sends one chunk to its right
  neighbour (rank r -> rank r + 1 mod N), all at the same time.  In the
  reduce-scatter phase the receiver adds the message into its own copy of
  that chunk; in the all-gather phase the receiver overwrites its copy.
* "Tips": in reduce-scatter step t rank r sends chunk (r - t) mod N; after the
  phase rank r holds the finished chunk (r + 1) mod N, so in all-gather step t
  it sends chunk (r + 1 - t) mod N.  Every message of a step is built first
  (with a copy of its data) and only then are all of them delivered.
  Bytes are counted with ``nbytes`` of what is sent.

Chunk boundaries follow ``numpy.array_split`` (the first ``len mod N`` chunks
are one element longer); the page's test only uses lengths divisible by N.

Pins (tests/test_oracle_ring.py): the N = 3 schedule table of s.1 cell by cell
(tests/golden/ring_n3_schedule.txt), the byte counts 512 / 768 / 896 for 64
float64 values at N = 2 / 4 / 8 and the naive rank-0 receive 512 / 1536 /
3584 (s.1), Eq. (13.5.1) of "13.5 Multi-GPU from First Principles", exact sums
on integer-valued data against ``numpy.sum``, and the "Common bugs" case
(all-gather started from chunk r corrupts the result).
"""

import numpy as np


def chunk_bounds(length, nranks):
    """Half-open [start, stop) of each of the ``nranks`` chunks of ``length``.

    The first ``length % nranks`` chunks get one extra element (the
    ``numpy.array_split`` rule).
    """
    q, rem = divmod(int(length), int(nranks))
    out = []
    start = 0
    for c in range(nranks):
        size = q + (1 if c < rem else 0)
        out.append((start, start + size))
        start += size
    return out


def ring_all_reduce(arrays, ag_start_offset=1, wire_round=None):
    """Run the ring all-reduce on copies of ``arrays`` (one 1-D array per rank).

    Returns ``(results, sent, log)``:

    * ``results[r]`` -- rank r's vector after both phases,
    * ``sent[r]``    -- bytes rank r sent (``nbytes`` of its messages),
    * ``log``        -- one entry per message:
      ``(phase, step, sender, receiver, chunk, payload_copy)`` with phase
      ``"RS"`` or ``"AG"``.

    ``ag_start_offset`` is the chunk rank r sends first in the all-gather,
    relative to r: 1 is the rule of the page ((r + 1 - t) mod N); 0 is the
    "wrong chunk" bug listed under "Common bugs" and exists only so a test can
    show that it corrupts the sums.
    """
    n = len(arrays)
    data = [np.array(a, copy=True) for a in arrays]
    length = data[0].shape[0]
    for a in data:
        assert a.shape == (length,) and a.dtype == data[0].dtype
    bounds = chunk_bounds(length, n)
    sent = [0] * n
    log = []

    # Phase 1: reduce-scatter.  Step t: rank r sends chunk (r - t) mod N.
    for t in range(n - 1):
        messages = []
        for r in range(n):
            c = (r - t) % n
            lo, hi = bounds[c]
            messages.append((r, (r + 1) % n, c, data[r][lo:hi].copy()))
        for src, dst, c, payload in messages:
            lo, hi = bounds[c]
            summed = data[dst][lo:hi] + payload
            data[dst][lo:hi] = summed if wire_round is None else wire_round(summed)
            sent[src] += payload.nbytes
            log.append(("RS", t, src, dst, c, payload))

    # Phase 2: all-gather.  Step t: rank r sends chunk (r + 1 - t) mod N.
    for t in range(n - 1):
        messages = []
        for r in range(n):
            c = (r + ag_start_offset - t) % n
            lo, hi = bounds[c]
            messages.append((r, (r + 1) % n, c, data[r][lo:hi].copy()))
        for src, dst, c, payload in messages:
            lo, hi = bounds[c]
            data[dst][lo:hi] = payload
            sent[src] += payload.nbytes
            log.append(("AG", t, src, dst, c, payload))

    return data, sent, log


def ring_reduce_scatter(arrays):
    """Only the reduce-scatter phase.

    Returns ``(owned, sent)`` where ``owned[r] = (chunk, values)`` is the chunk
    rank r holds fully summed after N - 1 steps, read from rank r's own
    buffer, and ``sent[r]`` is the bytes rank r sent in the phase.
    """
    n = len(arrays)
    data = [np.array(a, copy=True) for a in arrays]
    bounds = chunk_bounds(data[0].shape[0], n)
    sent = [0] * n
    for t in range(n - 1):
        messages = []
        for r in range(n):
            c = (r - t) % n
            lo, hi = bounds[c]
            messages.append((r, (r + 1) % n, c, data[r][lo:hi].copy()))
        for src, dst, c, payload in messages:
            lo, hi = bounds[c]
            data[dst][lo:hi] = data[dst][lo:hi] + payload
            sent[src] += payload.nbytes
    owned = []
    for r in range(n):
        c = (r + 1) % n
        lo, hi = bounds[c]
        owned.append((c, data[r][lo:hi].copy()))
    return owned, sent


def naive_gather_receive_bytes(nbytes, nranks):
    """Bytes rank 0 receives when it gathers every vector and broadcasts back.

    s.1 of "Lab 09": rank 0 receives (N - 1) * S.
    """
    return (nranks - 1) * nbytes
