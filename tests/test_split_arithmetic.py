"""The index arithmetic of the balanced decode split, checked on the CPU by brute force.

The decode kernel lays the requests' blocks end to end (T blocks) and gives worker w
of W = min(workers, T) the blocks [w*T/W, (w+1)*T/W). A worker cuts its range at
request boundaries into segments; a segment that is not a whole request stores its
partial in slot (request + worker). The merge finds a request's partials from its
block range alone: workers worker_of(c0) .. worker_of(c1 - 1), slot (request +
worker). When requests outnumber workers, each worker records the request whose
first cut between workers falls at the start of its range, and the merge runs over
those records only. This file restates those formulas (as the kernels compute them)
and checks them against plain enumeration: ranges partition the blocks and none is
empty, worker_of names the owner of every block, slots never collide, the merge
reads exactly the slots the segments wrote, and every split request is recorded
exactly once.
"""
import numpy as np
import pytest


def worker_of(b, T, W):
    """Worker holding global block b (as the kernels compute it)."""
    return ((b + 1) * W + T - 1) // T - 1


def split(blocks, workers):
    """Segments and split-request records of one call, enumerated directly."""
    blocks = np.asarray(blocks, dtype=np.int64)
    cum = np.concatenate([[0], np.cumsum(blocks)])
    T = int(cum[-1])
    W = min(workers, T)
    ranges = [(w * T // W, (w + 1) * T // W) for w in range(W)]
    segments = []  # (request, worker, first block, end block)
    for w, (lo, hi) in enumerate(ranges):
        for s in range(len(blocks)):
            a, b = max(lo, int(cum[s])), min(hi, int(cum[s + 1]))
            if a < b:
                segments.append((s, w, a, b))
    records = []
    for w, (lo, hi) in enumerate(ranges):
        first = int(np.searchsorted(cum[1:], lo, side="right"))  # first request whose blocks pass lo
        rec = first if (lo > cum[first] and worker_of(int(cum[first]), T, W) == w - 1) else -1
        records.append(rec)
    return cum, T, W, ranges, segments, records + [-1] * (workers - W)


CASES = [([3, 1, 4, 1, 5, 9, 2, 6], 3), ([1] * 50, 7), ([100], 256), ([5, 0, 7, 0, 0, 9], 4),
         ([2, 2, 2, 2], 8), ([0, 0, 0], 5), ([1, 700, 2, 3, 900, 1], 16)]


def random_cases(n=200):
    rng = np.random.default_rng(11)
    for _ in range(n):
        S = int(rng.integers(1, 80))
        blocks = rng.integers(0, 40, S)
        blocks[rng.random(S) < 0.05] = 0  # some empty requests
        if rng.random() < 0.3:
            blocks[rng.integers(0, S)] = int(rng.integers(100, 600))  # one long request
        yield blocks.tolist(), int(rng.integers(1, 300))


@pytest.mark.parametrize("blocks,workers", CASES + list(random_cases()))
def test_balanced_split_arithmetic(blocks, workers):
    cum, T, W, ranges, segments, records = split(blocks, workers)
    if T == 0:
        assert not segments and all(r == -1 for r in records)
        return
    # ranges partition [0, T) and none is empty (W <= T)
    assert ranges[0][0] == 0 and ranges[-1][1] == T
    assert all(lo < hi for lo, hi in ranges)
    assert all(ranges[i][1] == ranges[i + 1][0] for i in range(W - 1))
    # worker_of names the owner of every block
    owner = np.repeat(np.arange(W), [hi - lo for lo, hi in ranges])
    assert all(worker_of(b, T, W) == owner[b] for b in range(T))
    # slots (request + worker) strictly increase along the block axis: unique
    slots = [s + w for s, w, _, _ in segments]
    assert all(slots[i] < slots[i + 1] for i in range(len(slots) - 1))
    assert max(slots) < len(blocks) + W  # within the workspace's S + W rows
    # the merge reads exactly the slots the request's segments wrote
    for s in range(len(blocks)):
        c0, c1 = int(cum[s]), int(cum[s + 1])
        mine = [(w, s + w) for r, w, _, _ in segments if r == s]
        if c1 == c0:
            assert not mine
            continue
        w0, w1 = worker_of(c0, T, W), worker_of(c1 - 1, T, W)
        assert [w for w, _ in mine] == list(range(w0, w1 + 1))
        assert [slot for _, slot in mine] == [s + w0 + i for i in range(w1 - w0 + 1)]
    # every request with more than one segment is recorded exactly once, no other
    split_requests = sorted(s for s in range(len(blocks))
                            if sum(1 for r, *_ in segments if r == s) > 1)
    recorded = [r for r in records if r >= 0]
    assert sorted(recorded) == split_requests
    assert len(records) == workers
