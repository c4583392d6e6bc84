"""CPU model of the work-queue protocol of attn_fwd_queued_kernel
(ba_att_forward_queued), run under random interleavings of the workgroups.

The model takes the kernel's steps as its source states them: each
workgroup's thread 0 draws tickets from its own XCD's counter and then from
the other XCDs' counters (nearest first), dropping a counter once a ticket
lands past that XCD's range; a workgroup leaves when every counter it tried
is exhausted, counts itself out on word 8, and the last one out stores zeros
back.  Every atomic is one indivisible step; workgroups interleave at random
between steps.  It checks what the kernel relies on: every tile is taken
exactly once, every workgroup leaves after finitely many steps, the queue is
zero again afterwards (so a second launch on it sees every tile), and a
queue that does not start at zero still ends (with stale tickets, tiles are
skipped; with a stale leaver count, the queue is cleared early and tiles are
drawn again: results undefined, as the header states, but no hang)."""

import random

import pytest

N_XCD = 8


class QueueModel:
    def __init__(self, total: int, grid: int, queue=None):
        self.total, self.grid = total, grid
        self.per = (total + N_XCD - 1) // N_XCD
        self.q = list(queue) if queue is not None else [0] * 16
        self.taken = []

    def workgroup(self, w: int):
        """One workgroup as a generator: yields after each atomic step."""
        xcd = w % N_XCD
        open_mask = (1 << N_XCD) - 1
        while True:
            t = -1
            for i in range(N_XCD):
                if t >= 0:
                    break
                y = (xcd + i) % N_XCD
                if not (open_mask >> y) & 1:
                    continue
                lo = y * self.per
                length = min(self.per, self.total - lo)
                if length > 0:
                    ticket = self.q[y]          # atomicAdd(&queue[y], 1)
                    self.q[y] = (ticket + 1) & 0xFFFFFFFF
                    yield
                else:
                    ticket = 0xFFFFFFFF
                if length > 0 and ticket < length:
                    t = lo + ticket
                else:
                    open_mask &= ~(1 << y)
            if t < 0:
                break
            self.taken.append(t)                # the tile body
            yield
        left = self.q[N_XCD]                    # atomic add on the leaver count
        self.q[N_XCD] = left + 1
        yield
        if left == self.grid - 1:
            for i in range(N_XCD + 1):
                self.q[i] = 0
        yield


def run(model: QueueModel, seed: int, max_steps: int = 10 ** 6) -> int:
    rng = random.Random(seed)
    live = {w: model.workgroup(w) for w in range(model.grid)}
    steps = 0
    while live:
        w = rng.choice(list(live))
        try:
            next(live[w])
        except StopIteration:
            del live[w]
        steps += 1
        assert steps < max_steps, "a workgroup did not leave"
    return steps


@pytest.mark.parametrize("total,grid", [(1, 8), (3, 8), (36, 768), (2048, 768), (16384, 768), (777, 16),
                                        (8, 8), (9, 8), (100, 24)])
def test_every_tile_once_and_the_queue_returns_to_zero(total, grid):
    m = QueueModel(total, grid)
    for launch in range(2):                     # a second launch on the same queue
        m.taken = []
        run(m, seed=total * 7 + grid + launch)
        assert sorted(m.taken) == list(range(total))
        assert m.q == [0] * 16


def test_random_interleavings():
    rng = random.Random(5)
    for seed in range(40):
        total = rng.randint(1, 400)
        grid = 8 * rng.randint(1, 12)
        m = QueueModel(total, grid)
        run(m, seed)
        assert sorted(m.taken) == list(range(total))
        assert m.q == [0] * 16


def test_stale_tickets_end_the_launch_and_skip_tiles():
    total, grid = 500, 64
    stale = [3, 1000, 0, 70, 2, 0, 64, 9] + [0] * 8
    m = QueueModel(total, grid, queue=stale)
    run(m, seed=11)
    assert len(m.taken) == len(set(m.taken))    # no tile twice
    assert len(m.taken) < total                 # the stale tickets' tiles are skipped
    assert m.q == [0] * 16                      # the last workgroup out still clears it


@pytest.mark.parametrize("seed", range(10))
def test_a_stale_leaver_count_still_ends_the_launch(seed):
    """A leaver count not at zero makes some workgroup see itself last
    while others still run: it clears the queue early and tiles are drawn
    again (results undefined, as the header states), but every workgroup
    still leaves: no draw waits on another workgroup."""
    total, grid = 300, 32
    m = QueueModel(total, grid, queue=[0] * 8 + [5] + [0] * 7)
    steps = run(m, seed)
    assert set(m.taken) == set(range(total))    # every tile at least once
    assert steps < 20 * (total + grid) * N_XCD  # and a bounded number of steps
