"""Host model of the hand-over in mat_forward_ring_kernel (csrc/wkv_mat.hip).

Four producer waves and four consumer waves share a ring of six LDS slots
(chunk q in slot q mod 6).  Producer p prepares chunks p, p + 4, ...: it
waits until the slot's `done` count reaches 4 * (q / 6) (the consumers are
through the slot's previous chunk, six back), writes that chunk's y tile out
of the slot (unless it ran token by token), writes the new operands and the
chunk's form flag, and publishes `ready`.  After its chunks it waits for the
consumers once more on each slot s = p, p + 4, ... below six and writes the
tile of that slot's last chunk.  The consumer waves take the chunks in pairs, each waiting for `ready`,
reading the operands, writing its quarter of the y tile (or y itself for a
token-by-token chunk) and counting itself in `done`.

The model runs every wave's steps in random interleavings and checks that no
schedule deadlocks, that every operand read sees its own chunk, that a y tile
is written out only once all four consumer waves have filled it in and before
the next chunk in the slot overwrites it, and that every chunk's y is written
exactly once.  CPU only.
"""
import random

import pytest

SLOTS = 6
WAVES = 4


class Ring:
    def __init__(self, nch, exact):
        self.nch = nch
        self.exact_of = exact                     # chunk -> runs token by token
        self.ready = [-1] * SLOTS
        self.done = [0] * SLOTS
        self.exact = [0] * SLOTS
        self.operands = [None] * SLOTS            # chunk whose operands the slot holds
        self.tile = [None] * SLOTS                # (chunk, set of consumer waves that wrote)
        self.y_written = {}                       # chunk -> times its y was written out

    def write_y(self, q):
        self.y_written[q] = self.y_written.get(q, 0) + 1

    def store_tile(self, s, q):
        """A producer writes chunk q's tile out of slot s (when it ran on the
        matrix cores)."""
        if self.exact[s]:
            return
        chunk, parts = self.tile[s]
        assert chunk == q and parts == set(range(WAVES)), (q, self.tile[s])
        self.write_y(q)


def producer(ring, p):
    """Generator of the producer's steps; yields a predicate while it waits."""
    q = p
    while q < ring.nch:
        s = q % SLOTS
        want = WAVES * (q // SLOTS)
        yield lambda s=s, want=want: ring.done[s] == want
        if q >= SLOTS:
            ring.store_tile(s, q - SLOTS)
        yield None
        ring.operands[s] = q
        yield None
        ring.exact[s] = 1 if ring.exact_of[q] else 0
        ring.ready[s] = q
        yield None
        q += WAVES
    for s in range(p, SLOTS, WAVES):
        if s < ring.nch:
            last = s + (ring.nch - 1 - s) // SLOTS * SLOTS
            want = WAVES * (last // SLOTS + 1)
            yield lambda s=s, want=want: ring.done[s] == want
            ring.store_tile(s, last)


def consumer(ring, w):
    for q in range(0, ring.nch, 2):
        pair = [c for c in (q, q + 1) if c < ring.nch]
        for c in pair:
            s = c % SLOTS
            yield lambda s=s, c=c: ring.ready[s] == c
        for c in pair:
            s = c % SLOTS
            assert ring.operands[s] == c, (w, c, ring.operands[s])
            yield None
            if ring.exact[s]:
                if w == 0:
                    ring.write_y(c)        # token by token: y goes out at once
            else:
                chunk, parts = ring.tile[s] if ring.tile[s] is not None else (None, set())
                if chunk != c:
                    # the slot's previous tile must be out before it is overwritten
                    if chunk is not None and not ring.exact_of[chunk]:
                        assert ring.y_written.get(chunk, 0) == 1, (c, chunk)
                    chunk, parts = c, set()
                parts = parts | {w}
                ring.tile[s] = (chunk, parts)
            yield None
        for c in pair:
            ring.done[c % SLOTS] += 1
            yield None


def run(nch, exact, rng):
    ring = Ring(nch, exact)
    threads = [producer(ring, p) for p in range(WAVES)] + [consumer(ring, w) for w in range(WAVES)]
    waiting = [None] * len(threads)      # predicate a thread is blocked on
    alive = set(range(len(threads)))
    while alive:
        runnable = [i for i in alive if waiting[i] is None or waiting[i]()]
        assert runnable, f"deadlock with nch={nch}"
        i = rng.choice(runnable)
        try:
            waiting[i] = next(threads[i])
        except StopIteration:
            alive.discard(i)
    assert ring.y_written == {q: 1 for q in range(nch)}, ring.y_written


@pytest.mark.parametrize("nch", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 11, 12, 13, 16, 25])
def test_ring_hand_over_random_schedules(nch):
    rng = random.Random(1000 + nch)
    for trial in range(60):
        exact = {q: rng.random() < 0.2 for q in range(nch)}
        run(nch, exact, rng)


def test_ring_model_catches_an_early_release():
    """The model is not vacuous: a producer that waits for one completion too
    few overwrites a slot its consumers still read."""
    def early_producer(ring, p):
        q = p
        while q < ring.nch:
            s = q % SLOTS
            want = max(0, WAVES * (q // SLOTS) - 1)
            yield lambda s=s, want=want: ring.done[s] >= want
            ring.operands[s] = q
            ring.exact[s] = 1
            ring.ready[s] = q
            yield None
            q += WAVES

    rng = random.Random(7)
    caught = False
    for trial in range(200):
        ring = Ring(12, {q: True for q in range(12)})
        threads = [early_producer(ring, p) for p in range(WAVES)] + [consumer(ring, w) for w in range(WAVES)]
        waiting = [None] * len(threads)
        alive = set(range(len(threads)))
        try:
            while alive:
                runnable = [i for i in alive if waiting[i] is None or waiting[i]()]
                if not runnable:
                    break
                i = rng.choice(runnable)
                try:
                    waiting[i] = next(threads[i])
                except StopIteration:
                    alive.discard(i)
        except AssertionError:
            caught = True
            break
    assert caught
