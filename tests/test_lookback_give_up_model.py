"""Host model of the chunked forward path's look-back and of what a wait that
gives up leaves behind (forward_chunked_kernel and look_back in
csrc/wkv_forward.hip).

Tiles of one column group run in ticket order.  Tile j publishes its
aggregate (unless it is the first), looks back over tiles j-1, j-2, ...
combining published aggregates until it meets an inclusive prefix, publishes
its own inclusive prefix (unless it is the last) and writes its outputs from
the exclusive prefix.  Each wait for a flag is bounded; one that runs out, or
that sees the shared error word already set, gives up: the error word is set,
the failure is counted, and the carry becomes NaN.

The model stands in for the state with a scalar that combines by addition (the
look-back's correctness only needs an associative combine) and checks, over
random schedules: without a stall every tile's prefix is exact; with one tile
that stalls before publishing, the run still ends, the error word is set and
counted, every tile after the stalled one is NaN, and every tile before it is
exact or NaN (never a finite wrong value).  CPU only.
"""
import math
import random

import pytest

EMPTY, AGGREGATE, INCLUSIVE = 0, 1, 2


def run(ntiles, rng, stall=None, patience=3):
    """Simulate the tiles with a random interleaving.  `stall`: a tile that
    never publishes anything (its wave is stuck before it), or None.
    `patience`: polls a wait makes before giving up."""
    vals = [rng.uniform(0.5, 2.0) for _ in range(ntiles)]
    flags = [EMPTY] * ntiles
    desc = [[None, None] for _ in range(ntiles)]       # aggregate, inclusive
    shared = {"error": 0, "failures": 0}
    out = [None] * ntiles

    def tile(j):
        if j == stall:
            return
        if j > 0 and j < ntiles - 1:
            desc[j][0] = vals[j]
            flags[j] = AGGREGATE
            yield
        if j == 0:
            x = 0.0
        else:
            sfx = 0.0
            jj = j - 1
            while True:
                polls = 0
                while flags[jj] == EMPTY:
                    if shared["error"] or polls >= patience:
                        break
                    polls += 1
                    yield
                if flags[jj] == EMPTY:
                    # give up: recorded, and the carry is poisoned
                    shared["error"] = 1
                    shared["failures"] += 1
                    x = math.nan
                    break
                kind = 1 if flags[jj] == INCLUSIVE else 0
                d = desc[jj][kind] + sfx
                if kind == 1:
                    x = d
                    break
                sfx = d
                jj -= 1
        if j < ntiles - 1:
            desc[j][1] = x + vals[j]
            flags[j] = INCLUSIVE
            yield
        out[j] = x                                       # exclusive prefix of tile j

    # tiles start in ticket order, then interleave at random
    live = []
    for j in range(ntiles):
        live.append(tile(j))
        # a few random steps of the started tiles before the next one starts
        for _ in range(rng.randrange(3)):
            if live:
                g = rng.choice(live)
                try:
                    next(g)
                except StopIteration:
                    live.remove(g)
    while live:
        g = rng.choice(live)
        try:
            next(g)
        except StopIteration:
            live.remove(g)
    return vals, out, shared


@pytest.mark.parametrize("seed", range(40))
def test_look_back_prefixes_without_a_stall(seed):
    rng = random.Random(seed)
    n = rng.randrange(2, 12)
    vals, out, shared = run(n, rng, patience=10 ** 9)
    assert shared == {"error": 0, "failures": 0}
    for j in range(n):
        assert out[j] == pytest.approx(sum(vals[:j]))


@pytest.mark.parametrize("seed", range(60))
def test_a_give_up_is_never_silent(seed):
    rng = random.Random(1000 + seed)
    n = rng.randrange(3, 12)
    stall = rng.randrange(0, n - 1)
    vals, out, shared = run(n, rng, stall=stall, patience=rng.randrange(1, 4))
    # the run ends (run() returned), and the miss is recorded
    assert shared["error"] == 1 and shared["failures"] >= 1
    # tiles before the stalled one do not need it: exact, or NaN when they
    # were still waiting once the error word was set (they then give up at
    # once, so the kernel ends) -- never a finite wrong value
    for j in range(stall):
        assert math.isnan(out[j]) or out[j] == pytest.approx(sum(vals[:j]))
    assert out[stall] is None                     # the stalled tile wrote nothing
    # every tile after it depends on it: NaN, never a finite wrong value
    for j in range(stall + 1, n):
        assert math.isnan(out[j]), (stall, j, out[j])


def test_model_sees_silent_continuation():
    """The check above fails for the old behaviour, which continued a give-up
    with the partial suffix it had combined so far."""
    import types
    src = open(__file__).read()
    old = "                    x = math.nan\n"
    assert src.count(old) == 1
    mod = types.ModuleType("lookback_old")
    exec(compile(src.replace(old, "                    x = sfx\n"), "<old look-back>", "exec"),
         mod.__dict__)
    rng = random.Random(7)
    silent = 0
    for _ in range(50):
        n = rng.randrange(3, 12)
        stall = rng.randrange(0, n - 1)
        _, out, _ = mod.run(n, rng, stall=stall, patience=1)
        silent += sum(1 for j in range(stall + 1, n) if out[j] is not None and not math.isnan(out[j]))
    assert silent > 0
