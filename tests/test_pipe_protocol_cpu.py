"""A CPU model of the LDS hand-over of the 16-token chunk kernel
(csrc/kda_chunk_pipe.hip): eight producer waves (chunk ci goes to producer
ci % 8) and four consumer waves share a ring of R slots through per-slot
"ready" counters and per-slot, per-consumer "released" counters, plus one
triangular-solve scratch per slot.  Every wave runs its own program of LDS
operations in order (the LDS serves each wave's operations in order); the
model interleaves the waves at random, one operation at a time, and checks
after every step that

* a consumer reads a slot only while it holds the chunk the consumer wants,
  completely written (tiles and M' and beta);
* a producer writes a slot only after every consumer has released the chunk
  it held, and the scratch of a slot is never shared by two chunks at once;
* every chunk is consumed by every consumer, in order, and nobody waits
  forever (the run ends).

The consumer reads the next slot's counter early (before releasing the
current slot) and trusts a value already at the target, as the kernel does.
Ring sizes 4 .. 12 are checked, also those that do not divide the producer
count (a producer then changes slots from one chunk to the next)."""
import random

import pytest

NP, NC = 8, 4


def run(R, nch, seed, max_steps=2_000_000):
    rng = random.Random(seed)
    ready = [0] * R
    released = [[0] * NC for _ in range(R)]
    slot = [None] * R            # (chunk, parts written) of each slot
    scratch = [None] * R         # chunk whose -N columns the scratch holds
    consumed = [[] for _ in range(NC)]

    def producer(p):
        for ci in range(p, nch, NP):
            s, rnd = ci % R, ci // R
            # poll the four release counters until all reach the round
            while True:
                seen = []
                for c in range(NC):
                    seen.append(released[s][c])
                    yield
                if min(seen) >= rnd:
                    break
            # the slot must no longer be read by anyone
            assert all(released[s][c] >= rnd for c in range(NC)), (ci, s)
            assert slot[s] is None or slot[s][0] == ci - R, (ci, slot[s])
            slot[s] = (ci, 0)
            yield
            for part in range(1, 4):           # -Kt, Qt, Ki, V ... then A_qk
                slot[s] = (ci, part)
                yield
            # the triangular solve through this slot's scratch
            assert scratch[s] is None or scratch[s] < ci, (ci, scratch[s])
            scratch[s] = ci
            yield
            assert scratch[s] == ci, (ci, scratch[s])
            slot[s] = (ci, 4)                  # M' written
            yield
            ready[s] = rnd + 1                 # publish
            yield

    def consumer(w):
        def wait_ready(ci):
            s = ci % R
            while ready[s] < ci // R + 1:
                yield
        yield from wait_ready(0)
        for ci in range(nch):
            s = ci % R
            assert slot[s] == (ci, 4), (w, ci, slot[s])
            yield                                  # read the slot's operands
            assert slot[s] == (ci, 4), (w, ci, slot[s])
            cn = ci + 1
            peek = ready[cn % R] if cn < nch else None   # read early
            yield
            consumed[w].append(ci)
            released[s][w] = ci // R + 1           # release after the reads
            yield
            if cn < nch and not (peek >= cn // R + 1):
                yield from wait_ready(cn)

    waves = [producer(p) for p in range(NP)] + [consumer(w) for w in range(NC)]
    live = list(range(len(waves)))
    steps = 0
    while live:
        i = rng.choice(live)
        try:
            next(waves[i])
        except StopIteration:
            live.remove(i)
        steps += 1
        assert steps < max_steps, "no progress (a wait never ends)"
    assert all(c == list(range(nch)) for c in consumed)


@pytest.mark.parametrize("R", [4, 6, 8, 9, 10, 12])
def test_hand_over_protocol_any_interleaving(R):
    for seed in range(200):
        run(R, nch=3 * R + 11, seed=seed)


def test_model_catches_a_release_before_the_reads():
    """The model is not vacuous: a consumer that releases its slot before
    reading it is caught (a producer overwrites the slot under it)."""
    R, nch = 8, 40

    def broken(seed):
        rng = random.Random(seed)
        ready = [0] * R
        released = [[0] * NC for _ in range(R)]
        slot = [None] * R

        def producer(p):
            for ci in range(p, nch, NP):
                s, rnd = ci % R, ci // R
                while min(released[s]) < rnd:
                    yield
                slot[s] = (ci, 0)
                yield
                slot[s] = (ci, 4)
                ready[s] = rnd + 1
                yield

        def consumer(w):
            for ci in range(nch):
                s = ci % R
                while ready[s] < ci // R + 1:
                    yield
                released[s][w] = ci // R + 1       # released too early
                yield
                yield
                assert slot[s] == (ci, 4), (w, ci, slot[s])

        waves = [producer(p) for p in range(NP)] + [consumer(w) for w in range(NC)]
        live = list(range(len(waves)))
        while live:
            i = rng.choice(live)
            try:
                next(waves[i])
            except StopIteration:
                live.remove(i)

    with pytest.raises(AssertionError):
        for seed in range(200):
            broken(seed)
