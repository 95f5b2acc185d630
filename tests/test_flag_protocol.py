"""CPU model of the readiness protocol of the one-launch bf16 prefill
(`csrc/kda_prefill_bf16.hip`).

Prep blocks publish the record of each (chunk slot, head) by setting its
flag, in whatever order the blocks run; a state task may load a chunk's
record only once its flag is seen.  The task does not poll every chunk: it
keeps `upto`, the last chunk known to be published with every earlier one,
and when a step needs chunk c beyond it, its 16 lanes read the flags of
chunks upto + 1 ... upto + 16 (clamped to the last chunk) and `upto` moves to
the end of the published run that starts right after it, until it reaches c.
Steps check ahead by a schedule fixed at compile time: the prologue checks
chunks 0 .. NB - 1, steps 1 .. 11 of each twelve-step loop iteration check
the chunk their loads need (c + NB - 1), the last one a chunk further for the
first step of the next iteration, which checks nothing, and the tail steps
check their own.

These tests replay that schedule against prep blocks that publish in random
order, interleaved lane by lane with the polls, and check that every record
load finds its record published; a copy of the poll that starts its window
at c instead of right after `upto` (a mistake once made in the kernel) must
be caught.  A second model checks the progress argument of the bounded prep
lead: with blocks dispatched in slot order into a few slots, prep items that
wait for the pass to consume the chunk `lead` behind them never stall it.
"""
import os
import random
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "gated_delta_rule_88_amd", "csrc", "kda_prefill_bf16.hip")
LANES = 16


def schedule(nch, nb):
    """(kind, chunk) events of one state task, in program order: "need"
    (a readiness check) and "load" (the record loads of a step)."""
    ev = []
    if nch > 0:
        ev += [("need", 0), ("load", 0)]
        if nb == 3:
            ev += [("need", 1), ("load", 1)]
        ev.append(("need", nb - 1))
    c0 = 0
    while c0 + 12 <= nch:
        for u in range(12):
            c = c0 + u
            if u > 0:
                ev.append(("need", c + nb - 1 + (1 if u == 11 else 0)))
            ev.append(("load", c + nb - 1))
        c0 += 12
    for c in range(c0, nch):
        ev += [("need", c + nb - 1), ("load", c + nb - 1)]
    return ev


class Prep:
    """Records published one at a time, each tick with probability `rate`,
    in an order that is random within a window of `spread` chunks (the prep
    runs roughly in slot order, its blocks finishing out of order)."""

    def __init__(self, nch, rng, rate, spread=6):
        keys = [c + rng.uniform(0, spread) for c in range(nch)]
        self.order = sorted(range(nch), key=lambda c: -keys[c])
        self.published = [False] * nch
        self.rng = rng
        self.rate = rate

    def tick(self, p=None):
        if self.order and self.rng.random() < (self.rate if p is None else p):
            self.published[self.order.pop()] = True

    def read(self, c):
        self.tick()
        return self.published[c]


def need_record(prep, nch, c, st, window_at_c=False):
    """The task's poll.  st["upto"]: last chunk known to be published, every
    earlier one included."""
    if c <= st["upto"]:
        return
    while True:
        first = c if window_at_c else st["upto"] + 1
        ready = [prep.read(min(first + i, nch - 1)) for i in range(LANES)]
        run = next((i for i, r in enumerate(ready) if not r), LANES)
        st["upto"] = max(st["upto"], first + run - 1)
        if st["upto"] >= c:
            return
        for _ in range(4):   # the wave sleeps; other blocks publish meanwhile
            prep.tick()


def run_task(nch, nb, seed, window_at_c=False, rate=0.05):
    """Replay one state task; returns the loads that found their record
    unpublished.  With a low publication rate the task runs at the prep's
    frontier, where the order of publication matters."""
    rng = random.Random(seed)
    prep = Prep(nch, rng, rate)
    st = {"upto": -1}
    bad = []
    for kind, c in schedule(nch, nb):
        if kind == "need":
            need_record(prep, nch, c, st, window_at_c)
        else:
            rec = min(c, nch - 1)   # past the end the last record is loaded again
            if not prep.published[rec]:
                bad.append(rec)
            assert st["upto"] >= rec or bad, "a load the schedule never checked"
        prep.tick()
    return bad


def test_the_schedule_checks_every_record_before_it_is_loaded():
    for nb in (2, 3):
        for nch in (1, 2, 3, 11, 12, 13, 14, 23, 24, 25, 36, 37, 50):
            loads = [c for k, c in schedule(nch, nb) if k == "load"]
            # one load per step, in chunk order, NB - 1 ahead
            assert loads[: nb - 1] == list(range(nb - 1))[: len(loads)]
            assert len(loads) == nch + nb - 1 - (nb - 1 if nch == 0 else 0)
            st = {"upto": -1}
            for kind, c in schedule(nch, nb):   # every load covered by an earlier check
                if kind == "need":
                    st["upto"] = max(st["upto"], c)
                else:
                    assert st["upto"] >= c, (nb, nch, c)


@pytest.mark.parametrize("nb", [2, 3])
def test_no_record_is_loaded_before_it_is_published(nb):
    for rate in (0.02, 0.05, 0.3, 1.0):
        for nch in (1, 5, 12, 13, 24, 29, 40):
            for seed in range(40):
                assert run_task(nch, nb, 1000 * nch + seed, rate=rate) == [], (nb, nch, seed, rate)


@pytest.mark.parametrize("nb", [2, 3])
def test_a_poll_window_starting_at_the_needed_chunk_is_caught(nb):
    # chunks are published out of order: a published run starting at c says
    # nothing of the chunks between upto and c
    caught = sum(bool(run_task(nch, nb, seed, window_at_c=True)) for nch in (13, 24, 40) for seed in range(60))
    assert caught > 0


def lead_model(nchunks, lead, nb, slots, seed):
    """Discrete-time model of one head: the state task holds its own block
    from the start; prep items are dispatched in chunk order into `slots`
    free slots and each, if its chunk is `lead` or more past the start, first
    waits (in its slot) until the task has consumed the chunk `lead` behind
    it; an item then takes one to three ticks and publishes.  The task's step
    c needs records c .. c + nb - 1 (clamped) and then marks c consumed.
    Returns the tick at which the task finished, or None on a stall."""
    rng = random.Random(seed)
    published = [False] * nchunks
    consumed = [False] * nchunks
    running = []          # [chunk, ticks left or None while waiting]
    nxt = 0
    c = 0
    for t in range(100 * nchunks + 100):
        while nxt < nchunks and len(running) < slots:
            running.append([nxt, None])
            nxt += 1
        for item in running:
            ch = item[0]
            if item[1] is None and (ch < lead or consumed[ch - lead]):
                item[1] = rng.randint(1, 3)
            elif item[1] is not None:
                item[1] -= 1
                if item[1] == 0:
                    published[ch] = True
        running = [it for it in running if not published[it[0]]]
        if c < nchunks and all(published[x] for x in range(c, min(c + nb, nchunks))):
            consumed[c] = True
            c += 1
        if c == nchunks:
            return t
    return None


def test_bounded_prep_lead_never_stalls_the_pass():
    text = open(SRC).read()
    lead = int(re.search(r"#define KDA_LEAD_CHUNKS (\d+)", text).group(1))
    for nb in (2, 3):
        assert lead >= nb   # the chunks a pass step needs come from items dispatched earlier
        for slots in (1, 2, 5, 40):
            for seed in range(10):
                assert lead_model(3 * lead + 7, lead, nb, slots, seed) is not None, (nb, slots, seed)
                # and so for any lead the argument allows
                assert lead_model(40, nb, nb, slots, seed) is not None, (nb, slots, seed)


def test_a_lead_shorter_than_the_pass_lookahead_can_stall():
    # lead < nb: the item of chunk c waits for chunk c - lead, whose step needs
    # chunk c itself -- with one slot nothing moves
    assert lead_model(20, 1, 2, 1, 0) is None
