"""Host model of the query-tile kernel's LDS ring protocol (no GPU).

The kernel's waves meet at no barrier in its pair loop: they synchronise
through per-slot release counts, per-slot landed-load counts and a job word
(csrc/attn.hip, attn_gqa_tile_kernel).  This model runs the same rules as a
set of interleaved state machines under random schedules and checks what the
kernel relies on: every wave finishes (no wait lasts forever), a slot is never
overwritten while a wave may still read it, a wave never computes on a pair
whose loads have not all landed, and every load job is issued exactly once.
"""
import random

import pytest

RING, JOBS = 4, 2


def run_model(n_waves, active, seed, slot_rule=True, max_steps=10 ** 6):
    """active[w][u]: wave w computes pair u.  Returns the number of scheduler
    steps taken; raises AssertionError on a protocol violation.  slot_rule
    False drops the slot checks (entering pair u and claiming its loads before
    every wave released pair u - RING), to show that the model detects it."""
    rng = random.Random(seed)
    n_pairs = len(active[0])
    rel = [0] * RING          # releases per slot, over all its pairs
    rdy = [0] * RING          # landed jobs per slot, over all its pairs
    job = [0]                 # the next job to claim
    slot_pair = [None] * RING  # the pair whose rows the slot holds (None while a load is in flight)
    readers = [set() for _ in range(RING)]
    issued = []
    # wave state: (pc, u, pending job or None)
    st = [{"u": 0, "pc": "enter", "job": None, "landed_at": 0} for _ in range(n_waves)]
    t = 0

    def try_claim(w):
        j = job[0]
        pj = j // JOBS
        if pj >= n_pairs:
            return False
        if slot_rule and pj >= RING and rel[pj % RING] < n_waves * (pj // RING):
            return False
        job[0] = j + 1      # the compare-and-swap succeeds (one claimer at a time)
        s = pj % RING
        assert not readers[s], "a load into a slot that a wave still reads"
        issued.append(j)
        st[w]["job"] = j
        st[w]["landed_at"] = t + rng.randint(1, 20)
        return True

    steps = 0
    while any(x["pc"] != "done" for x in st):
        steps += 1
        assert steps < max_steps, "no progress: a wait never ends"
        t += 1
        w = rng.randrange(n_waves)
        x = st[w]
        if x["pc"] == "done":
            continue
        if x["job"] is not None:            # a claimed job: wait for it, then count it
            if t >= x["landed_at"]:
                j = x["job"]
                s = (j // JOBS) % RING
                rdy[s] += 1
                if rdy[s] % JOBS == 0:
                    slot_pair[s] = j // JOBS
                x["job"] = None
            continue
        u = x["u"]
        if u >= n_pairs:
            x["pc"] = "done"
            continue
        s, gen = u % RING, u // RING
        if x["pc"] == "enter":
            if slot_rule and u >= RING and rel[s] < n_waves * gen:
                try_claim(w)
                continue
            x["pc"] = "loads" if active[w][u] else "release"
            continue
        if x["pc"] == "loads":
            if rdy[s] < JOBS * (gen + 1):
                try_claim(w)
                continue
            assert slot_pair[s] == u, "computing on a slot that does not hold the pair"
            readers[s].add(w)
            x["pc"] = "compute"
            continue
        if x["pc"] == "compute":
            readers[s].discard(w)
            x["pc"] = "release"
            continue
        if x["pc"] == "release":
            rel[s] += 1
            x["u"] = u + 1
            x["pc"] = "enter"
    assert sorted(issued) == list(range(JOBS * n_pairs)), "every job issued exactly once"
    assert rel == [n_waves * ((n_pairs - s + RING - 1) // RING) for s in range(RING)]
    return steps


@pytest.mark.parametrize("n_pairs", [1, 2, 3, 5, 17, 40])
@pytest.mark.parametrize("density", [0.1, 0.46, 1.0])
def test_ring_protocol_finishes_and_never_overwrites(n_pairs, density):
    for seed in range(6):
        rng = random.Random(1000 * seed + n_pairs)
        n_waves = 16
        active = [[rng.random() < density for _ in range(n_pairs)] for _ in range(n_waves)]
        for u in range(n_pairs):   # every pair is needed by some wave (the kernel lists needed tiles only)
            if not any(active[w][u] for w in range(n_waves)):
                active[rng.randrange(n_waves)][u] = True
        run_model(n_waves, active, seed)


def test_ring_protocol_model_catches_a_missing_slot_wait():
    # the model is not vacuous: without the slot rule a fast wave's loads land
    # in a slot that a slower wave still reads (or a wave computes on a slot
    # that holds another pair), which the model reports for some schedule
    caught = 0
    for seed in range(20):
        rng = random.Random(seed)
        active = [[rng.random() < 0.46 for _ in range(24)] for _ in range(16)]
        for u in range(24):
            if not any(a[u] for a in active):
                active[0][u] = True
        try:
            run_model(16, active, seed, slot_rule=False, max_steps=10 ** 5)
        except AssertionError:
            caught += 1
    assert caught > 0
