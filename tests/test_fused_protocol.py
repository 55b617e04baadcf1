"""The fused launch's scheduling protocol, simulated on the host over the
planner's real queues (muon_describe, kind MUON_KIND_FUSED).

A block claims the next entry of its XCD's queue (one iteration's tiles,
repeated T times), waits until its matrix's finished-tile counter reaches the
entry's target, runs it and counts it finished.  The targets are the kernel's:
    Gram t:   (t - 1) tot            poly t:   (t - 1) tot + ng
    update t: (t - 1) tot + ng + npl           (tot = ng + npl + nu)
The simulation runs every queue with a few resident blocks or many, and
random tile durations, and checks that
  * every queue drains (claims in queue order, waits on earlier entries only:
    no deadlock, whatever the number of resident blocks);
  * a tile starts only after every tile whose output it reads has finished
    (X_t for Gram and update, A for the polynomial, B for the update);
  * a tile that overwrites a buffer (A, B, or the X copy it writes) starts
    only after every reader of that buffer's previous contents has finished.
"""
import heapq
import random

import pytest

from muon_newton_schulz_03_amd import _lib, describe, inputs

GRAM, POLY, UPD = 1, 2, 3


def queues(shapes):
    d, q = describe(shapes, kind=_lib.KIND_FUSED, fused=True)
    per_xcd = {}
    for x, prod, i, ti, tj in q:
        per_xcd.setdefault(x, []).append((prod, i, ti, tj))
    counts = {}
    for lst in per_xcd.values():
        for prod, i, _, _ in lst:
            c = counts.setdefault(i, [0, 0, 0])
            c[prod - 1] += 1
    return per_xcd, counts


def target(counts, i, t, prod):
    ng, npl, nu = counts[i]
    return (t - 1) * (ng + npl + nu) + (ng if prod >= POLY else 0) + (npl if prod == UPD else 0)


def simulate(per_xcd, counts, T, resident, seed):
    """Discrete-event run of every XCD's queue; returns the (start, end) time of
    every (xcd, entry index)."""
    rng = random.Random(seed)
    times = {}
    for x, lst in per_xcd.items():
        total = len(lst) * T
        dep = {i: 0 for i in counts}
        head = 0
        clock = 0.0
        # blocks: each either holds a claimed entry waiting on its target, or runs one
        waiting = []   # (entry) claimed, not yet started
        running = []   # heap of (end time, entry)
        free = resident
        guard = 0
        while head < total or waiting or running:
            guard += 1
            assert guard < 10 * total + 100, f"XCD {x}: no progress (deadlock) with {resident} blocks"
            # free blocks claim in queue order
            while free and head < total:
                waiting.append(head)
                head += 1
                free -= 1
            # start every claimed entry whose target is met
            started = False
            for e in list(waiting):
                t = e // len(lst) + 1
                prod, i, _, _ = lst[e % len(lst)]
                if dep[i] >= target(counts, i, t, prod):
                    waiting.remove(e)
                    dur = rng.uniform(0.5, 2.0) * (4.0 if prod == GRAM else 1.0)
                    heapq.heappush(running, (clock + dur, e))
                    times[(x, e)] = [clock, None]
                    started = True
            if not running:
                assert started or not waiting, f"XCD {x}: claimed entries wait on nothing running (deadlock)"
                continue
            # finish the earliest running tile
            clock, e = heapq.heappop(running)
            times[(x, e)][1] = clock
            _, i, _, _ = lst[e % len(lst)]
            dep[i] += 1
            free += 1
    return times


def check_order(per_xcd, T, times):
    """Reads after writes and overwrites after reads, per matrix."""
    for x, lst in per_xcd.items():
        n = len(lst)
        ev = {}  # (matrix, t, prod) -> list of (start, end)
        for e in range(n * T):
            t = e // n + 1
            prod, i, _, _ = lst[e % n]
            ev.setdefault((i, t, prod), []).append(times[(x, e)])
        for (i, t, prod), spans in ev.items():
            first_start = min(s for s, _ in spans)
            # inputs finished: X_t (updates of t - 1), A (Grams of t), B (polys of t)
            deps = []
            if t > 1 and prod in (GRAM, UPD):
                deps.append((i, t - 1, UPD))
            if prod == POLY:
                deps.append((i, t, GRAM))
            if prod == UPD:
                deps.append((i, t, POLY))
            for d in deps:
                assert max(end for _, end in ev[d]) <= first_start, f"{(i, t, prod)} read {d} before it finished"
            # previous contents' readers finished before the overwrite
            prev_readers = []
            if prod == GRAM and t > 1:
                prev_readers.append((i, t - 1, POLY))           # A of t - 1
            if prod == POLY and t > 1:
                prev_readers.append((i, t - 1, UPD))            # B of t - 1
            if prod == UPD and t > 1:
                prev_readers += [(i, t - 1, GRAM), (i, t - 1, UPD)]  # X_{t-1}: the copy X_{t+1} reuses
            for d in prev_readers:
                assert max(end for _, end in ev[d]) <= first_start, f"{(i, t, prod)} overwrote what {d} reads"


SETS = {
    "gpt2_small": inputs.workload("gpt2_small").shapes,
    "mixed": [(300, 700), (700, 300), (129, 4100), (1000, 130), (64, 64), (256, 256), (512, 1536),
              (1536, 512), (384, 384)],
}


@pytest.mark.parametrize("name", sorted(SETS))
@pytest.mark.parametrize("resident", [1, 3, 64])
def test_fused_protocol_drains_and_orders(name, resident):
    per_xcd, counts = queues(SETS[name])
    for seed in range(3):
        times = simulate(per_xcd, counts, T=3, resident=resident, seed=seed)
        assert len(times) == 3 * sum(len(v) for v in per_xcd.values())
        assert all(end is not None for _, end in times.values())
        check_order(per_xcd, 3, times)


def test_the_check_catches_a_wrong_target():
    """The order check is not vacuous: with the polynomial allowed to start
    after half of its matrix's Gram tiles, it fails."""
    per_xcd, counts = queues([(768, 768), (768, 3072)])
    half = {i: [max(1, c[0] // 2), c[1], c[2]] for i, c in counts.items()}
    real_target = target

    def early(c, i, t, prod):
        if prod == POLY:
            return real_target(c, i, t, GRAM) + half[i][0]
        return real_target(c, i, t, prod)

    globals()["target"] = early
    try:
        times = simulate(per_xcd, counts, T=2, resident=64, seed=0)
        with pytest.raises(AssertionError, match="read"):
            check_order(per_xcd, 2, times)
    finally:
        globals()["target"] = real_target
