"""A CPU model of the one-launch (persistent) expert FFN's work-queue
protocol: workgroups take gate-up and down tiles from a queue, and a down tile
of an expert waits until every gate-up tile of that expert has finished (the
Ling-2.6-1T page, §4-5: the V2 schedule, one kernel whose FFN1 and FFN2
stages overlap).  No GPU: the model checks the protocol's bookkeeping and
forward progress, and how it behaves under two memory models of a chip
whose eight XCDs each have their own L2:

* ``coherent``: a counter increment is seen by every poller once performed
  (the compiler's agent-scope atomics on gfx950 follow this model: an
  increment is a ``global_atomic_add`` without ``sc1`` after ``buffer_wbl2
  sc1``, a poll a ``global_load ... sc1`` followed by ``buffer_inv sc1``);
* ``xcd_local``: an increment is seen only by pollers on the XCD that
  performed it (what a hang would look like if increments stayed in one
  XCD's L2).

Two queue layouts: one global queue (every gate-up tile before every down
tile), and one queue per XCD holding whole experts, each workgroup taking
work only from the queue of the XCD it runs on (the hardware's XCC_ID), so
that no wait crosses an XCD.  Polls are bounded: a poll that exceeds its
budget raises the kernel's error flag and the workgroup exits, so that a
broken protocol ends as a reported error, never as a hang.
"""

import random

import pytest

N_XCD = 8


def tiles(rows, bm):
    return (rows + bm - 1) // bm


def make_items(counts, bm, n1, n2):
    """Gate-up items (g, mt, c) and down items (g, mt, c) of every group with
    rows; target[g] = gate-up items of group g (what its down items wait for).
    The tile count per group is the tile prefix's ceil(rows / bm)."""
    gate, down, target = [], [], {}
    for g, r in enumerate(counts):
        mt = tiles(r, bm)
        target[g] = mt * n1
        gate += [("gate", g, m, c) for m in range(mt) for c in range(n1)]
        down += [("down", g, m, c) for m in range(mt) for c in range(n2)]
    return gate, down, target


def xcd_of_group(counts):
    """Whole groups to XCDs, largest first onto the least-loaded XCD."""
    load, where = [0] * N_XCD, {}
    for g in sorted(range(len(counts)), key=lambda g: -counts[g]):
        x = min(range(N_XCD), key=lambda x: load[x])
        where[g] = x
        load[x] += counts[g]
    return where


def simulate(counts, *, layout, memory, slots_per_xcd, bm=32, n1=4, n2=4, seed=0, poll_budget=10_000):
    """Runs the protocol with `slots_per_xcd` resident workgroups per XCD,
    an adversarial (random) interleaving of their steps.  Returns
    (finished items, error flag)."""
    rng = random.Random(seed)
    gate, down, target = make_items(counts, bm, n1, n2)
    if layout == "global":
        queues = {None: gate + down}
        qof = lambda x: None  # noqa: E731
    else:
        where = xcd_of_group(counts)
        queues = {x: [it for it in gate if where[it[1]] == x] + [it for it in down if where[it[1]] == x]
                  for x in range(N_XCD)}
        qof = lambda x: x  # noqa: E731
    head = {q: 0 for q in queues}
    # performed increments per group, and per (group, xcd) for the XCD-local model
    done_total = {g: 0 for g in target}
    done_on = {(g, x): 0 for g in target for x in range(N_XCD)}
    wgs = [{"xcd": x, "item": None, "polls": 0, "alive": True} for x in range(N_XCD) for _ in range(slots_per_xcd)]
    finished, error = [], False

    def seen(g, x):
        return done_total[g] if memory == "coherent" else done_on[(g, x)]

    while any(w["alive"] for w in wgs):
        w = rng.choice([w for w in wgs if w["alive"]])
        if w["item"] is None:                      # dequeue (an atomic fetch-add on the queue head)
            q = qof(w["xcd"])
            if head[q] >= len(queues[q]):
                w["alive"] = False                 # queue drained: exit
                continue
            w["item"], w["polls"] = queues[q][head[q]], 0
            head[q] += 1
            continue
        kind, g, m, c = w["item"]
        if kind == "down" and seen(g, w["xcd"]) < target[g]:
            w["polls"] += 1                        # bounded poll of the group's counter
            if w["polls"] > poll_budget:
                error = True
                w["alive"] = False
            continue
        if kind == "gate":                         # tile done: release, then count it
            done_total[g] += 1
            done_on[(g, w["xcd"])] += 1
        finished.append(w["item"])
        w["item"] = None
    return finished, error


COUNTS = {
    "decode_8x16": [16] * 8,                       # 64 tokens top-2 over 8 experts
    "ragged": [5, 0, 17, 1, 40, 0, 3, 32, 77, 2],  # empty groups, partial tiles
    "skewed": [300, 1, 0, 64, 129, 7, 7, 250, 31, 33, 0, 12],
}


@pytest.mark.parametrize("case", list(COUNTS))
@pytest.mark.parametrize("slots", [1, 3])
def test_bookkeeping_and_progress_coherent(case, slots):
    """Every item finishes exactly once, no poll runs out, under any
    interleaving, with one or several resident workgroups per XCD, in both
    layouts (the target of each group equals its enqueued gate-up items,
    groups without rows have neither items nor waits)."""
    counts = COUNTS[case]
    gate, down, target = make_items(counts, 32, 4, 4)
    assert all(target[g] == 0 for g, r in enumerate(counts) if r == 0)
    for layout in ("global", "per_xcd"):
        for seed in range(5):
            fin, err = simulate(counts, layout=layout, memory="coherent", slots_per_xcd=slots, seed=seed)
            assert not err
            assert sorted(fin) == sorted(gate + down)


@pytest.mark.parametrize("case", list(COUNTS))
def test_global_queue_stalls_if_increments_stay_in_one_xcd(case):
    """With one global queue, a down tile's poller is in general on another
    XCD than the workgroups that counted its group's gate-up tiles: under
    the XCD-local model the polls run out (the error flag is raised; in a
    kernel without a bound this is a hang)."""
    _, err = simulate(COUNTS[case], layout="global", memory="xcd_local", slots_per_xcd=2, seed=1, poll_budget=2000)
    assert err


@pytest.mark.parametrize("case", list(COUNTS))
@pytest.mark.parametrize("slots", [1, 3])
def test_per_xcd_queues_complete_under_either_model(case, slots):
    """One queue per XCD holding whole groups: every wait is on counters
    incremented on the poller's own XCD, so the protocol completes under
    the XCD-local model too."""
    counts = COUNTS[case]
    gate, down, _ = make_items(counts, 32, 4, 4)
    for memory in ("coherent", "xcd_local"):
        for seed in range(3):
            fin, err = simulate(counts, layout="per_xcd", memory=memory, slots_per_xcd=slots, seed=seed)
            assert not err
            assert sorted(fin) == sorted(gate + down)


def test_out_of_order_dequeue_can_deadlock():
    """The forward-progress argument rests on the queue order: if a down tile
    could be dequeued while a gate-up tile it waits for is still queued, and
    every resident workgroup holds such a down tile, nothing runs the
    gate-up tile.  Planted: down tiles first, one resident workgroup."""
    counts = [40]
    gate, down, target = make_items(counts, 32, 4, 4)

    def run_order(order):
        done, held = 0, None
        for it in order:                   # one workgroup: takes items in queue order
            held = it
            if it[0] == "down" and done < target[0]:
                return False               # waits for a gate-up tile still in the queue
            if it[0] == "gate":
                done += 1
        return held is not None

    assert run_order(gate + down)
    assert not run_order(down + gate)
