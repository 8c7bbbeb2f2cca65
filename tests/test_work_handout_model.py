"""A step-by-step model of the one-launch path's work hand-out, under random interleavings (CPU).

The one-launch kernel (gla_fused) hands segments to its persistent workgroups through one 64-bit
work word per XCD, a batch counter shared by all XCDs and a mask of XCDs that have begun
(take_work and work_add in csrc/gla_kernels.hip).  The GPU tests run it as the hardware schedules
it; they cannot make an XCD run no workgroup at all, the case the take-over of starting batches
exists for.  This model restates those rules in Python, one shared-memory access per step, and runs
workgroups in random orders, with all XCDs present and with some missing, checking that

  * every segment of every sequence is worked exactly once;
  * every workgroup ends (none waits forever on a work word or on an earlier segment);
  * an XCD that takes over a batch at launch works it with all its workgroups.

A segment waits until every earlier segment of its sequence has been worked (the real kernel waits
for the earlier segments of its fold block and the previous block's prefix, which depends on all of
them).  The model shares no code with the library: it is checked by reading both side by side.
"""
import random

import pytest

DONE, STOLEN = 0xFFFFFFFF, 0xFFFFFFFE


class Shared:
    def __init__(self, n_slots):
        self.word = [(0, 0)] * n_slots  # (tag, next ticket)
        self.next_batch = 0
        self.started = 0
        self.worked = {}                 # (seq, seg) -> (slot, id) of the workgroup that worked it
        self.takers = {}                 # batch -> slots that took tickets of it after a take-over


def workgroup(sh, p, slot, wg_id=0, join=True, takeover=True):
    """One workgroup of XCD `slot`; yields at every access to shared memory.  join=False and
    takeover=False plant the two mistakes the checks below must catch: workgroups without a batch
    of their own leaving instead of joining one taken over, and no take-over at all."""
    def work_add():
        tag, t = sh.word[slot]
        sh.word[slot] = (tag, t + 1)
        return tag, t

    def take_work(v):
        while True:
            tag, t = v
            if tag == DONE:
                return None
            b = (slot if slot < p["n_pre"] else -1) if tag == 0 else (-1 if tag == STOLEN else tag - 1)
            first = b * p["batch"]
            k = 0 if b < 0 else min(p["batch"], p["bh"] - first)
            n_in = k * p["n_seg"]
            if t < n_in:
                if tag == 0 and t == 0:
                    sh.started |= 1 << slot
                    yield
                return first + t % k, t // k, b
            if t == n_in:
                if p["n_pre"] >= p["n_batch"]:
                    nb = p["n_batch"]
                else:
                    nb = p["n_pre"] + sh.next_batch
                    sh.next_batch += 1
                    yield
                if nb < p["n_batch"]:
                    sh.word[slot] = (nb + 1, 1)
                    yield
                    return nb * p["batch"], 0, nb
                started = sh.started
                yield
                for y in range(p["n_pre"] if takeover else 0):
                    if y != slot and not (started >> y & 1):
                        if sh.word[y] == (0, 0):  # compare-exchange 0 -> (STOLEN, 0)
                            sh.word[y] = (STOLEN, 0)
                            yield
                            sh.word[slot] = (y + 1, 1)
                            yield
                            return y * p["batch"], 0, y
                        yield
                sh.word[slot] = (DONE, 0)
                yield
                return None
            if p["n_pre"] >= p["n_batch"] and (b >= 0 or not join):
                return None
            while sh.word[slot][0] == tag:  # wait for the workgroup taking the next batch
                yield
            v = work_add()
            yield

    v = work_add()
    yield
    got = yield from take_work(v)
    while got is not None:
        seq, seg, b = got
        nv = work_add()  # the next ticket's increment goes out before the segment is worked
        yield
        while any((seq, s) not in sh.worked for s in range(seg)):
            yield
        assert (seq, seg) not in sh.worked, f"segment {seq, seg} worked twice"
        sh.worked[(seq, seg)] = (slot, wg_id)
        sh.takers.setdefault(b, set()).add(slot)
        yield
        got = yield from take_work(nv)


def run(bh, n_seg, batch, xcds, wgs_per_slot, seed, max_steps=2_000_000, **plant):
    n_batch = (bh + batch - 1) // batch
    p = dict(bh=bh, n_seg=n_seg, batch=batch, n_batch=n_batch, n_pre=min(n_batch, min(xcds, 16)))
    slots = sorted(wgs_per_slot)
    sh = Shared(max(16, max(slots) + 1))
    live = [workgroup(sh, p, s, i, **plant) for s in slots for i in range(wgs_per_slot[s])]
    rng = random.Random(seed)
    steps = 0
    while live:
        i = rng.randrange(len(live))
        try:
            next(live[i])
        except StopIteration:
            live.pop(i)
        steps += 1
        assert steps < max_steps, f"no progress: {len(live)} workgroups still running"
    expect = {(q, s) for q in range(bh) for s in range(n_seg)}
    assert set(sh.worked) == expect, f"missing {sorted(expect - set(sh.worked))[:5]}"
    return sh


# (sequences, segments per sequence, batch, XCDs the device reports, workgroups on each XCD that runs)
CASES = [
    (16, 32, 2, 8, {x: 64 for x in range(8)}),      # one batch per XCD, one round
    (12, 32, 2, 8, {x: 64 for x in range(8)}),      # 6 batches: two XCDs start with none
    (6, 25, 1, 8, {x: 25 for x in range(8)}),       # fewer sequences than XCDs
    (40, 6, 2, 8, {x: 8 for x in range(8)}),        # 20 batches: the counter hands out 12
    (48, 9, 6, 8, {x: 20 for x in range(8)}),       # fewer workgroups than tickets: several rounds
    (16, 8, 2, 8, {x: 16 for x in range(6)}),       # XCDs 6 and 7 run no workgroup
    (12, 8, 2, 8, {x: 16 for x in (1, 4, 6, 7)}),   # half the XCDs missing, some without batches
    (4, 5, 1, 1, {3: 6}),                           # one XCD reported, running as XCD 3
    (5, 3, 1, 8, {7: 4}),                           # only XCD 7 runs: it takes over every batch
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"bh{c[0]}_seg{c[1]}_b{c[2]}_xcds{len(c[4])}")
def test_every_segment_once_and_every_workgroup_ends(case):
    bh, n_seg, batch, xcds, wgs = case
    for seed in range(12):
        run(bh, n_seg, batch, xcds, wgs, seed)


def taken_over_at_launch(join):
    """6 sequences on 8 XCDs, XCD 7 first: it takes over a starting batch before that batch's XCD
    begins.  Returns the workgroups of XCD 7 that worked segments of the batch it took."""
    bh, n_seg, batch = 6, 25, 1
    p = dict(bh=bh, n_seg=n_seg, batch=batch, n_batch=6, n_pre=6)
    sh = Shared(16)
    xcd7 = [workgroup(sh, p, 7, i, join=join) for i in range(25)]
    # XCD 7's workgroups run alone for a few steps each: enough for the first to take over a batch
    # and for the others to take tickets of it or decide to leave, not enough to finish the batch
    for _ in range(6):
        for g in xcd7:
            try:
                next(g)
            except StopIteration:
                pass
    others = [workgroup(sh, p, x, i, join=join) for x in range(6) for i in range(25)]
    live = xcd7 + others
    rng = random.Random(5)
    while live:
        i = rng.randrange(len(live))
        try:
            next(live[i])
        except StopIteration:
            live.pop(i)
    assert len(sh.worked) == bh * n_seg
    stolen = [b for b, s in sh.takers.items() if s == {7}]
    assert len(stolen) == 1, "XCD 7 took over no batch"
    assert sum(1 for (q, _), (x, _) in sh.worked.items() if q == stolen[0] and x == 7) == n_seg
    return {wg for (q, _), (x, wg) in sh.worked.items() if q == stolen[0]}


def test_batch_taken_over_at_launch_is_worked_by_the_whole_xcd():
    assert len(taken_over_at_launch(join=True)) > 5
    # planted: workgroups leaving instead of joining leave the batch to the one that took it
    assert len(taken_over_at_launch(join=False)) == 1


@pytest.mark.parametrize("case", [CASES[5], CASES[7], CASES[8]], ids=["xcds_6_7_missing", "one_xcd_as_3", "only_xcd_7"])
def test_planted_missing_takeover_is_caught(case):
    """Without the take-over, the batches of XCDs that run no workgroup are never worked."""
    bh, n_seg, batch, xcds, wgs = case
    with pytest.raises(AssertionError, match="missing"):
        run(bh, n_seg, batch, xcds, wgs, 0, takeover=False)
