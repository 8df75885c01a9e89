"""The backward kernels' LDS buffer schedules, modelled on the host (no GPU).

dK/dV kernel (eight waves per workgroup, two roles): Q, dO and the row terms of a 64-row block go
into buffer set t % 3 (three sets); at step t every wave waits for its own copies, passes the
workgroup barrier and then requests block t + 1's copies into set (t + 1) % 3.  The dV waves
read set t % 3 (block t) and store the block's P into P buffer t % 2; the dK waves work one
block behind: they read set (t - 1) % 3 and the P that the dV waves stored in buffer (t - 1) % 2
during the previous step.  One barrier per step orders all of it.

dQ kernel (four waves, one role): K and V blocks go into two buffer pairs; step t waits, passes
the barrier, requests block t + 1 into pair (t + 1) % 2 and reads pair t % 2.

The replay checks, for every step count up to 40, the two properties the barrier placement has
to give:

  * every read sees its block: the block's copy (or store) into that buffer happened in an
    earlier barrier epoch, a copy was waited for by its issuing waves before that barrier, and
    nothing else was written into the buffer from then until the read's epoch ends;
  * nothing is written into a buffer that a wave may still read: all reads of the buffer's
    previous contents happened in earlier barrier epochs.
"""
import pytest


def dkdv_events(n_steps):
    """(role, kind, buffer, tag, epoch) in program order; kind 'copy' is an asynchronous copy
    that the issuing wave waits for before its next barrier, 'store' a plain LDS store."""
    ev = []
    epoch = 0
    if n_steps > 0:  # prologue: stage(0) into set 0 by both roles
        for role in ("dV", "dK"):
            ev.append((role, "copy", ("set", 0), ("blk", 0), epoch))
    for t in range(n_steps + 1):
        epoch += 1  # wait for own copies, then the barrier that opens step t
        if t + 1 < n_steps:
            for role in ("dV", "dK"):
                ev.append((role, "copy", ("set", (t + 1) % 3), ("blk", t + 1), epoch))
        if t < n_steps:  # dV waves: block t
            ev.append(("dV", "read", ("set", t % 3), ("blk", t), epoch))
            ev.append(("dV", "store", ("P", t % 2), ("P", t), epoch))
        if 1 <= t <= n_steps:  # dK waves: block t - 1 and its P
            ev.append(("dK", "read", ("set", (t - 1) % 3), ("blk", t - 1), epoch))
            ev.append(("dK", "read", ("P", (t - 1) % 2), ("P", t - 1), epoch))
    return ev


def dq_events(n_blk):
    ev = []
    epoch = 0
    if n_blk > 0:
        ev.append(("w", "copy", ("kv", 0), ("blk", 0), epoch))
    for t in range(n_blk):
        epoch += 1
        if t + 1 < n_blk:
            ev.append(("w", "copy", ("kv", (t + 1) % 2), ("blk", t + 1), epoch))
        ev.append(("w", "read", ("kv", t % 2), ("blk", t), epoch))
    return ev


def check(ev):
    """Raise AssertionError on the first violation of the two properties above.  A copy issued in
    epoch e lands before the barrier that ends epoch e (its waves wait for it there), so it is
    visible from epoch e + 1 on; a store in epoch e likewise becomes visible from e + 1."""
    writes = {}  # buffer -> list of (epoch, tag) in program order
    reads = {}   # buffer -> list of (epoch, tag)
    for role, kind, buf, tag, epoch in ev:
        if kind in ("copy", "store"):
            # every read of what the buffer held must lie in an earlier epoch
            for r_epoch, r_tag in reads.get(buf, []):
                prev = writes[buf][-1][1] if writes.get(buf) else None
                if r_tag == prev:
                    assert r_epoch < epoch, (role, kind, buf, tag, epoch, "overwrites a read of", r_tag, r_epoch)
            writes.setdefault(buf, []).append((epoch, tag))
        else:
            hist = writes.get(buf, [])
            assert hist, (role, buf, tag, epoch, "read before any write")
            w_epoch, w_tag = hist[-1]
            assert w_tag == tag, (role, buf, tag, epoch, "buffer holds", w_tag)
            assert w_epoch < epoch, (role, buf, tag, epoch, "write not yet visible", w_epoch)
            reads.setdefault(buf, []).append((epoch, tag))
    # a write later in program order but in the same epoch as a read of the old contents would
    # also be a race: re-check every read against every write of its buffer
    for role, kind, buf, tag, epoch in ev:
        if kind != "read":
            continue
        for w_epoch, w_tag in writes[buf]:
            if w_tag != tag:
                assert not (w_epoch == epoch), (role, buf, tag, epoch, "written in the same epoch by", w_tag)
    return True


@pytest.mark.parametrize("n_steps", list(range(0, 41)))
def test_dkdv_schedule(n_steps):
    assert check(dkdv_events(n_steps))


@pytest.mark.parametrize("n_blk", list(range(0, 41)))
def test_dq_schedule(n_blk):
    assert check(dq_events(n_blk))


def test_the_checker_catches_a_two_set_dkdv_schedule():
    # with two Q / dO sets instead of three, the copy of block t + 1 lands in the set that the
    # dK waves are still reading (block t - 1) in the same step
    ev = []
    epoch = 0
    n = 6
    ev.append(("dV", "copy", ("set", 0), ("blk", 0), epoch))
    for t in range(n + 1):
        epoch += 1
        if t + 1 < n:
            ev.append(("dV", "copy", ("set", (t + 1) % 2), ("blk", t + 1), epoch))
        if t < n:
            ev.append(("dV", "read", ("set", t % 2), ("blk", t), epoch))
        if 1 <= t <= n:
            ev.append(("dK", "read", ("set", (t - 1) % 2), ("blk", t - 1), epoch))
    with pytest.raises(AssertionError):
        check(ev)


def test_the_checker_catches_a_single_p_buffer():
    # one P buffer: the dV waves' store of P(t) meets the dK waves' read of P(t - 1) in step t
    ev = []
    epoch = 0
    for t in range(5):
        epoch += 1
        ev.append(("dV", "store", ("P", 0), ("P", t), epoch))
        if t >= 1:
            ev.append(("dK", "read", ("P", 0), ("P", t - 1), epoch))
    with pytest.raises(AssertionError):
        check(ev)


def test_the_checker_catches_a_read_in_the_copy_epoch():
    # reading block t + 1 in the step that requests it (no barrier between wait and read)
    ev = [("w", "copy", ("kv", 0), ("blk", 0), 0)]
    ev.append(("w", "read", ("kv", 0), ("blk", 0), 0))
    with pytest.raises(AssertionError):
        check(ev)
