"""The forward kernel's LDS double-buffer schedule, modelled on the host (no GPU).

The prefill kernel keeps two K buffers and two V buffers in LDS; block t's keys live in K
buffer t % 2 and its values in V buffer t % 2, and K runs one block ahead of V.  Per step t
(after the prologue) every wave waits for all of its own copies and then passes the workgroup
barrier; after the barrier it issues the copies of K[t+2] and V[t+1]; during the step it reads
K[t+1] (the next block's scores) and V[t] (this block's products).  The prologue issues K[0],
V[0], K[1], V[1], waits for K[0] only, passes a barrier and reads K[0].

This test replays that order for every tile count up to 40 and checks the two properties the
barrier placement has to give (so a single-buffer build would need extra barriers, while this
schedule needs none beyond one per step):

  * no copy is issued into a buffer that a wave may still read: the buffer's last reads all
    happened before a barrier that the issuing wave has passed;
  * every read sees its block: the copy of that block into that buffer was issued and waited for
    by every wave before a barrier the reading wave has passed, and no later copy into the
    buffer was issued before the read.
"""
import pytest


def replay(n_tiles):
    """Events (kind, buffer, block, barrier epoch) in program order of one wave (all waves run
    the same order); a barrier ends an epoch.  Kinds: 'issue', 'wait_all', 'wait_k0', 'read'."""
    ev, epoch = [], 0

    def buf(kind, t):
        return (kind, t % 2)

    if n_tiles == 0:
        return ev
    issued = []
    for kind, t in (("K", 0), ("V", 0), ("K", 1), ("V", 1)):
        if t < n_tiles:
            ev.append(("issue", buf(kind, t), (kind, t), epoch))
            issued.append((kind, t))
    ev.append(("wait", None, ("K", 0), epoch))  # loads complete in order: K[0] has landed
    epoch += 1  # barrier
    ev.append(("read", buf("K", 0), ("K", 0), epoch))
    for t in range(n_tiles):
        ev.append(("wait", None, "all", epoch))
        epoch += 1  # barrier at the start of step t
        if t + 2 < n_tiles:
            ev.append(("issue", buf("K", t + 2), ("K", t + 2), epoch))
        if t + 1 < n_tiles and t >= 1:
            ev.append(("issue", buf("V", t + 1), ("V", t + 1), epoch))
        if t + 1 < n_tiles:
            ev.append(("read", buf("K", t + 1), ("K", t + 1), epoch))
        ev.append(("read", buf("V", t), ("V", t), epoch))
    return ev


def check(n_tiles):
    ev = replay(n_tiles)
    # per buffer: the block it holds (last issued copy), the epoch of that issue, whether the
    # issuing waves have waited for it (and in which epoch), and the last epoch it was read in
    holds, issue_epoch, landed_epoch, last_read = {}, {}, {}, {}
    pending = []  # issued, not yet waited for (in order)
    for kind, b, what, epoch in ev:
        if kind == "issue":
            # every earlier read of this buffer must lie in an earlier epoch (before a barrier)
            assert last_read.get(b, -1) < epoch, f"n={n_tiles}: {what} overwrites {b} still read"
            holds[b], issue_epoch[b] = what, epoch
            landed_epoch.pop(b, None)
            pending.append(b)
        elif kind == "wait":
            if what == "all":
                done, pending[:] = list(pending), []
            else:  # in-order completion up to and including that copy
                i = [holds[p] for p in pending].index(what)
                done, pending[:] = pending[:i + 1], pending[i + 1:]
            for p in done:
                landed_epoch[p] = epoch
        else:  # read
            assert holds.get(b) == what, f"n={n_tiles}: read of {what} finds {holds.get(b)}"
            # waited for by every wave before a barrier that this read follows
            assert landed_epoch.get(b, epoch) < epoch, f"n={n_tiles}: {what} read before it landed"
            last_read[b] = epoch
    return ev


@pytest.mark.parametrize("n_tiles", range(0, 41))
def test_double_buffer_schedule(n_tiles):
    ev = check(n_tiles)
    reads = [e[2] for e in ev if e[0] == "read"]
    # every block's K and V is read (K[0] in the prologue, K[t+1] and V[t] in step t)
    assert sorted(reads) == sorted([("K", t) for t in range(n_tiles)] +
                                   [("V", t) for t in range(n_tiles)])


def test_model_catches_a_third_block_in_flight():
    # a schedule that issued K[t+3] (a third K block in flight in two buffers) would overwrite
    # K[t+1] while step t still reads it: the same checks must reject it
    ev = replay(6)
    bad = []
    for e in ev:
        bad.append(e)
        if e[0] == "issue" and e[2][0] == "K" and e[2][1] >= 2:
            t3 = e[2][1] + 1
            if t3 < 6:
                bad.append(("issue", ("K", t3 % 2), ("K", t3), e[3]))
    holds, last_read = {}, {}
    with pytest.raises(AssertionError):
        for kind, b, what, epoch in bad:
            if kind == "issue":
                assert last_read.get(b, -1) < epoch
                holds[b] = what
            elif kind == "read":
                assert holds.get(b) == what
                last_read[b] = epoch
