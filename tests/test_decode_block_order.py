"""The decode split kernel's block schedule, restated on the host (no GPU).

A split of nkb 32-key blocks is streamed by NW waves (1 or 4); wave w takes the blocks at steps
w, w + NW, w + 2 NW, ... and keeps NB of them in flight in registers (NB = 2 for a lone wave, 1
for each of four), refilling a register slot with the block NB * NW steps further on as soon as
the slot's block is staged.  Step j reads block (j + rot) mod nkb, with rot = (7 s + 5 p) mod nkb
for split s of (batch, KV head) pair p, so concurrent splits start at different offsets.

For every block count up to 40 and a spread of (s, p), the replay checks that each block of the
split is computed exactly once, that the block computed from a register slot is the one last
loaded into it, and that nothing is loaded past the split.
"""
import itertools

import pytest


def replay(nkb, NW, s, p):
    NB = 2 if NW == 1 else 1
    rot = (s * 7 + p * 5) % nkb if nkb > 0 else 0

    def phys(j):
        k = j + rot
        return k - nkb if k >= nkb else k

    computed = []
    for w in range(NW):
        slots = {}
        for u in range(NB):  # prologue
            if w + u * NW < nkb:
                slots[u] = phys(w + u * NW)
        kb = w
        while kb < nkb:
            for u in range(NB):
                kbu = kb + u * NW
                if kbu < nkb:
                    staged = slots.pop(u)  # the slot's registers go to LDS
                    assert staged == phys(kbu), (nkb, NW, s, p, w, kbu)
                    if kbu + NB * NW < nkb:
                        slots[u] = phys(kbu + NB * NW)
                    computed.append(phys(kbu))
            kb += NB * NW
        assert not slots, "a block was loaded but never computed"
    return computed


@pytest.mark.parametrize("NW", [1, 4])
def test_every_block_once(NW):
    for nkb, s, p in itertools.product(range(0, 41), range(0, 17), (0, 1, 3, 7, 63)):
        blocks = replay(nkb, NW, s, p)
        assert sorted(blocks) == list(range(nkb)), (nkb, NW, s, p)
        assert all(0 <= b < nkb for b in blocks)


def test_rotation_spreads_the_starting_block():
    # the GQA decode workload: 64 pairs x 16 splits of 16 blocks; every starting offset is used
    # by the same number of splits
    starts = [((s * 7 + p * 5) % 16) for s in range(16) for p in range(64)]
    counts = [starts.count(k) for k in range(16)]
    assert min(counts) == max(counts) == 64
