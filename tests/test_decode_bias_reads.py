"""The split-KV decode kernel's bias reads, modelled on the host (no GPU).

The split kernel reads, for each 4-key group it needs (keys key .. key+3 of its own bias row,
key = ks0 + 32 kb + 16 hh + 4 grp), one or two aligned 8-byte units of four keys and shifts the
group out of them.  This test restates that address arithmetic and checks, for every split
shape the GPU tests use with a bias plus a seeded sweep (with and without per-batch key
lengths), that

  * every unit read is 8-byte aligned and lies inside the row (so no read leaves the caller's
    bias tensor, whatever the split length L = ceil(Nk / S) is mod 4);
  * every key of a group that lies inside the split is supplied by a unit that was read;
  * the shift takes exactly keys key .. key+3 out of the one or two units.
"""
import numpy as np
import pytest

KB = 32  # keys per wave block of the split kernel


def _groups(Nk_cap, S, Nk):
    """(ks0, ks1, key) of every 4-key group the split kernel handles for one batch element."""
    L = -(-Nk_cap // S)
    for s in range(S):
        ks0 = min(s * L, Nk)
        ks1 = min(ks0 + L, Nk)
        nkb = -(-(ks1 - ks0) // KB)
        for kb in range(nkb):
            for hh in range(2):
                for grp in range(4):
                    yield ks0, ks1, ks0 + KB * kb + 16 * hh + 4 * grp


def _reads(ks0, ks1, key):
    """The units (first key of each aligned 4-key unit) the kernel loads for one group, and the
    misalignment a used to shift the group out of them."""
    a = ks0 & 3
    unit = key - a
    units = []
    if unit + a < ks1:
        units.append(unit)
    if a != 0 and unit + 4 < ks1:
        units.append(unit + 4)
    return a, unit, units


def _check_row(Nk_cap, S, Nk, row):
    """row: int array [Nk_cap] of distinct values standing in for one bias row."""
    assert Nk_cap % 4 == 0
    for ks0, ks1, key in _groups(Nk_cap, S, Nk):
        assert key % 4 == ks0 % 4
        a, unit, units = _reads(ks0, ks1, key)
        for u in units:
            assert u % 4 == 0, f"unaligned unit {u} (Nk_cap={Nk_cap} S={S})"
            assert 0 <= u and u + 4 <= Nk_cap, f"unit {u} outside row of {Nk_cap} keys"
        covered = {u + i for u in units for i in range(4)}
        for j in range(key, key + 4):
            if ks0 <= j < ks1:
                assert j in covered, f"key {j} of split [{ks0},{ks1}) not read"
        # the kernel's shift of the 64-bit units (four 16-bit keys each, little-endian)
        lo = sum(int(row[unit + i]) << (16 * i) for i in range(4)) if unit in units else 0
        hi = (sum(int(row[unit + 4 + i]) << (16 * i) for i in range(4))
              if (unit + 4) in units else 0)
        w = lo if a == 0 else ((lo >> (16 * a)) | (hi << (64 - 16 * a))) & ((1 << 64) - 1)
        for i in range(4):
            if key + i < ks1:
                assert (w >> (16 * i)) & 0xFFFF == row[key + i], (Nk_cap, S, key, i)


# (Nk capacity, n_splits) of the GPU tests that pass a bias to the split kernel, and the
# GQA decode workload with the bias of the benchmark
GPU_TEST_SHAPES = [(1000, 16), (1000, 5), (512, 4), (64, 64), (8192, 16)]


@pytest.mark.parametrize("Nk_cap,S", GPU_TEST_SHAPES)
def test_bias_reads_of_gpu_test_shapes(Nk_cap, S):
    row = np.arange(Nk_cap) % 65521
    _check_row(Nk_cap, S, Nk_cap, row)
    # and with the per-batch key lengths the extras tests draw (0, 1, a few ragged values)
    for Nk in sorted({0, 1, 3, Nk_cap - 1, Nk_cap // 3, Nk_cap // 2 + 5}):
        _check_row(Nk_cap, S, max(0, min(Nk, Nk_cap)), row)


def test_bias_reads_seeded_sweep():
    rng = np.random.default_rng(2024)
    for _ in range(300):
        Nk_cap = 4 * int(rng.integers(1, 700))
        S = int(rng.integers(1, min(Nk_cap, 256) + 1))
        Nk = int(rng.integers(0, Nk_cap + 1)) if rng.integers(0, 2) else Nk_cap
        row = rng.integers(0, 1 << 16, size=Nk_cap)
        _check_row(Nk_cap, S, Nk, row)


def test_every_misalignment_occurs():
    # the sweep above exercises all four offsets of the split start mod 4
    seen = set()
    for Nk_cap, S in GPU_TEST_SHAPES:
        L = -(-Nk_cap // S)
        seen |= {(s * L) % 4 for s in range(S) if s * L < Nk_cap}
    assert seen == {0, 1, 2, 3}
