"""A CPU model of how bevpool_forward writes every output cell exactly once.

The forward kernel has no memset: cells that own no interval are zeroed by
the owners, under these rules (forward_kernels.hip, zero_end_slices,
zero_interior_gap, zero_chunk_if_empty):
  * the owner of each interval writes its cell once, and zeroes the gap
    between the previous interval's cell and its own -- except the aligned
    256-cell chunks lying wholly inside that gap;
  * those chunks are zeroed by chunk checks: a check of chunk [c0, c1) zeroes
    it when it lies between the first and last occupied cells and no point
    falls in it (the first point at or after c0, found by a 64-way search
    over the sorted ranks_bev, lies at or past c1);
  * the empty head [0, first cell) and tail (last cell, n_cells) are cut into
    up to 64 slices of at least 64 cells; slice s of the head is zeroed by
    the owner of interval s and slice s of the tail by the owner of interval
    I - 1 - s.
This model restates those rules and checks, on random maps of many shapes,
that every cell is written exactly once; it also checks the 64-way search
against bisect.  It pins the design of the rules; the GPU tests check the
kernel's output on maps with large empty regions.
"""
import bisect
import math

import numpy as np
import pytest

WAVE = 64
SLICE_CELLS = 64
CHUNK_CELLS = 256
INT32_MAX = 2 ** 31 - 1


def end_slice(lo, hi, s, owners):
    size = hi - lo
    k = max(1, min(min(WAVE, owners), -(-size // SLICE_CELLS)))
    if s >= k or size <= 0:
        return 0, 0
    length = -(-size // k)
    return min(hi, lo + s * length), min(hi, lo + (s + 1) * length)


def search64(ranks_bev, c0):
    """The kernel's 64-way search: ranks_bev[t] for the first t with
    ranks_bev[t] >= c0, or INT32_MAX when there is none."""
    n = len(ranks_bev)
    lo, hi, hv = 0, n, INT32_MAX
    lanes = np.arange(WAVE)
    while lo < hi:
        step = -(-(hi - lo) // WAVE)
        t = lo + lanes * step
        valid = t < hi
        v = np.where(valid, ranks_bev[np.minimum(t, n - 1)], INT32_MAX)
        ge = v >= c0
        j = int(np.argmax(ge)) if ge.any() else WAVE
        new_lo = lo if j == 0 else lo + (j - 1) * step + 1
        if j < WAVE and lo + j * step < hi:
            hi = lo + j * step
            hv = int(v[j])
        lo = new_lo
    return hv


def write_counts(cells, lengths, n_cells):
    """How many times each output cell is stored, under the rules above."""
    cells = np.asarray(cells, np.int64)
    I = len(cells)
    diff = np.zeros(n_cells + 1, np.int64)

    def zero(lo, hi):
        if hi > lo:
            diff[lo] += 1
            diff[hi] -= 1

    def zero_interior_gap(lo, hi):
        if hi - lo >= CHUNK_CELLS:
            kf, kl = -(-lo // CHUNK_CELLS), hi // CHUNK_CELLS
            if kf < kl:
                zero(lo, kf * CHUNK_CELLS)
                lo = kl * CHUNK_CELLS
        zero(lo, hi)

    first, last = int(cells[0]), int(cells[-1])
    for iv in range(I):
        zero(int(cells[iv]), int(cells[iv]) + 1)             # the owned cell
        if iv > 0:
            zero_interior_gap(int(cells[iv - 1]) + 1, int(cells[iv]))
        if iv < WAVE:
            zero(*end_slice(0, first, iv, I))
        if I - 1 - iv < WAVE:
            zero(*end_slice(last + 1, n_cells, I - 1 - iv, I))
    ranks_bev = np.repeat(cells, lengths)
    for chunk in range(-(-n_cells // CHUNK_CELLS)):
        c0, c1 = chunk * CHUNK_CELLS, min(n_cells, (chunk + 1) * CHUNK_CELLS)
        if c1 <= first or c0 > last:
            continue
        if search64(ranks_bev, c0) >= c1:
            zero(c0, c1)
    return np.cumsum(diff)[:n_cells]


def _random_map(rng, kind):
    n_cells = int(rng.choice([1, 7, 255, 256, 257, 1000, 5000, 16384, 40000, 65536]))
    if kind == "uniform":
        k = int(rng.integers(1, min(n_cells, 3000) + 1))
        cells = rng.choice(n_cells, size=k, replace=False)
    elif kind == "clusters":
        centres = rng.integers(0, n_cells, size=int(rng.integers(1, 6)))
        spread = int(rng.integers(1, 600))
        cells = np.unique(np.clip(rng.choice(centres, 2000) + rng.integers(-spread, spread, 2000),
                                  0, n_cells - 1))
    elif kind == "head_or_tail_only":
        band = min(n_cells, int(rng.integers(1, max(2, n_cells // 8) + 1)))
        lo = 0 if rng.random() < 0.5 else n_cells - band
        cells = np.unique(rng.integers(lo, lo + band, size=int(rng.integers(1, 200))))
    elif kind == "few":
        cells = rng.choice(n_cells, size=int(rng.integers(1, min(n_cells, 70) + 1)), replace=False)
    else:  # "chunk_edges": occupied cells on and around multiples of 256
        base = np.arange(0, n_cells, CHUNK_CELLS * int(rng.integers(1, 4)))
        cells = np.unique(np.clip(base + rng.integers(-1, 2, size=base.size), 0, n_cells - 1))
    cells = np.sort(np.unique(cells)).astype(np.int64)
    lengths = rng.integers(1, 5, size=cells.size)
    return cells, lengths, n_cells


@pytest.mark.parametrize("kind", ["uniform", "clusters", "head_or_tail_only", "few", "chunk_edges"])
def test_every_cell_written_exactly_once(kind):
    rng = np.random.default_rng(["uniform", "clusters", "head_or_tail_only", "few",
                                 "chunk_edges"].index(kind))
    for trial in range(120):
        cells, lengths, n_cells = _random_map(rng, kind)
        counts = write_counts(cells, lengths, n_cells)
        bad = np.nonzero(counts != 1)[0]
        assert bad.size == 0, (f"{kind} trial {trial}: cells {bad[:5].tolist()} written "
                               f"{counts[bad[:5]].tolist()} times (n_cells {n_cells}, "
                               f"{cells.size} intervals)")


def test_long_runs_are_shared_out():
    """No single owner zeroes a long run: with three intervals in the middle
    of a 65,536-cell grid, the head is cut into three slices (one per owner,
    at most 64 owners), and the interior gap's whole chunks go to the chunk
    checks; still every cell is written once."""
    n_cells = 65536
    cells = np.array([30000, 30001, 40000])
    I = cells.size
    sizes = [end_slice(0, 30000, s, I) for s in range(WAVE)]
    assert max(hi - lo for lo, hi in sizes) <= math.ceil(30000 / I)
    np.testing.assert_array_equal(write_counts(cells, [3, 1, 2], n_cells), np.ones(n_cells))


def test_search64_matches_bisect():
    rng = np.random.default_rng(9)
    for trial in range(400):
        n = int(rng.choice([1, 2, 63, 64, 65, 4095, 4096, 4097, 300000]))
        rb = np.sort(rng.integers(0, int(rng.choice([3, 1000, 1 << 30])), size=n))
        for c0 in list(rng.integers(-1, int(rb[-1]) + 3, size=6)) + [int(rb[0]), int(rb[-1])]:
            t = bisect.bisect_left(rb.tolist(), int(c0)) if n < 5000 else int(np.searchsorted(rb, c0))
            want = int(rb[t]) if t < n else INT32_MAX
            assert search64(rb, int(c0)) == want, f"trial {trial}, n {n}, c0 {c0}"
