"""Host check of the workgroup -> work-item mappings of `csrc/common.h`
(xcd_contiguous, xcd_windowed), restated here: each must be a permutation of
the item list, and the workgroups the hardware deals to one XCD (equal pid mod
8) must take contiguous runs (inside each window for the windowed form).
No GPU involved."""

import itertools


def xcd_contiguous(j, S, R):
    x, off = (S + j) & 7, S & 7
    base = 0
    for y in range(x):
        j0 = (y - off) & 7
        base += (R - 1 - j0) // 8 + 1 if j0 < R else 0
    return base + (j - ((x - off) & 7)) // 8


def xcd_windowed(j, S, R, W):
    base = (j // W) * W
    return base + xcd_contiguous(j - base, S + base, min(W, R - base))


def _runs_are_contiguous(items_of_xcd):
    return all(b == a + 1 for a, b in zip(items_of_xcd, items_of_xcd[1:]))


def test_xcd_contiguous_is_a_permutation_with_contiguous_runs():
    for S, R in itertools.product(range(0, 17), list(range(0, 40)) + [511, 512, 513, 1000]):
        items = [xcd_contiguous(j, S, R) for j in range(R)]
        assert sorted(items) == list(range(R)), (S, R)
        for x in range(8):
            mine = [items[j] for j in range(R) if (S + j) & 7 == x]
            assert _runs_are_contiguous(mine), (S, R, x)


def test_xcd_windowed_is_a_permutation_and_keeps_window_order():
    for S, R, W in itertools.product((0, 3, 8, 13), (1, 7, 64, 511, 512, 513, 1500, 3072), (8, 64, 512)):
        items = [xcd_windowed(j, S, R, W) for j in range(R)]
        assert sorted(items) == list(range(R)), (S, R, W)
        for w0 in range(0, R, W):
            win = items[w0:w0 + W]
            # a window covers exactly its own slice of the list
            assert sorted(win) == list(range(w0, min(w0 + W, R)))
            for x in range(8):
                mine = [win[j] for j in range(len(win)) if (S + w0 + j) & 7 == x]
                assert _runs_are_contiguous(mine), (S, R, W, w0, x)
