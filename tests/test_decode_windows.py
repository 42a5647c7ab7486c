"""The decode kernel's walk over page-table windows, replayed on the host.

A decode wave reads the page ids of up to 64 logical pages at a time (one per
lane) and finds each 16-token group's page by its index inside that window.
Split lengths are multiples of 16 while pages may hold up to 256 rows, so a
split can start inside a page.  The window must then end at the end of its
64th page, not 64 pages' worth of tokens after the split's start, or the last
groups would index a 65th page (lane 64, which wraps to lane 0).  This test
replays the kernel's window and group arithmetic in Python for page sizes
16..256 and the split lengths that start splits inside pages, and checks that
every group indexes a page inside its window and that the groups cover each
split exactly once."""

import itertools

import pytest


def _walk(n, split, ps, fixed=True):
    """Yield (split index, group start, window page index) as the kernel
    visits them; ``fixed=False`` replays the window end the kernel first had."""
    shift = ps.bit_length() - 1
    ns = (n + split - 1) // split
    for s in range(ns):
        t_begin, t_end = s * split, min(n, (s + 1) * split)
        w0 = t_begin
        while w0 < t_end:
            lp_base = w0 >> shift
            if fixed:
                w_end = min(t_end, (lp_base + 64) << shift)
            else:
                w_end = min(t_end, w0 + (64 << shift))
            for t0 in range(w0, w_end, 16):
                yield s, t0, (t0 >> shift) - lp_base
            w0 = w_end


SPLITS = [16, 48, 128, 320, 1040, 2064, 4112, 16400, 20000]


@pytest.mark.parametrize("ps", [16, 32, 64, 128, 256])
def test_every_group_indexes_its_window(ps):
    for split, n in itertools.product(SPLITS, [1, 15, 17, 1000, 4200, 32800, 40000]):
        seen = []
        for s, t0, i in _walk(n, split, ps):
            assert 0 <= i < 64, (ps, split, n, s, t0, i)
            assert t0 % 16 == 0
            seen.append(t0)
        # the groups tile 0 .. n exactly once, in order
        assert seen == list(range(0, n, 16)), (ps, split, n)


@pytest.mark.parametrize("n,split,ps", [(4200, 2064, 32), (32800, 16400, 256),
                                        (40000, 20000, 256)])
def test_the_first_window_end_left_the_window(n, split, ps):
    # the cases where the first kernel's window end indexed page 64
    assert any(i >= 64 for _, _, i in _walk(n, split, ps, fixed=False))
    assert all(i < 64 for _, _, i in _walk(n, split, ps))
