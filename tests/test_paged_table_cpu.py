"""Host bookkeeping of the generation loop (int4_weight_kv_amd.block.PagedTable):
pages are taken from the free list only when a sequence first needs a
position on them, no page is shared, release returns them, and running out
of pages or of block-table room is an error."""

import numpy as np
import pytest

from int4_weight_kv_amd.block import PagedTable


def test_pages_taken_at_boundaries():
    t = PagedTable(num_pages=10, batch=3, max_pages_per_seq=4, page_size=64, seed=7)
    for b, L in enumerate([61, 0, 127]):
        t.ensure(b, L)
        t.lens[b] = L
    assert [int((t.table[b] >= 0).sum()) for b in range(3)] == [1, 0, 2]
    taken = []
    for step in range(8):  # positions 61..68, 0..7, 127..134
        before = (t.table >= 0).sum(axis=1).copy()
        for b in range(3):
            t.ensure(b, int(t.lens[b]) + 1)
        after = (t.table >= 0).sum(axis=1)
        # a page is taken exactly when the new token starts a page
        want = [int(t.lens[b] % 64 == 0 and t.lens[b] // 64 >= before[b]) for b in range(3)]
        assert list(after - before) == want, (step, t.lens.tolist())
        taken.append(list(after - before))
        t.lens += 1
    assert sum(map(sum, taken)) == 3  # seq 0 at 64, seq 1 at 0, seq 2 at 128
    used = t.table[t.table >= 0]
    assert len(set(used.tolist())) == len(used)  # no page shared
    assert len(used) + len(t.free) == 10
    # slots follow the table
    s = t.slots(2, [0, 63, 64, 128])
    assert s.tolist() == [t.table[2, 0] * 64, t.table[2, 0] * 64 + 63, t.table[2, 1] * 64, t.table[2, 2] * 64]


def test_release_and_exhaustion():
    t = PagedTable(num_pages=3, batch=2, max_pages_per_seq=4, page_size=64)
    t.ensure(0, 130)  # three pages
    assert len(t.free) == 0
    with pytest.raises(RuntimeError):
        t.ensure(1, 1)
    t.release(0)
    assert len(t.free) == 3 and np.all(t.table[0] < 0) and t.lens[0] == 0
    t.ensure(1, 64)
    assert int((t.table[1] >= 0).sum()) == 1
    with pytest.raises(RuntimeError):
        t.ensure(1, 4 * 64 + 1)  # beyond the block table row
