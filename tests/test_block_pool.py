"""Host block pool (include/pa_blocks.h): unit cases and a randomized
comparison with a small reference model written here from the behaviour the
header states (on-demand blocks, sharing by fork, copy-on-write of a shared
partially filled block, lowest free id first)."""

import heapq

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

BS = 16


@pytest.fixture(scope="module")
def pa():
    import __graft_entry__
    b = __graft_entry__._build_module()
    import os
    if not os.path.exists(b.LIB_PATH):
        b.build()
    import decode_attention_paged_07_amd as mod
    return mod


def row(n=8):
    return np.full(n, -1, np.int32)


def test_growth_takes_lowest_free_ids(pa):
    p = pa.BlockPool(10, BS)
    r = row()
    assert p.append(r, 0, 17) is None                # 17 tokens -> 2 blocks
    assert r[:2].tolist() == [0, 1] and p.num_free == 8
    assert p.append(r, 17, 15) is None               # fills block 1 (slots 1..15): no new block
    assert p.num_free == 8
    assert p.append(r, 32, 1) is None                # position 32 starts block 2
    assert r[2] == 2 and p.num_free == 7
    assert [p.refcount(b) for b in range(4)] == [1, 1, 1, 0]


def test_fork_shares_and_copy_on_write(pa):
    p = pa.BlockPool(8, BS)
    a, b = row(), row()
    p.append(a, 0, 20)                               # blocks 0, 1 (block 1 holds 4 tokens)
    p.fork(a, 20, b)
    assert b[:2].tolist() == [0, 1] and p.refcount(0) == 2 and p.refcount(1) == 2
    cow = p.append(b, 20, 1)                         # b writes into shared block 1: copy it
    assert cow == (1, 2) and b[:2].tolist() == [0, 2]
    assert p.refcount(1) == 1 and p.refcount(2) == 1 and p.refcount(0) == 2
    assert p.append(a, 20, 1) is None                # a now owns block 1 alone: no copy
    assert a[:2].tolist() == [0, 1]


def test_no_copy_when_the_next_token_starts_a_block(pa):
    p = pa.BlockPool(8, BS)
    a, b = row(), row()
    p.append(a, 0, 32)
    p.fork(a, 32, b)
    assert p.append(b, 32, 1) is None                # shared blocks stay shared
    assert b[:3].tolist() == [0, 1, 2] and p.refcount(0) == 2 and p.refcount(1) == 2


def test_release_frees_at_zero_and_rejects_overrelease(pa):
    p = pa.BlockPool(4, BS)
    a, b = row(), row()
    p.append(a, 0, 40)
    p.fork(a, 40, b)
    p.release(a, 40)
    assert p.num_free == 1 and p.refcount(0) == 1
    p.release(b, 40)
    assert p.num_free == 4
    with pytest.raises(ValueError):
        p.release(b, 40)                             # names free blocks now


def test_exhaustion_changes_nothing(pa):
    p = pa.BlockPool(3, BS)
    a = row()
    p.append(a, 0, 30)
    before = a.copy()
    with pytest.raises(pa.PoolExhausted):
        p.append(a, 30, 40)                          # needs 3 more blocks, 1 free
    assert np.array_equal(a, before) and p.num_free == 1
    p2 = pa.BlockPool(2, BS)
    x, y = row(), row()
    p2.append(x, 0, 5)
    p2.fork(x, 5, y)
    p2.append(y, 5, 1)                               # copy takes the last free block
    with pytest.raises(pa.PoolExhausted):
        p2.fork(x, 5, row()) or p2.append(x, 5, 20)


def test_argument_errors(pa):
    p = pa.BlockPool(4, BS)
    with pytest.raises(ValueError):
        p.append(row(2), 0, 33)                      # does not fit in 2 blocks
    with pytest.raises(ValueError):
        p.append(row(), 5, 1)                        # row names no live block
    with pytest.raises(ValueError):
        p.append(row(), 0, 0)
    with pytest.raises(TypeError):
        p.append(np.zeros(4, np.int64), 0, 1)
    with pytest.raises(ValueError):
        pa.BlockPool(0, BS)
    assert pa.pa_copy_blocks(0x1000, 0x2000, 0x3000, 0x4000, 1, 4, 100, None) == pa.PA_ERR_SHAPE
    assert pa.pa_copy_blocks(0x1008, 0x2000, 0x3000, 0x4000, 1, 4, 4096, None) == pa.PA_ERR_ALIGN
    assert pa.pa_copy_blocks(None, 0x2000, 0x3000, 0x4000, 1, 4, 4096, None) == pa.PA_ERR_NULL
    assert pa.pa_copy_blocks(None, None, None, None, 0, 4, 4096, None) == pa.PA_OK


# ---------------------------------------------------------------------------
# Randomized comparison with a reference model.
# ---------------------------------------------------------------------------

class ModelPool:
    """Reference behaviour: reference counts, a min-heap of free ids."""

    def __init__(self, n, bs):
        self.refs = [0] * n
        self.free = list(range(n))
        heapq.heapify(self.free)
        self.bs = bs

    def _take(self):
        b = heapq.heappop(self.free)
        self.refs[b] = 1
        return b

    def _drop(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            heapq.heappush(self.free, b)

    def append(self, r, n, k):
        have, need = -(-n // self.bs), -(-(n + k) // self.bs)
        if n + k > len(r) * self.bs:
            return "shape"
        cow = n % self.bs != 0 and self.refs[r[have - 1]] > 1
        if len(self.free) < need - have + cow:
            return "nomem"
        pair = None
        if cow:
            old = r[have - 1]
            nb = self._take()
            self._drop(old)
            r[have - 1] = nb
            pair = (old, nb)
        for i in range(have, need):
            r[i] = self._take()
        return pair

    def fork(self, src, n, dst):
        for i in range(-(-n // self.bs)):
            self.refs[src[i]] += 1
            dst[i] = src[i]

    def release(self, r, n):
        for i in range(-(-n // self.bs)):
            self._drop(r[i])


ops = st.lists(st.tuples(st.sampled_from(["append", "append", "fork", "release"]), st.integers(0, 9),
                         st.integers(0, 9), st.integers(1, 40)), min_size=1, max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops)
def test_random_operations_match_the_model(pa, seq_ops):
    n_blocks, max_blocks = 24, 6
    p = pa.BlockPool(n_blocks, BS)
    m = ModelPool(n_blocks, BS)
    rows, mrows, lens = {}, {}, {}
    for op, a, b, k in seq_ops:
        if op == "append":
            if a not in rows:
                rows[a], mrows[a], lens[a] = row(max_blocks), [-1] * max_blocks, 0
            expect = m.append(mrows[a], lens[a], k)
            if expect == "shape":
                with pytest.raises(ValueError):
                    p.append(rows[a], lens[a], k)
                continue
            if expect == "nomem":
                with pytest.raises(pa.PoolExhausted):
                    p.append(rows[a], lens[a], k)
                continue
            assert p.append(rows[a], lens[a], k) == expect
            lens[a] += k
        elif op == "fork":
            if a not in rows or b in rows:
                continue
            rows[b], mrows[b], lens[b] = row(max_blocks), [-1] * max_blocks, lens[a]
            p.fork(rows[a], lens[a], rows[b])
            m.fork(mrows[a], lens[a], mrows[b])
        else:
            if a not in rows:
                continue
            p.release(rows[a], lens[a])
            m.release(mrows[a], lens[a])
            del rows[a], mrows[a], lens[a]
        for s in rows:
            nb = -(-lens[s] // BS)
            assert rows[s][:nb].tolist() == mrows[s][:nb]
        assert [p.refcount(i) for i in range(n_blocks)] == m.refs
        assert p.num_free == len(m.free)
        # every live block is referenced exactly as often as rows name it
        count = [0] * n_blocks
        for s in rows:
            for i in rows[s][:-(-lens[s] // BS)]:
                count[i] += 1
        assert count == m.refs
