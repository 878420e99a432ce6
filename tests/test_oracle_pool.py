"""Pins of oracle.pool / oracle.store: the pages' worked example and invariant list."""

import os

import numpy as np
import pytest

from oracle import pool as OP
from oracle.store import OracleStore
from workloads.gen import bf16_normal, rng_for

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _fork_example():
    with open(os.path.join(GOLD, "fork_worked_example.txt")) as f:
        return {k: int(v) for k, v in (ln.split() for ln in f if ln.strip() and not ln.startswith("#"))}


def _check_invariants(pool: OP.OraclePool):
    alloc, reserved, avail = pool.stats()
    assert alloc + reserved + avail == pool.M                       # lease accounting
    refs = np.zeros(pool.M, dtype=np.int64)
    for s in pool.spaces.values():
        assert len(set(s.pages)) == len(s.pages)                    # one logical block per page
        for g in s.pages:
            refs[g] += 1
        row = pool.table[s.row]
        assert list(row[: len(s.pages)]) == s.pages and np.all(row[len(s.pages):] == -1)
        assert s.frontier <= 64 * len(s.pages)
    assert np.array_equal(refs, pool.refs)                          # refs == memberships
    assert set(pool.free) == set(np.flatnonzero(refs == 0))         # free <=> unreferenced
    assert alloc == int(np.count_nonzero(refs))                     # aliases counted once


def test_fork_worked_example():
    ex = _fork_example()
    P, F = ex["P"], ex["F"]
    pool = OP.OraclePool(S=4096, C=2, M=128)
    a = pool.open(0)
    assert pool.ensure_mapped(a, F) == (OP.OK, 0)
    pool.commit(a, F)
    b = pool.fork(a, F, 1)
    assert pool.frontier_of(b) == F != ex["not_rounded_to"]
    pa, pb = pool.pages_of(a), pool.pages_of(b)
    full = F // P
    assert full == ex["full_pages"] and pa[:full] == pb[:full]
    # the partial tail is shared until the writer copies it
    assert pb[full] == pa[full] and pool.refs[pa[full]] == 2
    assert pool.ensure_mapped(b, F + 1) == (OP.SHARED_WRITE, 0)
    st, (src, dst, cols) = pool.cow_tail(b)
    assert st == OP.OK and cols == ex["tail_columns"] and src == pa[full] and dst != src
    assert pool.pages_of(b)[:full] == pa[:full] and pool.pages_of(b)[full] == dst
    assert pool.ensure_mapped(b, F + 1) == (OP.OK, 0)
    # both writers now own a private tail; full pages stay shared
    assert all(pool.refs[g] == 2 for g in pa[:full]) and pool.refs[pa[full]] == 1
    _check_invariants(pool)


def test_aligned_fork_needs_no_copy():
    pool = OP.OraclePool(S=8192, C=2, M=200)
    a = pool.open(0)
    pool.ensure_mapped(a, 4096)
    pool.commit(a, 4096)
    b = pool.fork(a, 4096, 1)
    assert pool.cow_tail(b) == (OP.OK, None)
    # growth past an aligned fork lands on a fresh private page
    assert pool.ensure_mapped(b, 4097) == (OP.OK, 0)
    assert pool.pages_of(b)[64] not in pool.pages_of(a) and pool.refs[pool.pages_of(b)[64]] == 1
    _check_invariants(pool)


def test_shortfall_is_returned_not_raised_and_allocates_nothing():
    pool = OP.OraclePool(S=1024, C=2, M=16)
    a, b = pool.open(0), pool.open(1)
    assert pool.ensure_mapped(a, 640) == (OP.OK, 0)                  # 10 pages
    before = pool.stats()
    assert pool.ensure_mapped(b, 8 * 64 + 1) == (OP.CAPACITY, 3)    # needs 9, 6 left
    assert pool.stats() == before and pool.pages_of(b) == []
    assert pool.ensure_mapped(b, 6 * 64) == (OP.OK, 0)
    assert pool.stats() == (16, 0, 0)
    assert pool.ensure_mapped(a, 2000) == (OP.INVALID, 0)            # beyond S
    _check_invariants(pool)


def test_decode_allocates_only_at_page_crossings():
    pool = OP.OraclePool(S=2048, C=1, M=32)
    a = pool.open(0)
    for n in range(0, 700):
        before = pool.stats()[0]
        assert pool.ensure_mapped(a, n + 1) == (OP.OK, 0)
        assert pool.stats()[0] - before == (1 if n % 64 == 0 else 0)
        pool.commit(a, n + 1)
    # a lower bound never trims
    assert pool.ensure_mapped(a, 10) == (OP.OK, 0) and len(pool.pages_of(a)) == 11


def test_release_frees_on_last_reference_in_block_order():
    pool = OP.OraclePool(S=1024, C=3, M=48, free_order=list(range(47, -1, -1)))
    a = pool.open(0)
    pool.ensure_mapped(a, 200)
    pool.commit(a, 200)
    b = pool.fork(a, 130, 1)
    pa = pool.pages_of(a)
    assert pa == [47, 46, 45, 44]
    pool.release(a)
    # pages still referenced by b stay allocated, the rest go back in block order
    assert list(pool.free)[-1:] == [44] and pool.refs[47] == 1
    pool.release(b)
    assert list(pool.free)[-3:] == [47, 46, 45]
    assert pool.stats() == (0, 0, 48)
    assert np.all(pool.table == -1)


def test_random_operation_sequences_keep_invariants():
    rng = np.random.default_rng(7)
    for trial in range(30):
        C = int(rng.integers(1, 9))
        S = int(rng.integers(64, 2048))
        lo, hi = -(-S // 64), C * -(-S // 64)
        lo = max(lo, C)
        M = int(rng.integers(lo, hi + 1))
        pool = OP.OraclePool(S=S, C=C, M=M, free_order=rng.permutation(M))
        live = {}
        for _ in range(200):
            op = rng.integers(0, 6)
            free_rows = [r for r in range(C) if r not in live.values()]
            if op == 0 and free_rows:
                live[pool.open(free_rows[0])] = free_rows[0]
            elif op == 1 and live:
                sid = list(live)[int(rng.integers(len(live)))]
                n = pool.frontier_of(sid) + int(rng.integers(0, 100))
                st, deficit = pool.ensure_mapped(sid, min(n, S))
                if st == OP.OK:
                    pool.commit(sid, min(n, S))
                elif st == OP.CAPACITY:
                    assert deficit > 0
            elif op == 2 and live and free_rows:
                src = list(live)[int(rng.integers(len(live)))]
                F = int(rng.integers(0, pool.frontier_of(src) + 1))
                live[pool.fork(src, F, free_rows[0])] = free_rows[0]
            elif op == 3 and live:
                pool.cow_tail(list(live)[int(rng.integers(len(live)))])
            elif op == 4 and live:
                sid = list(live)[int(rng.integers(len(live)))]
                pool.release(sid)
                del live[sid]
            _check_invariants(pool)


def test_store_cow_copies_only_committed_columns_of_every_plane():
    pool = OP.OraclePool(S=1024, C=2, M=32)
    st = OracleStore(pool, "K8V4", H=2, D=256, layers=2)
    a = pool.open(0)
    pool.ensure_mapped(a, 100)
    rng = rng_for(8)
    for layer in range(2):
        k, v = bf16_normal(rng, (100, 2, 256)), bf16_normal(rng, (100, 2, 256))
        st.append(layer, 0, 0, k, v)
    pool.commit(a, 100)
    b = pool.fork(a, 100, 1)
    _, (src, dst, cols) = pool.cow_tail(b)
    st.cow_copy(src, dst, cols)
    for lp in st.planes:
        for arr in lp.values():
            assert np.array_equal(arr[dst, :, :cols], arr[src, :, :cols])
            assert not np.any(arr[dst, :, cols:])
    for layer in range(2):
        ka, va = st.gather(layer, 0, 100)
        kb, vb = st.gather(layer, 1, 100)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)


def test_open_rejects_leased_row_and_fork_beyond_frontier():
    pool = OP.OraclePool(S=1024, C=2, M=16)
    a = pool.open(0)
    with pytest.raises(ValueError):
        pool.open(0)
    pool.ensure_mapped(a, 10)
    pool.commit(a, 10)
    with pytest.raises(ValueError):
        pool.fork(a, 11, 1)
