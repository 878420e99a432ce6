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
    held = [g for s in pool.spaces.values() for g in s.reserve]
    assert len(set(held)) == len(held) == reserved                  # a group sits in one reservation
    assert not set(held) & set(pool.free)
    assert set(pool.free) | set(held) == set(np.flatnonzero(refs == 0))   # free or held <=> unreferenced
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
            op = rng.integers(0, 9)
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
            elif op == 5 and live:
                sid = list(live)[int(rng.integers(len(live)))]
                st, deficit = pool.reserve(sid, int(rng.integers(0, 4)))
                assert (st == OP.OK) == (deficit == 0)
            elif op == 6 and live:
                # a speculative unit: map the draft rows, commit a prefix, trim
                sid = list(live)[int(rng.integers(len(live)))]
                F = pool.frontier_of(sid)
                T = int(rng.integers(1, 80))
                if F + T <= S and pool.ensure_mapped(sid, F + T)[0] == OP.OK:
                    a = int(rng.integers(1, T + 1))
                    assert pool.commit_accepted(sid, T, a) == OP.OK
                    assert pool.frontier_of(sid) == F + a
                    assert len(pool.pages_of(sid)) == -(-(F + a) // 64)
            elif op == 7 and live:
                sid = list(live)[int(rng.integers(len(live)))]
                pool.trim(sid, int(rng.integers(0, S + 1)))
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


# ------------------------------------------------------------------ speculative units --
def test_draft_pool_pages_closed_form_and_worst_lead():
    from oracle.geometry import draft_pool_pages
    M, C = 4096, 8
    assert draft_pool_pages(M, C, 1) == M                 # no draft window: no lead
    for K in (2, 5, 64, 65):
        assert draft_pool_pages(M, C, K) == M + C          # a lead of 1..64 tokens: one page per row
    assert draft_pool_pages(M, C, 66) == M + 2 * C
    # the extra pages of one row for a K - 1 token lead, over every frontier,
    # never exceed the per-row term, and reach it
    for K in (2, 17, 64, 65, 66, 130):
        worst = max(-(-(f + K - 1) // 64) - -(-f // 64) for f in range(0, 256))
        assert worst == (draft_pool_pages(M, 1, K) - M)
    with pytest.raises(ValueError):
        draft_pool_pages(M, C, 0)


def test_commit_accepted_trims_and_returns_leases_to_the_reservation():
    M = 64
    pool = OP.OraclePool(S=4096, C=2, M=M, free_order=np.arange(M)[::-1])
    sid = pool.open(0)
    assert pool.ensure_mapped(sid, 1000) == (OP.OK, 0)
    pool.commit(sid, 1000)                                   # 16 pages, tail at 40 columns
    assert pool.ensure_mapped(sid, 1300) == (OP.OK, 0)       # draft rows [1000, 1300): 21 pages
    drafted = pool.pages_of(sid)
    assert len(drafted) == 21 and pool.stats() == (21, 0, M - 21)
    assert pool.commit_accepted(sid, 300, 10) == OP.OK       # frontier 1010: ceil(1010/64) = 16 pages kept
    assert pool.frontier_of(sid) == 1010
    assert pool.pages_of(sid) == drafted[:16]                # the last partial page stays
    assert pool.reserved_of(sid) == drafted[16:]             # removed leases, in block order
    assert pool.stats() == (16, 5, M - 21)                   # not back to the global capacity
    assert np.all(pool.table[0, 16:] == -1)
    # the next unit maps from the reservation first, in its order
    assert pool.ensure_mapped(sid, 1010 + 150) == (OP.OK, 0)
    assert pool.pages_of(sid)[16:] == drafted[16:19]
    assert pool.stats() == (19, 2, M - 21)
    # release returns reservation to the back of the free list, after the pages
    pool.release(sid)
    assert list(pool.free)[-2:] == drafted[19:21]
    assert pool.stats() == (0, 0, M)
    _check_invariants(pool)


def test_commit_accepted_bounds_and_cancelled_rows():
    pool = OP.OraclePool(S=1024, C=1, M=16)
    sid = pool.open(0)
    pool.ensure_mapped(sid, 70)
    pool.commit(sid, 60)
    assert pool.commit_accepted(sid, 5, 0) == OP.INVALID          # a live row accepts at least one token
    assert pool.commit_accepted(sid, 5, 6) == OP.INVALID          # never more than it produced
    assert pool.commit_accepted(sid, 0, 0, cancelled=True) == OP.INVALID
    assert pool.commit_accepted(sid, 5, 1, cancelled=True) == OP.INVALID   # a cancelled row accepts none
    assert pool.commit_accepted(sid, 80, 1) == OP.UNMAPPED        # produced rows must have been mapped
    assert pool.frontier_of(sid) == 60 and len(pool.pages_of(sid)) == 2
    assert pool.commit_accepted(sid, 5, 0, cancelled=True) == OP.OK
    assert pool.frontier_of(sid) == 60 and len(pool.pages_of(sid)) == 1   # trimmed to the frontier
    assert pool.stats() == (1, 1, 14)
    # a trim never cuts below the committed frontier, whatever the provisional extent
    pool.ensure_mapped(sid, 200)
    assert pool.trim(sid, 0) == OP.OK and len(pool.pages_of(sid)) == 1
    pool.ensure_mapped(sid, 200)
    assert pool.trim(sid, 129) == OP.OK and len(pool.pages_of(sid)) == 3  # provisional 129 keeps 3 pages
    _check_invariants(pool)


def test_reserve_shortfall_moves_nothing():
    pool = OP.OraclePool(S=1024, C=2, M=16)
    a, b = pool.open(0), pool.open(1)
    assert pool.reserve(a, 10) == (OP.OK, 0)
    assert pool.reserve(b, 7) == (OP.CAPACITY, 1)
    assert pool.stats() == (0, 10, 6)
    # b can map only what is left globally; a maps from its reservation
    assert pool.ensure_mapped(b, 64 * 7) == (OP.CAPACITY, 1)
    assert pool.ensure_mapped(a, 64 * 12) == (OP.OK, 0)      # 10 held + 2 from the free list
    assert pool.stats() == (12, 0, 4)
    _check_invariants(pool)


def test_rejected_rows_past_the_frontier_are_outside_the_valid_domain():
    """After a speculative unit keeps 3 of 7 draft rows, the rejected rows stay
    in the tail page; the next unit's rows overwrite them, and decode equals
    contiguous attention over the accepted history alone (brute force)."""
    from oracle import attention as A
    from oracle.codecs import bf16_to_f32
    H, D, Hq = 2, 64, 4
    pool = OP.OraclePool(S=512, C=1, M=8, free_order=np.arange(8)[::-1])
    st = OracleStore(pool, "BF16", H, D, 1)
    r = rng_for(77, 0)
    sid = pool.open(0)
    hist_k, hist_v = bf16_normal(r, (100, H, D)), bf16_normal(r, (100, H, D))
    pool.ensure_mapped(sid, 100)
    st.append(0, 0, 0, hist_k, hist_v)
    pool.commit(sid, 100)
    dk, dv = bf16_normal(r, (7, H, D), 1.0, 30.0), bf16_normal(r, (7, H, D), 1.0, 30.0)   # loud draft rows
    pool.ensure_mapped(sid, 107)
    st.append(0, 0, 100, dk, dv)
    assert pool.commit_accepted(sid, 7, 3) == OP.OK
    nk, nv = bf16_normal(r, (1, H, D)), bf16_normal(r, (1, H, D))
    pool.ensure_mapped(sid, 104)
    st.append(0, 0, 103, nk, nv)                             # the next canonical row at 103
    q = bf16_normal(r, (1, Hq, D))
    got = A.paged_decode(st, 0, [0], [104], q, 0.125)
    K = bf16_to_f32(np.concatenate([hist_k, dk[:3], nk])).astype(np.float64)
    V = bf16_to_f32(np.concatenate([hist_v, dv[:3], nv])).astype(np.float64)
    qf = bf16_to_f32(q).astype(np.float64)
    for j in range(Hq):
        s_ = K[:, j // 2] @ qf[0, j] * 0.125
        w = np.exp(s_ - s_.max())
        ref = (w / w.sum()) @ V[:, j // 2]
        assert np.max(np.abs(got[0, j] - ref)) < 1e-12


def test_store_refuses_writes_into_shared_pages():
    # writer-cardinality rule: a page two address spaces reference is immutable.
    # Both a shared full page and a shared partial tail refuse a write; after
    # the tail copy the fork writes its private page and the parent's bytes stay.
    pool = OP.OraclePool(S=1024, C=2, M=32)
    st = OracleStore(pool, "INT8_G64", H=1, D=64, layers=1)
    a = pool.open(0)
    pool.ensure_mapped(a, 100)
    rng = rng_for(81)
    k, v = bf16_normal(rng, (100, 1, 64)), bf16_normal(rng, (100, 1, 64))
    st.append(0, 0, 0, k, v)
    pool.commit(a, 100)
    b = pool.fork(a, 100, 1)
    row = bf16_normal(rng, (1, 1, 64))
    with pytest.raises(ValueError, match="shared"):
        st.append(0, 1, 10, row, row)          # a full page both rows map
    with pytest.raises(ValueError, match="shared"):
        st.append(0, 1, 100, row, row)         # the shared tail, at the fork's frontier
    with pytest.raises(ValueError, match="shared"):
        st.append(0, 0, 100, row, row)         # the parent may not write it either
    before = {r: arr.copy() for r, arr in st.planes[0].items()}
    _, (src, dst, cols) = pool.cow_tail(b)
    st.cow_copy(src, dst, cols)
    st.append(0, 1, 100, row, row)             # now private
    st.append(0, 0, 100, row, row)
    for r, arr in st.planes[0].items():
        assert np.array_equal(arr[src, :, :100 - 64], before[r][src, :, :100 - 64])
