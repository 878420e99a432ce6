"""Page-group allocator, address spaces and block table (oracle side).

Source: NInfer "Paged KV Context Store" maintainer page --
  * lease accounting equation: allocated + reserved + available = capacity;
  * KVAddressSpace descriptor: ordered logical-block -> page membership,
    committed frontier, execution-row lease;
  * device block-table matrix block_tables[N_logical, C] of I32 page IDs, one
    row per active address space (C-order [C][L] here; unmapped = -1);
  * ensure_mapped_to_tokens rules: lower-bound coverage, allocate only what
    is missing, fail only on a shortfall (returned, not raised), never move
    the frontier;
  * Fork: full pages before the frontier gain a reference; a partial tail is
    shared too and must be copied (COW) before any write; worked example
    F = 1000 -> 15 full pages + 40 tail columns, frontier not rounded down;
  * writer-cardinality rules: a page with several address-space references
    is immutable; a write into a shared tail is refused until it is copied;
  * finish/release rules: drop references, free a page on its last one;
  * speculative units: the accepted prefix is committed
    (1 <= accepted <= produced for a row that is not cancelled, 0 for a
    cancelled one), then the retained membership is
    NeededPages = ceil(max(committed, provisional) / P): trailing mappings past
    it are removed, the last partial page stays, and the removed device leases
    go back to the address space's own active reservation, not to the global
    available capacity; bytes past the frontier inside the kept page are not
    in the valid domain and are overwritten by the next canonical write;
  * the active reservation (growth entitlement) is released at finish.

The free-list discipline is this library's reading (the pages leave it open and
say correctness must not depend on it): pages are taken from the front of a
FIFO seeded with a caller-given order of [0, M), and freed pages are appended
at its back in logical-block order.  A reservation is a FIFO of concrete page
groups held by one address space: reserve() moves groups from the front of
the pool's FIFO to the back of the reservation, a trim appends the removed
groups there in logical-block order, a mapping takes from the reservation's
front before the pool's, and release returns the reservation to the back of
the pool's FIFO in its order.  The C ABI follows the same rules, so block
tables can be compared bit for bit.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np

from .geometry import P, ceil_div, logical_pages, m_bounds

OK, CAPACITY, SHARED_WRITE, INVALID, STALE, UNMAPPED = "OK", "CAPACITY", "SHARED_WRITE", "INVALID", "STALE", "UNMAPPED"


@dataclass
class AddressSpace:
    row: int
    pages: list = field(default_factory=list)   # logical block -> page-group id
    frontier: int = 0                            # committed frontier (tokens)
    reserve: deque = field(default_factory=deque)   # active reservation: held page groups


class OraclePool:
    def __init__(self, S: int, C: int, M: int, free_order=None):
        lo, hi = m_bounds(S, C)
        if not lo <= M <= hi:
            raise ValueError(f"M={M} outside [{lo}, {hi}]")
        self.S, self.C, self.M, self.L = S, C, M, logical_pages(S)
        order = list(range(M)) if free_order is None else [int(g) for g in free_order]
        if sorted(order) != list(range(M)):
            raise ValueError("free_order must be a permutation of [0, M)")
        self.free = deque(order)
        self.refs = np.zeros(M, dtype=np.int64)
        self.table = np.full((C, self.L), -1, dtype=np.int32)
        self.spaces: dict[int, AddressSpace] = {}
        self._next_id = 0

    # --------------------------------------------------------- accounting --
    def stats(self) -> tuple[int, int, int]:
        """(allocated, reserved, available): groups with references, groups
        held in reservations, groups in the pool's free list."""
        reserved = sum(len(s.reserve) for s in self.spaces.values())
        available = len(self.free)
        return self.M - reserved - available, reserved, available

    def _alloc(self, s: AddressSpace | None = None) -> int:
        g = s.reserve.popleft() if s is not None and s.reserve else self.free.popleft()
        assert self.refs[g] == 0
        self.refs[g] = 1
        return g

    def _unref(self, g: int) -> None:
        self.refs[g] -= 1
        assert self.refs[g] >= 0
        if self.refs[g] == 0:
            self.free.append(g)

    def _row_free(self, row: int) -> bool:
        return 0 <= row < self.C and all(s.row != row for s in self.spaces.values())

    def _new_space(self, row: int) -> int:
        sid = self._next_id
        self._next_id += 1
        self.spaces[sid] = AddressSpace(row=row)
        self.table[row, :] = -1
        return sid

    # --------------------------------------------------------- operations --
    def open(self, row: int) -> int:
        if not self._row_free(row):
            raise ValueError("table row not available")
        return self._new_space(row)

    def fork(self, src: int, F: int, row: int) -> int:
        """New address space sharing src's pages covering [0, F)."""
        s = self.spaces[src]
        if not 0 <= F <= s.frontier:
            raise ValueError("fork frontier beyond the committed frontier")
        if not self._row_free(row):
            raise ValueError("table row not available")
        sid = self._new_space(row)
        d = self.spaces[sid]
        n = ceil_div(F, P)
        d.pages = list(s.pages[:n])
        for g in d.pages:
            self.refs[g] += 1
        d.frontier = F
        self.table[row, :n] = d.pages
        return sid

    def ensure_mapped(self, sid: int, tokens: int) -> tuple[str, int]:
        """Map pages so [0, tokens) is covered; returns (status, deficit)."""
        s = self.spaces[sid]
        if tokens > self.S:
            return INVALID, 0
        if tokens > s.frontier and s.frontier % P:
            tail = s.frontier // P
            if tail < len(s.pages) and self.refs[s.pages[tail]] > 1:
                return SHARED_WRITE, 0
        need = ceil_div(tokens, P) - len(s.pages)
        if need <= 0:
            return OK, 0
        have = len(s.reserve) + len(self.free)
        if need > have:
            return CAPACITY, need - have
        for _ in range(need):
            g = self._alloc(s)
            s.pages.append(g)
            self.table[s.row, len(s.pages) - 1] = g
        return OK, 0

    def reserve(self, sid: int, n: int) -> tuple[str, int]:
        """Move n page groups from the pool's free list into the address
        space's reservation; a shortfall returns the deficit, moves nothing."""
        s = self.spaces[sid]
        if n > len(self.free):
            return CAPACITY, n - len(self.free)
        for _ in range(n):
            s.reserve.append(self.free.popleft())
        return OK, 0

    def trim(self, sid: int, provisional: int) -> str:
        """Keep NeededPages = ceil(max(frontier, provisional) / P) mappings;
        the trailing ones are removed and their groups, once unreferenced, go
        to the address space's reservation (in logical-block order)."""
        s = self.spaces[sid]
        if provisional > self.S:
            return INVALID
        keep = ceil_div(max(s.frontier, provisional), P)
        for b in range(keep, len(s.pages)):
            g = s.pages[b]
            self.refs[g] -= 1
            assert self.refs[g] >= 0
            if self.refs[g] == 0:
                s.reserve.append(g)
            self.table[s.row, b] = -1
        del s.pages[keep:]
        return OK

    def commit_accepted(self, sid: int, produced: int, accepted: int, cancelled: bool = False) -> str:
        """Close a speculative unit that wrote `produced` rows from the
        committed frontier: commit the accepted prefix, then trim to it."""
        s = self.spaces[sid]
        if produced < 1 or (accepted != 0 if cancelled else not 1 <= accepted <= produced):
            return INVALID
        if s.frontier + produced > P * len(s.pages):
            return UNMAPPED
        s.frontier += accepted
        return self.trim(sid, s.frontier)

    def commit(self, sid: int, frontier: int) -> str:
        s = self.spaces[sid]
        if frontier < s.frontier or frontier > P * len(s.pages):
            return INVALID
        s.frontier = frontier
        return OK

    def cow_tail(self, sid: int):
        """Private copy of a shared partial tail page.

        Returns (status, (src_page, dst_page, columns) or None).  Nothing to do
        when the frontier is page-aligned or the tail is already private.
        """
        s = self.spaces[sid]
        cols = s.frontier % P
        if cols == 0:
            return OK, None
        b = s.frontier // P
        g = s.pages[b]
        if self.refs[g] == 1:
            return OK, None
        if not s.reserve and not self.free:
            return CAPACITY, None
        g2 = self._alloc(s)
        s.pages[b] = g2
        self.table[s.row, b] = g2
        self._unref(g)
        return OK, (g, g2, cols)

    def release(self, sid: int) -> None:
        s = self.spaces.pop(sid)
        for g in s.pages:
            self._unref(g)
        self.free.extend(s.reserve)
        self.table[s.row, :] = -1

    # ------------------------------------------------------------ queries --
    def pages_of(self, sid: int) -> list:
        return list(self.spaces[sid].pages)

    def row_of(self, sid: int) -> int:
        return self.spaces[sid].row

    def frontier_of(self, sid: int) -> int:
        return self.spaces[sid].frontier

    def reserved_of(self, sid: int) -> list:
        return list(self.spaces[sid].reserve)
