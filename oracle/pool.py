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
  * finish/release rules: drop references, free a page on its last one.

The free-list discipline is this build's reading (the pages leave it open and
say correctness must not depend on it): pages are taken from the front of a
FIFO seeded with a caller-given order of [0, M), and freed pages are appended
at its back in logical-block order.  The C ABI follows the same rule, so block
tables can be compared bit for bit.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import numpy as np

from .geometry import P, ceil_div, logical_pages, m_bounds

OK, CAPACITY, SHARED_WRITE, INVALID, STALE = "OK", "CAPACITY", "SHARED_WRITE", "INVALID", "STALE"


@dataclass
class AddressSpace:
    row: int
    pages: list = field(default_factory=list)   # logical block -> page-group id
    frontier: int = 0                            # committed frontier (tokens)


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
        """(allocated, reserved, available); reserved is always 0 here."""
        available = len(self.free)
        return self.M - available, 0, available

    def _alloc(self) -> int:
        g = self.free.popleft()
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
        if need > len(self.free):
            return CAPACITY, need - len(self.free)
        for _ in range(need):
            g = self._alloc()
            s.pages.append(g)
            self.table[s.row, len(s.pages) - 1] = g
        return OK, 0

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
        if not self.free:
            return CAPACITY, None
        g2 = self._alloc()
        s.pages[b] = g2
        self.table[s.row, b] = g2
        self._unref(g)
        return OK, (g, g2, cols)

    def release(self, sid: int) -> None:
        s = self.spaces.pop(sid)
        for g in s.pages:
            self._unref(g)
        self.table[s.row, :] = -1

    # ------------------------------------------------------------ queries --
    def pages_of(self, sid: int) -> list:
        return list(self.spaces[sid].pages)

    def row_of(self, sid: int) -> int:
        return self.spaces[sid].row

    def frontier_of(self, sid: int) -> int:
        return self.spaces[sid].frontier
