"""Drive one workload through the oracle and through the device pool, in the same order.

History construction: roots in sequence order (open, map, append, commit),
then forks (fork at the source's frontier, map, append own history, commit).
Step: optional tail copy, map the step's tokens, one batched append of every
entry's new rows per layer, then decode (last token) or verify (the chunk).
"""

from __future__ import annotations

import sys

import numpy as np

from oracle.pool import OraclePool
from oracle.store import OracleStore


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ oracle --
def build_oracle(wl, free_order=None, privatize=False, layers=None):
    layers = range(wl.layers) if layers is None else layers
    pool = OraclePool(wl.S, wl.C, wl.M, free_order=wl.free_order if free_order is None else free_order)
    st = OracleStore(pool, wl.profile, wl.H, wl.D, wl.layers, scale_bytes=wl.scale_bytes)
    sids = {}
    for b in wl.order():
        row = wl.table_rows[b]
        if wl.fork[b] is None or privatize:
            sids[b] = pool.open(row)
            n_inh = 0
        else:
            src, F = wl.fork[b]
            sids[b] = pool.fork(sids[src], F, row)
            n_inh = F
            if wl.hist[b] > F and F % 64:          # own history starts inside the shared tail
                _, info = pool.cow_tail(sids[b])
                st.cow_copy(*info)
        if wl.hist[b] > n_inh:
            assert pool.ensure_mapped(sids[b], wl.hist[b]) == ("OK", 0)
            for layer in layers:
                k, v = wl.logical_kv(layer, b, wl.hist[b])
                st.append(layer, row, n_inh, k[n_inh:], v[n_inh:])
        pool.commit(sids[b], wl.hist[b])
    for b in range(wl.B):                           # every tail copy before any write of the step
        if wl.cow[b]:
            _, info = pool.cow_tail(sids[b])
            if info is not None:
                st.cow_copy(*info)
    for b in range(wl.B):
        assert pool.ensure_mapped(sids[b], wl.hist[b] + wl.step[b]) == ("OK", 0)
        for layer in layers:
            k, v = wl.step_kv(layer, b)
            st.append(layer, wl.table_rows[b], wl.hist[b], k, v)
    return pool, st, sids


def oracle_pool_only(wl, free_order=None):
    """Block-table bookkeeping alone (cheap at any size)."""
    pool = OraclePool(wl.S, wl.C, wl.M, free_order=wl.free_order if free_order is None else free_order)
    sids = {}
    for b in wl.order():
        row = wl.table_rows[b]
        if wl.fork[b] is None:
            sids[b] = pool.open(row)
        else:
            sids[b] = pool.fork(sids[wl.fork[b][0]], wl.fork[b][1], row)
            if wl.hist[b] > wl.fork[b][1] and wl.fork[b][1] % 64:
                pool.cow_tail(sids[b])
        assert pool.ensure_mapped(sids[b], wl.hist[b])[0] == "OK"
        pool.commit(sids[b], wl.hist[b])
    for b in range(wl.B):
        if wl.cow[b]:
            pool.cow_tail(sids[b])
    for b in range(wl.B):
        assert pool.ensure_mapped(sids[b], wl.hist[b] + wl.step[b])[0] == "OK"
    return pool, sids


# ------------------------------------------------------------------ device --
from workloads.device_driver import build_device, device_decode, device_verify, plane_np  # noqa: E402,F401
