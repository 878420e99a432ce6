"""GPU parity of speculative units against the oracle: verify a draft chunk,
commit the accepted prefix, trim the trailing pages into each sequence's
reservation, then run the next unit from the new frontiers.

Bar: block tables, lease accounting and reservations bit-exact after every
step; verify outputs within max-abs 2e-3 of the fp64 oracle.  Planes start as
0xFF bytes (NaN) so a read past any frontier would show.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from tests.drivers import build_device, build_oracle, say
from workloads.device_driver import _dev
from workloads.gen import bf16_normal, rng_for

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _state_equal(dp, pool, seqs, sids, B):
    assert np.array_equal(dp.table.cpu().numpy(), pool.table)
    assert dp.stats() == pool.stats()
    for b in range(B):
        row, frontier, mapped = dp.info(seqs[b])
        assert (row, frontier, mapped) == (pool.row_of(sids[b]), pool.frontier_of(sids[b]),
                                           len(pool.pages_of(sids[b])))
        assert dp.reservation(seqs[b]) == len(pool.reserved_of(sids[b]))


def _verify_both(dp, st, wl, n0, T, q_bits, layer=0):
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    dev = dp.device
    cu = [0]
    for t in T:
        cu.append(cu[-1] + t)
    out = torch.empty((cu[-1], wl.Hq, wl.D), dtype=torch.float32, device=dev)
    msl, mql = max(n + t for n, t in zip(n0, T)), max(T)
    ws = dp.workspace(wl.B, wl.Hq, msl, mql)
    dp.verify(layer, wl.Hq, i32(wl.table_rows, dev), i32(n0, dev), i32(cu, dev), cu[-1], mql, msl,
              _dev(q_bits, dev), wl.sm_scale, out, ws)
    torch.cuda.synchronize()
    ref = A.paged_verify(st, layer, wl.table_rows, n0, cu, q_bits, wl.sm_scale)
    return float(np.max(np.abs(out.cpu().numpy() - ref)))


@pytest.mark.parametrize("gq,D", [(4, 128), (8, 64)])
def test_speculative_rounds_commit_trim_and_reuse(gq, D):
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    H = 2
    # frontiers mid-page, at a page end, and at 0; draft windows crossing pages
    hist, T1 = [700, 1023, 0], [70, 9, 130]
    wl = workloads.small(120 + gq, "BF16", hist=hist, step=T1, C=4, S=2048, Hq=H * gq, H=H, D=D, mode="verify")
    pool, st, sids = build_oracle(wl)
    dp, seqs, _ = build_device(wl, fill=0xFF)
    _state_equal(dp, pool, seqs, sids, wl.B)
    err = _verify_both(dp, st, wl, hist, T1, wl.q(0))
    say(f"round 1 gq={gq} D={D}: max abs err {err:.3g}")
    assert err <= TOL

    r = rng_for(9100 + gq, 0)
    n0 = list(hist)
    for rnd, accepted in enumerate(([3, 9, 1], [1, 2, 64])):
        Tp = T1 if rnd == 0 else T2
        for b in range(wl.B):
            a = min(accepted[b], Tp[b])
            assert pool.commit_accepted(sids[b], Tp[b], a) == "OK"
            dp.commit_accepted(seqs[b], Tp[b], a)
            n0[b] += a
        _state_equal(dp, pool, seqs, sids, wl.B)
        assert sum(len(pool.reserved_of(s)) for s in sids.values()) > 0   # trailing pages went to reservations
        # the next unit: map the draft rows (from the reservations first), append, verify
        T2 = [int(x) for x in r.integers(1, 100, size=wl.B)]
        k = bf16_normal(r, (sum(T2), H, D))
        v = bf16_normal(r, (sum(T2), H, D))
        q = bf16_normal(r, (sum(T2), wl.Hq, D))
        cu = np.concatenate([[0], np.cumsum(T2)]).astype(int)
        for b in range(wl.B):
            assert pool.ensure_mapped(sids[b], n0[b] + T2[b]) == ("OK", 0)
            dp.ensure_mapped(seqs[b], n0[b] + T2[b])
            st.append(0, wl.table_rows[b], n0[b], k[cu[b]:cu[b + 1]], v[cu[b]:cu[b + 1]])
        dev = dp.device
        dp.append(0, i32(wl.table_rows, dev), i32(n0, dev), i32(list(cu), dev), int(cu[-1]), _dev(k, dev),
                  _dev(v, dev))
        torch.cuda.synchronize()
        _state_equal(dp, pool, seqs, sids, wl.B)
        err = _verify_both(dp, st, wl, n0, T2, q)
        say(f"round {rnd + 2} gq={gq} D={D} n0={n0} T={T2}: max abs err {err:.3g}")
        assert err <= TOL
    for b in range(wl.B):
        pool.release(sids[b])
        dp.release(seqs[b])
    torch.cuda.synchronize()
    assert dp.stats() == pool.stats() == (0, 0, wl.M)
    dp.close()
