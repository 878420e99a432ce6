"""GPU parity of the matrix-core page stream (BF16 decode) against the CPU oracle.

Covers what the stream's own structure adds on top of the generic decode
tests: a block range crossing more segments than its cached query rows, the
shapes it instantiates (with NaN bytes in every row past the frontiers, which
the page loads' ranges must keep out), bitwise invariance to physical page
placement, and repeated calls on one workspace.
Bar: max-abs 2e-3 against the fp64 oracle.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from tests.drivers import build_device, build_oracle, device_decode, say

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _check(wl, tag, **kw):
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl, **kw)
    assert np.array_equal(dp.table.cpu().numpy(), pool.table)
    got = device_decode(dp, wl, 0)
    ref = A.paged_decode(st, 0, wl.table_rows, wl.seq_lens, wl.q(0), wl.sm_scale)
    err = float(np.max(np.abs(got - ref)))
    say(f"  {tag}: max abs err {err:.3g}")
    assert err <= TOL
    return dp, got


@pytest.mark.parametrize("D", [128, 256])
def test_stream_block_crossing_many_segments(D):
    # one long entry and seven short ones: the block that reaches the short
    # entries crosses ~15 segments (past the partials kept in registers and
    # past the cached query rows)
    hist = [65000, 40, 10, 63, 64, 1, 100, 20]
    wl = workloads.small(61, "BF16", hist=hist, C=8, S=65536, Hq=16, H=4, D=D, M=1100)
    say(f"decode {wl.name} B={wl.B} H={wl.H}")
    dp, _ = _check(wl, "many segments")
    dp.close()


@pytest.mark.parametrize("gq,D", [(8, 128), (8, 64), (4, 64), (1, 128), (2, 64), (4, 256), (1, 256), (8, 256)])
def test_stream_shapes(gq, D):
    # planes start as 0xFF bytes (NaN bf16): rows past every frontier hold them
    H = 2
    hist = [0, 63, 64, 777, 1500, 1500, 5]
    fork = [None, None, None, None, None, (4, 1500), None]
    cow = [False] * 5 + [True, False]
    wl = workloads.small(70 + gq + D, "BF16", hist=hist, fork=fork, cow=cow, C=7, S=2048, Hq=H * gq, H=H, D=D)
    say(f"decode BF16 gq={gq} D={D}, planes filled with 0xFF")
    dp, _ = _check(wl, f"gq={gq} D={D}", fill=0xFF)
    dp.close()


def test_stream_bitwise_invariant_to_page_permutation():
    # shared pages are read once for all sharers; the same histories in
    # private pages take another split (equal within rounding)
    wl = workloads.small(63, "BF16", hist=[700, 1000, 1000, 130], fork=[None, (0, 640), (0, 700), None],
                         cow=[False, False, True, False], C=4, S=2048, Hq=8, H=2, D=128)
    outs = []
    for fo in (None, np.arange(wl.M)[::-1].copy(), np.random.default_rng(1).permutation(wl.M)):
        dp, _, _ = build_device(wl, free_order=fo)
        outs.append(device_decode(dp, wl, 0))
        dp.close()
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    dp, _, _ = build_device(wl, privatize=True)
    private = device_decode(dp, wl, 0)
    dp.close()
    assert float(np.max(np.abs(private - outs[0]))) <= 1e-5


def test_stream_repeated_calls_on_one_workspace():
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev
    wl = workloads.small(64, "BF16", hist=[3000, 2000, 1, 900], C=4, S=4096, Hq=8, H=2, D=128)
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    dev = dp.device
    q = _dev(wl.q(0), dev)
    msl = max(wl.seq_lens)
    ws = dp.workspace(wl.B, wl.Hq, msl)
    rows, lens = i32(wl.table_rows, dev), i32(wl.seq_lens, dev)
    outs = []
    for _ in range(3):
        out = torch.full((wl.B, wl.Hq, wl.D), float("nan"), dtype=torch.float32, device=dev)
        dp.decode(0, wl.Hq, rows, lens, msl, q, wl.sm_scale, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    ref = A.paged_decode(st, 0, wl.table_rows, wl.seq_lens, wl.q(0), wl.sm_scale)
    assert float(np.max(np.abs(outs[0] - ref))) <= TOL
    # the arrival counters are back at zero: a smaller batch on the same workspace
    sub = [1, 3]
    out = torch.full((2, wl.Hq, wl.D), float("nan"), dtype=torch.float32, device=dev)
    sub_lens = [wl.seq_lens[b] for b in sub]
    dp.decode(0, wl.Hq, i32([wl.table_rows[b] for b in sub], dev), i32(sub_lens, dev), max(sub_lens),
              q[sub].contiguous(), wl.sm_scale, out, ws)
    torch.cuda.synchronize()
    ref_sub = A.paged_decode(st, 0, [wl.table_rows[b] for b in sub], sub_lens, wl.q(0)[sub], wl.sm_scale)
    assert float(np.max(np.abs(out.cpu().numpy() - ref_sub))) <= TOL
    dp.close()


@pytest.mark.parametrize("profile", ["BF16", "INT8_G64"])
@pytest.mark.parametrize("npages", [32, 33, 56, 57])
def test_combine_piece_counts_at_round_edges(profile, npages):
    # one entry of npages pages at two KV heads: 2 * npages stream positions
    # over the 512 blocks of the run, one page each, so each (entry, head)
    # output folds exactly npages pieces -- the combine's rounds end at 32
    # (scalar ids) and 56 (the record's inline ids); 57 takes the overflow list
    wl = workloads.small(90 + npages, profile, hist=[64 * npages - 7], C=1, S=4096, Hq=8, H=2, D=128)
    say(f"decode {profile}: one entry of {npages} pages, {npages} pieces per output")
    dp, _ = _check(wl, f"{npages} pieces")
    dp.close()
