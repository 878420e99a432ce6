"""GPU parity of decode over shared pages, and of the plan / run split.

Entries that share leading pages (forks) read them once: the page stream
carries the query heads of every sharing entry in one matrix-core tile.  The
cases build fork trees (a chain, siblings, unaligned fork points with a copied
tail, a shared tail page that two entries see to different depths) at every
head grouping (tiles hold 16/GQ entries, so trees are capped differently),
compare with the fp64 oracle, and with the same histories in private pages
(a different split: equal within rounding, not bitwise).  The plan / run
split must give exactly the one-call result on every layer, and a run on a
plan of another batch shape must mark its outputs (NaN).  A run that appends
the step's rows itself must leave the same planes and outputs, bit for bit, as
kv_append followed by a run, on BF16 pages (also when a block holds more
new-token pages than it stages) and on every quantized profile (also when a
block writes many new rows).  Bar: max-abs 2e-3.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from tests.drivers import build_device, build_oracle, device_decode, say

pytestmark = pytest.mark.gpu

TOL = 2e-3

# entry 1 forks entry 0 at a page boundary, entry 2 inside a page (its own
# history starts in the shared tail: copied), entry 3 forks the fork 1 (a
# chain), entry 5 forks entry 4 at its frontier and appends into a fresh page
TREE_HIST = [2000, 2000, 1500, 3000, 1000, 640]
TREE_FORK = [None, (0, 1024), (0, 1000), (1, 1900), None, (4, 640)]


def _decode_vs_oracle(wl, tag):
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    assert np.array_equal(dp.table.cpu().numpy(), pool.table)
    got = device_decode(dp, wl, 0)
    dp.close()
    ref = A.paged_decode(st, 0, wl.table_rows, wl.seq_lens, wl.q(0), wl.sm_scale)
    err = float(np.max(np.abs(got - ref)))
    say(f"  {tag}: max abs err {err:.3g}")
    assert err <= TOL
    return got


@pytest.mark.parametrize("gq,D", [(4, 128), (8, 128), (1, 128), (2, 64), (4, 64), (4, 256), (2, 256)])
def test_decode_fork_tree(gq, D):
    H = 2
    wl = workloads.small(110 + gq + D, "BF16", hist=TREE_HIST, fork=TREE_FORK, C=6, S=4096, Hq=H * gq, H=H, D=D)
    say(f"fork tree gq={gq} D={D}")
    shared = _decode_vs_oracle(wl, f"gq={gq} D={D}")
    dp, _, _ = build_device(wl, privatize=True)
    private = device_decode(dp, wl, 0)
    dp.close()
    assert float(np.max(np.abs(shared - private))) <= 1e-5


def test_decode_shared_tail_seen_to_different_depths():
    # no step tokens: entry 1 forks entry 0 at 650 and attends [0, 650) while
    # entry 0 attends [0, 700) of the same tail page; entry 2 forks entry 1 at
    # 650 too (three entries on one tail page)
    wl = workloads.small(120, "BF16", hist=[700, 650, 650, 300], fork=[None, (0, 650), (1, 650), None],
                         step=[0, 0, 0, 0], C=4, S=2048, Hq=8, H=2, D=128)
    say("shared tail, step 0")
    _decode_vs_oracle(wl, "shared tail")


def test_decode_eight_entries_share_one_prefix():
    # GQ = 1: a tile holds all eight entries of the call
    fork = [None] + [(0, 4096)] * 7
    hist = [5000, 4096, 4100, 4200, 6000, 4500, 7000, 4160]
    wl = workloads.small(121, "BF16", hist=hist, fork=fork, C=8, S=8192, Hq=4, H=4, D=128)
    say("eight entries on one prefix")
    _decode_vs_oracle(wl, "eight sharers")


def test_decode_plan_once_run_every_layer():
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev
    wl = workloads.small(122, "BF16", hist=TREE_HIST, fork=TREE_FORK, C=6, S=4096, Hq=8, H=2, D=128, layers=3)
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    dev = dp.device
    msl = max(wl.seq_lens)
    rows, lens = i32(wl.table_rows, dev), i32(wl.seq_lens, dev)
    ws = dp.workspace(wl.B, wl.Hq, msl)
    dp.decode_plan(wl.Hq, rows, lens, msl, ws)
    for layer in range(wl.layers):
        q = _dev(wl.q(layer), dev)
        out = torch.full((wl.B, wl.Hq, wl.D), float("nan"), dtype=torch.float32, device=dev)
        dp.decode_run(layer, wl.B, wl.Hq, msl, q, wl.sm_scale, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        one_call = device_decode(dp, wl, layer)
        assert np.array_equal(got.view(np.uint32), one_call.view(np.uint32)), layer
        ref = A.paged_decode(st, layer, wl.table_rows, wl.seq_lens, wl.q(layer), wl.sm_scale)
        err = float(np.max(np.abs(got - ref)))
        say(f"  layer {layer}: max abs err {err:.3g}")
        assert err <= TOL
    dp.close()


def test_decode_run_on_a_plan_of_another_batch_marks_outputs():
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev
    wl = workloads.small(123, "BF16", hist=[900, 300, 1200, 64], C=4, S=2048, Hq=8, H=2, D=128)
    dp, _, _ = build_device(wl)
    dev = dp.device
    msl = max(wl.seq_lens)
    ws = dp.workspace(wl.B, wl.Hq, msl)
    dp.decode_plan(wl.Hq, i32(wl.table_rows, dev), i32(wl.seq_lens, dev), msl, ws)
    q = _dev(wl.q(0), dev)[:3].contiguous()
    out = torch.zeros((3, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    dp.decode_run(0, 3, wl.Hq, msl, q, wl.sm_scale, out, ws)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all())
    dp.close()


def _append_run_case(wl, tag):
    """Pool without the step rows + decode_append_run == kv_append + decode_run, bitwise (outputs and planes)."""
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev, plane_np
    pool, st, _ = build_oracle(wl)
    dp_a, _, step_a = build_device(wl, step_append=False)
    dp_b, _, _ = build_device(wl)
    dev = dp_a.device
    msl = max(wl.seq_lens)
    rows, lens = i32(wl.table_rows, dev), i32(wl.seq_lens, dev)
    ws_a, ws_b = dp_a.workspace(wl.B, wl.Hq, msl), dp_b.workspace(wl.B, wl.Hq, msl)
    dp_a.decode_plan(wl.Hq, rows, lens, msl, ws_a)
    dp_b.decode_plan(wl.Hq, rows, lens, msl, ws_b)
    for layer in range(wl.layers):
        q = _dev(wl.q(layer), dev)
        k, v = step_a[layer]
        out_a = torch.full((wl.B, wl.Hq, wl.D), float("nan"), dtype=torch.float32, device=dev)
        out_b = torch.full((wl.B, wl.Hq, wl.D), float("nan"), dtype=torch.float32, device=dev)
        dp_a.decode_append_run(layer, wl.B, wl.Hq, msl, k, v, q, wl.sm_scale, out_a, ws_a)
        dp_b.decode_run(layer, wl.B, wl.Hq, msl, q, wl.sm_scale, out_b, ws_b)
        torch.cuda.synchronize()
        ga, gb = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.array_equal(ga.view(np.uint32), gb.view(np.uint32)), (tag, layer)
        for role in dp_a.planes[layer]:
            assert np.array_equal(plane_np(dp_a, layer, role), plane_np(dp_b, layer, role)), (tag, layer, role)
        ref = A.paged_decode(st, layer, wl.table_rows, wl.seq_lens, wl.q(layer), wl.sm_scale)
        err = float(np.max(np.abs(ga - ref)))
        say(f"  {tag} layer {layer}: max abs err {err:.3g}")
        assert err <= TOL
    dp_a.close()
    dp_b.close()


@pytest.mark.parametrize("gq,D", [(4, 128), (2, 64), (4, 256)])
def test_decode_append_run_matches_append_then_run(gq, D):
    # forks with shared prefixes; new tokens at page starts, mid-page and page ends
    hist = [2000, 2000, 1500, 3000, 1000, 640]
    fork = [None, (0, 1024), (0, 1000), (1, 1900), None, (4, 640)]
    wl = workloads.small(130 + gq + D, "BF16", hist=hist, fork=fork, C=6, S=4096, Hq=2 * gq, H=2, D=D, layers=2)
    say(f"append in the run gq={gq} D={D}")
    _append_run_case(wl, f"gq={gq} D={D}")


@pytest.mark.parametrize("profile,gq,D,sb", [("INT8_G64", 4, 128, 4), ("INT8_G64", 2, 64, 4), ("INT8_G64", 8, 256, 4),
                                           ("FP8_E4M3FN_ROW256", 4, 128, 4), ("FP8_E4M3FN_ROW256", 1, 64, 4), ("NVFP4_G16", 4, 128, 4),
                                           ("NVFP4_G16", 2, 256, 4), ("K8V4", 8, 256, 4), ("K8V4", 4, 128, 4),
                                           ("INT8_G64", 4, 128, 2), ("K8V4", 8, 256, 2)])
def test_decode_append_run_quantized(profile, gq, D, sb):
    # the quantized stream writes the step's rows itself (the append kernel's
    # codec) before it loads their pages: planes and outputs bit for bit as
    # kv_append + decode_run; forks, new tokens at page starts, mid-page and
    # page ends, some in a fresh page
    wl = workloads.small(140 + gq + D + sb, profile, hist=TREE_HIST, fork=TREE_FORK, C=6, S=4096, Hq=2 * gq, H=2,
                         D=D, layers=2, scale_bytes=sb, outlier_frac=0.01 if profile == "INT8_G64" else 0.0)
    say(f"append in the quantized run {profile} gq={gq} D={D} scale bytes {sb}")
    _append_run_case(wl, f"{profile} gq={gq} D={D} sb={sb}")


@pytest.mark.parametrize("profile,D", [("INT8_G64", 128), ("K8V4", 256)])
def test_decode_append_run_quantized_many_new_rows_in_a_block(profile, D):
    # seven short entries and one long one over 16 KV heads: the short
    # entries' 112 one-page units share the first blocks' ranges, so a block
    # writes many new rows, in every wave
    hist = [10, 63, 0, 40, 1, 62, 30, 66000]
    wl = workloads.small(141, profile, hist=hist, C=8, S=66048, Hq=16, H=16, D=D)
    say(f"append in the quantized run, many new rows per block, {profile} D={D}")
    _append_run_case(wl, f"{profile} many new rows")


@pytest.mark.parametrize("D", [128, 256])
def test_decode_append_run_more_new_rows_than_staged(D):
    # seven one-page entries and one long one: the first block's range holds
    # nine new-token pages, more than it stages (eight rows at D = 128, four
    # at D = 256)
    hist = [10, 63, 0, 40, 1, 62, 30, 66000]
    wl = workloads.small(131, "BF16", hist=hist, C=8, S=66048, Hq=8, H=2, D=D)
    say("append in the run, more new rows than staged")
    _append_run_case(wl, "many new rows")
