"""Invariances of decode where the page stream's blocks each stream many pages.

The work split gives every block an equal share of the flat page stream; with
long histories each block streams 10-25 pages, so partial boundaries inside a
block, the register-carried merge of a unit's pages and the combine order all
decide the output bits.  Checked on the BF16, INT8-G64 and K8V4 streams:

* physical page placement ("Paged KV Context Store" page: physical ids of a
  page group may be any permutation; kernel correctness does not depend on
  their contiguity) -- two other free orders give bitwise-equal outputs;
* plane order (PagedKVStorageLayout passage: the head-major order differs
  only in strides) -- a head-major pool gives bitwise-equal outputs;
* sharing (fork passage) -- the same histories in private pages take another
  split (shared pages are read once for every sharer): the sums run in
  another order, with other running maxima, so the two agree to rounding of
  the value terms: within 1e-5 x max(1, max|v|), max|v| the largest
  dequantized value (about 5 for N(0,1) values, about 90 with the INT8
  workload's 1% of outliers x20);
* the fp64 oracle over every output, within 2e-3.
"""

import numpy as np
import pytest

import workloads
from tests.drivers import build_device, device_decode, oracle_decode_all, oracle_logical, say

pytestmark = pytest.mark.gpu

TOL = 2e-3

# entry 1 forks entry 0 at a page boundary, entry 2 inside a page (its own
# history starts in the copied tail), entry 3 is private
HIST = [64000, 60000, 50011, 62000]
FORK = [None, (0, 20480), (0, 30001), None]

CASES = [("BF16", 4, 128, 4), ("BF16", 8, 256, 2), ("INT8_G64", 4, 128, 4), ("K8V4", 8, 256, 2)]


def _pages_per_block(wl):
    # distinct (page, KV head) slices read once, over the stream's blocks
    # (two per compute unit, one for the BF16 stream at D = 256)
    own = sum(-(-(wl.hist[b] + wl.step[b] - wl.own_start(b)) // 64) for b in range(wl.B))
    return own * wl.H / (256.0 if wl.profile == "BF16" and wl.D == 256 else 512.0)


@pytest.mark.parametrize("profile,gq,D,H", CASES)
def test_decode_invariances_with_many_pages_per_block(profile, gq, D, H):
    wl = workloads.small(400 + gq + D, profile, hist=HIST, fork=FORK, C=4, S=65536, Hq=H * gq, H=H, D=D,
                         outlier_frac=0.01 if profile == "INT8_G64" else 0.0)
    say(f"{profile} gq={gq} D={D} H={H}: about {_pages_per_block(wl):.1f} pages per block")
    runs = [("default order", {}),
            ("reversed order", {"free_order": np.arange(wl.M)[::-1].copy()}),
            ("random order", {"free_order": np.random.default_rng(7).permutation(wl.M).astype(np.int32)}),
            ("head-major", {"head_major": True})]
    outs = []
    for tag, kw in runs:
        dp, _, _ = build_device(wl, zero=False, **kw)
        outs.append(device_decode(dp, wl, 0))
        dp.close()
        say(f"  {tag}: done")
        if len(outs) > 1:
            assert np.array_equal(outs[-1].view(np.uint32), outs[0].view(np.uint32)), tag
    dp, _, _ = build_device(wl, zero=False, privatize=True)
    private = device_decode(dp, wl, 0)
    dp.close()
    d = float(np.max(np.abs(private - outs[0])))
    vmax = max(float(np.max(np.abs(oracle_logical(wl, 0, b, wl.seq_lens[b])[1]))) for b in range(wl.B))
    say(f"  private copies: max abs difference {d:.3g} (max|v| {vmax:.3g})")
    assert d <= 1e-5 * max(1.0, vmax)
    ref = oracle_decode_all(wl, 0)
    err = float(np.max(np.abs(outs[0] - ref)))
    say(f"  oracle: max abs err {err:.3g}")
    assert err <= TOL
