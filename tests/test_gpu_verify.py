"""GPU parity of verify / chunked prefill (causal, several query tokens per
entry) against the CPU oracle.

Chunks of at most 32 query columns (tokens x GQ) go through the page stream in
chunk mode; longer chunks through 128-column tiles on the matrix cores.  The
cases mix both in one call, put frontiers at every kind of in-page offset,
end tiles with partial columns, and fork histories.  Bar: max-abs 2e-3
against the fp64 oracle.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from tests.drivers import build_device, build_oracle, device_verify, say

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _check(wl, tag):
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    assert np.array_equal(dp.table.cpu().numpy(), pool.table)
    got = device_verify(dp, wl, 0)
    ref = A.paged_verify(st, 0, wl.table_rows, wl.hist, wl.cu_q, wl.q(0), wl.sm_scale)
    err = float(np.max(np.abs(got - ref)))
    say(f"  {tag}: max abs err {err:.3g}")
    assert err <= TOL
    dp.close()


@pytest.mark.parametrize("gq,D", [(8, 128), (2, 64), (4, 128), (1, 128)])
def test_verify_mixed_chunks(gq, D):
    H = 2
    # query columns per entry: 3*gq .. well above 128; frontiers at 0, mid-page, page end
    hist = [0, 100, 333, 64, 1000, 700]
    step = [3, 9, 40, 17, 100, 1]
    fork = [None, None, None, None, (2, 320), None]
    wl = workloads.small(80 + gq + D, "BF16", hist=hist, step=step, fork=fork, C=6, S=2048, Hq=H * gq, H=H, D=D,
                         mode="verify")
    say(f"verify gq={gq} D={D} columns={[t * gq for t in step]}")
    _check(wl, f"gq={gq} D={D}")


def test_verify_long_prefill_tiles_share_pages():
    # one long prefill across many pages and tiles, next to a short verify
    wl = workloads.small(90, "BF16", hist=[3000, 2500], step=[300, 5], C=2, S=4096, Hq=8, H=2, D=128,
                         mode="verify")
    _check(wl, "prefill 300 + verify 5")


def test_verify_long_histories_one_term_pages():
    # long histories: past the first pages no key weighs more than 1/256 of
    # its column's running sum, and the tiles take P as one bf16 term there
    wl = workloads.small(91, "BF16", hist=[12000, 19937], step=[200, 141], C=2, S=20480, Hq=8, H=2, D=128,
                         mode="verify")
    _check(wl, "prefill 200 + 141 at 12K/20K keys")


@pytest.mark.parametrize("scale_mul", [1.0, 4.0])
def test_verify_one_term_pages_with_outlier_values(scale_mul):
    # 1% of the K and V elements x20 (values up to about 90): a key on a
    # one-term page moves its column by at most 2^-17 |v - o|, so even heavy
    # values stay inside the bar; with the softmax scale x4 some columns are
    # peaked as well
    wl = workloads.small(93, "BF16", hist=[30000, 20011], step=[256, 97], C=2, S=32768, Hq=8, H=2, D=128,
                         mode="verify", outlier_frac=0.01, scale_mul=scale_mul)
    _check(wl, f"outliers x20, scale x{scale_mul}")


@pytest.mark.parametrize("scale_mul", [4.0, 16.0])
def test_verify_peaked_softmax_keeps_two_terms(scale_mul):
    # softmax scale x4 and x16: a few keys carry most of every column, the
    # pages that hold them keep P as p_hi + p_lo
    wl = workloads.small(92, "BF16", hist=[6000, 3001], step=[160, 64], C=2, S=8192, Hq=8, H=2, D=128,
                         mode="verify", scale_mul=scale_mul)
    _check(wl, f"peaked x{scale_mul}")
