"""GPU parity of paged_attn_verify on every closed profile and at head_dim 256.

The pool sets of the Paged KV Context Store page put Main Text and MTP
pages on the engine-selected profile, so a prefill chunk or a speculative
verify runs on whatever profile the pool holds.  Cases: INT8-G64 (fp32 and
binary16 scales), FP8-row, NVFP4-G16 and K8V4 pools at D = 128 and 256, and
BF16 pools at D = 256; frontiers mid-page, at a page end and at 0; a fork
sharing full pages and one whose own history starts in a copied tail; chunks
from one token to several 128-column tiles; planes filled with 0xFF bytes
(NaN codes and scales past every frontier).  Bar: max-abs 2e-3 against the
fp64 oracle on the same dequantized values.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from tests.drivers import build_device, build_oracle, device_verify, say

pytestmark = pytest.mark.gpu

TOL = 2e-3

CASES = [("INT8_G64", 4, 128, 4), ("INT8_G64", 4, 128, 2), ("FP8_E4M3FN_ROW256", 4, 128, 4),
         ("NVFP4_G16", 2, 128, 4), ("K8V4", 4, 128, 4), ("K8V4", 8, 256, 4), ("INT8_G64", 2, 256, 4),
         ("FP8_E4M3FN_ROW256", 1, 256, 2), ("BF16", 4, 256, 4), ("BF16", 8, 256, 4), ("BF16", 1, 256, 4)]


@pytest.mark.parametrize("profile,gq,D,sb", CASES)
def test_verify_every_profile_matches_oracle(profile, gq, D, sb):
    H = 2
    # entry 1 forks entry 0 at a page boundary; entry 2's own history starts
    # in a copied tail; chunks of 5, 40, 1, 100 and 64 tokens
    hist = [700, 1000, 1000, 130, 0]
    step = [5, 40, 1, 100, 64]
    fork = [None, (0, 640), (0, 700), None, None]
    wl = workloads.small(700 + gq + D + sb, profile, hist=hist, step=step, fork=fork, C=5, S=2048, Hq=H * gq, H=H,
                         D=D, mode="verify", outlier_frac=0.01 if profile == "INT8_G64" else 0.0, scale_bytes=sb)
    say(f"verify {profile} gq={gq} D={D} scale bytes {sb}")
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl, fill=0xFF)
    assert np.array_equal(dp.table.cpu().numpy(), pool.table)
    got = device_verify(dp, wl, 0)
    dp.close()
    ref = A.paged_verify(st, 0, wl.table_rows, wl.hist, wl.cu_q, wl.q(0), wl.sm_scale)
    err = float(np.max(np.abs(got - ref)))
    say(f"  max abs err {err:.3g}")
    assert err <= TOL


@pytest.mark.parametrize("profile,gq,D", [("K8V4", 8, 256), ("INT8_G64", 4, 128), ("BF16", 4, 256)])
def test_verify_profiles_long_history_mid_page(profile, gq, D):
    # a 10K-token history with the chunk starting mid-page, a short verify and
    # a prefill chunk over several tiles, and a T = 1 chunk equal to decode
    wl = workloads.small(760 + D, profile, hist=[10000 + 35, 9000 + 1, 4000 + 63], step=[5, 300, 1], C=3, S=16384,
                         Hq=2 * gq, H=2, D=D, mode="verify")
    say(f"verify {profile} gq={gq} D={D} long history")
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    got = device_verify(dp, wl, 0)
    dp.close()
    ref = A.paged_verify(st, 0, wl.table_rows, wl.hist, wl.cu_q, wl.q(0), wl.sm_scale)
    err = float(np.max(np.abs(got - ref)))
    say(f"  max abs err {err:.3g}")
    assert err <= TOL


def test_verify_tiles_without_page_split():
    # 8 entries x 4 KV heads x 16 tiles of 512-token chunks: enough tiles to
    # fill the chip, so every tile streams its whole range (no parts, no
    # combine) -- the other cases here run split tiles
    hist = [100, 700, 1000, 64, 0, 333, 1500, 63]
    wl = workloads.small(780, "INT8_G64", hist=hist, step=[512] * 8, C=8, S=2048, Hq=16, H=4, D=128,
                         mode="verify", outlier_frac=0.01)
    say("verify INT8-G64, 512 tiles, no page split")
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl, fill=0xFF)
    got = device_verify(dp, wl, 0)
    dp.close()
    ref = A.paged_verify(st, 0, wl.table_rows, wl.hist, wl.cu_q, wl.q(0), wl.sm_scale)
    err = float(np.max(np.abs(got - ref)))
    say(f"  max abs err {err:.3g}")
    assert err <= TOL
