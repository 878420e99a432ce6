"""GPU parity of the head-major plane order [X, P, N, H] (storage [H][M][64][X]).

The PagedKVStorageLayout passage gives two closed physical orders whose
address-translation equations differ only in which of the head and
page-group terms carries the larger stride.  Results do not depend on the
order: planes (read back as [M][H][64][X]) are bit-exact against the oracle,
decode and verify outputs are within 2e-3 of the fp64 oracle and bitwise
equal to those of a page-major pool built from the same inputs, and the host
replica (the packed logical-order host image) is covered in test_gpu_replica.py.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from tests.drivers import build_device, build_oracle, device_decode, device_verify, plane_np, say

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _planes_equal(dp, st, layer):
    for role, ref in st.planes[layer].items():
        got = plane_np(dp, layer, role)
        if ref.dtype == np.float32:
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), role
        else:
            assert np.array_equal(got, ref), role


# page stream (BF16, INT8, FP8, K8V4), and the split kernel (NVFP4 at D = 64)
CASES = [("BF16", 4, 128), ("INT8_G64", 4, 128), ("FP8_E4M3FN_ROW256", 8, 256), ("K8V4", 8, 256),
         ("NVFP4_G16", 2, 64)]


@pytest.mark.parametrize("profile,gq,D", CASES)
def test_head_major_decode_matches_oracle_and_page_major(profile, gq, D):
    H = 3
    # ragged tails, an empty history, a fork with a copied tail (the copy runs per (group, head) slice)
    hist = [0, 63, 64, 777, 1500, 1500]
    fork = [None, None, None, None, None, (4, 1500)]
    cow = [False] * 5 + [True]
    wl = workloads.small(300 + gq + D, profile, hist=hist, fork=fork, cow=cow, C=6, S=2048, Hq=H * gq, H=H, D=D)
    say(f"head-major decode {profile} gq={gq} D={D}")
    pool, st, _ = build_oracle(wl)
    outs = []
    for hm in (True, False):
        dp, _, _ = build_device(wl, head_major=hm)
        assert np.array_equal(dp.table.cpu().numpy(), pool.table)
        _planes_equal(dp, st, 0)
        outs.append(device_decode(dp, wl, 0))
        dp.close()
    ref = A.paged_decode(st, 0, wl.table_rows, wl.seq_lens, wl.q(0), wl.sm_scale)
    err = np.max(np.abs(outs[0] - ref))
    say(f"  max abs err {err:.3g}")
    assert err <= TOL
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("gq,D", [(4, 128), (1, 64)])
def test_head_major_verify_matches_oracle_and_page_major(gq, D):
    H = 2
    wl = workloads.small(340 + gq, "BF16", hist=[0, 100, 333, 640], step=[7, 1, 40, 300], C=4, S=1024, Hq=H * gq,
                         H=H, D=D, mode="verify")
    say(f"head-major verify gq={gq} D={D}")
    pool, st, _ = build_oracle(wl)
    outs = []
    for hm in (True, False):
        dp, _, _ = build_device(wl, head_major=hm)
        _planes_equal(dp, st, 0)
        outs.append(device_verify(dp, wl, 0))
        dp.close()
    ref = A.paged_verify(st, 0, wl.table_rows, wl.hist, wl.cu_q, wl.q(0), wl.sm_scale)
    assert np.max(np.abs(outs[0] - ref)) <= TOL
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_head_major_storage_order():
    # the storage itself is [H][M][64][X]: slice (g, h) sits at slice number h * M + g
    wl = workloads.small(350, "BF16", hist=[200, 64], C=2, S=512, Hq=4, H=2, D=64)
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl, head_major=True)
    raw = dp.planes[0]["K_CODE"].permute(1, 0, 2, 3).contiguous().cpu().numpy()   # storage order
    assert dp.planes[0]["K_CODE"].permute(1, 0, 2, 3).is_contiguous()
    flat = raw.reshape(-1, 64, wl.D)
    ref = st.planes[0]["K_CODE"]
    for g in np.unique(pool.table[pool.table >= 0]):
        for h in range(wl.H):
            assert np.array_equal(flat[h * wl.M + g].view(np.uint16), ref[g, h].view(np.uint16)), (g, h)
    dp.close()
