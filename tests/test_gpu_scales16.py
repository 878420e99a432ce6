"""GPU parity of 2-byte (binary16) INT8-G64 and FP8-row scale planes.

The page's D256 payload table sizes the scale planes at 2 bytes; these pools
store each scale as binary16 (the fp32 quotient rounded half to even,
saturated at 65504) and take the codes against the stored scale.  Bar: codes
and scales bit-exact against the oracle for every finite bf16 input; decode
within max-abs 2e-3 of the fp64 oracle on the matrix-core quantized stream
(pages filled with 0xFF past every frontier) and on the chunked split kernel
(more KV heads than the stream's plan takes).
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from oracle import codecs as Q
from tests.drivers import build_device, build_oracle, device_decode, plane_np, say
from tests.test_gpu_parity import KINDS, _codec_rows, _compare_planes, _table

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.mark.parametrize("profile", ["INT8_G64", "FP8_E4M3FN_ROW256", "K8V4"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_codec_two_byte_scales_bit_exact_all_bf16_inputs(profile, D):
    import torch
    from paged_kv_cache_03_amd.device_pool import DevicePool, i32
    rows = _codec_rows(D, 60 + D)
    n = rows.shape[0]
    S = 64 * -(-n // 64)
    L = S // 64
    say(f"codec {profile} D={D} 2-byte scales rows={n}")
    dp = DevicePool(profile, 1, D, 1, S, 1, L, free_order=np.arange(L)[::-1].copy(), scale_bytes=2)
    seq = dp.open(0)
    dp.ensure_mapped(seq, n)
    k = torch.from_numpy(rows.view(np.int16).reshape(n, 1, D)).cuda()
    v = torch.from_numpy(rows[::-1].copy().view(np.int16).reshape(n, 1, D)).cuda()
    dp.append(0, i32([0], "cuda"), i32([0], "cuda"), i32([0, n], "cuda"), n, k, v)
    torch.cuda.synchronize()
    table = _table(dp)[0]
    pos = np.arange(n)
    for side, x in (("K", rows), ("V", rows[::-1])):
        kind = KINDS[profile][0 if side == "K" else 1]
        code, scale = Q.quantize(kind, x, 2)
        gc = plane_np(dp, 0, f"{side}_CODE")[table[pos >> 6], 0, pos & 63]
        assert np.array_equal(gc, code), (side, kind)
        if scale is not None:
            gs = plane_np(dp, 0, f"{side}_SCALE")[table[pos >> 6], 0, pos & 63]
            assert np.array_equal(gs.view(np.uint8), scale.reshape(n, -1).view(np.uint8)), (side, kind)
    dp.close()


@pytest.mark.parametrize("profile,gq,D", [("INT8_G64", 4, 128), ("INT8_G64", 1, 64), ("INT8_G64", 8, 256),
                                          ("FP8_E4M3FN_ROW256", 4, 128), ("FP8_E4M3FN_ROW256", 8, 64),
                                          ("K8V4", 8, 256), ("K8V4", 4, 128)])
def test_qstream_two_byte_scales_with_stale_bytes(profile, gq, D):
    H = 2
    hist = [0, 63, 64, 777, 1500, 1500, 5, 2000]
    fork = [None, None, None, None, None, (4, 1500), None, (4, 1024)]
    cow = [False] * 5 + [True, False, False]
    wl = workloads.small(160 + gq + D, profile, hist=hist, fork=fork, cow=cow, C=8, S=4096, Hq=H * gq, H=H, D=D,
                         outlier_frac=0.01 if profile == "INT8_G64" else 0.0, scale_bytes=2)
    say(f"decode {profile} gq={gq} D={D}, 2-byte scales, planes filled with 0xFF")
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl, fill=0xFF)
    assert np.array_equal(_table(dp), pool.table)
    got = device_decode(dp, wl, 0)
    ref = A.paged_decode(st, 0, wl.table_rows, wl.seq_lens, wl.q(0), wl.sm_scale)
    err = float(np.max(np.abs(got - ref)))
    say(f"  max abs err {err:.3g}")
    assert err <= TOL
    dp.close()


@pytest.mark.parametrize("profile", ["INT8_G64", "K8V4"])
def test_split_kernel_two_byte_scales(profile):
    # 72 KV heads: past the 64 the stream's plan takes, so the chunked split kernel runs
    D = 64 if profile == "INT8_G64" else 128
    wl = workloads.small(170, profile, hist=[300, 1000, 63], C=3, S=1024, Hq=72, H=72, D=D, scale_bytes=2)
    say(f"split decode {profile} H=72 D={D}, 2-byte scales")
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    _compare_planes(dp, st, [0])
    got = device_decode(dp, wl, 0)
    ref = A.paged_decode(st, 0, wl.table_rows, wl.seq_lens, wl.q(0), wl.sm_scale)
    err = float(np.max(np.abs(got - ref)))
    say(f"  max abs err {err:.3g}")
    assert err <= TOL
    dp.close()
