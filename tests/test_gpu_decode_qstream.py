"""GPU parity of the matrix-core page stream on quantized pages.

The quantized profiles (INT8-G64, FP8-E4M3FN-row256, NVFP4-G16, K8V4) run the
page stream with codes converted to bf16 operands in registers and the fp32
scales applied to scores and probabilities.  The cases cover every
instantiated (K codec, V codec, D) with the head groupings, ragged frontiers,
forks with shared and copied tails, pages whose unwritten rows hold 0xFF
bytes (NaN codes and scales that must not leak into the output), blocks
crossing many segments past the cached query rows, bitwise invariance to
physical page placement, and plan-once / run-every-layer.
Bar: max-abs 2e-3 against the fp64 oracle.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from tests.drivers import build_device, build_oracle, device_decode, say

pytestmark = pytest.mark.gpu

TOL = 2e-3

CASES = [
    ("INT8_G64", 4, 128), ("INT8_G64", 1, 64), ("INT8_G64", 8, 256), ("INT8_G64", 2, 128),
    ("FP8_E4M3FN_ROW256", 4, 128), ("FP8_E4M3FN_ROW256", 8, 64), ("FP8_E4M3FN_ROW256", 2, 256),
    ("NVFP4_G16", 4, 128), ("NVFP4_G16", 1, 256),
    ("K8V4", 8, 256), ("K8V4", 4, 128), ("K8V4", 2, 256),
]


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


@pytest.mark.parametrize("profile,gq,D", CASES)
def test_qstream_shapes_with_stale_bytes(profile, gq, D):
    H = 2
    hist = [0, 63, 64, 777, 1500, 1500, 5, 2000]
    fork = [None, None, None, None, None, (4, 1500), None, (4, 1024)]
    cow = [False] * 5 + [True, False, False]
    wl = workloads.small(80 + gq + D, profile, hist=hist, fork=fork, cow=cow, C=8, S=4096, Hq=H * gq, H=H, D=D,
                         outlier_frac=0.01 if profile == "INT8_G64" else 0.0)
    say(f"decode {profile} gq={gq} D={D}, planes filled with 0xFF")
    dp, _ = _check(wl, f"{profile} gq={gq} D={D}", fill=0xFF)
    dp.close()


@pytest.mark.parametrize("profile,D", [("INT8_G64", 128), ("K8V4", 256)])
def test_qstream_block_crossing_many_segments(profile, D):
    # one long entry and seven short ones: the block that reaches the short
    # entries crosses ~15 segments (past the cached query rows)
    hist = [65000, 40, 10, 63, 64, 1, 100, 20]
    Hq = 16 if profile == "INT8_G64" else 8
    wl = workloads.small(91, profile, hist=hist, C=8, S=65536, Hq=Hq, H=4 if profile == "INT8_G64" else 2, D=D,
                         M=1100)
    say(f"decode {profile} B={wl.B} H={wl.H} D={D}")
    dp, _ = _check(wl, f"{profile} many segments")
    dp.close()


@pytest.mark.parametrize("profile,gq,D", [("INT8_G64", 4, 128), ("K8V4", 8, 256)])
def test_qstream_bitwise_invariant_to_page_permutation(profile, gq, D):
    wl = workloads.small(93, profile, hist=[700, 1000, 1000, 130], fork=[None, (0, 640), (0, 700), None],
                         cow=[False, False, True, False], C=4, S=2048, Hq=2 * gq, H=2, D=D)
    outs = []
    for fo in (None, np.arange(wl.M)[::-1].copy(), np.random.default_rng(2).permutation(wl.M)):
        dp, _, _ = build_device(wl, free_order=fo)
        outs.append(device_decode(dp, wl, 0))
        dp.close()
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    dp, _, _ = build_device(wl, privatize=True)
    private = device_decode(dp, wl, 0)
    dp.close()
    assert float(np.max(np.abs(private - outs[0]))) <= 1e-5


def test_qstream_plan_once_run_every_layer():
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev
    wl = workloads.small(94, "INT8_G64", hist=[2000, 2000, 1500, 3000], fork=[None, (0, 1024), (0, 1000), None],
                         C=4, S=4096, Hq=8, H=2, D=128, layers=3)
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    dev = dp.device
    msl = max(wl.seq_lens)
    ws = dp.workspace(wl.B, wl.Hq, msl)
    dp.decode_plan(wl.Hq, i32(wl.table_rows, dev), i32(wl.seq_lens, dev), msl, ws)
    for layer in range(wl.layers):
        q = _dev(wl.q(layer), dev)
        out = torch.full((wl.B, wl.Hq, wl.D), float("nan"), dtype=torch.float32, device=dev)
        dp.decode_run(layer, wl.B, wl.Hq, msl, q, wl.sm_scale, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), device_decode(dp, wl, layer).view(np.uint32)), layer
        ref = A.paged_decode(st, layer, wl.table_rows, wl.seq_lens, wl.q(layer), wl.sm_scale)
        err = float(np.max(np.abs(got - ref)))
        say(f"  layer {layer}: max abs err {err:.3g}")
        assert err <= TOL
    dp.close()
