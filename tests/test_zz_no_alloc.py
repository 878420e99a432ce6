"""GPU test of paged_attn_decode_noalloc: decode on the library's static
scratch, for callers that cannot allocate, against paged_attn_decode with a
caller workspace (the same kernels: outputs bit for bit) and the fp64
oracle (max-abs 2e-3).  Two calls in a row, the second on a smaller batch
with shorter contexts, then a shape whose workspace exceeds the scratch is
refused on the host before any launch."""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from tests.drivers import build_device, build_oracle, say
from workloads.device_driver import _dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


def test_decode_noalloc_matches_workspace_decode_and_oracle():
    import torch
    from paged_kv_cache_03_amd import _abi as abi
    from paged_kv_cache_03_amd.device_pool import i32
    hist = [3000, 2000, 1, 900, 64, 1500]
    fork = [None, None, None, None, None, (0, 1500)]
    cow = [False] * 5 + [True]
    for profile, gq, D in (("BF16", 4, 128), ("INT8_G64", 4, 128)):
        wl = workloads.small(600 + D, profile, hist=hist, fork=fork, cow=cow, C=6, S=4096, Hq=2 * gq, H=2, D=D)
        say(f"noalloc decode {profile} gq={gq} D={D}")
        pool, st, _ = build_oracle(wl)
        dp, _, _ = build_device(wl)
        dev = dp.device
        q = _dev(wl.q(0), dev)
        calls = [(list(range(wl.B)), wl.seq_lens), ([4, 1, 3], [64, 1700, 901])]   # second: smaller, shorter
        for sel, lens in calls:
            rows = [wl.table_rows[b] for b in sel]
            msl = max(lens)
            qs = q[sel].contiguous()
            out_n = torch.full((len(sel), wl.Hq, wl.D), float("nan"), dtype=torch.float32, device=dev)
            out_w = torch.full_like(out_n, float("nan"))
            dp.decode_noalloc(0, wl.Hq, i32(rows, dev), i32(lens, dev), msl, qs, wl.sm_scale, out_n)
            ws = dp.workspace(len(sel), wl.Hq, msl)
            dp.decode(0, wl.Hq, i32(rows, dev), i32(lens, dev), msl, qs, wl.sm_scale, out_w, ws)
            torch.cuda.synchronize()
            got, ref_w = out_n.cpu().numpy(), out_w.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref_w.view(np.uint32)), (profile, sel)
            ref = A.paged_decode(st, 0, rows, lens, wl.q(0)[sel], wl.sm_scale)
            err = float(np.max(np.abs(got - ref)))
            say(f"  B={len(sel)} max_seq_len={msl}: bitwise equal to the workspace decode, oracle err {err:.3g}")
            assert err <= TOL
        dp.close()


def test_decode_noalloc_refuses_a_workspace_beyond_the_scratch():
    import torch
    from paged_kv_cache_03_amd import _abi as abi
    from paged_kv_cache_03_amd.device_pool import DevicePool, i32
    # 72 KV heads (past the 64 the page stream's plan takes) x 8 entries at
    # head_dim 256 over 32768-token contexts take the split kernel, whose
    # partials exceed the scratch
    dp = DevicePool("BF16", 72, 256, 1, 32768, 8, 512, zero=True)
    need = abi._lib.paged_attn_workspace_bytes(dp.handle, 8, 144, 32768, 0)
    assert need > abi.KV_DECODE_SCRATCH_BYTES
    dev = dp.device
    q = torch.zeros((8, 144, 256), dtype=torch.int16, device=dev)
    out = torch.zeros((8, 144, 256), dtype=torch.float32, device=dev)
    with pytest.raises(abi.KVError) as ei:
        dp.decode_noalloc(0, 144, i32(list(range(8)), dev), i32([0] * 8, dev), 32768, q, 0.0625, out)
    assert ei.value.status == abi.KV_E_INVALID and "scratch" in ei.value.message
    torch.cuda.synchronize()
    assert bool((out == 0).all())
    dp.close()
