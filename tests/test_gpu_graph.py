"""GPU test of the decode step captured as a HIP graph (kv_decode_step_graph_create).

One graph per batch shape, replayed while the data changes in place: lengths
advance (one of them across a page boundary, the new page mapped and published
before the replay), queries and the step's rows change, and eager work runs
between replays.  Every replay equals an eager step on the same inputs bit for
bit (the same kernels on the same data) and the oracle within max-abs 2e-3;
block tables stay bit-exact.  The step appends its rows inside the run (BF16,
INT8-G64 and K8V4 pages) or through kv_append + run (INT8-G64 pages).
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


@pytest.mark.parametrize("profile,fused", [("BF16", True), ("INT8_G64", False), ("INT8_G64", True), ("K8V4", True)])
def test_step_graph_replays_match_eager_and_oracle(profile, fused):
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    H, gq, D, layers = 2, 4, 128, 3
    hist = [300, 1000, 62, 0]
    wl = workloads.small(130, profile, hist=hist, step=[1] * 4, C=4, S=2048, Hq=H * gq, H=H, D=D, layers=layers,
                         mode="decode")
    pool, st, sids = build_oracle(wl)
    dp, seqs, step_inputs = build_device(wl)
    dev = dp.device
    B, Hq = wl.B, wl.Hq
    lens = list(wl.seq_lens)
    rows_t, lens_t = i32(wl.table_rows, dev), i32(lens, dev)
    pos0_t, cu_t = i32([n - 1 for n in lens], dev), i32(list(range(B + 1)), dev)
    kbuf = [step_inputs[l][0].clone() for l in range(layers)]
    vbuf = [step_inputs[l][1].clone() for l in range(layers)]
    qbuf = [_dev(wl.q(l), dev) for l in range(layers)]
    out_g = [torch.empty((B, Hq, D), dtype=torch.float32, device=dev) for _ in range(layers)]
    out_e = [torch.empty_like(o) for o in out_g]
    msl = wl.S                                   # fixed bound: the grid does not change between replays
    ws = dp.workspace(B, Hq, msl)

    def eager(outs):
        dp.decode_plan(Hq, rows_t, lens_t, msl, ws)
        for l in range(layers):
            if fused:
                dp.decode_append_run(l, B, Hq, msl, kbuf[l], vbuf[l], qbuf[l], wl.sm_scale, outs[l], ws)
            else:
                dp.append(l, rows_t, pos0_t, cu_t, B, kbuf[l], vbuf[l])
                dp.decode_run(l, B, Hq, msl, qbuf[l], wl.sm_scale, outs[l], ws)

    # fused: the append inside the run (no positions); otherwise kv_append with positions
    g = dp.step_graph(B, Hq, rows_t, lens_t, msl, qbuf, wl.sm_scale, out_g, ws, ks=kbuf, vs=vbuf,
                      pos0=None if fused else pos0_t, cu=None if fused else cu_t)
    r = rng_for(9300, 1)
    qs = [wl.q(l) for l in range(layers)]
    try:
        for it in range(4):
            if it > 0:
                # the next token of every entry: frontier commit, mapping (a page
                # crossing for the entry at 63 -> 64 -> 65), new rows and queries
                for b in range(B):
                    dp.commit(seqs[b], lens[b])
                    assert pool.commit(sids[b], lens[b]) == "OK"
                    lens[b] += 1
                    dp.ensure_mapped(seqs[b], lens[b])
                    assert pool.ensure_mapped(sids[b], lens[b]) == ("OK", 0)
                for l in range(layers):
                    k, v = bf16_normal(r, (B, H, D)), bf16_normal(r, (B, H, D))
                    qs[l] = bf16_normal(r, (B, Hq, D))
                    for b in range(B):
                        st.append(l, wl.table_rows[b], lens[b] - 1, k[b:b + 1], v[b:b + 1])
                    kbuf[l].copy_(_dev(k, dev))
                    vbuf[l].copy_(_dev(v, dev))
                    qbuf[l].copy_(_dev(qs[l], dev))
                lens_t.copy_(i32(lens, dev))
                pos0_t.copy_(i32([n - 1 for n in lens], dev))
            dp.graph_launch(g)
            torch.cuda.synchronize()
            eager(out_e)
            torch.cuda.synchronize()
            assert np.array_equal(dp.table.cpu().numpy(), pool.table)
            worst = 0.0
            for l in range(layers):
                got = out_g[l].cpu().numpy()
                assert np.array_equal(got, out_e[l].cpu().numpy()), f"replay {it} layer {l} differs from eager"
                ref = A.paged_decode(st, l, wl.table_rows, lens, qs[l], wl.sm_scale)
                worst = max(worst, float(np.max(np.abs(got - ref))))
            say(f"{profile} replay {it} lens={lens}: max abs err {worst:.3g}")
            assert worst <= TOL
    finally:
        dp.graph_destroy(g)
    dp.close()


def test_step_graph_kv_append_form_with_ragged_rows():
    # BF16 pages with positions given: the graph takes kv_append + run, whatever
    # the rows per entry (2, 1, 3 and 0 here, one crossing a page); every
    # replay with new rows and queries equals the eager calls and the oracle
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    H, gq, D, layers = 2, 4, 128, 2
    wl = workloads.small(131, "BF16", hist=[300, 1000, 62, 5], step=[2, 1, 3, 0], C=4, S=2048, Hq=H * gq, H=H,
                         D=D, layers=layers, mode="decode")
    pool, st, _ = build_oracle(wl)
    dp, _, step_inputs = build_device(wl)
    dev = dp.device
    B, Hq, total = wl.B, wl.Hq, int(wl.cu_q[-1])
    rows_t, lens_t = i32(wl.table_rows, dev), i32(wl.seq_lens, dev)
    pos0_t, cu_t = i32(wl.hist, dev), i32(wl.cu_q, dev)
    kbuf = [step_inputs[l][0].clone() for l in range(layers)]
    vbuf = [step_inputs[l][1].clone() for l in range(layers)]
    qbuf = [_dev(wl.q(l), dev) for l in range(layers)]
    out_g = [torch.empty((B, Hq, D), dtype=torch.float32, device=dev) for _ in range(layers)]
    out_e = [torch.empty_like(o) for o in out_g]
    msl = max(wl.seq_lens)
    ws = dp.workspace(B, Hq, msl)
    g = dp.step_graph(B, Hq, rows_t, lens_t, msl, qbuf, wl.sm_scale, out_g, ws, ks=kbuf, vs=vbuf, pos0=pos0_t,
                      cu=cu_t, total_tokens=total)
    r = rng_for(9301, 1)
    qs = [wl.q(l) for l in range(layers)]
    try:
        for it in range(3):
            if it > 0:
                for l in range(layers):
                    k, v = bf16_normal(r, (total, H, D)), bf16_normal(r, (total, H, D))
                    qs[l] = bf16_normal(r, (B, Hq, D))
                    for b in range(B):
                        a, e = wl.cu_q[b], wl.cu_q[b + 1]
                        if e > a:
                            st.append(l, wl.table_rows[b], wl.hist[b], k[a:e], v[a:e])
                    kbuf[l].copy_(_dev(k, dev))
                    vbuf[l].copy_(_dev(v, dev))
                    qbuf[l].copy_(_dev(qs[l], dev))
            dp.graph_launch(g)
            torch.cuda.synchronize()
            dp.decode_plan(Hq, rows_t, lens_t, msl, ws)
            for l in range(layers):
                dp.append(l, rows_t, pos0_t, cu_t, total, kbuf[l], vbuf[l])
                dp.decode_run(l, B, Hq, msl, qbuf[l], wl.sm_scale, out_e[l], ws)
            torch.cuda.synchronize()
            worst = 0.0
            for l in range(layers):
                got = out_g[l].cpu().numpy()
                assert np.array_equal(got, out_e[l].cpu().numpy()), f"replay {it} layer {l} differs from eager"
                ref = A.paged_decode(st, l, wl.table_rows, wl.seq_lens, qs[l], wl.sm_scale)
                worst = max(worst, float(np.max(np.abs(got - ref))))
                for role, arr in st.planes[l].items():
                    p = dp.planes[l][role].cpu().numpy()
                    assert np.array_equal(p.view(np.uint8), arr.view(np.uint8)), (it, l, role)
            say(f"ragged rows replay {it}: max abs err {worst:.3g}")
            assert worst <= TOL
    finally:
        dp.graph_destroy(g)
    dp.close()


def test_step_graph_fused_form_refuses_what_it_cannot_take():
    # no positions asks for the append inside the run: NVFP4 pages at head_dim
    # 64 decode on the split kernel, which has none
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from paged_kv_cache_03_amd import _abi as abi
    wl = workloads.small(132, "NVFP4_G16", hist=[100, 200], step=[1, 1], C=2, S=512, Hq=8, H=2, D=64)
    dp, _, step_inputs = build_device(wl)
    dev = dp.device
    rows_t, lens_t = i32(wl.table_rows, dev), i32(wl.seq_lens, dev)
    ws = dp.workspace(wl.B, wl.Hq, 512)
    q = [_dev(wl.q(0), dev)]
    out = [torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev)]
    with pytest.raises(abi.KVError) as ei:
        dp.step_graph(wl.B, wl.Hq, rows_t, lens_t, 512, q, wl.sm_scale, out, ws, ks=[step_inputs[0][0]],
                      vs=[step_inputs[0][1]])
    assert ei.value.status == abi.KV_E_UNSUPPORTED
    dp.close()
