"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: codes, scales and block tables bit-exact; attention outputs (fp32) within
max-abs 2e-3 of the fp64 oracle on identical dequantized inputs.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as A
from oracle import codecs as Q
from tests.drivers import (build_device, build_oracle, device_decode, device_verify, oracle_decode_all,
                           oracle_pool_only, oracle_verify_rows, plane_np, say)

pytestmark = pytest.mark.gpu

TOL = 2e-3
KINDS = {"BF16": ("bf16", "bf16"), "INT8_G64": ("int8_g64",) * 2, "FP8_E4M3FN_ROW256": ("fp8_row",) * 2,
         "NVFP4_G16": ("nvfp4_g16",) * 2, "K8V4": ("fp8_row", "nvfp4_g16")}


def _table(dp):
    return np.array(dp.table.cpu().numpy())


def _compare_planes(dp, st, layers, pages=None):
    for layer in layers:
        for role, ref in st.planes[layer].items():
            got = plane_np(dp, layer, role)
            sel = slice(None) if pages is None else pages
            g, r = got[sel], ref[sel]
            if r.dtype == np.float32:
                assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), (layer, role)
            else:
                assert np.array_equal(g, r), (layer, role)


# ----------------------------------------------------------------- codecs --
def _codec_rows(D, seed):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7F80) != 0x7F80]
    rng = np.random.default_rng(seed)
    finite = finite[rng.permutation(len(finite))]
    n_rows = -(-len(finite) // D)
    rows = np.zeros(n_rows * D, dtype=np.uint16)
    rows[: len(finite)] = finite
    rows = rows.reshape(n_rows, D)
    special = np.zeros((4, D), dtype=np.uint16)
    special[1, 3] = 0xC040            # single non-zero element (-3.0)
    special[2, :] = 0x8000            # all negative zero
    special[3, :] = 0x0001            # smallest subnormal everywhere
    normal = workloads.bf16_normal(workloads.rng_for(seed), (60, D), outlier_frac=0.01)
    return np.concatenate([rows, special, normal])


@pytest.mark.parametrize("profile", ["BF16", "INT8_G64", "FP8_E4M3FN_ROW256", "NVFP4_G16", "K8V4"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_codec_bit_exact_all_bf16_inputs(profile, D):
    import torch
    from paged_kv_cache_03_amd.device_pool import DevicePool, i32
    rows = _codec_rows(D, 30 + D)
    n = rows.shape[0]
    S = 64 * -(-n // 64)
    L = S // 64
    say(f"codec {profile} D={D} rows={n}")
    dp = DevicePool(profile, 1, D, 1, S, 1, L, free_order=np.arange(L)[::-1].copy())
    seq = dp.open(0)
    dp.ensure_mapped(seq, n)
    k = torch.from_numpy(rows.view(np.int16).reshape(n, 1, D)).cuda()
    v = torch.from_numpy(rows[::-1].copy().view(np.int16).reshape(n, 1, D)).cuda()
    dp.append(0, i32([0], "cuda"), i32([0], "cuda"), i32([0, n], "cuda"), n, k, v)
    torch.cuda.synchronize()
    table = _table(dp)[0]
    for side, x in (("K", rows), ("V", rows[::-1])):
        kind = KINDS[profile][0 if side == "K" else 1]
        code, scale = Q.quantize(kind, x)
        got_c = plane_np(dp, 0, f"{side}_CODE")
        pos = np.arange(n)
        gc = got_c[table[pos >> 6], 0, pos & 63]
        assert np.array_equal(gc, code), (side, kind)
        if scale is not None:
            gs = plane_np(dp, 0, f"{side}_SCALE")[table[pos >> 6], 0, pos & 63]
            assert np.array_equal(gs.view(np.uint8), scale.reshape(n, -1).view(np.uint8)), (side, kind)
    dp.close()


# ---------------------------------------------------------- tiny decode ----
def test_tiny_bf16_decode_full_parity():
    wl = workloads.get(1)
    say(f"workload {wl.name}")
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    assert np.array_equal(_table(dp), pool.table)
    _compare_planes(dp, st, [0])
    for lens in ([301], [300]):          # with the appended step token, and without it
        got = device_decode(dp, wl, 0, seq_lens=lens)
        ref = A.paged_decode(st, 0, wl.table_rows, lens, wl.q(0), wl.sm_scale)
        assert np.max(np.abs(got - ref)) <= TOL, lens
    dp.close()


# ---------------------------------------------------- randomized shapes ----
CASES = [
    ("BF16", 4, 128), ("BF16", 1, 64), ("BF16", 8, 256), ("BF16", 2, 128),
    ("INT8_G64", 4, 128), ("INT8_G64", 8, 256), ("INT8_G64", 1, 64),
    ("FP8_E4M3FN_ROW256", 4, 128), ("FP8_E4M3FN_ROW256", 8, 256),
    ("NVFP4_G16", 4, 128), ("NVFP4_G16", 2, 64),
    ("K8V4", 8, 256), ("K8V4", 4, 128),
]


@pytest.mark.parametrize("profile,gq,D", CASES)
def test_small_decode_parity(profile, gq, D):
    H = 2
    # several pages per sequence, ragged tails, an empty history, a fork with a copied tail
    hist = [0, 63, 64, 777, 1500, 1500]
    fork = [None, None, None, None, None, (4, 1500)]
    cow = [False] * 5 + [True]
    wl = workloads.small(100 + gq + D, profile, hist=hist, fork=fork, cow=cow, C=6, S=2048, Hq=H * gq, H=H, D=D,
                         outlier_frac=0.01 if profile == "INT8_G64" else 0.0)
    say(f"decode {profile} gq={gq} D={D}")
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    assert np.array_equal(_table(dp), pool.table)
    _compare_planes(dp, st, [0])
    got = device_decode(dp, wl, 0)
    ref = A.paged_decode(st, 0, wl.table_rows, wl.seq_lens, wl.q(0), wl.sm_scale)
    err = np.max(np.abs(got - ref))
    say(f"  max abs err {err:.3g}")
    assert err <= TOL
    dp.close()


def test_decode_zero_length_and_single_token():
    wl = workloads.small(7, "BF16", hist=[0, 0, 5], step=[0, 1, 1], C=3, S=256)
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    got = device_decode(dp, wl, 0)
    assert np.all(got[0] == 0)
    ref = A.paged_decode(st, 0, wl.table_rows, wl.seq_lens, wl.q(0), wl.sm_scale)
    assert np.max(np.abs(got - ref)) <= TOL
    # ctx 1: the output is the single value row exactly
    v1 = Q.bf16_to_f32(wl.step_kv(0, 1)[1])[0]
    assert np.max(np.abs(got[1] - np.repeat(v1, wl.Hq // wl.H, axis=0))) <= 1e-6
    dp.close()


@pytest.mark.parametrize("gq,D", [(4, 128), (1, 64), (8, 256)])
def test_small_verify_parity(gq, D):
    H = 2
    wl = workloads.small(40 + gq, "BF16", hist=[0, 100, 333, 64], step=[7, 1, 40, 64], C=4, S=1024, Hq=H * gq,
                         H=H, D=D, mode="verify")
    say(f"verify gq={gq} D={D}")
    pool, st, _ = build_oracle(wl)
    dp, _, _ = build_device(wl)
    got = device_verify(dp, wl, 0)
    ref = A.paged_verify(st, 0, wl.table_rows, wl.hist, wl.cu_q, wl.q(0), wl.sm_scale)
    assert np.max(np.abs(got - ref)) <= TOL
    dp.close()


# ------------------------------------------------------------ invariances --
def test_gpu_outputs_bitwise_invariant_to_page_permutation_and_sharing():
    wl = workloads.small(8, "INT8_G64", hist=[700, 1000, 1000, 130], fork=[None, (0, 640), (0, 700), None],
                         cow=[False, False, True, False], C=4, S=2048, Hq=8, H=2, D=128)
    say("invariance")
    outs = []
    for fo, priv in ((None, False), (np.arange(wl.M)[::-1].copy(), False),
                     (np.random.default_rng(1).permutation(wl.M), False), (None, True)):
        dp, _, _ = build_device(wl, free_order=fo, privatize=priv)
        outs.append(device_decode(dp, wl, 0))
        dp.close()
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def test_gpu_decode_identical_before_and_after_tail_cow():
    import torch
    wl = workloads.small(9, "K8V4", hist=[1000, 1000], fork=[None, (0, 1000)], cow=[False, False], step=[0, 0],
                         C=2, S=2048, Hq=16, H=2, D=256)
    dp, seqs, _ = build_device(wl)
    before = device_decode(dp, wl, 0)
    t0 = _table(dp).copy()
    dp.cow_tail(seqs[1])
    torch.cuda.synchronize()
    t1 = _table(dp)
    row1 = wl.table_rows[1]
    assert t1[row1, 15] != t0[row1, 15] and np.array_equal(t1[row1, :15], t0[row1, :15])
    after = device_decode(dp, wl, 0)
    assert np.array_equal(before.view(np.uint32), after.view(np.uint32))
    # the copy moved exactly the 40 committed columns of every plane
    for role in dp.planes[0]:
        p = plane_np(dp, 0, role)
        assert np.array_equal(p[t1[row1, 15], :, :40], p[t0[row1, 15], :, :40])
    dp.close()


# --------------------------------------------------------- full sizes ------
def _full_decode_check(wl, layers):
    """Every decode output of the given layers against the fp64 oracle, and
    every row the step appended (codes and scales, bit for bit), at the full
    size, in the launch configuration the benchmark times (plan + run)."""
    import torch
    pool, _ = oracle_pool_only(wl)
    dp, _, _ = build_device(wl, layers=layers, zero=False)
    assert np.array_equal(_table(dp), pool.table)
    kind_k, kind_v = KINDS[wl.profile]
    worst = 0.0
    for layer in layers:
        got = device_decode(dp, wl, layer)
        say(f"  layer {layer}: device done, oracle reference of all {wl.B}x{wl.Hq} outputs")
        ref = oracle_decode_all(wl, layer)
        err = float(np.max(np.abs(got - ref)))
        say(f"  layer {layer}: max abs err over every output {err:.3g}")
        worst = max(worst, err)
        # every appended row: its page through the table, codes and scales bit-exact
        planes = {role: plane_np(dp, layer, role) for role in dp.planes[layer]}
        for b in range(wl.B):
            k, v = wl.step_kv(layer, b)
            pos = wl.hist[b] + np.arange(wl.step[b])
            gg = pool.table[wl.table_rows[b], pos >> 6]
            for side, x, kind in (("K", k, kind_k), ("V", v, kind_v)):
                code, scale = Q.quantize(kind, x, wl.scale_bytes)
                got_c = planes[f"{side}_CODE"][gg, :, pos & 63]
                assert np.array_equal(got_c, code), (layer, b, side)
                if scale is not None:
                    got_s = planes[f"{side}_SCALE"][gg, :, pos & 63]
                    assert np.array_equal(got_s.view(np.uint8), scale.reshape(got_s.shape).view(np.uint8)), \
                        (layer, b, side)
        del planes
        crossing = sum(int((wl.hist[b] >> 6) != ((wl.hist[b] + wl.step[b] - 1) >> 6)) for b in range(wl.B))
        say(f"  layer {layer}: {sum(wl.step)} appended rows bit-exact ({crossing} entries cross a page)")
    assert worst <= TOL
    dp.close()
    torch.cuda.empty_cache()


def test_full_bf16_decode_c8_32k():
    wl = workloads.get(2)
    say(f"workload {wl.name} (layers 0 and 31)")
    _full_decode_check(wl, [0, 31])


def test_full_int8_decode_c8_32k():
    wl = workloads.get(3)
    say(f"workload {wl.name} (layer 0)")
    _full_decode_check(wl, [0])


def test_full_k8v4_decode_c8_64k():
    wl = workloads.get(4)
    say(f"workload {wl.name}")
    _full_decode_check(wl, [0])


def test_full_verify_prefill_c4_128k():
    """Every row of both 5-token verify chunks, and all 32 heads of the first
    and last token of each 32-token (128-column) tile of both 512-token prefill
    chunks, plus 16 more seeded tokens of each, against the fp64 oracle."""
    import torch
    wl = workloads.get(5)
    say(f"workload {wl.name}")
    pool, _ = oracle_pool_only(wl)
    dp, _, _ = build_device(wl, zero=False)
    assert np.array_equal(_table(dp), pool.table)
    got = device_verify(dp, wl, 0)
    dp.close()
    torch.cuda.empty_cache()
    rng = np.random.default_rng(5)
    tokens = {}
    for b in range(wl.B):
        T = wl.step[b]
        if T <= 32:
            tokens[b] = list(range(T))
        else:
            sel = {x for t in range(0, T, 32) for x in (t, min(T, t + 32) - 1)}
            sel |= {int(x) for x in rng.integers(0, T, 16)}
            tokens[b] = sorted(sel)
    say(f"  device done; oracle reference of {sum(len(t) for t in tokens.values())} tokens x {wl.Hq} heads")
    ref = oracle_verify_rows(wl, 0, tokens)
    worst = 0.0
    for (b, i), r in ref.items():
        worst = max(worst, float(np.max(np.abs(got[wl.cu_q[b] + i] - r))))
    say(f"  max abs err over {len(ref)} tokens x {wl.Hq} heads {worst:.3g}")
    assert worst <= TOL
