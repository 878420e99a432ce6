"""Pins of oracle.attention: brute force, library SDPA, special cases, invariances."""

import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as A
from oracle import codecs as Q
from oracle.pool import OraclePool
from oracle.store import OracleStore
from tests.drivers import build_oracle
from workloads.gen import bf16_normal, f32_to_bf16_bits, rng_for


def _brute(qv, K, V, scale):
    # pure-Python loops: softmax over dot products, no max subtraction needed at this size
    n, D = len(K), len(qv)
    s = [sum(float(qv[d]) * float(K[i][d]) for d in range(D)) * scale for i in range(n)]
    w = [math.exp(x) for x in s]
    tot = sum(w)
    return [sum(w[i] * float(V[i][d]) for i in range(n)) / tot for d in range(D)]


def test_attend_matches_brute_force():
    rng = np.random.default_rng(10)
    for n in (1, 2, 7, 30):
        qv, K, V = rng.standard_normal(16), rng.standard_normal((n, 16)), rng.standard_normal((n, 16))
        got = A.attend(qv, K, V, 0.25)
        assert np.allclose(got, _brute(qv, K, V, 0.25), rtol=1e-12, atol=1e-12)


def test_gqa_decode_matches_torch_sdpa_fp64():
    rng = rng_for(11)
    Hq, H, D, n = 8, 2, 64, 37
    q = bf16_normal(rng, (Hq, D))
    K = Q.bf16_to_f32(bf16_normal(rng, (n, H, D)))
    V = Q.bf16_to_f32(bf16_normal(rng, (n, H, D)))
    scale = 1.0 / math.sqrt(D)
    got = A.decode_dense(q, K, V, scale)
    qt = torch.from_numpy(Q.bf16_to_f32(q).astype(np.float64))[:, None, :]          # [Hq, 1, D]
    kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // H, 0)
    vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // H, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0].numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_causal_chunk_matches_torch_sdpa_with_explicit_mask():
    rng = rng_for(12)
    Hq, H, D, n0, T = 4, 2, 32, 45, 9
    q = bf16_normal(rng, (T, Hq, D))
    K = Q.bf16_to_f32(bf16_normal(rng, (n0 + T, H, D)))
    V = Q.bf16_to_f32(bf16_normal(rng, (n0 + T, H, D)))
    got = A.causal_dense(q, K, V, n0, 0.125)
    qt = torch.from_numpy(Q.bf16_to_f32(q).astype(np.float64)).permute(1, 0, 2)        # [Hq, T, D]
    kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // H, 0)
    vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // H, 0)
    mask = torch.arange(n0 + T)[None, :] <= (n0 + torch.arange(T))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.125)
    assert np.allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_special_cases():
    rng = np.random.default_rng(13)
    D = 32
    v0 = rng.standard_normal((1, D))
    assert np.array_equal(A.attend(rng.standard_normal(D), rng.standard_normal((1, D)), v0, 0.3), v0[0])
    V = rng.standard_normal((50, D))
    mean = V.mean(0)
    assert np.allclose(A.attend(np.zeros(D), rng.standard_normal((50, D)), V, 0.3), mean, atol=1e-14)
    k = rng.standard_normal(D)
    assert np.allclose(A.attend(rng.standard_normal(D), np.tile(k, (50, 1)), V, 0.3), mean, atol=1e-14)
    assert np.array_equal(A.attend(np.ones(D), np.zeros((0, D)), np.zeros((0, D)), 1.0), np.zeros(D))
    # a hugely dominant key returns its value (max subtraction keeps this finite)
    K = np.zeros((5, D))
    K[3] = 1000.0
    out = A.attend(np.ones(D), K, V[:5], 1.0)
    assert np.allclose(out, V[3])


def test_mha_is_gqa_with_one_query_head_per_kv_head():
    rng = rng_for(14)
    q = bf16_normal(rng, (3, 16))
    K = Q.bf16_to_f32(bf16_normal(rng, (20, 3, 16)))
    V = Q.bf16_to_f32(bf16_normal(rng, (20, 3, 16)))
    out = A.decode_dense(q, K, V, 0.25)
    for j in range(3):
        assert np.array_equal(out[j], A.attend(Q.bf16_to_f32(q[j]), K[:, j], V[:, j], 0.25))


def _build(wl, free_order=None, privatize=False):
    pool, st, _ = build_oracle(wl, free_order=free_order, privatize=privatize)
    return pool, st


def _decode(wl, st, layer=0):
    return A.paged_decode(st, layer, wl.table_rows, wl.seq_lens, wl.q(layer), wl.sm_scale)


@pytest.mark.parametrize("profile", ["BF16", "INT8_G64", "FP8_E4M3FN_ROW256", "NVFP4_G16", "K8V4"])
def test_paged_decode_equals_dense_over_logical_kv(profile):
    wl = workloads.small(1, profile, hist=[0, 63, 64, 200, 511], C=5, S=1024, D=128)
    pool, st = _build(wl)
    out = _decode(wl, st)
    kind_k, kind_v = {"BF16": ("bf16", "bf16"), "INT8_G64": ("int8_g64",) * 2,
                      "FP8_E4M3FN_ROW256": ("fp8_row",) * 2, "NVFP4_G16": ("nvfp4_g16",) * 2,
                      "K8V4": ("fp8_row", "nvfp4_g16")}[profile]
    for b in range(wl.B):
        k, v = wl.logical_kv(0, b, wl.seq_lens[b])
        K = Q.dequantize(kind_k, *Q.quantize(kind_k, k))
        V = Q.dequantize(kind_v, *Q.quantize(kind_v, v))
        ref = A.decode_dense(wl.q(0)[b], K, V, wl.sm_scale)
        assert np.array_equal(out[b], ref)


def test_every_in_page_frontier():
    # frontiers ending at each offset 1..64 of a page, and the first token of a page
    hist = list(range(64, 129))
    wl = workloads.small(2, "BF16", hist=hist, C=8, S=256, M=8 * 4 + 40, Hq=2, H=1, D=64)
    wl.table_rows = [b % 8 for b in range(len(hist))]
    for b in range(wl.B):
        pool = OraclePool(256, 1, 4, free_order=[3, 1, 0, 2])
        st = OracleStore(pool, "BF16", 1, 64, 1)
        sid = pool.open(0)
        k, v = wl.logical_kv(0, b, wl.seq_lens[b])
        pool.ensure_mapped(sid, len(k))
        st.append(0, 0, 0, k, v)
        out = A.paged_decode(st, 0, [0], [len(k)], wl.q(0)[b:b + 1], wl.sm_scale)
        ref = A.decode_dense(wl.q(0)[b], Q.bf16_to_f32(k), Q.bf16_to_f32(v), wl.sm_scale)
        assert np.array_equal(out[0], ref)


def test_results_invariant_under_page_permutation():
    wl = workloads.small(3, "INT8_G64", hist=[130, 700, 5], C=3, S=1024)
    _, st1 = _build(wl)
    _, st2 = _build(wl, free_order=np.arange(wl.M)[::-1].copy())
    _, st3 = _build(wl, free_order=np.random.default_rng(0).permutation(wl.M))
    o1, o2, o3 = _decode(wl, st1), _decode(wl, st2), _decode(wl, st3)
    assert np.array_equal(o1, o2) and np.array_equal(o1, o3)


def test_shared_prefix_equals_private_copies():
    wl = workloads.small(4, "K8V4", hist=[640, 900, 1000], C=3, S=1024, D=256, Hq=4, H=2,
                         fork=[None, (0, 640), (0, 320)])
    pool, st = _build(wl)
    assert pool.pages_of(0)[:5] == pool.pages_of(2)[:5]            # really shared
    _, st_priv = _build(wl, privatize=True)
    assert np.array_equal(_decode(wl, st), _decode(wl, st_priv))


def test_results_identical_before_and_after_tail_cow():
    wl = workloads.small(5, "NVFP4_G16", hist=[1000, 1000], C=2, S=2048, D=128,
                         fork=[None, (0, 1000)], cow=[False, True], step=[1, 1])
    # before the step: both rows read the shared tail
    pool = OraclePool(wl.S, wl.C, wl.M, free_order=wl.free_order)
    st = OracleStore(pool, wl.profile, wl.H, wl.D, 1)
    a = pool.open(wl.table_rows[0])
    pool.ensure_mapped(a, 1000)
    k, v = wl.logical_kv(0, 0, 1000)
    st.append(0, wl.table_rows[0], 0, k, v)
    pool.commit(a, 1000)
    b = pool.fork(a, 1000, wl.table_rows[1])
    q = wl.q(0)
    before = A.paged_decode(st, 0, wl.table_rows, [1000, 1000], q, wl.sm_scale)
    _, info = pool.cow_tail(b)
    st.cow_copy(*info)
    after = A.paged_decode(st, 0, wl.table_rows, [1000, 1000], q, wl.sm_scale)
    assert info[2] == 1000 % 64 and np.array_equal(before, after)


def test_verify_t1_equals_decode_and_chunk_equals_contiguous():
    wl = workloads.small(6, "BF16", hist=[100, 333, 64], step=[1, 1, 1], C=3, S=1024)
    _, st = _build(wl)
    dec = _decode(wl, st)
    ver = A.paged_verify(st, 0, wl.table_rows, wl.hist, wl.cu_q, wl.q(0), wl.sm_scale)
    assert np.array_equal(dec, ver)
    wl2 = workloads.small(7, "BF16", hist=[100, 333, 64], step=[20, 1, 37], C=3, S=1024, mode="verify")
    _, st2 = _build(wl2)
    ver2 = A.paged_verify(st2, 0, wl2.table_rows, wl2.hist, wl2.cu_q, wl2.q(0), wl2.sm_scale)
    for b in range(3):
        k, v = wl2.logical_kv(0, b, wl2.seq_lens[b])
        a, e = wl2.cu_q[b], wl2.cu_q[b + 1]
        ref = A.causal_dense(wl2.q(0)[a:e], Q.bf16_to_f32(k), Q.bf16_to_f32(v), wl2.hist[b], wl2.sm_scale)
        assert np.array_equal(ver2[a:e], ref)


def test_planted_index_error_is_caught():
    # a dropped GQA offset (every query head reading KV head 0) must not pass the SDPA pin
    rng = rng_for(15)
    q = bf16_normal(rng, (4, 16))
    K = Q.bf16_to_f32(bf16_normal(rng, (9, 2, 16)))
    V = Q.bf16_to_f32(bf16_normal(rng, (9, 2, 16)))
    good = A.decode_dense(q, K, V, 0.25)
    bad = np.stack([A.attend(Q.bf16_to_f32(q[j]), K[:, 0], V[:, 0], 0.25) for j in range(4)])
    assert not np.allclose(good, bad)
    assert f32_to_bf16_bits(np.float32([1.0]))[0] == 0x3F80


def test_attend_many_equals_attend_per_row_and_sdpa():
    # each row is the per-vector definition over its own key range, including an
    # empty range, one key and the whole of K; the explicit-mask SDPA of torch
    # (fp64, CPU) is the library pin of the same thing
    rng = np.random.default_rng(21)
    n, D = 300, 32
    K, V = rng.standard_normal((n, D)), rng.standard_normal((n, D))
    Qm = rng.standard_normal((9, D)) * 3.0
    lim = [0, 1, 2, 63, 64, 65, 200, 299, 300]
    got = A.attend_many(Qm, lim, K, V, 0.2)
    for r in range(len(lim)):
        assert np.allclose(got[r], A.attend(Qm[r], K[:lim[r]], V[:lim[r]], 0.2), rtol=1e-12, atol=1e-13), r
    assert np.array_equal(got[0], np.zeros(D))
    assert np.array_equal(got[1], V[0])
    mask = torch.arange(n)[None, :] < torch.tensor(lim[1:])[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qm[1:])[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None], attn_mask=mask[None],
        scale=0.2)[0].numpy()
    assert np.allclose(got[1:], ref, rtol=1e-12, atol=1e-13)
    # a planted off-by-one in the limits is caught
    bad = A.attend_many(Qm, [x + 1 if 0 < x < n else x for x in lim], K, V, 0.2)
    assert not np.allclose(bad[2], got[2], atol=1e-6)
