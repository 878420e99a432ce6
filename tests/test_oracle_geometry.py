"""Pins of oracle.geometry against the pages' printed values and closed forms."""

import os

import numpy as np
import pytest

from oracle import geometry as G

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_d256_payload_table_matches_pages():
    # the page's table implies 2-byte INT8/FP8 scale elements
    for prof, kc, ks, vc, vs, tot in _rows("d256_payload_table.txt"):
        b = G.payload_bytes_per_token_head(prof, 256, scale_bytes=2)
        assert (b["K_CODE"], b["K_SCALE"], b["V_CODE"], b["V_SCALE"], b["KV"]) == tuple(
            int(x) for x in (kc, ks, vc, vs, tot)), prof


def test_payload_with_fp32_scales():
    # the workloads store INT8-G64 and FP8-row scales as fp32: only the scale
    # columns change (4 INT8 groups at D=256, one FP8 row scale per side)
    got = {p: G.payload_bytes_per_token_head(p, 256, 4)["KV"] for p in G.PROFILES}
    assert got == {"BF16": 1024, "INT8_G64": 544, "FP8_E4M3FN_ROW256": 520, "NVFP4_G16": 288, "K8V4": 404}
    # K8V4 is asymmetric: not 2 * a per-side vector size
    b = G.payload_bytes_per_token_head("K8V4", 256, 4)
    assert b["K"] != b["V"]


def test_page_bytes_is_sum_over_planes():
    # PageBytes = sum_plane bytes/token * P, over every plane of every layer
    D, H, layers = 128, 8, 32
    per_plane_bytes = {s.role: s.x_extent * s.elem_bytes for s in G.plane_schema("INT8_G64", D)}
    assert per_plane_bytes == {"K_CODE": 128, "K_SCALE": 8, "V_CODE": 128, "V_SCALE": 8}
    assert G.page_bytes("INT8_G64", D, H, layers) == 272 * H * layers * 64


def test_capacity_bounds_on_named_workloads():
    # 8-sequence decode at S=32768: pool M = C * ceil(32768/64) = 4096 = M_max
    assert G.logical_pages(32768) == 512
    assert G.m_bounds(32768, 8) == (512, 4096)
    # tiny decode: C=1, M=16 is only legal for L=16, i.e. 960 < S <= 1024
    for S in range(1, 4096):
        lo, hi = G.m_bounds(S, 1)
        assert (lo <= 16 <= hi) == (960 < S <= 1024)
    assert G.m_bounds(65536, 8) == (1024, 8192)
    assert G.m_bounds(131072, 4) == (2048, 8192)
    # M_min guarantees at least one page per active lane even for tiny S
    assert G.m_bounds(10, 8) == (8, 8)


def test_capacity_bounds_brute_force():
    # M_min: smallest pool in which one sequence reaches S AND every lane holds a page;
    # M_max: all C sequences at the ceiling simultaneously.  Counted by enumeration.
    for S in (1, 63, 64, 65, 1000, 4097):
        for C in range(1, 9):
            pages_one_seq = next(n for n in range(1, 10 ** 6) if n * 64 >= S)
            m_min = next(M for M in range(1, 10 ** 6) if M >= pages_one_seq and M >= C)
            m_max = sum(pages_one_seq for _ in range(C))
            assert G.m_bounds(S, C) == (m_min, m_max)


def test_explicit_capacity_policy():
    assert G.explicit_capacity(32768 * 8, 32768, 8) == 4096
    assert G.explicit_capacity(32768 + 1, 32768, 8) == 513
    with pytest.raises(ValueError):
        G.explicit_capacity(1000, 32768, 8)           # K_main < S
    with pytest.raises(ValueError):
        G.explicit_capacity(32768 * 9, 32768, 8)       # above M_max


def test_check_geometry_rejections():
    ok = dict(page_size=64, S=1024, C=2, M=16, H=2, D=128, Hq=8)
    G.check_geometry(**ok)
    for bad in (dict(page_size=32), dict(C=9), dict(C=0), dict(M=15), dict(M=33), dict(Hq=5), dict(Hq=1),
                dict(D=96, profile="INT8_G64"), dict(D=40, profile="NVFP4_G16")):
        with pytest.raises(ValueError):
            G.check_geometry(**{**ok, **bad})


def test_element_index_matches_c_order_layout():
    # address-translation equation with contiguous strides == C-order [M][H][P][X]
    rng = np.random.default_rng(0)
    M, H, X = 7, 3, 40
    for _ in range(2000):
        g, h, o, d = (int(rng.integers(0, n)) for n in (M, H, 64, X))
        assert G.element_index(d, o, h, g, X, H) == np.ravel_multi_index((g, h, o, d), (M, H, 64, X))


def test_head_major_index_is_c_order_and_a_bijection():
    # head-major [X, P, N, H] == C-order [H][M][P][X]; every element once, no gaps
    M, H, X = 5, 3, 6
    seen = np.zeros(M * H * 64 * X, dtype=np.int64)
    for g in range(M):
        for h in range(H):
            for o in range(64):
                for d in range(X):
                    i = G.element_index_head_major(d, o, h, g, X, M)
                    assert i == np.ravel_multi_index((h, g, o, d), (H, M, 64, X))
                    seen[i] += 1
    assert (seen == 1).all()
    # the two orders agree only when there is one head (or one page group)
    assert G.element_index_head_major(1, 2, 0, 3, X, M) == G.element_index(1, 2, 0, 3, X, 1)
    assert G.element_index_head_major(1, 2, 1, 0, X, 1) == G.element_index(1, 2, 1, 0, X, H)


def test_translation_shift_mask():
    p = np.arange(1 << 20)
    assert np.array_equal(p >> 6, p // 64) and np.array_equal(p & 63, p % 64)
    table = np.arange(100, 100 + 40)
    assert G.translate(1000, table) == (15, 40, 115)
    # logical block b covers [b*P, (b+1)*P)
    for b in range(5):
        assert {G.translate(q, table)[0] for q in range(b * 64, (b + 1) * 64)} == {b}


def test_attention_pairs_brute_force():
    for B in (0, 1, 7, 64):
        for S in (0, 1, 5, 33):
            pairs = sum(1 for i in range(S) for k in range(B + i + 1))
            assert G.attention_pairs(B, S) == pairs
