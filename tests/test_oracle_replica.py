"""Pins of the oracle's host replica (logical-order packed HostKVPageLayout).

What the store page fixes: a replica holds no device page ids or table holes,
each page carries the payload of every grouped plane, and only the actual
page count is paid for.  Pinned here by a round trip, by independence from
physical placement, by the size formula of the geometry module, and by
reading single elements at the offsets the layout defines.
"""

import numpy as np
import pytest

from oracle import geometry as G
from oracle.pool import OraclePool
from oracle.store import OracleStore
from workloads.gen import bf16_normal, rng_for


def _filled(profile, D, H, layers, n, free_order, seed=5):
    pool = OraclePool(S=2048, C=3, M=48, free_order=free_order)
    st = OracleStore(pool, profile, H, D, layers)
    sid = pool.open(0)
    pool.ensure_mapped(sid, n)
    r = rng_for(seed, 0)
    for layer in range(layers):
        st.append(layer, 0, 0, bf16_normal(r, (n, H, D), 0.01), bf16_normal(r, (n, H, D), 0.01))
    pool.commit(sid, n)
    return pool, st, sid


@pytest.mark.parametrize("profile,D", [("BF16", 64), ("INT8_G64", 128), ("K8V4", 256), ("NVFP4_G16", 128)])
def test_replica_round_trip_restores_every_plane(profile, D):
    H, layers, n = 2, 2, 300                      # 4 full pages and a 44-row tail
    pool, st, sid = _filled(profile, D, H, layers, n, np.random.default_rng(1).permutation(48))
    data, f = st.replica(sid)
    assert f == n and data.size == -(-n // 64) * G.page_bytes(profile, D, H, layers)
    s2 = st.restore(1, data, f)
    assert pool.frontier_of(s2) == n
    assert not set(pool.pages_of(s2)) & set(pool.pages_of(sid))     # new page groups
    for layer in range(layers):
        k0, v0 = st.gather(layer, 0, n)
        k1, v1 = st.gather(layer, 1, n)
        assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
        for role, arr in st.planes[layer].items():
            for b, (g0, g1) in enumerate(zip(pool.pages_of(sid), pool.pages_of(s2))):
                assert np.array_equal(arr[g0], arr[g1]), (role, b)


def test_replica_is_independent_of_page_placement():
    a = _filled("INT8_G64", 128, 2, 3, 777, np.arange(48))[1:]
    b = _filled("INT8_G64", 128, 2, 3, 777, np.random.default_rng(9).permutation(48))[1:]
    da, _ = a[0].replica(a[1])
    db, _ = b[0].replica(b[1])
    assert a[0].pool.pages_of(a[1]) != b[0].pool.pages_of(b[1])
    assert np.array_equal(da, db)


def test_replica_offsets_hold_the_logical_elements():
    profile, D, H, layers, n = "K8V4", 256, 2, 2, 200
    pool, st, sid = _filled(profile, D, H, layers, n, np.random.default_rng(4).permutation(48))
    data, _ = st.replica(sid)
    pb = G.page_bytes(profile, D, H, layers)
    schema = G.plane_schema(profile, D)
    rng = np.random.default_rng(0)
    for _ in range(500):
        p = int(rng.integers(0, n))
        layer = int(rng.integers(0, layers))
        j = int(rng.integers(0, len(schema)))
        spec = schema[j]
        h, x = int(rng.integers(0, H)), int(rng.integers(0, spec.x_extent))
        # page p // 64 of the replica; layers in order, planes in schema order
        before = layer * sum(H * 64 * s.x_extent * s.elem_bytes for s in schema) + \
            sum(H * 64 * s.x_extent * s.elem_bytes for s in schema[:j])
        off = (p // 64) * pb + before + ((h * 64 + p % 64) * spec.x_extent + x) * spec.elem_bytes
        got = data[off:off + spec.elem_bytes]
        arr = st.planes[layer][spec.role]
        want = np.ascontiguousarray(arr[pool.table[0, p // 64], h, p % 64, x:x + 1]).view(np.uint8)
        assert np.array_equal(got, want)


def test_replica_of_an_empty_history_is_empty():
    pool = OraclePool(S=1024, C=2, M=16)
    st = OracleStore(pool, "BF16", 2, 64, 1)
    sid = pool.open(0)
    data, f = st.replica(sid)
    assert f == 0 and data.size == 0
    s2 = st.restore(1, data, 0)
    assert pool.pages_of(s2) == [] and pool.frontier_of(s2) == 0
