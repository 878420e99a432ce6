"""Pins of oracle.codecs: library casts, brute force, format constants, bounds.

Format constants come from the published minifloat definitions (OCP 8-bit
floating point: E4M3FN, bias 7, max 448, no infinities; OCP MX: E2M1 values
0, 0.5, 1, 1.5, 2, 3, 4, 6).
"""

import numpy as np
import pytest
import torch

from oracle import codecs as Q

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _finite_bf16_f32():
    x = Q.bf16_to_f32(ALL_BF16)
    return x[np.isfinite(x)]


def test_bf16_decode_is_bit_shift():
    x = Q.bf16_to_f32(np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x8000], dtype=np.uint16))
    assert x[0] == 1.0 and x[1] == -1.0 and x[2] == np.float32(3.140625)
    assert x[3] == np.float32(2.0 ** -133) and np.signbit(x[4]) and x[4] == 0


def test_e4m3fn_grid_constants():
    g = Q.E4M3FN_GRID
    assert len(g) == 127 and g[0] == 0 and np.all(np.diff(g) > 0)
    assert g[-1] == 448.0 and g[1] == 2.0 ** -9 and g[8] == 2.0 ** -6 and g[0x38] == 1.0


def test_e4m3fn_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = Q.decode_e4m3fn(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan].view(np.uint32), got[~nan].view(np.uint32))


def _torch_e4m3(y):
    # torch's CPU cast rounds half to even but maps overflow to NaN: clamp first
    yc = np.clip(y, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(yc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3fn_encode_matches_torch_on_all_bf16_and_random_fp32():
    y = _finite_bf16_f32()
    assert np.array_equal(Q.encode_e4m3fn(y), _torch_e4m3(y))
    rng = np.random.default_rng(1)
    z = (rng.choice([-1.0, 1.0], 400_000) * np.exp2(rng.uniform(-14, 10, 400_000))).astype(np.float32)
    assert np.array_equal(Q.encode_e4m3fn(z), _torch_e4m3(z))


def test_e4m3fn_ties_and_saturation():
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 5 * 2.0 ** -10: 0x02,
             448.0: 0x7E, 464.0: 0x7E, 500.0: 0x7E, 1e30: 0x7E, 0.0: 0x00}
    for v, code in cases.items():
        assert int(Q.encode_e4m3fn(np.float32(v))) == code, v
        assert int(Q.encode_e4m3fn(np.float32(-v))) == code | 0x80, v


def _brute_nearest(a, grid):
    # nearest grid value, ties to the even index, by exhaustive comparison
    best = np.zeros(a.shape, dtype=np.int64)
    bestd = np.full(a.shape, np.inf)
    for i, gv in enumerate(grid):
        d = np.abs(a - gv)
        better = (d < bestd) | ((d == bestd) & (i % 2 == 0))
        best = np.where(better, i, best)
        bestd = np.where(better, d, bestd)
    return best


def test_e2m1_brute_force_all_bf16():
    y = _finite_bf16_f32()
    a = np.minimum(np.abs(y).astype(np.float64), 6.0)
    want = _brute_nearest(a, [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]) | np.where(np.signbit(y), 8, 0)
    assert np.array_equal(Q.encode_e2m1(y), want.astype(np.uint8))


def test_e2m1_tie_table():
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0, 7.0: 6.0, 1e9: 6.0}
    for v, want in ties.items():
        assert Q.decode_e2m1(Q.encode_e2m1(np.float32(v))) == want
        assert Q.decode_e2m1(Q.encode_e2m1(np.float32(-v))) == -want


def test_e4m3fn_brute_force_random():
    rng = np.random.default_rng(2)
    y = (rng.standard_normal(200_000) * np.exp2(rng.integers(-12, 9, 200_000))).astype(np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), 448.0)
    want = _brute_nearest(a, Q.E4M3FN_GRID) | np.where(np.signbit(y), 0x80, 0)
    assert np.array_equal(Q.encode_e4m3fn(y), want.astype(np.uint8))


def _groups_with_specials(rng, n, D):
    x = rng.standard_normal((n, D)).astype(np.float32)
    x[0] = 0.0                                  # all-zero row
    x[1] = 0.0
    x[1, 5] = -3.0                              # single non-zero element
    x[2] *= np.float32(20.0)                    # outliers
    x[3] = np.float32(1e-30)                    # tiny but normal
    return Q.bf16_to_f32(_round_bf16(x))


def _round_bf16(x):
    u = x.astype(np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_int8_g64_nearest_and_bounds():
    rng = np.random.default_rng(3)
    x = _groups_with_specials(rng, 300, 256)
    q, s = Q.quant_int8_g64(x)
    assert q.dtype == np.int8 and s.shape == (300, 4)
    xg, qg = x.reshape(300, 4, 64), q.reshape(300, 4, 64).astype(np.int64)
    # scale: absmax / 127 within one fp32 rounding
    a = np.abs(xg).max(-1)
    assert np.all(np.abs(s.astype(np.float64) * 127 - a) <= a * 2.0 ** -23)
    nz = s > 0
    # each code is the nearest integer (ties to even) to the fp32 quotient x/s
    quot = (xg / np.where(nz, s, 1)[..., None]).astype(np.float32).astype(np.float64)
    ks = np.arange(-127, 128)
    d = np.abs(quot[..., None] - ks)
    dmin = d.min(-1, keepdims=True)
    cand = (d == dmin)
    even = cand & (ks % 2 == 0)
    pick = np.where(even.any(-1), ks[np.argmax(even, -1)], ks[np.argmax(cand, -1)])
    assert np.array_equal(np.where(nz[..., None], pick, 0), qg)
    # reconstruction error within half a step (plus fp32 rounding)
    err = np.abs(Q.dequant_int8_g64(q, s).reshape(300, 4, 64) - xg)
    assert np.all(err <= s[..., None] * (0.5 + 2 * 128 * 2.0 ** -24))
    # the group maximum maps to +-127; zero groups give zero codes and scale
    assert np.all(np.abs(qg).max(-1)[nz] == 127)
    assert np.all(qg[~nz] == 0) and np.all(s[0] == 0)


def test_fp8_row_codes_and_roundtrip():
    rng = np.random.default_rng(4)
    x = _groups_with_specials(rng, 300, 256)
    c, s = Q.quant_fp8_row(x)
    assert s.shape == (300, 1) and c.dtype == np.uint8
    nz = s[:, 0] > 0
    # the row maximum encodes to +-448
    amax = np.argmax(np.abs(x), axis=1)
    assert np.all((c[np.arange(300), amax] & 0x7F)[nz] == 0x7E)
    # codes equal the clamped torch cast of the fp32 quotient
    y = (x[nz] / s[nz]).astype(np.float32)
    assert np.array_equal(c[nz], _torch_e4m3(y))
    # relative error of a normal E4M3 value is at most 2^-4 (half of 3 mantissa bits)
    dq = Q.dequant_fp8_row(c, s)
    big = np.abs(x) >= s * 2.0 ** -6
    assert np.all(np.abs(dq - x)[big] <= np.abs(x)[big] * 2.0 ** -4 * 1.0001)
    assert np.all(c[~nz] == 0)


def test_nvfp4_g16_codes_pack_and_scale():
    rng = np.random.default_rng(5)
    x = _groups_with_specials(rng, 200, 256)
    packed, sc = Q.quant_nvfp4_g16(x)
    assert packed.shape == (200, 128) and sc.shape == (200, 16)
    nib = Q.unpack_nibbles(packed)
    # low nibble holds the even element
    assert np.array_equal(nib[:, 0::2], packed & 0xF) and np.array_equal(nib[:, 1::2], packed >> 4)
    xg = x.reshape(200, 16, 16)
    a = np.abs(xg).max(-1)
    # the scale is the E4M3FN rounding of absmax/6 (torch cast pin)
    assert np.array_equal(sc, _torch_e4m3((a / np.float32(6)).astype(np.float32)))
    vs = Q.decode_e4m3fn(sc)
    nz = vs > 0
    # the group maximum always lands on +-6 (scale rounding is at most 1/16 relative)
    ng = nib.reshape(200, 16, 16)
    amax = np.argmax(np.abs(xg), -1)
    top = np.take_along_axis(ng, amax[..., None], -1)[..., 0]
    assert np.all((top & 7)[nz] == 7)
    # element codes: brute-force nearest of the fp32 quotient
    quot = (xg / np.where(nz, vs, 1)[..., None]).astype(np.float32)
    want = _brute_nearest(np.minimum(np.abs(quot).astype(np.float64), 6.0),
                          [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]) | np.where(np.signbit(quot), 8, 0)
    assert np.array_equal(np.where(nz[..., None], want, 0), ng)
    # dequantization is exact in fp32: value(nibble) * value(scale)
    dq = Q.dequant_nvfp4_g16(packed, sc).reshape(200, 16, 16).astype(np.float64)
    assert np.array_equal(dq, Q.decode_e2m1(ng).astype(np.float64) * vs[..., None].astype(np.float64))


@pytest.mark.parametrize("kind", ["bf16", "int8_g64", "fp8_row", "nvfp4_g16"])
def test_quantize_dispatch_shapes(kind):
    rng = np.random.default_rng(6)
    xb = _round_bf16(rng.standard_normal((5, 3, 128)).astype(np.float32))
    code, scale = Q.quantize(kind, xb)
    back = Q.dequantize(kind, code, scale)
    assert back.shape == (5, 3, 128) and back.dtype == np.float32
    if kind == "bf16":
        assert np.array_equal(back, Q.bf16_to_f32(xb))
    else:
        assert np.max(np.abs(back - Q.bf16_to_f32(xb))) < 1.0


# ----------------------------------------------------- 2-byte scale planes --
def test_f16_scale_rounding_matches_torch_half_conversion():
    import torch
    from oracle.codecs import to_f16_bits
    rng = np.random.default_rng(11)
    # random magnitudes over the binary16 range, exact midpoints between
    # neighbouring binary16 values (ties), subnormals, zero
    vals = [np.float32(x) for x in np.exp(rng.uniform(np.log(1e-9), np.log(6e4), 20000))]
    h = np.arange(1, 0x7BFF, 37, dtype=np.uint16).view(np.float16).astype(np.float32)
    mids = ((h[:-1].astype(np.float64) + h[1:].astype(np.float64)) / 2).astype(np.float32)
    x = np.concatenate([np.array(vals, np.float32), h, mids, np.float32([0.0, 2.0 ** -25, 3 * 2.0 ** -26])])
    want = torch.from_numpy(x).to(torch.float16).numpy().view(np.uint16)
    assert np.array_equal(to_f16_bits(x), want)
    # saturation at the largest finite value instead of infinity
    assert to_f16_bits(np.float32([65520.0, 1e9]))[0] == 0x7BFF == to_f16_bits(np.float32([1e9]))[0]


def test_int8_g64_f16_scale_equals_fp32_scale_when_exact():
    from oracle.codecs import quant_int8_g64
    rng = np.random.default_rng(12)
    # absmax of every group exactly 127 * 2^k: a/127 is exact in binary16 and in fp32
    amax = (127.0 * 2.0 ** rng.integers(-8, 6, size=(500, 2))).astype(np.float32)
    x = (rng.uniform(-0.99, 0.99, (500, 2, 64)) * amax[..., None]).astype(np.float32)
    j = rng.integers(0, 64, size=(500, 2))
    np.put_along_axis(x, j[..., None], (amax * np.where(rng.random((500, 2)) < 0.5, -1, 1))[..., None], axis=-1)
    x = x.reshape(500, 128)
    q4, s4 = quant_int8_g64(x, 4)
    q2, s2 = quant_int8_g64(x, 2)
    assert np.array_equal(q4, q2)
    assert np.array_equal(s2.view(np.float16).astype(np.float32), s4)


def test_int8_g64_f16_scale_error_bound():
    from oracle.codecs import dequant_int8_g64, quant_int8_g64, scale_values
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((4000, 128)) * np.exp(rng.uniform(-6, 6, (4000, 1)))).astype(np.float32)
    q, s16 = quant_int8_g64(x, 2)
    sv = np.repeat(scale_values(s16), 64, axis=-1)
    err = np.abs(dequant_int8_g64(q, s16) - x)
    over = np.maximum(np.abs(x) - 127 * sv, 0)        # a scale rounded down clips at 127
    assert np.all(err <= sv / 2 * (1 + 2 ** -20) + over + 1e-30)
    normal = sv >= 2.0 ** -14                          # normal binary16 scales: half an ulp is 2^-11 relative
    assert np.all(over[normal] <= 127 * sv[normal] * 2.0 ** -11 * 1.01)


def test_fp8_row_f16_scale_equals_fp32_scale_when_exact():
    from oracle.codecs import quant_fp8_row
    rng = np.random.default_rng(14)
    amax = (448.0 * 2.0 ** rng.integers(-10, 4, size=300)).astype(np.float32)
    x = (rng.uniform(-0.99, 0.99, (300, 256)) * amax[:, None]).astype(np.float32)
    x[np.arange(300), rng.integers(0, 256, size=300)] = amax
    c4, s4 = quant_fp8_row(x, 4)
    c2, s2 = quant_fp8_row(x, 2)
    assert np.array_equal(c4, c2)
    assert np.array_equal(s2.view(np.float16).astype(np.float32), s4)


@pytest.mark.parametrize("profile,table_bytes", [("BF16", 1024), ("INT8_G64", 528), ("FP8_E4M3FN_ROW256", 516),
                                                 ("NVFP4_G16", 288), ("K8V4", 402)])
def test_store_with_two_byte_scales_reproduces_the_d256_payload_table(profile, table_bytes):
    from oracle.pool import OraclePool
    from oracle.store import OracleStore
    pool = OraclePool(S=1024, C=1, M=16)
    st = OracleStore(pool, profile, 2, 256, 1, scale_bytes=2)
    per_token_head = sum(arr[0, 0, 0].nbytes for arr in st.planes[0].values())
    assert per_token_head == table_bytes
    assert st.replica_page_bytes() == table_bytes * 2 * 64
