"""Pins of the dense / grouped oracle against facts independent of it.

* 16-bit float decoding is checked exhaustively against numpy's float16 and
  against the definition of bf16 (the upper half of an fp32 pattern).
* RNE encoding is checked against numpy's float64->float16 conversion and, for
  bf16, against the nearest-representable property on constructed midpoints.
* The W4A16 definition (Humming article, quantization descriptor: group INT4
  weights, per-group scale and zero point; MSD page §4.2-4.3: scale of shape
  (K/128, N)) is pinned by special cases that reduce to other computations:
  integer activations with unit scales equal an int64 matmul; a unit row of x
  picks one dequantised weight row (pins nibble order, group index, scale and
  zero indexing); signed weights equal the unsigned encoding q+8 with zero 8.
* Scale groups of 32, 64 and 256 rows (Humming article: the descriptor keeps
  the scale granularity as a parameter): the unit-row probe at the group
  edges, and integer activations with power-of-two scales per group equal an
  int64 reduction (per-group int64 matmuls, each scaled exactly).
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_f16_decode_exhaustive(orc):
    L = orc.lib()
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([L.oracle_f16_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_bf16_decode_exhaustive(orc):
    L = orc.lib()
    bits = np.arange(65536, dtype=np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([L.oracle_bf16_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_f16_encode_matches_numpy(orc):
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        # exact midpoints between adjacent fp16 values (ties) and their neighbours
        (np.arange(0, 65504, dtype=np.float64)[::97] + 0.5),
        np.array([65519.99, 65520.0, 6.0e-8, 2.98e-8, 2.9802322387695312e-08, 0.0, -0.0]),
    ])
    got = orc.round_array(v, orc.F16)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def _bf16_val(b):
    return (np.uint32(b) << np.uint32(16)).view(np.float32).astype(np.float64) if np.isscalar(b) else \
        (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_bf16_encode_nearest_even(orc):
    rng = np.random.default_rng(2)
    base = rng.integers(0x0080, 0x7F00, 5000).astype(np.uint16)      # normal bf16 patterns
    lo = _bf16_val(base)
    hi = _bf16_val(base + 1)
    mids = (lo + hi) / 2.0                                            # exact ties in fp64
    frac = lo + (hi - lo) * rng.random(5000)
    v = np.concatenate([mids, -mids, frac])
    got = orc.round_array(v, orc.BF16)
    gv = _bf16_val(got)
    # nearest: no representable neighbour is strictly closer
    for nb in (got.astype(np.int64) - 1, got.astype(np.int64) + 1):
        nv = _bf16_val(nb.astype(np.uint16))
        assert np.all(np.abs(v - gv) <= np.abs(v - nv))
    # ties go to the even mantissa
    t = np.abs(v[:10000]) == np.abs(mids.tolist() * 2)
    assert np.all((got[:10000][t] & 1) == 0)


def test_integer_case_equals_int64_matmul(orc):
    """scale = 1, no zero point, integer x: the product is an exact int matmul."""
    M, K, N = 5, 384, 192
    rng = np.random.default_rng(3)
    xi = rng.integers(-20, 21, size=(M, K))
    q = rng.integers(-8, 8, size=(K, N))
    for dt in (orc.F16, orc.BF16):
        x = synth.to_bits(xi.astype(np.float32), dt)
        w = synth.pack_nibbles((q & 0xF).astype(np.uint8))
        s = synth.to_bits(np.ones((K // 128, N), np.float32), dt)
        y64, _ = orc.w4a16(x, w, s, None, M, K, N, dt)
        assert np.array_equal(y64, (xi.astype(np.int64) @ q.astype(np.int64)).astype(np.float64))


def test_unit_row_probe_pins_indexing(orc):
    """x = e_k selects dequant(W)[k, :] = (q[k,:] - z[g,:]) * s[g,:]."""
    p = synth.make_dense(1, 512, 64, synth.BF16, signed=False, seed=5)
    K, N = p.K, p.N
    s = synth.bits_to_f32(p.scale, p.dtype).astype(np.float64)
    z = synth.unpack_nibbles(p.zero).astype(np.int64)
    for k in (0, 1, 2, 127, 128, 129, 300, 511):
        xk = np.zeros((1, K), np.float32)
        xk[0, k] = 1.0
        x = synth.to_bits(xk, p.dtype)
        y64, _ = orc.w4a16(x, p.w, p.scale, p.zero, 1, K, N, p.dtype)
        g = k // 128
        expect = (p.q[k].astype(np.int64) - z[g]) * s[g]
        assert np.array_equal(y64[0], expect), k


def test_signed_equals_unsigned_plus_8(orc):
    p = synth.make_dense(3, 256, 128, synth.F16, signed=True, seed=6)
    y_s, _ = orc.w4a16(p.x, p.w, p.scale, None, p.M, p.K, p.N, p.dtype)
    u = (p.q.astype(np.int64) + 8).astype(np.uint8)
    w_u = synth.pack_nibbles(u)
    z8 = synth.pack_nibbles(np.full((p.G, p.N), 8, np.uint8))
    y_u, _ = orc.w4a16(p.x, w_u, p.scale, z8, p.M, p.K, p.N, p.dtype)
    assert np.array_equal(y_s, y_u)


def test_power_of_two_scale_is_linear(orc):
    p = synth.make_dense(4, 256, 64, synth.BF16, signed=True, seed=7)
    s2 = synth.to_bits(synth.bits_to_f32(p.scale, p.dtype) * 4.0, p.dtype)
    y1, _ = orc.w4a16(p.x, p.w, p.scale, None, p.M, p.K, p.N, p.dtype)
    y2, _ = orc.w4a16(p.x, p.w, s2, None, p.M, p.K, p.N, p.dtype)
    assert np.array_equal(y2, 4.0 * y1)


def test_points_match_full(orc):
    p = synth.make_dense(6, 384, 128, synth.BF16, signed=False, seed=8)
    y64, y = orc.w4a16(p.x, p.w, p.scale, p.zero, p.M, p.K, p.N, p.dtype)
    rng = np.random.default_rng(0)
    rows = rng.integers(0, p.M, 50)
    cols = rng.integers(0, p.N, 50)
    pts = orc.w4a16_points(p.x, p.w, p.scale, p.zero, p.M, p.K, p.N, p.dtype, rows, cols)
    assert np.array_equal(pts, y64[rows, cols])
    assert np.array_equal(y, orc.round_array(y64, p.dtype))


def test_grouped_reduces_to_dense(orc):
    counts = [5, 0, 17, 1, 0, 9]
    p = synth.make_grouped(len(counts), 20, 2, 256, 128, synth.BF16, counts=counts, seed=9)
    y64, y = orc.grouped(p.x, p.offsets, p.w, p.scale, None, p.E, p.M, p.K, p.N, p.dtype)
    for e, c in enumerate(counts):
        r0, r1 = p.offsets[e], p.offsets[e + 1]
        assert r1 - r0 == c
        if c == 0:
            continue
        ye, _ = orc.w4a16(np.ascontiguousarray(p.x[r0:r1]), np.ascontiguousarray(p.w[e]),
                          np.ascontiguousarray(p.scale[e]), None, c, p.K, p.N, p.dtype)
        assert np.array_equal(y64[r0:r1], ye)


def test_moe_routing_shape():
    p = synth.moe()
    assert p.M == 512 * 8 and p.offsets[-1] == p.M and p.E == 64
    counts = np.diff(p.offsets)
    assert counts.min() >= 0 and counts.max() > 4 * np.median(counts)   # skewed


@pytest.mark.parametrize("group", [32, 64, 256])
@pytest.mark.parametrize("signed", [False, True])
def test_unit_row_probe_small_groups(orc, group, signed):
    p = synth.make_dense(1, 512, 64, synth.F16, signed=signed, seed=11 + group, group=group)
    K, N = p.K, p.N
    s = synth.bits_to_f32(p.scale, p.dtype).astype(np.float64)
    z = synth.unpack_nibbles(p.zero).astype(np.int64) if p.zero is not None else np.zeros((K // group, N), np.int64)
    for k in sorted({0, 1, group - 1, group, group + 1, 2 * group - 1, 255, 256, 511}):
        xk = np.zeros((1, K), np.float32)
        xk[0, k] = 1.0
        y64, _ = orc.w4a16(synth.to_bits(xk, p.dtype), p.w, p.scale, p.zero, 1, K, N, p.dtype, group=group)
        g = k // group
        expect = (p.q[k].astype(np.int64) - z[g]) * s[g]
        assert np.array_equal(y64[0], expect), (group, k)


@pytest.mark.parametrize("group", [32, 64])
def test_small_groups_integer_reduction(orc, group):
    """Integer x, zero points, scales 2^e (e in [-3, 3]) per (group, column):
    8 * y equals sum_g x_g . ((q - z)_g * 2^(e_g + 3)) in int64."""
    M, K, N = 6, 384, 128
    rng = np.random.default_rng(group)
    G = K // group
    xi = rng.integers(-30, 31, size=(M, K))
    u = rng.integers(0, 16, size=(K, N))
    zq = rng.integers(0, 16, size=(G, N))
    e = rng.integers(-3, 4, size=(G, N))
    for dt in (orc.F16, orc.BF16):
        x = synth.to_bits(xi.astype(np.float32), dt)
        s = synth.to_bits(np.exp2(e).astype(np.float32), dt)
        y64, _ = orc.w4a16(x, synth.pack_nibbles(u.astype(np.uint8)), s, synth.pack_nibbles(zq.astype(np.uint8)),
                           M, K, N, dt, group=group)
        acc = np.zeros((M, N), np.int64)
        for g in range(G):
            rows = slice(g * group, (g + 1) * group)
            wg = (u[rows] - zq[g]) * (2 ** (e[g] + 3))
            acc += xi[:, rows].astype(np.int64) @ wg.astype(np.int64)
        assert np.array_equal(y64 * 8, acc.astype(np.float64)), dt


def test_grouped_small_groups_reduce_to_dense(orc):
    counts = [7, 0, 33, 2]
    p = synth.make_grouped(len(counts), 20, 2, 256, 128, synth.F16, counts=counts, seed=12, group=32)
    y64, _ = orc.grouped(p.x, p.offsets, p.w, p.scale, None, p.E, p.M, p.K, p.N, p.dtype, group=32)
    for ex, c in enumerate(counts):
        r0, r1 = p.offsets[ex], p.offsets[ex + 1]
        if c == 0:
            continue
        ye, _ = orc.w4a16(np.ascontiguousarray(p.x[r0:r1]), np.ascontiguousarray(p.w[ex]),
                          np.ascontiguousarray(p.scale[ex]), None, c, p.K, p.N, p.dtype, group=32)
        assert np.array_equal(y64[r0:r1], ye)
