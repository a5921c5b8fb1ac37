"""Pins of the W8A16 oracle (Humming article: the WNA16 setting with 8-bit
integer weights, 16-bit activations, group scales and optional zero points)
against facts independent of it:

* integer activations with unit scales: the result equals numpy's int64
  matmul of x and (q - z) exactly;
* unit rows of x pick single dequantized weight rows, computed here from the
  bytes (two's complement int8 without zero points, uint8 minus its group's
  zero point otherwise), which pins the sign rule and the group and zero
  indexing;
* signed weights equal their unsigned encoding q + 128 with zero point 128;
* doubling one group's scales doubles exactly that group's share;
* weights within [-8, 7] give the same result as the independent W4A16 oracle;
* the 16-bit result is the fp64 sum rounded once to nearest even.
"""
import numpy as np
import pytest

import synth
from test_oracle_moe import rne


def _problem(rng, M, K, N, dtype, signed, group=128, int_x=False, unit_scale=False):
    G = K // group
    x = rng.integers(-3, 4, (M, K)).astype(np.float32) if int_x else rng.standard_normal((M, K)).astype(np.float32)
    xb = synth.to_bits(x, dtype)
    w = rng.integers(0, 256, (K, N), dtype=np.uint8)
    s = np.ones((G, N), np.float32) if unit_scale else (0.001 + 0.01 * rng.random((G, N))).astype(np.float32)
    sb = synth.to_bits(s, dtype)
    z = None if signed else rng.integers(100, 156, (G, N), dtype=np.uint8)
    return xb, w, sb, z


def _deq(w, s_bits, z, dtype, group):
    K, N = w.shape
    q = w.astype(np.int8).astype(np.int64) if z is None else w.astype(np.int64)
    zz = 0 if z is None else np.repeat(z.astype(np.int64), group, axis=0)
    sv = np.repeat(synth.bits_to_f32(s_bits, dtype).astype(np.float64), group, axis=0)
    return (q - zz).astype(np.float64) * sv, q - zz


@pytest.mark.parametrize("signed", [True, False])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
def test_integer_inputs_equal_int64_matmul(orc, signed, dtype):
    rng = np.random.default_rng(1)
    M, K, N = 5, 256, 48
    x, w, s, z = _problem(rng, M, K, N, dtype, signed, int_x=True, unit_scale=True)
    y64, _ = orc.w8a16(x, w, s, z, M, K, N, dtype)
    _, qz = _deq(w, s, z, dtype, 128)
    xi = synth.bits_to_f32(x, dtype).astype(np.int64)
    assert np.array_equal(y64, (xi @ qz).astype(np.float64))


@pytest.mark.parametrize("signed", [True, False])
@pytest.mark.parametrize("group", [128, 256])
def test_unit_rows_pick_dequantized_rows(orc, signed, group):
    rng = np.random.default_rng(2)
    K, N, dt = 512, 64, synth.BF16
    _, w, s, z = _problem(rng, 1, K, N, dt, signed, group=group)
    ks = [0, 1, 127, 128, 255, 300, 511]
    x = np.zeros((len(ks), K), np.float32)
    x[np.arange(len(ks)), ks] = 1.0
    y64, _ = orc.w8a16(synth.to_bits(x, dt), w, s, z, len(ks), K, N, dt, group=group)
    wd, _ = _deq(w, s, z, dt, group)
    assert np.array_equal(y64, wd[ks])
    # the sign rule on its own: byte 0xFF is -1 without zero points, 255 - z with them
    w2 = np.zeros_like(w)
    w2[0, :] = 0xFF
    y2, _ = orc.w8a16(synth.to_bits(x[:1], dt), w2, s, z, 1, K, N, dt, group=group)
    sv = synth.bits_to_f32(s[0], dt).astype(np.float64)
    assert np.array_equal(y2[0], -sv if z is None else (255.0 - z[0]) * sv)


def test_signed_equals_unsigned_with_zero_128(orc):
    rng = np.random.default_rng(3)
    M, K, N, dt = 3, 384, 64, synth.F16
    x, w, s, _ = _problem(rng, M, K, N, dt, True)
    y_s, _ = orc.w8a16(x, w, s, None, M, K, N, dt)
    u = (w.astype(np.int8).astype(np.int16) + 128).astype(np.uint8)
    y_u, _ = orc.w8a16(x, u, s, np.full((K // 128, N), 128, np.uint8), M, K, N, dt)
    assert np.array_equal(y_s, y_u)


def test_group_scale_linearity_and_rounding(orc):
    rng = np.random.default_rng(4)
    M, K, N, dt = 4, 512, 32, synth.BF16
    x, w, s, z = _problem(rng, M, K, N, dt, False)
    base, y = orc.w8a16(x, w, s, z, M, K, N, dt)
    assert np.array_equal(y, rne(base, dt))
    s2 = synth.to_bits(synth.bits_to_f32(s, dt) * np.float32(2.0), dt)
    s2[[0, 2, 3]] = s[[0, 2, 3]]                           # only group 1 doubled
    y2, _ = orc.w8a16(x, w, s2, z, M, K, N, dt)
    x1 = np.zeros_like(x)
    x1[:, 128:256] = x[:, 128:256]
    share, _ = orc.w8a16(x1, w, s, z, M, K, N, dt)
    assert np.allclose(y2 - base, share, rtol=1e-12, atol=1e-300)


def test_small_weights_match_w4a16_oracle(orc):
    rng = np.random.default_rng(5)
    M, K, N, dt = 6, 256, 64, synth.BF16
    q = rng.integers(-8, 8, (K, N)).astype(np.int8)
    x = synth.to_bits(rng.standard_normal((M, K)).astype(np.float32), dt)
    s = synth.to_bits((0.002 + 0.01 * rng.random((K // 128, N))).astype(np.float32), dt)
    y8, _ = orc.w8a16(x, q.view(np.uint8), s, None, M, K, N, dt)
    y4, _ = orc.w4a16(x, synth.pack_nibbles(q.view(np.uint8) & 0xF), s, None, M, K, N, dt)
    assert np.array_equal(y8, y4)


def test_channel_scale_composition(orc):
    """The secondary per-column scale: t = 1 leaves the product unchanged,
    t = 2^k shifts every 16-bit result by k in the exponent (no overflow,
    no subnormals here), and the result is the fp64 product rounded once."""
    rng = np.random.default_rng(9)
    M, K, N, dt = 3, 256, 32, synth.BF16
    q = rng.integers(-8, 8, (K, N)).astype(np.int8)
    x = synth.to_bits(rng.standard_normal((M, K)).astype(np.float32), dt)
    s = synth.to_bits((0.002 + 0.01 * rng.random((K // 128, N))).astype(np.float32), dt)
    y64, y = orc.w8a16(x, q.view(np.uint8), s, None, M, K, N, dt)
    v1, b1 = orc.channel_scaled(y64, np.ones(N, np.float32), dt)
    assert np.array_equal(v1, y64) and np.array_equal(b1, y)
    k = rng.integers(-3, 4, N)
    v2, b2 = orc.channel_scaled(y64, np.exp2(k).astype(np.float32), dt)
    ybits = y.astype(np.int64)
    shifted = np.where(ybits & 0x7FFF, ybits + (k[None, :] << 7), ybits)   # bf16 exponent field starts at bit 7
    assert np.array_equal(b2.astype(np.int64), shifted)
    t = rng.uniform(0.5, 2.0, N).astype(np.float32)
    v3, b3 = orc.channel_scaled(y64, t, dt)
    assert np.array_equal(b3, rne(y64 * t.astype(np.float64), dt))


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
def test_float_zero_points(orc, dtype):
    """W4A16 with floating-point zero points: integer-valued zero points give
    the integer-zero-point oracle's result; zero points 0 with integer x and
    unit scales give numpy's int64 matmul of the unsigned codes; raising one
    group's zero points by d moves the result by exactly -d * s * (row sum of
    x over that group)."""
    rng = np.random.default_rng(12)
    M, K, N, group = 4, 512, 32, 256
    G = K // group
    u = rng.integers(0, 16, (K, N)).astype(np.uint8)
    w = synth.pack_nibbles(u)
    x = synth.to_bits(rng.standard_normal((M, K)).astype(np.float32), dtype)
    s = synth.to_bits((0.002 + 0.01 * rng.random((G, N))).astype(np.float32), dtype)
    zi = rng.integers(0, 16, (G, N)).astype(np.uint8)
    y_int, _ = orc.w4a16(x, w, s, synth.pack_nibbles(zi), M, K, N, dtype, group=group)
    y_f, _ = orc.w4a16_fzero(x, w, s, synth.to_bits(zi.astype(np.float32), dtype), M, K, N, dtype, group=group)
    assert np.array_equal(y_int, y_f)
    xi = rng.integers(-3, 4, (M, K)).astype(np.float32)
    ones = synth.to_bits(np.ones((G, N), np.float32), dtype)
    zeros = synth.to_bits(np.zeros((G, N), np.float32), dtype)
    y0, _ = orc.w4a16_fzero(synth.to_bits(xi, dtype), w, ones, zeros, M, K, N, dtype, group=group)
    assert np.array_equal(y0, (xi.astype(np.int64) @ u.astype(np.int64)).astype(np.float64))
    zf = (rng.random((G, N)) * 15).astype(np.float32)
    zb = synth.to_bits(zf, dtype)
    base, _ = orc.w4a16_fzero(x, w, s, zb, M, K, N, dtype, group=group)
    zb2 = zb.copy()
    zb2[1] = synth.to_bits(synth.bits_to_f32(zb[1], dtype) + np.float32(0.5), dtype)
    y2, _ = orc.w4a16_fzero(x, w, s, zb2, M, K, N, dtype, group=group)
    d = synth.bits_to_f32(zb2[1], dtype).astype(np.float64) - synth.bits_to_f32(zb[1], dtype).astype(np.float64)
    xv = synth.bits_to_f32(x, dtype).astype(np.float64)
    S1 = xv[:, group:2 * group].sum(axis=1)
    sv = synth.bits_to_f32(s[1], dtype).astype(np.float64)
    assert np.allclose(y2 - base, -S1[:, None] * (d * sv)[None, :], rtol=1e-9, atol=1e-12)


def test_w8_float_zero_points(orc):
    """8-bit codes with floating-point zero points: integer-valued zero points
    reproduce the uint8-zero-point oracle; a half-unit shift of one group's
    zero points moves the result by -0.5 * s * (that group's row sum of x)."""
    rng = np.random.default_rng(13)
    M, K, N, dt = 3, 256, 32, synth.F16
    x, w, s, z = _problem(rng, M, K, N, dt, False)
    y_int, _ = orc.w8a16(x, w, s, z, M, K, N, dt)
    y_f, _ = orc.w8a16_fzero(x, w, s, synth.to_bits(z.astype(np.float32), dt), M, K, N, dt)
    assert np.array_equal(y_int, y_f)
    zf = z.astype(np.float32)
    zf[0] += 0.5
    y_h, _ = orc.w8a16_fzero(x, w, s, synth.to_bits(zf, dt), M, K, N, dt)
    S0 = synth.bits_to_f32(x, dt).astype(np.float64)[:, :128].sum(axis=1)
    sv = synth.bits_to_f32(s[0], dt).astype(np.float64)
    assert np.allclose(y_h - y_f, -0.5 * S0[:, None] * sv[None, :], rtol=1e-9, atol=1e-12)
