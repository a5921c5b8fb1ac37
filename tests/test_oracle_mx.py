"""Pins of the W4A8-MXFP4 oracle (Humming article: the W4A8-MXFP4 path, MXFP4
weights with 8-bit activations; element and scale formats per the OCP
Microscaling Formats (MX) v1.0 specification: E2M1 and E4M3 elements, E8M0
shared scales, blocks of 32 along K) against facts independent of it:

* E4M3 and E8M0 decoding of all 256 codes equals torch's float8_e4m3fn and
  float8_e8m0fnu types; E2M1 decoding equals the bit-field formula (sign,
  2-bit exponent with bias 1, 1-bit mantissa, subnormal at exponent 0);
* MXFP8 quantization: the shared exponent is floor(log2 amax) - 8 computed by
  numpy, the element codes equal torch's round-to-nearest-even cast of the
  clamped scaled values, the block maximum lands in [256, 448], values that
  are exactly representable round-trip, and an all-zero block gets the
  smallest scale;
* the product with unit scales equals an fp64 matmul of the decoded operands;
  one scale step doubles exactly the contribution of its block (so a
  transposed or misplaced scale index fails); the low nibble holds the even
  column.
"""
import numpy as np
import pytest
import torch

import synth
from test_oracle_moe import rne


def _torch_decode(codes, dt):
    return torch.from_numpy(np.asarray(codes, np.uint8).copy()).view(dt).double().numpy()


def _e2m1_bitfield(c):
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e.astype(np.float64) - 1))
    return np.where(s == 1, -mag, mag)


def test_element_and_scale_decoding(orc):
    L = orc.lib()
    codes = np.arange(256, dtype=np.uint8)
    e4 = np.array([L.oracle_e4m3_to_double(int(c)) for c in codes])
    ref = _torch_decode(codes, torch.float8_e4m3fn)
    assert np.array_equal(np.isnan(e4), np.isnan(ref)) and np.isnan(e4).sum() == 2
    assert np.array_equal(e4[~np.isnan(e4)], ref[~np.isnan(ref)])
    e8 = np.array([L.oracle_e8m0_to_double(int(c)) for c in codes])
    ref8 = _torch_decode(codes, torch.float8_e8m0fnu)
    assert np.isnan(e8[255]) and np.array_equal(e8[:255], ref8[:255])
    e2 = np.array([L.oracle_e2m1_to_double(int(c)) for c in range(16)])
    assert np.array_equal(e2, _e2m1_bitfield(np.arange(16)))
    assert e2.max() == 6.0 and e4[0x7E] == 448.0 and e8[127] == 1.0


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
def test_mxfp8_quantize_definition(orc, dtype):
    rng = np.random.default_rng(11)
    M, K = 5, 256
    x = synth.to_bits((rng.standard_normal((M, K)) * np.exp2(rng.integers(-6, 7, (M, 1)))).astype(np.float32),
                      dtype)
    xv = synth.bits_to_f32(x, dtype).astype(np.float64)
    qx, sx = orc.mxfp8_quantize(x, M, K, dtype)
    blocks = np.abs(xv).reshape(M, K // 32, 32).max(axis=2)
    e = np.floor(np.log2(blocks)).astype(np.int64) - 8
    assert np.array_equal(sx.astype(np.int64), e + 127)
    scaled = xv / np.exp2(np.repeat(e, 32, axis=1))
    ref = torch.from_numpy(np.clip(scaled, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(qx, ref)
    dec = _torch_decode(qx, torch.float8_e4m3fn).reshape(M, K // 32, 32)
    top = np.abs(dec).max(axis=2)
    assert (top >= 256).all() and (top <= 448).all()


def test_mxfp8_exact_values_round_trip_and_zero_block(orc):
    # every element a multiple of 2^-3 times a power of two within E4M3's
    # range relative to the block maximum -> exact round trip
    dt = synth.BF16
    vals = np.array([1.0, -1.5, 0.75, 2.0, 3.5, -0.125, 0.0, 1.875] * 4, np.float32)
    x = np.stack([vals, vals * 64.0, np.zeros(32, np.float32)])
    xb = synth.to_bits(x, dt)
    qx, sx = orc.mxfp8_quantize(xb, 3, 32, dt)
    dec = _torch_decode(qx, torch.float8_e4m3fn) * np.exp2(sx.astype(np.float64) - 127)
    assert np.array_equal(dec[:2], x[:2].astype(np.float64))
    assert sx[2, 0] == 0 and not qx[2].any()
    assert sx[1, 0] == sx[0, 0] + 6                            # 64 = 2^6
    # a block maximum of 500 (shared exponent 0) saturates to 448; 17 sits
    # halfway between 16 and 18 and rounds to the even mantissa (16)
    y = np.zeros((1, 32), np.float32)
    y[0, :3] = [500.0, -500.0, 17.0]
    qy, sy = orc.mxfp8_quantize(synth.to_bits(y, dt), 1, 32, dt)
    assert sy[0, 0] == 127 and qy[0, 0] == 0x7E and qy[0, 1] == 0xFE
    assert _torch_decode(qy[0, 2:3], torch.float8_e4m3fn)[0] == 16.0


def _problem(rng, M, K, N):
    qx = rng.integers(0, 256, (M, K), dtype=np.uint8)
    qx[(qx & 0x7F) == 0x7F] = 0x30                            # no NaN codes
    sx = rng.integers(120, 135, (M, K // 32), dtype=np.uint8)
    w = rng.integers(0, 256, (K, N // 2), dtype=np.uint8)
    sw = rng.integers(118, 130, (K // 32, N), dtype=np.uint8)
    return qx, sx, w, sw


def _decoded(qx, sx, w, sw):
    M, K = qx.shape
    N = w.shape[1] * 2
    a = _torch_decode(qx, torch.float8_e4m3fn) * np.exp2(np.repeat(sx.astype(np.float64) - 127, 32, axis=1))
    codes = np.empty((K, N), np.int64)
    codes[:, 0::2] = w & 0xF
    codes[:, 1::2] = w >> 4
    b = _e2m1_bitfield(codes) * np.exp2(np.repeat(sw.astype(np.float64) - 127, 32, axis=0))
    return a, b


@pytest.mark.parametrize("M,K,N", [(1, 128, 32), (3, 256, 48), (7, 96, 16)])
def test_product_is_decoded_matmul(orc, M, K, N):
    rng = np.random.default_rng(M * K + N)
    qx, sx, w, sw = _problem(rng, M, K, N)
    y64, y = orc.w4a8_mxfp4(qx, sx, w, sw, M, K, N, synth.BF16)
    a, b = _decoded(qx, sx, w, sw)
    ref = a @ b
    assert np.allclose(y64, ref, rtol=1e-12, atol=1e-300)
    # unit scales: the raw element matmul
    ones_x, ones_w = np.full_like(sx, 127), np.full_like(sw, 127)
    y64u, _ = orc.w4a8_mxfp4(qx, ones_x, w, ones_w, M, K, N, synth.BF16)
    a1, b1 = _decoded(qx, ones_x, w, ones_w)
    assert np.allclose(y64u, a1 @ b1, rtol=1e-12, atol=1e-300)
    # the 16-bit result is the fp64 sum rounded once to nearest even
    assert np.array_equal(y, rne(y64, synth.BF16))


def test_scale_steps_and_nibble_order(orc):
    rng = np.random.default_rng(5)
    M, K, N = 2, 128, 8
    qx, sx, w, sw = _problem(rng, M, K, N)
    base, _ = orc.w4a8_mxfp4(qx, sx, w, sw, M, K, N, synth.F16)
    a, b = _decoded(qx, sx, w, sw)
    # weight scale of block 2, column 5, one step up: only column 5 changes, by
    # exactly that block's partial product
    sw2 = sw.copy()
    sw2[2, 5] += 1
    y2, _ = orc.w4a8_mxfp4(qx, sx, w, sw2, M, K, N, synth.F16)
    part = a[:, 64:96] @ b[64:96, 5]
    assert np.allclose(y2[:, 5] - base[:, 5], part, rtol=1e-12, atol=1e-300)
    assert np.array_equal(np.delete(y2, 5, axis=1), np.delete(base, 5, axis=1))
    # activation scale of row 1, block 3
    sx2 = sx.copy()
    sx2[1, 3] += 1
    y3, _ = orc.w4a8_mxfp4(qx, sx2, w, sw, M, K, N, synth.F16)
    assert np.allclose(y3[1] - base[1], a[1, 96:] @ b[96:], rtol=1e-12, atol=1e-300)
    assert np.array_equal(y3[0], base[0])
    # low nibble = even column: a weight of 1.0 (code 2) at (k=0, n=2) only
    qx1 = np.zeros_like(qx)
    qx1[:, 0] = 0x38                                          # 1.0
    w1 = np.zeros_like(w)
    w1[0, 1] = 0x02                                           # byte 1, low nibble -> column 2
    y4, _ = orc.w4a8_mxfp4(qx1, np.full_like(sx, 127), w1, np.full_like(sw, 127), M, K, N, synth.BF16)
    exp = np.zeros((M, N))
    exp[:, 2] = 1.0
    assert np.array_equal(y4, exp)
