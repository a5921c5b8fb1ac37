"""Pins of the step-by-step MSD oracle (WeightQuantBatchMatmulExperiment
operator deep-dive, A16W4 PerGroup pseudo-quant MatMul, §4.1 eqs. 1-11).

What pins what:
* eq.1 A_max: numpy max(|x|) over each (row, 128-group).
* eqs.2-7: (a) worked values derived in exact real arithmetic (no tie is
  near, so binary32 rounding cannot change them); (b) tie witnesses
  (tests/golden/msd_tie_witnesses.txt) re-evaluated with an exact rational
  model of binary32 arithmetic: pins the operation order, the absence of FMA
  contraction and round-half-to-even; (c) exhaustive fp16 sweeps: every layer
  lies in [-7, 7] and the reconstruction error after layer j is below the
  closed-form bound 0.5*A_max/(7.49*14.98^(j-1)) and does not grow with j.
* eq.9 Y_int: numpy int64 matmul of the layers and the integer weights.
* eqs.10-11 (merge, group accumulation): |y_msd - x.dequant(W)| per element is
  bounded by sum_g 0.5*A_max[m,g]/(7.49*14.98^2) * s[g,n] * sum_k|q[k,n]|; a
  dropped layer, a wrong factor, sign or group index breaks the bound.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
C1 = Fraction(float(np.float32(7.49)))
C2 = Fraction(float(np.float32(14.98)))


# ---- exact rational model of binary32 round-to-nearest-even -----------------

def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_half_even(v: Fraction) -> Fraction:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return Fraction(fl)


def f32(v: Fraction) -> Fraction:
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = max(_floor_log2(a), -126)
    q = Fraction(2) ** (e - 23)
    return s * _round_half_even(a / q) * q


def exact_decompose(a: float, amax: float):
    a, amax = Fraction(a), Fraction(amax)
    t1 = f32(f32(C1 * a) / amax)
    A1 = _round_half_even(t1)
    d1 = t1 - A1
    assert f32(d1) == d1
    t2 = f32(d1 * C2)
    A2 = _round_half_even(t2)
    d2 = t2 - A2
    assert f32(d2) == d2
    t3 = f32(d2 * C2)
    A3 = _round_half_even(t3)
    return (int(A1), int(A2), int(A3)), (t1, t2, t3)


def f16(bits):
    return float(np.uint16(bits).view(np.float16))


# ---- tests ------------------------------------------------------------------

def test_factors_are_the_fp32_constants():
    assert float(C1) == 7.489999771118164 and float(C2) == 14.979999542236328
    assert C2 == 2 * C1


@pytest.mark.parametrize("ratio,expect", [
    # a/amax = 1:   7.49 -> 7; 0.49*14.98 = 7.340 -> 7; 0.3402*14.98 = 5.096 -> 5
    (1.0, (7, 7, 5)),
    # 1/2:  3.745 -> 4; -0.255*14.98 = -3.820 -> -4; 0.1801*14.98 = 2.698 -> 3
    (0.5, (4, -4, 3)),
    # 1/4:  1.8725 -> 2; -0.1275*14.98 = -1.910 -> -2; 0.0900*14.98 = 1.349 -> 1
    (0.25, (2, -2, 1)),
    # 3/4:  5.6175 -> 6; -0.3825*14.98 = -5.730 -> -6; 0.2701*14.98 = 4.047 -> 4
    (0.75, (6, -6, 4)),
    (-1.0, (-7, -7, -5)),
    (0.0, (0, 0, 0)),
])
def test_worked_values(orc, ratio, expect):
    for amax in (1.0, 3.0, 0.125, 2048.0):
        layers, _ = orc.msd_decompose_one(ratio * amax, amax)
        assert tuple(int(v) for v in layers) == expect


def test_zero_group_gives_zero_layers(orc):
    x = np.zeros((2, 256), np.float32)
    x[1, 128:] = 0.5
    xb = synth.to_bits(x, synth.F16)
    amax = orc.msd_amax(xb, 2, 256)
    assert amax[0, 0] == 0 and amax[0, 1] == 0 and amax[1, 0] == 0 and amax[1, 1] == 0.5
    layers = orc.msd_layers(xb, amax, 2, 256)
    assert not layers[:, 0, :].any() and not layers[:, 1, :128].any()
    assert tuple(layers[:, 1, 200]) == (7, 7, 5)


def test_tie_witnesses_round_half_even(orc):
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "msd_tie_witnesses.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) >= 8
    for amax_b, a_b, step in rows:
        amax, a, step = f16(int(amax_b, 16)), f16(int(a_b, 16)), int(step)
        expect, ts = exact_decompose(a, amax)
        t = ts[step - 1]
        assert t.denominator == 2, (amax_b, a_b)            # an exact tie at that step
        got, t_or = orc.msd_decompose_one(a, amax)
        assert tuple(int(v) for v in got) == expect, (amax_b, a_b, got, expect)
        assert [Fraction(float(v)) for v in t_or] == list(ts)
        # half-away-from-zero would have given another integer at that step
        away = int(t + (Fraction(1, 2) if t > 0 else Fraction(-1, 2)))
        assert away != expect[step - 1]


def test_random_pairs_match_exact_model(orc):
    rng = np.random.default_rng(11)
    for _ in range(300):
        amax = abs(float(np.float16(rng.standard_normal() * 10.0 ** rng.integers(-3, 4))))
        if amax == 0 or not np.isfinite(amax):
            continue
        a = float(np.float16(amax * rng.uniform(-1, 1)))
        expect, _ = exact_decompose(a, amax)
        got, _ = orc.msd_decompose_one(a, amax)
        assert tuple(int(v) for v in got) == expect


@pytest.mark.parametrize("amax", [1.0, 3.0, 65504.0, 6.103515625e-05, 0.333251953125])
def test_exhaustive_fp16_sweep_bounds(orc, amax):
    allb = np.arange(0, 0x7C00, dtype=np.uint16)
    a = allb.view(np.float16).astype(np.float32)
    a = a[a <= np.float32(amax)]
    a = np.concatenate([a, -a])
    # lay the values out as groups of 128 whose first element is amax
    n_per = 127
    pad = (-a.size) % n_per
    vals = np.concatenate([a, np.zeros(pad, np.float32)]).reshape(-1, n_per)
    x = np.concatenate([np.full((vals.shape[0], 1), amax, np.float32), vals], axis=1)
    M = x.shape[0]
    xb = synth.to_bits(x, synth.F16).reshape(1, -1)
    K = xb.shape[1]
    amx = orc.msd_amax(xb, 1, K)
    assert np.all(amx == np.float32(amax))
    L = orc.msd_layers(xb, amx, 1, K).astype(np.float64)[:, 0, :]
    assert L.min() >= -7 and L.max() <= 7
    av = synth.bits_to_f32(xb, synth.F16).astype(np.float64)[0]
    c1, c2 = float(C1), float(C2)
    r1 = L[0] / c1
    r2 = r1 + L[1] / (c1 * c2)
    r3 = r2 + L[2] / (c1 * c2 * c2)
    errs = [np.abs(av / amax - r) for r in (r1, r2, r3)]
    bounds = [0.5 / c1, 0.5 / (c1 * c2), 0.5 / (c1 * c2 * c2)]
    slack = 4e-7
    for e, b in zip(errs, bounds):
        assert e.max() <= b + slack
        assert e.max() >= 0.9 * b          # the sweep reaches the bound
    assert np.all(errs[1] <= errs[0] + slack)
    assert np.all(errs[2] <= errs[1] + slack)


def test_amax_matches_numpy(orc):
    p = synth.msd(M=5, K=512, N=64)
    a = orc.msd_amax(p.x, p.M, p.K)
    ref = np.abs(synth.bits_to_f32(p.x, synth.F16)).reshape(p.M, p.G, 128).max(axis=2)
    assert np.array_equal(a, ref)


def test_yint_matches_int_matmul(orc):
    p = synth.msd(M=7, K=384, N=96, seed=3)
    amax = orc.msd_amax(p.x, p.M, p.K)
    L = orc.msd_layers(p.x, amax, p.M, p.K)
    Y = orc.msd_yint(L, p.w, p.M, p.K, p.N)
    q = p.q.astype(np.int64)
    for g in range(p.G):
        ks = slice(128 * g, 128 * (g + 1))
        for j in range(3):
            assert np.array_equal(Y[g, j], L[j][:, ks].astype(np.int64) @ q[ks])
    assert np.abs(Y).max() <= 7 * 8 * 128


@pytest.mark.parametrize("seed", [0, 1])
def test_msd_result_within_closed_form_bound(orc, seed):
    p = synth.msd(M=6, K=1024, N=192, seed=seed)
    y64, y, amax, layers = orc.msd(p.x, p.w, p.scale, p.M, p.K, p.N, intermediates=True)
    ye64, _ = orc.w4a16(p.x, p.w, p.scale, None, p.M, p.K, p.N, synth.F16)
    s = synth.bits_to_f32(p.scale, synth.F16).astype(np.float64)          # [G][N]
    absq = np.abs(p.q.astype(np.float64)).reshape(p.G, 128, p.N).sum(axis=1)  # [G][N]
    eps3 = 0.5 / (float(C1) * float(C2) ** 2)
    bound = (amax.astype(np.float64) * (eps3 + 4e-7)) @ (s * absq)          # [M][N]
    err = np.abs(y64 - ye64)
    assert np.all(err <= bound * 1.0001 + 1e-12)
    # the bound is not vacuous: MSD error is visible but much smaller than the signal
    assert err.max() > 0 and err.max() < 0.05 * np.abs(ye64).max()
    # Intermediates agree with the separately exposed steps
    assert np.array_equal(amax, orc.msd_amax(p.x, p.M, p.K))
    assert np.array_equal(layers, orc.msd_layers(p.x, amax, p.M, p.K))
    assert np.array_equal(y, orc.round_array(y64, synth.F16))


def test_msd_dropping_a_layer_breaks_the_bound(orc):
    """Sensitivity check of the bound test: a reconstruction that stops after
    two layers violates it (a planted mistake, made on the CPU side)."""
    p = synth.msd(M=4, K=512, N=64, seed=5)
    _, _, amax, L = orc.msd(p.x, p.w, p.scale, p.M, p.K, p.N, intermediates=True)
    ye64, _ = orc.w4a16(p.x, p.w, p.scale, None, p.M, p.K, p.N, synth.F16)
    c1, c2 = float(C1), float(C2)
    q = p.q.astype(np.float64)
    s = synth.bits_to_f32(p.scale, synth.F16).astype(np.float64)
    y2 = np.zeros((p.M, p.N))
    for g in range(p.G):
        ks = slice(128 * g, 128 * (g + 1))
        Y1 = L[0][:, ks].astype(np.float64) @ q[ks]
        Y2 = L[1][:, ks].astype(np.float64) @ q[ks]
        y2 += ((Y1 / c1 + Y2 / (c1 * c2)) * amax[:, g:g + 1]) * s[g]
    absq = np.abs(q).reshape(p.G, 128, p.N).sum(axis=1)
    bound = (amax.astype(np.float64) * (0.5 / (c1 * c2 * c2) + 4e-7)) @ (s * absq)
    assert np.any(np.abs(y2 - ye64) > bound)
