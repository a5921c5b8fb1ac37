"""Pins of the fused-experts (MoE chain) oracle against facts independent of it.

The chain is the one the pages name (pwwt.cn notes, §5: fused_experts_impl runs
an expert GEMM, a fused SiLU-and-multiply and a second expert GEMM;
FlagGems-vLLM operator list, MoE and activation tables: moe_align_block_size,
silu_and_mul, moe_sum).  Each step is pinned by something other than the
oracle itself:

* routing prep equals numpy's stable argsort of the expert ids, with entries
  outside [0, E) dropped;
* silu_and_mul equals scipy's logistic function times the gate times the up
  half, rounded once (round-to-nearest-even checked by an independent
  fp64 -> bf16/fp16 rounding), and SiLU's closed forms (0 at 0, 1/(1+e^-1)
  at 1, ~g for large g, ~0 for very negative g);
* moe_sum with one-hot routing weights selects a row exactly, and otherwise
  equals an fp64 numpy sum rounded once;
* the whole chain with one expert and top-1 reduces to dense oracle GEMMs
  around silu_and_mul, is invariant under relabelling the experts, equals one
  expert when the top-2 experts are identical copies with weights summing to
  1, and ignores unrouted entries.
"""
import numpy as np
import pytest
from scipy.special import expit

import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _f64_of(bits, dtype):
    return synth.bits_to_f32(bits, dtype).astype(np.float64)


def rne(v, dtype):
    """Independent round-to-nearest-even of fp64 values to 16-bit patterns:
    pick the nearest of the neighbouring patterns of a first guess (ties to
    the even pattern)."""
    v = np.asarray(v, dtype=np.float64)
    guess = synth.to_bits(v.astype(np.float32), dtype).astype(np.int64)
    best = guess.copy()
    bestd = np.abs(_f64_of(guess.astype(np.uint16), dtype) - v)
    for delta in (-1, 1):
        cand = (guess + delta) & 0xFFFF
        cv = _f64_of(cand.astype(np.uint16), dtype)
        d = np.abs(cv - v)
        better = (d < bestd) | ((d == bestd) & (cand % 2 == 0) & (best % 2 == 1))
        best = np.where(better & np.isfinite(cv), cand, best)
        bestd = np.where(better & np.isfinite(cv), d, bestd)
    return best.astype(np.uint16)


@pytest.mark.parametrize("E", [1, 5, 64])
def test_align_is_stable_argsort(orc, E):
    rng = np.random.default_rng(E)
    ids = rng.integers(-1, E + 1, size=(37, 4)).astype(np.int32)      # includes -1 and E (not routed)
    off, srt, row_of = orc.moe_align(ids, E)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    order = np.argsort(np.where(valid, flat, E), kind="stable")[: int(valid.sum())]
    assert np.array_equal(srt, order)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat[valid], minlength=E))]))
    inv = np.full(flat.size, -1)
    inv[order] = np.arange(order.size)
    assert np.array_equal(row_of, inv)


def test_align_empty_and_all_unrouted(orc):
    off, srt, row_of = orc.moe_align(np.full((3, 2), -1, np.int32), 4)
    assert off.tolist() == [0, 0, 0, 0, 0] and srt.size == 0 and (row_of == -1).all()


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
def test_silu_and_mul_matches_logistic(orc, dtype):
    rng = np.random.default_rng(3)
    R, I = 9, 64
    h = synth.to_bits((rng.standard_normal((R, 2 * I)) * 3).astype(np.float32), dtype)
    a = orc.silu_and_mul(h, dtype)
    hv = _f64_of(h, dtype)
    g, u = hv[:, :I], hv[:, I:]
    assert np.array_equal(a, rne(g * expit(g) * u, dtype))
    # the gate is the first half: swapping the halves changes the result
    assert not np.array_equal(a, rne(u * expit(u) * g, dtype))


def test_silu_closed_forms(orc):
    dt = synth.BF16
    g = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 200.0, -200.0], np.float32)
    h = synth.to_bits(np.concatenate([g, np.ones_like(g)]).reshape(1, -1), dt)
    a = _f64_of(orc.silu_and_mul(h, dt), dt)[0]
    assert a[0] == 0.0
    assert a[1] == _f64_of(rne(1.0 / (1.0 + np.exp(-1.0)), dt), dt)     # 0.7310585786...
    assert a[2] == _f64_of(rne(-1.0 / (1.0 + np.exp(1.0)), dt), dt)     # -0.2689414213...
    assert a[3] == 40.0 and a[5] == 200.0                               # silu(g) -> g
    assert abs(a[4]) < 1e-15 and a[6] == 0.0                            # silu(g) -> 0


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
def test_moe_sum(orc, dtype):
    rng = np.random.default_rng(5)
    T, topk, N = 7, 3, 40
    ids = rng.integers(0, 4, size=(T, topk)).astype(np.int32)
    ids[2, 1] = -1                                                      # one unrouted entry
    _, _, row_of = orc.moe_align(ids, 4)
    R = int((row_of >= 0).sum())
    o = synth.to_bits(rng.standard_normal((R, N)).astype(np.float32), dtype)
    # one-hot weights select a row exactly
    onehot = np.zeros((T, topk), np.float32)
    onehot[:, 0] = 1.0
    out = orc.moe_sum(o, row_of, onehot, dtype)
    assert np.array_equal(out, o[row_of.reshape(T, topk)[:, 0]])
    # general weights: fp64 sum over routed k, rounded once
    w = rng.random((T, topk)).astype(np.float32)
    out = orc.moe_sum(o, row_of, w, dtype)
    ov = _f64_of(o, dtype)
    ref = np.zeros((T, N))
    for t in range(T):
        for k in range(topk):
            r = row_of[t * topk + k]
            if r >= 0:
                ref[t] += np.float64(w[t, k]) * ov[r]
    assert np.array_equal(out, rne(ref, dtype))


@pytest.mark.parametrize("signed", [True, False])
def test_chain_one_expert_is_dense(orc, signed):
    dt = synth.BF16
    c = synth.make_moe_chain(6, 1, 1, 256, 128, dt, signed=signed, seed=2)
    c.topk_w[:] = 1.0
    out = orc.fused_moe(c)
    _, h = orc.w4a16(c.x, c.w13[0], c.s13[0], None if signed else c.z13[0], c.T, c.H, 2 * c.I, dt)
    a = orc.silu_and_mul(h, dt)
    _, o = orc.w4a16(a, c.w2[0], c.s2[0], None if signed else c.z2[0], c.T, c.I, c.H, dt)
    assert np.array_equal(out, o)


def test_chain_relabel_invariant(orc):
    c = synth.make_moe_chain(10, 2, 4, 128, 128, synth.BF16, seed=4)
    base = orc.fused_moe(c)
    perm = np.array([2, 0, 3, 1])                                      # new label of old expert e
    inv = np.argsort(perm)
    c2 = synth.MoeChain(**{**c.__dict__})
    c2.topk_ids = perm[c.topk_ids].astype(np.int32)
    c2.w13, c2.s13, c2.w2, c2.s2 = c.w13[inv], c.s13[inv], c.w2[inv], c.s2[inv]
    assert np.array_equal(orc.fused_moe(c2), base)


def test_chain_duplicate_experts_and_unrouted(orc):
    c = synth.make_moe_chain(5, 2, 2, 128, 128, synth.BF16, seed=6)
    # expert 1 is an exact copy of expert 0; every token routes to both
    for a in ("w13", "s13", "w2", "s2"):
        getattr(c, a)[1] = getattr(c, a)[0]
    c.topk_ids[:] = [0, 1]
    c.topk_w[:] = [0.25, 0.75]
    one = synth.MoeChain(**{**c.__dict__})
    one.topk_ids = np.array([[0, -1]] * c.T, np.int32)                 # second entry not routed
    one.topk_w = np.array([[1.0, 0.5]] * c.T, np.float32)
    assert np.array_equal(orc.fused_moe(c), orc.fused_moe(one))
    none = synth.MoeChain(**{**c.__dict__})
    none.topk_ids = np.full((c.T, 2), -1, np.int32)
    assert not orc.fused_moe(none).any()


@pytest.mark.parametrize("cfg", [dict(T=9, topk=2, E=3, H=256, I=128, dtype=synth.BF16, signed=True),
                                 dict(T=21, topk=4, E=7, H=128, I=256, dtype=synth.F16, signed=False)])
def test_chain_from_steps_equals_per_token_chain(orc, cfg):
    """The chain composed from the oracle's steps over all routed rows (used at
    full size) equals the per-token chain bit for bit, including tokens with
    unrouted entries."""
    c = synth.make_moe_chain(seed=cfg["T"], **cfg)
    c.topk_ids[0, 0] = -1
    c.topk_ids[-1, -1] = cfg["E"]
    assert np.array_equal(orc.fused_moe_steps(c), orc.fused_moe(c))
