"""Fused-experts chain (routing prep, gather, gate/up grouped W4A16, SiLU and
multiply, down grouped W4A16, weighted sum) against the oracle, through the
C ABI.  Integer work (routing prep, gather) is compared bit for bit;
silu_and_mul within one unit in the last place of the 16-bit result (fp32 on
the GPU vs fp64 in the oracle, one rounding each); moe_sum bit-identical in
more than 99% of the outputs and everywhere within one unit in the last place
plus the fp32 accumulation bound; the chain with the float tolerance
(max |d| <= 1e-2 max |ref|, relative L1 <= 2e-3)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _ulp_diff(a_bits, b_bits):
    """Distance in 16-bit patterns between two arrays of same-type floats
    (sign-magnitude mapped to a monotone integer line)."""
    def line(b):
        b = np.asarray(b, np.uint16).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(line(a_bits) - line(b_bits))


def _routing(T, topk, E, invalid, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(max(E, topk))[:topk] for _ in range(T)]).astype(np.int32) % E if T else \
        np.zeros((0, topk), np.int32)
    if invalid and T:
        m = rng.random(ids.shape) < 0.1
        ids[m] = rng.choice([-1, E, -7], size=int(m.sum()))
    return ids


@pytest.mark.parametrize("T,topk,E,invalid", [(1, 1, 1, False), (37, 4, 5, True), (700, 3, 64, True),
                                              (512, 8, 64, False), (64, 2, 1024, True), (300, 8, 7, False),
                                              (1100, 8, 16, True), (200, 8, 33, True), (128, 8, 64, False),
                                              (1100, 8, 300, True), (300, 8, 256, False), (150, 8, 257, True)])
def test_align_bit_exact(orc, T, topk, E, invalid):
    import weight_only_quantized_amd as w4
    print(f"[case] align T={T} topk={topk} E={E} invalid={invalid}", flush=True)
    ids = _routing(T, topk, E, invalid, seed=T + E)
    off_ref, srt_ref, row_ref = orc.moe_align(ids, E)
    n = T * topk
    off = torch.full((E + 1,), -5, dtype=torch.int32, device=DEV)
    srt = torch.full((max(n, 1),), -5, dtype=torch.int32, device=DEV)
    row = torch.full((max(n, 1),), -5, dtype=torch.int32, device=DEV)
    w4.w4a16_moe_align(_i32(ids), T, topk, E, off, srt, row)
    torch.cuda.synchronize()
    R = int(off_ref[-1])
    assert np.array_equal(off.cpu().numpy(), off_ref)
    assert np.array_equal(srt.cpu().numpy()[:R], srt_ref)
    assert np.array_equal(row.cpu().numpy()[:n], row_ref)


def test_gather_bit_exact(orc):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_dev, to_host_u16
    T, topk, E, H = 50, 4, 6, 384
    ids = _routing(T, topk, E, True, seed=3)
    off_ref, srt_ref, _ = orc.moe_align(ids, E)
    x = synth.to_bits(np.random.default_rng(1).standard_normal((T, H)).astype(np.float32), synth.BF16)
    xs = torch.zeros((T * topk, H), dtype=torch.int16, device=DEV)
    srt_full = np.zeros(T * topk, np.int32)
    srt_full[:srt_ref.size] = srt_ref
    w4.w4a16_moe_gather(to_dev(x), _i32(srt_full), _i32(off_ref), T, topk, E, H, xs, synth.BF16)
    torch.cuda.synchronize()
    got = to_host_u16(xs)
    R = int(off_ref[-1])
    assert np.array_equal(got[:R], x[srt_ref // topk])
    assert not got[R:].any()                                  # rows past the routed ones untouched


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16])
def test_silu_and_mul(orc, dt):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_dev, to_host_u16
    R, I, rows = 67, 1408, 50
    h = synth.to_bits((np.random.default_rng(dt).standard_normal((R, 2 * I)) * 4).astype(np.float32), dt)
    ref = orc.silu_and_mul(h, dt)
    a = torch.full((R, I), 0x1234, dtype=torch.int16, device=DEV)
    w4.w4a16_silu_and_mul(to_dev(h), _i32([rows]), R, I, a, dt)
    torch.cuda.synchronize()
    got = to_host_u16(a)
    d = _ulp_diff(got[:rows], ref[:rows])
    print(f"[parity] silu_and_mul dt={dt} exact={np.mean(d == 0):.5f} max_ulp={d.max()}", flush=True)
    assert d.max() <= 1 and np.mean(d == 0) > 0.99
    assert (got[rows:] == 0x1234).all()                       # rows past the count untouched
    w4.w4a16_silu_and_mul(to_dev(h), None, R, I, a, dt)
    torch.cuda.synchronize()
    assert _ulp_diff(to_host_u16(a), ref).max() <= 1


@pytest.mark.parametrize("dt", [synth.BF16, synth.F16])
def test_moe_sum(orc, dt):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_dev, to_host_u16
    T, topk, E, N = 93, 8, 16, 2048
    rng = np.random.default_rng(7)
    ids = _routing(T, topk, E, True, seed=9)
    _, _, row_of = orc.moe_align(ids, E)
    R = int((row_of >= 0).sum())
    o = synth.to_bits(rng.standard_normal((R, N)).astype(np.float32), dt)
    w = rng.random((T, topk)).astype(np.float32)
    ref = orc.moe_sum(o, row_of, w, dt)
    out = torch.empty((T, N), dtype=torch.int16, device=DEV)
    w4.w4a16_moe_sum(to_dev(o), _i32(row_of), torch.from_numpy(w).to(DEV), T, topk, N, out, dt)
    torch.cuda.synchronize()
    got = to_host_u16(out)
    d = _ulp_diff(got, ref)
    print(f"[parity] moe_sum dt={dt} exact={np.mean(d == 0):.5f} max_ulp={d.max()}", flush=True)
    assert np.mean(d == 0) > 0.99
    # error bound: one rounding of the result (one unit of the reference's last
    # place) plus fp32 accumulation of topk products, relative to sum |w o|
    # (a sum that nearly cancels can be off by more than one unit of its own
    # last place)
    ov = synth.bits_to_f32(o, dt).astype(np.float64)
    mag = np.zeros((T, N))
    for t in range(T):
        for k in range(topk):
            r = row_of[t * topk + k]
            if r >= 0:
                mag[t] += abs(float(w[t, k])) * np.abs(ov[r])
    refv = synth.bits_to_f32(ref, dt).astype(np.float64)
    nxt = synth.bits_to_f32((ref.astype(np.int64) + 1).astype(np.uint16), dt).astype(np.float64)
    ulp = np.abs(nxt - refv)
    err = np.abs(synth.bits_to_f32(got, dt).astype(np.float64) - refv)
    assert np.all(err <= ulp + topk * 2.0 ** -23 * mag)


class DevChain:
    """A fused-experts problem resident on the GPU (prepacked weights)."""

    def __init__(self, c):
        import weight_only_quantized_amd as w4
        from gpu_helpers import to_dev
        self.c = c
        self.x = to_dev(c.x)
        self.ids = _i32(c.topk_ids)
        self.w = torch.from_numpy(np.ascontiguousarray(c.topk_w, np.float32)).to(DEV)

        def pack(wplain, K, N):
            w = to_dev(wplain.reshape(-1))
            out = torch.empty(w4.w4a16_prepacked_bytes(c.E, K, N), dtype=torch.uint8, device=DEV)
            w4.w4a16_prepack(w, out, c.E, K, N, int(c.signed))
            return out
        self.w13 = pack(c.w13, c.H, 2 * c.I)
        self.w2 = pack(c.w2, c.I, c.H)
        self.s13, self.s2 = to_dev(c.s13), to_dev(c.s2)
        self.z13 = to_dev(c.z13) if c.z13 is not None else None
        self.z2 = to_dev(c.z2) if c.z2 is not None else None
        self.nbytes = w4.w4a16_fused_moe_workspace_bytes(c.T, c.topk, c.E, c.H, c.I)
        self.ws = torch.empty(self.nbytes, dtype=torch.uint8, device=DEV)

    def run(self):
        import weight_only_quantized_amd as w4
        c = self.c
        out = torch.empty((c.T, c.H), dtype=torch.int16, device=DEV)
        w4.w4a16_fused_moe(self.x, self.ids, self.w, self.w13, self.s13, self.z13, self.w2, self.s2, self.z2,
                           out, c.T, c.topk, c.E, c.H, c.I, 128, c.dtype, self.ws, self.nbytes)
        return out


CHAINS = [
    dict(T=1, topk=1, E=1, H=128, I=128, dtype=synth.BF16, signed=True),
    dict(T=16, topk=2, E=4, H=256, I=128, dtype=synth.BF16, signed=True),
    dict(T=40, topk=3, E=6, H=384, I=256, dtype=synth.F16, signed=False),
    dict(T=33, topk=4, E=5, H=256, I=384, dtype=synth.BF16, signed=True, invalid=True),
    dict(T=200, topk=8, E=64, H=512, I=256, dtype=synth.BF16, signed=True),
]


@pytest.mark.parametrize("cfg", range(len(CHAINS)))
def test_fused_moe_small(orc, cfg):
    from gpu_helpers import check_tol, to_host_u16
    k = dict(CHAINS[cfg])
    invalid = k.pop("invalid", False)
    ids = _routing(k["T"], k["topk"], k["E"], True, seed=cfg) if invalid else None
    c = synth.make_moe_chain(seed=cfg, ids=ids, **k)
    print(f"[case] fused_moe cfg={cfg} {CHAINS[cfg]}", flush=True)
    out = DevChain(c).run()
    torch.cuda.synchronize()
    check_tol(to_host_u16(out), orc.fused_moe(c), c.dtype, label=f"fused_moe_cfg{cfg}")


def test_fused_moe_full(orc):
    """The chain at the sizes the benchmark times (512 tokens, top-8 of 64
    experts, H=2048, I=1408, the same seeded inputs), every token compared
    against the oracle's steps composed over all routed rows."""
    from gpu_helpers import check_tol, to_host_u16
    c = synth.moe_chain()
    print("[case] fused_moe full T=512 topk=8 E=64 H=2048 I=1408", flush=True)
    out = to_host_u16(DevChain(c).run())
    torch.cuda.synchronize()
    check_tol(out, orc.fused_moe_steps(c), c.dtype, label="fused_moe_full all tokens")


@pytest.mark.parametrize("cfg", [0, 2])
def test_silu_epilogue_equals_separate_kernel(cfg):
    """The gate/up projection with SiLU-and-multiply in its epilogue (tile
    configurations 0 and 2: a gate and an up tile per wave) against the same
    chain through the stored projection and the separate kernel
    (configuration 4, one column tile per wave): bit for bit, since both round
    the projection to the dtype before the same fp32 SiLU and product, and with
    half items off every tile configuration accumulates each output in the same
    order."""
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_host_u16
    k = dict(CHAINS[4])
    c = synth.make_moe_chain(seed=9, **k)
    print(f"[case] silu epilogue cfg={cfg} vs separate kernel {CHAINS[4]}", flush=True)
    d = DevChain(c)
    prev = w4.w4a16_test_tile_halves(0)
    try:
        w4.w4a16_test_tile_config(cfg)
        fused = to_host_u16(d.run())
        w4.w4a16_test_tile_config(4)
        separate = to_host_u16(d.run())
    finally:
        w4.w4a16_test_tile_config(-1)
        w4.w4a16_test_tile_halves(prev)
    assert np.array_equal(fused, separate)


@pytest.mark.parametrize("halves", [0, 1])
def test_fused_moe_full_half_items(orc, halves):
    """The benchmark-size chain with half items on and off: both within the
    bar against the oracle's steps (the gate/up projection's plan splits some
    items' K range between two wave pairs when they are on)."""
    import weight_only_quantized_amd as w4
    from gpu_helpers import check_tol, to_host_u16
    c = synth.moe_chain()
    print(f"[case] fused_moe full halves={halves}", flush=True)
    prev = w4.w4a16_test_tile_halves(halves)
    try:
        out = to_host_u16(DevChain(c).run())
        torch.cuda.synchronize()
    finally:
        w4.w4a16_test_tile_halves(prev)
    check_tol(out, orc.fused_moe_steps(c), c.dtype, label=f"fused_moe_full halves={halves}")
