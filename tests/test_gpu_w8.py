"""W8A16 (8-bit integer weights, 16-bit activations) through the C ABI against
the oracle.  Prepack bytes bit for bit against the documented layout; products
with the float acceptance bar (max |d| <= 1e-2 max |ref|, relative L1 <= 2e-3)
and, tighter, within eps16 |y| + (K + 64) 2^-23 sum_k |x| (u + z) s: every
product of a 16-bit activation and an 8-bit code is exact in fp32, so only the
fp32 sums (including the row-sum correction of the bf16 path, whose terms are
u and z rather than u - z) and the final rounding can differ."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


class DevW8:
    def __init__(self, p):
        import weight_only_quantized_amd as w4
        from gpu_helpers import to_dev
        self.p = p
        self.x = to_dev(p.x)
        self.scale = to_dev(p.scale)
        self.zero = _u8(p.zero) if p.zero is not None else None
        self.wp = torch.empty(w4.w8a16_prepacked_bytes(1, p.K, p.N), dtype=torch.uint8, device=DEV)
        w4.w8a16_prepack(_u8(p.w), self.wp, 1, p.K, p.N, int(p.zero is None))

    def gemm(self):
        import weight_only_quantized_amd as w4
        p = self.p
        y = torch.empty((p.M, p.N), dtype=torch.int16, device=DEV)
        w4.w8a16_gemm(self.x, self.wp, self.scale, self.zero, y, p.M, p.K, p.N, p.group, p.dtype)
        return y


def _check(orc, got, p, label, cols=None):
    from gpu_helpers import check_tol
    w, s, z = p.w, p.scale, p.zero
    if cols is not None:
        w, s = w[:, cols], s[:, cols]
        z = None if z is None else z[:, cols]
    N = w.shape[1]
    y64, ref = orc.w8a16(p.x, w, s, z, p.M, p.K, N, p.dtype, group=p.group)
    xa = np.abs(synth.bits_to_f32(p.x, p.dtype).astype(np.float64))
    u = (w.astype(np.int8).astype(np.float64) + 128.0) if z is None else w.astype(np.float64)
    zz = np.full((p.K // p.group, N), 128.0) if z is None else z.astype(np.float64)
    sv = np.abs(synth.bits_to_f32(s, p.dtype).astype(np.float64))
    wmag = (u + np.repeat(zz, p.group, axis=0)) * np.repeat(sv, p.group, axis=0)
    mag = xa @ wmag
    eps16 = 2.0 ** -8 if p.dtype == synth.BF16 else 2.0 ** -11
    bound = eps16 * np.abs(y64) + (p.K + 64) * 2.0 ** -23 * mag + 2.0 ** -24
    err = np.abs(synth.bits_to_f32(got, p.dtype).astype(np.float64) - y64)
    print(f"[parity] {label} max err/bound={np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound), (label, np.unravel_index(np.argmax(err / bound), err.shape))
    check_tol(got, ref, p.dtype, label=label)


def _documented_layout(w, K, N, signed):
    G, NB = K // 128, N // 16
    codes = (w ^ 0x80) if signed else w
    out = np.zeros((NB, G, 2048), np.uint8)
    for nb in range(NB):
        for g in range(G):
            for L in range(64):
                col, k0 = 16 * nb + L % 16, 128 * g + 32 * (L // 16)
                out[nb, g, 32 * L:32 * L + 32] = codes[k0:k0 + 32, col]
    return out.reshape(-1)


@pytest.mark.parametrize("signed", [True, False])
def test_prepack_layout(signed):
    p = synth.make_w8(1, 256, 128, signed=signed, seed=3)
    d = DevW8(p)
    torch.cuda.synchronize()
    assert np.array_equal(d.wp.cpu().numpy(), _documented_layout(p.w, p.K, p.N, signed))


CASES = [(1, 4096, 256), (5, 384, 192), (16, 8192, 128), (3, 128, 64),
         (17, 256, 64), (40, 1024, 320), (48, 4096, 128), (49, 512, 128), (100, 2048, 576), (300, 1024, 1088)]


@pytest.mark.parametrize("signed", [True, False])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
@pytest.mark.parametrize("M,K,N", CASES)
def test_gemm(orc, M, K, N, dtype, signed):
    from gpu_helpers import to_host_u16
    print(f"[case] w8 gemm M={M} K={K} N={N} dtype={dtype} signed={signed}", flush=True)
    p = synth.make_w8(M, K, N, dtype, signed=signed, seed=M + K + N)
    got = to_host_u16(DevW8(p).gemm())
    _check(orc, got, p, f"w8_{M}x{K}x{N}_{dtype}_{int(signed)}")


@pytest.mark.parametrize("group", [256, 1024, 4096])
@pytest.mark.parametrize("M", [4, 70])
def test_group_sizes(orc, group, M):
    from gpu_helpers import to_host_u16
    print(f"[case] w8 group={group} M={M}", flush=True)
    p = synth.make_w8(M, 4096, 192, synth.BF16, signed=False, seed=group + M, group=group)
    got = to_host_u16(DevW8(p).gemm())
    _check(orc, got, p, f"w8_group{group}_m{M}")


def test_all_variants(orc):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_host_u16
    counts = w4.w4a16_test_w8_config(-1, -1)
    n_small, n_tile = counts // 100, counts % 100
    try:
        for dtype in (synth.BF16, synth.F16):
            ps = synth.make_w8(7, 1024, 256, dtype, signed=False, seed=11)
            pt = synth.make_w8(90, 1024, 512, dtype, signed=True, seed=12)
            ds, dtl = DevW8(ps), DevW8(pt)
            for c in range(n_small):
                w4.w4a16_test_w8_config(c, -1)
                print(f"[case] w8 small config {c} dtype={dtype}", flush=True)
                _check(orc, to_host_u16(ds.gemm()), ps, f"w8_small_cfg{c}_{dtype}")
            for c in range(n_tile):
                w4.w4a16_test_w8_config(-1, c)
                print(f"[case] w8 tile config {c} dtype={dtype}", flush=True)
                _check(orc, to_host_u16(dtl.gemm()), pt, f"w8_tile_cfg{c}_{dtype}")
    finally:
        w4.w4a16_test_w8_config(-1, -1)


@pytest.mark.parametrize("M", [1, 16])
def test_tile_forced_small_m(orc, M):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_host_u16
    p = synth.make_w8(M, 512, 320, synth.F16, signed=False, seed=50 + M)
    d = DevW8(p)
    old = w4.w4a16_test_force_variant(2)
    try:
        print(f"[case] w8 tile forced M={M}", flush=True)
        got = to_host_u16(d.gemm())
    finally:
        w4.w4a16_test_force_variant(old)
    _check(orc, got, p, f"w8_forced_m{M}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_full_size(orc, M):
    """The decode shape the benchmark times (K = 4096, N = 14336, bf16, uint8
    weights with uint8 zero points, the same seeded inputs), every output
    compared."""
    from gpu_helpers import to_host_u16
    print(f"[case] w8 decode full M={M}", flush=True)
    p = synth.make_w8(M, 4096, 14336, synth.BF16, signed=False, seed=0)
    got = to_host_u16(DevW8(p).gemm())
    _check(orc, got, p, f"w8_decode_full_m{M}")


def test_prefill_full_size(orc):
    """The prefill shape the benchmark times (M = N = K = 4096, bf16, int8
    weights, the same seeded inputs), every output compared."""
    from gpu_helpers import to_host_u16
    print("[case] w8 prefill full 4096^3 int8", flush=True)
    p = synth.make_w8(4096, 4096, 4096, synth.BF16, signed=True, seed=0)
    got = to_host_u16(DevW8(p).gemm())
    _check(orc, got, p, "w8_prefill_full")
