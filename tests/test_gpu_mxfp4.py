"""W4A8-MXFP4 (MXFP4 weights x MXFP8 activations) through the C ABI against the
oracle.

* MXFP8 quantization: codes and scales bit for bit (the decision is taken in
  fp32 on both sides, and every step of it is exact there).
* Weight prepack: bytes equal the layout the header documents.
* Products: with one nonzero weight per column the product is a single exact
  term, so the GEMM output must equal the oracle bit for bit; that exposes the
  activation quantization done inside the fused decode kernel.  General
  products: both sides multiply the same quantized operands exactly, so the
  only difference is fp32 accumulation and the final rounding:
  |y - y64| <= eps16 |y64| + (K + 16) 2^-24 sum_k |a b|, with sum |a b| from
  the oracle on the operands' magnitudes; plus the float acceptance bar.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


class DevMx:
    def __init__(self, p):
        import weight_only_quantized_amd as w4
        from gpu_helpers import to_dev
        self.p = p
        self.x = to_dev(p.x) if p.M else torch.empty((0, p.K), dtype=torch.int16, device=DEV)
        self.wp = torch.empty(w4.w4a8_mxfp4_prepacked_bytes(1, p.K, p.N), dtype=torch.uint8, device=DEV)
        w4.w4a8_mxfp4_prepack(_u8(p.w), _u8(p.sw), self.wp, 1, p.K, p.N)

    def gemm(self):
        import weight_only_quantized_amd as w4
        p = self.p
        y = torch.empty((p.M, p.N), dtype=torch.int16, device=DEV)
        nb = w4.w4a8_mxfp4_workspace_bytes(p.M, p.K)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
        w4.w4a8_mxfp4_gemm(self.x, self.wp, y, p.M, p.K, p.N, p.dtype, ws, nb)
        return y

    def gemm_prequant(self, qx, sx):
        import weight_only_quantized_amd as w4
        p = self.p
        y = torch.empty((p.M, p.N), dtype=torch.int16, device=DEV)
        w4.w4a8_mxfp4_gemm_prequant(_u8(qx), _u8(sx), self.wp, y, p.M, p.K, p.N, p.dtype)
        return y


def _x_mix(M, K, dtype, seed):
    """Activations with blocks of very different magnitude: all-zero blocks,
    blocks that saturate (max/2^e in (448, 512)), tiny values, outliers."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * np.exp2(rng.integers(-8, 9, (M, K // 32))).repeat(32, axis=1)
    x[:, :32] = 0.0                                            # zero block
    if K >= 96:
        x[:, 64:96] *= 1e-3                                    # small block
        x[:, 70] = 500.0 if dtype == synth.F16 else 1e4        # outlier in it
    if K >= 128:
        x[:, 96:128] = np.linspace(-1, 1, 32)
        x[:, 100] = 1.9375                                     # max/2^e = 496 -> saturates to 448
    hi = 60000.0 if dtype == synth.F16 else 1e30
    return synth.to_bits(np.clip(x, -hi, hi).astype(np.float32), dtype)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
@pytest.mark.parametrize("M,K", [(1, 128), (5, 256), (37, 4096), (300, 1024), (2, 8192)])
def test_quantize_bit_exact(orc, dtype, M, K):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_dev
    print(f"[case] mxfp8_quantize dtype={dtype} M={M} K={K}", flush=True)
    x = _x_mix(M, K, dtype, seed=M + K)
    qref, sref = orc.mxfp8_quantize(x, M, K, dtype)
    qx = torch.full((M, K), 0x55, dtype=torch.uint8, device=DEV)
    sx = torch.full((M, K // 32), 0x55, dtype=torch.uint8, device=DEV)
    w4.w4a8_mxfp8_quantize(to_dev(x), qx, sx, M, K, dtype)
    torch.cuda.synchronize()
    q, s = qx.cpu().numpy(), sx.cpu().numpy()
    assert np.array_equal(s, sref), np.argwhere(s != sref)[:5]
    bad = np.argwhere(q != qref)
    assert bad.size == 0, [(tuple(b), q[tuple(b)], qref[tuple(b)]) for b in bad[:5]]


def _documented_layout(w, sw, K, N):
    """The packed bytes as the header describes them (1088-byte tiles ordered
    (16-column block, 128-row group); slot L: column 16nb + L%16, rows
    128g + 32(L/16) + r as nibble r; byte 1024 + L its scale)."""
    codes = synth.unpack_nibbles(w)                            # [K][N]
    G, NB = K // 128, N // 16
    out = np.zeros((NB, G, 1088), np.uint8)
    for nb in range(NB):
        for g in range(G):
            for L in range(64):
                col, k0 = 16 * nb + L % 16, 128 * g + 32 * (L // 16)
                nib = codes[k0:k0 + 32, col]
                out[nb, g, 16 * L:16 * L + 16] = nib[0::2] | (nib[1::2] << 4)
                out[nb, g, 1024 + L] = sw[4 * g + L // 16, col]
    return out.reshape(-1)


@pytest.mark.parametrize("K,N", [(128, 64), (384, 192)])
def test_prepack_layout(K, N):
    p = synth.make_mx(1, K, N, seed=K + N)
    d = DevMx(p)
    torch.cuda.synchronize()
    assert np.array_equal(d.wp.cpu().numpy(), _documented_layout(p.w, p.sw, K, N))


def _one_per_column(p, seed):
    """Each column n has a single nonzero weight, at row perm[n] (K == N), of
    value +-1 or +-0.5 times its scale."""
    rng = np.random.default_rng(seed)
    codes = np.zeros((p.K, p.N), np.uint8)
    perm = rng.permutation(p.K)[:p.N]
    codes[perm, np.arange(p.N)] = rng.choice([0x2, 0xA, 0x1, 0x9], size=p.N)
    p.w = synth.pack_nibbles(codes)
    return p


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
@pytest.mark.parametrize("M,K", [(1, 512), (16, 512), (7, 1024), (16, 8192), (40, 256)])
def test_single_term_products_bit_exact(orc, dtype, M, K):
    """One nonzero weight per column: y[m][n] = a[m][k] * b[k][n] exactly, so the
    16-bit outputs must match bit for bit, including the quantization the fused
    kernel does in registers (M <= 16) or the separate kernel (M > 16)."""
    print(f"[case] mx single-term dtype={dtype} M={M} K={K}", flush=True)
    p = synth.make_mx(M, K, K, dtype, seed=K + M, scale_exp=(-3, 3))
    p.x = _x_mix(M, K, dtype, seed=M * 7 + K)
    p = _one_per_column(p, seed=M + K)
    from gpu_helpers import to_host_u16
    got = to_host_u16(DevMx(p).gemm())
    qx, sx = orc.mxfp8_quantize(p.x, M, K, dtype)
    _, ref = orc.w4a8_mxfp4(qx, sx, p.w, p.sw, M, K, K, dtype)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, [(tuple(b), got[tuple(b)], ref[tuple(b)]) for b in bad[:5]]


def _check_bound(orc, got_bits, qx, sx, p, label):
    from gpu_helpers import check_tol
    M, K, N, dt = p.M, p.K, p.N, p.dtype
    y64, ref = orc.w4a8_mxfp4(qx, sx, p.w, p.sw, M, K, N, dt)
    # sum_k |a b|: the same product on the operands' magnitudes (sign bits cleared)
    mag, _ = orc.w4a8_mxfp4(qx & 0x7F, sx, p.w & 0x77, p.sw, M, K, N, dt)
    got = synth.bits_to_f32(got_bits, dt).astype(np.float64)
    eps16 = 2.0 ** -8 if dt == synth.BF16 else 2.0 ** -11
    tiny = 2.0 ** -133 if dt == synth.BF16 else 2.0 ** -24
    bound = eps16 * np.abs(y64) + (K + 16) * 2.0 ** -24 * mag + tiny
    err = np.abs(got - y64)
    print(f"[parity] {label} max err/bound={np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound), (label, np.unravel_index(np.argmax(err / bound), err.shape))
    check_tol(got_bits, ref, dt, label=label)


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
@pytest.mark.parametrize("M,K,N", [(1, 128, 64), (3, 384, 192), (16, 1024, 320), (9, 4096, 256),
                                   (16, 8192, 128), (17, 256, 64), (33, 1024, 192), (48, 4096, 128),
                                   (49, 512, 64), (100, 2048, 512)])
def test_gemm(orc, dtype, M, K, N):
    print(f"[case] mx gemm dtype={dtype} M={M} K={K} N={N}", flush=True)
    from gpu_helpers import to_host_u16
    p = synth.make_mx(M, K, N, dtype, seed=M + K + N, outlier_frac=0.01)
    got = to_host_u16(DevMx(p).gemm())
    qx, sx = orc.mxfp8_quantize(p.x, M, K, dtype)
    _check_bound(orc, got, qx, sx, p, f"mx_gemm_{M}x{K}x{N}")


@pytest.mark.parametrize("M", [1, 16, 33, 60])
def test_gemm_prequant(orc, M):
    from gpu_helpers import to_host_u16
    p = synth.make_mx(M, 1024, 256, synth.BF16, seed=M)
    qx, sx = orc.mxfp8_quantize(p.x, M, p.K, p.dtype)
    got = to_host_u16(DevMx(p).gemm_prequant(qx, sx))
    _check_bound(orc, got, qx, sx, p, f"mx_prequant_m{M}")


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
@pytest.mark.parametrize("M,K,N", [(300, 2048, 512), (1000, 1024, 1088), (129, 16384, 192)])
def test_gemm_tile(orc, dtype, M, K, N):
    """The tile kernel: several row and column tiles with ragged tails, and a K
    beyond the split-K kernel's reach."""
    print(f"[case] mx tile dtype={dtype} M={M} K={K} N={N}", flush=True)
    from gpu_helpers import to_host_u16
    p = synth.make_mx(M, K, N, dtype, seed=M + K + N, outlier_frac=0.01)
    got = to_host_u16(DevMx(p).gemm())
    qx, sx = orc.mxfp8_quantize(p.x, M, K, dtype)
    _check_bound(orc, got, qx, sx, p, f"mx_tile_{M}x{K}x{N}")


@pytest.mark.parametrize("M", [1, 5, 16])
def test_tile_forced_small_m(orc, M):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_host_u16
    p = synth.make_mx(M, 1024, 320, synth.BF16, seed=40 + M)
    d = DevMx(p)
    old = w4.w4a16_test_force_variant(2)
    try:
        print(f"[case] mx tile forced M={M}", flush=True)
        got = to_host_u16(d.gemm())
    finally:
        w4.w4a16_test_force_variant(old)
    qx, sx = orc.mxfp8_quantize(p.x, M, p.K, p.dtype)
    _check_bound(orc, got, qx, sx, p, f"mx_tile_forced_m{M}")


def test_tile_configs(orc):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_host_u16
    p = synth.make_mx(200, 1024, 576, synth.F16, seed=8)
    d = DevMx(p)
    qx, sx = orc.mxfp8_quantize(p.x, p.M, p.K, p.dtype)
    n = w4.w4a16_test_mx_tile_config(-1)
    try:
        for c in range(n):
            w4.w4a16_test_mx_tile_config(c)
            print(f"[case] mx tile config {c}", flush=True)
            _check_bound(orc, to_host_u16(d.gemm()), qx, sx, p, f"mx_tile_cfg{c}")
    finally:
        w4.w4a16_test_mx_tile_config(-1)


def test_small_configs(orc):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_host_u16
    p = synth.make_mx(5, 2048, 512, synth.BF16, seed=3)
    d = DevMx(p)
    qx, sx = orc.mxfp8_quantize(p.x, p.M, p.K, p.dtype)
    n = w4.w4a16_test_mx_small_config(-1)
    try:
        for c in range(n):
            w4.w4a16_test_mx_small_config(c)
            print(f"[case] mx small config {c}", flush=True)
            _check_bound(orc, to_host_u16(d.gemm()), qx, sx, p, f"mx_cfg{c}")
    finally:
        w4.w4a16_test_mx_small_config(-1)


def test_empty_and_errors():
    import weight_only_quantized_amd as w4
    p = synth.make_mx(0, 256, 64, synth.BF16)
    d = DevMx(p)
    y = torch.empty((0, 64), dtype=torch.int16, device=DEV)
    w4.w4a8_mxfp4_gemm(d.x, d.wp, y, 0, 256, 64, synth.BF16, None, 0)      # M == 0: no-op
    x = torch.zeros((49, 256), dtype=torch.int16, device=DEV)
    y = torch.empty((49, 64), dtype=torch.int16, device=DEV)
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a8_mxfp4_gemm(x, d.wp, y, 49, 256, 64, synth.BF16, None, 0)     # M > 48 needs a workspace
    assert e.value.status == 5


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_full_size(orc, M):
    """The decode shape the benchmark times (K = 4096, N = 14336, bf16 x
    quantized inside the GEMM, the same seeded inputs), every output
    compared."""
    from gpu_helpers import to_host_u16
    print(f"[case] mx decode full M={M}", flush=True)
    p = synth.mx_decode(M)
    got = to_host_u16(DevMx(p).gemm())
    qx, sx = orc.mxfp8_quantize(p.x, M, p.K, p.dtype)
    _check_bound(orc, got, qx, sx, p, f"mx_decode_full_m{M}")


def test_prefill_full_size(orc):
    """The prefill shape the benchmark times (M = N = K = 4096, bf16 x
    quantized into the workspace, then the tile kernel; the same seeded
    inputs), every output compared."""
    from gpu_helpers import to_host_u16
    print("[case] mx prefill full 4096^3", flush=True)
    p = synth.make_mx(4096, 4096, 4096, synth.BF16, name="mx_prefill")
    got = to_host_u16(DevMx(p).gemm())
    qx, sx = orc.mxfp8_quantize(p.x, p.M, p.K, p.dtype)
    _check_bound(orc, got, qx, sx, p, "mx_prefill_full")


class DevMxGrouped:
    def __init__(self, p):
        import weight_only_quantized_amd as w4
        from gpu_helpers import to_dev
        self.p = p
        self.x = to_dev(p.x) if p.R else torch.zeros((1, p.K), dtype=torch.int16, device=DEV)
        self.off = torch.from_numpy(np.ascontiguousarray(p.offsets, np.int32)).to(DEV)
        self.wp = torch.empty(w4.w4a8_mxfp4_prepacked_bytes(p.E, p.K, p.N), dtype=torch.uint8, device=DEV)
        w4.w4a8_mxfp4_prepack(_u8(p.w.reshape(-1)), _u8(p.sw.reshape(-1)), self.wp, p.E, p.K, p.N)
        self.nb = w4.w4a8_mxfp4_grouped_workspace_bytes(p.R, p.K)
        self.ws = torch.empty(max(self.nb, 16), dtype=torch.uint8, device=DEV)

    def run(self):
        import weight_only_quantized_amd as w4
        p = self.p
        y = torch.full((max(p.R, 1), p.N), 0x1234, dtype=torch.int16, device=DEV)
        w4.w4a8_mxfp4_grouped_gemm(self.x, self.off, self.wp, y, p.E, p.R, p.K, p.N, p.dtype, self.ws, self.nb)
        return y


def _check_grouped(orc, got, p, label, experts=None):
    qx, sx = orc.mxfp8_quantize(p.x, p.R, p.K, p.dtype)
    for e in (range(p.E) if experts is None else experts):
        r0, r1 = int(p.offsets[e]), int(p.offsets[e + 1])
        if r1 == r0:
            continue
        sub = synth.MxProblem(x=p.x[r0:r1], w=p.w[e], sw=p.sw[e], M=r1 - r0, K=p.K, N=p.N, dtype=p.dtype)
        _check_bound(orc, np.ascontiguousarray(got[r0:r1]), np.ascontiguousarray(qx[r0:r1]),
                     np.ascontiguousarray(sx[r0:r1]), sub, f"{label}_e{e}")


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
@pytest.mark.parametrize("E,tokens,topk,K,N,counts", [
    (4, 40, 2, 256, 128, None),
    (8, 100, 3, 512, 192, None),
    (6, 0, 1, 256, 64, [0, 37, 0, 1, 130, 5]),          # experts without rows, ragged tiles
    (3, 0, 1, 1024, 320, [300, 0, 64]),
])
def test_grouped(orc, dtype, E, tokens, topk, K, N, counts):
    from gpu_helpers import to_host_u16
    print(f"[case] mx grouped E={E} tokens={tokens} K={K} N={N} counts={counts} dtype={dtype}", flush=True)
    p = synth.make_mx_grouped(E, tokens, topk, K, N, dtype, seed=E + K, counts=counts)
    got = to_host_u16(DevMxGrouped(p).run())
    _check_grouped(orc, got, p, f"mx_grouped_E{E}")


def test_grouped_tile_configs(orc):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_host_u16
    p = synth.make_mx_grouped(5, 0, 1, 512, 576, synth.BF16, seed=3, counts=[70, 0, 1, 200, 33])
    d = DevMxGrouped(p)
    n = w4.w4a16_test_mx_tile_config(-1)
    try:
        for c in range(n):
            w4.w4a16_test_mx_tile_config(c)
            print(f"[case] mx grouped config {c}", flush=True)
            _check_grouped(orc, to_host_u16(d.run()), p, f"mx_grouped_cfg{c}")
    finally:
        w4.w4a16_test_mx_tile_config(-1)


def test_grouped_full_size(orc):
    """The MoE grouped shape the benchmark times (64 experts, 4096 routed rows,
    K=2048, N=1408, the same seeded inputs), every expert's rows compared."""
    from gpu_helpers import to_host_u16
    print("[case] mx grouped full", flush=True)
    p = synth.mx_moe()
    got = to_host_u16(DevMxGrouped(p).run())
    assert int(np.count_nonzero(np.diff(p.offsets))) == p.E
    _check_grouped(orc, got, p, "mx_grouped_full")
