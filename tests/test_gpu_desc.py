"""The weight-descriptor entry point (w4a16_gemm_desc): 4- and 8-bit weights,
with and without zero points, with the optional per-column secondary scale,
on both kernel families, against the oracle product scaled per column in
fp64 and rounded once (acceptance bar: max |d| <= 1e-2 max |ref|, relative L1
<= 2e-3).  Without a secondary scale the result is bit-identical to the
dedicated entry points (same kernels)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("signed", [True, False])
@pytest.mark.parametrize("M", [1, 16, 24, 100])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
def test_gemm_desc(orc, bits, signed, M, dtype):
    import weight_only_quantized_amd as w4
    from gpu_helpers import check_tol, to_dev, to_host_u16
    K, N, group = 1024, 320, 256
    print(f"[case] desc bits={bits} signed={signed} M={M} dtype={dtype}", flush=True)
    t = np.random.default_rng(M + bits).uniform(0.25, 4.0, N).astype(np.float32)
    if bits == 4:
        p = synth.make_dense(M, K, N, dtype, signed=signed, seed=M + 1, group=group)
        w = to_dev(p.w.reshape(-1))
        wp = torch.empty(w4.w4a16_prepacked_bytes(1, K, N), dtype=torch.uint8, device=DEV)
        w4.w4a16_prepack(w, wp, 1, K, N, int(signed))
        zero = to_dev(p.zero) if p.zero is not None else None
        y64, _ = orc.w4a16(p.x, p.w, p.scale, p.zero, M, K, N, dtype, group=group)
    else:
        p = synth.make_w8(M, K, N, dtype, signed=signed, seed=M + 1, group=group)
        wp = torch.empty(w4.w8a16_prepacked_bytes(1, K, N), dtype=torch.uint8, device=DEV)
        w4.w8a16_prepack(_u8(p.w), wp, 1, K, N, int(signed))
        zero = _u8(p.zero) if p.zero is not None else None
        y64, _ = orc.w8a16(p.x, p.w, p.scale, p.zero, M, K, N, dtype, group=group)
    x, sc = to_dev(p.x), to_dev(p.scale)
    ts = torch.from_numpy(t).to(DEV)
    y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    w4.w4a16_gemm_desc(x, wp, y, M, K, N, sc, zero, ts, weight_bits=bits, group_size=group, dt=dtype)
    _, ref = orc.channel_scaled(y64, t, dtype)
    check_tol(to_host_u16(y), ref, dtype, label=f"desc_b{bits}_s{int(signed)}_m{M}")
    # without a secondary scale: bit-identical to the dedicated entry point
    y1 = torch.empty((M, N), dtype=torch.int16, device=DEV)
    y2 = torch.empty((M, N), dtype=torch.int16, device=DEV)
    w4.w4a16_gemm_desc(x, wp, y1, M, K, N, sc, zero, None, weight_bits=bits, group_size=group, dt=dtype)
    if bits == 4:
        w4.w4a16_gemm(x, wp, sc, zero, y2, M, K, N, group, dtype)
    else:
        w4.w8a16_gemm(x, wp, sc, zero, y2, M, K, N, group, dtype)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [1, 16, 24, 100])
@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
@pytest.mark.parametrize("with_t", [False, True])
def test_float_zero_points(orc, bits, M, dtype, with_t):
    """Floating-point zero points (values of the activation dtype, arbitrary
    fractions) through the descriptor, with and without a secondary scale."""
    import weight_only_quantized_amd as w4
    from gpu_helpers import check_tol, to_dev, to_host_u16
    K, N, group = 1024, 320, 256
    G = K // group
    rng = np.random.default_rng(M * 10 + bits + int(with_t))
    print(f"[case] float zero bits={bits} M={M} dtype={dtype} t={with_t}", flush=True)
    top = 15.0 if bits == 4 else 255.0
    zf = synth.to_bits((rng.random((G, N)) * top).astype(np.float32), dtype)
    if bits == 4:
        p = synth.make_dense(M, K, N, dtype, signed=False, seed=M + 3, group=group)
        wp = torch.empty(w4.w4a16_prepacked_bytes(1, K, N), dtype=torch.uint8, device=DEV)
        w4.w4a16_prepack(to_dev(p.w.reshape(-1)), wp, 1, K, N, 0)
        y64, _ = orc.w4a16_fzero(p.x, p.w, p.scale, zf, M, K, N, dtype, group=group)
    else:
        p = synth.make_w8(M, K, N, dtype, signed=False, seed=M + 3, group=group)
        wp = torch.empty(w4.w8a16_prepacked_bytes(1, K, N), dtype=torch.uint8, device=DEV)
        w4.w8a16_prepack(_u8(p.w), wp, 1, K, N, 0)
        y64, _ = orc.w8a16_fzero(p.x, p.w, p.scale, zf, M, K, N, dtype, group=group)
    t = rng.uniform(0.25, 4.0, N).astype(np.float32) if with_t else np.ones(N, np.float32)
    ts = torch.from_numpy(t).to(DEV) if with_t else None
    x, sc, zd = to_dev(p.x), to_dev(p.scale), to_dev(zf)
    d = w4.weight_desc(sc, zd, ts, bits, group, zero_format=1)
    nb = w4.w4a16_gemm_desc_workspace_bytes(d, M, K, N)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    w4.w4a16_gemm_desc(x, wp, y, M, K, N, sc, zd, ts, weight_bits=bits, group_size=group, dt=dtype, zero_format=1,
                       workspace=ws, workspace_bytes=nb)
    _, ref = orc.channel_scaled(y64, t, dtype)
    check_tol(to_host_u16(y), ref, dtype, label=f"fzero_b{bits}_m{M}_t{int(with_t)}")


@pytest.mark.parametrize("dtype", [synth.BF16, synth.F16])
def test_float_zero_points_many_groups(orc, dtype):
    """Floating-point zero points over 18 scale groups: the correction kernel
    takes groups eight at a time (two full chunks and a ragged one)."""
    import weight_only_quantized_amd as w4
    from gpu_helpers import check_tol, to_dev, to_host_u16
    M, K, N, group = 3, 2304, 192, 128
    G = K // group
    rng = np.random.default_rng(77)
    print(f"[case] float zero many groups M={M} K={K} N={N} dtype={dtype}", flush=True)
    zf = synth.to_bits((rng.random((G, N)) * 15.0).astype(np.float32), dtype)
    p = synth.make_dense(M, K, N, dtype, signed=False, seed=5, group=group)
    wp = torch.empty(w4.w4a16_prepacked_bytes(1, K, N), dtype=torch.uint8, device=DEV)
    w4.w4a16_prepack(to_dev(p.w.reshape(-1)), wp, 1, K, N, 0)
    y64, ref = orc.w4a16_fzero(p.x, p.w, p.scale, zf, M, K, N, dtype, group=group)
    x, sc, zd = to_dev(p.x), to_dev(p.scale), to_dev(zf)
    d = w4.weight_desc(sc, zd, None, 4, group, zero_format=1)
    nb = w4.w4a16_gemm_desc_workspace_bytes(d, M, K, N)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    w4.w4a16_gemm_desc(x, wp, y, M, K, N, sc, zd, None, weight_bits=4, group_size=group, dt=dtype, zero_format=1,
                       workspace=ws, workspace_bytes=nb)
    check_tol(to_host_u16(y), ref, dtype, label="fzero_many_groups")


@pytest.mark.parametrize("group,signed,M,dtype", [(32, True, 1, synth.BF16), (64, False, 16, synth.F16),
                                                  (32, False, 100, synth.BF16), (64, True, 40, synth.F16)])
def test_gemm_desc_small_scale_groups(orc, group, signed, M, dtype):
    """The descriptor with 32/64-row scale groups (4-bit weights prepacked by
    w4a16_prepack_g) and a per-column secondary scale, both kernel families."""
    import weight_only_quantized_amd as w4
    from gpu_helpers import check_tol, prepack, to_dev, to_host_u16
    K, N = 1024, 320
    print(f"[case] desc group={group} signed={signed} M={M} dtype={dtype}", flush=True)
    t = np.random.default_rng(M + group).uniform(0.25, 4.0, N).astype(np.float32)
    p = synth.make_dense(M, K, N, dtype, signed=signed, seed=M + group, group=group)
    wp = prepack(p)
    zero = to_dev(p.zero) if p.zero is not None else None
    y64, _ = orc.w4a16(p.x, p.w, p.scale, p.zero, M, K, N, dtype, group=group)
    y = torch.empty((M, N), dtype=torch.int16, device=DEV)
    w4.w4a16_gemm_desc(to_dev(p.x), wp, y, M, K, N, to_dev(p.scale), zero, torch.from_numpy(t).to(DEV),
                       weight_bits=4, group_size=group, dt=dtype)
    _, ref = orc.channel_scaled(y64, t, dtype)
    check_tol(to_host_u16(y), ref, dtype, label=f"desc_group{group}_m{M}")
