"""MSD parity: A_max, the three int8 layers and the per-group int32 products
are bit-exact against the step-by-step oracle (exposed by the test hook from
the production kernels); the fp16 output meets the float tolerance against the
oracle's MSD result (WeightQuantBatchMatmulExperiment operator deep-dive,
§4.1 eqs. 1-11)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _intermediates(p):
    import weight_only_quantized_amd as w4
    from gpu_helpers import Dev, DEV
    d = Dev(p)
    G = p.K // 128
    amax = torch.empty((p.M, G), dtype=torch.float32, device=DEV)
    layers = torch.empty((3, p.M, p.K), dtype=torch.int8, device=DEV)
    yint = torch.empty((G, 3, p.M, p.N), dtype=torch.int32, device=DEV)
    nbytes = w4.w4a16_msd_workspace_bytes(p.M, p.K, p.N)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    w4.w4a16_test_msd_intermediates(d.x, d.wp, p.M, p.K, p.N, amax, layers, yint, ws, nbytes)
    torch.cuda.synchronize()
    return amax.cpu().numpy(), layers.cpu().numpy(), yint.cpu().numpy()


@pytest.mark.parametrize("M,K,N,seed", [(1, 128, 64, 0), (5, 384, 128, 1), (17, 256, 64, 2), (64, 512, 192, 3),
                                        (70, 256, 128, 4), (1, 2176, 128, 5), (1, 3072, 192, 6),
                                        (1, 8192, 12288, 7)])
def test_intermediates_bit_exact(orc, M, K, N, seed):
    print(f"[case] msd intermediates M={M} K={K} N={N}", flush=True)
    p = synth.msd(M=M, K=K, N=N, seed=seed)
    amax, layers, yint = _intermediates(p)
    ra = orc.msd_amax(p.x, M, K)
    rl = orc.msd_layers(p.x, ra, M, K)
    ry = orc.msd_yint(rl, p.w, M, K, N)
    assert np.array_equal(amax.view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(layers, rl)
    assert np.array_equal(yint, ry)


@pytest.mark.parametrize("amax", [1.0, 3.0, 65504.0, 6.103515625e-05, 0.333251953125])
def test_exhaustive_fp16_layers(orc, amax):
    """Every fp16 value |a| <= amax through the GPU decomposition, bit-compared
    with the oracle (groups of 128 whose first element is amax)."""
    print(f"[case] msd sweep amax={amax}", flush=True)
    a = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    a = a[a <= np.float32(amax)]
    a = np.concatenate([a, -a])
    pad = (-a.size) % 127
    vals = np.concatenate([a, np.zeros(pad, np.float32)]).reshape(-1, 127)
    x = np.concatenate([np.full((vals.shape[0], 1), amax, np.float32), vals], axis=1).reshape(-1)
    K = 128 * 64
    rows = (x.size + K - 1) // K
    x = np.concatenate([x, np.zeros(rows * K - x.size, np.float32)]).reshape(rows, K)
    p = synth.make_dense(rows, K, 64, synth.F16, signed=True, seed=0)
    p.x = synth.to_bits(x, synth.F16)
    amx, layers, _ = _intermediates(p)
    ra = orc.msd_amax(p.x, rows, K)
    assert np.array_equal(amx.view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(layers, orc.msd_layers(p.x, ra, rows, K))


def _check_msd(orc, p, label):
    from gpu_helpers import Dev, check_tol, to_host_u16
    print(f"[case] {label} M={p.M} K={p.K} N={p.N}", flush=True)
    d = Dev(p)
    y = d.msd()
    torch.cuda.synchronize()
    _, y_ref = orc.msd(p.x, p.w, p.scale, p.M, p.K, p.N)
    return check_tol(to_host_u16(y), y_ref, synth.F16, label=label)


def test_msd_full(orc):
    _check_msd(orc, synth.msd(), "msd")


def test_msd_page_example(orc):
    _check_msd(orc, synth.msd_page_example(), "msd_page")


@pytest.mark.parametrize("M,K,N", [(1, 128, 64), (3, 1024, 320), (33, 2048, 192), (100, 512, 128),
                                   (1, 2176, 192), (1, 1920, 64)])
def test_msd_shapes(orc, M, K, N):
    _check_msd(orc, synth.msd(M=M, K=K, N=N, seed=M), f"msd_{M}x{K}x{N}")


def test_msd_zero_rows(orc):
    p = synth.msd(M=4, K=512, N=128, seed=9)
    xf = synth.bits_to_f32(p.x, synth.F16)
    xf[1] = 0.0
    xf[2, 128:256] = 0.0
    p.x = synth.to_bits(xf, synth.F16)
    mx, _ = _check_msd(orc, p, "msd_zero_rows")


def test_msd_zero_groups_single_row(orc):
    """One row (the one-launch kernel) with all-zero groups (A_max = 0: zero
    layers and coefficients) next to ordinary ones."""
    p = synth.msd(M=1, K=2048, N=192, seed=11)
    xf = synth.bits_to_f32(p.x, synth.F16)
    xf[0, 0:128] = 0.0
    xf[0, 1024:1280] = 0.0
    p.x = synth.to_bits(xf, synth.F16)
    _check_msd(orc, p, "msd_zero_groups_1row")
    amax, layers, yint = _intermediates(p)
    ra = orc.msd_amax(p.x, 1, p.K)
    rl = orc.msd_layers(p.x, ra, 1, p.K)
    assert np.array_equal(yint, orc.msd_yint(rl, p.w, 1, p.K, p.N))


def test_msd_workspace_errors():
    import weight_only_quantized_amd as w4
    from gpu_helpers import Dev, to_host_u16, DEV
    p = synth.msd(M=4, K=256, N=128)
    d = Dev(p)
    y = d.new_y(fill=0x2222)
    nbytes = w4.w4a16_msd_workspace_bytes(p.M, p.K, p.N)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    with pytest.raises(w4.W4A16Error) as ei:
        w4.w4a16_msd_gemm(d.x, d.wp, d.scale, y, p.M, p.K, p.N, 128, ws, nbytes - 16)
    assert ei.value.status == 5
    torch.cuda.synchronize()
    assert np.all(to_host_u16(y) == 0x2222)


@pytest.mark.parametrize("cfg", range(6))
def test_msd_configs(orc, cfg):
    """Every configuration of the MSD product kernel: bit-exact per-group
    int32 products and the merged output, with ragged row and column tiles."""
    import weight_only_quantized_amd as w4
    count = w4.w4a16_test_msd_config(-1)
    if cfg >= count:
        pytest.skip(f"only {count} MSD configurations")
    M, K, N = 70, 512, 320
    p = synth.msd(M=M, K=K, N=N, seed=20 + cfg)
    w4.w4a16_test_msd_config(cfg)
    try:
        print(f"[case] msd config {cfg} M={M} K={K} N={N}", flush=True)
        amax, layers, yint = _intermediates(p)
        ra = orc.msd_amax(p.x, M, K)
        rl = orc.msd_layers(p.x, ra, M, K)
        assert np.array_equal(yint, orc.msd_yint(rl, p.w, M, K, N))
        _check_msd(orc, p, f"msd_cfg{cfg}")
    finally:
        w4.w4a16_test_msd_config(-1)


@pytest.mark.parametrize("which", ["page", "shape", "msd"])
def test_msd_basic_pipeline(orc, which):
    """The page's basic pipeline (products through memory, separate merge)
    meets the same bar against the oracle as the fused kernel."""
    import weight_only_quantized_amd as w4
    from gpu_helpers import Dev, DEV, check_tol, to_host_u16
    p = {"page": synth.msd_page_example, "shape": lambda: synth.msd(M=33, K=2048, N=192, seed=4),
         "msd": synth.msd}[which]()
    print(f"[case] msd_basic {which} M={p.M} K={p.K} N={p.N}", flush=True)
    d = Dev(p)
    nbytes = w4.w4a16_test_msd_basic_workspace_bytes(p.M, p.K, p.N)
    assert nbytes >= w4.w4a16_msd_workspace_bytes(p.M, p.K, p.N) + 4 * 3 * p.M * p.N * (p.K // 128)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    y = d.new_y()
    w4.w4a16_test_msd_basic(d.x, d.wp, d.scale, y, p.M, p.K, p.N, 128, ws, nbytes)
    torch.cuda.synchronize()
    _, y_ref = orc.msd(p.x, p.w, p.scale, p.M, p.K, p.N)
    check_tol(to_host_u16(y), y_ref, synth.F16, label=f"msd_basic_{which}")
