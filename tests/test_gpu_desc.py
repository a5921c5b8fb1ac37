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
@pytest.mark.parametrize("M", [1, 16, 100])
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


def test_desc_validation():
    import weight_only_quantized_amd as w4
    import ctypes as C
    L = w4.lib()
    F = 1 << 40
    d = w4.WeightDesc(5, 0, 128, F, None, None)
    assert L.w4a16_gemm_desc(F, F, C.byref(d), F, 1, 128, 64, 1, None) == 3     # weight_bits
    d = w4.WeightDesc(4, 1, 128, F, None, None)
    assert L.w4a16_gemm_desc(F, F, C.byref(d), F, 1, 128, 64, 1, None) == 3     # reserved
    d = w4.WeightDesc(8, 0, 128, F, None, F + 2)
    assert L.w4a16_gemm_desc(F, F, C.byref(d), F, 1, 128, 64, 1, None) == 4     # channel_scale alignment
    assert L.w4a16_gemm_desc(F, F, None, F, 1, 128, 64, 1, None) == 1
