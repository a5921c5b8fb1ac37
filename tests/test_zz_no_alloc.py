"""w4a16_msd_gemm_noalloc (the MSD call whose workspace is the library's
static per-device scratch) against w4a16_msd_gemm with a caller workspace:
both run the same kernels on the same plan, so the outputs must be equal bit
for bit (a stricter bar than the float acceptance bar, which is also checked
against the oracle).  Two calls in a row, the second with a smaller input,
so the second reuses the scratch the first left behind; then a problem too
large for the scratch is rejected on the host."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _run_both(p):
    import weight_only_quantized_amd as w4
    from gpu_helpers import Dev, to_host_u16
    d = Dev(p)
    ref = d.msd()
    y = torch.full((p.M, p.N), 0x7BFF, dtype=torch.int16, device="cuda:0")
    w4.w4a16_msd_gemm_noalloc(d.x, d.wp, d.scale, y, p.M, p.K, p.N, 128)
    torch.cuda.synchronize()
    return to_host_u16(y), to_host_u16(ref)


@pytest.mark.parametrize("first,second", [((64, 8192, 8192), (5, 1024, 640)),
                                          ((37, 2048, 1024), (1, 8192, 12288))])
def test_noalloc_equals_workspace_call(orc, first, second):
    from gpu_helpers import check_tol
    for M, K, N in (first, second):
        print(f"[case] msd noalloc M={M} K={K} N={N}", flush=True)
        p = synth.msd(M=M, K=K, N=N, seed=M + K)
        got, ref = _run_both(p)
        assert np.array_equal(got, ref), np.argwhere(got != ref)[:5]
        _, y_ref = orc.msd(p.x, p.w, p.scale, p.M, p.K, p.N)
        check_tol(got, y_ref, synth.F16, label=f"msd_noalloc_{M}x{K}x{N}")


def test_noalloc_too_large_rejected():
    import weight_only_quantized_amd as w4
    M, K, N = 4096, 8192, 8192
    x = torch.zeros((M, K), dtype=torch.int16, device="cuda:0")
    wp = torch.zeros(K * N // 2, dtype=torch.uint8, device="cuda:0")
    sc = torch.zeros((K // 128, N), dtype=torch.int16, device="cuda:0")
    y = torch.full((M, N), 0x1234, dtype=torch.int16, device="cuda:0")
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_msd_gemm_noalloc(x, wp, sc, y, M, K, N, 128)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert int((y != 0x1234).sum()) == 0          # nothing was enqueued
