"""GPU prepack / unpack are bit-exact against the oracle's layout reference."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("E,K,N,signed", [
    (1, 128, 64, True), (1, 256, 64, False), (3, 384, 192, True), (2, 1024, 1408, False), (1, 4096, 320, True),
])
def test_prepack_bit_exact_and_round_trip(orc, E, K, N, signed):
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_dev, DEV
    print(f"[case] prepack E={E} K={K} N={N} signed={signed}", flush=True)
    rng = np.random.default_rng(E * 1000 + K + N)
    w = rng.integers(0, 256, size=(E, K, N // 2), dtype=np.uint8)
    wd = to_dev(w.reshape(-1))
    packed = torch.empty(E * K * N // 2, dtype=torch.uint8, device=DEV)
    w4.w4a16_prepack(wd, packed, E, K, N, int(signed))
    back = torch.zeros_like(wd)
    w4.w4a16_test_unpack(packed, back, E, K, N, int(signed))
    torch.cuda.synchronize()
    ref = orc.prepack(w.reshape(-1), E, K, N, signed)
    assert np.array_equal(packed.cpu().numpy(), ref)
    assert np.array_equal(back.cpu().numpy(), w.reshape(-1))


@pytest.mark.parametrize("name", ["decode", "moe", "msd"])
def test_prepack_full_size(orc, name):
    from gpu_helpers import prepack
    print(f"[case] prepack full {name}", flush=True)
    p = {"decode": lambda: synth.decode(1), "moe": synth.moe, "msd": synth.msd}[name]()
    got = prepack(p).cpu().numpy()
    ref = orc.prepack(p.w.reshape(-1), p.E, p.K, p.N, p.signed)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("E,K,N,signed,group", [(1, 128, 64, True, 32), (2, 384, 192, False, 64),
                                                (3, 256, 128, True, 64), (1, 4096, 14336, False, 32)])
def test_prepack_group_aligned_bytes(orc, E, K, N, signed, group):
    """w4a16_prepack_g with 32/64-row groups writes the group-aligned layout:
    bytes equal to the oracle's statement of it; with a 128-multiple group
    it writes the standard layout."""
    import weight_only_quantized_amd as w4
    from gpu_helpers import to_dev
    print(f"[case] prepack_g E={E} K={K} N={N} signed={signed} group={group}", flush=True)
    rng = np.random.default_rng(K + N + group)
    w = rng.integers(0, 256, size=(E, K, N // 2), dtype=np.uint8)
    out = torch.empty(E * K * N // 2, dtype=torch.uint8, device="cuda:0")
    w4.w4a16_prepack_g(to_dev(w.reshape(-1)), out, E, K, N, int(signed), group)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), orc.prepack(w, E, K, N, signed, layout=1))
    w4.w4a16_prepack_g(to_dev(w.reshape(-1)), out, E, K, N, int(signed), 128)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), orc.prepack(w, E, K, N, signed, layout=0))
