"""The C-ABI library loads and exports every declared entry point; host-side
validation rejects bad arguments before touching the device.  No compute
calls are made here (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

import weight_only_quantized_amd as w4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("w4a16.h", "w4a16_test.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(w[48]a(?:16|8)_[a-z0-9_]+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = w4.lib()
    declared = _declared()
    assert {"w4a16_prepack", "w4a16_gemm", "w4a16_msd_gemm", "w4a16_grouped_gemm",
            "w4a16_msd_workspace_bytes", "w4a16_prepacked_bytes", "w4a16_status_str"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(w4.EXPORTED)


def test_status_strings():
    for s in range(8):
        assert w4.w4a16_status_str(s).startswith(w4.STATUS_NAMES[s])
    assert "UNKNOWN" in w4.w4a16_status_str(99)


def test_size_queries():
    assert w4.w4a16_prepacked_bytes(1, 4096, 14336) == 4096 * 14336 // 2
    assert w4.w4a16_prepacked_bytes(64, 2048, 1408) == 64 * 2048 * 1408 // 2
    assert w4.w4a16_prepacked_bytes(0, 128, 64) == 0
    ws = w4.w4a16_msd_workspace_bytes(64, 8192, 8192)
    # at least A_max/coefficients + three int8 layers
    assert ws >= 3 * 64 * 8192 and ws % 256 == 0
    assert w4.w4a16_msd_workspace_bytes(64, 8192, 8192, 64) == 0     # unsupported group
    assert w4.w4a16_msd_workspace_bytes(0, 8192, 8192) == 0
    assert w4.w4a16_msd_workspace_bytes(1, 100, 8192) == 0            # K % 128 != 0


FAKE = 1 << 40          # never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status", [
    (dict(group_size=48), 3),             # below 128: only 32 and 64
    (dict(group_size=16), 3),
    (dict(group_size=192), 3),            # not a multiple of 128
    (dict(group_size=512), 2),            # does not divide K = 256
    (dict(dt=7), 3),
    (dict(K=100), 2),
    (dict(K=0), 2),
    (dict(N=96), 2),
    (dict(M=-1), 2),
])
def test_gemm_validation(kw, status):
    args = dict(M=4, K=256, N=256, group_size=128, dt=0)
    args.update(kw)
    st = w4.lib().w4a16_gemm(FAKE, FAKE, FAKE, None, FAKE, args["M"], args["K"], args["N"],
                            args["group_size"], args["dt"], None)
    assert st == status


def test_gemm_null_and_align():
    L = w4.lib()
    assert L.w4a16_gemm(None, FAKE, FAKE, None, FAKE, 4, 256, 256, 128, 0, None) == 1
    assert L.w4a16_gemm(FAKE, FAKE, None, None, FAKE, 4, 256, 256, 128, 0, None) == 1
    assert L.w4a16_gemm(FAKE + 8, FAKE, FAKE, None, FAKE, 4, 256, 256, 128, 0, None) == 4
    assert L.w4a16_gemm(FAKE, FAKE + 4, FAKE, None, FAKE, 4, 256, 256, 128, 0, None) == 4
    assert L.w4a16_gemm(FAKE, FAKE, FAKE + 1, None, FAKE, 4, 256, 256, 128, 0, None) == 4


def test_m_zero_is_noop():
    L = w4.lib()
    assert L.w4a16_gemm(None, None, None, None, None, 0, 256, 256, 128, 1, None) == 0
    assert L.w4a16_msd_gemm(None, None, None, None, 0, 256, 256, 128, None, 0, None) == 0
    assert L.w4a16_grouped_gemm(None, None, None, None, None, None, 4, 0, 256, 256, 128, 1, None) == 0


def test_msd_validation():
    L = w4.lib()
    ws = w4.w4a16_msd_workspace_bytes(4, 256, 256)
    assert L.w4a16_msd_gemm(FAKE, FAKE, FAKE, FAKE, 4, 256, 256, 64, FAKE, ws, None) == 3
    assert L.w4a16_msd_gemm(FAKE, FAKE, FAKE, FAKE, 4, 250, 256, 128, FAKE, ws, None) == 2
    assert L.w4a16_msd_gemm(FAKE, FAKE, FAKE, FAKE, 4, 256, 256, 128, None, ws, None) == 5
    assert L.w4a16_msd_gemm(FAKE, FAKE, FAKE, FAKE, 4, 256, 256, 128, FAKE, ws - 1, None) == 5
    assert L.w4a16_msd_gemm(FAKE, FAKE, None, FAKE, 4, 256, 256, 128, FAKE, ws, None) == 1
    assert L.w4a16_msd_gemm(FAKE, FAKE, FAKE, FAKE, 4, 256, 256, 128, FAKE + 8, ws, None) == 4


def test_grouped_and_prepack_validation():
    L = w4.lib()
    assert L.w4a16_grouped_gemm(FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 16, 256, 256, 128, 1, None) == 2
    assert L.w4a16_grouped_gemm(FAKE, None, FAKE, FAKE, None, FAKE, 4, 16, 256, 256, 128, 1, None) == 1
    assert L.w4a16_grouped_gemm(FAKE, FAKE + 2, FAKE, FAKE, None, FAKE, 4, 16, 256, 256, 128, 1, None) == 4
    assert L.w4a16_grouped_gemm(FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 16, 256, 256, 128, 5, None) == 3
    assert L.w4a16_prepack(FAKE, FAKE, 0, 256, 256, 1, None) == 2
    assert L.w4a16_prepack(FAKE, FAKE, 1, 200, 256, 1, None) == 2
    assert L.w4a16_prepack(None, FAKE, 1, 256, 256, 1, None) == 1
    assert L.w4a16_prepack(FAKE + 1, FAKE, 1, 256, 256, 1, None) == 4


def test_binding_raises_on_error():
    with pytest.raises(w4.W4A16Error) as ei:
        w4.w4a16_gemm(FAKE, FAKE, FAKE, None, FAKE, 4, 256, 256, group_size=48, dt=0, stream=0)
    assert ei.value.status == 3


def test_variant_table():
    assert "small" in w4.w4a16_test_variant_name(1, 4096, 14336, 1, 1)
    assert "small" in w4.w4a16_test_variant_name(16, 4096, 14336, 1, 1)
    assert "small" in w4.w4a16_test_variant_name(17, 4096, 4096, 1, 0)      # two 16-row tiles
    assert "small" in w4.w4a16_test_variant_name(32, 4096, 14336, 1, 1)
    assert "tile" in w4.w4a16_test_variant_name(17, 4224, 4096, 1, 0)       # past 32 groups
    assert "small" in w4.w4a16_test_variant_name(64, 4096, 4096, 1, 0)      # two 32-row groups
    assert "tile" in w4.w4a16_test_variant_name(65, 4096, 4096, 1, 0)
    assert "tile" in w4.w4a16_test_variant_name(4096, 4096, 4096, 1, 0)


def test_no_bit_cast_of_vector_subscript():
    """Guard for a compiler issue: __builtin_bit_cast applied directly to a
    vector-subscript expression (v[i]) is lowered as a read of element 0.  The
    kernels must route such elements through a scalar (the `as<T>` helper)."""
    csrc = os.path.join(ROOT, "weight_only_quantized_amd", "csrc")
    bad = []
    for f in os.listdir(csrc):
        if f.endswith((".hip", ".hpp", ".cpp")):
            for i, line in enumerate(open(os.path.join(csrc, f)), 1):
                if re.search(r"__builtin_bit_cast\([^,]+,\s*[^()]*\[[^\]]+\]\s*\)", line):
                    bad.append(f"{f}:{i}: {line.strip()}")
    assert not bad, bad


def test_moe_chain_validation():
    """Host-side argument checks of the fused-experts entry points (no launch)."""
    L = w4.lib()
    # routing: E outside [1, 1024], topk < 1, misaligned or missing buffers
    assert L.w4a16_moe_align(FAKE, 8, 2, 0, FAKE, FAKE, FAKE, None) == 2
    assert L.w4a16_moe_align(FAKE, 8, 2, 1025, FAKE, FAKE, FAKE, None) == 3
    assert L.w4a16_moe_align(FAKE, 8, 0, 4, FAKE, FAKE, FAKE, None) == 2
    assert L.w4a16_moe_align(FAKE, 8, 2, 4, None, FAKE, FAKE, None) == 1
    assert L.w4a16_moe_align(FAKE + 2, 8, 2, 4, FAKE, FAKE, FAKE, None) == 4
    assert L.w4a16_moe_gather(FAKE, FAKE, FAKE, 8, 2, 4, 100, FAKE, 1, None) == 2      # H % 8
    assert L.w4a16_moe_gather(FAKE, FAKE, FAKE, 8, 2, 4, 128, FAKE + 8, 1, None) == 4
    assert L.w4a16_moe_gather(FAKE, FAKE, FAKE, 0, 2, 4, 128, FAKE, 1, None) == 0       # no tokens
    assert L.w4a16_silu_and_mul(FAKE, None, 4, 12, FAKE, 1, None) == 2                 # I % 8
    assert L.w4a16_silu_and_mul(FAKE, None, 4, 16, FAKE, 7, None) == 3
    assert L.w4a16_silu_and_mul(FAKE, FAKE + 2, 4, 16, FAKE, 1, None) == 4
    assert L.w4a16_silu_and_mul(FAKE, None, 0, 16, FAKE, 1, None) == 0
    assert L.w4a16_moe_sum(FAKE, FAKE, FAKE, 4, 2, 20, FAKE, 1, None) == 2             # N % 8
    assert L.w4a16_moe_sum(FAKE, None, FAKE, 4, 2, 16, FAKE, 1, None) == 1
    ws = w4.w4a16_fused_moe_workspace_bytes(16, 2, 4, 256, 128)
    assert ws > 16 * 2 * (2 * 128 + 128 + 256) * 2                                       # h, a, o
    assert w4.w4a16_fused_moe_workspace_bytes(16, 2, 4, 256, 100) == 0
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 16, 2, 4, 256, 128, 128, 1, FAKE, ws, None]
    a = list(args); a[15] = 64
    assert L.w4a16_fused_moe(*a) == 3                                                   # group size
    a = list(args); a[14] = 96
    assert L.w4a16_fused_moe(*a) == 2                                                   # I % 128
    a = list(args); a[5] = FAKE
    assert L.w4a16_fused_moe(*a) == 1                                                   # one zero pointer only
    a = list(args); a[18] = ws - 1
    assert L.w4a16_fused_moe(*a) == 5
    a = list(args); a[17] = FAKE + 8
    assert L.w4a16_fused_moe(*a) == 4


def test_group_sizes_accepted_by_gemm_only():
    """Scale groups that are multiples of 128 dividing K pass validation for the
    dense and grouped GEMMs (they fail later only on the fake pointers'
    alignment), while the MSD path keeps group 128."""
    L = w4.lib()
    for gs in (128, 256, 512, 1024):
        assert L.w4a16_gemm(FAKE, FAKE, FAKE + 1, None, FAKE, 4, 1024, 256, gs, 0, None) == 4
        assert L.w4a16_grouped_gemm(FAKE, FAKE, FAKE, FAKE + 1, None, FAKE, 4, 16, 1024, 256, gs, 1, None) == 4
    ws = w4.w4a16_msd_workspace_bytes(4, 1024, 256)
    assert L.w4a16_msd_gemm(FAKE, FAKE, FAKE, FAKE, 4, 1024, 256, 256, FAKE, ws, None) == 3


def test_mxfp4_sizes_and_validation():
    assert w4.w4a8_mxfp4_prepacked_bytes(1, 4096, 14336) == 32 * 896 * 1088
    assert w4.w4a8_mxfp4_prepacked_bytes(0, 128, 64) == 0
    # the size does not depend on the kernel a call picks (the split-K kernel,
    # M <= 48, uses none of it but may be given it)
    assert w4.w4a8_mxfp4_workspace_bytes(16, 4096) == 16 * 4096 + 16 * 128
    assert w4.w4a8_mxfp4_workspace_bytes(48, 4096) == 48 * 4096 + 48 * 128
    assert w4.w4a8_mxfp4_workspace_bytes(0, 4096) == 0
    assert w4.w4a8_mxfp4_workspace_bytes(16, 16384) >= 16 * 16384     # K beyond the split-K kernel
    ws = w4.w4a8_mxfp4_workspace_bytes(49, 4096)
    assert ws >= 49 * 4096 + 49 * 128 and (49 * 4096 + 255) // 256 * 256 <= ws
    L = w4.lib()
    F = FAKE
    # (call, expected status): shapes, dtype, nulls, alignment, workspace; all
    # rejected on the host before any device call
    cases = [
        (lambda: L.w4a8_mxfp4_gemm(F, F, F, 1, 100, 64, 1, None, 0, None), 2),        # K % 128
        (lambda: L.w4a8_mxfp4_gemm(F, F, F, 1, 128, 32, 1, None, 0, None), 2),        # N % 64
        (lambda: L.w4a8_mxfp4_gemm(F, F, F, 1, 16384, 64, 1, None, 0, None), 5),      # K > 8192: tile kernel
        (lambda: L.w4a8_mxfp4_gemm(F, F, F, 1, 8192, 1 << 20, 1, None, 0, None), 2),  # packed > 2 GiB
        (lambda: L.w4a8_mxfp4_gemm(F, F, F, -1, 128, 64, 1, None, 0, None), 2),
        (lambda: L.w4a8_mxfp4_gemm(F, F, F, 1, 128, 64, 5, None, 0, None), 3),        # dtype
        (lambda: L.w4a8_mxfp4_gemm(None, F, F, 1, 128, 64, 1, None, 0, None), 1),
        (lambda: L.w4a8_mxfp4_gemm(F + 8, F, F, 1, 128, 64, 1, None, 0, None), 4),    # x alignment
        (lambda: L.w4a8_mxfp4_gemm(F, F, F, 49, 128, 64, 1, None, 0, None), 5),       # workspace
        (lambda: L.w4a8_mxfp4_gemm(F, F, F, 49, 128, 64, 1, F, 16, None), 5),
        (lambda: L.w4a8_mxfp4_gemm_prequant(F, F, F, F, 1, 128, 48, 1, None), 2),
        (lambda: L.w4a8_mxfp4_gemm_prequant(F, None, F, F, 1, 128, 64, 1, None), 1),
        (lambda: L.w4a8_mxfp8_quantize(F, F, F, 1, 96, 1, None), 2),
        (lambda: L.w4a8_mxfp8_quantize(F, F + 4, F, 1, 128, 1, None), 4),
        (lambda: L.w4a8_mxfp4_prepack(F, F, F, 0, 128, 64, None), 2),
        (lambda: L.w4a8_mxfp4_prepack(F, None, F, 1, 128, 64, None), 1),
    ]
    for i, (call, st) in enumerate(cases):
        assert call() == st, i
    assert L.w4a8_mxfp4_gemm(F, F, F, 0, 128, 64, 1, None, 0, None) == 0              # M == 0: no-op


def test_weight_desc_validation():
    import ctypes as C
    L = w4.lib()
    F = 1 << 40
    d = w4.WeightDesc(5, 0, 128, F, None, None)
    assert L.w4a16_gemm_desc(F, F, C.byref(d), F, 1, 128, 64, 1, None, 0, None) == 3     # weight_bits
    d = w4.WeightDesc(4, 2, 128, F, None, None)
    assert L.w4a16_gemm_desc(F, F, C.byref(d), F, 1, 128, 64, 1, None, 0, None) == 3     # zero_format
    d = w4.WeightDesc(8, 0, 128, F, None, F + 2)
    assert L.w4a16_gemm_desc(F, F, C.byref(d), F, 1, 128, 64, 1, None, 0, None) == 4     # channel_scale alignment
    assert L.w4a16_gemm_desc(F, F, None, F, 1, 128, 64, 1, None, 0, None) == 1
    d = w4.WeightDesc(4, 1, 128, F, None, None)
    assert L.w4a16_gemm_desc(F, F, C.byref(d), F, 1, 128, 64, 1, None, 0, None) == 1     # float zeros need zero
    d = w4.WeightDesc(4, 1, 128, F, F, None)
    assert L.w4a16_gemm_desc(F, F, C.byref(d), F, 1, 128, 64, 1, None, 0, None) == 5     # and a workspace
    assert L.w4a16_gemm_desc_workspace_bytes(C.byref(d), 3, 256, 64) >= 3 * 64 * 4


def test_msd_noalloc_validation():
    L = w4.lib()
    # the scratch bound is checked on the host, before any device call
    assert w4.w4a16_msd_workspace_bytes(4096, 8192, 8192) > w4.MSD_SCRATCH_BYTES
    assert L.w4a16_msd_gemm_noalloc(FAKE, FAKE, FAKE, FAKE, 4096, 8192, 8192, 128, None) == 7
    assert L.w4a16_msd_gemm_noalloc(None, FAKE, FAKE, FAKE, 64, 8192, 8192, 128, None) == 1
    assert L.w4a16_msd_gemm_noalloc(FAKE, FAKE, FAKE, FAKE, 64, 8192, 8192, 64, None) == 3
    assert L.w4a16_msd_gemm_noalloc(FAKE, FAKE, FAKE, FAKE, 64, 8000, 8192, 128, None) == 2
    assert L.w4a16_msd_gemm_noalloc(FAKE + 8, FAKE, FAKE, FAKE, 64, 8192, 8192, 128, None) == 4
    assert L.w4a16_msd_gemm_noalloc(FAKE, FAKE, FAKE, FAKE, 0, 8192, 8192, 128, None) == 0


def test_prepack_g_validation():
    L = w4.lib()
    assert L.w4a16_prepack_g(FAKE, FAKE, 1, 256, 64, 1, 48, None) == 3       # unsupported group
    assert L.w4a16_prepack_g(FAKE, FAKE, 1, 256, 64, 1, 512, None) == 2      # does not divide K
    assert L.w4a16_prepack_g(FAKE, FAKE, 1, 200, 64, 1, 32, None) == 2       # K % 128 != 0
    assert L.w4a16_prepack_g(None, FAKE, 1, 256, 64, 1, 32, None) == 1
    assert L.w4a16_prepack_g(FAKE + 4, FAKE, 1, 256, 64, 1, 64, None) == 4
    # 32/64-row groups in the descriptor: 4-bit weights with integer zero points only
    for bits, zf in ((8, 0), (4, 1)):
        d = w4.WeightDesc(weight_bits=bits, group_size=32, scale=FAKE, zero=FAKE, zero_format=zf)
        assert L.w4a16_gemm_desc(FAKE, FAKE, C.byref(d), FAKE, 4, 256, 64, 0, None, 0, None) == 3
