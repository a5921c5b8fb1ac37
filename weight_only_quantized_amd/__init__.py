"""Python binding of libw4a16 (weight-only quantized matmul on MI355X).

Argument marshalling only: every function has the name of the C entry point
it calls (include/w4a16.h, include/w4a16_test.h), takes device tensors (torch
tensors on a ROCm device, or raw integer device addresses) plus sizes, and
enqueues on the given stream (default: torch's current stream).  Every step of
the computation runs in the HIP kernels of libw4a16.so; there is no fallback.
A non-OK status raises :class:`W4A16Error`.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

W4A16_F16 = 0
W4A16_BF16 = 1
GROUP_SIZE = 128

W4A16_OK = 0
STATUS_NAMES = {0: "W4A16_OK", 1: "W4A16_ERR_NULL", 2: "W4A16_ERR_SHAPE", 3: "W4A16_ERR_UNSUPPORTED",
                4: "W4A16_ERR_ALIGN", 5: "W4A16_ERR_WORKSPACE", 6: "W4A16_ERR_DEVICE", 7: "W4A16_ERR_SCRATCH"}


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {w4a16_status_str(status)} (status {status})")


class WeightDesc(C.Structure):
    """w4a16_weight_desc (include/w4a16.h): weight bits, group size, scale,
    zero points and the optional per-column secondary scale (device pointers)."""
    _fields_ = [("weight_bits", C.c_int32), ("zero_format", C.c_int32), ("group_size", C.c_int64),
                ("scale", C.c_void_p), ("zero", C.c_void_p), ("channel_scale", C.c_void_p)]


_lib = None
_p = C.c_void_p
_i64 = C.c_int64
_SIGS = {
    "w4a16_status_str": ([C.c_int], C.c_char_p),
    "w4a16_prepacked_bytes": ([_i64, _i64, _i64], C.c_size_t),
    "w4a16_prepack": ([_p, _p, _i64, _i64, _i64, C.c_int, _p], C.c_int),
    "w4a16_prepack_g": ([_p, _p, _i64, _i64, _i64, C.c_int, _i64, _p], C.c_int),
    "w4a16_gemm": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, C.c_int, _p], C.c_int),
    "w4a16_msd_workspace_bytes": ([_i64, _i64, _i64, _i64], C.c_size_t),
    "w4a16_msd_gemm": ([_p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, C.c_size_t, _p], C.c_int),
    "w4a16_msd_gemm_noalloc": ([_p, _p, _p, _p, _i64, _i64, _i64, _i64, _p], C.c_int),
    "w4a16_grouped_gemm": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, C.c_int, _p], C.c_int),
    "w4a16_moe_align": ([_p, _i64, _i64, _i64, _p, _p, _p, _p], C.c_int),
    "w4a16_moe_gather": ([_p, _p, _p, _i64, _i64, _i64, _i64, _p, C.c_int, _p], C.c_int),
    "w4a16_silu_and_mul": ([_p, _p, _i64, _i64, _p, C.c_int, _p], C.c_int),
    "w4a16_moe_sum": ([_p, _p, _p, _i64, _i64, _i64, _p, C.c_int, _p], C.c_int),
    "w4a16_fused_moe_workspace_bytes": ([_i64, _i64, _i64, _i64, _i64], C.c_size_t),
    "w4a16_fused_moe": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64, C.c_int,
                         _p, C.c_size_t, _p], C.c_int),
    "w4a16_gemm_desc_workspace_bytes": ([C.POINTER(WeightDesc), _i64, _i64, _i64], C.c_size_t),
    "w4a16_gemm_desc": ([_p, _p, C.POINTER(WeightDesc), _p, _i64, _i64, _i64, C.c_int, _p, C.c_size_t, _p],
                        C.c_int),
    "w8a16_prepacked_bytes": ([_i64, _i64, _i64], C.c_size_t),
    "w8a16_prepack": ([_p, _p, _i64, _i64, _i64, C.c_int, _p], C.c_int),
    "w8a16_gemm": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, C.c_int, _p], C.c_int),
    "w4a8_mxfp4_prepacked_bytes": ([_i64, _i64, _i64], C.c_size_t),
    "w4a8_mxfp4_prepack": ([_p, _p, _p, _i64, _i64, _i64, _p], C.c_int),
    "w4a8_mxfp8_quantize": ([_p, _p, _p, _i64, _i64, C.c_int, _p], C.c_int),
    "w4a8_mxfp4_gemm_prequant": ([_p, _p, _p, _p, _i64, _i64, _i64, C.c_int, _p], C.c_int),
    "w4a8_mxfp4_workspace_bytes": ([_i64, _i64], C.c_size_t),
    "w4a8_mxfp4_gemm": ([_p, _p, _p, _i64, _i64, _i64, C.c_int, _p, C.c_size_t, _p], C.c_int),
    "w4a8_mxfp4_grouped_workspace_bytes": ([_i64, _i64], C.c_size_t),
    "w4a8_mxfp4_grouped_gemm": ([_p, _p, _p, _p, _i64, _i64, _i64, _i64, C.c_int, _p, C.c_size_t, _p], C.c_int),
    "w4a16_test_unpack": ([_p, _p, _i64, _i64, _i64, C.c_int, _p], C.c_int),
    "w4a16_test_msd_intermediates": ([_p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, C.c_size_t, _p], C.c_int),
    "w4a16_test_msd_basic_workspace_bytes": ([_i64, _i64, _i64, _i64], C.c_size_t),
    "w4a16_test_msd_basic": ([_p, _p, _p, _p, _i64, _i64, _i64, _i64, _p, C.c_size_t, _p], C.c_int),
    "w4a16_test_force_variant": ([C.c_int], C.c_int),
    "w4a16_test_variant_name": ([_i64, _i64, _i64, C.c_int, C.c_int], C.c_char_p),
    "w4a16_test_small_config": ([C.c_int], C.c_int),
    "w4a16_test_tile_config": ([C.c_int], C.c_int),
    "w4a16_test_tile_halves": ([C.c_int], C.c_int),
    "w4a16_test_msd_config": ([C.c_int], C.c_int),
    "w4a16_test_mx_small_config": ([C.c_int], C.c_int),
    "w4a16_test_mx_tile_config": ([C.c_int], C.c_int),
    "w4a16_test_w8_config": ([C.c_int, C.c_int], C.c_int),
}
EXPORTED = tuple(_SIGS)

# size of the static per-device scratch of w4a16_msd_gemm_noalloc (W4A16_MSD_SCRATCH_BYTES)
MSD_SCRATCH_BYTES = 32 << 20


def lib():
    """Load libw4a16.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != W4A16_OK:
        raise W4A16Error(status, where)


def w4a16_status_str(status: int) -> str:
    return lib().w4a16_status_str(int(status)).decode()


def w4a16_prepacked_bytes(E: int, K: int, N: int) -> int:
    return lib().w4a16_prepacked_bytes(E, K, N)


def w4a16_prepack(w, w_packed, E, K, N, is_signed, stream=None):
    _check(lib().w4a16_prepack(_ptr(w), _ptr(w_packed), E, K, N, int(is_signed), _stream(stream)), "w4a16_prepack")


def w4a16_prepack_g(w, w_packed, E, K, N, is_signed, group_size, stream=None):
    _check(lib().w4a16_prepack_g(_ptr(w), _ptr(w_packed), E, K, N, int(is_signed), group_size, _stream(stream)),
           "w4a16_prepack_g")


def w4a16_gemm(x, w_packed, scale, zero, y, M, K, N, group_size=GROUP_SIZE, dt=W4A16_BF16, stream=None):
    _check(lib().w4a16_gemm(_ptr(x), _ptr(w_packed), _ptr(scale), _ptr(zero), _ptr(y), M, K, N, group_size,
                            int(dt), _stream(stream)), "w4a16_gemm")


def w4a16_msd_workspace_bytes(M, K, N, group_size=GROUP_SIZE) -> int:
    return lib().w4a16_msd_workspace_bytes(M, K, N, group_size)


def w4a16_msd_gemm(x, w_packed, antiquant_scale, y, M, K, N, group_size=GROUP_SIZE, workspace=None,
                   workspace_bytes=0, stream=None):
    _check(lib().w4a16_msd_gemm(_ptr(x), _ptr(w_packed), _ptr(antiquant_scale), _ptr(y), M, K, N, group_size,
                                _ptr(workspace), int(workspace_bytes), _stream(stream)), "w4a16_msd_gemm")


def w4a16_msd_gemm_noalloc(x, w_packed, antiquant_scale, y, M, K, N, group_size=GROUP_SIZE, stream=None):
    _check(lib().w4a16_msd_gemm_noalloc(_ptr(x), _ptr(w_packed), _ptr(antiquant_scale), _ptr(y), M, K, N,
                                        group_size, _stream(stream)), "w4a16_msd_gemm_noalloc")


def w4a16_grouped_gemm(x, expert_offsets, w_packed, scale, zero, y, E, R, K, N, group_size=GROUP_SIZE,
                       dt=W4A16_BF16, stream=None):
    _check(lib().w4a16_grouped_gemm(_ptr(x), _ptr(expert_offsets), _ptr(w_packed), _ptr(scale), _ptr(zero),
                                    _ptr(y), E, R, K, N, group_size, int(dt), _stream(stream)),
           "w4a16_grouped_gemm")


def w4a16_moe_align(topk_ids, T, topk, E, expert_offsets, sorted_ids, row_of, stream=None):
    _check(lib().w4a16_moe_align(_ptr(topk_ids), T, topk, E, _ptr(expert_offsets), _ptr(sorted_ids),
                                 _ptr(row_of), _stream(stream)), "w4a16_moe_align")


def w4a16_moe_gather(x, sorted_ids, expert_offsets, T, topk, E, H, x_sorted, dt=W4A16_BF16, stream=None):
    _check(lib().w4a16_moe_gather(_ptr(x), _ptr(sorted_ids), _ptr(expert_offsets), T, topk, E, H,
                                  _ptr(x_sorted), int(dt), _stream(stream)), "w4a16_moe_gather")


def w4a16_silu_and_mul(h, row_count, R, I, a, dt=W4A16_BF16, stream=None):
    _check(lib().w4a16_silu_and_mul(_ptr(h), _ptr(row_count), R, I, _ptr(a), int(dt), _stream(stream)),
           "w4a16_silu_and_mul")


def w4a16_moe_sum(o, row_of, topk_w, T, topk, N, out, dt=W4A16_BF16, stream=None):
    _check(lib().w4a16_moe_sum(_ptr(o), _ptr(row_of), _ptr(topk_w), T, topk, N, _ptr(out), int(dt),
                               _stream(stream)), "w4a16_moe_sum")


def w4a16_fused_moe_workspace_bytes(T, topk, E, H, I) -> int:
    return lib().w4a16_fused_moe_workspace_bytes(T, topk, E, H, I)


def w4a16_fused_moe(x, topk_ids, topk_w, w13_packed, s13, z13, w2_packed, s2, z2, out, T, topk, E, H, I,
                    group_size=GROUP_SIZE, dt=W4A16_BF16, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().w4a16_fused_moe(_ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(w13_packed), _ptr(s13), _ptr(z13),
                                 _ptr(w2_packed), _ptr(s2), _ptr(z2), _ptr(out), T, topk, E, H, I, group_size,
                                 int(dt), _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "w4a16_fused_moe")


def weight_desc(scale, zero=None, channel_scale=None, weight_bits=4, group_size=GROUP_SIZE, zero_format=0):
    return WeightDesc(int(weight_bits), int(zero_format), int(group_size), _ptr(scale), _ptr(zero),
                      _ptr(channel_scale))


def w4a16_gemm_desc_workspace_bytes(desc, M, K, N) -> int:
    return lib().w4a16_gemm_desc_workspace_bytes(C.byref(desc), M, K, N)


def w4a16_gemm_desc(x, w_packed, y, M, K, N, scale, zero=None, channel_scale=None, weight_bits=4,
                    group_size=GROUP_SIZE, dt=W4A16_BF16, zero_format=0, workspace=None, workspace_bytes=0,
                    stream=None):
    d = weight_desc(scale, zero, channel_scale, weight_bits, group_size, zero_format)
    _check(lib().w4a16_gemm_desc(_ptr(x), _ptr(w_packed), C.byref(d), _ptr(y), M, K, N, int(dt), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream)), "w4a16_gemm_desc")


def w8a16_prepacked_bytes(E: int, K: int, N: int) -> int:
    return lib().w8a16_prepacked_bytes(E, K, N)


def w8a16_prepack(w, w_packed, E, K, N, is_signed, stream=None):
    _check(lib().w8a16_prepack(_ptr(w), _ptr(w_packed), E, K, N, int(is_signed), _stream(stream)), "w8a16_prepack")


def w8a16_gemm(x, w_packed, scale, zero, y, M, K, N, group_size=GROUP_SIZE, dt=W4A16_BF16, stream=None):
    _check(lib().w8a16_gemm(_ptr(x), _ptr(w_packed), _ptr(scale), _ptr(zero), _ptr(y), M, K, N, group_size,
                            int(dt), _stream(stream)), "w8a16_gemm")


def w4a8_mxfp4_prepacked_bytes(E: int, K: int, N: int) -> int:
    return lib().w4a8_mxfp4_prepacked_bytes(E, K, N)


def w4a8_mxfp4_prepack(w, w_scale, w_packed, E, K, N, stream=None):
    _check(lib().w4a8_mxfp4_prepack(_ptr(w), _ptr(w_scale), _ptr(w_packed), E, K, N, _stream(stream)),
           "w4a8_mxfp4_prepack")


def w4a8_mxfp8_quantize(x, qx, sx, M, K, dt=W4A16_BF16, stream=None):
    _check(lib().w4a8_mxfp8_quantize(_ptr(x), _ptr(qx), _ptr(sx), M, K, int(dt), _stream(stream)),
           "w4a8_mxfp8_quantize")


def w4a8_mxfp4_gemm_prequant(qx, sx, w_packed, y, M, K, N, dt=W4A16_BF16, stream=None):
    _check(lib().w4a8_mxfp4_gemm_prequant(_ptr(qx), _ptr(sx), _ptr(w_packed), _ptr(y), M, K, N, int(dt),
                                          _stream(stream)), "w4a8_mxfp4_gemm_prequant")


def w4a8_mxfp4_workspace_bytes(M: int, K: int) -> int:
    return lib().w4a8_mxfp4_workspace_bytes(M, K)


def w4a8_mxfp4_gemm(x, w_packed, y, M, K, N, dt=W4A16_BF16, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().w4a8_mxfp4_gemm(_ptr(x), _ptr(w_packed), _ptr(y), M, K, N, int(dt), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream)), "w4a8_mxfp4_gemm")


def w4a8_mxfp4_grouped_workspace_bytes(R: int, K: int) -> int:
    return lib().w4a8_mxfp4_grouped_workspace_bytes(R, K)


def w4a8_mxfp4_grouped_gemm(x, expert_offsets, w_packed, y, E, R, K, N, dt=W4A16_BF16, workspace=None,
                            workspace_bytes=0, stream=None):
    _check(lib().w4a8_mxfp4_grouped_gemm(_ptr(x), _ptr(expert_offsets), _ptr(w_packed), _ptr(y), E, R, K, N,
                                         int(dt), _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "w4a8_mxfp4_grouped_gemm")


# ---- test hooks (include/w4a16_test.h) ----------------------------------------

def w4a16_test_unpack(w_packed, w, E, K, N, is_signed, stream=None):
    _check(lib().w4a16_test_unpack(_ptr(w_packed), _ptr(w), E, K, N, int(is_signed), _stream(stream)),
           "w4a16_test_unpack")


def w4a16_test_msd_intermediates(x, w_packed, M, K, N, amax, layers, yint, workspace, workspace_bytes,
                                 group_size=GROUP_SIZE, stream=None):
    _check(lib().w4a16_test_msd_intermediates(_ptr(x), _ptr(w_packed), M, K, N, group_size, _ptr(amax),
                                              _ptr(layers), _ptr(yint), _ptr(workspace), int(workspace_bytes),
                                              _stream(stream)), "w4a16_test_msd_intermediates")


def w4a16_test_msd_basic_workspace_bytes(M, K, N, group_size=GROUP_SIZE) -> int:
    return lib().w4a16_test_msd_basic_workspace_bytes(M, K, N, group_size)


def w4a16_test_msd_basic(x, w_packed, antiquant_scale, y, M, K, N, group_size=GROUP_SIZE, workspace=None,
                         workspace_bytes=0, stream=None):
    _check(lib().w4a16_test_msd_basic(_ptr(x), _ptr(w_packed), _ptr(antiquant_scale), _ptr(y), M, K, N, group_size,
                                      _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "w4a16_test_msd_basic")


def w4a16_test_force_variant(variant: int) -> int:
    return lib().w4a16_test_force_variant(int(variant))


def w4a16_test_variant_name(M, K, N, dt, has_zero) -> str:
    return lib().w4a16_test_variant_name(M, K, N, int(dt), int(has_zero)).decode()


def w4a16_test_small_config(idx: int) -> int:
    return lib().w4a16_test_small_config(int(idx))


def w4a16_test_tile_config(idx: int) -> int:
    return lib().w4a16_test_tile_config(int(idx))


def w4a16_test_tile_halves(enable: int) -> int:
    return lib().w4a16_test_tile_halves(int(enable))


def w4a16_test_msd_config(idx: int) -> int:
    return lib().w4a16_test_msd_config(int(idx))


def w4a16_test_mx_small_config(idx: int) -> int:
    return lib().w4a16_test_mx_small_config(int(idx))


def w4a16_test_mx_tile_config(idx: int) -> int:
    return lib().w4a16_test_mx_tile_config(int(idx))


def w4a16_test_w8_config(small_idx: int, tile_idx: int) -> int:
    return lib().w4a16_test_w8_config(int(small_idx), int(tile_idx))
