"""ctypes wrapper of the C oracle (``oracle.c``).

TEST INFRASTRUCTURE: only the tests, the package smoke check and the
benchmark's CPU-baseline leg import this module.  The HIP library never does,
and this module never imports the library.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

F16 = 0
BF16 = 1

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
             "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose=False):
    """Compile the oracle with gcc (no GPU code involved)."""
    cmd = ["gcc", *GCC_FLAGS, _SRC, "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    global _lib
    _lib = None


_lib = None

_p = C.c_void_p
_i64 = C.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        sig = {
            "oracle_num_threads": ([], C.c_int),
            "oracle_set_num_threads": ([C.c_int], None),
            "oracle_f16_to_double": ([C.c_uint16], C.c_double),
            "oracle_bf16_to_double": ([C.c_uint16], C.c_double),
            "oracle_double_to_f16": ([C.c_double], C.c_uint16),
            "oracle_double_to_bf16": ([C.c_double], C.c_uint16),
            "oracle_round_array": ([_p, _p, _i64, C.c_int], None),
            "oracle_w4a16": ([_p, _p, _p, _p, _i64, _i64, _i64, _i64, C.c_int, _p, _p], None),
            "oracle_w4a16_points": ([_p, _p, _p, _p, _i64, _i64, _i64, _i64, C.c_int, _p, _p, _i64, _p], None),
            "oracle_grouped": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, C.c_int, _p, _p], None),
            "oracle_msd_amax": ([_p, _i64, _i64, _i64, _p], None),
            "oracle_msd_layers": ([_p, _p, _i64, _i64, _i64, _p], None),
            "oracle_msd_decompose_one": ([C.c_float, C.c_float, _p, _p], None),
            "oracle_msd_yint": ([_p, _p, _i64, _i64, _i64, _i64, _p], None),
            "oracle_msd": ([_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p], None),
            "oracle_moe_align": ([_p, _i64, _i64, _i64, _p, _p, _p], _i64),
            "oracle_silu_and_mul": ([_p, _i64, _i64, C.c_int, _p], None),
            "oracle_moe_sum": ([_p, _p, _p, _i64, _i64, _i64, C.c_int, _p], None),
            "oracle_fused_moe": ([_p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                  C.c_int, _p, _i64, _p], None),
            "oracle_w8a16": ([_p, _p, _p, _p, _i64, _i64, _i64, _i64, C.c_int, _p, _p], None),
            "oracle_w4a16_fzero": ([_p, _p, _p, _p, _i64, _i64, _i64, _i64, C.c_int, _p, _p], None),
            "oracle_w8a16_fzero": ([_p, _p, _p, _p, _i64, _i64, _i64, _i64, C.c_int, _p, _p], None),
            "oracle_e4m3_to_double": ([C.c_uint8], C.c_double),
            "oracle_e2m1_to_double": ([C.c_uint8], C.c_double),
            "oracle_e8m0_to_double": ([C.c_uint8], C.c_double),
            "oracle_mxfp8_quantize": ([_p, _i64, _i64, C.c_int, _p, _p], None),
            "oracle_w4a8_mxfp4": ([_p, _p, _p, _p, _i64, _i64, _i64, C.c_int, _p, _p], None),
            "oracle_prepack": ([_p, _p, _i64, _i64, _i64, C.c_int], None),
            "oracle_unpack": ([_p, _p, _i64, _i64, _i64, C.c_int], None),
            "oracle_prepack_layout": ([_p, _p, _i64, _i64, _i64, C.c_int, C.c_int], None),
            "oracle_unpack_layout": ([_p, _p, _i64, _i64, _i64, C.c_int, C.c_int], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return a.ctypes.data


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's parallel loops from now on."""
    lib().oracle_set_num_threads(int(n))


def f16_to_double(bits: int) -> float:
    return lib().oracle_f16_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits))


def round_array(v: np.ndarray, dtype: int) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_round_array(_ptr(v), _ptr(out), v.size, dtype)
    return out


def channel_scaled(y64, channel_scale, dtype):
    """Secondary (per-output-column) scale of the weight descriptor (Humming
    article: the descriptor's optional secondary scales, read as one fp32
    factor per column on top of the group scales): y = RNE(t[n] * y64[m][n]),
    the product in fp64.  Returns (scaled y64, 16-bit bits)."""
    t = np.asarray(channel_scale, dtype=np.float32).astype(np.float64)
    v = np.asarray(y64, dtype=np.float64) * t[None, :]
    return v, round_array(v, dtype)


def w4a16(x, w, scale, zero, M, K, N, dtype, group=128):
    """Return (y64 [M,N] float64, y [M,N] uint16 bits)."""
    y64 = np.empty((M, N), dtype=np.float64)
    y = np.empty((M, N), dtype=np.uint16)
    lib().oracle_w4a16(_ptr(x), _ptr(w), _ptr(scale), _ptr(zero), M, K, N, group, dtype,
                       _ptr(y64), _ptr(y))
    return y64, y


def w4a16_points(x, w, scale, zero, M, K, N, dtype, rows, cols, group=128):
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(rows.shape[0], dtype=np.float64)
    lib().oracle_w4a16_points(_ptr(x), _ptr(w), _ptr(scale), _ptr(zero), M, K, N, group, dtype,
                              _ptr(rows), _ptr(cols), rows.shape[0], _ptr(out))
    return out


def grouped(x, offsets, w, scale, zero, E, R, K, N, dtype, group=128):
    y64 = np.zeros((R, N), dtype=np.float64)
    y = np.zeros((R, N), dtype=np.uint16)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    lib().oracle_grouped(_ptr(x), _ptr(offsets), _ptr(w), _ptr(scale), _ptr(zero), E, R, K, N,
                         group, dtype, _ptr(y64), _ptr(y))
    return y64, y


def msd_amax(x, M, K, group=128):
    out = np.empty((M, K // group), dtype=np.float32)
    lib().oracle_msd_amax(_ptr(x), M, K, group, _ptr(out))
    return out


def msd_layers(x, amax, M, K, group=128):
    out = np.empty((3, M, K), dtype=np.int8)
    am = np.ascontiguousarray(amax, np.float32)        # bound: outlives the call
    lib().oracle_msd_layers(_ptr(x), _ptr(am), M, K, group, _ptr(out))
    return out


def msd_decompose_one(a: float, amax: float):
    out = np.zeros(3, dtype=np.int8)
    t = np.zeros(3, dtype=np.float32)
    lib().oracle_msd_decompose_one(float(np.float32(a)), float(np.float32(amax)), _ptr(out), _ptr(t))
    return out, t


def msd_yint(layers, w, M, K, N, group=128):
    out = np.empty((K // group, 3, M, N), dtype=np.int32)
    ly = np.ascontiguousarray(layers, np.int8)
    lib().oracle_msd_yint(_ptr(ly), _ptr(w), M, K, N, group, _ptr(out))
    return out


def msd(x, w, scale, M, K, N, group=128, intermediates=False):
    y64 = np.empty((M, N), dtype=np.float64)
    y = np.empty((M, N), dtype=np.uint16)
    amax = np.empty((M, K // group), dtype=np.float32) if intermediates else None
    layers = np.empty((3, M, K), dtype=np.int8) if intermediates else None
    lib().oracle_msd(_ptr(x), _ptr(w), _ptr(scale), M, K, N, group, _ptr(y64), _ptr(y),
                     _ptr(amax), _ptr(layers))
    if intermediates:
        return y64, y, amax, layers
    return y64, y


def moe_align(topk_ids, E):
    """Stable routing prep: returns (offsets [E+1], sorted [R], row_of [T*topk])."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    T, topk = ids.shape
    offsets = np.zeros(E + 1, dtype=np.int32)
    sorted_ = np.zeros(max(T * topk, 1), dtype=np.int32)
    row_of = np.zeros(max(T * topk, 1), dtype=np.int32)
    R = lib().oracle_moe_align(_ptr(ids), T, topk, E, _ptr(offsets), _ptr(sorted_), _ptr(row_of))
    return offsets, sorted_[:R].copy(), row_of[:T * topk].copy()


def silu_and_mul(h, dtype):
    """h: uint16 bits [R][2I] -> a [R][I] bits."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    R, I2 = h.shape
    a = np.empty((R, I2 // 2), dtype=np.uint16)
    lib().oracle_silu_and_mul(_ptr(h), R, I2 // 2, dtype, _ptr(a))
    return a


def moe_sum(o, row_of, topk_w, dtype):
    """o: uint16 bits [R][N]; row_of [T*topk]; topk_w fp32 [T][topk] -> [T][N] bits."""
    o = np.ascontiguousarray(o, dtype=np.uint16)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, topk = w.shape
    N = o.shape[1]
    out = np.empty((T, N), dtype=np.uint16)
    ro = np.ascontiguousarray(row_of, np.int32)
    lib().oracle_moe_sum(_ptr(o), _ptr(ro), _ptr(w), T, topk, N, dtype, _ptr(out))
    return out


def fused_moe(c, tokens=None):
    """Whole fused-experts chain of a synth.MoeChain for the given tokens
    (default: all); returns [P][H] bits."""
    tok = np.arange(c.T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
    out = np.empty((tok.shape[0], c.H), dtype=np.uint16)
    ids = np.ascontiguousarray(c.topk_ids, np.int32)
    tw = np.ascontiguousarray(c.topk_w, np.float32)
    lib().oracle_fused_moe(_ptr(c.x), _ptr(ids), _ptr(tw), _ptr(c.w13), _ptr(c.s13),
                           _ptr(c.z13), _ptr(c.w2), _ptr(c.s2), _ptr(c.z2), c.T, c.topk, c.E, c.H, c.I,
                           128, c.dtype, _ptr(tok), tok.shape[0], _ptr(out))
    return out


def fused_moe_steps(c):
    """The whole fused-experts chain of a synth.MoeChain for every token, composed
    from the oracle's own steps in the chain's order (routing prep, gate/up
    grouped W4A16 on the routed rows, silu_and_mul, down grouped W4A16,
    weighted moe_sum); returns [T][H] bits.  Each routed row is computed once,
    so this is far cheaper than fused_moe at full size; every row and sum is
    taken in the same order as fused_moe, so the two agree bit for bit."""
    offsets, sorted_, row_of = moe_align(c.topk_ids, c.E)
    R = int(offsets[-1])
    if R == 0:
        return moe_sum(np.zeros((1, c.H), np.uint16), row_of, c.topk_w, c.dtype)
    xs = np.ascontiguousarray(np.asarray(c.x)[sorted_ // c.topk], dtype=np.uint16)   # token of each routed row
    _, h = grouped(xs, offsets, np.ascontiguousarray(c.w13), np.ascontiguousarray(c.s13),
                   None if c.z13 is None else np.ascontiguousarray(c.z13), c.E, R, c.H, 2 * c.I, c.dtype)
    a = silu_and_mul(h, c.dtype)
    _, o = grouped(a, offsets, np.ascontiguousarray(c.w2), np.ascontiguousarray(c.s2),
                   None if c.z2 is None else np.ascontiguousarray(c.z2), c.E, R, c.I, c.H, c.dtype)
    return moe_sum(o, row_of, c.topk_w, c.dtype)


def w4a16_fzero(x, w, scale, zf, M, K, N, dtype, group=128):
    """W4A16 with floating-point zero points: w [K][N/2] unsigned codes, zf
    [K/group][N] 16-bit patterns of dtype; returns (y64, y bits)."""
    y64 = np.empty((M, N), dtype=np.float64)
    y = np.empty((M, N), dtype=np.uint16)
    xc, wc, sc, zc = (np.ascontiguousarray(x, np.uint16), np.ascontiguousarray(w, np.uint8),
                      np.ascontiguousarray(scale, np.uint16), np.ascontiguousarray(zf, np.uint16))
    lib().oracle_w4a16_fzero(_ptr(xc), _ptr(wc), _ptr(sc), _ptr(zc), M, K, N, group, dtype, _ptr(y64), _ptr(y))
    return y64, y


def w8a16_fzero(x, w, scale, zf, M, K, N, dtype, group=128):
    """W8A16 with floating-point zero points: w [K][N] uint8 codes, zf
    [K/group][N] 16-bit patterns of dtype; returns (y64, y bits)."""
    y64 = np.empty((M, N), dtype=np.float64)
    y = np.empty((M, N), dtype=np.uint16)
    xc, wc, sc, zc = (np.ascontiguousarray(x, np.uint16), np.ascontiguousarray(w, np.uint8),
                      np.ascontiguousarray(scale, np.uint16), np.ascontiguousarray(zf, np.uint16))
    lib().oracle_w8a16_fzero(_ptr(xc), _ptr(wc), _ptr(sc), _ptr(zc), M, K, N, group, dtype, _ptr(y64), _ptr(y))
    return y64, y


def w8a16(x, w, scale, zero, M, K, N, dtype, group=128):
    """W8A16: w [K][N] bytes (int8, or uint8 with zero [K/group][N]); returns
    (y64 [M,N] float64, y [M,N] uint16 bits)."""
    y64 = np.empty((M, N), dtype=np.float64)
    y = np.empty((M, N), dtype=np.uint16)
    # contiguous copies are bound to names so they outlive the call
    xc, wc, sc = (np.ascontiguousarray(x, np.uint16), np.ascontiguousarray(w, np.uint8),
                  np.ascontiguousarray(scale, np.uint16))
    zc = None if zero is None else np.ascontiguousarray(zero, np.uint8)
    lib().oracle_w8a16(_ptr(xc), _ptr(wc), _ptr(sc), _ptr(zc), M, K, N, group, dtype, _ptr(y64), _ptr(y))
    return y64, y


def mxfp8_quantize(x, M, K, dtype):
    """x bits [M][K] -> (E4M3 codes [M][K] uint8, E8M0 scales [M][K/32] uint8)."""
    qx = np.empty((M, K), dtype=np.uint8)
    sx = np.empty((M, K // 32), dtype=np.uint8)
    xc = np.ascontiguousarray(x, np.uint16)
    lib().oracle_mxfp8_quantize(_ptr(xc), M, K, dtype, _ptr(qx), _ptr(sx))
    return qx, sx


def w4a8_mxfp4(qx, sx, w, sw, M, K, N, dtype):
    """Return (y64 [M,N], y [M,N] bits) of the MXFP8 x MXFP4 product."""
    y64 = np.empty((M, N), dtype=np.float64)
    y = np.empty((M, N), dtype=np.uint16)
    qc, sc, wc, swc = (np.ascontiguousarray(a, np.uint8) for a in (qx, sx, w, sw))
    lib().oracle_w4a8_mxfp4(_ptr(qc), _ptr(sc), _ptr(wc), _ptr(swc), M, K, N, dtype, _ptr(y64), _ptr(y))
    return y64, y


def prepack(w, E, K, N, is_signed, layout=0):
    """layout 0: the standard tile layout; 1: the group-aligned layout used for
    scale groups of 32 or 64 rows."""
    out = np.empty(E * K * N // 2, dtype=np.uint8)
    wc = np.ascontiguousarray(w, np.uint8)
    lib().oracle_prepack_layout(_ptr(wc), _ptr(out), E, K, N, int(is_signed), int(layout))
    return out


def unpack(packed, E, K, N, is_signed, layout=0):
    out = np.empty(E * K * N // 2, dtype=np.uint8)
    pc = np.ascontiguousarray(packed, np.uint8)
    lib().oracle_unpack_layout(_ptr(pc), _ptr(out), E, K, N, int(is_signed), int(layout))
    return out


def compare(y_bits, y_ref_bits, dtype):
    """Tolerance check used across the suite: returns (max_ratio, rel_l1), where
    max_ratio = max|y - y_ref| / max|y_ref| (bar 1e-2) and rel_l1 =
    sum|y - y_ref| / sum|y_ref| (bar 2e-3); y_ref is the once-rounded oracle."""
    if dtype == BF16:
        conv = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        conv = lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64)
    y = conv(y_bits)
    r = conv(y_ref_bits)
    d = np.abs(y - r)
    mref = np.max(np.abs(r)) if r.size else 0.0
    sref = np.sum(np.abs(r))
    max_ratio = float(np.max(d) / mref) if r.size and mref > 0 else float(np.max(d) if d.size else 0.0)
    rel_l1 = float(np.sum(d) / sref) if sref > 0 else float(np.sum(d))
    return max_ratio, rel_l1
