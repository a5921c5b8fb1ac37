"""Seeded synthetic inputs for the weight-only quantized matmul workloads.

This module only *produces* input tensors (activations, packed int4 weights,
scales, zero points, MoE routing).  It contains none of the method's
arithmetic: no dequantisation, no matmul, no MSD decomposition.  Both the CPU
oracle (``oracle/``) and the HIP path (``weight_only_quantized_amd``) consume
exactly the bytes produced here, so the two sides never share computation.

Storage conventions (the plain, user-facing layout; the pages only say "two
int4 per byte", see the WeightQuantBatchMatmulExperiment operator deep-dive,
§4.3):

* activations ``x``: ``[M][K]`` raw 16-bit patterns (``np.uint16``) of fp16 or
  bf16 values, row-major;
* weights ``w``: ``[K][N/2]`` bytes (``[E][K][N/2]`` for grouped), element
  ``(k, n)`` in byte ``k*N/2 + n//2``, low nibble for even ``n``;
  signed weights are 4-bit two's complement in [-8, 7], unsigned ones are
  plain [0, 15];
* scales: ``[G][N]`` (``[E][G][N]``) raw 16-bit patterns, same dtype as ``x``;
* zero points: ``[G][N/2]`` bytes packed like ``w`` (unsigned 4-bit).

Random streams: one ``numpy`` PCG64 generator per (seed, tensor tag), so each
tensor is reproducible on its own.  Normal draws are made in fp64, rounded once
to fp32 and then once, round-to-nearest-even, to the 16-bit type.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional

import numpy as np

F16 = 0
BF16 = 1
GROUP = 128

_TAGS = ("x", "w", "s", "z", "mask", "route", "tokens")


def stream(seed: int, tag: str) -> np.random.Generator:
    """Independent generator for one tensor tag."""
    return np.random.Generator(np.random.PCG64([int(seed), zlib.crc32(tag.encode())]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even), return raw bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to fp16 (numpy's conversion is round-to-nearest-even)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(a: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == BF16 else f32_to_f16_bits(a)


def bits_to_f32(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact widening of 16-bit patterns to fp32 (for test diagnostics)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


def pack_nibbles(vals: np.ndarray) -> np.ndarray:
    """Pack a [..., N] array of 4-bit codes (0..15) two per byte along the last
    axis, low nibble = even index."""
    v = np.ascontiguousarray(vals, dtype=np.uint8) & 0xF
    assert v.shape[-1] % 2 == 0
    return (v[..., 0::2] | (v[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_nibbles` (4-bit codes, unsigned)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


@dataclasses.dataclass
class Problem:
    """One W4A16 (or MSD) problem instance in the plain storage layout."""
    x: np.ndarray                 # uint16 [M][K] (or [R][K] for grouped)
    w: np.ndarray                 # uint8 [K][N/2] or [E][K][N/2]
    scale: np.ndarray             # uint16 [G][N] or [E][G][N]
    zero: Optional[np.ndarray]    # uint8 [G][N/2] or [E][G][N/2], or None
    q: np.ndarray                 # int8 integer weight values, [K][N] / [E][K][N]
    M: int
    K: int
    N: int
    dtype: int
    E: int = 1
    offsets: Optional[np.ndarray] = None   # int32 [E+1] for grouped
    name: str = ""
    group: int = GROUP                     # K rows per scale group (multiple of 128)

    @property
    def signed(self) -> bool:
        return self.zero is None

    @property
    def G(self) -> int:
        return self.K // self.group


def _normal(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(shape, dtype=np.float64).astype(np.float32)


def _weights(seed, shape_kn, signed, tag="w"):
    g = stream(seed, tag)
    if signed:
        q = g.integers(-8, 8, size=shape_kn, dtype=np.int8)
    else:
        q = g.integers(0, 16, size=shape_kn, dtype=np.int8)
    return q, pack_nibbles(q.view(np.uint8) & 0xF)


def _scales(seed, shape, lo, hi, dtype, tag="s"):
    g = stream(seed, tag)
    s = (lo + (hi - lo) * g.random(shape, dtype=np.float64)).astype(np.float32)
    return to_bits(s, dtype)


def make_dense(M, K, N, dtype, signed=True, scale_range=(0.002, 0.01),
               zero_range=(6, 9), seed=0, outlier_frac=0.0, outlier_mult=20.0,
               x_scale=1.0, name="", group=GROUP) -> Problem:
    """Dense W4A16 problem: x ~ N(0,1) (optionally with outliers), W int4,
    scale uniform, zero points uniform integers (unsigned weights only); one
    scale (and zero) row per ``group`` K rows."""
    assert K % group == 0 and N % 2 == 0
    G = K // group
    x = _normal(stream(seed, "x"), (M, K)) * np.float32(x_scale)
    if outlier_frac > 0:
        mask = stream(seed, "mask").random((M, K)) < outlier_frac
        x = np.where(mask, x * np.float32(outlier_mult), x).astype(np.float32)
    xb = to_bits(x, dtype)
    q, w = _weights(seed, (K, N), signed)
    s = _scales(seed, (G, N), scale_range[0], scale_range[1], dtype)
    z = None
    if not signed:
        zq = stream(seed, "z").integers(zero_range[0], zero_range[1] + 1, size=(G, N), dtype=np.int8)
        z = pack_nibbles(zq.view(np.uint8))
    return Problem(x=xb, w=w, scale=s, zero=z, q=q, M=M, K=K, N=N, dtype=dtype, name=name, group=group)


def zipf_routing(tokens, experts, topk, alpha, seed):
    """Per-token top-k expert choice: ``topk`` distinct experts drawn without
    replacement from a Zipf(alpha) law truncated to ``experts`` ranks,
    P(e) proportional to (e+1)^-alpha.  Returns int array [tokens, topk]."""
    p = (np.arange(1, experts + 1, dtype=np.float64)) ** (-alpha)
    p /= p.sum()
    g = stream(seed, "route")
    out = np.empty((tokens, topk), dtype=np.int64)
    for t in range(tokens):
        out[t] = g.choice(experts, size=topk, replace=False, p=p)
    return out


def _routed_rows(E, tokens, topk, K, dtype, alpha, seed, counts=None):
    """Rows of token activations gathered and sorted by (expert, token) under
    Zipf routing (or the given rows per expert); returns (offsets [E+1], x bits)."""
    if counts is None:
        route = zipf_routing(tokens, E, topk, alpha, seed)
        pairs = sorted((int(e), t) for t in range(tokens) for e in route[t])
        tok_of_row = np.array([t for _, t in pairs], dtype=np.int64)
        counts = np.bincount(np.array([e for e, _ in pairs]), minlength=E)
    else:
        counts = np.asarray(counts, dtype=np.int64)
        tok_of_row = np.concatenate([np.arange(c) % max(tokens, 1) for c in counts]).astype(np.int64) \
            if counts.sum() else np.zeros(0, np.int64)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    xt = _normal(stream(seed, "tokens"), (max(tokens, 1), K))
    x = xt[tok_of_row] if R else np.zeros((0, K), np.float32)
    return offsets, to_bits(x, dtype)


def make_grouped(E, tokens, topk, K, N, dtype, alpha=1.1, signed=True,
                 scale_range=(0.002, 0.01), seed=0, name="",
                 counts: Optional[np.ndarray] = None, group=GROUP) -> Problem:
    """MoE grouped problem.  Rows of ``x`` are token activations gathered and
    sorted by (expert, token); ``offsets[e]..offsets[e+1]`` are expert e's rows.
    If ``counts`` is given it overrides the routing draw (rows per expert)."""
    G = K // group
    offsets, xb = _routed_rows(E, tokens, topk, K, dtype, alpha, seed, counts)
    R = int(offsets[-1])
    q, w = _weights(seed, (E, K, N), signed)
    s = _scales(seed, (E, G, N), scale_range[0], scale_range[1], dtype)
    z = None
    if not signed:
        zq = stream(seed, "z").integers(6, 10, size=(E, G, N), dtype=np.int8)
        z = pack_nibbles(zq.view(np.uint8))
    return Problem(x=xb, w=w, scale=s, zero=z, q=q, M=R, K=K, N=N, dtype=dtype,
                   E=E, offsets=offsets, name=name, group=group)


# ---------------------------------------------------------------------------
# The five workloads (shapes and distributions of the benchmark configurations)
# ---------------------------------------------------------------------------

def tiny(seed=0) -> Problem:
    """M=4, K=256, N=256; x fp16 N(0,1); signed int4; scale fp16 U[0.005,0.02]."""
    return make_dense(4, 256, 256, F16, signed=True, scale_range=(0.005, 0.02), seed=seed, name="tiny")


def decode(M, seed=0, N=14336, K=4096) -> Problem:
    """Decode: K=4096, N=14336; x bf16 N(0,1); unsigned int4 with per-group
    uint4 zero points U{6..9}; scale bf16 U[0.002,0.01]."""
    return make_dense(M, K, N, BF16, signed=False, scale_range=(0.002, 0.01),
                      zero_range=(6, 9), seed=seed, name=f"decode_m{M}")


def prefill(seed=0, M=4096, K=4096, N=4096) -> Problem:
    """Prefill: M=N=K=4096; x bf16 N(0,1); signed int4; scale bf16 U[0.002,0.01]."""
    return make_dense(M, K, N, BF16, signed=True, scale_range=(0.002, 0.01), seed=seed, name="prefill")


def msd(seed=0, M=64, K=8192, N=8192) -> Problem:
    """MSD A16W4: M=64, K=N=8192; x fp16 N(0,1) with 1% of entries x20;
    signed int4; antiquant_scale fp16 U[0.005,0.02]."""
    return make_dense(M, K, N, F16, signed=True, scale_range=(0.005, 0.02), seed=seed,
                      outlier_frac=0.01, outlier_mult=20.0, name="msd")


def msd_page_example(seed=0) -> Problem:
    """The MSD page's own example shape (M=1, N=12288, K=8192): x U[-3,3],
    weights in [-7,7], scale U[-3,3] (WeightQuantBatchMatmulExperiment
    operator deep-dive, §4.3)."""
    M, K, N = 1, 8192, 12288
    G = K // GROUP
    x = (-3 + 6 * stream(seed, "x").random((M, K))).astype(np.float32)
    q = stream(seed, "w").integers(-7, 8, size=(K, N), dtype=np.int8)
    s = (-3 + 6 * stream(seed, "s").random((G, N))).astype(np.float32)
    return Problem(x=to_bits(x, F16), w=pack_nibbles(q.view(np.uint8) & 0xF),
                   scale=to_bits(s, F16), zero=None, q=q, M=M, K=K, N=N, dtype=F16,
                   name="msd_page")


def moe(seed=0) -> Problem:
    """MoE grouped: 64 experts, 512 tokens, top-8 Zipf(1.1) routing,
    K=2048, N=1408; x bf16 N(0,1); signed int4; scale bf16 U[0.002,0.01]."""
    return make_grouped(64, 512, 8, 2048, 1408, BF16, alpha=1.1, signed=True, seed=seed, name="moe")


# ---------------------------------------------------------------------------
# MoE fused-experts chain (routing, gate/up and down expert weights)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class MoeChain:
    """Inputs of one fused-experts call in the plain layouts: tokens x
    [T][H], routing ids/weights [T][topk], gate/up weights W13 [E][H][2I]
    (gate columns 0..I-1, up columns I..2I-1) and down weights W2 [E][I][H],
    each with per-group scales (and zero points when unsigned)."""
    x: np.ndarray                  # uint16 [T][H]
    topk_ids: np.ndarray           # int32 [T][topk]
    topk_w: np.ndarray             # float32 [T][topk]
    w13: np.ndarray                # uint8 [E][H][I]      (2I nibbles per row)
    s13: np.ndarray                # uint16 [E][H/128][2I]
    z13: Optional[np.ndarray]      # uint8 [E][H/128][I] or None
    w2: np.ndarray                 # uint8 [E][I][H/2]
    s2: np.ndarray                 # uint16 [E][I/128][H]
    z2: Optional[np.ndarray]       # uint8 [E][I/128][H/2] or None
    T: int
    topk: int
    E: int
    H: int
    I: int
    dtype: int
    name: str = ""

    @property
    def signed(self) -> bool:
        return self.z13 is None


def make_moe_chain(T, topk, E, H, I, dtype=BF16, alpha=1.1, signed=True, seed=0,
                   scale_range=(0.002, 0.01), ids: Optional[np.ndarray] = None, name="") -> MoeChain:
    """Fused-experts inputs: x ~ N(0,1); routing ids from :func:`zipf_routing`
    (``ids`` overrides them, e.g. with out-of-range entries); routing weights
    drawn U[0.05, 1) and normalised to sum 1 per token; int4 weights and
    uniform scales as in :func:`make_grouped`."""
    assert H % GROUP == 0 and I % GROUP == 0
    x = to_bits(_normal(stream(seed, "tokens"), (T, H)), dtype)
    if ids is None:
        ids = zipf_routing(T, E, topk, alpha, seed) if T else np.zeros((0, topk), np.int64)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    wr = 0.05 + 0.95 * stream(seed, "mask").random((T, topk))
    wr = (wr / wr.sum(axis=1, keepdims=True)).astype(np.float32) if T else wr.astype(np.float32)
    _, w13 = _weights(seed, (E, H, 2 * I), signed, tag="w")
    s13 = _scales(seed, (E, H // GROUP, 2 * I), scale_range[0], scale_range[1], dtype, tag="s")
    _, w2 = _weights(seed, (E, I, H), signed, tag="w2")
    s2 = _scales(seed, (E, I // GROUP, H), scale_range[0], scale_range[1], dtype, tag="s2")
    z13 = z2 = None
    if not signed:
        z13 = pack_nibbles(stream(seed, "z").integers(6, 10, size=(E, H // GROUP, 2 * I), dtype=np.int8).view(np.uint8))
        z2 = pack_nibbles(stream(seed, "z2").integers(6, 10, size=(E, I // GROUP, H), dtype=np.int8).view(np.uint8))
    return MoeChain(x=x, topk_ids=ids, topk_w=wr, w13=w13, s13=s13, z13=z13, w2=w2, s2=s2, z2=z2,
                    T=T, topk=topk, E=E, H=H, I=I, dtype=dtype, name=name)


def moe_chain(seed=0) -> MoeChain:
    """Fused-experts chain at the MoE workload's sizes: 64 experts, 512
    tokens, top-8 Zipf(1.1) routing, hidden H=2048, expert width I=1408 (the
    grouped GEMM's K and N); x bf16 N(0,1); signed int4; scales bf16
    U[0.002,0.01]."""
    return make_moe_chain(512, 8, 64, 2048, 1408, BF16, alpha=1.1, signed=True, seed=seed, name="moe_chain")


@dataclasses.dataclass
class MxProblem:
    """W4A8-MXFP4 problem in the plain layout: 16-bit activations ``x [M][K]``,
    E2M1 weight codes ``w [K][N/2]`` (low nibble = even n) and E8M0 weight
    scale bytes ``sw [K/32][N]``."""
    x: np.ndarray
    w: np.ndarray
    sw: np.ndarray
    M: int
    K: int
    N: int
    dtype: int
    name: str = ""


def make_mx(M, K, N, dtype=BF16, seed=0, scale_exp=(-9, -6), x_scale=1.0, outlier_frac=0.0,
            outlier_mult=20.0, name="") -> MxProblem:
    """x ~ N(0,1) * x_scale (optionally with outliers); weight codes uniform
    over the 16 E2M1 patterns; weight scale exponents uniform integers in
    ``scale_exp`` (stored as exponent + 127)."""
    assert K % 32 == 0 and N % 2 == 0
    x = _normal(stream(seed, "x"), (M, K)) * np.float32(x_scale)
    if outlier_frac > 0:
        mask = stream(seed, "mask").random((M, K)) < outlier_frac
        x = np.where(mask, x * np.float32(outlier_mult), x).astype(np.float32)
    codes = stream(seed, "w").integers(0, 16, size=(K, N), dtype=np.uint8)
    sw = (127 + stream(seed, "s").integers(scale_exp[0], scale_exp[1] + 1, size=(K // 32, N))).astype(np.uint8)
    return MxProblem(x=to_bits(x, dtype), w=pack_nibbles(codes), sw=sw, M=M, K=K, N=N, dtype=dtype, name=name)


def mx_decode(M, seed=0, N=14336, K=4096) -> MxProblem:
    """W4A8-MXFP4 decode: the decode shape (K=4096, N=14336), x bf16 N(0,1)."""
    return make_mx(M, K, N, BF16, seed=seed, name=f"mx_decode_m{M}")


@dataclasses.dataclass
class W8Problem:
    """W8A16 problem in the plain layout: 16-bit activations ``x [M][K]``, one
    byte per weight ``w [K][N]`` (int8 when ``zero`` is None, else uint8),
    ``scale [K/group][N]`` 16-bit patterns, ``zero [K/group][N]`` uint8."""
    x: np.ndarray
    w: np.ndarray
    scale: np.ndarray
    zero: Optional[np.ndarray]
    M: int
    K: int
    N: int
    dtype: int
    group: int = GROUP
    name: str = ""


def make_w8(M, K, N, dtype=BF16, signed=True, scale_range=(1e-4, 5e-4), zero_range=(100, 156), seed=0,
            group=GROUP, name="") -> W8Problem:
    """x ~ N(0,1); weight bytes uniform over [0, 255] (read as int8 when signed);
    scales uniform in ``scale_range``; zero points uniform integers in
    ``zero_range`` (unsigned weights only)."""
    assert K % group == 0
    G = K // group
    x = to_bits(_normal(stream(seed, "x"), (M, K)), dtype)
    w = stream(seed, "w").integers(0, 256, size=(K, N), dtype=np.uint8)
    s = _scales(seed, (G, N), scale_range[0], scale_range[1], dtype)
    z = None if signed else stream(seed, "z").integers(zero_range[0], zero_range[1] + 1, size=(G, N)).astype(np.uint8)
    return W8Problem(x=x, w=w, scale=s, zero=z, M=M, K=K, N=N, dtype=dtype, group=group, name=name)


@dataclasses.dataclass
class MxGrouped:
    """Grouped W4A8-MXFP4 problem: routed rows ``x [R][K]`` sorted by expert,
    ``offsets [E+1]``, E2M1 codes ``w [E][K][N/2]``, E8M0 scales
    ``sw [E][K/32][N]``."""
    x: np.ndarray
    offsets: np.ndarray
    w: np.ndarray
    sw: np.ndarray
    E: int
    R: int
    K: int
    N: int
    dtype: int
    name: str = ""


def make_mx_grouped(E, tokens, topk, K, N, dtype=BF16, alpha=1.1, seed=0, counts=None, scale_exp=(-9, -6),
                    name="") -> MxGrouped:
    """Routing as for the W4A16 grouped problems; weight codes uniform over the
    16 E2M1 patterns, scale exponents uniform in ``scale_exp``."""
    offsets, x = _routed_rows(E, tokens, topk, K, dtype, alpha, seed, counts)
    codes = stream(seed, "w").integers(0, 16, size=(E, K, N), dtype=np.uint8)
    sw = (127 + stream(seed, "s").integers(scale_exp[0], scale_exp[1] + 1, size=(E, K // 32, N))).astype(np.uint8)
    return MxGrouped(x=x, offsets=offsets, w=pack_nibbles(codes), sw=sw, E=E, R=int(offsets[-1]), K=K, N=N,
                     dtype=dtype, name=name)


def mx_moe(seed=0) -> MxGrouped:
    """W4A8-MXFP4 at the MoE grouped shape: 64 experts, 512 tokens, top-8
    Zipf(1.1), K=2048, N=1408, bf16 x."""
    return make_mx_grouped(64, 512, 8, 2048, 1408, BF16, alpha=1.1, seed=seed, name="mx_moe")
