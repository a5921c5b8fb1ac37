#!/usr/bin/env python3
"""Benchmark of libw4a16 on one MI355X.

Headline workload (one JSON line on stdout): the decode W4A16 configuration,
M in {1, 4, 16}, K=4096, N=14336, group 128, bf16 activations, unsigned int4
weights with per-group uint4 zero points.  One step = the three GEMM calls
(M=1, M=4, M=16) on inputs already resident in HBM.  Weight buffers rotate over
more than 600 MB of distinct copies so the 256 MB Infinity Cache cannot hold
them: every step streams its weights from HBM.

value    = algorithmic bytes of K steps / wall time of the K steps
           (synchronized on both sides) -> GB/s.  The K steps are launched
           from one captured HIP graph (a decode loop is launch-bound when
           each call goes through Python: a call costs more host time than
           the kernel takes on the GPU).
roofline = the dominant kernel (the small-M split-K kernel): algorithmic
           bytes per launch / its average launch duration, timed with HIP
           events on the launch stream, against the 8 TB/s HBM peak.
cpu_baseline = the CPU oracle on the same decode step (host cores).

per_config adds the same measurement for the other workloads (tiny, prefill,
mrange = W4A16 at M = 32..2048 on the decode weights,
MSD, MoE grouped, and the MoE fused-experts chain: routing prep, gather, gate/up
grouped GEMM, SiLU and multiply, down grouped GEMM, weighted sum); they are
reported for completeness, the headline is decode.  msd_page is the MSD
page's own example shape (M=1, K=8192, N=12288); msd_page and msd_basic also time
the page's basic pipeline (integer products written to memory, separate merge)
next to the fused kernel.  The chain's algorithmic
bytes: tokens in and out (T*H*2 each), routing ids and weights (T*topk*8), and
the active experts' gate/up and down weights with their scales.  mx_decode is
W4A8-MXFP4 at the decode shape (bf16 x quantized to MXFP8 inside the GEMM,
MXFP4 weights); its bytes: x + E2M1 codes (K*N/2) + E8M0 scales (K/32*N) + y.
mx_prefill is W4A8-MXFP4 at M=N=K=4096 (activation quantization into a
workspace, then the LDS-staged tile kernel); judged on flops against the
5.0 PFLOP/s dense fp8 peak.  mx_moe is W4A8-MXFP4 at the MoE grouped shape
(quantization of the routed rows, then the grouped tile kernel).  w8_decode / w8_prefill are W8A16 (8-bit integer
weights) at the decode shape (uint8 with zero points) and at 4096^3 (int8);
bytes: x + K*N weight bytes + scales (+ zero points, one byte each) + y.

Algorithmic bytes of one dense call: x (M*K*2) + packed weights (K*N/2) +
scales (K/128*N*2) + zero points (K/128*N/2, if any) + y (M*N*2).
Algorithmic flops: 2*M*N*K (MSD also reports 6*M*N*K int8 ops).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16/fp16 MFMA
INT8_PEAK_TOPS = 5000.0        # dense int8 MFMA
ROTATE_BYTES = 600 * 2 ** 20   # distinct bytes touched before a buffer is reused

METRIC = "TFLOP/s + effective HBM GB/s (% of roofline), W4A16 g128, M=1..4096"


# Sources that define the decode kernel (the dominant kernel of the headline
# step): committed HBM-traffic counts are valid only for these exact files.
DECODE_KERNEL_SOURCES = ("gemm_small.hip", "common.hpp")


def kernel_source_hash(files=None) -> str:
    """Hash of kernel sources (all of csrc/ by default)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_quantized_amd", "csrc")
    names = sorted(files) if files else sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp", ".cpp")))
    for f in names:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def dense_bytes(M, K, N, zero):
    G = K // 128
    return M * K * 2 + K * N // 2 + G * N * 2 + (G * N // 2 if zero else 0) + M * N * 2


# ---------------------------------------------------------------------------
# GPU workloads
# ---------------------------------------------------------------------------

class Workload:
    """Inputs resident on the GPU plus a launch(i) closure (i selects the
    rotated buffer set)."""
    name: str
    calls: list          # list of (label, launch(i), bytes, flops)
    nsets: int


def _dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda:0")


def _prepack(p, w_dev):
    import torch
    import weight_only_quantized_amd as w4
    out = torch.empty(w4.w4a16_prepacked_bytes(p.E, p.K, p.N), dtype=torch.uint8, device="cuda:0")
    w4.w4a16_prepack(w_dev, out, p.E, p.K, p.N, int(p.signed))
    return out


def _copies(t, nbytes_per_set):
    n = max(1, -(-ROTATE_BYTES // max(nbytes_per_set, 1)))
    return [t] + [t.clone() for _ in range(n - 1)]


def decode_workload():
    import torch
    import synth
    import weight_only_quantized_amd as w4
    ps = {M: synth.decode(M) for M in (1, 4, 16)}
    p1 = ps[1]
    wp = _prepack(p1, _dev(p1.w.reshape(-1)))            # same weights for the three M
    sc, zr = _dev(p1.scale), _dev(p1.zero)
    per_set = wp.numel() + sc.numel() * 2 + zr.numel()
    wps = _copies(wp, per_set)
    scs = [sc] + [sc.clone() for _ in range(len(wps) - 1)]
    zrs = [zr] + [zr.clone() for _ in range(len(wps) - 1)]
    xs = {M: _dev(ps[M].x) for M in ps}
    ys = {M: torch.empty((M, p1.N), dtype=torch.int16, device="cuda:0") for M in ps}
    K, N = p1.K, p1.N
    calls = []
    for M in (1, 4, 16):
        def launch(i, M=M):
            j = i % len(wps)
            w4.w4a16_gemm(xs[M], wps[j], scs[j], zrs[j], ys[M], M, K, N, 128, synth.BF16)
        calls.append((f"decode_m{M}", launch, dense_bytes(M, K, N, True), 2 * M * N * K))
    return calls, len(wps)


def mrange_workload():
    """W4A16 over the middle of the M range on the decode weights (K=4096,
    N=14336, uint4 + zero points, bf16): M in {32, 64, 128, 256, 512, 1024,
    2048}, each with the kernel variant the dispatcher picks for it."""
    import torch
    import synth
    import weight_only_quantized_amd as w4
    Ms = (32, 64, 128, 256, 512, 1024, 2048)
    p = synth.make_dense(max(Ms), 4096, 14336, synth.BF16, signed=False, scale_range=(0.002, 0.01),
                         zero_range=(6, 9), seed=0, name="mrange")
    K, N = p.K, p.N
    wp = _prepack(p, _dev(p.w.reshape(-1)))
    sc, zr = _dev(p.scale), _dev(p.zero)
    xfull = _dev(p.x)
    xs = {M: xfull[:M].contiguous() for M in Ms}
    ys = {M: torch.empty((M, N), dtype=torch.int16, device="cuda:0") for M in Ms}
    calls = []
    for M in Ms:
        def launch(i, M=M):
            w4.w4a16_gemm(xs[M], wp, sc, zr, ys[M], M, K, N, 128, synth.BF16)
        calls.append((f"mrange_m{M}", launch, dense_bytes(M, K, N, True), 2 * M * N * K))
    return calls, 1


def tiny_workload():
    import torch
    import synth
    import weight_only_quantized_amd as w4
    p = synth.tiny()
    wp = _prepack(p, _dev(p.w.reshape(-1)))
    x, sc = _dev(p.x), _dev(p.scale)
    y = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda:0")

    def launch(i):
        w4.w4a16_gemm(x, wp, sc, None, y, p.M, p.K, p.N, 128, synth.F16)
    return [("tiny", launch, dense_bytes(p.M, p.K, p.N, False), 2 * p.M * p.N * p.K)], 1


def prefill_workload():
    import torch
    import synth
    import weight_only_quantized_amd as w4
    p = synth.prefill()
    wp = _prepack(p, _dev(p.w.reshape(-1)))
    x, sc = _dev(p.x), _dev(p.scale)
    y = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda:0")
    per_set = wp.numel() + x.numel() * 2 + sc.numel() * 2
    wps = _copies(wp, per_set)
    xs = [x] + [x.clone() for _ in range(len(wps) - 1)]

    def launch(i):
        j = i % len(wps)
        w4.w4a16_gemm(xs[j], wps[j], sc, None, y, p.M, p.K, p.N, 128, synth.BF16)
    return [("prefill", launch, dense_bytes(p.M, p.K, p.N, False), 2 * p.M * p.N * p.K)], len(wps)


def msd_workload():
    import torch
    import synth
    import weight_only_quantized_amd as w4
    p = synth.msd()
    wp = _prepack(p, _dev(p.w.reshape(-1)))
    x, sc = _dev(p.x), _dev(p.scale)
    y = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda:0")
    nb = w4.w4a16_msd_workspace_bytes(p.M, p.K, p.N)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    wps = _copies(wp, wp.numel() + sc.numel() * 2)
    scs = [sc] + [sc.clone() for _ in range(len(wps) - 1)]

    def launch(i):
        j = i % len(wps)
        w4.w4a16_msd_gemm(x, wps[j], scs[j], y, p.M, p.K, p.N, 128, ws, nb)
    return [("msd", launch, dense_bytes(p.M, p.K, p.N, False), 2 * p.M * p.N * p.K)], len(wps)


def _msd_calls(p, name):
    """Fused MSD call and the page's basic pipeline (products through memory)
    on the same problem."""
    import torch
    import synth
    import weight_only_quantized_amd as w4
    wp = _prepack(p, _dev(p.w.reshape(-1)))
    x, sc = _dev(p.x), _dev(p.scale)
    y = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda:0")
    nb = w4.w4a16_msd_workspace_bytes(p.M, p.K, p.N)
    nbb = w4.w4a16_test_msd_basic_workspace_bytes(p.M, p.K, p.N)
    ws = torch.empty(max(nb, nbb), dtype=torch.uint8, device="cuda:0")
    wps = _copies(wp, wp.numel() + sc.numel() * 2)
    scs = [sc] + [sc.clone() for _ in range(len(wps) - 1)]

    def fused(i):
        j = i % len(wps)
        w4.w4a16_msd_gemm(x, wps[j], scs[j], y, p.M, p.K, p.N, 128, ws, nb)

    def basic(i):
        j = i % len(wps)
        w4.w4a16_test_msd_basic(x, wps[j], scs[j], y, p.M, p.K, p.N, 128, ws, nbb)
    nbytes, flops = dense_bytes(p.M, p.K, p.N, False), 2 * p.M * p.N * p.K
    return [(name, fused, nbytes, flops), (name + "_basic", basic, nbytes, flops)], len(wps)


def msd_page_workload():
    """The MSD page's own example shape (M=1, K=8192, N=12288), fused and
    basic pipelines."""
    import synth
    return _msd_calls(synth.msd_page_example(), "msd_page")


def msd_basic_workload():
    """The MSD configuration (M=64, K=N=8192) through the basic pipeline, next
    to the fused kernel."""
    import synth
    return _msd_calls(synth.msd(), "msd")


def moe_workload():
    import numpy as np
    import torch
    import synth
    import weight_only_quantized_amd as w4
    p = synth.moe()
    wp = _prepack(p, _dev(p.w.reshape(-1)))
    x, sc, off = _dev(p.x), _dev(p.scale), _dev(p.offsets)
    y = torch.empty((p.M, p.N), dtype=torch.int16, device="cuda:0")
    active = int(np.count_nonzero(np.diff(p.offsets)))
    G = p.K // 128
    nbytes = p.M * p.K * 2 + active * (p.K * p.N // 2 + G * p.N * 2) + p.M * p.N * 2 + (p.E + 1) * 4
    wps = _copies(wp, wp.numel() + sc.numel() * 2)
    scs = [sc] + [sc.clone() for _ in range(len(wps) - 1)]

    def launch(i):
        j = i % len(wps)
        w4.w4a16_grouped_gemm(x, off, wps[j], scs[j], None, y, p.E, p.M, p.K, p.N, 128, synth.BF16)
    return [("moe", launch, nbytes, 2 * p.M * p.N * p.K)], len(wps)


def moe_chain_workload():
    """Fused-experts chain (routing prep, gather, gate/up grouped GEMM, SiLU and
    multiply, down grouped GEMM, weighted sum) at the MoE workload's sizes."""
    import numpy as np
    import torch
    import synth
    import weight_only_quantized_amd as w4
    c = synth.moe_chain()
    dev = "cuda:0"

    def pack(wplain, K, N):
        out = torch.empty(w4.w4a16_prepacked_bytes(c.E, K, N), dtype=torch.uint8, device=dev)
        w4.w4a16_prepack(_dev(wplain.reshape(-1)), out, c.E, K, N, int(c.signed))
        return out
    w13, w2 = pack(c.w13, c.H, 2 * c.I), pack(c.w2, c.I, c.H)
    s13, s2 = _dev(c.s13), _dev(c.s2)
    x, ids = _dev(c.x), _dev(np.ascontiguousarray(c.topk_ids, np.int32))
    tw = _dev(np.ascontiguousarray(c.topk_w, np.float32))
    out = torch.empty((c.T, c.H), dtype=torch.int16, device=dev)
    nb = w4.w4a16_fused_moe_workspace_bytes(c.T, c.topk, c.E, c.H, c.I)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    per_set = w13.numel() + w2.numel() + (s13.numel() + s2.numel()) * 2
    sets = _copies(w13, per_set)
    w2s = [w2] + [w2.clone() for _ in range(len(sets) - 1)]
    s13s = [s13] + [s13.clone() for _ in range(len(sets) - 1)]
    s2s = [s2] + [s2.clone() for _ in range(len(sets) - 1)]
    active = np.unique(c.topk_ids[(c.topk_ids >= 0) & (c.topk_ids < c.E)]).size
    R = int(((c.topk_ids >= 0) & (c.topk_ids < c.E)).sum())
    wbytes = c.H * 2 * c.I // 2 + c.H // 128 * 2 * c.I * 2 + c.I * c.H // 2 + c.I // 128 * c.H * 2
    nbytes = c.T * c.H * 2 * 2 + c.T * c.topk * 8 + active * wbytes
    flops = 2 * R * c.H * 2 * c.I + 2 * R * c.I * c.H

    def launch(i):
        j = i % len(sets)
        w4.w4a16_fused_moe(x, ids, tw, sets[j], s13s[j], None, w2s[j], s2s[j], None, out, c.T, c.topk, c.E,
                           c.H, c.I, 128, synth.BF16, ws, nb)
    return [("moe_chain", launch, nbytes, flops)], len(sets)


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def mx_bytes(M, K, N):
    """Algorithmic bytes of one W4A8-MXFP4 call: x (16-bit) + E2M1 codes + E8M0
    scales (one per 32 rows and column) + y."""
    return M * K * 2 + K * N // 2 + K // 32 * N + M * N * 2


def mx_decode_workload():
    """W4A8-MXFP4 at the decode shape: M in {1, 4, 16}, K=4096, N=14336, bf16 x
    quantized to MXFP8 inside the GEMM, MXFP4 weights."""
    import torch
    import synth
    import weight_only_quantized_amd as w4
    ps = {M: synth.mx_decode(M) for M in (1, 4, 16)}
    p1 = ps[1]
    K, N = p1.K, p1.N
    wp = torch.empty(w4.w4a8_mxfp4_prepacked_bytes(1, K, N), dtype=torch.uint8, device="cuda:0")
    w4.w4a8_mxfp4_prepack(_dev(p1.w), _dev(p1.sw), wp, 1, K, N)
    wps = _copies(wp, wp.numel())
    xs = {M: _dev(ps[M].x) for M in ps}
    ys = {M: torch.empty((M, N), dtype=torch.int16, device="cuda:0") for M in ps}
    calls = []
    for M in (1, 4, 16):
        def launch(i, M=M):
            w4.w4a8_mxfp4_gemm(xs[M], wps[i % len(wps)], ys[M], M, K, N, synth.BF16, None, 0)
        calls.append((f"mx_decode_m{M}", launch, mx_bytes(M, K, N), 2 * M * N * K))
    return calls, len(wps)


def mx_prefill_workload():
    """W4A8-MXFP4 at the prefill shape (M=N=K=4096): bf16 x quantized to MXFP8
    into a workspace, then the tile kernel; one call = both launches."""
    import torch
    import synth
    import weight_only_quantized_amd as w4
    M = K = N = 4096
    p = synth.make_mx(M, K, N, synth.BF16, name="mx_prefill")
    wp = torch.empty(w4.w4a8_mxfp4_prepacked_bytes(1, K, N), dtype=torch.uint8, device="cuda:0")
    w4.w4a8_mxfp4_prepack(_dev(p.w), _dev(p.sw), wp, 1, K, N)
    x = _dev(p.x)
    y = torch.empty((M, N), dtype=torch.int16, device="cuda:0")
    nb = w4.w4a8_mxfp4_workspace_bytes(M, K)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")

    def launch(i):
        w4.w4a8_mxfp4_gemm(x, wp, y, M, K, N, synth.BF16, ws, nb)
    return [("mx_prefill", launch, mx_bytes(M, K, N), 2 * M * N * K)], 1


def mx_moe_workload():
    """W4A8-MXFP4 at the MoE grouped shape (64 experts, 512 tokens, top-8
    Zipf(1.1), K=2048, N=1408, bf16 x): quantization of the 4096 routed rows
    into a workspace, then the grouped tile kernel; one call = both launches."""
    import numpy as np
    import torch
    import synth
    import weight_only_quantized_amd as w4
    p = synth.mx_moe()
    wp = torch.empty(w4.w4a8_mxfp4_prepacked_bytes(p.E, p.K, p.N), dtype=torch.uint8, device="cuda:0")
    w4.w4a8_mxfp4_prepack(_dev(p.w.reshape(-1)), _dev(p.sw.reshape(-1)), wp, p.E, p.K, p.N)
    x = _dev(p.x)
    off = _dev(np.ascontiguousarray(p.offsets, np.int32))
    y = torch.empty((p.R, p.N), dtype=torch.int16, device="cuda:0")
    nb = w4.w4a8_mxfp4_grouped_workspace_bytes(p.R, p.K)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    active = int(np.count_nonzero(np.diff(p.offsets)))
    nbytes = p.R * p.K * 2 + active * (p.K * p.N // 2 + p.K // 32 * p.N) + p.R * p.N * 2

    def launch(i):
        w4.w4a8_mxfp4_grouped_gemm(x, off, wp, y, p.E, p.R, p.K, p.N, synth.BF16, ws, nb)
    return [("mx_moe", launch, nbytes, 2 * p.R * p.N * p.K)], 1


def w8_bytes(M, K, N, zero):
    """Algorithmic bytes of one W8A16 call: x + 8-bit weights + scales (+ zero
    points, one byte each) + y."""
    G = K // 128
    return M * K * 2 + K * N + G * N * 2 + (G * N if zero else 0) + M * N * 2


def w8_decode_workload():
    """W8A16 at the decode shape: M in {1, 4, 16}, K=4096, N=14336, bf16 x,
    uint8 weights with uint8 zero points, bf16 scales, group 128."""
    import torch
    import synth
    import weight_only_quantized_amd as w4
    ps = {M: synth.make_w8(M, 4096, 14336, synth.BF16, signed=False, seed=0) for M in (1, 4, 16)}
    p1 = ps[1]
    K, N = p1.K, p1.N
    wp = torch.empty(w4.w8a16_prepacked_bytes(1, K, N), dtype=torch.uint8, device="cuda:0")
    w4.w8a16_prepack(_dev(p1.w), wp, 1, K, N, 0)
    sc, zr = _dev(p1.scale), _dev(p1.zero)
    wps = _copies(wp, wp.numel())
    xs = {M: _dev(ps[M].x) for M in ps}
    ys = {M: torch.empty((M, N), dtype=torch.int16, device="cuda:0") for M in ps}
    calls = []
    for M in (1, 4, 16):
        def launch(i, M=M):
            w4.w8a16_gemm(xs[M], wps[i % len(wps)], sc, zr, ys[M], M, K, N, 128, synth.BF16)
        calls.append((f"w8_decode_m{M}", launch, w8_bytes(M, K, N, True), 2 * M * N * K))
    return calls, len(wps)


def w8_prefill_workload():
    """W8A16 at the prefill shape (M=N=K=4096), bf16 x, int8 weights."""
    import torch
    import synth
    import weight_only_quantized_amd as w4
    M = K = N = 4096
    p = synth.make_w8(M, K, N, synth.BF16, signed=True, seed=0)
    wp = torch.empty(w4.w8a16_prepacked_bytes(1, K, N), dtype=torch.uint8, device="cuda:0")
    w4.w8a16_prepack(_dev(p.w), wp, 1, K, N, 1)
    x, sc = _dev(p.x), _dev(p.scale)
    y = torch.empty((M, N), dtype=torch.int16, device="cuda:0")

    def launch(i):
        w4.w8a16_gemm(x, wp, sc, None, y, M, K, N, 128, synth.BF16)
    return [("w8_prefill", launch, w8_bytes(M, K, N, False), 2 * M * N * K)], 1


def _capture(calls, first, count):
    """One HIP graph holding `count` steps (every call once per step, buffer set
    first + i for step i), captured on a side stream.  Replaying it launches the
    kernels back to back with no host work in between, as a serving loop that
    captures its decode step would."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(count):
            for _, launch, _, _ in calls:
                launch(first + i)
    return g


def run_steps(calls, steps, warmup):
    """Wall time of exactly `steps` steps, synchronized on both sides.

    Warmup: `warmup` eager steps, then the same `warmup` steps replayed from a
    graph of their own (loads the graph path).  Timed: one replay of a graph
    holding the `steps` steps."""
    import torch
    for i in range(warmup):
        for _, launch, _, _ in calls:
            launch(i)
    torch.cuda.synchronize()
    gw = _capture(calls, 0, max(warmup, 1))
    g = _capture(calls, warmup, steps)
    gw.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def per_launch_ms(calls, steps, warmup):
    """Average duration of each call: a graph of `steps` back-to-back launches of
    that one call (rotating buffer sets), replayed once to warm up and once
    between two HIP events on the replay stream (torch's current stream)."""
    import torch
    out = []
    for ci in range(len(calls)):
        one = [calls[ci]]
        g = _capture(one, warmup, steps)
        g.replay()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / steps)
    return out


def measure(name, builder, steps, warmup):
    calls, nsets = builder()
    wall = run_steps(calls, steps, warmup)
    lat = per_launch_ms(calls, steps, 2)
    step_bytes = sum(c[2] for c in calls)
    step_flops = sum(c[3] for c in calls)
    out = {
        "ms_per_step": wall / steps * 1e3,
        "GBps": step_bytes * steps / wall / 1e9,
        "TFLOPs": step_flops * steps / wall / 1e12,
        "rotated_sets": nsets,
        "calls": {},
    }
    for (label, _, nb, nf), ms in zip(calls, lat):
        out["calls"][label] = {
            "event_ms": ms,
            "bytes": nb,
            "flops": nf,
            "GBps": nb / (ms * 1e-3) / 1e9,
            "TFLOPs": nf / (ms * 1e-3) / 1e12,
            "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": nf / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        }
    return calls, out


def cpu_baseline(min_seconds=10.0):
    """The oracle (as it stands) on the decode step, repeated for >= min_seconds."""
    import oracle
    import synth
    ps = [synth.decode(M) for M in (1, 4, 16)]
    step_bytes = sum(dense_bytes(p.M, p.K, p.N, True) for p in ps)
    n = 0
    t0 = time.perf_counter()
    while True:
        for p in ps:
            oracle.w4a16(p.x, p.w, p.scale, p.zero, p.M, p.K, p.N, p.dtype)
        n += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": step_bytes * n / el / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": el,
            "sample": f"{n} full decode steps (M=1,4,16; K=4096, N=14336) in fp64, OpenMP"}


def load_traffic(kernel_key):
    """HBM traffic per launch from committed rocprofv3 counter runs, or None if
    missing or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != kernel_source_hash(DECODE_KERNEL_SOURCES):
        return None
    return e.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=["decode", "tiny", "prefill", "msd", "moe", "moe_chain", "msd_page",
                                       "msd_basic", "mx_decode", "mx_prefill", "w8_decode", "w8_prefill", "mrange", "mx_moe"],
                    default=None,
                    help="run only this workload (profiling); no JSON headline unless decode")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the per-config extras")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.copy_mb:
        a = torch.empty(args.copy_mb * 2 ** 20 // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch_read": a.numel() * 4, "write": b.numel() * 4,
                          "launches": args.steps}))
        return

    builders = {"decode": decode_workload, "tiny": tiny_workload, "prefill": prefill_workload,
                "msd": msd_workload, "moe": moe_workload, "moe_chain": moe_chain_workload,
                "msd_page": msd_page_workload, "msd_basic": msd_basic_workload, "mx_decode": mx_decode_workload,
                "mx_prefill": mx_prefill_workload, "w8_decode": w8_decode_workload,
                "w8_prefill": w8_prefill_workload, "mrange": mrange_workload,
                "mx_moe": mx_moe_workload}
    if args.only and args.only != "decode":
        _, out = measure(args.only, builders[args.only], args.steps, args.warmup)
        print(json.dumps({"workload": args.only, **out}), flush=True)
        return

    print("[bench] decode workload", file=sys.stderr, flush=True)
    calls, dec = measure("decode", decode_workload, args.steps, args.warmup)
    ms_step = dec["ms_per_step"]
    step_bytes = sum(c[2] for c in calls)
    launch_ms = sum(v["event_ms"] for v in dec["calls"].values())
    achieved = step_bytes / (launch_ms * 1e-3) / 1e9
    traffic = load_traffic("gemm_small_kernel")

    extra = {}
    if not args.no_extra and not args.only:
        for name in ("tiny", "prefill", "mrange", "msd", "moe", "moe_chain", "msd_page", "msd_basic",
                     "mx_decode", "mx_prefill", "mx_moe", "w8_decode", "w8_prefill"):
            print(f"[bench] {name} workload", file=sys.stderr, flush=True)
            _, extra[name] = measure(name, builders[name], max(10, args.steps // 2), args.warmup)
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline()

    line = {
        "metric": METRIC,
        "value": step_bytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode W4A16 g128: M in {1,4,16}, K=4096, N=14336, bf16 x, uint4 weights "
                        "+ uint4 zero points, bf16 scales (one step = the three GEMM calls)",
            "weight_buffers_rotated": dec["rotated_sets"],
            "tflops": dec["TFLOPs"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gemm_small_kernel<bf16, zero, NB=4, SG=2, D=4 (M<=4) or D=8 (M=16)>",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "per_launch_ms": {k: v["event_ms"] for k, v in dec["calls"].items()},
        },
        "cpu_baseline": cpu,
        "per_config": extra,
        "kernel_source_hash": kernel_source_hash(),
        "decode_kernel_source_hash": kernel_source_hash(DECODE_KERNEL_SOURCES),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
