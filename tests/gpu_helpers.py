"""Device-side helpers for the GPU tests: move synthetic inputs to the GPU,
prepack, run the library entry points, read results back as raw 16-bit
patterns.  Only marshalling; all computation runs in libw4a16."""
from __future__ import annotations

import numpy as np
import torch

import synth
import weight_only_quantized_amd as w4

DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def prepack(p: synth.Problem) -> torch.Tensor:
    """Prepacked weights of p: the group-aligned layout for scale groups of 32
    or 64 rows, the standard one otherwise."""
    w = to_dev(p.w.reshape(-1))
    out = torch.empty(w4.w4a16_prepacked_bytes(p.E, p.K, p.N), dtype=torch.uint8, device=DEV)
    if p.group < 128:
        w4.w4a16_prepack_g(w, out, p.E, p.K, p.N, int(p.signed), p.group)
    else:
        w4.w4a16_prepack(w, out, p.E, p.K, p.N, int(p.signed))
    return out


class Dev:
    """A problem resident on the GPU (inputs and prepacked weights)."""

    def __init__(self, p: synth.Problem):
        self.p = p
        self.x = to_dev(p.x) if p.M else torch.empty((0, p.K), dtype=torch.int16, device=DEV)
        self.scale = to_dev(p.scale)
        self.zero = to_dev(p.zero) if p.zero is not None else None
        self.wp = prepack(p)
        self.offsets = to_dev(p.offsets) if p.offsets is not None else None

    def new_y(self, fill=None):
        y = torch.empty((self.p.M, self.p.N), dtype=torch.int16, device=DEV)
        if fill is not None:
            y.fill_(fill)
        return y

    def gemm(self, y=None):
        p = self.p
        y = self.new_y() if y is None else y
        w4.w4a16_gemm(self.x, self.wp, self.scale, self.zero, y, p.M, p.K, p.N, p.group, p.dtype)
        return y

    def grouped(self, y=None):
        p = self.p
        y = self.new_y() if y is None else y
        w4.w4a16_grouped_gemm(self.x, self.offsets, self.wp, self.scale, self.zero, y, p.E, p.M, p.K, p.N,
                              p.group, p.dtype)
        return y

    def msd(self, y=None, ws=None):
        p = self.p
        y = self.new_y() if y is None else y
        nbytes = w4.w4a16_msd_workspace_bytes(p.M, p.K, p.N)
        if ws is None:
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
        w4.w4a16_msd_gemm(self.x, self.wp, self.scale, y, p.M, p.K, p.N, 128, ws, nbytes)
        return y


def check_tol(y_bits, y_ref_bits, dtype, max_bar=1e-2, l1_bar=2e-3, label=""):
    """Float acceptance: max|y - y_ref| <= 1e-2 max|y_ref| and relative L1 <= 2e-3."""
    import oracle
    mx, l1 = oracle.compare(y_bits, y_ref_bits, dtype)
    print(f"[parity] {label} max_ratio={mx:.3e} rel_l1={l1:.3e}", flush=True)
    assert np.all(np.isfinite(synth.bits_to_f32(y_bits, dtype))), label
    assert mx <= max_bar, (label, mx)
    assert l1 <= l1_bar, (label, l1)
    return mx, l1
