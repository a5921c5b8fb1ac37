"""Grouped (MoE) W4A16 parity against the oracle: the MoE workload with
Zipf(1.1) top-8 routing, and skewed / empty expert edge cases."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _check(orc, p, label):
    from gpu_helpers import Dev, check_tol, to_host_u16
    print(f"[case] {label} E={p.E} R={p.M} K={p.K} N={p.N} counts={np.diff(p.offsets).tolist()[:16]}", flush=True)
    d = Dev(p)
    y = d.grouped(d.new_y(fill=0))
    torch.cuda.synchronize()
    _, y_ref = orc.grouped(p.x, p.offsets, p.w, p.scale, p.zero, p.E, p.M, p.K, p.N, p.dtype, group=p.group)
    return check_tol(to_host_u16(y), y_ref, p.dtype, label=label)


def test_moe_full(orc):
    _check(orc, synth.moe(), "moe")


@pytest.mark.parametrize("halves", [0, 1])
def test_moe_full_half_items_on_off(orc, halves):
    """The MoE workload with the grouped kernel's half items (K range split
    between two wave pairs) turned off and on."""
    import weight_only_quantized_amd as w4
    prev = w4.w4a16_test_tile_halves(halves)
    try:
        _check(orc, synth.moe(), f"moe halves={halves}")
    finally:
        w4.w4a16_test_tile_halves(prev)


@pytest.mark.parametrize("counts,K,N", [
    ([3, 0, 40, 1, 65], 384, 320),     # odd group count: the second half runs one empty step
    ([64] * 3 + [0, 7], 128, 192),     # one group: the second half has no groups
    ([33, 31, 2], 1408, 1408),         # the MoE down projection's K and N
])
def test_half_items_shapes(orc, counts, K, N):
    """Few items: the plan turns whole items into half items (every item fits
    in one round as halves), with odd and single group counts and natural
    half column blocks."""
    p = synth.make_grouped(len(counts), sum(counts), 1, K, N, synth.BF16, signed=True, counts=counts,
                           seed=K + N)
    _check(orc, p, f"grouped_half_{counts[:4]}_{K}_{N}")


@pytest.mark.parametrize("counts,dt,signed", [
    ([5, 0, 17, 1, 0, 9], synth.BF16, True),
    ([0, 0, 0, 40], synth.BF16, False),
    ([300], synth.F16, True),
    ([129, 0, 128, 1, 0], synth.F16, False),
    ([0] * 10 + [3] + [0] * 50 + [200], synth.BF16, True),
])
def test_edge_counts(orc, counts, dt, signed):
    p = synth.make_grouped(len(counts), max(sum(counts), 1), 1, 256, 320, dt, signed=signed,
                           counts=counts, seed=len(counts))
    _check(orc, p, f"grouped_{counts[:6]}")


def test_many_experts_over_workgroup_scan(orc):
    """E larger than one workgroup's scan width (512) exercises the carry."""
    rng = np.random.default_rng(4)
    counts = rng.integers(0, 3, size=700)
    counts[rng.integers(0, 700, 5)] = 70
    p = synth.make_grouped(700, int(counts.sum()), 1, 128, 64, synth.BF16, counts=counts, seed=2)
    _check(orc, p, "many_experts")


@pytest.mark.parametrize("cfg", range(8))
@pytest.mark.parametrize("dt,signed", [(synth.BF16, True), (synth.F16, False)])
def test_tile_configs(orc, cfg, dt, signed):
    """Every workgroup tile configuration of the tile kernel, grouped form:
    partial row tiles, an empty expert, a partial column tile."""
    import weight_only_quantized_amd as w4
    count = w4.w4a16_test_tile_config(-1)
    if cfg >= count:
        pytest.skip(f"only {count} tile configurations")
    counts = [5, 0, 70, 33, 1, 129]
    p = synth.make_grouped(len(counts), sum(counts), 1, 384, 320, dt, signed=signed, counts=counts, seed=cfg)
    prev = w4.w4a16_test_tile_config(cfg)
    try:
        _check(orc, p, f"grouped_tile_cfg{cfg}")
    finally:
        w4.w4a16_test_tile_config(-1)


@pytest.mark.parametrize("counts,n", [([1, 1, 1], 64), ([2, 0, 31], 192), ([40] * 9, 64)])
def test_fewer_items_than_xcds(orc, counts, n):
    """Fewer (row tile, column block) items than XCDs, or a count that is not a
    multiple of it: most per-XCD ranges are empty or uneven."""
    p = synth.make_grouped(len(counts), sum(counts), 1, 256, n, synth.BF16, signed=True, counts=counts,
                           seed=sum(counts))
    _check(orc, p, f"grouped_small_{counts[:4]}_{n}")


@pytest.mark.parametrize("group,dt,signed", [(256, synth.BF16, True), (1024, synth.F16, False)])
def test_grouped_group_sizes(orc, group, dt, signed):
    """Grouped GEMM with scale groups of 256 rows and with one scale per column."""
    counts = [5, 0, 70, 33, 1, 129]
    p = synth.make_grouped(len(counts), sum(counts), 1, 1024, 320, dt, signed=signed, counts=counts,
                           seed=group, group=group)
    _check(orc, p, f"grouped_group{group}")


@pytest.mark.parametrize("group,dt,signed,counts", [
    (32, synth.BF16, True, [5, 0, 70, 33, 1, 129]),
    (64, synth.F16, False, [200, 3, 0, 97]),
    (32, synth.F16, False, [40] * 9),
    (64, synth.BF16, True, [0, 0, 17]),
])
def test_grouped_small_scale_groups(orc, group, dt, signed, counts):
    """Grouped GEMM with scale groups of 32 and 64 rows (group-aligned
    weights): ragged experts, experts without rows, both tile shapes."""
    p = synth.make_grouped(len(counts), sum(counts), 1, 1024, 320, dt, signed=signed, counts=counts,
                           seed=group + len(counts), group=group)
    _check(orc, p, f"grouped_group{group}_{counts[:4]}")
