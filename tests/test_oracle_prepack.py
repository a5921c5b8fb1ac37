"""Pins of the prepacked-layout reference (the library's own format).

The layout is this project's design (the pages only motivate an offline
reorder of int4 weights: "Marlin layout" in the pwwt.cn notes §6.2, QUICK's
offline interleave that skips the shared-memory write-back after dequant, and
Humming's "reorder into the target kernel's layout").  Its statement, in
words: 1024-byte tiles ordered (expert, 16-column block, 128-row group); slot
L of a tile holds column 16*nb + L%16 for rows 128*g + 32*(L//16) + r; word t
of the slot holds r = 8t + i with the code of row r at bit 4*(i//2) + 16*(i%2);
codes are u (unsigned) or q+8 (signed).

Pins: spot positions taken from that statement; a bijection over all bits;
the round trip over every byte value at every position.  The group-aligned
layout (scale groups of 32 or 64 rows) exchanges the roles of the chunk
c = L // 16 and the word t: word t of slot L holds rows 128*g + 32*t +
8*(L//16) + i.  Its pins: its own spot positions, the round trip, and the
statement that it is layout 0 with rows permuted inside each 32x32 block of
(chunk, word) positions.
"""
import numpy as np
import pytest

import synth


def _single(K, N, k, n, code, E=1, e=0):
    codes = np.zeros((E, K, N), np.uint8)
    codes[e, k, n] = code
    return synth.pack_nibbles(codes)


@pytest.mark.parametrize("k,n,byte,shift", [
    (0, 0, 0, 0),        # slot 0, word 0, i=0 -> bit 0
    (1, 0, 2, 0),        # i=1 -> bit 16 -> byte 2 low nibble
    (2, 0, 0, 4),        # i=2 -> bit 4
    (3, 0, 2, 4),        # i=3 -> bit 20
    (7, 0, 3, 4),        # i=7 -> bit 28 -> byte 3 high nibble
    (8, 0, 4, 0),        # word 1
    (31, 0, 15, 4),      # word 3, i=7
    (32, 0, 256, 0),     # next 32-row chunk: slot 16
    (0, 1, 16, 0),       # next column: slot 1
    (0, 15, 240, 0),     # slot 15
    (128, 0, 1024, 0),   # next group: next tile
    (0, 16, 2 * 1024, 0),  # next column block: after G=2 tiles
    (255, 31, 3 * 1024 + 63 * 16 + 15, 4),
])
def test_spot_positions(orc, k, n, byte, shift):
    K, N = 256, 64
    w = _single(K, N, k, n, 0x5)
    p = orc.prepack(w, 1, K, N, is_signed=False)
    nz = np.nonzero(p)[0]
    assert list(nz) == [byte]
    assert p[byte] == (0x5 << shift)


def test_signed_code_is_q_plus_8(orc):
    K, N = 128, 16
    q = np.arange(-8, 8)
    codes = np.zeros((K, N), np.uint8)
    codes[0, :] = (q & 0xF).astype(np.uint8)        # row 0, columns hold -8..7
    p = orc.prepack(synth.pack_nibbles(codes), 1, K, N, is_signed=True)
    # row 0 of column j sits in slot j, bit 0 of word 0
    got = np.array([p[16 * j] & 0xF for j in range(16)])
    assert np.array_equal(got, q + 8)


def test_bijection(orc):
    E, K, N = 2, 256, 64
    rng = np.random.default_rng(0)
    # every input nibble position gets a distinct marker through 4 one-hot planes
    codes = rng.integers(0, 16, size=(E, K, N)).astype(np.uint8)
    p = orc.prepack(synth.pack_nibbles(codes), E, K, N, False)
    assert np.array_equal(np.sort(synth.unpack_nibbles(p.reshape(-1))), np.sort(codes.reshape(-1)))
    # one position at a time lands in exactly one distinct nibble
    seen = set()
    for (e, k, n) in [(0, 0, 0), (1, 255, 63), (0, 100, 17), (1, 3, 40), (0, 200, 33)]:
        pk = orc.prepack(_single(K, N, k, n, 0xF, E, e), E, K, N, False)
        nzb = np.nonzero(pk)[0]
        assert len(nzb) == 1
        key = (int(nzb[0]), int(pk[nzb[0]]))
        assert key not in seen
        seen.add(key)


@pytest.mark.parametrize("signed", [False, True])
def test_round_trip_all_byte_values(orc, signed):
    E, K, N = 2, 384, 128
    # each byte position sees every value 0..255 across 256 shifted copies is too
    # slow; instead cover all 256 values at every byte offset class mod 256
    base = (np.arange(E * K * N // 2) % 256).astype(np.uint8)
    for shift in (0, 1, 17, 128):
        w = np.roll(base, shift).reshape(E, K, N // 2)
        p = orc.prepack(w, E, K, N, signed)
        back = orc.unpack(p, E, K, N, signed)
        assert np.array_equal(back, w.reshape(-1))


@pytest.mark.parametrize("k,n,byte,shift", [
    (0, 0, 0, 0),        # slot 0, word 0, i=0
    (1, 0, 2, 0),        # i=1 -> bit 16
    (7, 0, 3, 4),        # i=7 -> bit 28
    (8, 0, 256, 0),      # rows 8..15 of the 32-row block: chunk 1 -> slot 16, word 0
    (16, 0, 512, 0),     # chunk 2 -> slot 32
    (24, 0, 768, 0),     # chunk 3 -> slot 48
    (32, 0, 4, 0),       # next 32-row block: word 1 of slot 0
    (96, 0, 12, 0),      # word 3
    (127, 15, 768 + 15 * 16 + 12 + 3, 4),  # chunk 3, column 15, word 3, i=7
    (128, 0, 1024, 0),   # next 128-row block: next tile
    (0, 16, 2 * 1024, 0),
])
def test_group_aligned_spot_positions(orc, k, n, byte, shift):
    K, N = 256, 64
    p = orc.prepack(_single(K, N, k, n, 0x5), 1, K, N, is_signed=False, layout=1)
    nz = np.nonzero(p)[0]
    assert list(nz) == [byte]
    assert p[byte] == (0x5 << shift)


@pytest.mark.parametrize("signed", [False, True])
def test_group_aligned_round_trip(orc, signed):
    E, K, N = 2, 384, 128
    base = (np.arange(E * K * N // 2) % 251).astype(np.uint8)
    w = base.reshape(E, K, N // 2)
    p = orc.prepack(w, E, K, N, signed, layout=1)
    assert np.array_equal(orc.unpack(p, E, K, N, signed, layout=1), w.reshape(-1))


def test_group_aligned_is_a_row_permutation_of_layout0(orc):
    """Layout 1 of W equals layout 0 of W with the rows of every 128-row block
    permuted by k = 32t + 8c + i -> 32c + 8t + i."""
    E, K, N = 1, 256, 64
    codes = np.random.default_rng(4).integers(0, 16, size=(K, N)).astype(np.uint8)
    perm = np.empty(K, np.int64)
    for g in range(K // 128):
        for t in range(4):
            for c in range(4):
                for i in range(8):
                    perm[128 * g + 32 * c + 8 * t + i] = 128 * g + 32 * t + 8 * c + i
    p1 = orc.prepack(synth.pack_nibbles(codes), E, K, N, False, layout=1)
    p0 = orc.prepack(synth.pack_nibbles(codes[perm]), E, K, N, False, layout=0)
    assert np.array_equal(p1, p0)
