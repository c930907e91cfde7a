"""Pins of the oracle's packed-layout statement: hand-computed byte offsets
and exact round trips."""

import numpy as np

from oracle import layout


def test_codes_roundtrip_and_size():
    rng = np.random.default_rng(0)
    for N, K in ((16, 128), (32, 256), (128, 640), (48, 384)):
        c = rng.integers(0, 256, (N, K), dtype=np.uint8)
        p = layout.pack_codes(c)
        assert p.size == layout.packed_codes_bytes(N, K)
        assert np.array_equal(layout.unpack_codes(p, N, K), c)


def test_codes_hand_computed_offsets():
    # Element (n=17, k=200) of a 32x256 matrix: row band j=1, r=1; k-tile t=1,
    # column in tile c=72 -> h=1, q=0, b=8; lane = 1 + 16*0 = 1.
    # offset = (1*2 + 1)*2048 + 1*1024 + 1*16 + 8 = 7192.
    N, K = 32, 256
    c = np.zeros((N, K), dtype=np.uint8)
    c[17, 200] = 0xAB
    p = layout.pack_codes(c)
    assert np.flatnonzero(p).tolist() == [7192]
    # (n=0, k=47): c=47 -> h=0, q=2, b=15, lane 32 -> 32*16 + 15 = 527.
    # (n=0, k=63): h=0, q=3, b=15, lane 48 -> 783.  (n=0, k=64): h=1, q=0,
    # b=0, lane 0 -> 1024.
    c = np.zeros((N, K), dtype=np.uint8)
    c[0, 47] = 1
    c[0, 63] = 2
    c[0, 64] = 3
    p = layout.pack_codes(c)
    assert p[527] == 1 and p[783] == 2 and p[1024] == 3 and np.count_nonzero(p) == 3


def test_each_lane_owns_two_16_column_runs_of_one_row():
    N, K = 16, 128
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    ids = (n * K + k).astype(np.int64)
    # pack the element ids through the same permutation by packing each byte plane
    lo = layout.pack_codes((ids & 0xFF).astype(np.uint8)).astype(np.int64)
    hi = layout.pack_codes((ids >> 8).astype(np.uint8)).astype(np.int64)
    pid = lo | (hi << 8)
    for lane in range(64):
        got = np.concatenate([pid[lane * 16: lane * 16 + 16],
                              pid[1024 + lane * 16: 1024 + lane * 16 + 16]])
        row, col0 = lane % 16, 16 * (lane // 16)
        want = [row * K + col0 + i for i in range(16)] + [row * K + 64 + col0 + i for i in range(16)]
        assert got.tolist() == want


def test_mx_scales_roundtrip_padding_and_offsets():
    rng = np.random.default_rng(1)
    for N, K in ((16, 128), (32, 256), (32, 512), (64, 1152)):
        s = rng.integers(0, 255, (N, K // 32), dtype=np.uint8)
        p = layout.pack_mx_scales(s)
        assert p.size == layout.packed_mx_scales_bytes(N, K)
        assert np.array_equal(layout.unpack_mx_scales(p, N, K), s)
    # (n=17, kb=9) of N=32, K=512: t=2, q=1 -> g=0, i=2; lane = 1 + 16 = 17;
    # offset = ((1*1 + 0)*64 + 17)*4 + 2 = 326.
    s = np.zeros((32, 16), dtype=np.uint8)
    s[17, 9] = 7
    p = layout.pack_mx_scales(s)
    assert np.flatnonzero(p).tolist() == [326]
    # K=256 has 2 k-tiles: one group of 4 with two zero-padded tiles
    assert layout.packed_mx_scales_bytes(32, 256) == 2 * 256
