"""The packed ("pre-shuffled") weight layout, written from its definition
(CPU oracle; test infrastructure only).

This layout is this library's own (the pages only teach that the scale
layout a kernel assumes must be pinned by a round-trip test: fish.audio
blog, section "Estrategia de cuantización FP8", the weight_scale stride bug).
It is stated here in words and implemented with reshapes, independently of
the GPU packer's index arithmetic, so packed buffers can be compared
byte for byte.

Codes of a weight W [N, K] (N % 16 == 0, K % 128 == 0), KT = K / 128:

* The matrix is cut into tiles of 16 rows x 128 columns.  Tile (j, t) covers
  rows 16j..16j+15 and columns 128t..128t+127 and occupies the 2048 bytes at
  offset (j * KT + t) * 2048: tiles of one row band are consecutive along K.
* Inside a tile, element (r, c) (r = row within the tile, c = column within
  the tile) sits at byte  h * 1024 + lane * 16 + b  with
  h = c // 64, q = (c % 64) // 16, b = c % 16 and lane = r + 16 * q.
  So wavefront lane `lane` owns row lane % 16, columns 16q..16q+15 (first
  16 bytes) and 64+16q..64+16q+15 (second 16 bytes, 1024 bytes later), which
  is the operand order of gfx950's 16x16x128 fp8 matrix instruction; each
  1024-byte half of a tile is read by one 64-lane, 16-bytes-per-lane load.

MX scales (E8M0 bytes, logical [N, K/32]) with KG = ceil(KT / 4):

* For row band j and k-tile group g (k-tiles 4g..4g+3) there are 256 bytes at
  offset (j * KG + g) * 256; byte  lane * 4 + i  holds the scale of row
  16j + (lane % 16) and 32-column block  4 * (4g + i) + lane // 16.  Bytes of
  k-tiles past KT are zero.

Block scales (fp32, logical [N/128, K/128]) are stored as is, row-major.
"""

import numpy as np

TILE_N = 16
TILE_K = 128


def packed_codes_bytes(N, K):
    return N * K


def packed_mx_scales_bytes(N, K):
    KT = K // TILE_K
    KG = (KT + 3) // 4
    return (N // TILE_N) * KG * 256


def _check(N, K):
    if N % TILE_N or K % TILE_K:
        raise ValueError(f"N={N} must be a multiple of 16 and K={K} of 128")


def pack_codes(codes):
    """Row-major uint8 codes [N, K] -> packed 1-D uint8 array."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    _check(N, K)
    # axes: j, r, t, h, q, b   (column in tile c = 64h + 16q + b)
    v = codes.reshape(N // 16, 16, K // 128, 2, 4, 16)
    # target order: j, t, h, q, r, b  (lane = q*16 + r)
    return np.ascontiguousarray(v.transpose(0, 2, 3, 4, 1, 5)).reshape(-1)


def unpack_codes(packed, N, K):
    """Packed 1-D uint8 array -> row-major codes [N, K]."""
    _check(N, K)
    v = np.asarray(packed, dtype=np.uint8).reshape(N // 16, K // 128, 2, 4, 16, 16)
    # axes: j, t, h, q, r, b  -> j, r, t, h, q, b
    return np.ascontiguousarray(v.transpose(0, 4, 1, 2, 3, 5)).reshape(N, K)


def pack_mx_scales(scales):
    """Logical E8M0 scales [N, K/32] -> packed 1-D uint8 array."""
    s = np.asarray(scales, dtype=np.uint8)
    N, KB = s.shape
    K = KB * 32
    _check(N, K)
    KT = K // 128
    KG = (KT + 3) // 4
    pad = np.zeros((N, KG * 16), dtype=np.uint8)
    pad[:, :KB] = s
    # axes: j, r, g, i, q   (32-block index = 4*(4g+i) + q)
    v = pad.reshape(N // 16, 16, KG, 4, 4)
    # target order: j, g, q, r, i  (lane = q*16 + r, byte = lane*4 + i)
    return np.ascontiguousarray(v.transpose(0, 2, 4, 1, 3)).reshape(-1)


def unpack_mx_scales(packed, N, K):
    """Packed 1-D uint8 array -> logical E8M0 scales [N, K/32]."""
    _check(N, K)
    KT = K // 128
    KG = (KT + 3) // 4
    v = np.asarray(packed, dtype=np.uint8).reshape(N // 16, KG, 4, 16, 4)
    # axes: j, g, q, r, i -> j, r, g, i, q
    full = np.ascontiguousarray(v.transpose(0, 3, 1, 4, 2)).reshape(N, KG * 16)
    return full[:, : K // 32]
