"""Storage order of this library's 4-bit expert weights, written with numpy
for the tests.

This is a storage format of the library (the lane order of the 16x16x32
MFMA B operand that its 4-bit GEMM reads), not a step of the layer the
pages describe, so it lives with the tests rather than in the oracle.  The
oracle decides the codes, scales and offsets (``oracle.quantize_int4``);
these helpers only say where the library keeps each of them, so that the
GPU quantiser's bytes can be compared with the oracle's codes bit for bit.
The layout is pinned by hand-worked offsets in
``tests/golden/int4_format.json`` (``pin_int4_packing_hand_example``).
"""

from __future__ import annotations

import numpy as np

Q4_GROUP = 128


def pack_int4(q):
    """Pack codes [rows, K] (rows a multiple of 16) into the library's
    storage bytes, returned as [rows/16, K/128, 64, 16].

    Storage is tiled for the GEMM's MFMA operand order (a storage format
    of this library, not of the pages): one 1024-byte tile per 16 rows x
    one group of 128 weights, tiles row-block-major then group; inside a
    tile, 16-byte slot m = col + 16*kq holds row col's weights
    kq*32 .. kq*32+31 of the group as four little-endian 32-bit words
    (word h: weights kq*32 + 8h + 0..7).  In a word of eight consecutive
    weights k0..k7, nibble i (bits 4i..4i+3) holds k_(2i) for i < 4 and
    k_(2(i-4)+1) for i >= 4: even weights in the low half-word, odd
    weights in the high half-word."""
    q = np.asarray(q, np.uint32)
    rows, K = q.shape
    assert rows % 16 == 0 and K % Q4_GROUP == 0
    # [row block, col, group, kq, h, 8 weights]
    k8 = q.reshape(rows // 16, 16, K // Q4_GROUP, 4, 4, 8)
    word = np.zeros(k8.shape[:-1], np.uint32)
    for i in range(4):
        word |= k8[..., 2 * i] << np.uint32(4 * i)
        word |= k8[..., 2 * i + 1] << np.uint32(16 + 4 * i)
    # -> [row block, group, kq, col, h]: slot m = col + 16*kq
    tiles = word.transpose(0, 2, 3, 1, 4).reshape(rows // 16,
                                                   K // Q4_GROUP, 64, 4)
    return np.ascontiguousarray(tiles).astype("<u4").view(np.uint8)


def unpack_int4(packed, rows, K):
    """Inverse of :func:`pack_int4`: codes [rows, K] from the stored
    bytes (any shape holding rows*K/2 bytes in storage order)."""
    b = np.ascontiguousarray(np.asarray(packed, np.uint8)).reshape(-1)
    word = b.view("<u4").reshape(rows // 16, K // Q4_GROUP, 4, 16, 4)
    # [row block, group, kq, col, h] -> [row block, col, group, kq, h]
    word = word.transpose(0, 3, 1, 2, 4)
    q = np.zeros(word.shape + (8,), np.uint8)
    for i in range(4):
        q[..., 2 * i] = (word >> np.uint32(4 * i)) & 15
        q[..., 2 * i + 1] = (word >> np.uint32(16 + 4 * i)) & 15
    return q.reshape(rows, K)


def pack_qparams(scale, offset):
    """Store the per-group (scale, offset) pairs [rows, K/128] in the
    library's tiled order [rows/16, K/128, 16, 2]: one 128-byte tile per
    16 rows x one group, row col's pair at position col."""
    s = np.asarray(scale, np.float32)
    o = np.asarray(offset, np.float32)
    rows, G = s.shape
    st = np.stack([s, o], axis=-1).reshape(rows // 16, 16, G, 2)
    return np.ascontiguousarray(st.transpose(0, 2, 1, 3))


def int4_bytes(rows, K):
    """Storage bytes of a [rows, K] matrix in this format: K/2 code bytes
    per row plus a float32 scale and offset per group."""
    return rows * (K // 2) + rows * (K // Q4_GROUP) * 8
